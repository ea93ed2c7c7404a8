// lpc_device.hpp -- device-side building blocks for the gfx950 FP8 codec kernels.
//
// Two element layouts are used:
//   * granule (quantize): one lane owns 16 contiguous elements, so the 8
//     adjacent lanes of a wavefront-aligned group own one 128-element scale
//     block; the block absmax is reduced across those 8 lanes with DPP.
//   * lane vector of W elements (reduce-scatter, all-gather, dequantize, fused):
//     one lane owns W contiguous elements, chosen so that a lane writes 16
//     bytes of output (W = 4 for fp32, 8 for bf16; 4 where the output is
//     codes), and a wavefront's loads and stores are single contiguous runs.
//     128/W lanes own a block (32 or 16); the absmax is reduced with DPP
//     inside each 16-lane row and, for W = 4, one ds_swizzle between the two
//     rows of the half-wavefront.
// No kernel allocates LDS for these reductions.
//
// FP8 is OCP E4M3FN (the gfx950 native FP8 format): the conversions below use
// the gfx950 instructions v_cvt_pk_fp8_f32 (round to nearest even) and
// v_cvt_pk_f32_fp8 (exact).  Values are clamped to +-448 first with v_med3,
// which makes the conversion saturating whatever the instruction does on
// overflow.
//
// Large outputs are written with non-temporal stores: they are not read again
// by the kernel, and streaming them past the L2 leaves no dirty lines for the
// end-of-kernel write-back.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#pragma clang fp contract(off)

namespace lpc {

constexpr int kBlock = 128;        // elements per scale
constexpr int kGranule = 16;       // elements per lane (granule layout)
constexpr int kLanesPerBlock = kBlock / kGranule;  // 8
constexpr float kFp8Max = 448.0f;
constexpr int kMaxRanks = 8;

// clang vector types: the forms the non-temporal load/store builtins accept
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));

struct RankCodes {
    const uint8_t* codes[kMaxRanks];
    const float* scales[kMaxRanks];
};

struct RankBufs {
    const void* p[kMaxRanks];
};

// per-rank outputs of the all-ranks launches of the emulated collectives
struct RankQuant {
    uint8_t* codes[kMaxRanks];
    float* scales[kMaxRanks];
};

struct RankOut {
    void* p[kMaxRanks];
};

// ---------------------------------------------------------------------------
// cross-lane block max (DPP inside 16-lane rows, ds_swizzle across rows)
// ---------------------------------------------------------------------------

// Max over each aligned group of 8 lanes: quad_perm [1,0,3,2] (xor 1),
// quad_perm [2,3,0,1] (xor 2), row_half_mirror (lane i <-> 7-i inside each
// 8-lane half row: joins the two quads).
__device__ __forceinline__ float group8_max(float v) {
    int x = __float_as_int(v);
    v = fmaxf(v, __int_as_float(__builtin_amdgcn_update_dpp(x, x, 0xB1, 0xF, 0xF, false)));
    x = __float_as_int(v);
    v = fmaxf(v, __int_as_float(__builtin_amdgcn_update_dpp(x, x, 0x4E, 0xF, 0xF, false)));
    x = __float_as_int(v);
    v = fmaxf(v, __int_as_float(__builtin_amdgcn_update_dpp(x, x, 0x141, 0xF, 0xF, false)));
    return v;
}

// Max over each 16-lane row: group8_max, then row_mirror (lane i <-> 15-i
// joins the two 8-lane halves of the row).
__device__ __forceinline__ float group16_max(float v) {
    v = group8_max(v);
    const int x = __float_as_int(v);
    return fmaxf(v, __int_as_float(__builtin_amdgcn_update_dpp(x, x, 0x140, 0xF, 0xF, false)));
}

// Max over each 32-lane half-wavefront: group16_max, then ds_swizzle in bit
// mode with xor mask 16 (swaps the two 16-lane rows of each 32-lane group).
__device__ __forceinline__ float group32_max(float v) {
    v = group16_max(v);
    const int x = __float_as_int(v);
    constexpr int kSwapRows = 0x1F | (0x10 << 10);  // and_mask 0x1F, or_mask 0, xor_mask 0x10
    return fmaxf(v, __int_as_float(__builtin_amdgcn_ds_swizzle(x, kSwapRows)));
}

// ---------------------------------------------------------------------------
// XCD-aware tile order
// ---------------------------------------------------------------------------

// Workgroups of a launch are handed to the 8 XCDs round-robin by workgroup
// id.  This maps blockIdx.x to a tile index so that each XCD gets one
// contiguous run of tiles: neighbouring tiles share scale cache lines, and
// this way they share them inside one XCD's L2.  A bijection on
// [0, gridDim.x) for any grid size.
__device__ __forceinline__ size_t xcd_tile() {
    constexpr unsigned kXcds = 8;
    const unsigned nwg = gridDim.x, b = blockIdx.x;
    const unsigned per = nwg / kXcds, rem = nwg % kXcds;
    const unsigned x = b % kXcds, k = b / kXcds;
    return (size_t)(x * per + (x < rem ? x : rem) + k);
}

// ---------------------------------------------------------------------------
// E4M3 codec
// ---------------------------------------------------------------------------

__device__ __forceinline__ float clamp448(float q) {
    return __builtin_amdgcn_fmed3f(q, -kFp8Max, kFp8Max);
}

// four already-scaled values -> four codes in one dword (element 0 in byte 0)
__device__ __forceinline__ uint32_t encode4(float a, float b, float c, float d) {
    int w = __builtin_amdgcn_cvt_pk_fp8_f32(clamp448(a), clamp448(b), 0, false);
    w = __builtin_amdgcn_cvt_pk_fp8_f32(clamp448(c), clamp448(d), w, true);
    return (uint32_t)w;
}

// Blocks whose scale is at least this take the reciprocal route below; the
// rest divide.  It keeps every residual and quotient that can change a code
// clear of underflow.
constexpr float kMinRecipScale = 0x1p-80f;

// fl32(v / s), the correctly rounded quotient, from r = fl32(1 / s): q0 =
// fl32(v * r) is within 1.5 ulp of v / s; a correction step q + fl32(v - q*s)
// * r (two FMAs, the residual exact) brings it within one ulp, and a second
// step then gives the correctly rounded quotient (Markstein's theorem: with r
// within half an ulp of 1/s and q within one ulp of v/s, the corrected
// quotient is v/s rounded to nearest).  The sign is copied from v so that -0
// stays -0.  Quotients below 2^-10 in magnitude, the only ones an underflow
// could touch when s >= kMinRecipScale, encode as signed zero either way.
__device__ __forceinline__ float quotient(float v, float s, float r) {
    const float q0 = v * r;
    const float q1 = __builtin_fmaf(__builtin_fmaf(-q0, s, v), r, q0);
    const float q2 = __builtin_fmaf(__builtin_fmaf(-q1, s, v), r, q1);
    return __builtin_copysignf(q2, v);
}

// codes of fl32(v[j] / s), four per dword, for a block scale s > 0
template <int N>
__device__ __forceinline__ void encode_quotients(const float (&v)[N], float s, uint32_t (&w)[N / 4]) {
    float q[N];
    if (s >= kMinRecipScale) {
        const float r = 1.0f / s;
#pragma unroll
        for (int j = 0; j < N; ++j) q[j] = quotient(v[j], s, r);
    } else {
#pragma unroll
        for (int j = 0; j < N; ++j) q[j] = v[j] / s;
    }
#pragma unroll
    for (int k = 0; k < N / 4; ++k) w[k] = encode4(q[4 * k], q[4 * k + 1], q[4 * k + 2], q[4 * k + 3]);
}

// exact decode of the four codes in a dword
__device__ __forceinline__ void decode4(uint32_t w, float* out) {
    auto lo = __builtin_amdgcn_cvt_pk_f32_fp8((int)w, false);
    auto hi = __builtin_amdgcn_cvt_pk_f32_fp8((int)w, true);
    out[0] = lo[0];
    out[1] = lo[1];
    out[2] = hi[0];
    out[3] = hi[1];
}

// ---------------------------------------------------------------------------
// granule layout (16 elements per lane, 8 lanes per block)
// ---------------------------------------------------------------------------

// Blockwise quantization of a granule whose 8-lane group forms one block:
// returns the codes of fl32(v[j] / s) and sets *scale = fl32(absmax / 448)
// (identical in all 8 lanes).  The scale is an IEEE division; the quotients
// are correctly rounded (quotient()), as the quantization rule requires.
__device__ __forceinline__ uint4 quantize_granule(const float (&v)[kGranule], float* scale) {
    float amax = 0.0f;
#pragma unroll
    for (int j = 0; j < kGranule; ++j) amax = fmaxf(amax, fabsf(v[j]));
    amax = group8_max(amax);
    const float s = amax / kFp8Max;
    *scale = s;
    if (s == 0.0f) return make_uint4(0u, 0u, 0u, 0u);
    uint32_t w[4];
    encode_quotients(v, s, w);
    return make_uint4(w[0], w[1], w[2], w[3]);
}

// ---------------------------------------------------------------------------
// bfloat16
// ---------------------------------------------------------------------------

__device__ __forceinline__ float bf16lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }

// two floats -> two bf16 (round to nearest even) packed low/high
__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
    __bf16 ha = (__bf16)a;
    __bf16 hb = (__bf16)b;
    return (uint32_t)__builtin_bit_cast(uint16_t, ha) |
           ((uint32_t)__builtin_bit_cast(uint16_t, hb) << 16);
}

// granule loads: four 16-byte loads for fp32, two for bf16 (widened exactly)
__device__ __forceinline__ void load16(const float* __restrict__ p, float (&v)[kGranule]) {
    const float4* q = reinterpret_cast<const float4*>(p);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        float4 t = q[j];
        v[4 * j] = t.x;
        v[4 * j + 1] = t.y;
        v[4 * j + 2] = t.z;
        v[4 * j + 3] = t.w;
    }
}

__device__ __forceinline__ void load16(const uint16_t* __restrict__ p, float (&v)[kGranule]) {
    const uint4* q = reinterpret_cast<const uint4*>(p);
#pragma unroll
    for (int j = 0; j < 2; ++j) {
        uint4 t = q[j];
        uint32_t w[4] = {t.x, t.y, t.z, t.w};
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            v[8 * j + 2 * k] = bf16lo(w[k]);
            v[8 * j + 2 * k + 1] = bf16hi(w[k]);
        }
    }
}

// ---------------------------------------------------------------------------
// lane vectors of W = 4 or 8 elements (128/W lanes per block)
// ---------------------------------------------------------------------------

template <int W> struct LaneCodes;
template <> struct LaneCodes<4> { using T = uint32_t; };
template <> struct LaneCodes<8> { using T = uint2; };

// Elements per lane that make one lane's output 16 bytes.
template <typename Out> constexpr int lane_width() { return 16 / (int)sizeof(Out); }

// W codes; NT = non-temporal (streaming) load
template <int W, bool NT>
__device__ __forceinline__ typename LaneCodes<W>::T load_codes(const uint8_t* __restrict__ p) {
    if constexpr (W == 4) {
        if constexpr (NT) return __builtin_nontemporal_load(reinterpret_cast<const uint32_t*>(p));
        else return *reinterpret_cast<const uint32_t*>(p);
    } else {
        if constexpr (NT) {
            const u32x2_t v = __builtin_nontemporal_load(reinterpret_cast<const u32x2_t*>(p));
            return make_uint2(v.x, v.y);
        } else {
            return *reinterpret_cast<const uint2*>(p);
        }
    }
}

template <int W>
__device__ __forceinline__ void store_codes(uint8_t* __restrict__ p, typename LaneCodes<W>::T c) {
    *reinterpret_cast<typename LaneCodes<W>::T*>(p) = c;
}

// d[j] = fl32(E4M3(code j) * s)
__device__ __forceinline__ void dequant_lane(uint32_t c, float s, float (&d)[4]) {
    decode4(c, d);
#pragma unroll
    for (int j = 0; j < 4; ++j) d[j] = d[j] * s;
}

__device__ __forceinline__ void dequant_lane(uint2 c, float s, float (&d)[8]) {
    decode4(c.x, d);
    decode4(c.y, d + 4);
#pragma unroll
    for (int j = 0; j < 8; ++j) d[j] = d[j] * s;
}

// Blockwise quantization of a lane vector whose 128/W-lane group forms one
// block: returns the codes and sets *scale (identical across the group).
__device__ __forceinline__ uint32_t quantize_lane(const float (&v)[4], float* scale) {
    float amax = fmaxf(fmaxf(fabsf(v[0]), fabsf(v[1])), fmaxf(fabsf(v[2]), fabsf(v[3])));
    amax = group32_max(amax);
    const float s = amax / kFp8Max;
    *scale = s;
    if (s == 0.0f) return 0u;
    uint32_t w[1];
    encode_quotients(v, s, w);
    return w[0];
}

__device__ __forceinline__ uint2 quantize_lane(const float (&v)[8], float* scale) {
    float amax = 0.0f;
#pragma unroll
    for (int j = 0; j < 8; ++j) amax = fmaxf(amax, fabsf(v[j]));
    amax = group16_max(amax);
    const float s = amax / kFp8Max;
    *scale = s;
    if (s == 0.0f) return make_uint2(0u, 0u);
    uint32_t w[2];
    encode_quotients(v, s, w);
    return make_uint2(w[0], w[1]);
}

// 16-byte non-temporal stores of a lane's output (W = 4 fp32, W = 8 bf16)
__device__ __forceinline__ void store_lane_nt(float* __restrict__ p, const float (&d)[4]) {
    const f32x4_t v = {d[0], d[1], d[2], d[3]};
    __builtin_nontemporal_store(v, reinterpret_cast<f32x4_t*>(p));
}

__device__ __forceinline__ void store_lane_nt(uint16_t* __restrict__ p, const float (&d)[8]) {
    const u32x4_t v = {pack_bf16x2(d[0], d[1]), pack_bf16x2(d[2], d[3]), pack_bf16x2(d[4], d[5]),
                       pack_bf16x2(d[6], d[7])};
    __builtin_nontemporal_store(v, reinterpret_cast<u32x4_t*>(p));
}

}  // namespace lpc
