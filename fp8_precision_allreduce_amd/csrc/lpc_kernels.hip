// lpc_kernels.hip -- gfx950 kernels of the FP8 low-precision collective path
// and their launchers.  Arguments reaching these launchers have been checked
// by the C ABI layer (lpc_api.hip); nothing here validates again.
//
// The quantizers use one 16-element granule per lane (a wavefront covers 8
// scale blocks); the reduce-scatter, all-gather, fused and dequantize kernels
// give each lane a vector of 4 or 8 elements, so that every lane writes 16
// bytes (see lpc_device.hpp); DDA flat and DDA tree's one-rank reduce-scatter
// give each lane one 32-bit word of every rank's buffer, in 64-lane
// workgroups.  The other kernels use 256-lane workgroups.
// Rank loops are unrolled by template parameter so that all N loads of a lane
// are in flight before the first add.
#include <tuple>

#include "lpc_device.hpp"
#include "lpc_launch.hpp"

namespace lpc {

constexpr int kThreads = 256;
constexpr int kGranPerWG = kThreads;

static inline dim3 grid_for(size_t granules, unsigned y = 1) {
    return dim3((unsigned)((granules + kGranPerWG - 1) / kGranPerWG), y, 1);
}

__device__ __forceinline__ size_t granule_id() {
    return (size_t)blockIdx.x * kThreads + threadIdx.x;
}

// Every kernel of the library is launched through this helper.  It converts
// the arguments to the kernel's parameter types and returns the status of
// this launch itself (not whatever error an earlier call left behind).
template <typename... P, typename... A>
static hipError_t launch(void (*kernel)(P...), dim3 grid, dim3 block, uint32_t shmem, hipStream_t stream,
                         A... args) {
    static_assert(sizeof...(P) == sizeof...(A) && sizeof...(P) > 0, "argument count");
    std::tuple<P...> vals(args...);
    return std::apply(
        [&](auto&... v) {
            void* ptrs[] = {static_cast<void*>(&v)...};
            return hipLaunchKernel(reinterpret_cast<const void*>(kernel), grid, block, ptrs, shmem, stream);
        },
        vals);
}

// ---------------------------------------------------------------------------
// (1) quantize
// ---------------------------------------------------------------------------

// A wavefront quantizes 64 granules (1,024 elements) in one piece: its input, 4 KiB of fp32 or
// 2 KiB of bf16, comes in with loads that each cover one contiguous KiB (lane l reads bytes
// 16l..16l+15 of every KiB), non-temporal; LDS then regroups the rows so that each lane holds one
// whole 16-element granule, and the granule arithmetic follows (one block max and scale per 8
// lanes).  The non-temporal loads leave no freshly read input in the caches: the launch that
// follows a quantization (the reduce-scatter) measured about 2 us slower after plain loads at
// 16 MiB.  Loaded as granules (32 or 64 contiguous bytes a lane), non-temporal loads fetched lines
// more than once; with ordinary granule loads the bf16 quantizer measured 68.8 us at 256 MiB
// against 66.9 us regrouped (cold HBM, same run).
constexpr int kWaveGranules = 64;

// Input rows of one KiB per wavefront (4 fp32, 2 bf16), and 16-byte chunks per granule (as many).
template <typename In> constexpr uint32_t wave_rows() { return (uint32_t)sizeof(In); }

// LDS byte offset of 16-byte chunk j of granule G within a wavefront's rows: the chunk's slot is
// rotated by G/4 so that consecutive lanes touch distinct 16-byte bank groups, both when a loaded
// row is written (4 or 2 lanes per granule) and when a granule is read back (one lane each).
template <typename In>
__device__ __forceinline__ uint32_t regroup_slot(uint32_t G, uint32_t j) {
    constexpr uint32_t R = wave_rows<In>();
    return G * (16u * R) + (((j + (G >> 2)) & (R - 1)) * 16u);
}

// Lane l of a wavefront gets granule l of the `left` (64, or fewer, a multiple of 8) granules that
// start at src, through `lds` (the wavefront's 1 KiB per row).  Lanes l >= left get nothing.
template <typename In>
__device__ __forceinline__ void load_wave_granules(const In* __restrict__ src, uint32_t left, uint32_t l,
                                                   uint8_t* lds, float (&v)[kGranule]) {
    constexpr uint32_t R = wave_rows<In>();
    const u32x4_t* rows = reinterpret_cast<const u32x4_t*>(src);
    u32x4_t r[R];
    if (left == kWaveGranules) {
        // every wavefront but possibly the last: all rows in flight at once
#pragma unroll
        for (uint32_t k = 0; k < R; ++k) r[k] = __builtin_nontemporal_load(rows + k * 64 + l);
#pragma unroll
        for (uint32_t k = 0; k < R; ++k)
            *reinterpret_cast<u32x4_t*>(lds + regroup_slot<In>(k * (64 / R) + l / R, l % R)) = r[k];
    } else {
#pragma unroll
        for (uint32_t k = 0; k < R; ++k) {
            const uint32_t G = k * (64 / R) + l / R;
            if (G < left) {
                r[k] = __builtin_nontemporal_load(rows + k * 64 + l);
                *reinterpret_cast<u32x4_t*>(lds + regroup_slot<In>(G, l % R)) = r[k];
            }
        }
    }
    // LDS operations of one wavefront complete in order: the reads below see every lane's writes
    __builtin_amdgcn_wave_barrier();
    if (l >= left) return;
#pragma unroll
    for (uint32_t j = 0; j < R; ++j) {
        const u32x4_t t = *reinterpret_cast<const u32x4_t*>(lds + regroup_slot<In>(l, j));
        if constexpr (R == 4) {
#pragma unroll
            for (int q = 0; q < 4; ++q) v[4 * j + q] = __uint_as_float(t[q]);
        } else {
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                v[8 * j + 2 * q] = bf16lo(t[q]);
                v[8 * j + 2 * q + 1] = bf16hi(t[q]);
            }
        }
    }
}

// codes of granule g (non-temporal) and, from the block's first lane, its scale
__device__ __forceinline__ void store_granule(const uint4& c, float sc, size_t g, uint32_t l,
                                              uint8_t* __restrict__ codes, float* __restrict__ scales) {
    const u32x4_t cv = {c.x, c.y, c.z, c.w};
    __builtin_nontemporal_store(cv, reinterpret_cast<u32x4_t*>(codes + g * kGranule));
    if ((l & (kLanesPerBlock - 1)) == 0) scales[g / kLanesPerBlock] = sc;
}

template <typename In>
__global__ __launch_bounds__(kThreads) void quantize_kernel(const In* __restrict__ x, size_t ngran,
                                                            uint8_t* __restrict__ codes,
                                                            float* __restrict__ scales) {
    __shared__ __attribute__((aligned(16))) uint8_t lds[kThreads / 64][kWaveGranules * 16 * sizeof(In)];
    // the wavefront index read as a wave-uniform value, so that g0, left and the branches on them
    // are scalar
    const uint32_t w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), l = threadIdx.x & 63;
    const size_t g0 = (xcd_tile() * (kThreads / 64) + w) * kWaveGranules;
    if (g0 >= ngran) return;  // whole wavefronts past the end
    // granules of this wavefront that exist: all 64, or (the last wavefront) a multiple of 8
    const uint32_t left = (uint32_t)(ngran - g0 < kWaveGranules ? ngran - g0 : kWaveGranules);
    float v[kGranule];
    load_wave_granules(x + g0 * kGranule, left, l, lds[w], v);
    if (l >= left) return;  // whole 8-lane groups
    float sc;
    const uint4 c = quantize_granule(v, &sc);
    store_granule(c, sc, g0 + l, l, codes, scales);
}

hipError_t launch_quantize(const void* x, int in_bf16, size_t n, uint8_t* codes, float* scales,
                           hipStream_t stream) {
    const size_t ngran = n / kGranule;
    const size_t waves = (ngran + kWaveGranules - 1) / kWaveGranules;
    const dim3 grid((unsigned)((waves + kThreads / 64 - 1) / (kThreads / 64)));
    if (in_bf16)
        return launch(quantize_kernel<uint16_t>, grid, dim3(kThreads), 0, stream, static_cast<const uint16_t*>(x),
                      ngran, codes, scales);
    return launch(quantize_kernel<float>, grid, dim3(kThreads), 0, stream, static_cast<const float*>(x), ngran,
                  codes, scales);
}

// ---------------------------------------------------------------------------
// Lane-vector kernels: one lane owns W contiguous elements of a chunk (W = 4
// when the lane writes fp32 or codes, 8 when it writes bf16, so that every
// lane stores 16 bytes), 128/W lanes a scale block; tiles are taken in
// XCD-aware order.
// ---------------------------------------------------------------------------

template <int W>
static inline dim3 lane_grid(size_t elems, unsigned y = 1) {
    const size_t lanes = elems / W;
    return dim3((unsigned)((lanes + kThreads - 1) / kThreads), y, 1);
}

template <int W>
__device__ __forceinline__ size_t lane_elem() {
    return (xcd_tile() * kThreads + threadIdx.x) * W;
}

// Rank-order FP32 sum of the W elements at rank-buffer offset e over N ranks:
// all N code and scale loads are issued before the first add.
template <int N, int W>
__device__ __forceinline__ void rank_sum(const RankCodes& in, size_t e, float (&acc)[W]) {
    typename LaneCodes<W>::T c[N];
    float s[N];
#pragma unroll
    for (int p = 0; p < N; ++p) {
        c[p] = load_codes<W, true>(in.codes[p] + e);
        s[p] = in.scales[p][e / kBlock];
    }
    dequant_lane(c[0], s[0], acc);
#pragma unroll
    for (int p = 1; p < N; ++p) {
        float d[W];
        dequant_lane(c[p], s[p], d);
#pragma unroll
        for (int j = 0; j < W; ++j) acc[j] = acc[j] + d[j];
    }
}

// ---------------------------------------------------------------------------
// (2) reduce-scatter step: N-way dequant + rank-order FP32 sum of one chunk,
// requantized (kRequant, W = 4) or written out as the sum (kSumF32, W = 4;
// kSumBF16, W = 8).
// ---------------------------------------------------------------------------

enum RsOut { kRequant = 0, kSumF32 = 1, kSumBF16 = 2 };

template <int Mode> constexpr int rs_width() { return Mode == kSumBF16 ? 8 : 4; }

template <int N, int Mode>
__global__ __launch_bounds__(kThreads) void reduce_scatter_kernel(RankCodes in, size_t chunk_off, size_t C,
                                                                  uint8_t* __restrict__ cc,
                                                                  float* __restrict__ cs,
                                                                  void* __restrict__ out) {
    constexpr int W = rs_width<Mode>();
    const size_t i = lane_elem<W>();
    if (i >= C) return;  // whole blocks of 128/W lanes drop out together (C % 128 == 0)
    float acc[W];
    rank_sum<N, W>(in, chunk_off + i, acc);
    if constexpr (Mode == kRequant) {
        float s;
        const auto c = quantize_lane(acc, &s);
        store_codes<W>(cc + i, c);
        if ((threadIdx.x & (kBlock / W - 1)) == 0) cs[i / kBlock] = s;
    } else if constexpr (Mode == kSumF32) {
        store_lane_nt(static_cast<float*>(out) + i, acc);
    } else {
        store_lane_nt(static_cast<uint16_t*>(out) + i, acc);
    }
}

template <int Mode>
static hipError_t launch_rs_n(const RankCodes& in, int nranks, size_t chunk_off, size_t C, uint8_t* cc, float* cs,
                              void* out, hipStream_t stream) {
    const dim3 grid = lane_grid<rs_width<Mode>()>(C), block(kThreads);
    switch (nranks) {
#define LPC_RS_CASE(NR) \
    case NR: return launch(reduce_scatter_kernel<NR, Mode>, grid, block, 0, stream, in, chunk_off, C, cc, cs, out);
        LPC_RS_CASE(1) LPC_RS_CASE(2) LPC_RS_CASE(3) LPC_RS_CASE(4)
        LPC_RS_CASE(5) LPC_RS_CASE(6) LPC_RS_CASE(7) LPC_RS_CASE(8)
#undef LPC_RS_CASE
    }
    return hipErrorInvalidValue;
}

hipError_t launch_reduce_scatter_chunk(const RankCodes& in, int nranks, int rank, size_t n,
                                       uint8_t* cc, float* cs, hipStream_t stream) {
    const size_t C = n / nranks;
    return launch_rs_n<kRequant>(in, nranks, (size_t)rank * C, C, cc, cs, nullptr, stream);
}

hipError_t launch_reduce_scatter_out(const RankCodes& in, int nranks, int rank, size_t n, void* out,
                                     int out_bf16, hipStream_t stream) {
    const size_t C = n / nranks;
    if (out_bf16) return launch_rs_n<kSumBF16>(in, nranks, (size_t)rank * C, C, nullptr, nullptr, out, stream);
    return launch_rs_n<kSumF32>(in, nranks, (size_t)rank * C, C, nullptr, nullptr, out, stream);
}

// ---------------------------------------------------------------------------
// (3) all-gather dequantization (grid.y = chunk);  flat dequantization
// ---------------------------------------------------------------------------

// Wavefronts a full MI355X runs at once at 8 per SIMD (256 CUs x 4 SIMDs).
constexpr size_t kRoundWaves = 8192;

// Lane vectors per lane of a launch whose grid.y has `slices` slices of C / W lane vectors each:
// 2 (half a slice apart) for fp32 output (W = 4) when one per lane would take more than one round
// of wavefronts and C splits into two halves of whole blocks (C % 256 == 0), else 1.  On cold HBM
// a lane's first conversion waits a full load latency, so the launch pays about one latency per
// round of wavefronts (the all-gather at 16 MiB fp32, N = 8: 5.45 us with one vector per lane,
// 4.59 us with two).
static int lane_vectors(size_t slices, size_t C, int W) {
    if (W != 4 || C % (2 * kBlock) != 0) return 1;
    const size_t wgs = (C / W + kThreads - 1) / kThreads * slices;
    return wgs * (kThreads / 64) > kRoundWaves ? 2 : 1;
}

// chunk p = blockIdx.y; lane t dequantizes vectors t, t + H, ... of it
template <typename Out, int V>
__global__ __launch_bounds__(kThreads) void allgather_kernel(RankCodes chunks, size_t C, size_t H,
                                                             Out* __restrict__ out) {
    constexpr int W = lane_width<Out>();
    using Codes = typename LaneCodes<W>::T;
    const size_t t = xcd_tile() * kThreads + threadIdx.x;
    if (t >= H) return;  // whole blocks of 128/W lanes drop out together (H % (128/W) == 0)
    const int p = blockIdx.y;
    Codes c[V];
    float s[V];
#pragma unroll
    for (int k = 0; k < V; ++k) {
        const size_t i = (t + k * H) * W;
        c[k] = load_codes<W, true>(chunks.codes[p] + i);
        s[k] = chunks.scales[p][i / kBlock];
    }
#pragma unroll
    for (int k = 0; k < V; ++k) {
        const size_t i = (t + k * H) * W;
        float d[W];
        dequant_lane(c[k], s[k], d);
        store_lane_nt(out + (size_t)p * C + i, d);
    }
}

template <typename Out, int V>
static hipError_t launch_allgather_v(const RankCodes& chunks, int nranks, size_t C, void* out, hipStream_t stream) {
    const size_t H = C / lane_width<Out>() / V;
    const dim3 grid((unsigned)((H + kThreads - 1) / kThreads), nranks);
    return launch(allgather_kernel<Out, V>, grid, dim3(kThreads), 0, stream, chunks, C, H, static_cast<Out*>(out));
}

hipError_t launch_allgather(const RankCodes& chunks, int nranks, size_t n, void* out, int out_bf16,
                            hipStream_t stream) {
    const size_t C = n / nranks;
    if (out_bf16) return launch_allgather_v<uint16_t, 1>(chunks, nranks, C, out, stream);
    if (lane_vectors(nranks, C, lane_width<float>()) == 2)
        return launch_allgather_v<float, 2>(chunks, nranks, C, out, stream);
    return launch_allgather_v<float, 1>(chunks, nranks, C, out, stream);
}

template <typename Out>
__global__ __launch_bounds__(kThreads) void dequant_kernel(const uint8_t* __restrict__ codes,
                                                           const float* __restrict__ scales, size_t n,
                                                           Out* __restrict__ out) {
    constexpr int W = lane_width<Out>();
    const size_t i = lane_elem<W>();
    if (i >= n) return;
    float d[W];
    dequant_lane(load_codes<W, true>(codes + i), scales[i / kBlock], d);
    store_lane_nt(out + i, d);
}

hipError_t launch_dequant(const uint8_t* codes, const float* scales, size_t n, void* out, int out_bf16,
                          hipStream_t stream) {
    if (out_bf16)
        return launch(dequant_kernel<uint16_t>, lane_grid<lane_width<uint16_t>()>(n), dim3(kThreads), 0, stream,
                      codes, scales, n, static_cast<uint16_t*>(out));
    return launch(dequant_kernel<float>, lane_grid<lane_width<float>()>(n), dim3(kThreads), 0, stream, codes,
                  scales, n, static_cast<float*>(out));
}

// ---------------------------------------------------------------------------
// (2)+(3) fused.  A slice (grid.y) has H lanes, each owning lane vectors of W
// elements; the chunk has lanes = C / W vectors, H = lanes / V.
//   * Slices y < V reduce: lane t takes vector y*H + t of the own chunk,
//     loads it from all N ranks, sums in rank order, requantizes, writes the
//     requantized codes and their dequantization (from registers), and
//     dequantizes peer rank + 1's chunk at the same vector.
//   * Slice y >= V dequantizes peer rank + y - V + 2's chunk: lane t takes
//     vectors t, t + H, ..., t + (V-1)*H.
// Every lane issues all of its loads before its first conversion.  All code
// loads are non-temporal: each stream is read once.
//
// On cold HBM a lane's first conversion waits a full load latency, so the
// launch is bound by how many latencies lie on its path.  At 16 MiB fp32 and
// N = 8 one vector per lane (V = 1) is 14,336 wavefronts, two rounds of what
// the GPU holds at once (8 per SIMD): 6.7 us.  V = 2 is 8,192 wavefronts, one
// round, with the reduction spread over two slices of one vector per lane:
// 5.3 us (a reduction slice of two vectors per lane measured 5.4 us, a slice
// for the reduction alone 6.0-6.2 us).  Where V = 1 already fits in one round
// (8 MiB and below) it is faster, and with bf16 output (W = 8) V = 2 measured
// no faster at 16-256 MiB.
// ---------------------------------------------------------------------------

// slices of the fused launch: V reduction slices and one per peer other than rank + 1
__host__ __device__ constexpr int fused_slices(int N, int V) { return V + (N > 2 ? N - 2 : 0); }

template <int N, typename Out, int V>
__global__ __launch_bounds__(kThreads) void rs_ag_fused_kernel(RankCodes in, RankCodes peers, int rank,
                                                               size_t C, size_t H, uint8_t* __restrict__ cc,
                                                               float* __restrict__ cs,
                                                               Out* __restrict__ out) {
    constexpr int W = lane_width<Out>();
    using Codes = typename LaneCodes<W>::T;
    const size_t t = xcd_tile() * kThreads + threadIdx.x;
    if (t >= H) return;  // whole blocks of 128/W lanes drop out together (H % (128/W) == 0)
    const int y = blockIdx.y;
    float d[W];
    if (y < V) {
        const size_t i = ((size_t)y * H + t) * W;
        const size_t own = (size_t)rank * C + i;
        int q = rank + 1;
        if (q >= N) q -= N;
        Codes c[N], pc;
        float s[N], ps;
#pragma unroll
        for (int p = 0; p < N; ++p) {
            c[p] = load_codes<W, true>(in.codes[p] + own);
            s[p] = in.scales[p][own / kBlock];
        }
        if constexpr (N > 1) {
            pc = load_codes<W, true>(peers.codes[q] + i);
            ps = peers.scales[q][i / kBlock];
        }
        float acc[W];
        dequant_lane(c[0], s[0], acc);
#pragma unroll
        for (int p = 1; p < N; ++p) {
            dequant_lane(c[p], s[p], d);
#pragma unroll
            for (int j = 0; j < W; ++j) acc[j] = acc[j] + d[j];
        }
        float sc;
        const Codes code = quantize_lane(acc, &sc);
        store_codes<W>(cc + i, code);
        if ((threadIdx.x & (kBlock / W - 1)) == 0) cs[i / kBlock] = sc;
        dequant_lane(code, sc, d);  // own chunk straight from registers
        store_lane_nt(out + own, d);
        if constexpr (N > 1) {
            dequant_lane(pc, ps, d);
            store_lane_nt(out + (size_t)q * C + i, d);
        }
        return;
    }
    int q = rank + y - V + 2;  // this slice's peer
    if (q >= N) q -= N;
    Codes pc[V];
    float ps[V];
#pragma unroll
    for (int k = 0; k < V; ++k) {
        const size_t i = (t + k * H) * W;
        pc[k] = load_codes<W, true>(peers.codes[q] + i);
        ps[k] = peers.scales[q][i / kBlock];
    }
#pragma unroll
    for (int k = 0; k < V; ++k) {
        const size_t i = (t + k * H) * W;
        dequant_lane(pc[k], ps[k], d);
        store_lane_nt(out + (size_t)q * C + i, d);
    }
}

// Lane vectors per lane of the fused launch: 2 for fp32 output when one per lane would take more
// than one round of wavefronts and the chunk splits into two halves of whole blocks (C % 256 == 0),
// else 1.
static int fused_vectors(int nranks, size_t C, int out_bf16) {
    if (out_bf16) return 1;
    return lane_vectors(fused_slices(nranks, 1), C, lane_width<float>());
}

template <int N, typename Out, int V>
static hipError_t launch_fused_v(const RankCodes& in, const RankCodes& peers, int rank, size_t C, uint8_t* cc,
                                 float* cs, void* out, hipStream_t stream) {
    const size_t H = C / lane_width<Out>() / V;
    const dim3 grid((unsigned)((H + kThreads - 1) / kThreads), fused_slices(N, V));
    return launch(rs_ag_fused_kernel<N, Out, V>, grid, dim3(kThreads), 0, stream, in, peers, rank, C, H, cc, cs,
                  static_cast<Out*>(out));
}

hipError_t launch_rs_ag_fused(const RankCodes& in, const RankCodes& peers, int nranks, int rank, size_t n,
                              uint8_t* cc, float* cs, void* out, int out_bf16, hipStream_t stream) {
    const size_t C = n / nranks;
    const bool two = fused_vectors(nranks, C, out_bf16) == 2;
    switch (nranks) {
#define LPC_FUSED_CASE(NR)                                                                              \
    case NR:                                                                                            \
        if (out_bf16) return launch_fused_v<NR, uint16_t, 1>(in, peers, rank, C, cc, cs, out, stream); \
        if (two) return launch_fused_v<NR, float, 2>(in, peers, rank, C, cc, cs, out, stream);          \
        return launch_fused_v<NR, float, 1>(in, peers, rank, C, cc, cs, out, stream);
        LPC_FUSED_CASE(1) LPC_FUSED_CASE(2) LPC_FUSED_CASE(3) LPC_FUSED_CASE(4)
        LPC_FUSED_CASE(5) LPC_FUSED_CASE(6) LPC_FUSED_CASE(7) LPC_FUSED_CASE(8)
#undef LPC_FUSED_CASE
    }
    return hipErrorInvalidValue;
}

// ---------------------------------------------------------------------------
// DDA flat: N bf16 buffers -> FP32 rank-order sum -> bf16.  Small messages
// are latency-bound, so the launch spreads them thin: one lane owns one
// 32-bit word of every buffer (2 bf16, one 4-byte non-temporal load per
// rank), 64-lane workgroups in XCD-aware order.  On cold HBM at 64 KiB per
// rank this measured 2.29 us against 2.38 us with 4 bf16 a lane (8-byte
// loads) and 2.55-2.62 us with one rank a lane (16-byte loads exchanged
// through LDS); at 16 KiB 2.17 against 2.32 us.  A last odd element goes to
// a second, one-wavefront launch, which keeps the element-by-element tail
// out of the main kernel's code.
//
// The same word-wide reduce serves DDA tree's reduce-scatter of one chunk,
// bf16 or fp32 (2 or 1 elements a lane).
// ---------------------------------------------------------------------------

constexpr int kDdaThreads = 64;
constexpr int kDdaElems = 4;  // elements a lane of the all-ranks DDA flat launch

// A launch takes at most 2^31 - 1 lanes along a grid dimension.  One word a lane
// reaches that only for buffers near the largest accepted size (2^32 bf16, or a
// 2^32-element fp32 chunk); such a launch stops at kMaxWordGroups workgroups and
// its lanes take every grid-size-th word (the Strided variants below).
constexpr size_t kMaxWordGroups = ((size_t)1 << 31) / kDdaThreads - 1;

// The rank-order FP32 sum of the 32-bit word at byte offset off of every rank's
// buffer (two bf16, or one fp32), packed back into one word; non-temporal
// loads, each word is read once.
template <int N, bool BF16>
__device__ __forceinline__ uint32_t reduce_word(const RankBufs& b, size_t off) {
    uint32_t w[N];
#pragma unroll
    for (int p = 0; p < N; ++p)
        w[p] = __builtin_nontemporal_load(reinterpret_cast<const uint32_t*>(static_cast<const uint8_t*>(b.p[p]) + off));
    if constexpr (BF16) {
        float lo = bf16lo(w[0]), hi = bf16hi(w[0]);
#pragma unroll
        for (int p = 1; p < N; ++p) {
            lo = lo + bf16lo(w[p]);
            hi = hi + bf16hi(w[p]);
        }
        return pack_bf16x2(lo, hi);
    } else {
        float acc = __uint_as_float(w[0]);
#pragma unroll
        for (int p = 1; p < N; ++p) acc = acc + __uint_as_float(w[p]);
        return __float_as_uint(acc);
    }
}

// the rank-order sum of elements e .. e+3, written as bf16 (ordinary loads)
template <int N>
__device__ __forceinline__ void dda_flat_quad(const RankBufs& b, size_t e, uint16_t* __restrict__ out) {
    u32x2_t v[N];
#pragma unroll
    for (int p = 0; p < N; ++p) v[p] = *reinterpret_cast<const u32x2_t*>(static_cast<const uint16_t*>(b.p[p]) + e);
    float acc[kDdaElems] = {bf16lo(v[0][0]), bf16hi(v[0][0]), bf16lo(v[0][1]), bf16hi(v[0][1])};
#pragma unroll
    for (int p = 1; p < N; ++p) {
        acc[0] = acc[0] + bf16lo(v[p][0]);
        acc[1] = acc[1] + bf16hi(v[p][0]);
        acc[2] = acc[2] + bf16lo(v[p][1]);
        acc[3] = acc[3] + bf16hi(v[p][1]);
    }
    *reinterpret_cast<uint2*>(out + e) = make_uint2(pack_bf16x2(acc[0], acc[1]), pack_bf16x2(acc[2], acc[3]));
}

// the rank-order sum of element i alone
template <int N>
__device__ __forceinline__ void dda_flat_one(const RankBufs& b, size_t i, uint16_t* __restrict__ out) {
    float acc = __uint_as_float((uint32_t)static_cast<const uint16_t*>(b.p[0])[i] << 16);
#pragma unroll
    for (int p = 1; p < N; ++p) acc = acc + __uint_as_float((uint32_t)static_cast<const uint16_t*>(b.p[p])[i] << 16);
    const __bf16 h = (__bf16)acc;
    out[i] = __builtin_bit_cast(uint16_t, h);
}

// this lane's elements e .. e+3 (fewer at the tail) of the flat reduce
template <int N>
__device__ __forceinline__ void dda_flat_at(const RankBufs& b, size_t n, size_t e, uint16_t* __restrict__ out) {
    if (e + kDdaElems <= n) {
        dda_flat_quad<N>(b, e, out);
    } else {
        for (size_t i = e; i < n; ++i) dda_flat_one<N>(b, i, out);
    }
}

// lanes over the nw = n / 2 whole words
template <int N, bool Strided>
__global__ __launch_bounds__(kDdaThreads) void dda_flat_kernel(RankBufs b, size_t nw, uint32_t* __restrict__ out) {
    const size_t w = xcd_tile() * kDdaThreads + threadIdx.x;
    if constexpr (Strided) {
        const size_t stride = (size_t)gridDim.x * kDdaThreads;
        for (size_t v = w; v < nw; v += stride) out[v] = reduce_word<N, true>(b, v * 4);
    } else {
        if (w >= nw) return;
        out[w] = reduce_word<N, true>(b, w * 4);
    }
}

// one lane per element of [e0, n) (at most 1)
template <int N>
__global__ __launch_bounds__(kDdaThreads) void dda_flat_tail_kernel(RankBufs b, size_t e0, size_t n,
                                                                    uint16_t* __restrict__ out) {
    const size_t i = e0 + threadIdx.x;
    if (i >= n) return;
    dda_flat_one<N>(b, i, out);
}

template <int N>
static hipError_t launch_dda_flat_n(const RankBufs& b, size_t n, uint16_t* out, hipStream_t stream) {
    const size_t nw = n / 2;
    if (nw > 0) {
        const size_t groups = (nw + kDdaThreads - 1) / kDdaThreads;
        uint32_t* o = reinterpret_cast<uint32_t*>(out);
        const hipError_t e =
            groups <= kMaxWordGroups
                ? launch(dda_flat_kernel<N, false>, dim3((unsigned)groups), dim3(kDdaThreads), 0, stream, b, nw, o)
                : launch(dda_flat_kernel<N, true>, dim3((unsigned)kMaxWordGroups), dim3(kDdaThreads), 0, stream, b,
                         nw, o);
        if (e != hipSuccess) return e;
    }
    if (n % 2) return launch(dda_flat_tail_kernel<N>, dim3(1), dim3(kDdaThreads), 0, stream, b, nw * 2, n, out);
    return hipSuccess;
}

hipError_t launch_dda_flat(const RankBufs& b, int nranks, size_t n, void* out, hipStream_t stream) {
    uint16_t* o = static_cast<uint16_t*>(out);
    switch (nranks) {
#define LPC_DDA_CASE(NR) \
    case NR: return launch_dda_flat_n<NR>(b, n, o, stream);
        LPC_DDA_CASE(1) LPC_DDA_CASE(2) LPC_DDA_CASE(3) LPC_DDA_CASE(4)
        LPC_DDA_CASE(5) LPC_DDA_CASE(6) LPC_DDA_CASE(7) LPC_DDA_CASE(8)
#undef LPC_DDA_CASE
    }
    return hipErrorInvalidValue;
}

// ---------------------------------------------------------------------------
// DDA tree (unquantized): reduce-scatter of one chunk, and the gather copy.
// The all-ranks reduce-scatter and the gather copy move 16-byte granules (4
// fp32 or 8 bf16); the one-rank reduce-scatter moves 32-bit words.
// ---------------------------------------------------------------------------

// the rank-order sum of the 16-byte granule at byte offset `off` of every
// rank's buffer, written to dst
template <int N, bool BF16>
__device__ __forceinline__ void dda_tree_rs_at(const RankBufs& b, size_t off, void* __restrict__ dst) {
    uint4 v[N];
#pragma unroll
    for (int p = 0; p < N; ++p) v[p] = *reinterpret_cast<const uint4*>(static_cast<const uint8_t*>(b.p[p]) + off);
    if (BF16) {
        float acc[8];
        const uint32_t w0[4] = {v[0].x, v[0].y, v[0].z, v[0].w};
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            acc[2 * k] = bf16lo(w0[k]);
            acc[2 * k + 1] = bf16hi(w0[k]);
        }
#pragma unroll
        for (int p = 1; p < N; ++p) {
            const uint32_t w[4] = {v[p].x, v[p].y, v[p].z, v[p].w};
#pragma unroll
            for (int k = 0; k < 4; ++k) {
                acc[2 * k] = acc[2 * k] + bf16lo(w[k]);
                acc[2 * k + 1] = acc[2 * k + 1] + bf16hi(w[k]);
            }
        }
        *reinterpret_cast<uint4*>(dst) =
            make_uint4(pack_bf16x2(acc[0], acc[1]), pack_bf16x2(acc[2], acc[3]), pack_bf16x2(acc[4], acc[5]),
                       pack_bf16x2(acc[6], acc[7]));
    } else {
        float4 acc = *reinterpret_cast<const float4*>(&v[0]);
#pragma unroll
        for (int p = 1; p < N; ++p) {
            const float4 d = *reinterpret_cast<const float4*>(&v[p]);
            acc.x = acc.x + d.x;
            acc.y = acc.y + d.y;
            acc.z = acc.z + d.z;
            acc.w = acc.w + d.w;
        }
        *reinterpret_cast<float4*>(dst) = acc;
    }
}

// One rank's chunk: one 32-bit word a lane, like DDA flat, in 64-lane workgroups.  At
// 2 MiB bf16 per rank on cold HBM this measured 2.56 us against 2.95 us for 16-byte
// granules with ordinary loads in 256-lane workgroups.
template <int N, bool BF16, bool Strided>
__global__ __launch_bounds__(kDdaThreads) void dda_tree_rs_kernel(RankBufs b, size_t chunk_off_bytes, size_t nw,
                                                                  uint32_t* __restrict__ out) {
    const size_t w = (size_t)blockIdx.x * kDdaThreads + threadIdx.x;
    if constexpr (Strided) {
        const size_t stride = (size_t)gridDim.x * kDdaThreads;
        for (size_t v = w; v < nw; v += stride) out[v] = reduce_word<N, BF16>(b, chunk_off_bytes + v * 4);
    } else {
        if (w >= nw) return;
        out[w] = reduce_word<N, BF16>(b, chunk_off_bytes + w * 4);
    }
}

template <int N, bool BF16>
static hipError_t launch_tree_rs_n(const RankBufs& b, size_t off, size_t nw, uint32_t* out, hipStream_t stream) {
    const size_t groups = (nw + kDdaThreads - 1) / kDdaThreads;
    if (groups <= kMaxWordGroups)
        return launch(dda_tree_rs_kernel<N, BF16, false>, dim3((unsigned)groups), dim3(kDdaThreads), 0, stream, b,
                      off, nw, out);
    return launch(dda_tree_rs_kernel<N, BF16, true>, dim3((unsigned)kMaxWordGroups), dim3(kDdaThreads), 0, stream, b,
                  off, nw, out);
}

hipError_t launch_dda_tree_rs(const RankBufs& b, int bf16, int nranks, int rank, size_t n, void* out,
                              hipStream_t stream) {
    const size_t esz = bf16 ? 2 : 4;
    const size_t chunk_bytes = n / nranks * esz;
    const size_t nw = chunk_bytes / 4;
    const size_t off = (size_t)rank * chunk_bytes;
    uint32_t* o = static_cast<uint32_t*>(out);
    switch (nranks) {
#define LPC_TREE_CASE(NR)                                                    \
    case NR:                                                                 \
        if (bf16) return launch_tree_rs_n<NR, true>(b, off, nw, o, stream); \
        return launch_tree_rs_n<NR, false>(b, off, nw, o, stream);
        LPC_TREE_CASE(1) LPC_TREE_CASE(2) LPC_TREE_CASE(3) LPC_TREE_CASE(4)
        LPC_TREE_CASE(5) LPC_TREE_CASE(6) LPC_TREE_CASE(7) LPC_TREE_CASE(8)
#undef LPC_TREE_CASE
    }
    return hipErrorInvalidValue;
}

__global__ __launch_bounds__(kThreads) void gather_copy_kernel(RankBufs chunks, size_t ngran,
                                                               uint4* __restrict__ out) {
    const size_t g = granule_id();
    if (g >= ngran) return;
    const int p = blockIdx.y;
    const u32x4_t v = reinterpret_cast<const u32x4_t*>(chunks.p[p])[g];
    __builtin_nontemporal_store(v, reinterpret_cast<u32x4_t*>(out) + (size_t)p * ngran + g);
}

hipError_t launch_dda_tree_ag(const RankBufs& chunks, int bf16, int nranks, size_t n, void* out,
                              hipStream_t stream) {
    const size_t esz = bf16 ? 2 : 4;
    const size_t ngran = n / nranks * esz / 16;
    return launch(gather_copy_kernel, grid_for(ngran, nranks), dim3(kThreads), 0, stream, chunks, ngran,
                  static_cast<uint4*>(out));
}

// ---------------------------------------------------------------------------
// all-to-all-v routing.  Row k with destination j goes to packed position
// offsets[j] + (number of rows before k with destination j): a stable,
// destination-major permutation.
//
// Workgroup w places the rows of its own tile [w*T, (w+1)*T) and needs, for
// that, the per-destination counts of all rows (for the offsets) and of the
// rows before its tile.  There is no scratch memory through which workgroups
// could share partial counts, so every workgroup counts the whole destination
// array itself: 4 bytes a row, re-read from L2, and a handful of VALU
// operations per row, against a placement pass that would otherwise run on
// one CU.  The number of workgroups is capped, which bounds the re-reading.
//   counting  a lane loads 4 rows with one 16-byte load, 8 or 16 sub-tiles
//             at a time; a row adds one to its destination's byte of a 64-bit
//             per-lane counter, folded into 32-bit counters before a byte can
//             overflow; then a workgroup-wide sum.
//   placing   one sub-tile (4 contiguous rows per lane) at a time: each lane
//             counts its rows per destination in eight 16-bit fields, an
//             exclusive scan over the lanes gives each row the number of
//             earlier rows of its destination in the sub-tile, and the
//             destination's running base (kept in every lane's registers)
//             adds the rest.  The first sub-tile is loaded and scanned
//             together with the counting, so a tile of one sub-tile needs a
//             single barrier.
// Rows with an out-of-range destination are dropped; the workgroups fill the
// part of perm past the last placed row with -1.
// ---------------------------------------------------------------------------

constexpr int kRouteRowsPerLane = 4;
constexpr size_t kRouteMaxGroups = 128;

// Workgroup size and counting depth.  256 lanes with 16 sub-tiles in flight
// measured fastest up to about 18K rows (4.5 us at 16,384); 512 lanes with 8
// from there on (64K rows 9.2 -> 7.8 us, 256K rows 28.3 -> 20.2 us): the
// counting, which every workgroup repeats over all rows, then runs on twice
// the wavefronts of a CU.
template <int THREADS, int UNROLL>
struct RouteCfg {
    static constexpr int kThreads = THREADS;
    static constexpr int kWaves = THREADS / 64;
    static constexpr int kUnroll = UNROLL;                                 // sub-tiles in flight while counting
    static constexpr size_t kSubTile = (size_t)THREADS * kRouteRowsPerLane;  // rows placed per step
};
using RouteSmall = RouteCfg<256, 16>;
using RouteLarge = RouteCfg<512, 8>;
constexpr size_t kRouteLargeFrom = 18432;  // rows

// Wavefront totals of 16 per-lane counters, transposed: lane l ends with the
// total of counter l & 15.  Four DPP steps (row mirror, half-row mirror,
// quad xor 2, quad xor 1) each pair a lane with one that holds the same
// counters; the lane keeps the half selected by one bit of its row position
// (a bit the two partners differ in) and adds the partner's copy of that half.
// After them each lane of a row holds one counter summed over the row, and two
// gfx950 lane swaps add lane l ^ 32, then lane l ^ 16.  About 50 VALU
// operations, against 16 separate reductions.  Needs all 64 lanes active.
__device__ __forceinline__ uint32_t wave_sums16(const uint32_t (&c)[16]) {
    const unsigned l = threadIdx.x & 15;
    uint32_t a[8], b[4], d[2];
#pragma unroll
    for (int j = 0; j < 8; ++j) {
        const bool hi = (l & 8) != 0;
        const int send = (int)(hi ? c[j] : c[j + 8]);
        a[j] = (hi ? c[j + 8] : c[j]) + (uint32_t)__builtin_amdgcn_update_dpp(0, send, 0x140, 0xF, 0xF, false);
    }
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        const bool hi = (l & 4) != 0;
        const int send = (int)(hi ? a[j] : a[j + 4]);
        b[j] = (hi ? a[j + 4] : a[j]) + (uint32_t)__builtin_amdgcn_update_dpp(0, send, 0x141, 0xF, 0xF, false);
    }
#pragma unroll
    for (int j = 0; j < 2; ++j) {
        const bool hi = (l & 2) != 0;
        const int send = (int)(hi ? b[j] : b[j + 2]);
        d[j] = (hi ? b[j + 2] : b[j]) + (uint32_t)__builtin_amdgcn_update_dpp(0, send, 0x4E, 0xF, 0xF, false);
    }
    const bool hi = (l & 1) != 0;
    const int send = (int)(hi ? d[0] : d[1]);
    uint32_t v = (hi ? d[1] : d[0]) + (uint32_t)__builtin_amdgcn_update_dpp(0, send, 0xB1, 0xF, 0xF, false);
    const auto h = __builtin_amdgcn_permlane32_swap(v, v, false, false);  // lanes l and l ^ 32
    v = h[0] + h[1];
    const auto q = __builtin_amdgcn_permlane16_swap(v, v, false, false);  // lanes l and l ^ 16
    return q[0] + q[1];
}

// Inclusive prefix sum over the lanes of the wavefront: row_shr 1, 2, 4, 8
// inside each 16-lane row (a lane with no source lane in its row adds 0), then
// row_bcast 15 (rows 1 and 3 add the last lane of the row below) and row_bcast
// 31 (rows 2 and 3 add lane 31).  Needs all 64 lanes active.
__device__ __forceinline__ uint32_t wave_scan(uint32_t v) {
    int x = (int)v;
    x += __builtin_amdgcn_update_dpp(0, x, 0x111, 0xF, 0xF, true);
    x += __builtin_amdgcn_update_dpp(0, x, 0x112, 0xF, 0xF, true);
    x += __builtin_amdgcn_update_dpp(0, x, 0x114, 0xF, 0xF, true);
    x += __builtin_amdgcn_update_dpp(0, x, 0x118, 0xF, 0xF, true);
    x += __builtin_amdgcn_update_dpp(0, x, 0x142, 0xA, 0xF, false);
    x += __builtin_amdgcn_update_dpp(0, x, 0x143, 0xC, 0xF, false);
    return (uint32_t)x;
}

// rows k .. k+3 of dest (k % 4 == 0), -1 for a row at or past `end`
__device__ __forceinline__ int4 load_raw4(const int32_t* __restrict__ dest, size_t end, size_t k) {
    int4 v = make_int4(-1, -1, -1, -1);
    if (k + 4 <= end) {
        v = *reinterpret_cast<const int4*>(dest + k);
    } else {
        if (k < end) v.x = dest[k];
        if (k + 1 < end) v.y = dest[k + 1];
        if (k + 2 < end) v.z = dest[k + 2];
    }
    return v;
}

// one in byte d of a 64-bit counter for a destination d in [0, nranks),
// nothing for any other value
__device__ __forceinline__ uint64_t dest_byte(int32_t d, int nranks) {
    return (uint64_t)((uint32_t)d < (uint32_t)nranks ? 1u : 0u) << ((d & 7) * 8);
}

// The count bytes of four rows.  When all four name a destination in 0..7
// (the usual case) each adds one at byte d with no test against nranks: a row
// naming a destination in nranks..7 then lands in a byte that the kernel
// clears after the reduction.  Otherwise every row is tested (dest_byte).
// This saves about two VALU operations a row.
__device__ __forceinline__ uint64_t row_bytes4(int4 v, int nranks) {
    if ((uint32_t)(v.x | v.y | v.z | v.w) < 8u)
        return (1ull << ((uint32_t)v.x << 3)) + (1ull << ((uint32_t)v.y << 3)) + (1ull << ((uint32_t)v.z << 3)) +
               (1ull << ((uint32_t)v.w << 3));
    return dest_byte(v.x, nranks) + dest_byte(v.y, nranks) + dest_byte(v.z, nranks) + dest_byte(v.w, nranks);
}

// One round of count_rows: kUnroll sub-tiles from row s0, all loads in
// flight.  A full round (every row in range) loads plainly and counts through
// row_bytes4; the last, partial round loads only the sub-tiles that hold rows
// (a uniform test), each through load_raw4 (rows past the end read as -1), and
// tests every row.
template <typename Cfg, bool kFull>
__device__ __forceinline__ void count_round(const int32_t* __restrict__ dest, size_t rows, int nranks,
                                            size_t split, size_t s0, uint32_t (&before)[kMaxRanks],
                                            uint32_t (&after)[kMaxRanks]) {
    const size_t lane = (size_t)kRouteRowsPerLane * threadIdx.x;
    int4 v[Cfg::kUnroll];
#pragma unroll
    for (int u = 0; u < Cfg::kUnroll; ++u) {
        const size_t s = s0 + u * Cfg::kSubTile;
        if (kFull)
            v[u] = *reinterpret_cast<const int4*>(dest + s + lane);
        else if (s < rows)
            v[u] = load_raw4(dest, rows, s + lane);
    }
    uint64_t lo = 0, hi = 0;  // at most 64 per byte
#pragma unroll
    for (int u = 0; u < Cfg::kUnroll; ++u) {
        const size_t s = s0 + u * Cfg::kSubTile;
        if (kFull || s < rows) {
            const uint64_t b = kFull ? row_bytes4(v[u], nranks)
                                     : dest_byte(v[u].x, nranks) + dest_byte(v[u].y, nranks) +
                                           dest_byte(v[u].z, nranks) + dest_byte(v[u].w, nranks);
            if (s < split)
                lo += b;
            else
                hi += b;
        }
    }
#pragma unroll
    for (int j = 0; j < kMaxRanks; ++j) {
        before[j] += (uint32_t)(lo >> (8 * j)) & 0xFFu;
        after[j] += (uint32_t)(hi >> (8 * j)) & 0xFFu;
    }
}

// This lane's per-destination counts of the rows before row `split` and of
// the rest (split a multiple of the sub-tile).  The lane reads rows
// 4*t + kSubTile*u of each round; a sub-tile lies wholly on one side of
// `split`.
template <typename Cfg>
__device__ __forceinline__ void count_rows(const int32_t* __restrict__ dest, size_t rows, int nranks,
                                           size_t split, uint32_t (&before)[kMaxRanks],
                                           uint32_t (&after)[kMaxRanks]) {
    constexpr size_t kRound = Cfg::kUnroll * Cfg::kSubTile;
    size_t s0 = 0;
    for (; s0 + kRound <= rows; s0 += kRound) count_round<Cfg, true>(dest, rows, nranks, split, s0, before, after);
    if (s0 < rows) count_round<Cfg, false>(dest, rows, nranks, split, s0, before, after);
}

// 16-bit field d & 7 of four packed registers (destinations 2r, 2r+1 in
// register r).  The registers are paired into 64-bit values before the
// select: a select between array elements would be folded into an indexed
// load, and the array moved out of registers.
__device__ __forceinline__ uint32_t field16(const uint32_t (&f)[4], int32_t d) {
    const uint64_t lo = ((uint64_t)f[1] << 32) | f[0], hi = ((uint64_t)f[3] << 32) | f[2];
    const uint64_t x = (d & 4) ? hi : lo;
    return (uint32_t)(x >> ((d & 3) * 16)) & 0xFFFFu;
}

// v[d & 7], selected the same way
__device__ __forceinline__ uint32_t pick8(const uint32_t (&v)[kMaxRanks], int32_t d) {
    const uint64_t p01 = ((uint64_t)v[1] << 32) | v[0], p23 = ((uint64_t)v[3] << 32) | v[2];
    const uint64_t p45 = ((uint64_t)v[5] << 32) | v[4], p67 = ((uint64_t)v[7] << 32) | v[6];
    const uint64_t x = (d & 4) ? ((d & 2) ? p67 : p45) : ((d & 2) ? p23 : p01);
    return (uint32_t)(x >> ((d & 1) * 32));
}

// The lane's per-destination row counts (at most 4 each) as eight 16-bit
// fields in four registers: destinations 2r and 2r+1 in register r.
__device__ __forceinline__ void lane_fields(const int32_t (&d)[kRouteRowsPerLane], int nranks, uint32_t (&own)[4]) {
    uint64_t bytes = 0;
#pragma unroll
    for (int i = 0; i < kRouteRowsPerLane; ++i) bytes += dest_byte(d[i], nranks);
    const uint32_t lo = (uint32_t)bytes, hi = (uint32_t)(bytes >> 32);
    own[0] = (lo & 0xFFu) | ((lo << 8) & 0xFF0000u);
    own[1] = ((lo >> 16) & 0xFFu) | ((lo >> 8) & 0xFF0000u);
    own[2] = (hi & 0xFFu) | ((hi << 8) & 0xFF0000u);
    own[3] = ((hi >> 16) & 0xFFu) | ((hi >> 8) & 0xFF0000u);
}

// Scatter this lane's rows k .. k+3 of a sub-tile.  excl: the fields of the
// rows of its destinations in earlier lanes of the sub-tile; base: each
// destination's packed position of the sub-tile's first such row.
__device__ __forceinline__ void place_rows(const int32_t (&d)[kRouteRowsPerLane], int nranks, size_t k,
                                           const uint32_t (&excl)[4], const uint32_t (&base)[kMaxRanks],
                                           int32_t* __restrict__ perm) {
    uint32_t pos[kRouteRowsPerLane];
#pragma unroll
    for (int i = 0; i < kRouteRowsPerLane; ++i) {
        uint32_t same = 0;  // earlier rows of this lane with the same destination
#pragma unroll
        for (int e = 0; e < i; ++e) same += d[e] == d[i] ? 1u : 0u;
        pos[i] = pick8(base, d[i]) + field16(excl, d[i]) + same;
    }
#pragma unroll
    for (int i = 0; i < kRouteRowsPerLane; ++i)
        if ((uint32_t)d[i] < (uint32_t)nranks) perm[pos[i]] = (int32_t)(k + i);
}

template <typename Cfg>
__global__ __launch_bounds__(Cfg::kThreads) void a2av_route_kernel(const int32_t* __restrict__ dest,
                                                                   size_t rows, int nranks, size_t tile,
                                                                   int32_t* __restrict__ counts,
                                                                   int32_t* __restrict__ offsets,
                                                                   int32_t* __restrict__ perm) {
    __shared__ uint32_t wave_part[Cfg::kWaves][2 * kMaxRanks];
    __shared__ uint32_t wave_tot[Cfg::kWaves][4];
    const int t = threadIdx.x;
    const int w = __builtin_amdgcn_readfirstlane(t >> 6);  // wavefront index, kept scalar
    const size_t ts = (size_t)blockIdx.x * tile;
    const size_t te = ts + tile < rows ? ts + tile : rows;

    // The first sub-tile of this workgroup's rows is loaded with the counting
    // loads and scanned with the counts, so that one barrier serves both.
    size_t k = ts + (size_t)kRouteRowsPerLane * t;
    const int4 first = load_raw4(dest, te, k);
    uint32_t before[kMaxRanks], after[kMaxRanks];
#pragma unroll
    for (int j = 0; j < kMaxRanks; ++j) before[j] = after[j] = 0;
    count_rows<Cfg>(dest, rows, nranks, ts, before, after);

    int32_t d[kRouteRowsPerLane] = {first.x, first.y, first.z, first.w};
    uint32_t own[4], excl[4];
    lane_fields(d, nranks, own);
#pragma unroll
    for (int r = 0; r < 4; ++r) {
        const uint32_t incl = wave_scan(own[r]);
        excl[r] = incl - own[r];
        if ((t & 63) == 63) wave_tot[w][r] = incl;
    }
    static_assert(2 * kMaxRanks == 16, "one counter per lane of a row");
    uint32_t cnt[2 * kMaxRanks];
#pragma unroll
    for (int j = 0; j < kMaxRanks; ++j) {
        cnt[j] = before[j];
        cnt[kMaxRanks + j] = after[j];
    }
    const uint32_t wave_cnt = wave_sums16(cnt);
    if ((t & 63) < 2 * kMaxRanks) wave_part[w][t & 63] = wave_cnt;
    __syncthreads();

    // every lane: totals, offsets and the bases of this tile's first
    // sub-tile (destinations at or past nranks count zero rows)
    uint32_t bef[kMaxRanks], tot[kMaxRanks];
#pragma unroll
    for (int j = 0; j < kMaxRanks; ++j) {
        bef[j] = tot[j] = 0;
#pragma unroll
        for (int v = 0; v < Cfg::kWaves; ++v) {
            bef[j] += wave_part[v][j];
            tot[j] += wave_part[v][kMaxRanks + j];
        }
        tot[j] += bef[j];
        if (j >= nranks) bef[j] = tot[j] = 0;  // rows row_bytes4 counted for no destination
    }
    uint32_t base[kMaxRanks], off[kMaxRanks], placed = 0;
#pragma unroll
    for (int j = 0; j < kMaxRanks; ++j) {
        off[j] = placed;
        base[j] = placed + bef[j];
        placed += tot[j];
    }
    if (blockIdx.x == 0 && t == 0) {
#pragma unroll
        for (int j = 0; j < kMaxRanks; ++j) {
            if (j < nranks) {
                counts[j] = (int32_t)tot[j];
                offsets[j] = (int32_t)off[j];
            }
        }
    }

    for (size_t s = ts;;) {
        uint32_t sub[4];  // the sub-tile's fields, all lanes
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            sub[r] = 0;
#pragma unroll
            for (int v = 0; v < Cfg::kWaves; ++v) {
                const uint32_t c = wave_tot[v][r];
                excl[r] += v < w ? c : 0u;
                sub[r] += c;
            }
        }
        place_rows(d, nranks, k, excl, base, perm);
        s += Cfg::kSubTile;
        if (s >= te) break;
#pragma unroll
        for (int j = 0; j < kMaxRanks; ++j) base[j] += field16(sub, j);
        // the next sub-tile (tiles of more than 1024 rows only)
        k = s + (size_t)kRouteRowsPerLane * t;
        const int4 next = load_raw4(dest, te, k);
        d[0] = next.x;
        d[1] = next.y;
        d[2] = next.z;
        d[3] = next.w;
        lane_fields(d, nranks, own);
        __syncthreads();  // every lane has read wave_tot
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const uint32_t incl = wave_scan(own[r]);
            excl[r] = incl - own[r];
            if ((t & 63) == 63) wave_tot[w][r] = incl;
        }
        __syncthreads();
    }

    // the tail of perm past the placed rows
    const size_t q0 = placed > ts ? placed : ts;
    for (size_t q = q0 + t; q < te; q += Cfg::kThreads) perm[q] = -1;
}

// Workgroups and tile size: one sub-tile per workgroup up to kRouteMaxGroups
// workgroups, larger tiles (whole sub-tiles) beyond.
template <typename Cfg>
static hipError_t launch_route(const int32_t* dest, size_t rows, int nranks, int32_t* counts, int32_t* offsets,
                               int32_t* perm, hipStream_t stream) {
    const size_t subtiles = (rows + Cfg::kSubTile - 1) / Cfg::kSubTile;
    const size_t g = subtiles < kRouteMaxGroups ? subtiles : kRouteMaxGroups;
    const size_t tile = (subtiles + g - 1) / g * Cfg::kSubTile;
    const size_t groups = (rows + tile - 1) / tile;
    return launch(a2av_route_kernel<Cfg>, dim3((unsigned)groups), dim3(Cfg::kThreads), 0, stream, dest, rows, nranks,
                  tile, counts, offsets, perm);
}

hipError_t launch_a2av_route(const int32_t* dest, size_t rows, int nranks, int32_t* counts, int32_t* offsets,
                             int32_t* perm, hipStream_t stream) {
    if (rows < kRouteLargeFrom) return launch_route<RouteSmall>(dest, rows, nranks, counts, offsets, perm, stream);
    return launch_route<RouteLarge>(dest, rows, nranks, counts, offsets, perm, stream);
}

// ---------------------------------------------------------------------------
// gather + quantize rows: granules over the packed (row, column) space, in
// XCD-aware tile order.  A granule never straddles a row (row_len % 128 ==
// 0); its source row is perm[packed row].  An invalid perm entry quantizes a
// zero row: scale +0, codes 0x00.  When row_len is a multiple of 1,024, every
// wavefront's 64 granules lie in one row and come in as one piece, with the
// quantizer's regrouped non-temporal loads (measured at 16,384 x 7168 bf16,
// cold HBM); otherwise each lane loads its own granule.
// ---------------------------------------------------------------------------

template <typename In, bool kWave>
__global__ __launch_bounds__(kThreads) void quantize_rows_kernel(const In* __restrict__ x, size_t rows,
                                                                 size_t row_len, const int32_t* __restrict__ perm,
                                                                 uint8_t* __restrict__ codes,
                                                                 float* __restrict__ scales) {
    float v[kGranule];
    if constexpr (kWave) {
        __shared__ __attribute__((aligned(16))) uint8_t lds[kThreads / 64][kWaveGranules * 16 * sizeof(In)];
        const uint32_t w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), l = threadIdx.x & 63;
        const size_t g0 = (xcd_tile() * (kThreads / 64) + w) * kWaveGranules;  // packed granule index
        const size_t e0 = g0 * kGranule;
        if (e0 >= rows * row_len) return;  // whole wavefronts (rows * row_len % 1024 == 0)
        const size_t k = e0 / row_len;     // one packed row for the whole wavefront
        const int32_t src = perm[k];
        if (src < 0 || (size_t)src >= rows) {
#pragma unroll
            for (int j = 0; j < kGranule; ++j) v[j] = 0.0f;
        } else {
            load_wave_granules(x + (size_t)src * row_len + (e0 - k * row_len), kWaveGranules, l, lds[w], v);
        }
        float sc;
        const uint4 c = quantize_granule(v, &sc);
        store_granule(c, sc, g0 + l, l, codes, scales);
    } else {
        const size_t g = xcd_tile() * kThreads + threadIdx.x;  // packed granule index
        const size_t e = g * kGranule;
        if (e >= rows * row_len) return;  // whole 8-lane blocks drop out together
        const size_t k = e / row_len;
        const size_t col = e - k * row_len;
        const int32_t src = perm[k];
        if (src < 0 || (size_t)src >= rows) {
#pragma unroll
            for (int j = 0; j < kGranule; ++j) v[j] = 0.0f;
        } else {
            load16(x + (size_t)src * row_len + col, v);
        }
        float sc;
        const uint4 c = quantize_granule(v, &sc);
        store_granule(c, sc, g, threadIdx.x, codes, scales);
    }
}

template <typename In>
static hipError_t launch_quantize_rows_t(const In* x, size_t rows, size_t row_len, const int32_t* perm,
                                         uint8_t* codes, float* scales, hipStream_t stream) {
    const size_t ngran = rows * row_len / kGranule;
    if (row_len % (kWaveGranules * kGranule) == 0) {
        const size_t waves = ngran / kWaveGranules;
        const dim3 grid((unsigned)((waves + kThreads / 64 - 1) / (kThreads / 64)));
        return launch(quantize_rows_kernel<In, true>, grid, dim3(kThreads), 0, stream, x, rows, row_len, perm, codes,
                      scales);
    }
    return launch(quantize_rows_kernel<In, false>, grid_for(ngran), dim3(kThreads), 0, stream, x, rows, row_len,
                  perm, codes, scales);
}

hipError_t launch_quantize_rows(const void* x, int in_bf16, size_t rows, size_t row_len, const int32_t* perm,
                                uint8_t* codes, float* scales, hipStream_t stream) {
    if (in_bf16)
        return launch_quantize_rows_t(static_cast<const uint16_t*>(x), rows, row_len, perm, codes, scales, stream);
    return launch_quantize_rows_t(static_cast<const float*>(x), rows, row_len, perm, codes, scales, stream);
}

// ---------------------------------------------------------------------------
// raw codec: 4 values per lane, element-wise tail
// ---------------------------------------------------------------------------

__global__ __launch_bounds__(kThreads) void encode_kernel(const float* __restrict__ x, size_t n,
                                                          uint8_t* __restrict__ codes) {
    const size_t g = granule_id();
    const size_t e = g * 4;
    if (e >= n) return;
    if (e + 4 <= n) {
        const float4 v = *reinterpret_cast<const float4*>(x + e);
        *reinterpret_cast<uint32_t*>(codes + e) = encode4(v.x, v.y, v.z, v.w);
    } else {
        for (size_t i = e; i < n; ++i)
            codes[i] = (uint8_t)(__builtin_amdgcn_cvt_pk_fp8_f32(clamp448(x[i]), 0.0f, 0, false) & 0xFF);
    }
}

hipError_t launch_encode(const float* x, size_t n, uint8_t* codes, hipStream_t stream) {
    const size_t ngran = (n + 3) / 4;
    return launch(encode_kernel, grid_for(ngran), dim3(kThreads), 0, stream, x, n, codes);
}

// ---------------------------------------------------------------------------
// All ranks in one launch (the emulated collectives on one GPU).  Each kernel
// below runs the per-rank kernel of the same step for every rank at once,
// with the rank taken from a grid dimension: every lane does exactly the
// arithmetic of the per-rank kernel on the same elements, so the results are
// those of N separate launches, bit for bit, at a third of the launches.
// ---------------------------------------------------------------------------

// quantize every rank's buffer: grid.y = rank; each wavefront as in quantize_kernel
template <typename In>
__global__ __launch_bounds__(kThreads) void quantize_ranks_kernel(RankBufs x, size_t ngran, RankQuant q) {
    __shared__ __attribute__((aligned(16))) uint8_t lds[kThreads / 64][kWaveGranules * 16 * sizeof(In)];
    const uint32_t w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), l = threadIdx.x & 63;
    const size_t g0 = (xcd_tile() * (kThreads / 64) + w) * kWaveGranules;
    if (g0 >= ngran) return;
    const uint32_t left = (uint32_t)(ngran - g0 < kWaveGranules ? ngran - g0 : kWaveGranules);
    const int r = blockIdx.y;
    float v[kGranule];
    load_wave_granules(static_cast<const In*>(x.p[r]) + g0 * kGranule, left, l, lds[w], v);
    if (l >= left) return;
    float sc;
    const uint4 c = quantize_granule(v, &sc);
    store_granule(c, sc, g0 + l, l, q.codes[r], q.scales[r]);
}

hipError_t launch_quantize_ranks(const RankBufs& x, int in_bf16, int nranks, size_t n, const RankQuant& q,
                                 hipStream_t stream) {
    const size_t ngran = n / kGranule;
    const size_t waves = (ngran + kWaveGranules - 1) / kWaveGranules;
    const dim3 grid((unsigned)((waves + kThreads / 64 - 1) / (kThreads / 64)), nranks);
    if (in_bf16)
        return launch(quantize_ranks_kernel<uint16_t>, grid, dim3(kThreads), 0, stream, x, ngran, q);
    return launch(quantize_ranks_kernel<float>, grid, dim3(kThreads), 0, stream, x, ngran, q);
}

// reduce-scatter step of every rank: grid.y = the rank owning the chunk
template <int N>
__global__ __launch_bounds__(kThreads) void reduce_scatter_ranks_kernel(RankCodes in, size_t C, RankQuant chunks) {
    constexpr int W = rs_width<kRequant>();
    const size_t i = lane_elem<W>();
    if (i >= C) return;
    const int r = blockIdx.y;
    float acc[W];
    rank_sum<N, W>(in, (size_t)r * C + i, acc);
    float s;
    const auto c = quantize_lane(acc, &s);
    store_codes<W>(chunks.codes[r] + i, c);
    if ((threadIdx.x & (kBlock / W - 1)) == 0) chunks.scales[r][i / kBlock] = s;
}

hipError_t launch_reduce_scatter_ranks(const RankCodes& in, int nranks, size_t n, const RankQuant& chunks,
                                       hipStream_t stream) {
    const size_t C = n / nranks;
    const dim3 grid = lane_grid<rs_width<kRequant>()>(C, nranks), block(kThreads);
    switch (nranks) {
#define LPC_RSR_CASE(NR) \
    case NR: return launch(reduce_scatter_ranks_kernel<NR>, grid, block, 0, stream, in, C, chunks);
        LPC_RSR_CASE(1) LPC_RSR_CASE(2) LPC_RSR_CASE(3) LPC_RSR_CASE(4)
        LPC_RSR_CASE(5) LPC_RSR_CASE(6) LPC_RSR_CASE(7) LPC_RSR_CASE(8)
#undef LPC_RSR_CASE
    }
    return hipErrorInvalidValue;
}

// all-gather dequantization into every rank's output: grid.y = chunk, grid.z = rank
template <typename Out>
__global__ __launch_bounds__(kThreads) void allgather_ranks_kernel(RankCodes chunks, size_t C, RankOut outs) {
    constexpr int W = lane_width<Out>();
    const size_t i = lane_elem<W>();
    if (i >= C) return;
    const int p = blockIdx.y, r = blockIdx.z;
    float d[W];
    // every chunk is read once per rank (grid.z): ordinary loads, so the reads after the first hit
    // the caches (non-temporal loads measured 26.9 against 22.6 us at N=8 x 16 MiB)
    dequant_lane(load_codes<W, false>(chunks.codes[p] + i), chunks.scales[p][i / kBlock], d);
    store_lane_nt(static_cast<Out*>(outs.p[r]) + (size_t)p * C + i, d);
}

hipError_t launch_allgather_ranks(const RankCodes& chunks, int nranks, size_t n, const RankOut& outs, int out_bf16,
                                  hipStream_t stream) {
    const size_t C = n / nranks;
    if (out_bf16) {
        dim3 grid = lane_grid<lane_width<uint16_t>()>(C, nranks);
        grid.z = nranks;
        return launch(allgather_ranks_kernel<uint16_t>, grid, dim3(kThreads), 0, stream, chunks, C, outs);
    }
    dim3 grid = lane_grid<lane_width<float>()>(C, nranks);
    grid.z = nranks;
    return launch(allgather_ranks_kernel<float>, grid, dim3(kThreads), 0, stream, chunks, C, outs);
}

// DDA flat reduce of every rank into its own output: grid.y = rank
template <int N>
__global__ __launch_bounds__(kDdaThreads) void dda_flat_ranks_kernel(RankBufs b, size_t n, RankOut outs) {
    const size_t e = ((size_t)blockIdx.x * kDdaThreads + threadIdx.x) * kDdaElems;
    if (e >= n) return;
    dda_flat_at<N>(b, n, e, static_cast<uint16_t*>(outs.p[blockIdx.y]));
}

hipError_t launch_dda_flat_ranks(const RankBufs& b, int nranks, size_t n, const RankOut& outs, hipStream_t stream) {
    const size_t lanes = (n + kDdaElems - 1) / kDdaElems;
    const dim3 grid((unsigned)((lanes + kDdaThreads - 1) / kDdaThreads), nranks), block(kDdaThreads);
    switch (nranks) {
#define LPC_DDAR_CASE(NR) \
    case NR: return launch(dda_flat_ranks_kernel<NR>, grid, block, 0, stream, b, n, outs);
        LPC_DDAR_CASE(1) LPC_DDAR_CASE(2) LPC_DDAR_CASE(3) LPC_DDAR_CASE(4)
        LPC_DDAR_CASE(5) LPC_DDAR_CASE(6) LPC_DDAR_CASE(7) LPC_DDAR_CASE(8)
#undef LPC_DDAR_CASE
    }
    return hipErrorInvalidValue;
}

// DDA tree reduce-scatter of every rank: grid.y = the rank owning the chunk
template <int N, bool BF16>
__global__ __launch_bounds__(kThreads) void dda_tree_rs_ranks_kernel(RankBufs b, size_t chunk_bytes, size_t ngran,
                                                                     RankOut chunks) {
    const size_t g = granule_id();
    if (g >= ngran) return;
    const int r = blockIdx.y;
    dda_tree_rs_at<N, BF16>(b, (size_t)r * chunk_bytes + g * 16, static_cast<uint4*>(chunks.p[r]) + g);
}

hipError_t launch_dda_tree_rs_ranks(const RankBufs& b, int bf16, int nranks, size_t n, const RankOut& chunks,
                                    hipStream_t stream) {
    const size_t chunk_bytes = n / nranks * (bf16 ? 2 : 4);
    const size_t ngran = chunk_bytes / 16;
    const dim3 grid = grid_for(ngran, nranks), block(kThreads);
    switch (nranks) {
#define LPC_TREER_CASE(NR)                                                                                   \
    case NR:                                                                                                 \
        if (bf16)                                                                                            \
            return launch(dda_tree_rs_ranks_kernel<NR, true>, grid, block, 0, stream, b, chunk_bytes, ngran, \
                          chunks);                                                                           \
        return launch(dda_tree_rs_ranks_kernel<NR, false>, grid, block, 0, stream, b, chunk_bytes, ngran, chunks);
        LPC_TREER_CASE(1) LPC_TREER_CASE(2) LPC_TREER_CASE(3) LPC_TREER_CASE(4)
        LPC_TREER_CASE(5) LPC_TREER_CASE(6) LPC_TREER_CASE(7) LPC_TREER_CASE(8)
#undef LPC_TREER_CASE
    }
    return hipErrorInvalidValue;
}

// DDA tree all-gather (a gather copy) into every rank's output: grid.y =
// chunk, grid.z = rank
__global__ __launch_bounds__(kThreads) void gather_copy_ranks_kernel(RankBufs chunks, size_t ngran, RankOut outs) {
    const size_t g = granule_id();
    if (g >= ngran) return;
    const int p = blockIdx.y;
    const u32x4_t v = reinterpret_cast<const u32x4_t*>(chunks.p[p])[g];
    __builtin_nontemporal_store(v, static_cast<u32x4_t*>(outs.p[blockIdx.z]) + (size_t)p * ngran + g);
}

// copy `bytes` (even) from src.p[r] to dst.p[r] for every rank r = grid.y:
// 16-byte granules, and granule `full` takes the tail two bytes at a time
__global__ __launch_bounds__(kThreads) void copy_ranks_kernel(RankBufs src, size_t bytes, RankOut dst) {
    const size_t g = granule_id();
    const size_t full = bytes / 16;
    const int r = blockIdx.y;
    if (g < full) {
        reinterpret_cast<u32x4_t*>(dst.p[r])[g] = reinterpret_cast<const u32x4_t*>(src.p[r])[g];
    } else if (g == full) {
        const uint16_t* s = static_cast<const uint16_t*>(src.p[r]);
        uint16_t* d = static_cast<uint16_t*>(dst.p[r]);
        for (size_t i = full * 8; i < bytes / 2; ++i) d[i] = s[i];
    }
}

hipError_t launch_copy_ranks(const RankBufs& src, int nranks, size_t bytes, const RankOut& dst, hipStream_t stream) {
    return launch(copy_ranks_kernel, grid_for(bytes / 16 + 1, nranks), dim3(kThreads), 0, stream, src, bytes, dst);
}

hipError_t launch_dda_tree_ag_ranks(const RankBufs& chunks, int bf16, int nranks, size_t n, const RankOut& outs,
                                    hipStream_t stream) {
    const size_t ngran = n / nranks * (bf16 ? 2 : 4) / 16;
    dim3 grid = grid_for(ngran, nranks);
    grid.z = nranks;
    return launch(gather_copy_ranks_kernel, grid, dim3(kThreads), 0, stream, chunks, ngran, outs);
}

}  // namespace lpc
