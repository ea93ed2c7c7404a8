// lpc_kernels.hip -- gfx950 kernels of the FP8 low-precision collective path
// and their launchers.  Arguments reaching these launchers have been checked
// by the C ABI layer (lpc_api.hip); nothing here validates again.
//
// The quantizers use one 16-element granule per lane (a wavefront covers 8
// scale blocks); the reduce-scatter, all-gather, fused and dequantize kernels
// give each lane a vector of 4 or 8 elements, so that every lane writes 16
// bytes (see lpc_device.hpp).  Streaming kernels use 256-lane workgroups.
// Rank loops are unrolled by template parameter so that all N loads of a lane
// are in flight before the first add.
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

// Every kernel of the library is launched through this helper.
template <typename K, typename... Args>
static void launch(K kernel, dim3 grid, dim3 block, uint32_t shmem, hipStream_t stream, Args... args) {
    hipLaunchKernelGGL(kernel, grid, block, shmem, stream, args...);
}

// ---------------------------------------------------------------------------
// (1) quantize
// ---------------------------------------------------------------------------

template <typename In>
__global__ __launch_bounds__(kThreads) void quantize_kernel(const In* __restrict__ x, size_t ngran,
                                                            uint8_t* __restrict__ codes,
                                                            float* __restrict__ scales) {
    const size_t g = xcd_tile() * kThreads + threadIdx.x;
    if (g >= ngran) return;  // whole 8-lane groups drop out together (n % 128 == 0)
    float v[kGranule];
    load16(x + g * kGranule, v);
    float s;
    const uint4 c = quantize_granule(v, &s);
    const u32x4_t cv = {c.x, c.y, c.z, c.w};
    __builtin_nontemporal_store(cv, reinterpret_cast<u32x4_t*>(codes + g * kGranule));
    if ((threadIdx.x & (kLanesPerBlock - 1)) == 0) scales[g / kLanesPerBlock] = s;
}

hipError_t launch_quantize(const void* x, int in_bf16, size_t n, uint8_t* codes, float* scales,
                           hipStream_t stream) {
    const size_t ngran = n / kGranule;
    if (in_bf16)
        launch(quantize_kernel<uint16_t>, grid_for(ngran), dim3(kThreads), 0, stream,
                           static_cast<const uint16_t*>(x), ngran, codes, scales);
    else
        launch(quantize_kernel<float>, grid_for(ngran), dim3(kThreads), 0, stream,
                           static_cast<const float*>(x), ngran, codes, scales);
    return hipGetLastError();
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
        c[p] = load_codes<W, false>(in.codes[p] + e);
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
static void launch_rs_n(const RankCodes& in, int nranks, size_t chunk_off, size_t C, uint8_t* cc, float* cs,
                        void* out, hipStream_t stream) {
    const dim3 grid = lane_grid<rs_width<Mode>()>(C), block(kThreads);
    switch (nranks) {
#define LPC_RS_CASE(NR)                                                                              \
    case NR:                                                                                         \
        launch((reduce_scatter_kernel<NR, Mode>), grid, block, 0, stream, in, chunk_off, C, cc, cs,  \
               out);                                                                                 \
        break;
        LPC_RS_CASE(1) LPC_RS_CASE(2) LPC_RS_CASE(3) LPC_RS_CASE(4)
        LPC_RS_CASE(5) LPC_RS_CASE(6) LPC_RS_CASE(7) LPC_RS_CASE(8)
#undef LPC_RS_CASE
    }
}

hipError_t launch_reduce_scatter_chunk(const RankCodes& in, int nranks, int rank, size_t n,
                                       uint8_t* cc, float* cs, hipStream_t stream) {
    const size_t C = n / nranks;
    launch_rs_n<kRequant>(in, nranks, (size_t)rank * C, C, cc, cs, nullptr, stream);
    return hipGetLastError();
}

hipError_t launch_reduce_scatter_out(const RankCodes& in, int nranks, int rank, size_t n, void* out,
                                     int out_bf16, hipStream_t stream) {
    const size_t C = n / nranks;
    if (out_bf16)
        launch_rs_n<kSumBF16>(in, nranks, (size_t)rank * C, C, nullptr, nullptr, out, stream);
    else
        launch_rs_n<kSumF32>(in, nranks, (size_t)rank * C, C, nullptr, nullptr, out, stream);
    return hipGetLastError();
}

// ---------------------------------------------------------------------------
// (3) all-gather dequantization (grid.y = chunk);  flat dequantization
// ---------------------------------------------------------------------------

template <typename Out>
__global__ __launch_bounds__(kThreads) void allgather_kernel(RankCodes chunks, size_t C,
                                                             Out* __restrict__ out) {
    constexpr int W = lane_width<Out>();
    const size_t i = lane_elem<W>();
    if (i >= C) return;
    const int p = blockIdx.y;
    float d[W];
    dequant_lane(load_codes<W, false>(chunks.codes[p] + i), chunks.scales[p][i / kBlock], d);
    store_lane_nt(out + (size_t)p * C + i, d);
}

hipError_t launch_allgather(const RankCodes& chunks, int nranks, size_t n, void* out, int out_bf16,
                            hipStream_t stream) {
    const size_t C = n / nranks;
    if (out_bf16)
        launch(allgather_kernel<uint16_t>, lane_grid<lane_width<uint16_t>()>(C, nranks), dim3(kThreads), 0,
               stream, chunks, C, static_cast<uint16_t*>(out));
    else
        launch(allgather_kernel<float>, lane_grid<lane_width<float>()>(C, nranks), dim3(kThreads), 0, stream,
               chunks, C, static_cast<float*>(out));
    return hipGetLastError();
}

template <typename Out>
__global__ __launch_bounds__(kThreads) void dequant_kernel(const uint8_t* __restrict__ codes,
                                                           const float* __restrict__ scales, size_t n,
                                                           Out* __restrict__ out) {
    constexpr int W = lane_width<Out>();
    const size_t i = lane_elem<W>();
    if (i >= n) return;
    float d[W];
    dequant_lane(load_codes<W, false>(codes + i), scales[i / kBlock], d);
    store_lane_nt(out + i, d);
}

hipError_t launch_dequant(const uint8_t* codes, const float* scales, size_t n, void* out, int out_bf16,
                          hipStream_t stream) {
    if (out_bf16)
        launch(dequant_kernel<uint16_t>, lane_grid<lane_width<uint16_t>()>(n), dim3(kThreads), 0, stream, codes,
               scales, n, static_cast<uint16_t*>(out));
    else
        launch(dequant_kernel<float>, lane_grid<lane_width<float>()>(n), dim3(kThreads), 0, stream, codes,
               scales, n, static_cast<float*>(out));
    return hipGetLastError();
}

// ---------------------------------------------------------------------------
// (2)+(3) fused.  Every lane owns the same position i of every chunk.  The
// peers' chunks are split into slices of two (peer q = rank + 1 .. rank + N - 1,
// mod N): grid.y == 0 reduces and requantizes the own chunk at i, writes its
// dequantization from registers, and dequantizes peers q = 1, 2 at i;
// grid.y == y > 0 dequantizes peers q = 2y + 1, 2y + 2.  Each lane issues all
// of its loads before its first conversion.  With bf16 output (W = 8) the
// code loads are non-temporal: 15 streams are read once each, and keeping
// them out of the caches measured faster at large sizes.
// ---------------------------------------------------------------------------

constexpr int kPeersPerSlice = 2;

__host__ __device__ constexpr int fused_slices(int N) {
    return N <= 1 ? 1 : (N - 1 + kPeersPerSlice - 1) / kPeersPerSlice;
}

template <int N, typename Out>
__global__ __launch_bounds__(kThreads) void rs_ag_fused_kernel(RankCodes in, RankCodes peers, int rank,
                                                               size_t C, uint8_t* __restrict__ cc,
                                                               float* __restrict__ cs,
                                                               Out* __restrict__ out) {
    constexpr int W = lane_width<Out>();
    constexpr bool kNtLoads = W == 8;
    using Codes = typename LaneCodes<W>::T;
    const size_t i = lane_elem<W>();
    if (i >= C) return;
    const int y = blockIdx.y;
    const int q_first = kPeersPerSlice * y + 1;
    Codes pc[kPeersPerSlice];
    float ps[kPeersPerSlice];
    int pp[kPeersPerSlice];
#pragma unroll
    for (int k = 0; k < kPeersPerSlice; ++k) {
        int p = rank + q_first + k;
        if (p >= N) p -= N;
        pp[k] = p;
    }
    float d[W];
    if (y == 0) {
        const size_t own = (size_t)rank * C + i;
        Codes c[N];
        float s[N];
#pragma unroll
        for (int p = 0; p < N; ++p) {
            c[p] = load_codes<W, kNtLoads>(in.codes[p] + own);
            s[p] = in.scales[p][own / kBlock];
        }
#pragma unroll
        for (int k = 0; k < kPeersPerSlice; ++k) {
            if (q_first + k < N) {
                pc[k] = load_codes<W, kNtLoads>(peers.codes[pp[k]] + i);
                ps[k] = peers.scales[pp[k]][i / kBlock];
            }
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
    } else {
#pragma unroll
        for (int k = 0; k < kPeersPerSlice; ++k) {
            if (q_first + k < N) {
                pc[k] = load_codes<W, kNtLoads>(peers.codes[pp[k]] + i);
                ps[k] = peers.scales[pp[k]][i / kBlock];
            }
        }
    }
#pragma unroll
    for (int k = 0; k < kPeersPerSlice; ++k) {
        if (q_first + k < N) {
            dequant_lane(pc[k], ps[k], d);
            store_lane_nt(out + (size_t)pp[k] * C + i, d);
        }
    }
}

hipError_t launch_rs_ag_fused(const RankCodes& in, const RankCodes& peers, int nranks, int rank, size_t n,
                              uint8_t* cc, float* cs, void* out, int out_bf16, hipStream_t stream) {
    const size_t C = n / nranks;
    const dim3 block(kThreads);
    const dim3 grid_f32 = lane_grid<lane_width<float>()>(C, fused_slices(nranks));
    const dim3 grid_bf16 = lane_grid<lane_width<uint16_t>()>(C, fused_slices(nranks));
    switch (nranks) {
#define LPC_FUSED_CASE(NR)                                                                           \
    case NR:                                                                                         \
        if (out_bf16)                                                                                \
            launch((rs_ag_fused_kernel<NR, uint16_t>), grid_bf16, block, 0, stream, in, peers, rank, \
                   C, cc, cs, static_cast<uint16_t*>(out));                                          \
        else                                                                                         \
            launch((rs_ag_fused_kernel<NR, float>), grid_f32, block, 0, stream, in, peers, rank, C,  \
                   cc, cs, static_cast<float*>(out));                                                \
        break;
        LPC_FUSED_CASE(1) LPC_FUSED_CASE(2) LPC_FUSED_CASE(3) LPC_FUSED_CASE(4)
        LPC_FUSED_CASE(5) LPC_FUSED_CASE(6) LPC_FUSED_CASE(7) LPC_FUSED_CASE(8)
#undef LPC_FUSED_CASE
    }
    return hipGetLastError();
}

// ---------------------------------------------------------------------------
// DDA flat: N bf16 buffers -> FP32 rank-order sum -> bf16.  Small messages
// are latency-bound, so the launch spreads them thin: one lane owns 4 bf16
// (one 8-byte load per rank), 64-lane workgroups; the last partial quad goes
// element by element.
// ---------------------------------------------------------------------------

constexpr int kDdaThreads = 64;
constexpr int kDdaElems = 4;

template <int N>
__global__ __launch_bounds__(kDdaThreads) void dda_flat_kernel(RankBufs b, size_t n,
                                                               uint16_t* __restrict__ out) {
    const size_t e = ((size_t)blockIdx.x * kDdaThreads + threadIdx.x) * kDdaElems;
    if (e >= n) return;
    if (e + kDdaElems <= n) {
        uint2 v[N];
#pragma unroll
        for (int p = 0; p < N; ++p) v[p] = *reinterpret_cast<const uint2*>(static_cast<const uint16_t*>(b.p[p]) + e);
        float acc[kDdaElems] = {bf16lo(v[0].x), bf16hi(v[0].x), bf16lo(v[0].y), bf16hi(v[0].y)};
#pragma unroll
        for (int p = 1; p < N; ++p) {
            acc[0] = acc[0] + bf16lo(v[p].x);
            acc[1] = acc[1] + bf16hi(v[p].x);
            acc[2] = acc[2] + bf16lo(v[p].y);
            acc[3] = acc[3] + bf16hi(v[p].y);
        }
        *reinterpret_cast<uint2*>(out + e) = make_uint2(pack_bf16x2(acc[0], acc[1]), pack_bf16x2(acc[2], acc[3]));
    } else {
        for (size_t i = e; i < n; ++i) {
            float acc = __uint_as_float((uint32_t)static_cast<const uint16_t*>(b.p[0])[i] << 16);
#pragma unroll
            for (int p = 1; p < N; ++p)
                acc = acc + __uint_as_float((uint32_t)static_cast<const uint16_t*>(b.p[p])[i] << 16);
            const __bf16 h = (__bf16)acc;
            out[i] = __builtin_bit_cast(uint16_t, h);
        }
    }
}

hipError_t launch_dda_flat(const RankBufs& b, int nranks, size_t n, void* out, hipStream_t stream) {
    const size_t lanes = (n + kDdaElems - 1) / kDdaElems;
    const dim3 grid((unsigned)((lanes + kDdaThreads - 1) / kDdaThreads)), block(kDdaThreads);
    uint16_t* o = static_cast<uint16_t*>(out);
    switch (nranks) {
#define LPC_DDA_CASE(NR)                                                                 \
    case NR:                                                                             \
        launch((dda_flat_kernel<NR>), grid, block, 0, stream, b, n, o);      \
        break;
        LPC_DDA_CASE(1) LPC_DDA_CASE(2) LPC_DDA_CASE(3) LPC_DDA_CASE(4)
        LPC_DDA_CASE(5) LPC_DDA_CASE(6) LPC_DDA_CASE(7) LPC_DDA_CASE(8)
#undef LPC_DDA_CASE
    }
    return hipGetLastError();
}

// ---------------------------------------------------------------------------
// DDA tree (unquantized): reduce-scatter of one chunk, and the gather copy.
// Granule = 16 bytes (4 fp32 or 8 bf16).
// ---------------------------------------------------------------------------

template <int N, bool BF16>
__global__ __launch_bounds__(kThreads) void dda_tree_rs_kernel(RankBufs b, size_t chunk_off_bytes,
                                                               size_t ngran, void* __restrict__ out) {
    const size_t g = granule_id();
    if (g >= ngran) return;
    uint4 v[N];
#pragma unroll
    for (int p = 0; p < N; ++p)
        v[p] = *reinterpret_cast<const uint4*>(static_cast<const uint8_t*>(b.p[p]) + chunk_off_bytes + g * 16);
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
        reinterpret_cast<uint4*>(out)[g] =
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
        reinterpret_cast<float4*>(out)[g] = acc;
    }
}

hipError_t launch_dda_tree_rs(const RankBufs& b, int bf16, int nranks, int rank, size_t n, void* out,
                              hipStream_t stream) {
    const size_t esz = bf16 ? 2 : 4;
    const size_t chunk_bytes = n / nranks * esz;
    const size_t ngran = chunk_bytes / 16;
    const size_t off = (size_t)rank * chunk_bytes;
    const dim3 grid = grid_for(ngran), block(kThreads);
    switch (nranks) {
#define LPC_TREE_CASE(NR)                                                                              \
    case NR:                                                                                           \
        if (bf16)                                                                                      \
            launch((dda_tree_rs_kernel<NR, true>), grid, block, 0, stream, b, off, ngran, out); \
        else                                                                                           \
            launch((dda_tree_rs_kernel<NR, false>), grid, block, 0, stream, b, off, ngran, out); \
        break;
        LPC_TREE_CASE(1) LPC_TREE_CASE(2) LPC_TREE_CASE(3) LPC_TREE_CASE(4)
        LPC_TREE_CASE(5) LPC_TREE_CASE(6) LPC_TREE_CASE(7) LPC_TREE_CASE(8)
#undef LPC_TREE_CASE
    }
    return hipGetLastError();
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
    launch(gather_copy_kernel, grid_for(ngran, nranks), dim3(kThreads), 0, stream, chunks,
                       ngran, static_cast<uint4*>(out));
    return hipGetLastError();
}

// ---------------------------------------------------------------------------
// all-to-all-v routing: one workgroup of 1024 lanes (16 wavefronts).  Rows are
// taken in super-tiles of 16 x 1024: lane t holds rows st + b*1024 + t,
// b = 0..15, in registers (one batch of loads, then no global reads), so a
// super-tile costs one load latency.
//   pass 1: per-destination counts, from wavefront ballots; counts, and
//           offsets as their exclusive prefix.
//   pass 2: for each super-tile, the ballots give every row its rank among
//           the earlier lanes of its wavefront with the same destination, and
//           every (b, wavefront) its count per destination; an exclusive
//           prefix over (b, wavefront) in row order, started at the
//           destination's running base, places each row: a stable,
//           destination-major permutation.
// ---------------------------------------------------------------------------

constexpr int kRouteThreads = 1024;
constexpr int kRouteWaves = kRouteThreads / 64;
constexpr int kRouteBatch = 16;
constexpr size_t kRouteSuperTile = (size_t)kRouteBatch * kRouteThreads;

// number of lanes below this one whose bit is set in mask
__device__ __forceinline__ int lanes_below(uint64_t mask) {
    return (int)__builtin_amdgcn_mbcnt_hi((uint32_t)(mask >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)mask, 0u));
}

__device__ __forceinline__ void load_route_batch(const int32_t* __restrict__ dest, size_t rows, size_t st,
                                                 int nranks, int32_t (&d)[kRouteBatch]) {
#pragma unroll
    for (int b = 0; b < kRouteBatch; ++b) {
        const size_t k = st + (size_t)b * kRouteThreads + threadIdx.x;
        const int32_t v = k < rows ? dest[k] : -1;
        d[b] = (v >= 0 && v < nranks) ? v : -1;  // out-of-range destinations are dropped
    }
}

__global__ __launch_bounds__(kRouteThreads) void a2av_route_kernel(const int32_t* __restrict__ dest,
                                                                   size_t rows, int nranks,
                                                                   int32_t* __restrict__ counts,
                                                                   int32_t* __restrict__ offsets,
                                                                   int32_t* __restrict__ perm) {
    __shared__ int32_t wave_cnt[kRouteBatch][kRouteWaves][kMaxRanks];  // then the in-batch prefix
    __shared__ int32_t batch_base[kRouteBatch][kMaxRanks];
    __shared__ int32_t base[kMaxRanks];
    __shared__ int32_t placed;
    const int t = threadIdx.x, lane = t & 63, w = t >> 6;
    int32_t d[kRouteBatch];

    // pass 1: counts
    int32_t cnt[kMaxRanks];
#pragma unroll
    for (int j = 0; j < kMaxRanks; ++j) cnt[j] = 0;
    for (size_t st = 0; st < rows; st += kRouteSuperTile) {
        load_route_batch(dest, rows, st, nranks, d);
#pragma unroll
        for (int b = 0; b < kRouteBatch; ++b)
#pragma unroll
            for (int j = 0; j < kMaxRanks; ++j) cnt[j] += __popcll(__ballot(d[b] == j));
    }
    if (lane == 0) {
#pragma unroll
        for (int j = 0; j < kMaxRanks; ++j) wave_cnt[0][w][j] = cnt[j];
    }
    __syncthreads();
    if (t == 0) {
        int32_t acc = 0;
        for (int j = 0; j < kMaxRanks; ++j) {
            int32_t c = 0;
            for (int v = 0; v < kRouteWaves; ++v) c += wave_cnt[0][v][j];
            base[j] = acc;
            if (j < nranks) {
                counts[j] = c;
                offsets[j] = acc;
                acc += c;
            }
        }
        placed = acc;
    }
    __syncthreads();

    // pass 2: stable scatter, one super-tile at a time
    for (size_t st = 0; st < rows; st += kRouteSuperTile) {
        load_route_batch(dest, rows, st, nranks, d);
        int32_t rank_in_wave[kRouteBatch];
#pragma unroll
        for (int b = 0; b < kRouteBatch; ++b) {
            rank_in_wave[b] = 0;
#pragma unroll
            for (int j = 0; j < kMaxRanks; ++j) {
                const uint64_t m = __ballot(d[b] == j);
                if (d[b] == j) rank_in_wave[b] = lanes_below(m);
                if (lane == 0) wave_cnt[b][w][j] = __popcll(m);
            }
        }
        __syncthreads();
        if (t < kRouteBatch * kMaxRanks) {  // (b, j): exclusive prefix over the wavefronts of batch b
            const int b = t / kMaxRanks, j = t % kMaxRanks;
            int32_t run = 0;
            for (int v = 0; v < kRouteWaves; ++v) {
                const int32_t c = wave_cnt[b][v][j];
                wave_cnt[b][v][j] = run;
                run += c;
            }
            batch_base[b][j] = run;
        }
        __syncthreads();
        if (t < kMaxRanks) {  // j: exclusive prefix over the batches, from the running base
            int32_t run = base[t];
            for (int b = 0; b < kRouteBatch; ++b) {
                const int32_t c = batch_base[b][t];
                batch_base[b][t] = run;
                run += c;
            }
            base[t] = run;
        }
        __syncthreads();
#pragma unroll
        for (int b = 0; b < kRouteBatch; ++b) {
            if (d[b] >= 0) {
                const size_t k = st + (size_t)b * kRouteThreads + t;
                perm[batch_base[b][d[b]] + wave_cnt[b][w][d[b]] + rank_in_wave[b]] = (int32_t)k;
            }
        }
        __syncthreads();  // the next super-tile rewrites wave_cnt and batch_base
    }
    // rows with an out-of-range destination were dropped: mark perm's tail
    for (size_t k = (size_t)placed + t; k < rows; k += kRouteThreads) perm[k] = -1;
}

hipError_t launch_a2av_route(const int32_t* dest, size_t rows, int nranks, int32_t* counts, int32_t* offsets,
                             int32_t* perm, hipStream_t stream) {
    launch(a2av_route_kernel, dim3(1), dim3(kRouteThreads), 0, stream, dest, rows, nranks, counts,
           offsets, perm);
    return hipGetLastError();
}

// ---------------------------------------------------------------------------
// gather + quantize rows: flat granules over the packed (row, column) space,
// in XCD-aware tile order.  A granule never straddles a row (row_len % 128 ==
// 0); its source row is perm[packed row].  An invalid perm entry quantizes a
// zero row: scale +0, codes 0x00.
// ---------------------------------------------------------------------------

template <typename In>
__global__ __launch_bounds__(kThreads) void quantize_rows_kernel(const In* __restrict__ x, size_t rows,
                                                                 size_t row_len, const int32_t* __restrict__ perm,
                                                                 uint8_t* __restrict__ codes,
                                                                 float* __restrict__ scales) {
    const size_t g = xcd_tile() * kThreads + threadIdx.x;  // packed granule index
    const size_t e = g * kGranule;
    if (e >= rows * row_len) return;  // whole 8-lane blocks drop out together
    const size_t k = e / row_len;
    const size_t col = e - k * row_len;
    const int32_t src = perm[k];
    float v[kGranule];
    if (src < 0 || (size_t)src >= rows) {
#pragma unroll
        for (int j = 0; j < kGranule; ++j) v[j] = 0.0f;
    } else {
        load16(x + (size_t)src * row_len + col, v);
    }
    float s;
    const uint4 c = quantize_granule(v, &s);
    const u32x4_t cv = {c.x, c.y, c.z, c.w};
    __builtin_nontemporal_store(cv, reinterpret_cast<u32x4_t*>(codes + e));
    if ((threadIdx.x & (kLanesPerBlock - 1)) == 0) scales[g / kLanesPerBlock] = s;
}

hipError_t launch_quantize_rows(const void* x, int in_bf16, size_t rows, size_t row_len, const int32_t* perm,
                                uint8_t* codes, float* scales, hipStream_t stream) {
    const dim3 grid = grid_for(rows * row_len / kGranule), block(kThreads);
    if (in_bf16)
        launch(quantize_rows_kernel<uint16_t>, grid, block, 0, stream, static_cast<const uint16_t*>(x), rows,
               row_len, perm, codes, scales);
    else
        launch(quantize_rows_kernel<float>, grid, block, 0, stream, static_cast<const float*>(x), rows, row_len,
               perm, codes, scales);
    return hipGetLastError();
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
    launch(encode_kernel, grid_for(ngran), dim3(kThreads), 0, stream, x, n, codes);
    return hipGetLastError();
}

}  // namespace lpc
