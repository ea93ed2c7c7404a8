// lpc_kernels.hip -- gfx950 kernels of the FP8 low-precision collective path
// and their launchers.  Arguments reaching these launchers have been checked
// by the C ABI layer (lpc_api.hip); nothing here validates again.
//
// All streaming kernels use 256-lane workgroups and one 16-element granule
// per lane (see lpc_device.hpp), so a wavefront covers 8 scale blocks and a
// workgroup 4096 elements.  Rank loops are unrolled by template parameter so
// that all N loads of a lane are in flight before the first add.
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

// ---------------------------------------------------------------------------
// (1) quantize
// ---------------------------------------------------------------------------

template <typename In>
__global__ __launch_bounds__(kThreads) void quantize_kernel(const In* __restrict__ x, size_t ngran,
                                                            uint8_t* __restrict__ codes,
                                                            float* __restrict__ scales) {
    const size_t g = granule_id();
    if (g >= ngran) return;  // whole 8-lane groups drop out together (n % 128 == 0)
    float v[kGranule];
    load16(x + g * kGranule, v);
    float s;
    const uint4 c = quantize_granule(v, &s);
    *reinterpret_cast<uint4*>(codes + g * kGranule) = c;
    if ((threadIdx.x & (kLanesPerBlock - 1)) == 0) scales[g / kLanesPerBlock] = s;
}

hipError_t launch_quantize(const void* x, int in_bf16, size_t n, uint8_t* codes, float* scales,
                           hipStream_t stream) {
    const size_t ngran = n / kGranule;
    if (in_bf16)
        hipLaunchKernelGGL(quantize_kernel<uint16_t>, grid_for(ngran), dim3(kThreads), 0, stream,
                           static_cast<const uint16_t*>(x), ngran, codes, scales);
    else
        hipLaunchKernelGGL(quantize_kernel<float>, grid_for(ngran), dim3(kThreads), 0, stream,
                           static_cast<const float*>(x), ngran, codes, scales);
    return hipGetLastError();
}

// ---------------------------------------------------------------------------
// (2) reduce-scatter step: N-way dequant + rank-order FP32 sum of one chunk
// ---------------------------------------------------------------------------

// Sum of the granule at element offset `e` (rank-buffer index) over N ranks.
template <int N>
__device__ __forceinline__ void rank_sum16(const RankCodes& in, size_t e, float (&acc)[kGranule]) {
    uint4 c[N];
    float s[N];
#pragma unroll
    for (int p = 0; p < N; ++p) {
        c[p] = *reinterpret_cast<const uint4*>(in.codes[p] + e);
        s[p] = in.scales[p][e / kBlock];
    }
    dequant16(c[0], s[0], acc);
#pragma unroll
    for (int p = 1; p < N; ++p) {
        float d[kGranule];
        dequant16(c[p], s[p], d);
#pragma unroll
        for (int j = 0; j < kGranule; ++j) acc[j] = acc[j] + d[j];
    }
}

enum RsOut { kRequant = 0, kSumF32 = 1, kSumBF16 = 2 };

template <int N, int Mode>
__global__ __launch_bounds__(kThreads) void reduce_scatter_kernel(RankCodes in, size_t chunk_off,
                                                                  size_t cgran,
                                                                  uint8_t* __restrict__ cc,
                                                                  float* __restrict__ cs,
                                                                  void* __restrict__ out) {
    const size_t g = granule_id();
    if (g >= cgran) return;
    float acc[kGranule];
    rank_sum16<N>(in, chunk_off + g * kGranule, acc);
    if (Mode == kRequant) {
        float s;
        const uint4 c = quantize_granule(acc, &s);
        *reinterpret_cast<uint4*>(cc + g * kGranule) = c;
        if ((threadIdx.x & (kLanesPerBlock - 1)) == 0) cs[g / kLanesPerBlock] = s;
    } else if (Mode == kSumF32) {
        store16(static_cast<float*>(out) + g * kGranule, acc);
    } else {
        store16(static_cast<uint16_t*>(out) + g * kGranule, acc);
    }
}

template <int Mode>
static void launch_rs_n(const RankCodes& in, int nranks, size_t chunk_off, size_t cgran, uint8_t* cc,
                        float* cs, void* out, hipStream_t stream) {
    const dim3 grid = grid_for(cgran), block(kThreads);
    switch (nranks) {
#define LPC_RS_CASE(NR)                                                                              \
    case NR:                                                                                         \
        hipLaunchKernelGGL((reduce_scatter_kernel<NR, Mode>), grid, block, 0, stream, in, chunk_off, \
                           cgran, cc, cs, out);                                                      \
        break;
        LPC_RS_CASE(1) LPC_RS_CASE(2) LPC_RS_CASE(3) LPC_RS_CASE(4)
        LPC_RS_CASE(5) LPC_RS_CASE(6) LPC_RS_CASE(7) LPC_RS_CASE(8)
#undef LPC_RS_CASE
    }
}

hipError_t launch_reduce_scatter_chunk(const RankCodes& in, int nranks, int rank, size_t n,
                                       uint8_t* cc, float* cs, hipStream_t stream) {
    const size_t C = n / nranks;
    launch_rs_n<kRequant>(in, nranks, (size_t)rank * C, C / kGranule, cc, cs, nullptr, stream);
    return hipGetLastError();
}

hipError_t launch_reduce_scatter_out(const RankCodes& in, int nranks, int rank, size_t n, void* out,
                                     int out_bf16, hipStream_t stream) {
    const size_t C = n / nranks;
    if (out_bf16)
        launch_rs_n<kSumBF16>(in, nranks, (size_t)rank * C, C / kGranule, nullptr, nullptr, out, stream);
    else
        launch_rs_n<kSumF32>(in, nranks, (size_t)rank * C, C / kGranule, nullptr, nullptr, out, stream);
    return hipGetLastError();
}

// ---------------------------------------------------------------------------
// (3) all-gather dequantization;  flat dequantization
// ---------------------------------------------------------------------------

template <typename Out>
__device__ __forceinline__ void dequant_granule_to(const uint8_t* __restrict__ codes,
                                                   const float* __restrict__ scales, size_t g,
                                                   Out* __restrict__ out) {
    const uint4 c = *reinterpret_cast<const uint4*>(codes + g * kGranule);
    const float s = scales[g / kLanesPerBlock];
    float d[kGranule];
    dequant16(c, s, d);
    store16(out + g * kGranule, d);
}

// grid.y = chunk p; out chunk p at p*C
template <typename Out>
__global__ __launch_bounds__(kThreads) void allgather_kernel(RankCodes chunks, size_t cgran,
                                                             Out* __restrict__ out) {
    const size_t g = granule_id();
    if (g >= cgran) return;
    const int p = blockIdx.y;
    dequant_granule_to(chunks.codes[p], chunks.scales[p], g, out + (size_t)p * cgran * kGranule);
}

hipError_t launch_allgather(const RankCodes& chunks, int nranks, size_t n, void* out, int out_bf16,
                            hipStream_t stream) {
    const size_t cgran = n / nranks / kGranule;
    if (out_bf16)
        hipLaunchKernelGGL(allgather_kernel<uint16_t>, grid_for(cgran, nranks), dim3(kThreads), 0,
                           stream, chunks, cgran, static_cast<uint16_t*>(out));
    else
        hipLaunchKernelGGL(allgather_kernel<float>, grid_for(cgran, nranks), dim3(kThreads), 0,
                           stream, chunks, cgran, static_cast<float*>(out));
    return hipGetLastError();
}

template <typename Out>
__global__ __launch_bounds__(kThreads) void dequant_kernel(const uint8_t* __restrict__ codes,
                                                           const float* __restrict__ scales,
                                                           size_t ngran, Out* __restrict__ out) {
    const size_t g = granule_id();
    if (g >= ngran) return;
    dequant_granule_to(codes, scales, g, out);
}

hipError_t launch_dequant(const uint8_t* codes, const float* scales, size_t n, void* out, int out_bf16,
                          hipStream_t stream) {
    const size_t ngran = n / kGranule;
    if (out_bf16)
        hipLaunchKernelGGL(dequant_kernel<uint16_t>, grid_for(ngran), dim3(kThreads), 0, stream, codes,
                           scales, ngran, static_cast<uint16_t*>(out));
    else
        hipLaunchKernelGGL(dequant_kernel<float>, grid_for(ngran), dim3(kThreads), 0, stream, codes,
                           scales, ngran, static_cast<float*>(out));
    return hipGetLastError();
}

// ---------------------------------------------------------------------------
// (2)+(3) fused: grid.y == 0 reduces and requantizes the own chunk and writes
// its dequantization from registers; grid.y = q > 0 dequantizes peer chunk
// (rank + q) % N.  The own-chunk row is dispatched first.
// ---------------------------------------------------------------------------

template <int N, typename Out>
__global__ __launch_bounds__(kThreads) void rs_ag_fused_kernel(RankCodes in, RankCodes peers, int rank,
                                                               size_t cgran, uint8_t* __restrict__ cc,
                                                               float* __restrict__ cs,
                                                               Out* __restrict__ out) {
    const size_t g = granule_id();
    if (g >= cgran) return;
    const size_t C = cgran * kGranule;
    float d[kGranule];
    size_t out_off;
    if (blockIdx.y == 0) {
        const size_t chunk_off = (size_t)rank * C;
        float acc[kGranule];
        rank_sum16<N>(in, chunk_off + g * kGranule, acc);
        float s;
        const uint4 c = quantize_granule(acc, &s);
        *reinterpret_cast<uint4*>(cc + g * kGranule) = c;
        if ((threadIdx.x & (kLanesPerBlock - 1)) == 0) cs[g / kLanesPerBlock] = s;
        dequant16(c, s, d);  // own chunk straight from registers
        out_off = chunk_off + g * kGranule;
    } else {
        int p = rank + (int)blockIdx.y;
        if (p >= N) p -= N;
        const uint4 c = *reinterpret_cast<const uint4*>(peers.codes[p] + g * kGranule);
        dequant16(c, peers.scales[p][g / kLanesPerBlock], d);
        out_off = (size_t)p * C + g * kGranule;
    }
    store16(out + out_off, d);
}

hipError_t launch_rs_ag_fused(const RankCodes& in, const RankCodes& peers, int nranks, int rank, size_t n,
                              uint8_t* cc, float* cs, void* out, int out_bf16, hipStream_t stream) {
    const size_t cgran = n / nranks / kGranule;
    const dim3 grid = grid_for(cgran, nranks), block(kThreads);
    switch (nranks) {
#define LPC_FUSED_CASE(NR)                                                                           \
    case NR:                                                                                         \
        if (out_bf16)                                                                                \
            hipLaunchKernelGGL((rs_ag_fused_kernel<NR, uint16_t>), grid, block, 0, stream, in, peers, \
                               rank, cgran, cc, cs, static_cast<uint16_t*>(out));                    \
        else                                                                                         \
            hipLaunchKernelGGL((rs_ag_fused_kernel<NR, float>), grid, block, 0, stream, in, peers,    \
                               rank, cgran, cc, cs, static_cast<float*>(out));                       \
        break;
        LPC_FUSED_CASE(1) LPC_FUSED_CASE(2) LPC_FUSED_CASE(3) LPC_FUSED_CASE(4)
        LPC_FUSED_CASE(5) LPC_FUSED_CASE(6) LPC_FUSED_CASE(7) LPC_FUSED_CASE(8)
#undef LPC_FUSED_CASE
    }
    return hipGetLastError();
}

// ---------------------------------------------------------------------------
// DDA flat: N bf16 buffers -> FP32 rank-order sum -> bf16.  One lane owns 8
// bf16 (one 16-byte load per rank); the last partial granule goes element by
// element.
// ---------------------------------------------------------------------------

template <int N>
__global__ __launch_bounds__(kThreads) void dda_flat_kernel(RankBufs b, size_t n,
                                                            uint16_t* __restrict__ out) {
    const size_t g = granule_id();
    const size_t e = g * 8;
    if (e >= n) return;
    if (e + 8 <= n) {
        uint4 v[N];
#pragma unroll
        for (int p = 0; p < N; ++p) v[p] = *reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(b.p[p]) + e);
        float acc[8];
        {
            const uint32_t w[4] = {v[0].x, v[0].y, v[0].z, v[0].w};
#pragma unroll
            for (int k = 0; k < 4; ++k) {
                acc[2 * k] = bf16lo(w[k]);
                acc[2 * k + 1] = bf16hi(w[k]);
            }
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
        *reinterpret_cast<uint4*>(out + e) =
            make_uint4(pack_bf16x2(acc[0], acc[1]), pack_bf16x2(acc[2], acc[3]), pack_bf16x2(acc[4], acc[5]),
                       pack_bf16x2(acc[6], acc[7]));
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
    const size_t ngran = (n + 7) / 8;
    const dim3 grid = grid_for(ngran), block(kThreads);
    uint16_t* o = static_cast<uint16_t*>(out);
    switch (nranks) {
#define LPC_DDA_CASE(NR)                                                                 \
    case NR:                                                                             \
        hipLaunchKernelGGL((dda_flat_kernel<NR>), grid, block, 0, stream, b, n, o);      \
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
            hipLaunchKernelGGL((dda_tree_rs_kernel<NR, true>), grid, block, 0, stream, b, off, ngran, out); \
        else                                                                                           \
            hipLaunchKernelGGL((dda_tree_rs_kernel<NR, false>), grid, block, 0, stream, b, off, ngran, out); \
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
    out[(size_t)p * ngran + g] = reinterpret_cast<const uint4*>(chunks.p[p])[g];
}

hipError_t launch_dda_tree_ag(const RankBufs& chunks, int bf16, int nranks, size_t n, void* out,
                              hipStream_t stream) {
    const size_t esz = bf16 ? 2 : 4;
    const size_t ngran = n / nranks * esz / 16;
    hipLaunchKernelGGL(gather_copy_kernel, grid_for(ngran, nranks), dim3(kThreads), 0, stream, chunks,
                       ngran, static_cast<uint4*>(out));
    return hipGetLastError();
}

// ---------------------------------------------------------------------------
// all-to-all-v routing: one workgroup of 1024 lanes.  Lane t owns rows
// [t*R, (t+1)*R).  Per-lane destination counts go to LDS, one wavefront per
// destination turns them into exclusive prefixes, and each lane then places
// its rows in order: a stable destination-major permutation.
// ---------------------------------------------------------------------------

constexpr int kRouteThreads = 1024;

__global__ __launch_bounds__(kRouteThreads) void a2av_route_kernel(const int32_t* __restrict__ dest,
                                                                   size_t rows, int nranks,
                                                                   int32_t* __restrict__ counts,
                                                                   int32_t* __restrict__ offsets,
                                                                   int32_t* __restrict__ perm) {
    __shared__ int32_t pre[kMaxRanks][kRouteThreads];
    __shared__ int32_t total[kMaxRanks];
    __shared__ int32_t base[kMaxRanks];
    const int t = threadIdx.x;
    const size_t R = (rows + kRouteThreads - 1) / kRouteThreads;
    const size_t k0 = (size_t)t * R;
    const size_t k1 = k0 + R < rows ? k0 + R : rows;

    int32_t cnt[kMaxRanks];
#pragma unroll
    for (int d = 0; d < kMaxRanks; ++d) cnt[d] = 0;
    for (size_t k = k0; k < k1; ++k) {
        const int32_t d = dest[k];
#pragma unroll
        for (int j = 0; j < kMaxRanks; ++j) cnt[j] += (d == j && j < nranks) ? 1 : 0;
    }
#pragma unroll
    for (int d = 0; d < kMaxRanks; ++d) pre[d][t] = cnt[d];
    __syncthreads();

    // wavefront w < 8 scans destination w: lane l owns entries [16l, 16l+16)
    const int w = t / 64, lane = t % 64;
    if (w < kMaxRanks) {
        int32_t* row = pre[w];
        int32_t local[16];
        int32_t sum = 0;
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            local[i] = row[lane * 16 + i];
            sum += local[i];
        }
        // inclusive scan of per-lane sums across the wavefront
        int32_t inc = sum;
#pragma unroll
        for (int off = 1; off < 64; off <<= 1) {
            const int32_t y = __shfl_up(inc, off, 64);
            if (lane >= off) inc += y;
        }
        int32_t run = inc - sum;
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            row[lane * 16 + i] = run;
            run += local[i];
        }
        if (lane == 63) total[w] = inc;
    }
    __syncthreads();
    if (t == 0) {
        int32_t acc = 0;
        for (int d = 0; d < kMaxRanks; ++d) {
            base[d] = acc;
            if (d < nranks) {
                counts[d] = total[d];
                offsets[d] = acc;
                acc += total[d];
            }
        }
    }
    __syncthreads();
    int32_t pos[kMaxRanks];
#pragma unroll
    for (int d = 0; d < kMaxRanks; ++d) pos[d] = base[d] + pre[d][t];
    for (size_t k = k0; k < k1; ++k) {
        const int32_t d = dest[k];
#pragma unroll
        for (int j = 0; j < kMaxRanks; ++j) {
            if (d == j && j < nranks) {
                perm[pos[j]] = (int32_t)k;
                pos[j] += 1;
            }
        }
    }
    // rows with an out-of-range destination were dropped: mark perm's tail
    int32_t placed = 0;
    for (int d = 0; d < nranks; ++d) placed += total[d];
    for (size_t k = (size_t)placed + t; k < rows; k += kRouteThreads) perm[k] = -1;
}

hipError_t launch_a2av_route(const int32_t* dest, size_t rows, int nranks, int32_t* counts, int32_t* offsets,
                             int32_t* perm, hipStream_t stream) {
    hipLaunchKernelGGL(a2av_route_kernel, dim3(1), dim3(kRouteThreads), 0, stream, dest, rows, nranks, counts,
                       offsets, perm);
    return hipGetLastError();
}

// ---------------------------------------------------------------------------
// gather + quantize rows: grid.y walks packed rows, grid.x the granules of a row
// ---------------------------------------------------------------------------

template <typename In>
__global__ __launch_bounds__(1024) void quantize_rows_kernel(const In* __restrict__ x, size_t rows,
                                                             size_t row_len, const int32_t* __restrict__ perm,
                                                             uint8_t* __restrict__ codes,
                                                             float* __restrict__ scales) {
    const size_t lpr = row_len / kGranule;
    const size_t seg = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (seg >= lpr) return;
    for (size_t k = blockIdx.y; k < rows; k += gridDim.y) {
        const int32_t src = perm[k];
        const size_t g = k * lpr + seg;  // packed granule index
        if (src < 0 || (size_t)src >= rows) {
            *reinterpret_cast<uint4*>(codes + g * kGranule) = make_uint4(0u, 0u, 0u, 0u);
            if ((threadIdx.x & (kLanesPerBlock - 1)) == 0) scales[g / kLanesPerBlock] = 0.0f;
            continue;
        }
        float v[kGranule];
        load16(x + (size_t)src * row_len + seg * kGranule, v);
        float s;
        const uint4 c = quantize_granule(v, &s);
        *reinterpret_cast<uint4*>(codes + g * kGranule) = c;
        if ((threadIdx.x & (kLanesPerBlock - 1)) == 0) scales[g / kLanesPerBlock] = s;
    }
}

hipError_t launch_quantize_rows(const void* x, int in_bf16, size_t rows, size_t row_len, const int32_t* perm,
                                uint8_t* codes, float* scales, hipStream_t stream) {
    const size_t lpr = row_len / kGranule;
    // a row of up to 1024 granules is one workgroup (whole wavefronts); longer rows use 256-lane groups
    unsigned threads, gx;
    if (lpr <= 1024) {
        threads = (unsigned)((lpr + 63) / 64 * 64);
        gx = 1;
    } else {
        threads = kThreads;
        gx = (unsigned)((lpr + kThreads - 1) / kThreads);
    }
    const unsigned gy = (unsigned)(rows < 65535 ? rows : 65535);
    const dim3 grid(gx, gy, 1), block(threads);
    if (in_bf16)
        hipLaunchKernelGGL(quantize_rows_kernel<uint16_t>, grid, block, 0, stream, static_cast<const uint16_t*>(x),
                           rows, row_len, perm, codes, scales);
    else
        hipLaunchKernelGGL(quantize_rows_kernel<float>, grid, block, 0, stream, static_cast<const float*>(x), rows,
                           row_len, perm, codes, scales);
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
    hipLaunchKernelGGL(encode_kernel, grid_for(ngran), dim3(kThreads), 0, stream, x, n, codes);
    return hipGetLastError();
}

}  // namespace lpc
