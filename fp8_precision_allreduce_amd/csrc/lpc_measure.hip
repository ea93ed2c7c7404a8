// lpc_measure.hip -- reference kernels for measurement (include/lpc_measure.h).
// They are not part of any collective: a plain streaming kernel that moves a
// given number of bytes at a given read:write mix as simply as the hardware
// allows (the practical ceiling a path kernel with the same traffic is held
// against), and an empty launch of a given shape (the fixed cost every launch
// of that shape pays before it moves a byte).
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <algorithm>

#include "lpc.h"
#include "lpc_device.hpp"
#include "lpc_measure.h"

namespace {

constexpr int kThreads = 256;
using lpc::u32x4_t;

// Lane g of L launched lanes loads 16-byte vectors g, g + L, ..., g + (KR-1)*L
// of src (those below nr) and then stores 16-byte vectors g, g + L, ..., of dst
// (those below nw), loads and stores non-temporal, so that every wavefront
// instruction covers one contiguous KiB.  The stored value depends on every
// loaded one; with nothing to store, a store under a flag that the host always
// passes as 0 keeps the loads live.  Tiles in XCD-aware order, as the
// library's kernels take them.
template <int KR, int KW>
__global__ __launch_bounds__(kThreads) void stream_kernel(const uint4* __restrict__ src, size_t nr,
                                                          uint4* __restrict__ dst, size_t nw, int* sink,
                                                          int dump) {
    const size_t L = (size_t)gridDim.x * kThreads;
    const size_t g = lpc::xcd_tile() * kThreads + threadIdx.x;
    u32x4_t v = {(uint32_t)g, 0u, 0u, 0u};
#pragma unroll
    for (int k = 0; k < KR; ++k) {
        const size_t i = g + k * L;
        if (i < nr) v ^= __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(src + i));
    }
    if constexpr (KW == 0) {
        if (dump) *sink = (int)(v[0] ^ v[1] ^ v[2] ^ v[3]);
    } else {
#pragma unroll
        for (int k = 0; k < KW; ++k) {
            const size_t i = g + k * L;
            if (i < nw) {
                u32x4_t w = v;
                w[3] ^= (uint32_t)k;
                __builtin_nontemporal_store(w, reinterpret_cast<u32x4_t*>(dst + i));
            }
        }
    }
}

template <int KR, int KW>
hipError_t launch_stream(const void* src, size_t nr, void* dst, size_t nw, unsigned wgs, int* sink,
                         hipStream_t stream) {
    const uint4* s = static_cast<const uint4*>(src);
    uint4* d = static_cast<uint4*>(dst);
    int dump = 0;
    void* args[] = {&s, &nr, &d, &nw, &sink, &dump};
    return hipLaunchKernel(reinterpret_cast<const void*>(stream_kernel<KR, KW>), dim3(wgs), dim3(kThreads), args, 0,
                           stream);
}

// Per-lane counts are rounded up to 1, 2, 4 or 8 (0 when there is nothing to move).
int bucket(size_t k) { return k == 0 ? 0 : k <= 1 ? 1 : k <= 2 ? 2 : k <= 4 ? 4 : 8; }

// Workgroups of the streaming kernel.  per_lane == 0: one round of resident wavefronts (2,048
// workgroups of 256 lanes, 8 wavefronts per SIMD on 256 CUs) when that leaves at most 8 vectors per
// lane each way, fewer when there is less to move, more (8 vectors per lane) for larger transfers.
// per_lane == K: as many workgroups as K vectors per lane each way need.
size_t stream_workgroups(size_t nr, size_t nw, int per_lane) {
    constexpr size_t kRound = 2048, kMaxPerLane = 8;
    const size_t m = std::max(nr, nw);
    if (per_lane > 0) return (m + kThreads * per_lane - 1) / (kThreads * per_lane);
    const size_t need = (m + kThreads - 1) / kThreads;
    if (need <= kRound) return need;
    if (m <= kRound * kThreads * kMaxPerLane) return kRound;
    return (m + kThreads * kMaxPerLane - 1) / (kThreads * kMaxPerLane);
}

// A kernel-argument block of K bytes.
template <int K>
struct ArgBlock {
    uint64_t w[K / 8];
};

// Every wavefront loads the whole argument block and the grid size (as the
// library's kernels load their arguments and compute their tile order), and
// writes nothing: the store below needs a combination of argument values the
// host never passes.
template <int K>
__global__ void empty_kernel(ArgBlock<K> a, int* sink) {
    uint64_t h = 0;
#pragma unroll
    for (int k = 0; k < K / 8; ++k) h ^= a.w[k];
    if (h == 0x9E3779B97F4A7C15ull && blockIdx.x == gridDim.x) *sink = 1;
}

template <int K>
hipError_t launch_empty(dim3 grid, unsigned threads, int* sink, hipStream_t stream) {
    ArgBlock<K> a{};
    for (int k = 0; k < K / 8; ++k) a.w[k] = reinterpret_cast<uintptr_t>(sink);  // xor of the block is 0 or sink
    void* args[] = {&a, &sink};
    return hipLaunchKernel(reinterpret_cast<const void*>(empty_kernel<K>), grid, dim3(threads), args, 0, stream);
}

bool misaligned(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) != 0; }

}  // namespace

extern "C" {

lpc_status lpc_measure_stream(const void* src, size_t read_bytes, void* dst, size_t write_bytes, int per_lane,
                              hipStream_t stream) {
    if (read_bytes % 16 || write_bytes % 16) return LPC_ERR_SHAPE;
    if (per_lane != 0 && per_lane != 1 && per_lane != 2 && per_lane != 4 && per_lane != 8) return LPC_ERR_SHAPE;
    if (read_bytes == 0 && write_bytes == 0) return LPC_OK;
    if ((read_bytes && !src) || !dst) return LPC_ERR_NULL;
    if ((read_bytes && misaligned(src)) || misaligned(dst)) return LPC_ERR_ALIGN;
    int* sink = static_cast<int*>(dst);  // read only: never written
    const size_t nr = read_bytes / 16, nw = write_bytes / 16;
    const size_t wgs = stream_workgroups(nr, nw, per_lane);
    if (wgs > (size_t)INT32_MAX / kThreads) return LPC_ERR_SHAPE;
    const size_t L = wgs * kThreads;
    const int kr = bucket((nr + L - 1) / L), kw = bucket((nw + L - 1) / L);
    const unsigned g = (unsigned)wgs;
    hipError_t e = hipErrorInvalidValue;
    switch (kr * 16 + kw) {
#define LPC_STREAM_CASE(R, W) \
    case R * 16 + W: e = launch_stream<R, W>(src, nr, dst, nw, g, sink, stream); break;
        LPC_STREAM_CASE(1, 0) LPC_STREAM_CASE(2, 0) LPC_STREAM_CASE(4, 0) LPC_STREAM_CASE(8, 0)
        LPC_STREAM_CASE(0, 1) LPC_STREAM_CASE(0, 2) LPC_STREAM_CASE(0, 4) LPC_STREAM_CASE(0, 8)
        LPC_STREAM_CASE(1, 1) LPC_STREAM_CASE(1, 2) LPC_STREAM_CASE(1, 4) LPC_STREAM_CASE(1, 8)
        LPC_STREAM_CASE(2, 1) LPC_STREAM_CASE(2, 2) LPC_STREAM_CASE(2, 4) LPC_STREAM_CASE(2, 8)
        LPC_STREAM_CASE(4, 1) LPC_STREAM_CASE(4, 2) LPC_STREAM_CASE(4, 4) LPC_STREAM_CASE(4, 8)
        LPC_STREAM_CASE(8, 1) LPC_STREAM_CASE(8, 2) LPC_STREAM_CASE(8, 4) LPC_STREAM_CASE(8, 8)
#undef LPC_STREAM_CASE
    }
    return e == hipSuccess ? LPC_OK : LPC_ERR_HIP;
}

lpc_status lpc_measure_empty(unsigned grid_x, unsigned grid_y, unsigned threads, size_t kernarg_bytes, int* sink,
                             hipStream_t stream) {
    if (grid_x == 0 || grid_y == 0 || threads == 0 || threads > 1024 || kernarg_bytes > 512) return LPC_ERR_SHAPE;
    if (!sink) return LPC_ERR_NULL;
    if (misaligned(sink)) return LPC_ERR_ALIGN;
    const dim3 grid(grid_x, grid_y);
    hipError_t e;
    if (kernarg_bytes <= 16) e = launch_empty<16>(grid, threads, sink, stream);
    else if (kernarg_bytes <= 64) e = launch_empty<64>(grid, threads, sink, stream);
    else if (kernarg_bytes <= 128) e = launch_empty<128>(grid, threads, sink, stream);
    else if (kernarg_bytes <= 256) e = launch_empty<256>(grid, threads, sink, stream);
    else if (kernarg_bytes <= 320) e = launch_empty<320>(grid, threads, sink, stream);
    else e = launch_empty<512>(grid, threads, sink, stream);
    return e == hipSuccess ? LPC_OK : LPC_ERR_HIP;
}

}  // extern "C"
