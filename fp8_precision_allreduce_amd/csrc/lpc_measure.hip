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
// of src (those below nr) and stores 16-byte vectors g, g + L, ..., of dst
// (those below nw), non-temporally, so that every wavefront instruction
// covers one contiguous KiB.  The stored value depends on every loaded one.
// Tiles in XCD-aware order, as the library's kernels take them.
template <int KR, int KW>
__global__ __launch_bounds__(kThreads) void stream_kernel(const uint4* __restrict__ src, size_t nr,
                                                          uint4* __restrict__ dst, size_t nw) {
    const size_t L = (size_t)gridDim.x * kThreads;
    const size_t g = lpc::xcd_tile() * kThreads + threadIdx.x;
    uint4 v = make_uint4((uint32_t)g, 0u, 0u, 0u);
#pragma unroll
    for (int k = 0; k < KR; ++k) {
        const size_t i = g + k * L;
        if (i < nr) {
            const uint4 t = src[i];
            v.x ^= t.x;
            v.y ^= t.y;
            v.z ^= t.z;
            v.w ^= t.w;
        }
    }
#pragma unroll
    for (int k = 0; k < KW; ++k) {
        const size_t i = g + k * L;
        if (i < nw) {
            const u32x4_t w = {v.x, v.y, v.z, v.w ^ (uint32_t)k};
            __builtin_nontemporal_store(w, reinterpret_cast<u32x4_t*>(dst + i));
        }
    }
}

template <int KR, int KW>
hipError_t launch_stream(const void* src, size_t nr, void* dst, size_t nw, hipStream_t stream) {
    const size_t lanes = std::max((nr + KR - 1) / KR, (nw + KW - 1) / KW);
    const dim3 grid((unsigned)((lanes + kThreads - 1) / kThreads));
    const uint4* s = static_cast<const uint4*>(src);
    uint4* d = static_cast<uint4*>(dst);
    void* args[] = {&s, &nr, &d, &nw};
    return hipLaunchKernel(reinterpret_cast<const void*>(stream_kernel<KR, KW>), grid, dim3(kThreads), args, 0,
                           stream);
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

lpc_status lpc_measure_stream(const void* src, size_t read_bytes, void* dst, size_t write_bytes,
                              hipStream_t stream) {
    if (read_bytes % 16 || write_bytes % 16) return LPC_ERR_SHAPE;
    if (read_bytes == 0 && write_bytes == 0) return LPC_OK;
    if ((read_bytes && !src) || (write_bytes && !dst)) return LPC_ERR_NULL;
    if ((read_bytes && misaligned(src)) || (write_bytes && misaligned(dst))) return LPC_ERR_ALIGN;
    const size_t nr = read_bytes / 16, nw = write_bytes / 16;
    // loads and stores per lane in the ratio of the two byte counts, 1..4 each
    int kr = 1, kw = 1;
    if (nr >= nw) kr = nw == 0 ? 4 : (int)std::min<size_t>(4, (nr + nw / 2) / nw);
    else kw = nr == 0 ? 4 : (int)std::min<size_t>(4, (nw + nr / 2) / nr);
    if (std::max((nr + kr - 1) / kr, (nw + kw - 1) / kw) > (size_t)INT32_MAX) return LPC_ERR_SHAPE;
    hipError_t e = hipErrorInvalidValue;
    switch (kr * 8 + kw) {
        case 1 * 8 + 1: e = launch_stream<1, 1>(src, nr, dst, nw, stream); break;
        case 2 * 8 + 1: e = launch_stream<2, 1>(src, nr, dst, nw, stream); break;
        case 3 * 8 + 1: e = launch_stream<3, 1>(src, nr, dst, nw, stream); break;
        case 4 * 8 + 1: e = launch_stream<4, 1>(src, nr, dst, nw, stream); break;
        case 1 * 8 + 2: e = launch_stream<1, 2>(src, nr, dst, nw, stream); break;
        case 1 * 8 + 3: e = launch_stream<1, 3>(src, nr, dst, nw, stream); break;
        case 1 * 8 + 4: e = launch_stream<1, 4>(src, nr, dst, nw, stream); break;
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
