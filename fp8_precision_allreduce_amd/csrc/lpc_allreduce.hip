// lpc_allreduce.hip -- allreduce over emulated ranks on one GPU, and the
// size-based algorithm choice (the extern "C" calls of include/lpc.h's
// "Allreduce over emulated ranks" section).
//
// An emulated allreduce runs each step of the algorithm for all ranks at
// once: one launch per step, the rank taken from a grid dimension, each rank's
// share computed exactly as the per-rank entry point computes it, with the
// other ranks' buffers standing in for its peers' memory.  All arguments are
// checked before the first launch, so a validation error enqueues nothing.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <mutex>

#include "lpc.h"
#include "lpc_launch.hpp"

// Scratch of lpc_allreduce_emulated_noalloc: the workspace that
// lpc_allreduce_emulated takes as an argument, here a file-scope device array.
// Every GPU the library runs on holds its own copy until the process ends.
// Host code never passes the array's name to the runtime or a kernel: the name
// is a host-side stand-in, and the device address comes from
// hipGetSymbolAddress (scratch_address below).
static __device__ __align__(256) uint8_t scratch[LPC_NOALLOC_SCRATCH_BYTES];

namespace {

// Device address of `scratch` on each device, looked up once per device with
// that device current (each GPU holds the array at its own address).
constexpr int kMaxDevices = 64;
std::once_flag g_scratch_once[kMaxDevices];
void* g_scratch_ptr[kMaxDevices];
hipError_t g_scratch_err[kMaxDevices];

lpc_status scratch_address(void** out) {
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return LPC_ERR_HIP;
    std::call_once(g_scratch_once[dev], [dev] {
        void* p = nullptr;
        g_scratch_err[dev] = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        g_scratch_ptr[dev] = p;
    });
    if (g_scratch_err[dev] != hipSuccess || g_scratch_ptr[dev] == nullptr) return LPC_ERR_HIP;
    *out = g_scratch_ptr[dev];
    return LPC_OK;
}

constexpr size_t kRegionAlign = 256;  // every workspace region starts on a 256-byte boundary

size_t align_up(size_t x) { return (x + kRegionAlign - 1) / kRegionAlign * kRegionAlign; }

bool bad_dtype(lpc_dtype t) { return t != LPC_F32 && t != LPC_BF16; }

size_t elem_bytes(lpc_dtype t) { return t == LPC_BF16 ? 2 : 4; }

bool misaligned(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) != 0; }

// Workspace regions of the low-precision algorithm, in bytes from the start.
struct LpLayout {
    size_t codes[LPC_MAX_RANKS], scales[LPC_MAX_RANKS];   // every rank's quantized buffer
    size_t ccodes[LPC_MAX_RANKS], cscales[LPC_MAX_RANKS]; // every rank's requantized chunk
    size_t total;
};

LpLayout lp_layout(int nranks, size_t n) {
    LpLayout L{};
    const size_t C = n / (size_t)nranks;
    size_t off = 0;
    for (int r = 0; r < nranks; ++r) {
        L.codes[r] = off;
        off += align_up(n);
        L.scales[r] = off;
        off += align_up(n / LPC_BLOCK * sizeof(float));
    }
    for (int r = 0; r < nranks; ++r) {
        L.ccodes[r] = off;
        off += align_up(C);
        L.cscales[r] = off;
        off += align_up(C / LPC_BLOCK * sizeof(float));
    }
    L.total = off;
    return L;
}

// Argument checks shared by the workspace query and the allreduce itself.
lpc_status check_args(lpc_algo algo, int nranks, size_t n, lpc_dtype t) {
    if (bad_dtype(t)) return LPC_ERR_DTYPE;
    if (algo != LPC_ALGO_DDA_FLAT && algo != LPC_ALGO_DDA_TREE && algo != LPC_ALGO_LOW_PRECISION)
        return LPC_ERR_DTYPE;
    if (algo == LPC_ALGO_DDA_FLAT && t != LPC_BF16) return LPC_ERR_DTYPE;
    if (nranks < 1 || nranks > LPC_MAX_RANKS) return LPC_ERR_RANKS;
    if (n > LPC_MAX_ELEMS) return LPC_ERR_SHAPE;
    if (algo == LPC_ALGO_DDA_TREE && n % ((size_t)8 * nranks)) return LPC_ERR_SHAPE;
    if (algo == LPC_ALGO_LOW_PRECISION && n % ((size_t)LPC_BLOCK * nranks)) return LPC_ERR_SHAPE;
    return LPC_OK;
}

size_t workspace_bytes(lpc_algo algo, int nranks, size_t n, lpc_dtype t) {
    switch (algo) {
        case LPC_ALGO_DDA_FLAT: return (size_t)nranks * align_up(n * 2);
        case LPC_ALGO_DDA_TREE: return (size_t)nranks * align_up(n / (size_t)nranks * elem_bytes(t));
        case LPC_ALGO_LOW_PRECISION: return lp_layout(nranks, n).total;
        default: return 0;
    }
}

#define LPC_TRY(expr)                        \
    do {                                     \
        const lpc_status st_ = (expr);       \
        if (st_ != LPC_OK) return st_;       \
    } while (0)

#define LPC_TRY_HIP(expr)                              \
    do {                                               \
        if ((expr) != hipSuccess) return LPC_ERR_HIP;  \
    } while (0)

lpc_status check_bufs(void* const bufs[], int nranks) {
    for (int r = 0; r < nranks; ++r)
        if (!bufs[r]) return LPC_ERR_NULL;
    for (int r = 0; r < nranks; ++r)
        if (misaligned(bufs[r])) return LPC_ERR_ALIGN;
    return LPC_OK;
}

// Every rank's share of the allreduce, one launch per step, with the
// workspace at `ws` (arguments already checked).
lpc_status run_allreduce(void* const bufs[], int nranks, size_t n, lpc_dtype t, lpc_algo algo, uint8_t* ws,
                         hipStream_t stream);

}  // namespace

extern "C" {

lpc_algo lpc_select_algo(int nranks, size_t n, lpc_dtype t, int low_precision_enabled) {
    if (bad_dtype(t) || nranks < 1 || nranks > LPC_MAX_RANKS || n > LPC_MAX_ELEMS) return LPC_ALGO_AUTO;
    const size_t bytes = n * elem_bytes(t);
    if (t == LPC_BF16 && bytes <= LPC_DDA_FLAT_MAX_BYTES) return LPC_ALGO_DDA_FLAT;
    if (low_precision_enabled && bytes >= LPC_LOW_PRECISION_MIN_BYTES && n % ((size_t)LPC_BLOCK * nranks) == 0)
        return LPC_ALGO_LOW_PRECISION;
    if (n % ((size_t)8 * nranks) == 0) return LPC_ALGO_DDA_TREE;
    if (t == LPC_BF16) return LPC_ALGO_DDA_FLAT;
    return LPC_ALGO_AUTO;
}

lpc_status lpc_allreduce_workspace_bytes(lpc_algo algo, int nranks, size_t n, lpc_dtype t, size_t* bytes) {
    LPC_TRY(check_args(algo, nranks, n, t));
    if (!bytes) return LPC_ERR_NULL;
    *bytes = workspace_bytes(algo, nranks, n, t);
    return LPC_OK;
}

lpc_status lpc_allreduce_emulated(void* const bufs[], int nranks, size_t n, lpc_dtype t, lpc_algo algo,
                                  void* workspace, size_t ws_bytes, hipStream_t stream) {
    LPC_TRY(check_args(algo, nranks, n, t));
    if (n == 0) return LPC_OK;
    if (!bufs || !workspace) return LPC_ERR_NULL;
    LPC_TRY(check_bufs(bufs, nranks));
    if (misaligned(workspace)) return LPC_ERR_ALIGN;
    if (ws_bytes < workspace_bytes(algo, nranks, n, t)) return LPC_ERR_SHAPE;
    return run_allreduce(bufs, nranks, n, t, algo, static_cast<uint8_t*>(workspace), stream);
}

lpc_status lpc_allreduce_emulated_noalloc(void* const bufs[], int nranks, size_t n, lpc_dtype t, lpc_algo algo,
                                          hipStream_t stream) {
    LPC_TRY(check_args(algo, nranks, n, t));
    if (n == 0) return LPC_OK;
    if (!bufs) return LPC_ERR_NULL;
    LPC_TRY(check_bufs(bufs, nranks));
    if (workspace_bytes(algo, nranks, n, t) > LPC_NOALLOC_SCRATCH_BYTES) return LPC_ERR_SCRATCH;
    void* ws = nullptr;
    LPC_TRY(scratch_address(&ws));
    return run_allreduce(bufs, nranks, n, t, algo, static_cast<uint8_t*>(ws), stream);
}

}  // extern "C"

namespace {

lpc_status run_allreduce(void* const bufs[], int nranks, size_t n, lpc_dtype t, lpc_algo algo, uint8_t* ws,
                         hipStream_t stream) {
    lpc::RankBufs in{};
    for (int r = 0; r < nranks; ++r) in.p[r] = bufs[r];

    if (algo == LPC_ALGO_DDA_FLAT) {
        // every rank reduces all buffers into its own workspace output, then
        // one launch copies each output into its rank's buffer
        const size_t slot = align_up(n * 2);
        lpc::RankOut outs{}, back{};
        lpc::RankBufs slots{};
        for (int r = 0; r < nranks; ++r) {
            outs.p[r] = ws + r * slot;
            slots.p[r] = ws + r * slot;
            back.p[r] = bufs[r];
        }
        LPC_TRY_HIP(lpc::launch_dda_flat_ranks(in, nranks, n, outs, stream));
        LPC_TRY_HIP(lpc::launch_copy_ranks(slots, nranks, n * 2, back, stream));
        return LPC_OK;
    }
    if (algo == LPC_ALGO_DDA_TREE) {
        const size_t slot = align_up(n / (size_t)nranks * elem_bytes(t));
        lpc::RankOut chunks_out{}, outs{};
        lpc::RankBufs chunks{};
        for (int r = 0; r < nranks; ++r) {
            chunks_out.p[r] = ws + r * slot;
            chunks.p[r] = ws + r * slot;
            outs.p[r] = bufs[r];
        }
        LPC_TRY_HIP(lpc::launch_dda_tree_rs_ranks(in, t == LPC_BF16, nranks, n, chunks_out, stream));
        LPC_TRY_HIP(lpc::launch_dda_tree_ag_ranks(chunks, t == LPC_BF16, nranks, n, outs, stream));
        return LPC_OK;
    }
    // low precision: quantize every rank, reduce-scatter every chunk, all-gather into every buffer
    const LpLayout L = lp_layout(nranks, n);
    lpc::RankQuant q{}, cq{};
    lpc::RankCodes codes{}, chunks{};
    lpc::RankOut outs{};
    for (int r = 0; r < nranks; ++r) {
        q.codes[r] = ws + L.codes[r];
        q.scales[r] = reinterpret_cast<float*>(ws + L.scales[r]);
        cq.codes[r] = ws + L.ccodes[r];
        cq.scales[r] = reinterpret_cast<float*>(ws + L.cscales[r]);
        codes.codes[r] = q.codes[r];
        codes.scales[r] = q.scales[r];
        chunks.codes[r] = cq.codes[r];
        chunks.scales[r] = cq.scales[r];
        outs.p[r] = bufs[r];
    }
    LPC_TRY_HIP(lpc::launch_quantize_ranks(in, t == LPC_BF16, nranks, n, q, stream));
    LPC_TRY_HIP(lpc::launch_reduce_scatter_ranks(codes, nranks, n, cq, stream));
    LPC_TRY_HIP(lpc::launch_allgather_ranks(chunks, nranks, n, outs, t == LPC_BF16, stream));
    return LPC_OK;
}

}  // namespace
