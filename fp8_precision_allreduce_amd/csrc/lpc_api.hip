// lpc_api.hip -- the extern "C" entry points declared in include/lpc.h.
//
// Every entry point validates its arguments on the host, in the order the
// header states, before it touches the HIP runtime; on failure it returns the
// status and enqueues nothing.  Only then does it copy the host pointer
// arrays into kernel-argument structs and launch.
#include <stdint.h>

#include "lpc.h"
#include "lpc_launch.hpp"

namespace {

using lpc::RankBufs;
using lpc::RankCodes;

inline bool misaligned(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) != 0; }

inline bool bad_dtype(lpc_dtype t) { return t != LPC_F32 && t != LPC_BF16; }

inline bool bad_ranks(int nranks) { return nranks < 1 || nranks > LPC_MAX_RANKS; }

inline lpc_status hip_status(hipError_t e) { return e == hipSuccess ? LPC_OK : LPC_ERR_HIP; }

// pointer array of nranks entries; entry `skip` (if >= 0) is not required
template <typename T>
lpc_status check_array(const T* const* arr, int nranks, int skip = -1) {
    if (!arr) return LPC_ERR_NULL;
    for (int p = 0; p < nranks; ++p)
        if (p != skip && !arr[p]) return LPC_ERR_NULL;
    return LPC_OK;
}

template <typename T>
lpc_status check_array_align(const T* const* arr, int nranks, int skip = -1) {
    for (int p = 0; p < nranks; ++p)
        if (p != skip && misaligned(arr[p])) return LPC_ERR_ALIGN;
    return LPC_OK;
}

RankCodes rank_codes(const uint8_t* const* codes, const float* const* scales, int nranks, int skip = -1) {
    RankCodes r{};
    for (int p = 0; p < nranks; ++p) {
        if (p == skip) continue;
        r.codes[p] = codes[p];
        r.scales[p] = scales[p];
    }
    return r;
}

RankBufs rank_bufs(const void* const* bufs, int nranks) {
    RankBufs r{};
    for (int p = 0; p < nranks; ++p) r.p[p] = bufs[p];
    return r;
}

#define LPC_TRY(expr)                        \
    do {                                     \
        const lpc_status st_ = (expr);       \
        if (st_ != LPC_OK) return st_;       \
    } while (0)

}  // namespace

extern "C" {

int lpc_abi_version(void) { return LPC_ABI_VERSION; }

const char* lpc_status_string(lpc_status s) {
    switch (s) {
        case LPC_OK: return "LPC_OK";
        case LPC_ERR_NULL: return "LPC_ERR_NULL: a required pointer is NULL";
        case LPC_ERR_SHAPE: return "LPC_ERR_SHAPE: element count is not a whole number of blocks/chunks or is too large";
        case LPC_ERR_RANKS: return "LPC_ERR_RANKS: nranks outside 1..8 or rank outside 0..nranks-1";
        case LPC_ERR_DTYPE: return "LPC_ERR_DTYPE: unknown element type";
        case LPC_ERR_ALIGN: return "LPC_ERR_ALIGN: a pointer is not 16-byte aligned";
        case LPC_ERR_HIP: return "LPC_ERR_HIP: the HIP runtime refused the kernel launch";
        case LPC_ERR_SCRATCH:
            return "LPC_ERR_SCRATCH: the call needs more device scratch than the library's static array holds";
    }
    return "unknown lpc_status";
}

lpc_status lpc_quantize_fp8(const void* x, lpc_dtype in, size_t n, uint8_t* codes, float* scales,
                            hipStream_t stream) {
    if (bad_dtype(in)) return LPC_ERR_DTYPE;
    if (n == 0) return LPC_OK;
    if (!x || !codes || !scales) return LPC_ERR_NULL;
    if (misaligned(x) || misaligned(codes) || misaligned(scales)) return LPC_ERR_ALIGN;
    if (n % LPC_BLOCK || n > LPC_MAX_ELEMS) return LPC_ERR_SHAPE;
    return hip_status(lpc::launch_quantize(x, in == LPC_BF16, n, codes, scales, stream));
}

lpc_status lpc_reduce_scatter_chunk(const uint8_t* const codes[], const float* const scales[], int nranks,
                                    int rank, size_t n, uint8_t* chunk_codes, float* chunk_scales,
                                    hipStream_t stream) {
    if (bad_ranks(nranks) || rank < 0 || rank >= nranks) return LPC_ERR_RANKS;
    if (n == 0) return LPC_OK;
    LPC_TRY(check_array(codes, nranks));
    LPC_TRY(check_array(scales, nranks));
    if (!chunk_codes || !chunk_scales) return LPC_ERR_NULL;
    LPC_TRY(check_array_align(codes, nranks));
    LPC_TRY(check_array_align(scales, nranks));
    if (misaligned(chunk_codes) || misaligned(chunk_scales)) return LPC_ERR_ALIGN;
    if (n % ((size_t)LPC_BLOCK * nranks) || n > LPC_MAX_ELEMS) return LPC_ERR_SHAPE;
    return hip_status(lpc::launch_reduce_scatter_chunk(rank_codes(codes, scales, nranks), nranks, rank, n,
                                                       chunk_codes, chunk_scales, stream));
}

lpc_status lpc_reduce_scatter(const uint8_t* const codes[], const float* const scales[], int nranks, int rank,
                              size_t n, void* out, lpc_dtype out_t, hipStream_t stream) {
    if (bad_dtype(out_t)) return LPC_ERR_DTYPE;
    if (bad_ranks(nranks) || rank < 0 || rank >= nranks) return LPC_ERR_RANKS;
    if (n == 0) return LPC_OK;
    LPC_TRY(check_array(codes, nranks));
    LPC_TRY(check_array(scales, nranks));
    if (!out) return LPC_ERR_NULL;
    LPC_TRY(check_array_align(codes, nranks));
    LPC_TRY(check_array_align(scales, nranks));
    if (misaligned(out)) return LPC_ERR_ALIGN;
    if (n % ((size_t)LPC_BLOCK * nranks) || n > LPC_MAX_ELEMS) return LPC_ERR_SHAPE;
    return hip_status(lpc::launch_reduce_scatter_out(rank_codes(codes, scales, nranks), nranks, rank, n, out,
                                                     out_t == LPC_BF16, stream));
}

lpc_status lpc_allgather_dequant(const uint8_t* const chunk_codes[], const float* const chunk_scales[],
                                 int nranks, size_t n, void* out, lpc_dtype out_t, hipStream_t stream) {
    if (bad_dtype(out_t)) return LPC_ERR_DTYPE;
    if (bad_ranks(nranks)) return LPC_ERR_RANKS;
    if (n == 0) return LPC_OK;
    LPC_TRY(check_array(chunk_codes, nranks));
    LPC_TRY(check_array(chunk_scales, nranks));
    if (!out) return LPC_ERR_NULL;
    LPC_TRY(check_array_align(chunk_codes, nranks));
    LPC_TRY(check_array_align(chunk_scales, nranks));
    if (misaligned(out)) return LPC_ERR_ALIGN;
    if (n % ((size_t)LPC_BLOCK * nranks) || n > LPC_MAX_ELEMS) return LPC_ERR_SHAPE;
    return hip_status(lpc::launch_allgather(rank_codes(chunk_codes, chunk_scales, nranks), nranks, n, out,
                                            out_t == LPC_BF16, stream));
}

lpc_status lpc_rs_ag_fused(const uint8_t* const codes[], const float* const scales[], int nranks, int rank,
                           size_t n, uint8_t* chunk_codes, float* chunk_scales,
                           const uint8_t* const peer_chunk_codes[], const float* const peer_chunk_scales[],
                           void* out, lpc_dtype out_t, hipStream_t stream) {
    if (bad_dtype(out_t)) return LPC_ERR_DTYPE;
    if (bad_ranks(nranks) || rank < 0 || rank >= nranks) return LPC_ERR_RANKS;
    if (n == 0) return LPC_OK;
    LPC_TRY(check_array(codes, nranks));
    LPC_TRY(check_array(scales, nranks));
    LPC_TRY(check_array(peer_chunk_codes, nranks, rank));
    LPC_TRY(check_array(peer_chunk_scales, nranks, rank));
    if (!chunk_codes || !chunk_scales || !out) return LPC_ERR_NULL;
    LPC_TRY(check_array_align(codes, nranks));
    LPC_TRY(check_array_align(scales, nranks));
    LPC_TRY(check_array_align(peer_chunk_codes, nranks, rank));
    LPC_TRY(check_array_align(peer_chunk_scales, nranks, rank));
    if (misaligned(chunk_codes) || misaligned(chunk_scales) || misaligned(out)) return LPC_ERR_ALIGN;
    if (n % ((size_t)LPC_BLOCK * nranks) || n > LPC_MAX_ELEMS) return LPC_ERR_SHAPE;
    return hip_status(lpc::launch_rs_ag_fused(rank_codes(codes, scales, nranks),
                                              rank_codes(peer_chunk_codes, peer_chunk_scales, nranks, rank),
                                              nranks, rank, n, chunk_codes, chunk_scales, out,
                                              out_t == LPC_BF16, stream));
}

lpc_status dda_flat_reduce(const void* const bufs[], int nranks, size_t n, void* out, hipStream_t stream) {
    if (bad_ranks(nranks)) return LPC_ERR_RANKS;
    if (n == 0) return LPC_OK;
    LPC_TRY(check_array(bufs, nranks));
    if (!out) return LPC_ERR_NULL;
    LPC_TRY(check_array_align(bufs, nranks));
    if (misaligned(out)) return LPC_ERR_ALIGN;
    if (n > LPC_MAX_ELEMS) return LPC_ERR_SHAPE;
    return hip_status(lpc::launch_dda_flat(rank_bufs(bufs, nranks), nranks, n, out, stream));
}

lpc_status dda_tree_reduce_scatter(const void* const bufs[], lpc_dtype t, int nranks, int rank, size_t n,
                                   void* out, hipStream_t stream) {
    if (bad_dtype(t)) return LPC_ERR_DTYPE;
    if (bad_ranks(nranks) || rank < 0 || rank >= nranks) return LPC_ERR_RANKS;
    if (n == 0) return LPC_OK;
    LPC_TRY(check_array(bufs, nranks));
    if (!out) return LPC_ERR_NULL;
    LPC_TRY(check_array_align(bufs, nranks));
    if (misaligned(out)) return LPC_ERR_ALIGN;
    if (n % ((size_t)8 * nranks) || n > LPC_MAX_ELEMS) return LPC_ERR_SHAPE;
    return hip_status(lpc::launch_dda_tree_rs(rank_bufs(bufs, nranks), t == LPC_BF16, nranks, rank, n, out,
                                              stream));
}

lpc_status dda_tree_allgather(const void* const chunks[], lpc_dtype t, int nranks, size_t n, void* out,
                              hipStream_t stream) {
    if (bad_dtype(t)) return LPC_ERR_DTYPE;
    if (bad_ranks(nranks)) return LPC_ERR_RANKS;
    if (n == 0) return LPC_OK;
    LPC_TRY(check_array(chunks, nranks));
    if (!out) return LPC_ERR_NULL;
    LPC_TRY(check_array_align(chunks, nranks));
    if (misaligned(out)) return LPC_ERR_ALIGN;
    if (n % ((size_t)8 * nranks) || n > LPC_MAX_ELEMS) return LPC_ERR_SHAPE;
    return hip_status(lpc::launch_dda_tree_ag(rank_bufs(chunks, nranks), t == LPC_BF16, nranks, n, out, stream));
}

lpc_status lpc_a2av_route(const int32_t* dest, size_t rows, int nranks, int32_t* counts, int32_t* offsets,
                          int32_t* perm, hipStream_t stream) {
    if (bad_ranks(nranks)) return LPC_ERR_RANKS;
    if (rows == 0) return LPC_OK;
    if (!dest || !counts || !offsets || !perm) return LPC_ERR_NULL;
    if (misaligned(dest) || misaligned(counts) || misaligned(offsets) || misaligned(perm)) return LPC_ERR_ALIGN;
    if (rows >= ((size_t)1 << 31)) return LPC_ERR_SHAPE;
    return hip_status(lpc::launch_a2av_route(dest, rows, nranks, counts, offsets, perm, stream));
}

lpc_status lpc_quantize_fp8_rows(const void* x, lpc_dtype in, size_t rows, size_t row_len, const int32_t* perm,
                                 uint8_t* codes, float* scales, hipStream_t stream) {
    if (bad_dtype(in)) return LPC_ERR_DTYPE;
    if (rows == 0 || row_len == 0) return LPC_OK;
    if (!x || !perm || !codes || !scales) return LPC_ERR_NULL;
    if (misaligned(x) || misaligned(perm) || misaligned(codes) || misaligned(scales)) return LPC_ERR_ALIGN;
    if (row_len % LPC_BLOCK || rows >= ((size_t)1 << 31) || row_len > LPC_MAX_ELEMS ||
        rows * row_len > LPC_MAX_ELEMS)
        return LPC_ERR_SHAPE;
    return hip_status(lpc::launch_quantize_rows(x, in == LPC_BF16, rows, row_len, perm, codes, scales, stream));
}

lpc_status lpc_dequantize_fp8(const uint8_t* codes, const float* scales, size_t n, void* out, lpc_dtype out_t,
                              hipStream_t stream) {
    if (bad_dtype(out_t)) return LPC_ERR_DTYPE;
    if (n == 0) return LPC_OK;
    if (!codes || !scales || !out) return LPC_ERR_NULL;
    if (misaligned(codes) || misaligned(scales) || misaligned(out)) return LPC_ERR_ALIGN;
    if (n % LPC_BLOCK || n > LPC_MAX_ELEMS) return LPC_ERR_SHAPE;
    return hip_status(lpc::launch_dequant(codes, scales, n, out, out_t == LPC_BF16, stream));
}

lpc_status lpc_e4m3_encode(const float* x, size_t n, uint8_t* codes, hipStream_t stream) {
    if (n == 0) return LPC_OK;
    if (!x || !codes) return LPC_ERR_NULL;
    if (misaligned(x) || misaligned(codes)) return LPC_ERR_ALIGN;
    if (n > LPC_MAX_ELEMS) return LPC_ERR_SHAPE;
    return hip_status(lpc::launch_encode(x, n, codes, stream));
}

}  // extern "C"
