// lpc_launch.hpp -- launchers between the C ABI layer (lpc_api.hip) and the
// kernels (lpc_kernels.hip).  Internal to liblpc.so.  Each launcher enqueues
// one kernel on `stream` and returns the status of that launch; arguments
// have already been validated by the caller.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "lpc_device.hpp"

namespace lpc {

hipError_t launch_quantize(const void* x, int in_bf16, size_t n, uint8_t* codes, float* scales,
                           hipStream_t stream);
hipError_t launch_reduce_scatter_chunk(const RankCodes& in, int nranks, int rank, size_t n, uint8_t* cc,
                                       float* cs, hipStream_t stream);
hipError_t launch_reduce_scatter_out(const RankCodes& in, int nranks, int rank, size_t n, void* out,
                                     int out_bf16, hipStream_t stream);
hipError_t launch_allgather(const RankCodes& chunks, int nranks, size_t n, void* out, int out_bf16,
                            hipStream_t stream);
hipError_t launch_rs_ag_fused(const RankCodes& in, const RankCodes& peers, int nranks, int rank, size_t n,
                              uint8_t* cc, float* cs, void* out, int out_bf16, hipStream_t stream);
hipError_t launch_dequant(const uint8_t* codes, const float* scales, size_t n, void* out, int out_bf16,
                          hipStream_t stream);
hipError_t launch_dda_flat(const RankBufs& b, int nranks, size_t n, void* out, hipStream_t stream);
hipError_t launch_dda_tree_rs(const RankBufs& b, int bf16, int nranks, int rank, size_t n, void* out,
                              hipStream_t stream);
hipError_t launch_dda_tree_ag(const RankBufs& chunks, int bf16, int nranks, size_t n, void* out,
                              hipStream_t stream);
hipError_t launch_a2av_route(const int32_t* dest, size_t rows, int nranks, int32_t* counts, int32_t* offsets,
                             int32_t* perm, hipStream_t stream);
hipError_t launch_quantize_rows(const void* x, int in_bf16, size_t rows, size_t row_len, const int32_t* perm,
                                uint8_t* codes, float* scales, hipStream_t stream);
hipError_t launch_encode(const float* x, size_t n, uint8_t* codes, hipStream_t stream);

// every rank's share of one step in a single launch (emulated collectives)
hipError_t launch_quantize_ranks(const RankBufs& x, int in_bf16, int nranks, size_t n, const RankQuant& q,
                                 hipStream_t stream);
hipError_t launch_reduce_scatter_ranks(const RankCodes& in, int nranks, size_t n, const RankQuant& chunks,
                                       hipStream_t stream);
hipError_t launch_allgather_ranks(const RankCodes& chunks, int nranks, size_t n, const RankOut& outs, int out_bf16,
                                  hipStream_t stream);
hipError_t launch_dda_flat_ranks(const RankBufs& b, int nranks, size_t n, const RankOut& outs, hipStream_t stream);
hipError_t launch_dda_tree_rs_ranks(const RankBufs& b, int bf16, int nranks, size_t n, const RankOut& chunks,
                                    hipStream_t stream);
hipError_t launch_dda_tree_ag_ranks(const RankBufs& chunks, int bf16, int nranks, size_t n, const RankOut& outs,
                                    hipStream_t stream);
hipError_t launch_copy_ranks(const RankBufs& src, int nranks, size_t bytes, const RankOut& dst, hipStream_t stream);

}  // namespace lpc
