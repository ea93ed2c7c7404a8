/*
 * lpc_measure.h -- reference kernels for measuring liblpc.so's kernels
 * (exported by the same library).  They compute nothing of the collectives.
 *
 * The RCCLX pages measure their collectives with param-bench rccl-tests:
 * warm-up iterations, then the mean over the measured iterations (Meta
 * Engineering RCCLX post, es copy, section "Colectivos de mengua precisión",
 * last paragraph).  These two calls give that measurement its two reference
 * points on the GPU the library runs on:
 *   - lpc_measure_stream: the time a plain streaming kernel needs for the
 *     same bytes at the same read:write mix as a path kernel (the practical
 *     ceiling that kernel is held against, beside the HBM peak);
 *   - lpc_measure_empty: the time an empty launch of a given shape takes
 *     (the fixed cost a launch pays before it moves a byte).
 * Conventions as in lpc.h: device pointers, work enqueued on `stream`,
 * arguments checked on the host first (nothing enqueued on an error),
 * LPC_ERR_HIP when the launch is refused.
 */
#ifndef LPC_MEASURE_H
#define LPC_MEASURE_H

#include <stddef.h>

#include "lpc.h"

#ifdef __cplusplus
extern "C" {
#endif

/* Plain streaming kernel: reads read_bytes from src and writes write_bytes
 * to dst (the written values depend on the read ones; their content is
 * otherwise unspecified).  16-byte non-temporal loads and stores, every
 * wavefront instruction covering one contiguous KiB, tiles in the XCD-aware
 * order of the library's kernels.  A lane makes up to K loads, then up to K
 * stores, at a stride of the grid's lane count.  No single grid is fastest
 * for every size on cold HBM, so the grid is a parameter:
 *   per_lane == 0: one round of resident wavefronts (2,048 workgroups of 256
 *     lanes) or fewer, K <= 8 (larger transfers: more workgroups, K = 8);
 *     fastest of those tried up to tens of MB;
 *   per_lane == 1, 2, 4 or 8: K = per_lane and as many workgroups as that
 *     needs; one of these was fastest at hundreds of MB.
 *   src  [read_bytes], device, 16-byte aligned (may be NULL if read_bytes is 0)
 *   dst  [write_bytes], device, 16-byte aligned, must not overlap src.  With
 *        write_bytes == 0 it must still point to 16 valid bytes, which are not
 *        written (the kernel's store to it sits under a flag that is always off,
 *        which keeps the loads live)
 *   read_bytes, write_bytes  multiples of 16; per_lane one of 0, 1, 2, 4, 8
 *        (else LPC_ERR_SHAPE); both sizes 0 is a no-op */
lpc_status lpc_measure_stream(const void *src, size_t read_bytes, void *dst, size_t write_bytes, int per_lane,
                              hipStream_t stream);

/* Empty launch: grid_x x grid_y workgroups of `threads` lanes whose kernel
 * argument block is kernarg_bytes rounded up to 16, 64, 128, 256, 320 or 512
 * bytes (plus the grid size the runtime appends).  Every wavefront loads the
 * whole block and writes nothing.  At thousands of wavefronts the launch's
 * time grows with the argument bytes each wavefront loads (the scalar loads'
 * return bandwidth), so to match a kernel give the bytes one of its
 * wavefronts loads, not the size of its whole argument block.
 *   grid_x, grid_y >= 1; 1 <= threads <= 1024; kernarg_bytes <= 512 (else LPC_ERR_SHAPE)
 *   sink  a valid device pointer to at least 4 bytes, 16-byte aligned; never written */
lpc_status lpc_measure_empty(unsigned grid_x, unsigned grid_y, unsigned threads, size_t kernarg_bytes,
                             int *sink, hipStream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* LPC_MEASURE_H */
