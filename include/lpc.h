/*
 * lpc.h -- C ABI of the MI355X (gfx950) FP8 low-precision collective compute
 * library (liblpc.so).
 *
 * What the library computes is one GPU's share of the collectives described
 * on the RCCLX pages:
 *   - Meta Engineering RCCLX post (es copy, athrundataintelligence.com),
 *     section "Colectivos de mengua precisión": low-precision AllReduce,
 *     AllGather, AlltoAll and ReduceScatter; FP32 and BF16 data; FP8
 *     quantization for communication; FP32 compute; one quantization per
 *     collective, two for AllReduce.
 *   - dev.infolabhq.com "Meta open-sources RCCLX" (pt/es), sections on Direct
 *     Data Access (DDA flat: each rank reads every peer buffer and reduces
 *     locally; DDA tree: reduce-scatter then all-gather) and on low-precision
 *     collectives (FP8 compression up to 4:1, FP32 compute).
 *   - The same pages' Torchcomms quick-start: allreduce(t, SUM) is in place,
 *     on the current stream, and leaves the elementwise sum on every rank.
 *
 * The pages fix neither the FP8 format nor the block layout.  This library
 * uses: OCP FP8 E4M3FN (max 448, no infinities), round-to-nearest-even,
 * saturating; one FP32 scale s = absmax/448 per 128 contiguous elements;
 * code = E4M3(fl32(x / s)); value = fl32(E4M3(code) * s).  A block whose
 * scale is zero (all zeros, or an absmax so small that absmax/448 underflows)
 * has scale +0 and all codes 0x00.  Sums are FP32, in rank order 0..N-1,
 * multiply and add rounded separately.  With N ranks and n elements per
 * rank, rank r owns the chunk [r*C, (r+1)*C), C = n/N.
 *
 * Layout: a quantized buffer of n elements is two planar arrays, codes
 * uint8[n] and scales float[n/128]; element i uses scales[i/128].  bfloat16
 * data is passed as 16-bit patterns.
 *
 * Conventions for every call below:
 *   - All data pointers are DEVICE pointers; pointer arrays (codes[],
 *     scales[], bufs[], ...) are HOST arrays of nranks device pointers, read
 *     during the call and copied into kernel arguments.  The caller owns
 *     every buffer; the library allocates nothing and keeps no state, so
 *     calls are thread-safe.  The one exception is
 *     lpc_allreduce_emulated_noalloc, which works in a static device array
 *     of the library (see there).
 *   - Work is enqueued on `stream` (NULL: the default stream) and the call
 *     returns without waiting.
 *   - Arguments are checked on the host before anything is enqueued; on any
 *     status other than LPC_OK nothing was enqueued.  Checks, in order:
 *     dtype (LPC_ERR_DTYPE), 1 <= nranks <= 8 and 0 <= rank < nranks
 *     (LPC_ERR_RANKS), n == 0 (returns LPC_OK, no work), null pointers
 *     (LPC_ERR_NULL), 16-byte alignment of every pointer (LPC_ERR_ALIGN),
 *     shape (LPC_ERR_SHAPE).  A failed kernel launch gives LPC_ERR_HIP; a
 *     call that makes two launches (dda_flat_reduce with n odd, the
 *     emulated allreduce) may then leave the first one enqueued.
 *   - Inputs must be finite; NaN/Inf inputs give unspecified codes.  The
 *     FP32 rank-order sum of every element must be finite as well (for
 *     example |x| <= FLT_MAX / nranks everywhere): a block whose sum
 *     overflows has an infinite absmax, and its requantized codes and scale
 *     are unspecified.
 *   - Outputs must not overlap inputs unless a call says otherwise.
 *   - No call throws; every call is extern "C".
 */
#ifndef LPC_H
#define LPC_H

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

#define LPC_ABI_VERSION 1
#define LPC_BLOCK 128     /* elements per FP8 scale block */
#define LPC_MAX_RANKS 8   /* single node: the pages' low-precision collectives are tuned for one node */
#define LPC_FP8_MAX 448.0f

typedef enum {
    LPC_OK = 0,
    LPC_ERR_NULL = 1,   /* a required pointer is NULL */
    LPC_ERR_SHAPE = 2,  /* element count is not a whole number of blocks / chunks, or too large */
    LPC_ERR_RANKS = 3,  /* nranks outside 1..8, or rank outside 0..nranks-1 */
    LPC_ERR_DTYPE = 4,  /* unknown lpc_dtype */
    LPC_ERR_ALIGN = 5,  /* a pointer is not 16-byte aligned */
    LPC_ERR_HIP = 6,    /* the HIP runtime refused the kernel launch */
    LPC_ERR_SCRATCH = 7 /* the call needs more than the library's static scratch
                           (lpc_allreduce_emulated_noalloc only) */
} lpc_status;

typedef enum {
    LPC_F32 = 0,        /* IEEE binary32 */
    LPC_BF16 = 1        /* bfloat16 bit patterns (uint16) */
} lpc_dtype;

/* Largest element count accepted by any call: 2^32 elements (16 GiB of fp32).
 * A launch takes at most 2^31 - 1 lanes along a grid dimension: the kernels
 * give each lane 4 or more elements, except DDA flat and DDA tree's
 * reduce-scatter (one 32-bit word a lane), which near this size cap their grid
 * and let each lane take further words at the grid's stride.  Larger buffers
 * go in several calls. */
#define LPC_MAX_ELEMS ((size_t)1 << 32)

/* ---------------------------------------------------------------------- */
/* Low-precision AllReduce, one rank's steps                               */
/* ---------------------------------------------------------------------- */

/* (1) Quantize.  Blockwise FP8 quantization of one rank's buffer, the first
 * quantization of the low-precision collectives (RCCLX post, low-precision
 * section: FP8 for communication).
 *   x      [n] input of type `in` (LPC_F32 or LPC_BF16)
 *   codes  [n] output E4M3 codes;  scales [n/128] output FP32 scales
 *   n      elements; must be a multiple of 128 (else LPC_ERR_SHAPE)          */
lpc_status lpc_quantize_fp8(const void *x, lpc_dtype in, size_t n,
                            uint8_t *codes, float *scales, hipStream_t stream);

/* (2) Reduce-scatter step for the chunk owned by `rank`: read that chunk
 * from all nranks quantized buffers, dequantize, sum in FP32 in rank order,
 * and requantize the sum blockwise (the second quantization of AllReduce;
 * RCCLX post low-precision section; DDA tree's reduce-scatter phase on the
 * infolabhq pages).
 *   codes[p], scales[p]  rank p's whole quantized buffer ([n], [n/128])
 *   n            elements per rank; multiple of 128*nranks (else LPC_ERR_SHAPE)
 *   chunk_codes  [C] output codes;  chunk_scales [C/128] output scales        */
lpc_status lpc_reduce_scatter_chunk(const uint8_t *const codes[], const float *const scales[],
                                    int nranks, int rank, size_t n,
                                    uint8_t *chunk_codes, float *chunk_scales,
                                    hipStream_t stream);

/* (3) All-gather dequantization: out[p*C + i] = fl32(E4M3(chunk_codes[p][i])
 * * chunk_scales[p][i/128]), rounded to bf16 (nearest-even) when out_t is
 * LPC_BF16.  The owner's chunk is also taken from its requantized form, so
 * every rank ends with the same values.  This is the all-gather phase of the
 * two-phase allreduce (infolabhq pages, "Direct Data Access (DDA)" section,
 * DDA tree: reduce-scatter, then all-gather) carried out on the data of the
 * second quantization of a low-precision AllReduce (RCCLX post, es copy,
 * "Colectivos de mengua precisión": FP8 on the wire, FP32 compute, one or two
 * quantizations per collective).
 *   chunk_codes[p] [C], chunk_scales[p] [C/128]: rank p's requantized chunk
 *   n    elements of the output (= nranks*C); multiple of 128*nranks
 *   out  [n] of type out_t.  `out` may be the caller's original input buffer
 *        (in-place allreduce): it is not read.                               */
lpc_status lpc_allgather_dequant(const uint8_t *const chunk_codes[], const float *const chunk_scales[],
                                 int nranks, size_t n, void *out, lpc_dtype out_t,
                                 hipStream_t stream);

/* (2)+(3) in one launch: the reduce-scatter step for `rank`'s chunk (written
 * to chunk_codes/chunk_scales for the peers), its dequantization straight
 * from registers into out[rank*C ..], and the dequantization of the other
 * ranks' requantized chunks into the rest of `out`.  Results are
 * byte-identical to lpc_reduce_scatter_chunk followed by
 * lpc_allgather_dequant.  The operation is the low-precision AllReduce's two
 * phases after the first quantization, reduce-scatter with FP32 compute and
 * the second quantization, then all-gather (RCCLX post, es copy, "Colectivos
 * de mengua precisión"; the two phases as in infolabhq's "Direct Data Access
 * (DDA)" section, DDA tree).
 *   codes[], scales[]    as for lpc_reduce_scatter_chunk
 *   peer_chunk_codes[p], peer_chunk_scales[p]  rank p's requantized chunk
 *                        for p != rank ([rank] is ignored and may be NULL)
 *   out                  [n] of type out_t; may alias the caller's own
 *                        original input (not read), must not overlap any
 *                        code or scale array.                                 */
lpc_status lpc_rs_ag_fused(const uint8_t *const codes[], const float *const scales[],
                           int nranks, int rank, size_t n,
                           uint8_t *chunk_codes, float *chunk_scales,
                           const uint8_t *const peer_chunk_codes[],
                           const float *const peer_chunk_scales[],
                           void *out, lpc_dtype out_t, hipStream_t stream);

/* ---------------------------------------------------------------------- */
/* Low-precision ReduceScatter / AllGather (one quantization each)         */
/* ---------------------------------------------------------------------- */

/* Low-precision ReduceScatter: the reduce-scatter step without the second
 * quantization; the FP32 rank-order sum of `rank`'s chunk is the result,
 * written as float or rounded to bf16 (RCCLX post, low-precision section:
 * ReduceScatter, one quantization).
 *   out  [C] of type out_t, C = n/nranks.                                    */
lpc_status lpc_reduce_scatter(const uint8_t *const codes[], const float *const scales[],
                              int nranks, int rank, size_t n,
                              void *out, lpc_dtype out_t, hipStream_t stream);
/* Low-precision AllGather is lpc_quantize_fp8 on each rank's own chunk
 * followed by lpc_allgather_dequant over the N quantized chunks. */

/* ---------------------------------------------------------------------- */
/* DDA (unquantized)                                                        */
/* ---------------------------------------------------------------------- */

/* DDA flat local reduce (infolabhq pages, Direct Data Access section, DDA
 * flat): out[i] = bf16_rne(sum over p = 0..nranks-1, in order, of
 * f32(bufs[p][i])), FP32 accumulation.
 *   bufs[p]  [n] bfloat16 input of rank p;  out [n] bfloat16
 *   n        any element count (no block constraint).  One launch, or two
 *            when n is odd (the last element goes to a one-wavefront launch
 *            of its own).
 *   `out` must not alias any input (peers read the inputs concurrently).   */
lpc_status dda_flat_reduce(const void *const bufs[], int nranks, size_t n, void *out,
                           hipStream_t stream);

/* DDA tree, reduce-scatter phase, unquantized: out[i] = sum over p in rank
 * order of bufs[p][rank*C + i], FP32 accumulation, written in `t`
 * (infolabhq pages, "Direct Data Access (DDA)" section, DDA tree: the
 * allreduce split into reduce-scatter and all-gather, each phase reading the
 * peers' memory directly).
 *   bufs[p] [n] of type t;  out [C] of type t;  n multiple of 8*nranks.     */
lpc_status dda_tree_reduce_scatter(const void *const bufs[], lpc_dtype t, int nranks, int rank,
                                   size_t n, void *out, hipStream_t stream);

/* DDA tree, all-gather phase: out[p*C + i] = chunks[p][i] (a gather copy)
 * (infolabhq pages, "Direct Data Access (DDA)" section, DDA tree: the second
 * phase, every rank reading the peers' reduced chunks directly).
 *   chunks[p] [C] of type t;  out [n] of type t;  n multiple of 8*nranks.   */
lpc_status dda_tree_allgather(const void *const chunks[], lpc_dtype t, int nranks, size_t n,
                              void *out, hipStream_t stream);

/* ---------------------------------------------------------------------- */
/* Low-precision AlltoAll(v)                                                */
/* ---------------------------------------------------------------------- */

/* Routing for a variable all-to-all (RCCLX post: AllToAllvDynamic, a
 * GPU-resident collective): dest[k] in [0, nranks) is row k's destination.
 *   counts[d]  rows sent to d;  offsets[d]  exclusive prefix sum of counts
 *   perm[j]    source row of packed row j: destination-major, original row
 *              order kept within a destination (stable)
 * Rows with an out-of-range destination are dropped: they are not counted
 * and perm's tail past sum(counts) is filled with -1.
 *   rows < 2^31.  Each workgroup places one tile of rows and counts the
 *   whole of `dest` itself (no scratch memory), up to 128 workgroups.  */
lpc_status lpc_a2av_route(const int32_t *dest, size_t rows, int nranks,
                          int32_t *counts, int32_t *offsets, int32_t *perm,
                          hipStream_t stream);

/* Gather-and-quantize rows into the packed send buffer: packed row j is the
 * blockwise quantization of source row perm[j] of x (rows x row_len, row
 * major).  This is the one quantization of a low-precision AlltoAll (RCCLX
 * post, es copy, "Colectivos de mengua precisión": AlltoAll among the LP
 * collectives, FP8 on the wire), applied to the variable per-destination
 * row counts of AllToAllvDynamic (same post, introduction: CTran's
 * GPU-resident AllToAllvDynamic collective).  A perm entry outside [0, rows) gives an all-zero packed row
 * (codes 0, scales +0).
 *   codes [rows x row_len], scales [rows x row_len/128], packed order
 *   row_len multiple of 128 (else LPC_ERR_SHAPE).                             */
lpc_status lpc_quantize_fp8_rows(const void *x, lpc_dtype in, size_t rows, size_t row_len,
                                 const int32_t *perm, uint8_t *codes, float *scales,
                                 hipStream_t stream);

/* Dequantize a flat quantized buffer (e.g. received all-to-all rows):
 * out[i] = fl32(E4M3(codes[i]) * scales[i/128]) as float, or bf16 rounded.
 * The receive side of a low-precision AlltoAll: FP8 data back to FP32/BF16
 * for compute (RCCLX post, es copy, "Colectivos de mengua precisión").
 *   n multiple of 128.                                                        */
lpc_status lpc_dequantize_fp8(const uint8_t *codes, const float *scales, size_t n,
                              void *out, lpc_dtype out_t, hipStream_t stream);

/* ---------------------------------------------------------------------- */
/* Allreduce over emulated ranks, with algorithm selection                  */
/* ---------------------------------------------------------------------- */

/* Allreduce algorithms of the pages (infolabhq pages, Direct Data Access and
 * low-precision sections; RCCLX post, DDA and low-precision sections): DDA
 * flat for small messages, DDA tree (reduce-scatter + all-gather with direct
 * access) for slightly larger ones, low-precision FP8 for large messages when
 * enabled (the pages switch it on with an environment variable).          */
typedef enum {
    LPC_ALGO_AUTO = 0,           /* choose with lpc_select_algo */
    LPC_ALGO_DDA_FLAT = 1,       /* bf16 only */
    LPC_ALGO_DDA_TREE = 2,
    LPC_ALGO_LOW_PRECISION = 3
} lpc_algo;

/* Size thresholds of lpc_select_algo, in bytes per rank.  The pages give the
 * ordering (flat < tree < low precision) and the 16 MB floor of the
 * low-precision collectives, not the flat/tree boundary. */
#define LPC_DDA_FLAT_MAX_BYTES ((size_t)512 << 10)
#define LPC_LOW_PRECISION_MIN_BYTES ((size_t)16 << 20)

/* The algorithm an allreduce of n elements of type t per rank over nranks
 * ranks uses: LPC_ALGO_DDA_FLAT for bf16 up to LPC_DDA_FLAT_MAX_BYTES;
 * LPC_ALGO_LOW_PRECISION from LPC_LOW_PRECISION_MIN_BYTES when
 * low_precision_enabled != 0 and n is a multiple of 128*nranks;
 * LPC_ALGO_DDA_TREE otherwise when n is a multiple of 8*nranks; else
 * LPC_ALGO_DDA_FLAT for bf16.  Returns LPC_ALGO_AUTO when no algorithm
 * applies (bad arguments, or fp32 with n not a multiple of 8*nranks).
 * Pure function of its arguments, no HIP call.                              */
lpc_algo lpc_select_algo(int nranks, size_t n, lpc_dtype t, int low_precision_enabled);

/* Device workspace lpc_allreduce_emulated needs for (algo, nranks, n, t):
 *   DDA flat:       nranks outputs of n elements
 *   DDA tree:       nranks reduced chunks of n/nranks elements
 *   low precision:  nranks quantized buffers (n codes + n/128 scales) and
 *                   nranks requantized chunks, each region 256-byte aligned
 * Writes the byte count to *bytes.  Errors as for lpc_allreduce_emulated,
 * checked without HIP calls; LPC_ALGO_AUTO is LPC_ERR_DTYPE here.          */
lpc_status lpc_allreduce_workspace_bytes(lpc_algo algo, int nranks, size_t n, lpc_dtype t, size_t *bytes);

/* In-place allreduce (SUM) over nranks emulated ranks on one GPU: every
 * bufs[r] ends with the elementwise sum over ranks, as the pages' Torchcomms
 * allreduce(t, SUM) leaves it on every rank.  Each rank's share runs as that
 * rank would run it, with the other ranks' buffers as its peers; the ranks'
 * shares of one step go in one launch (the rank is a grid dimension):
 *   DDA flat:      every rank's dda_flat_reduce into its workspace output,
 *                  then each output is copied into that rank's buffer;
 *   DDA tree:      every rank's dda_tree_reduce_scatter into the workspace,
 *                  then every rank's dda_tree_allgather into its buffer;
 *   low precision: every rank's lpc_quantize_fp8, every rank's
 *                  lpc_reduce_scatter_chunk, then every rank's
 *                  lpc_allgather_dequant into its buffer (two quantizations).
 * Results are those of the per-rank entry points, bit for bit.
 *   bufs[r]    [n] of type t, device; distinct, non-overlapping
 *   algo       not LPC_ALGO_AUTO (LPC_ERR_DTYPE); LPC_ALGO_DDA_FLAT needs
 *              bf16 (LPC_ERR_DTYPE); shapes as the entry points it calls
 *   workspace  device, 16-byte aligned, at least the bytes
 *              lpc_allreduce_workspace_bytes gives (else LPC_ERR_SHAPE)
 * The work is enqueued on `stream`.  A validation error enqueues nothing; a
 * refused launch (LPC_ERR_HIP) may leave the steps before it enqueued.     */
lpc_status lpc_allreduce_emulated(void *const bufs[], int nranks, size_t n, lpc_dtype t, lpc_algo algo,
                                  void *workspace, size_t workspace_bytes, hipStream_t stream);

/* Size of the static device scratch of lpc_allreduce_emulated_noalloc (one
 * copy per GPU the library runs on, held until the process ends). */
#define LPC_NOALLOC_SCRATCH_BYTES ((size_t)64 << 20)

/* lpc_allreduce_emulated for callers that cannot allocate device memory:
 * code under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc.  Same arguments, checks, kernels and results, but no workspace
 * argument: the workspace is a file-scope device array of
 * LPC_NOALLOC_SCRATCH_BYTES bytes inside the library.  The call allocates
 * nothing (no hipMalloc/hipFree); its first call on a device looks up that
 * device's copy of the array (hipGetSymbolAddress), later calls reuse it.
 *   - The array belongs to the CURRENT device (hipGetDevice); `stream` must
 *     be a stream of that device.
 *   - A workspace need (lpc_allreduce_workspace_bytes) above
 *     LPC_NOALLOC_SCRATCH_BYTES returns LPC_ERR_SCRATCH, after the other
 *     argument checks and before any HIP call.  At 8 ranks that allows a
 *     low-precision allreduce of up to about 7.2M elements per rank, a DDA
 *     tree of up to 8M fp32 (16M bf16) elements per rank, and DDA flat of up
 *     to 4M bf16 elements per rank.
 *   - Every call on one GPU shares that GPU's array, and the array keeps the
 *     last call's contents.  Calls that overlap on one GPU (concurrent
 *     streams, or threads) race on it: the caller must order them.  Nothing
 *     in the array needs to start at zero (every byte is written before it
 *     is read), so the call clears nothing.
 * Errors: as lpc_allreduce_emulated (no workspace checks), plus
 * LPC_ERR_SCRATCH; LPC_ERR_HIP also when the device or the array's address
 * cannot be obtained. */
lpc_status lpc_allreduce_emulated_noalloc(void *const bufs[], int nranks, size_t n, lpc_dtype t,
                                          lpc_algo algo, hipStream_t stream);

/* ---------------------------------------------------------------------- */
/* Codec and library info                                                   */
/* ---------------------------------------------------------------------- */

/* Raw codec: codes[i] = E4M3 of the already-scaled value x[i], nearest-even,
 * saturating at +-448, sign kept (the conversion every quantizing kernel
 * applies to fl32(x / s)).  It is the FP8 encoding of the low-precision
 * collectives (RCCLX post, es copy, "Colectivos de mengua precisión", where
 * the range of FP8 decides what is representable); the pages name no FP8
 * variant, and this library reads it as OCP E4M3FN.  n: any count.          */
lpc_status lpc_e4m3_encode(const float *x, size_t n, uint8_t *codes, hipStream_t stream);

/* Human-readable name of a status code (static storage). */
const char *lpc_status_string(lpc_status status);

/* LPC_ABI_VERSION of the built library. */
int lpc_abi_version(void);

#ifdef __cplusplus
}
#endif

#endif /* LPC_H */
