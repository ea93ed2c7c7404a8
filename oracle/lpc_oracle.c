/*
 * lpc_oracle.c -- CPU oracle for the FP8 low-precision collective compute path.
 *
 * TEST INFRASTRUCTURE ONLY.  This file is the slow, plain, obviously-correct
 * statement of what the GPU library computes.  Only the test suite, the smoke
 * check and the benchmark's CPU-baseline leg may load or call it; the product
 * path never does.  It shares no source, header, table or helper with the HIP
 * library, and it includes nothing from it.
 *
 * Build: gcc -O2 -std=c11 -ffp-contract=off -fno-fast-math -fPIC -shared
 * (x86-64 SSE arithmetic: every float operation below is one IEEE binary32
 * operation rounded to nearest-even; no fused multiply-add, no flush to zero).
 *
 * Sources for what is computed (the web pages about RCCLX):
 *  - Meta Engineering RCCLX post, Spanish copy (athrundataintelligence.com),
 *    section "Colectivos de mengua precisión" (low-precision collectives):
 *    AllReduce / AllGather / AlltoAll / ReduceScatter with FP8-quantized
 *    communication for FP32 and BF16 data, compute steps kept in FP32,
 *    precision loss set by how many quantizations a collective applies.
 *  - dev.infolabhq.com "Meta open-sources RCCLX" (pt and es), section on
 *    low-precision collectives: FP8 compression up to 4:1 with FP32 compute;
 *    section on Direct Data Access: DDA flat (every rank loads all peers'
 *    buffers and reduces locally) and DDA tree (reduce-scatter + all-gather).
 * The pages give no FP8 variant, block size, scale rule or summation order.
 * Where they are silent this oracle takes these readings: OCP FP8 E4M3FN,
 * round-to-nearest-even, saturating at +-448, one FP32 scale
 * s = absmax/448 per 128 contiguous elements, FP32 sums in rank order
 * 0..N-1, the owned chunk of rank r is elements [r*C, (r+1)*C), C = n/N.
 *
 * Parity pins: every function here is checked, in the CPU test suite, against
 * something other than itself (torch's CPU float8/bfloat16 casts, closed
 * forms, exactness families, brute force and error bounds).  See the tests
 * named test_oracle_*.py.
 */
#include <math.h>
#include <stddef.h>
#include <stdint.h>
#include <string.h>

#define LPO_BLOCK 128
#define LPO_FP8_MAX 448.0f

/* ------------------------------------------------------------------------ */
/* OCP FP8 E4M3FN codec                                                     */
/* ------------------------------------------------------------------------ */

/* Decode one E4M3FN code: 1 sign bit, 4 exponent bits (bias 7), 3 mantissa
 * bits, no infinities, S.1111.111 is NaN.  Exponent field 0 is subnormal with
 * value m * 2^-9.  Every finite code is exact in binary32. */
float lpo_e4m3_decode(uint8_t c)
{
    int sign = (c >> 7) & 1;
    int e = (c >> 3) & 0xF;
    int m = c & 0x7;
    float v;
    if ((c & 0x7F) == 0x7F)
        return NAN;
    if (e == 0)
        v = ldexpf((float)m, -9);
    else
        v = ldexpf((float)(8 + m), e - 10);
    return sign ? -v : v;
}

/* The 127 non-negative finite values, ascending (codes 0x00..0x7E), taken
 * from the decoder above on first use. */
static float pos_table[0x7F];
static int pos_table_ready;

static float pos_value(int k)
{
    if (!pos_table_ready) {
        int j;
        for (j = 0; j < 0x7F; j++)
            pos_table[j] = lpo_e4m3_decode((uint8_t)j);
        pos_table_ready = 1;
    }
    return pos_table[k];
}

/* Encode a finite float: pick the nearest of the non-negative finite E4M3
 * values to |v|; on an exact tie between two neighbours take the one with the
 * even code; |v| >= 448 saturates to 448 (code 0x7E).  The sign bit of v is
 * copied into the code, so -0 and negative values that round to zero give
 * 0x80.  NaN input is outside the domain (returns the NaN code 0x7F). */
uint8_t lpo_e4m3_encode(float v)
{
    uint8_t sign = signbit(v) ? 0x80 : 0x00;
    float a = fabsf(v);
    int k;
    if (isnan(v))
        return 0x7F;
    if (a >= LPO_FP8_MAX)
        return (uint8_t)(sign | 0x7E);
    /* find k with value(k) <= a < value(k+1) by a plain scan */
    k = 0;
    while (k < 0x7E && !(a < pos_value(k + 1)))
        k++;
    {
        /* midpoint of two neighbours has <= 5 significant bits: exact */
        double lo = pos_value(k), hi = pos_value(k + 1);
        double mid = (lo + hi) / 2.0;
        double ad = a;
        int pick;
        if (ad < mid)
            pick = k;
        else if (ad > mid)
            pick = k + 1;
        else
            pick = (k % 2 == 0) ? k : k + 1;
        return (uint8_t)(sign | pick);
    }
}

/* ------------------------------------------------------------------------ */
/* bfloat16                                                                 */
/* ------------------------------------------------------------------------ */

float lpo_bf16_to_f32(uint16_t h)
{
    uint32_t u = (uint32_t)h << 16;
    float f;
    memcpy(&f, &u, 4);
    return f;
}

/* Round a finite float to the nearest bfloat16 (8 significant bits), ties to
 * the even bit pattern.  Written as: truncate to the two neighbouring bf16
 * patterns and compare the discarded 16 bits with the halfway value 0x8000.
 * NaN maps to the quiet NaN 0x7FC0 (with the input's sign). */
uint16_t lpo_bf16_rne(float f)
{
    uint32_t u;
    uint32_t down, rest;
    memcpy(&u, &f, 4);
    if (isnan(f))
        return (uint16_t)(((u >> 16) & 0x8000) | 0x7FC0);
    down = u >> 16;     /* truncated pattern (toward zero in magnitude) */
    rest = u & 0xFFFF;  /* discarded bits */
    if (rest > 0x8000 || (rest == 0x8000 && (down & 1)))
        down += 1;      /* magnitude rounds up; carries into the exponent */
    return (uint16_t)down;
}

/* ------------------------------------------------------------------------ */
/* Blockwise quantization                                                   */
/* ------------------------------------------------------------------------ */

/* One block of LPO_BLOCK floats: absmax, FP32 scale absmax/448, codes of
 * fl32(x/s).  A block whose scale is zero (all zeros, or absmax so small that
 * absmax/448 underflows) is stored as scale +0 and all codes 0x00. */
static void quantize_block(const float *x, uint8_t *codes, float *scale)
{
    float amax = 0.0f, s;
    int i;
    for (i = 0; i < LPO_BLOCK; i++) {
        float a = fabsf(x[i]);
        if (a > amax)
            amax = a;
    }
    s = amax / LPO_FP8_MAX;
    if (s == 0.0f) {
        *scale = 0.0f;
        memset(codes, 0, LPO_BLOCK);
        return;
    }
    *scale = s;
    for (i = 0; i < LPO_BLOCK; i++) {
        float q = x[i] / s;
        codes[i] = lpo_e4m3_encode(q);
    }
}

/* x: n floats (n % 128 == 0) -> codes[n], scales[n/128].  Returns 0, or -1
 * if n is not a whole number of blocks. */
int lpo_quantize_f32(const float *x, size_t n, uint8_t *codes, float *scales)
{
    size_t b;
    if (n % LPO_BLOCK)
        return -1;
    for (b = 0; b < n / LPO_BLOCK; b++)
        quantize_block(x + b * LPO_BLOCK, codes + b * LPO_BLOCK, scales + b);
    return 0;
}

/* Same for bfloat16 input, widened exactly to float first. */
int lpo_quantize_bf16(const uint16_t *x, size_t n, uint8_t *codes, float *scales)
{
    float tmp[LPO_BLOCK];
    size_t b;
    int i;
    if (n % LPO_BLOCK)
        return -1;
    for (b = 0; b < n / LPO_BLOCK; b++) {
        for (i = 0; i < LPO_BLOCK; i++)
            tmp[i] = lpo_bf16_to_f32(x[b * LPO_BLOCK + i]);
        quantize_block(tmp, codes + b * LPO_BLOCK, scales + b);
    }
    return 0;
}

/* Dequantize: out[i] = fl32(dec(code[i]) * scale[i/128]). */
int lpo_dequantize_f32(const uint8_t *codes, const float *scales, size_t n, float *out)
{
    size_t i;
    if (n % LPO_BLOCK)
        return -1;
    for (i = 0; i < n; i++)
        out[i] = lpo_e4m3_decode(codes[i]) * scales[i / LPO_BLOCK];
    return 0;
}

/* Dequantize to bfloat16: bf16_rne(fl32(dec * scale)). */
int lpo_dequantize_bf16(const uint8_t *codes, const float *scales, size_t n, uint16_t *out)
{
    size_t i;
    if (n % LPO_BLOCK)
        return -1;
    for (i = 0; i < n; i++)
        out[i] = lpo_bf16_rne(lpo_e4m3_decode(codes[i]) * scales[i / LPO_BLOCK]);
    return 0;
}

/* ------------------------------------------------------------------------ */
/* Low-precision allreduce, one step at a time                              */
/* ------------------------------------------------------------------------ */

/* Reduce-scatter step for the chunk owned by rank r: for each element of
 * [r*C, (r+1)*C), dequantize it from every rank and sum in FP32 in rank order
 * (acc = d_0, then acc = acc + d_p for p = 1..N-1, multiply and add rounded
 * separately), then requantize the summed chunk blockwise.
 * codes[p], scales[p]: rank p's full quantized buffer (n elements).
 * chunk_codes[C], chunk_scales[C/128]: the requantized owned chunk.
 * Returns -1 on a shape error (n % (128*N) != 0, N < 1, r out of range). */
int lpo_reduce_scatter_chunk(const uint8_t *const *codes, const float *const *scales,
                             int nranks, int rank, size_t n,
                             uint8_t *chunk_codes, float *chunk_scales)
{
    size_t C, b, i;
    int p;
    float acc[LPO_BLOCK];
    if (nranks < 1 || rank < 0 || rank >= nranks)
        return -1;
    if (n % ((size_t)LPO_BLOCK * (size_t)nranks))
        return -1;
    C = n / (size_t)nranks;
    for (b = 0; b < C / LPO_BLOCK; b++) {
        size_t base = (size_t)rank * C + b * LPO_BLOCK;   /* first element, rank-buffer index */
        size_t gblk = base / LPO_BLOCK;                    /* its block in the rank buffer */
        for (i = 0; i < LPO_BLOCK; i++) {
            acc[i] = lpo_e4m3_decode(codes[0][base + i]) * scales[0][gblk];
            for (p = 1; p < nranks; p++) {
                float d = lpo_e4m3_decode(codes[p][base + i]) * scales[p][gblk];
                acc[i] = acc[i] + d;
            }
        }
        quantize_block(acc, chunk_codes + b * LPO_BLOCK, chunk_scales + b);
    }
    return 0;
}

/* All-gather step: rank p's requantized chunk is chunk_codes[p] (C codes) and
 * chunk_scales[p] (C/128 scales); the output is their dequantization laid out
 * chunk after chunk, out[p*C + i].  The owning rank also takes its own chunk
 * from the requantized form, so every rank ends with identical values.
 * out_bf16 = 0: float output; 1: bfloat16 output (uint16 patterns). */
int lpo_allgather_dequant(const uint8_t *const *chunk_codes, const float *const *chunk_scales,
                          int nranks, size_t n, void *out, int out_bf16)
{
    size_t C, i;
    int p;
    if (nranks < 1 || n % ((size_t)LPO_BLOCK * (size_t)nranks))
        return -1;
    C = n / (size_t)nranks;
    for (p = 0; p < nranks; p++) {
        for (i = 0; i < C; i++) {
            float v = lpo_e4m3_decode(chunk_codes[p][i]) * chunk_scales[p][i / LPO_BLOCK];
            if (out_bf16)
                ((uint16_t *)out)[(size_t)p * C + i] = lpo_bf16_rne(v);
            else
                ((float *)out)[(size_t)p * C + i] = v;
        }
    }
    return 0;
}

/* ------------------------------------------------------------------------ */
/* Standalone reduce-scatter (one quantization)                             */
/* ------------------------------------------------------------------------ */

/* Low-precision ReduceScatter: as the reduce-scatter step above, but the
 * FP32 sum is the result (no second quantization), written as float or as
 * bfloat16.  out holds C = n/N elements. */
int lpo_reduce_scatter_out(const uint8_t *const *codes, const float *const *scales,
                           int nranks, int rank, size_t n, void *out, int out_bf16)
{
    size_t C, i;
    int p;
    if (nranks < 1 || rank < 0 || rank >= nranks)
        return -1;
    if (n % ((size_t)LPO_BLOCK * (size_t)nranks))
        return -1;
    C = n / (size_t)nranks;
    for (i = 0; i < C; i++) {
        size_t e = (size_t)rank * C + i;
        float acc = lpo_e4m3_decode(codes[0][e]) * scales[0][e / LPO_BLOCK];
        for (p = 1; p < nranks; p++) {
            float d = lpo_e4m3_decode(codes[p][e]) * scales[p][e / LPO_BLOCK];
            acc = acc + d;
        }
        if (out_bf16)
            ((uint16_t *)out)[i] = lpo_bf16_rne(acc);
        else
            ((float *)out)[i] = acc;
    }
    return 0;
}

/* ------------------------------------------------------------------------ */
/* DDA flat local reduce                                                    */
/* ------------------------------------------------------------------------ */

/* Every rank reads all N peers' bfloat16 buffers and reduces locally:
 * acc = f32(x_0[i]); acc = acc + f32(x_p[i]) for p = 1..N-1; out = bf16_rne.
 * (dev.infolabhq.com, section on Direct Data Access: DDA flat.) */
int lpo_dda_flat_bf16(const uint16_t *const *bufs, int nranks, size_t n, uint16_t *out)
{
    size_t i;
    int p;
    if (nranks < 1)
        return -1;
    for (i = 0; i < n; i++) {
        float acc = lpo_bf16_to_f32(bufs[0][i]);
        for (p = 1; p < nranks; p++)
            acc = acc + lpo_bf16_to_f32(bufs[p][i]);
        out[i] = lpo_bf16_rne(acc);
    }
    return 0;
}

/* Unquantized reduce-scatter + all-gather (DDA tree) for float data: the sum
 * of chunk r over ranks in rank order.  Same as DDA flat restricted to the
 * owned chunk; the all-gather part is a plain copy.  bf16 = 1 for bfloat16
 * buffers (sum in FP32, rounded once). */
int lpo_dda_tree_rs(const void *const *bufs, int bf16, int nranks, int rank, size_t n, void *out)
{
    size_t C, i;
    int p;
    if (nranks < 1 || rank < 0 || rank >= nranks || n % (size_t)nranks)
        return -1;
    C = n / (size_t)nranks;
    for (i = 0; i < C; i++) {
        size_t e = (size_t)rank * C + i;
        float acc;
        if (bf16) {
            acc = lpo_bf16_to_f32(((const uint16_t *)bufs[0])[e]);
            for (p = 1; p < nranks; p++)
                acc = acc + lpo_bf16_to_f32(((const uint16_t *)bufs[p])[e]);
            ((uint16_t *)out)[i] = lpo_bf16_rne(acc);
        } else {
            acc = ((const float *)bufs[0])[e];
            for (p = 1; p < nranks; p++)
                acc = acc + ((const float *)bufs[p])[e];
            ((float *)out)[i] = acc;
        }
    }
    return 0;
}

/* ------------------------------------------------------------------------ */
/* All-to-all-v: routing and per-row quantization                           */
/* ------------------------------------------------------------------------ */

/* Routing for a variable all-to-all: dest[k] in [0, N) is the destination of
 * row k.  counts[d] = rows going to d; offsets[d] = exclusive prefix sum of
 * counts; perm lists the source rows destination-major, keeping the original
 * row order inside each destination (a stable sort by destination).
 * Returns -1 if some dest is out of range. */
int lpo_a2av_route(const int32_t *dest, size_t rows, int nranks,
                   int32_t *counts, int32_t *offsets, int32_t *perm)
{
    size_t k;
    int d;
    size_t pos;
    if (nranks < 1)
        return -1;
    for (d = 0; d < nranks; d++)
        counts[d] = 0;
    for (k = 0; k < rows; k++) {
        if (dest[k] < 0 || dest[k] >= nranks)
            return -1;
        counts[dest[k]]++;
    }
    pos = 0;
    for (d = 0; d < nranks; d++) {
        offsets[d] = (int32_t)pos;
        pos += (size_t)counts[d];
    }
    /* stable: for each destination in turn, walk rows in order */
    pos = 0;
    for (d = 0; d < nranks; d++)
        for (k = 0; k < rows; k++)
            if (dest[k] == d)
                perm[pos++] = (int32_t)k;
    return 0;
}

/* Packed row k of the send buffer is the blockwise quantization of source
 * row perm[k].  x: rows x row_len (row_len % 128 == 0); bf16 selects the
 * input type (0 float, 1 bfloat16).  codes: rows x row_len, scales:
 * rows x row_len/128, both in packed (destination-major) row order. */
int lpo_quantize_rows(const void *x, int bf16, size_t rows, size_t row_len,
                      const int32_t *perm, uint8_t *codes, float *scales)
{
    size_t k;
    if (row_len % LPO_BLOCK)
        return -1;
    for (k = 0; k < rows; k++) {
        size_t src = (size_t)perm[k];
        if (perm[k] < 0 || src >= rows)
            return -1;
        if (bf16)
            lpo_quantize_bf16((const uint16_t *)x + src * row_len, row_len,
                              codes + k * row_len, scales + k * (row_len / LPO_BLOCK));
        else
            lpo_quantize_f32((const float *)x + src * row_len, row_len,
                             codes + k * row_len, scales + k * (row_len / LPO_BLOCK));
    }
    return 0;
}

/* ------------------------------------------------------------------------ */
/* Array helpers for the test loader                                        */
/* ------------------------------------------------------------------------ */

void lpo_e4m3_decode_array(const uint8_t *c, size_t n, float *out)
{
    size_t i;
    for (i = 0; i < n; i++)
        out[i] = lpo_e4m3_decode(c[i]);
}

void lpo_e4m3_encode_array(const float *v, size_t n, uint8_t *out)
{
    size_t i;
    for (i = 0; i < n; i++)
        out[i] = lpo_e4m3_encode(v[i]);
}

void lpo_bf16_rne_array(const float *v, size_t n, uint16_t *out)
{
    size_t i;
    for (i = 0; i < n; i++)
        out[i] = lpo_bf16_rne(v[i]);
}
