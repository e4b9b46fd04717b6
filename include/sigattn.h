/*
 * libsigattn — bidirectional sigmoid attention on padded variable-length
 * batches, for AMD Instinct MI355X (gfx950).
 *
 * What it computes.  For every sequence b and head h, on the valid rows
 * 0..n_b-1 (right padding):
 *
 *     X = Q K^T / sqrt(d) + b_b          scores, n_b x n_b
 *     P = sigma(X),  sigma(x) = 1/(1 + e^-x)   elementwise, no row normalisation
 *     O = P V
 *
 * ("Better Models, Faster Training: Sigmoid Attention for single-cell
 * Foundation Models", technical summary §2A: the SigmoidAttn formula and the
 * bias b = -log(n).)  By default there is no causal mask: the paper's models
 * are bidirectional (its abstract); args->mask selects the causal variant
 * (sigattn_mask).  The backward follows from the diagonal
 * Jacobian of §2B: with dP = dO V^T and dX = dP * P * (1 - P),
 *
 *     dQ = dX K / sqrt(d),   dK = dX^T Q / sqrt(d),   dV = P^T dO.
 *
 * As in §2C of the same summary, the forward is one fused pass and the
 * backward is split in two calls — one for dQ, one for dK and dV — so that no
 * output row has more than one writer and no atomics are needed; P is
 * recomputed, never stored.  Tiles that lie entirely in padding (query side or
 * key side) are never computed.
 *
 * Readings taken where the pages are silent: n in -log(n) is the sequence's
 * own valid length (other conventions selectable through bias_mode); log is
 * the natural log; d is the head dimension; padded output rows are written as
 * zero; a sequence with n_b = 0 produces all-zero outputs.
 *
 * Tensors.  Q, K, V, dO, O, dQ, dK, dV are device pointers to bf16 arrays
 * (or fp16, args->dtype) seen as [B, H, Lmax, d], 16-byte aligned.  By default each is contiguous
 * (row-major: d fastest); with args->strides each tensor argument may be any
 * strided view whose head dimension is contiguous (for example [B, Lmax, H, d]
 * activations, or the q/k/v slices of a fused QKV projection), so a caller
 * needs no transposes or copies.  The caller owns every buffer; the library
 * allocates no device or pinned memory and keeps no state between calls.
 * Rows n_b..Lmax-1 of the inputs may hold any bit pattern (including
 * NaN/Inf): they are never read.
 *
 * Streams and errors.  Every call validates all arguments on the host before
 * it enqueues anything, so a call that returns an error has no side effect.
 * On success the work is enqueued on args->stream (NULL: the default stream)
 * and the call returns; results are valid once the stream has reached that
 * point.  The dQ call and the dK/dV call are independent of each other and may
 * run on different streams.  Every output is fully overwritten.  The library
 * never prints and never aborts.
 */
#ifndef SIGATTN_H
#define SIGATTN_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum sigattn_status {
  SIGATTN_OK = 0,
  SIGATTN_ERR_NULL = 1,      /* args, a tensor pointer, seqlens, or (bias mode 3)
                                head_bias is NULL                                       */
  SIGATTN_ERR_SHAPE = 2,     /* B, H or Lmax < 1, d not 64 or 128, sizes overflow, or
                                (Lmax + 256) * d * 2 > 2^31 - 1 (32-bit slice offsets)  */
  SIGATTN_ERR_SEQLEN = 3,    /* some seqlens[b] outside [0, Lmax]                       */
  SIGATTN_ERR_ALIGN = 4,     /* a tensor pointer is not 16-byte aligned (head_bias and
                                sigattn_bias_grad's db: 4-byte)                         */
  SIGATTN_ERR_ALIAS = 5,     /* an output overlaps an input or another output (or the
                                per-head bias values)                                   */
  SIGATTN_ERR_BIAS = 6,      /* unknown bias_mode, non-finite bias_arg, or bias_arg <= 0
                                with SIGATTN_BIAS_NEG_LOG_N                             */
  SIGATTN_ERR_PRECISION = 7, /* unknown precision                                       */
  SIGATTN_ERR_HIP = 8,       /* the HIP runtime rejected a kernel launch                */
  SIGATTN_ERR_PASS = 9,      /* unknown pass id (sigattn_plan_stats only)               */
  SIGATTN_ERR_STRIDE = 10,   /* a stride is negative or not a multiple of 8 elements, a
                                row stride is below d or too large for 32-bit offsets
                                ((Lmax + 256) * l * 2 > 2^31 - 1), or an output view
                                maps two elements to one address                        */
  SIGATTN_ERR_MASK = 11,     /* unknown mask mode                                       */
  SIGATTN_ERR_DTYPE = 12     /* unknown element type                                    */
} sigattn_status;

/* Which keys a query sees. */
typedef enum sigattn_mask {
  SIGATTN_MASK_NONE = 0,   /* bidirectional: every valid key (the summary's models)   */
  SIGATTN_MASK_CAUSAL = 1  /* query i sees keys 0..i only: the autoregressive variant
                              (the language experiments of "Theory, Analysis, and Best
                              Practices for Sigmoid Self-Attention", abstract); tiles
                              above the diagonal are skipped like padded ones        */
} sigattn_mask;

/* Element type of every tensor argument of a call (all tensors share it). */
typedef enum sigattn_dtype {
  SIGATTN_DTYPE_BF16 = 0,  /* bfloat16 (the pages' precision)                          */
  SIGATTN_DTYPE_F16 = 1    /* IEEE binary16: the products use the fp16 MFMA; P and dX
                              are rounded to fp16 (11 significant bits against bf16's
                              8); outputs are fp16, so |values| must stay below 65504 */
} sigattn_dtype;

/* The bias b_b of the SigmoidAttn formula (summary §2A, b = -log(n)). */
typedef enum sigattn_bias_mode {
  SIGATTN_BIAS_NEG_LOG_SEQLEN = 0, /* b_b = -ln(n_b), n_b = valid length (default)  */
  SIGATTN_BIAS_NEG_LOG_N = 1,      /* b = -ln(bias_arg), a fixed n (e.g. Lmax)      */
  SIGATTN_BIAS_CONST = 2,          /* b = bias_arg                                  */
  SIGATTN_BIAS_PER_HEAD = 3        /* b_h = head_bias[h]: one value per head, read
                                      from device memory by the kernels, so that a
                                      trained bias needs no host round trip (the
                                      learnable variant; its gradient comes from
                                      sigattn_bwd_dkdv_dbias)                       */
} sigattn_bias_mode;

/* Arithmetic of the sigmoid and of the second matrix products (the tensors'
 * element type is written e16 below: bf16 or fp16).
 *
 * FAST is meant for the method's own regime, b = -ln n with scores of order
 * one, where every weight is about 1/n: P (forward, dV) and dX (dQ, dK) are
 * rounded once to e16, and the score scale log2(e)/sqrt(d) is folded into the
 * operand each wave holds for its whole tile (rounded to e16 once), which
 * saves one instruction per score.  Outside that regime - saturated scores
 * (|x| >> 10, e.g. inputs scaled x4), or a constant bias near 0 so that many
 * weights of order one sum - bf16 FAST exceeds |gpu - exact| <= 2e-2 (1 +
 * |exact|) and SPLIT is required. */
typedef enum sigattn_precision {
  SIGATTN_PREC_FAST = 0,  /* P and dX rounded once to e16; prescaled scores          */
  SIGATTN_PREC_SPLIT = 1  /* exact fp32 scores; P and dX as a pair hi = e16(x),
                             lo = e16(x - hi): two products, ~16 (bf16) or ~22
                             (fp16) significant bits                             */
} sigattn_precision;

/* Which pass sigattn_plan_stats describes. */
typedef enum sigattn_pass {
  SIGATTN_PASS_FWD = 0,
  SIGATTN_PASS_BWD_DQ = 1,
  SIGATTN_PASS_BWD_DKDV = 2,
  SIGATTN_PASS_BWD = 3       /* both backward sides, as sigattn_bwd runs them
                                (sigattn_validate and sigattn_plan_stats)       */
} sigattn_pass;

/* Element strides of one tensor argument seen as [B, H, Lmax, d]: element
 * (b, h, l, c) is at ptr[b * b_stride + h * h_stride + l * l_stride + c].  The
 * head dimension is always contiguous.  Contiguous [B, H, Lmax, d] is
 * {H*Lmax*d, Lmax*d, d}; [B, Lmax, H, d] is {Lmax*H*d, d, H*d}; the q slice of
 * a fused [B, Lmax, 3, H, d] projection is {Lmax*3*H*d, d, 3*H*d}.  Every
 * stride must be a non-negative multiple of 8 (16-byte rows) and l_stride >= d.
 * Inputs may overlap one another and may broadcast (a zero stride); an output
 * must map distinct elements to distinct addresses and may not overlap an
 * input or another output (checked exactly for outputs that share strides,
 * such as the dq/dk/dv slices of one fused buffer, and by address range
 * otherwise). */
typedef struct sigattn_strides {
  int64_t b, h, l;
} sigattn_strides;

typedef struct sigattn_args {
  int32_t B, H, Lmax, d;    /* batch, heads, padded length, head dim (64 or 128)    */
  const int32_t *seqlens;   /* HOST pointer to B valid lengths, 0 <= n_b <= Lmax;
                               read during the call only                            */
  int32_t bias_mode;        /* sigattn_bias_mode                                    */
  float bias_arg;           /* see sigattn_bias_mode; ignored for mode 0            */
  int32_t precision;        /* sigattn_precision                                    */
  void *stream;             /* hipStream_t to enqueue on; NULL = default stream     */
  const sigattn_strides *strides; /* HOST pointer, NULL = every tensor contiguous
                               [B, H, Lmax, d]; else one entry per tensor argument
                               of the call, in argument order (fwd: q, k, v, o;
                               dq: q, k, v, dout, dq; dkdv: q, k, v, dout, dk, dv);
                               read during the call only                            */
  int32_t mask;             /* sigattn_mask; 0 = bidirectional                      */
  const float *head_bias;   /* DEVICE pointer to H fp32 bias values, 4-byte aligned,
                               read by the kernels in bias mode 3 (the values must
                               be finite; they are not checked); ignored in the
                               other modes                                          */
  int32_t dtype;            /* sigattn_dtype of the tensors; 0 = bf16               */
} sigattn_args;

/* Forward: O = sigma(Q K^T / sqrt(d) + b) V on valid rows; padded rows of O = 0.
 * One fused kernel per launch chunk (summary §2C: fused forward). */
sigattn_status sigattn_fwd(const sigattn_args *args, const void *q, const void *k,
                           const void *v, void *o);

/* Backward, query side: dQ = (dO V^T * P * (1 - P)) K / sqrt(d); padded rows
 * of dQ = 0; padded rows of dO are ignored.  P is recomputed (§2B diagonal
 * Jacobian, §2C backward split into a dQ kernel and a dK/dV kernel). */
sigattn_status sigattn_bwd_dq(const sigattn_args *args, const void *q, const void *k,
                              const void *v, const void *dout, void *dq);

/* Backward, key side: dV = P^T dO and dK = (dO V^T * P * (1 - P))^T Q / sqrt(d);
 * padded rows of dK and dV = 0.  Each output row has a single writer: no
 * atomics (§2C). */
sigattn_status sigattn_bwd_dkdv(const sigattn_args *args, const void *q, const void *k,
                                const void *v, const void *dout, void *dk, void *dv);

/* The whole backward in one call: dQ (as sigattn_bwd_dq), dK and dV (as
 * sigattn_bwd_dkdv) and, if dbias is not NULL, the bias-gradient rows (as
 * sigattn_bwd_dkdv_dbias).  Results are bitwise those of the separate calls,
 * except in the short-sequence case below.
 * At d = 64 both sides normally run in ONE fused launch: the dK/dV
 * workgroups first, then the dQ workgroups, which fill the CUs the dK/dV work
 * leaves idle towards its end (§2C's two backward kernels, scheduled
 * together; still no atomics: every output row has one writer).  At d = 128
 * the two kernels run at different occupancies, and the dK/dV and dQ
 * launches run in turn on args->stream.
 * Short-sequence case: d = 64, fast precision, no mask and Lmax <= 256.
 * Then one workgroup per (sequence, head) writes all of its dQ, dK and dV
 * rows and its bias-gradient rows (one launch per 4096 sequences), computing
 * S, dP and dS once instead of once per side: dK, dV and the bias rows are
 * bitwise those of sigattn_bwd_dkdv(_dbias), and dQ is taken from the same
 * dS (the scores from K scaled by -log2(e)/sqrt(d) and rounded to the
 * element type, where sigattn_bwd_dq scales Q), so it differs from
 * sigattn_bwd_dq by rounding only.
 * args->strides, if set, has 7 entries: q, k, v, dout, dq, dk, dv.  Same
 * checks and errors as the separate calls (dq, dk, dv are outputs; dbias is
 * checked like a row output). */
sigattn_status sigattn_bwd(const sigattn_args *args, const void *q, const void *k, const void *v,
                           const void *dout, void *dq, void *dk, void *dv, float *dbias);

/* Backward, key side, with the gradient of the bias: as sigattn_bwd_dkdv, and
 * also, per key row, dbias[b, h, j] = sum over valid queries i of dX_ij, where
 * dX = dO V^T * P * (1 - P) is the gradient of the scores X_ij = q_i.k_j /
 * sqrt(d) + b (summary §2A formula, §2B derivative).  Because b enters every
 * score of its (sequence, head) with coefficient 1, dl/db for that (b, h) is
 * the sum of its row of dbias; a per-head bias sums over sequences too
 * (sigattn_bias_grad).  dbias: device fp32, contiguous [B, H, Lmax], 16-byte
 * aligned, written in full (0 on padded rows j >= n_b), must not overlap a
 * tensor argument.  Each row has a single writer: no atomics.  Any bias mode. */
sigattn_status sigattn_bwd_dkdv_dbias(const sigattn_args *args, const void *q, const void *k,
                                      const void *v, const void *dout, void *dk, void *dv,
                                      float *dbias);

/* Per-head bias gradient: db[h] = sum over b and j of dbias[b, h, j] (dbias as
 * written by sigattn_bwd_dkdv_dbias).  db: device fp32 [H], 4-byte aligned,
 * must not overlap dbias.  One workgroup per head sums in a fixed order, so
 * the result is deterministic.  Uses args' B, H, Lmax, seqlens (validated as
 * for the other calls) and stream; bias, precision and mask are ignored
 * except for validation. */
sigattn_status sigattn_bias_grad(const sigattn_args *args, const float *dbias, float *db);

/* Softmax attention on the same padded batches and schedule: the mechanism
 * sigmoid attention replaces, provided to compare the two on equal terms
 * ("Better Models, Faster Training: Sigmoid Attention for single-cell
 * Foundation Models", summary §4A, compares the sigmoid kernel with a softmax
 * FlashAttention kernel; the FlashAttention section of "Transformer
 * Attention機構の効率化と最新派生モデル" describes the tiled softmax with a
 * per-query log-sum-exp).  P = softmax over each query's valid keys of
 * Q K^T / sqrt(d); a constant bias cancels in a softmax, so bias_mode and
 * bias_arg are validated but have no effect.  lse2 and delta are fp32
 * [B, H, Lmax] contiguous arrays, 16-byte aligned:
 *   lse2_i  = log2 sum_j 2^(x_ij), x_ij = q_i.k_j * log2(e) / sqrt(d)  (the
 *             forward's per-row normaliser, base 2; 0 on padded rows),
 *   delta_i = sum_c dO_ic O_ic                    (0 on padded rows).
 * The backward is dV = P^T dO, dS = P * (dO V^T - delta), dQ = dS K / sqrt(d),
 * dK = dS^T Q / sqrt(d).  Tensor strides work as for the sigmoid calls
 * (args->strides entries in argument order, lse2/delta excluded). */
sigattn_status sigattn_softmax_fwd(const sigattn_args *args, const void *q, const void *k,
                                   const void *v, void *o, float *lse2);
sigattn_status sigattn_softmax_bwd_prep(const sigattn_args *args, const void *o,
                                        const void *dout, float *delta);
sigattn_status sigattn_softmax_bwd_dq(const sigattn_args *args, const void *q, const void *k,
                                      const void *v, const void *dout, const float *lse2,
                                      const float *delta, void *dq);
sigattn_status sigattn_softmax_bwd_dkdv(const sigattn_args *args, const void *q, const void *k,
                                        const void *v, const void *dout, const float *lse2,
                                        const float *delta, void *dk, void *dv);
/* Both softmax backward kernels (after sigattn_softmax_bwd_prep), in one
 * fused launch at d = 64 as sigattn_bwd does for sigmoid; strides order
 * q, k, v, dout, dq, dk, dv. */
sigattn_status sigattn_softmax_bwd(const sigattn_args *args, const void *q, const void *k, const void *v,
                                   const void *dout, const float *lse2, const float *delta, void *dq,
                                   void *dk, void *dv);

/* Runs every check the compute call for pass p would run (shape, lengths,
 * bias, precision, null pointers, alignment, strides, aliasing) on the
 * call's tensor arguments, given in argument order (fwd: q, k, v, o; dq: q,
 * k, v, dout, dq; dkdv: q, k, v, dout, dk, dv; SIGATTN_PASS_BWD: q, k, v,
 * dout, dq, dk, dv, as sigattn_bwd without bias rows), and returns the status
 * that call would return, without enqueuing anything and without
 * dereferencing the tensor pointers.  For callers that want to vet a layout
 * ahead of time. */
sigattn_status sigattn_validate(const sigattn_args *args, int32_t pass, const void *const *tensors);

/* Measurement helper, not part of the method: runs `blocks` workgroups of
 * 1024 threads, each wave issuing `iters` x 4 independent bf16 32x32x16 MFMAs
 * (the product every kernel here uses) on register operands, so that a
 * caller can time the sustained matrix-core rate of this chip under its
 * current clocks.  out: device, blocks * 1024 floats (per-thread sums, to
 * keep the work); clocks: device, 2 values written by block 0: shader-clock
 * ticks (s_memtime) and 100 MHz ticks (s_memrealtime) over the loop, whose
 * ratio gives the shader clock.  FLOP = blocks * 16 * iters * 4 * 32768.
 * SIGATTN_ERR_NULL / _ALIGN (out 4-byte, clocks 8-byte) / _SHAPE (blocks
 * outside [1, 65536], iters < 1) / _ALIAS before any launch. */
sigattn_status sigattn_probe_mfma(int32_t blocks, int32_t iters, float *out, uint64_t *clocks,
                                  void *stream);

/* Static description of a status code; never NULL. */
const char *sigattn_status_str(sigattn_status status);

/* Host-only description of the tile schedule a call would run, without
 * touching the GPU.  For pass p it reports the work items (one output tile
 * each), the (outer tile, inner tile) pairs those items visit — fully padded
 * tiles are not counted because they are never computed — and the number of
 * kernel launches.  For SIGATTN_PASS_BWD: the dK/dV and dQ sides summed,
 * and 1 launch when sigattn_bwd fuses them (d = 64, both sides fitting one
 * launch each), or the dK/dV side's launch count in sigattn_bwd's
 * short-sequence case (one launch per length table; the items and pairs are
 * still those of the two sides).
 * Any of the output pointers may be NULL.  Validates args (shape, seqlens,
 * bias, precision) as the compute calls do. */
sigattn_status sigattn_plan_stats(const sigattn_args *args, int32_t pass, int64_t *work_items,
                                  int64_t *tile_pairs, int32_t *launches);

/* Rows per output tile and per inner tile for pass p and head dim d
 * (written to *outer_rows, *inner_rows); SIGATTN_ERR_PASS / _SHAPE on a bad
 * pass or d. */
sigattn_status sigattn_tile_shape(int32_t pass, int32_t d, int32_t *outer_rows,
                                  int32_t *inner_rows);

#ifdef __cplusplus
}
#endif

#endif /* SIGATTN_H */
