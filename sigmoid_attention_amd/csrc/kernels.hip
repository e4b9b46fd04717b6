// Sigmoid attention kernels for gfx950: fused forward, backward-dQ,
// backward-dK/dV; padded output rows are zero-filled by the same launches.
//
// Method: "Better Models, Faster Training: Sigmoid Attention for single-cell
// Foundation Models", technical summary §2A (O = sigma(Q K^T / sqrt(d) + b) V,
// b = -log n), §2B (sigma' = sigma (1 - sigma), diagonal Jacobian) and §2C
// (fused forward, backward split into a dQ kernel and a dK/dV kernel so no
// atomics are needed, activations recomputed, fully padded blocks skipped).
//
// Design for MI355X (not a translation of the pages' Triton/H100 kernel):
// * one 256-thread workgroup (4 waves of 64) per output tile; each wave owns
//   32 output rows, so every product is a 32x32x16 MFMA (bf16, or fp16 in
//   the fp16 build of this file);
// * the tile streamed by the inner loop (K/V in the forward and dQ kernels,
//   Q/dO in the dK/dV kernel) is loaded straight from global memory into LDS
//   (buffer_load ... lds), two steps ahead, with hardware zero-fill past the
//   sequence end; one LDS copy per tile serves both the 16-byte fragment
//   reads and the transposing reads (see device_common.h): one barrier per
//   inner step and no VALU work for staging; in the d = 64 backward each
//   stage of the tile ring is an LDS array of its own (SIGATTN_RING), so the
//   step's reads do not wait for the load in flight;
// * fast precision folds the score scale into the operand a wave holds in
//   registers for its whole item, so sigma costs three VALU instructions per
//   score (exp, fma, rcp; see sigmoid_pre);
// * the score product's output registers are directly the B operand of the
//   second product (see device_common.h): P and dS never leave registers and
//   are never stored; the transposed A operand is read with ds_read_b64_tr_b16
//   from a row-major tile, so nothing is transposed on the VALU;
// * rows at or beyond n_b are zero-filled on load, never read, so no mask is
//   applied to P: a zero K row gives a finite score and a zero V (or dO, Q)
//   row contributes nothing;
// * with no row normaliser (§2A), partial products need no running max or
//   rescale, and the inner tiles may be visited in any order;
// * padded output rows are written as 0 by trailing workgroups of the same
//   launch (dispatched last, they fill the tail), so each call is one launch;
// * at d = 64 the two backward kernels run as one launch (bwd_kernel): the
//   dQ workgroups fill the CUs that the dK/dV workgroups leave idle at the
//   end; when every sequence fits 256 rows, one workgroup per (sequence,
//   head) computes S and dP once for dQ, dK and dV (bwd_small_kernel);
// * variants: a causal mask (tiles above the diagonal skipped, the straddling
//   tile masked in registers), a per-head bias read from device memory with
//   its gradient (per-key sums of dS), and softmax attention on the same
//   schedule for comparison.
#include "device_common.h"
#include "launch.h"
#include "plan.h"

namespace sigattn {
namespace SIGATTN_ELT {

namespace kern {

constexpr int kThreads = 256;

// The LDS tile ring of a workgroup: up to six tiles of `elems` 16-bit
// elements.  A load into one stage is issued while other stages are read.
// With SEP each stage is a __shared__ array of its own: the compiler can then
// tell that those reads do not touch the stage being filled and does not make
// them wait for the load (global -> LDS loads count as outstanding LDS writes
// until they land).  Without SEP the stages are slices of one array and every
// LDS read after a load waits for it; the scheduler then keeps fewer values
// live, which the head-dim-128 backward (one wave per SIMD, at the register
// limit) needs.  Stages are always named by compile-time indices, so with SEP
// every access resolves to one array.
struct Ring {
  uint16_t* p[6];
};
#define SIGATTN_RING(name, n, elems, sep)                                                                  \
  __shared__ __align__(16) uint16_t name##0[(sep) ? (elems) : (n) * (elems)], name##1[(sep) ? (elems) : 8], \
      name##2[(sep) ? (elems) : 8], name##3[(sep) ? (elems) : 8], name##4[(sep) ? (elems) : 8],             \
      name##5[(sep) && (n) > 5 ? (elems) : 8];                                                                \
  const Ring name = (sep) ? Ring{{name##0, name##1, name##2, name##3, name##4, (n) > 5 ? name##5 : nullptr}}  \
                          : Ring{{name##0, name##0 + (elems), name##0 + 2 * (elems), name##0 + 3 * (elems),    \
                                  name##0 + 4 * (elems), (n) > 5 ? name##0 + 5 * (elems) : nullptr}}
constexpr int kInner = 64;  // rows per inner tile

// Schedule per kernel and head dim (measured on MI355X, same-run A/B):
// LA = compute the next tile's scores while the VALU works on this tile (two
// tiles of scores live in registers); OCC = waves per SIMD the register
// budget is sized for.  At d = 64 more resident waves beat in-wave lookahead
// for the forward and dK/dV; dQ keeps the lookahead of its scores.  At
// d = 128 the forward fits lookahead and two waves per SIMD (1.43x faster
// than one wave per SIMD on the dense 8K batch).
// Forward waves per SIMD: 4 at d = 64 (split precision included: with the
// low part taken from the packed high part, see split_lo, it needs 117
// registers), 2 at d = 128.
template <int D, bool SPLIT = false> struct FwdCfg {
  static constexpr bool LA = D != 64;
  static constexpr int OCC = D == 64 ? 4 : 2;
};
// The dQ kernel runs two waves per SIMD at either head dim (at d = 128 one
// 16-byte value is spilled and reloaded once per step).  The dK/dV kernel
// runs one wave per SIMD at d = 128 (its accumulators alone take 128
// registers); with no other wave to overlap with, it computes the next
// tile's S and dP inside the chunk loop, with every LDS fragment read issued
// a chunk ahead (ROLL).  Their occupancies differ there, so at d = 128 the
// backward runs as two launches rather than the fused one.
template <int D> struct DqCfg {
  static constexpr int OCC = 2;
};
template <int D> struct DkdvCfg {
  static constexpr int BQ = 64;
  static constexpr int OCC = D == 64 ? 2 : 1;
  static constexpr bool ROLL = D == 128;
};

// sigma of one score value: from the raw score with the bias term c2, or
// (PRE, fast precision) from the prescaled score u with the bias factor m
// (see sigmoid_pre).
template <int D, bool PRE>
__device__ __forceinline__ float sigma_of(float score, float arg) {
  if constexpr (PRE) return sigmoid_pre(score, arg);
  else return sigmoid2(score, score_c1<D>(), arg);
}

// sigma of the eight score values of K-chunk c, rounded to the element type
// (hi) and, in split precision, the rounded remainder (lo).  arg: c2, or m
// with PRE.
template <int D, bool SPLIT, bool PRE>
__device__ __forceinline__ void sigmoid_chunk(const f32x16 (&sc)[2], int c, float arg, e16x8& hi, e16x8& lo) {
  f32x8 p = chunk8(sc[c >> 1], c & 1);
#pragma unroll
  for (int t = 0; t < 8; ++t) p[t] = sigma_of<D, PRE>(p[t], arg);
  hi = to_e16x8(p);
  if (SPLIT) lo = split_lo(p, hi);
}

// dS = dP * sigma * (1 - sigma) for K-chunk c (and optionally sigma itself;
// with DSUM, the chunk's eight fp32 dS values are also added to *dsum).
template <int D, bool SPLIT, bool PRE, bool WANT_P, bool DSUM = false, int NB>
__device__ __forceinline__ void dsigmoid_chunk(const f32x16 (&sc)[NB], const f32x16 (&dp)[NB], int c, float arg,
                                               e16x8& dh, e16x8& dl, e16x8& ph, e16x8& pl,
                                               float* dsum = nullptr) {
  // No contraction of dP * p (1 - p) into the sum below: the sum then rounds
  // the same in every kernel that inlines this, whatever else is scheduled
  // around it.
#pragma clang fp contract(off)
  const f32x8 sv = chunk8(sc[c >> 1], c & 1), gv = chunk8(dp[c >> 1], c & 1);
  f32x8 p8, ds;
#pragma unroll
  for (int t = 0; t < 8; ++t) {
    const float p = sigma_of<D, PRE>(sv[t], arg);
    p8[t] = p;
    ds[t] = gv[t] * __builtin_fmaf(-p, p, p);  // dP * p (1 - p)
  }
  dh = to_e16x8(ds);
  if (SPLIT) dl = split_lo(ds, dh);
  if (WANT_P) {
    ph = to_e16x8(p8);
    if (SPLIT) pl = split_lo(p8, ph);
  }
  if constexpr (DSUM)  // pairwise: keeps the eight values' live ranges short
    *dsum += ((ds[0] + ds[1]) + (ds[2] + ds[3])) + ((ds[4] + ds[5]) + (ds[6] + ds[7]));
}

// Causal mask (query i sees keys 0..i), applied only in tiles that straddle
// the diagonal.  `masked` is the score that gives weight 0: -inf for a raw
// score (sigma = 0, dS = 0; softmax weight 0), +inf for a prescaled one
// (u = c1 * score with c1 < 0).
// S^T layout (keys in registers, the query is the lane's column): keys after
// the lane's query.  key0 = first key of the tile.
__device__ __forceinline__ void mask_causal_cols(f32x16 (&sc)[2], int key0, int qrow, int hf, float masked) {
  const int lim = qrow - key0 - 4 * hf;
#pragma unroll
  for (int b = 0; b < 2; ++b)
#pragma unroll
    for (int r = 0; r < 16; ++r)
      if (32 * b + 8 * (r >> 2) + (r & 3) > lim) sc[b][r] = masked;
}

// S layout (queries in registers, the key is the lane's column): queries
// before the lane's key.  q0 = first query of the tile.
template <int NB>
__device__ __forceinline__ void mask_causal_rows(f32x16 (&sc)[NB], int q0, int krow, int hf, float masked) {
  const int lim = krow - q0 - 4 * hf;
#pragma unroll
  for (int b = 0; b < NB; ++b)
#pragma unroll
    for (int r = 0; r < 16; ++r)
      if (32 * b + 8 * (r >> 2) + (r & 3) < lim) sc[b][r] = masked;
}

// The same for one 32-row block of S whose first query is qb0.
__device__ __forceinline__ void mask_causal_block(f32x16& sc, int qb0, int krow, int hf, float masked) {
  const int lim = krow - qb0 - 4 * hf;
#pragma unroll
  for (int r = 0; r < 16; ++r)
    if (8 * (r >> 2) + (r & 3) < lim) sc[r] = masked;
}

// The masked score for a raw (PRE = false) or prescaled score.
template <bool PRE>
__device__ __forceinline__ constexpr float masked_score() {
  return PRE ? __builtin_inff() : -__builtin_inff();
}

// ---------------------------------------------------------------------------
// Softmax attention, the workload sigmoid attention replaces, on the same
// schedule (comparison path).  Per query row the forward keeps a running
// maximum and sum and hands the base-2 log-sum-exp of the row's scaled scores,
// lse2 = log2 sum_j 2^(s_ij c1s) with c1s = log2(e)/sqrt(d), to the backward,
// where P = 2^(s c1s - lse2) and dS = P (dP - delta), delta = rowsum(dO * O).
// ---------------------------------------------------------------------------
template <int D>
__device__ __forceinline__ constexpr float softmax_c1() {
  return (float)(1.4426950408889634074 / (D == 64 ? 8.0 : 11.313708498984760390));
}

// dS for K-chunk c when queries are the lane's column (dQ kernel): one lse2 and
// delta per lane.
template <int D, bool SPLIT, int NB>
__device__ __forceinline__ void dsoftmax_chunk_col(const f32x16 (&sc)[NB], const f32x16 (&dp)[NB], int c, float lse2,
                                                   float dlt, e16x8& dh, e16x8& dl) {
  const f32x8 sv = chunk8(sc[c >> 1], c & 1), gv = chunk8(dp[c >> 1], c & 1);
  f32x8 ds;
#pragma unroll
  for (int t = 0; t < 8; ++t) {
    const float p = __builtin_amdgcn_exp2f(__builtin_fmaf(sv[t], softmax_c1<D>(), -lse2));
    ds[t] = p * (gv[t] - dlt);
  }
  dh = to_e16x8(ds);
  if (SPLIT) dl = split_lo(ds, dh);
}

// P and dS for K-chunk c when queries are rows (dK/dV kernel): lse2 and delta
// of the chunk's eight rows held by the lane (rows 16c + 4hf + {0..3} and
// 16c + 8 + 4hf + {0..3}, in register order).
template <int D, bool SPLIT, int NB>
__device__ __forceinline__ void dsoftmax_chunk_row(const f32x16 (&sc)[NB], const f32x16 (&dp)[NB], int c,
                                                   const f32x8& lse8, const f32x8& dlt8, e16x8& dh, e16x8& dl,
                                                   e16x8& ph, e16x8& pl) {
  const f32x8 sv = chunk8(sc[c >> 1], c & 1), gv = chunk8(dp[c >> 1], c & 1);
  f32x8 p8, ds;
#pragma unroll
  for (int t = 0; t < 8; ++t) {
    const float p = __builtin_amdgcn_exp2f(__builtin_fmaf(sv[t], softmax_c1<D>(), -lse8[t]));
    p8[t] = p;
    ds[t] = p * (gv[t] - dlt8[t]);
  }
  dh = to_e16x8(ds);
  if (SPLIT) dl = split_lo(ds, dh);
  ph = to_e16x8(p8);
  if (SPLIT) pl = split_lo(p8, ph);
}

// Store 4 consecutive fp32 values of an output row in the element type (8 bytes).
__device__ __forceinline__ void store4(uint16_t* dst, const f32x16& acc, int i, float scale) {
  f32x8 v8;
#pragma unroll
  for (int t = 0; t < 4; ++t) {
    v8[t] = scale * acc[4 * i + t];
    v8[4 + t] = 0.0f;
  }
  const u32x4 packed = as_u32x4(to_e16x8(v8));
  *(uint2*)dst = (uint2){packed[0], packed[1]};
}

// Score-product helpers.  `tile` is an LDS tile; `bf` holds the B fragments
// (this wave's 32 rows of the other operand).  Block mb covers tile rows
// 32mb .. 32mb+31; K-steps s cover d = 16s .. 16s+15.
template <int D, int NB>
__device__ __forceinline__ void score_steps(f32x16 (&acc)[NB], const uint16_t* tile, const e16x8 (&bf)[D / 16],
                                            int s0, int s1, const FragAddr<D>& fa) {
#pragma unroll
  for (int s = s0; s < s1; ++s)
#pragma unroll
    for (int mb = 0; mb < NB; ++mb) acc[mb] = mfma(fa.read(tile, mb, s), bf[s], acc[mb]);
}

template <int D>
__device__ __forceinline__ void score_block(f32x16& acc, const uint16_t* tile, const e16x8 (&bf)[D / 16], int mb,
                                            const FragAddr<D>& fa) {
#pragma unroll
  for (int s = 0; s < D / 16; ++s) acc = mfma(fa.read(tile, mb, s), bf[s], acc);
}

// Second-product step for K-chunk c: acc[db] += A(tile rows d, K-chunk c) . B.
template <int D, bool SPLIT>
__device__ __forceinline__ void value_chunk(f32x16 (&acc)[D / 32], const TrFrag<D>& tr, const uint16_t* tile, int c,
                                            const e16x8& bh, const e16x8& bl) {
#pragma unroll
  for (int db = 0; db < D / 32; ++db) {
    const e16x8 a = tr.read(tile, db, c);
    acc[db] = mfma(a, bh, acc[db]);
    if (SPLIT) acc[db] = mfma(a, bl, acc[db]);
  }
}

// The same, with the A fragments read beforehand (see read_value_frags).
template <int D, bool SPLIT>
__device__ __forceinline__ void value_chunk_pre(f32x16 (&acc)[D / 32], const e16x8 (&a)[D / 32], const e16x8& bh,
                                                const e16x8& bl) {
#pragma unroll
  for (int db = 0; db < D / 32; ++db) {
    acc[db] = mfma(a[db], bh, acc[db]);
    if (SPLIT) acc[db] = mfma(a[db], bl, acc[db]);
  }
}

template <int D>
__device__ __forceinline__ void read_value_frags(e16x8 (&a)[D / 32], const TrFrag<D>& tr, const uint16_t* tile,
                                                 int c) {
#pragma unroll
  for (int db = 0; db < D / 32; ++db) a[db] = tr.read(tile, db, c);
}

// Keeps the compiler from moving instructions across this point, so LDS
// reads issued before a block of VALU work stay there and their latency is
// covered by that work.
__device__ __forceinline__ void sched_fence() { __builtin_amdgcn_sched_barrier(0); }

// Score product over all K-steps with the A fragments of step s+1 read while
// step s multiplies (one step of read-ahead).
template <int D, int NB>
__device__ __forceinline__ void score_pipelined(f32x16 (&acc)[NB], const uint16_t* tile, const e16x8 (&bf)[D / 16],
                                                const FragAddr<D>& fa) {
  e16x8 a0[NB], a1[NB];
#pragma unroll
  for (int mb = 0; mb < NB; ++mb) a0[mb] = fa.read(tile, mb, 0);
#pragma unroll
  for (int s = 0; s < D / 16; ++s) {
    if (s + 1 < D / 16) {
#pragma unroll
      for (int mb = 0; mb < NB; ++mb) a1[mb] = fa.read(tile, mb, s + 1);
    }
    sched_fence();
#pragma unroll
    for (int mb = 0; mb < NB; ++mb) acc[mb] = mfma(a0[mb], bf[s], acc[mb]);
    sched_fence();
#pragma unroll
    for (int mb = 0; mb < NB; ++mb) a0[mb] = a1[mb];
  }
}

// Scheduling hint: NM matrix products, each followed by NV vector ALU
// instructions, so the MFMA unit works while the VALU evaluates sigma.
template <int NM, int NV>
__device__ __forceinline__ void interleave() {
#pragma unroll
  for (int i = 0; i < NM; ++i) {
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
    __builtin_amdgcn_sched_group_barrier(0x002, NV, 0);
  }
}

template <int NB>
__device__ __forceinline__ void zero2(f32x16 (&a)[NB]) {
#pragma unroll
  for (int i = 0; i < NB; ++i) a[i] = (f32x16){};
}

// Inner loops are unrolled six times (the period of the 3-stage LDS ring and
// of the 2-way register ping-pong), so every LDS address is a lane offset
// plus a compile-time immediate.  Phase<P> is the step index modulo 6.
template <int P>
using Phase = std::integral_constant<int, P>;

template <int P, class T>
__device__ __forceinline__ T& pick(T& a, T& b) {
  if constexpr (P % 2 == 0) return a;
  else return b;
}

// Runs step(Phase<j % 6>, j) for j = 0 .. n-1 (n >= 1).
template <class Step>
__device__ __forceinline__ void run_steps(int n, Step&& step) {
  for (int j = 0;;) {
    step(Phase<0>{}, j);
    if (++j == n) break;
    sched_fence();
    step(Phase<1>{}, j);
    if (++j == n) break;
    sched_fence();
    step(Phase<2>{}, j);
    if (++j == n) break;
    sched_fence();
    step(Phase<3>{}, j);
    if (++j == n) break;
    sched_fence();
    step(Phase<4>{}, j);
    if (++j == n) break;
    sched_fence();
    step(Phase<5>{}, j);
    if (++j == n) break;
    sched_fence();
  }
}

// ---------------------------------------------------------------------------
// Forward.  Item = (b, h, 128-query tile).  Inner loop: 64-key tiles j.
// Per wave (32 queries): S^T_j (64 keys x 32 queries) = K_j . Q^T,
// P_j = sigma(S^T_j), O^T (d x 32 queries) += V_j^T . P_j.
// LDS: K in 3 stages (tile j+1 feeds the scores computed during step j while
// the VALU evaluates sigma of tile j; tile j+2 is loading), V in 2 stages.
// Tiles are loaded global -> LDS directly, one step ahead; loads past the
// sequence return zeros, so the steady state has no branches (the few
// products on such tiles are unused).
// ---------------------------------------------------------------------------
template <int D, bool SPLIT, bool LA = FwdCfg<D>::LA>
__global__ __launch_bounds__(kThreads, (FwdCfg<D, SPLIT>::OCC)) void fwd_kernel(const uint16_t* __restrict__ Q,
                                                                        const uint16_t* __restrict__ K,
                                                                        const uint16_t* __restrict__ V,
                                                                        uint16_t* __restrict__ O, const SeqTable T, const Sched S) {
  constexpr int BQ = 128, BK = kInner, TILE = BK * D;
  SIGATTN_RING(lds, 5, TILE, false);  // K0 K1 K2 V0 V1

  if ((int)blockIdx.x >= S.compute_blocks) {
    zero_padded_rows<D>(T, S, (int)blockIdx.x, O, 3, nullptr, 0);
    return;
  }
  Item it;
  if (!find_item(T, S, (int)blockIdx.x, it)) return;
  constexpr bool PRE = !SPLIT;  // fast precision: prescaled scores (sigmoid_pre)
  const int n = it.n;
  const int tid = threadIdx.x, lane = tid & 63, l32 = lane & 31, hf = lane >> 5;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const float c2 = item_c2(S, it);
  const float sarg = PRE ? item_bias_factor(S, it, c2) : c2;
  const TrFrag<D> tr(lane);
  const FragAddr<D> fa(l32, hf);
  const TileDma<BK, D> dma_k(w, lane, S.sl[1]), dma_v(w, lane, S.sl[2]);
  auto Kb = [&](int i) { return lds.p[i]; };
  auto Vb = [&](int i) { return lds.p[3 + i]; };
  const Slice qs(slice_base(Q, S, it.bh, 0), n, S.sl[0]), ks(slice_base(K, S, it.bh, 1), n, S.sl[1]),
      vs(slice_base(V, S, it.bh, 2), n, S.sl[2]);
  // the first tiles load while the fragments below are read
  dma_k.load(ks, 0, Kb(0));
  dma_k.load(ks, BK, Kb(1));
  dma_v.load(vs, 0, Vb(0));

  const int qrow = it.tile * BQ + 32 * w + l32;
  e16x8 qf[D / 16];
  if (PRE) load_bfrag_scaled<D>(qf, qs, qrow, hf, score_c1<D>());
  else load_bfrag<D>(qf, qs, qrow, hf);
  f32x16 acc[D / 32];
#pragma unroll
  for (int i = 0; i < D / 32; ++i) acc[i] = (f32x16){};

  const int nk = S.causal ? min((n + BK - 1) / BK, causal_inner_end(it.tile, BQ, BK)) : (n + BK - 1) / BK;
  const int q0w = it.tile * BQ + 32 * w;  // this wave's first query
  vm_drain();
  __syncthreads();
  f32x16 sA[2], sB[2];
  zero2(sA);
  score_steps<D>(sA, Kb(0), qf, 0, D / 16, fa);

  auto step = [&](auto phase, int j) {
    constexpr int P = decltype(phase)::value;
    constexpr int k1 = (P + 1) % 3, k2 = (P + 2) % 3;  // K stages of tiles j+1, j+2
    f32x16(&cur)[2] = pick<P>(sA, sB);
    f32x16(&nxt)[2] = pick<P + 1>(sA, sB);
    dma_k.load(ks, (j + 2) * BK, Kb(k2));        // stage of tile j-1: free since the last barrier
    dma_v.load(vs, (j + 1) * BK, Vb((P + 1) % 2));
    const uint16_t* Kn = Kb(k1);
    const uint16_t* Vc = Vb(P % 2);
    if (S.causal && j * BK + BK - 1 > q0w) mask_causal_cols(cur, j * BK, qrow, hf, masked_score<PRE>());
    zero2(nxt);
    e16x8 ph[4], pl[4];
    if (LA) {
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        score_steps<D>(nxt, Kn, qf, c * (D / 64), (c + 1) * (D / 64), fa);  // MFMA: tile j+1
        sigmoid_chunk<D, SPLIT, PRE>(cur, c, sarg, ph[c], pl[c]);              // VALU: tile j
        if (c > 0) value_chunk<D, SPLIT>(acc, tr, Vc, c - 1, ph[c - 1], pl[c - 1]);
      }
      value_chunk<D, SPLIT>(acc, tr, Vc, 3, ph[3], pl[3]);
    } else {
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        sigmoid_chunk<D, SPLIT, PRE>(cur, c, sarg, ph[c], pl[c]);
        if (c > 0) value_chunk<D, SPLIT>(acc, tr, Vc, c - 1, ph[c - 1], pl[c - 1]);
      }
      value_chunk<D, SPLIT>(acc, tr, Vc, 3, ph[3], pl[3]);
      score_steps<D>(nxt, Kn, qf, 0, D / 16, fa);
    }
    vm_drain();
    __syncthreads();
  };
  run_steps(nk, step);

  if (qrow < n) {
    uint16_t* dst = slice_base(O, S, it.bh, 3) + (size_t)qrow * S.sl[3];
#pragma unroll
    for (int db = 0; db < D / 32; ++db)
#pragma unroll
      for (int i = 0; i < 4; ++i) store4(dst + 32 * db + 8 * i + 4 * hf, acc[db], i, 1.0f);
  }
}

// ---------------------------------------------------------------------------
// Softmax forward (comparison path).  Same items, tiles and LDS pipeline as
// the sigmoid forward.  Per query (the lane's column of S^T) a running maximum
// m and running sum l, in base 2: per tile, the maximum over the lane's 32
// keys and its partner half's, m' = max(m, c1s * max), O and l scaled by
// 2^(m - m'), then P = 2^(s c1s - m').  Keys at or beyond n_b only occur in
// the last tile and are set to -inf there (their zero-filled rows would
// otherwise join the normalisation).  Epilogue: O / l and lse2 = m + log2 l.
// ---------------------------------------------------------------------------
template <int D, bool SPLIT>
__device__ __forceinline__ void softmax_chunk(const f32x16 (&sc)[2], int c, float m, float& l, e16x8& hi,
                                              e16x8& lo) {
  f32x8 p = chunk8(sc[c >> 1], c & 1);
#pragma unroll
  for (int t = 0; t < 8; ++t) {
    p[t] = __builtin_amdgcn_exp2f(__builtin_fmaf(p[t], softmax_c1<D>(), -m));
    l += p[t];
  }
  hi = to_e16x8(p);
  if (SPLIT) lo = split_lo(p, hi);
}

// Scores of keys >= nv (tile-relative) to -inf; lane half hf holds keys
// 32b + 8(r/4) + 4hf + r%4 in register r of block b.
__device__ __forceinline__ void mask_keys(f32x16 (&sc)[2], int nv, int hf) {
  const int lim = nv - 4 * hf;
#pragma unroll
  for (int b = 0; b < 2; ++b)
#pragma unroll
    for (int r = 0; r < 16; ++r)
      if (32 * b + 8 * (r >> 2) + (r & 3) >= lim) sc[b][r] = -__builtin_inff();
}

template <int D, bool SPLIT>
__global__ __launch_bounds__(kThreads, 2) void fwd_softmax_kernel(
    const uint16_t* __restrict__ Q, const uint16_t* __restrict__ K, const uint16_t* __restrict__ V,
    uint16_t* __restrict__ O, float* __restrict__ LSE, const SeqTable T, const Sched S) {
  constexpr int BQ = 128, BK = kInner, TILE = BK * D;
  SIGATTN_RING(lds, 5, TILE, false);  // K0 K1 K2 V0 V1

  if ((int)blockIdx.x >= S.compute_blocks) {
    zero_padded_rows<D>(T, S, (int)blockIdx.x, O, 3, nullptr, 0, LSE);
    return;
  }
  Item it;
  if (!find_item(T, S, (int)blockIdx.x, it)) return;
  const int n = it.n;
  const int tid = threadIdx.x, lane = tid & 63, l32 = lane & 31, hf = lane >> 5;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const TrFrag<D> tr(lane);
  const FragAddr<D> fa(l32, hf);
  const TileDma<BK, D> dma_k(w, lane, S.sl[1]), dma_v(w, lane, S.sl[2]);
  auto Kb = [&](int i) { return lds.p[i]; };
  auto Vb = [&](int i) { return lds.p[3 + i]; };
  const Slice qs(slice_base(Q, S, it.bh, 0), n, S.sl[0]), ks(slice_base(K, S, it.bh, 1), n, S.sl[1]),
      vs(slice_base(V, S, it.bh, 2), n, S.sl[2]);
  // the first tiles load while the fragments below are read
  dma_k.load(ks, 0, Kb(0));
  dma_k.load(ks, BK, Kb(1));
  dma_v.load(vs, 0, Vb(0));

  const int qrow = it.tile * BQ + 32 * w + l32;
  e16x8 qf[D / 16];
  load_bfrag<D>(qf, qs, qrow, hf);
  f32x16 acc[D / 32];
#pragma unroll
  for (int i = 0; i < D / 32; ++i) acc[i] = (f32x16){};
  float m = -__builtin_inff(), l = 0.0f;

  const int nk = S.causal ? min((n + BK - 1) / BK, causal_inner_end(it.tile, BQ, BK)) : (n + BK - 1) / BK;
  const int q0w = it.tile * BQ + 32 * w;  // this wave's first query
  vm_drain();
  __syncthreads();
  f32x16 sA[2], sB[2];
  zero2(sA);
  score_steps<D>(sA, Kb(0), qf, 0, D / 16, fa);

  auto step = [&](auto phase, int j) {
    constexpr int P = decltype(phase)::value;
    constexpr int k1 = (P + 1) % 3, k2 = (P + 2) % 3;
    f32x16(&cur)[2] = pick<P>(sA, sB);
    f32x16(&nxt)[2] = pick<P + 1>(sA, sB);
    dma_k.load(ks, (j + 2) * BK, Kb(k2));
    dma_v.load(vs, (j + 1) * BK, Vb((P + 1) % 2));
    const uint16_t* Kn = Kb(k1);
    const uint16_t* Vc = Vb(P % 2);
    zero2(nxt);
    if (S.causal && j * BK + BK - 1 > q0w) mask_causal_cols(cur, j * BK, qrow, hf, -__builtin_inff());
    if (j * BK + BK > n) mask_keys(cur, n - j * BK, hf);
    float mt = cur[0][0];
#pragma unroll
    for (int b = 0; b < 2; ++b)
#pragma unroll
      for (int r = 0; r < 16; ++r) mt = __builtin_fmaxf(mt, cur[b][r]);
    mt = __builtin_fmaxf(mt, __shfl_xor(mt, 32));
    const float mn = __builtin_fmaxf(m, mt * softmax_c1<D>());
    const float alpha = __builtin_amdgcn_exp2f(m - mn);
#pragma unroll
    for (int i = 0; i < D / 32; ++i) acc[i] *= alpha;
    l *= alpha;
    m = mn;
    e16x8 ph[4], pl[4];
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      softmax_chunk<D, SPLIT>(cur, c, mn, l, ph[c], pl[c]);
      if (c > 0) value_chunk<D, SPLIT>(acc, tr, Vc, c - 1, ph[c - 1], pl[c - 1]);
    }
    value_chunk<D, SPLIT>(acc, tr, Vc, 3, ph[3], pl[3]);
    score_steps<D>(nxt, Kn, qf, 0, D / 16, fa);
    vm_drain();
    __syncthreads();
  };
  run_steps(nk, step);

  l += __shfl_xor(l, 32);
  if (qrow < n) {
    const float inv = __builtin_amdgcn_rcpf(l);
    uint16_t* dst = slice_base(O, S, it.bh, 3) + (size_t)qrow * S.sl[3];
#pragma unroll
    for (int db = 0; db < D / 32; ++db)
#pragma unroll
      for (int i = 0; i < 4; ++i) store4(dst + 32 * db + 8 * i + 4 * hf, acc[db], i, inv);
    if (hf == 0) LSE[(size_t)it.bh * S.Lmax + qrow] = m + __builtin_amdgcn_logf(l);
  }
  // rows at or beyond n_b get lse2 = 0 from the trailing workgroups
}

// ---------------------------------------------------------------------------
// Backward, dQ.  Item = (b, h, 128-query tile).  Inner loop: 64-key tiles j.
// Per wave (32 queries): S^T_j = K_j . Q^T, dP^T_j = V_j . dO^T,
// dS^T_j = dP^T_j * P(1-P), dQ^T (d x 32 queries) += K_j^T . dS^T_j.
// LDS: K in 3 stages (tile j: transposing reads for dQ; tile j+1: scores;
// tile j+2: loading), V in 2 stages (tile j: dP; tile j+1: loading).
// ---------------------------------------------------------------------------
// The dQ work of block vb of schedule S (a kernel of its own, or the dQ part
// of the fused backward launch); lds: five stages of kInner x D elements.
template <int D, bool SPLIT, bool SOFTMAX>
__device__ __forceinline__ void dq_body(const Ring& lds, int vb, const uint16_t* __restrict__ Q,
                                        const uint16_t* __restrict__ K, const uint16_t* __restrict__ V,
                                        const uint16_t* __restrict__ dO, uint16_t* __restrict__ dQ,
                                        const float* __restrict__ LSE, const float* __restrict__ DELTA,
                                        const SeqTable& T, const Sched& S) {
  constexpr int BQ = 128, BK = kInner;

  if (vb >= S.compute_blocks) {
    zero_padded_rows<D>(T, S, vb, dQ, 4, nullptr, 0);
    return;
  }
  Item it;
  if (!find_item(T, S, vb, it)) return;
  constexpr bool PRE = !SPLIT && !SOFTMAX;  // fast precision: prescaled scores (sigmoid_pre)
  const int n = it.n;
  const int tid = threadIdx.x, lane = tid & 63, l32 = lane & 31, hf = lane >> 5;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const float c2 = item_c2(S, it);
  const float sarg = PRE ? item_bias_factor(S, it, c2) : c2;
  const TrFrag<D> tr(lane);
  const FragAddr<D> fa(l32, hf);
  const TileDma<BK, D> dma_k(w, lane, S.sl[1]), dma_v(w, lane, S.sl[2]);
  auto Kb = [&](int i) { return lds.p[i]; };
  auto Vb = [&](int i) { return lds.p[3 + i]; };
  const Slice qs(slice_base(Q, S, it.bh, 0), n, S.sl[0]), ks(slice_base(K, S, it.bh, 1), n, S.sl[1]),
      vs(slice_base(V, S, it.bh, 2), n, S.sl[2]), gs(slice_base(dO, S, it.bh, 3), n, S.sl[3]);
  // the first tiles load while the fragments below are read
  dma_k.load(ks, 0, Kb(0));
  dma_k.load(ks, BK, Kb(1));
  dma_v.load(vs, 0, Vb(0));

  const int qrow = it.tile * BQ + 32 * w + l32;
  e16x8 qf[D / 16], gf[D / 16];
  if (PRE) load_bfrag_scaled<D>(qf, qs, qrow, hf, score_c1<D>());
  else load_bfrag<D>(qf, qs, qrow, hf);
  load_bfrag<D>(gf, gs, qrow, hf);
  f32x16 acc[D / 32];
#pragma unroll
  for (int i = 0; i < D / 32; ++i) acc[i] = (f32x16){};
  float lse2 = 0.0f, dlt = 0.0f;  // softmax: this lane's query row
  if constexpr (SOFTMAX) {
    if (qrow < n) {
      lse2 = LSE[(size_t)it.bh * S.Lmax + qrow];
      dlt = DELTA[(size_t)it.bh * S.Lmax + qrow];
    }
  }

  const int nk = S.causal ? min((n + BK - 1) / BK, causal_inner_end(it.tile, BQ, BK)) : (n + BK - 1) / BK;
  const int q0w = it.tile * BQ + 32 * w;  // this wave's first query
  vm_drain();
  __syncthreads();
  f32x16 sA[2], sB[2];
  zero2(sA);
  score_steps<D>(sA, Kb(0), qf, 0, D / 16, fa);

  auto step = [&](auto phase, int j) {
    constexpr int P = decltype(phase)::value;
    constexpr int kc = P % 3, k1 = (P + 1) % 3, k2 = (P + 2) % 3;
    f32x16(&cur)[2] = pick<P>(sA, sB);
    f32x16(&nxt)[2] = pick<P + 1>(sA, sB);
    dma_k.load(ks, (j + 2) * BK, Kb(k2));
    dma_v.load(vs, (j + 1) * BK, Vb((P + 1) % 2));
    const uint16_t* Kt = Kb(kc);
    const uint16_t* Kn = Kb(k1);
    const uint16_t* Vc = Vb(P % 2);
    if (S.causal && j * BK + BK - 1 > q0w) mask_causal_cols(cur, j * BK, qrow, hf, masked_score<PRE>());
    f32x16 dp[2];
    zero2(dp);
    zero2(nxt);
    score_pipelined<D>(dp, Vc, gf, fa);
    e16x8 dh[4], dl[4], unused_h, unused_l;
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      score_steps<D>(nxt, Kn, qf, c * (D / 64), (c + 1) * (D / 64), fa);  // MFMA: tile j+1
      if constexpr (SOFTMAX)
        dsoftmax_chunk_col<D, SPLIT>(cur, dp, c, lse2, dlt, dh[c], dl[c]);
      else
        dsigmoid_chunk<D, SPLIT, PRE, false>(cur, dp, c, sarg, dh[c], dl[c], unused_h, unused_l);
      if (c > 0) value_chunk<D, SPLIT>(acc, tr, Kt, c - 1, dh[c - 1], dl[c - 1]);
    }
    value_chunk<D, SPLIT>(acc, tr, Kt, 3, dh[3], dl[3]);
    vm_drain();
    __syncthreads();
  };
  run_steps(nk, step);

  if (qrow < n) {
    const float scale = S.out_scale;
    uint16_t* dst = slice_base(dQ, S, it.bh, 4) + (size_t)qrow * S.sl[4];
#pragma unroll
    for (int db = 0; db < D / 32; ++db)
#pragma unroll
      for (int i = 0; i < 4; ++i) store4(dst + 32 * db + 8 * i + 4 * hf, acc[db], i, scale);
  }
}

template <int D, bool SPLIT, bool SOFTMAX = false>
__global__ __launch_bounds__(kThreads, DqCfg<D>::OCC) void dq_kernel(
    const uint16_t* __restrict__ Q, const uint16_t* __restrict__ K, const uint16_t* __restrict__ V,
    const uint16_t* __restrict__ dO, uint16_t* __restrict__ dQ, const float* __restrict__ LSE,
    const float* __restrict__ DELTA, const SeqTable T, const Sched S) {
  SIGATTN_RING(lds, 5, kInner * D, D == 64);  // K0 K1 K2 V0 V1
  dq_body<D, SPLIT, SOFTMAX>(lds, (int)blockIdx.x, Q, K, V, dO, dQ, LSE, DELTA, T, S);
}

// ---------------------------------------------------------------------------
// Backward, dK/dV.  Item = (b, h, 128-key tile).  Inner loop: 64-query tiles j.
// Per wave (32 keys): S_j = Q_j . K^T (64 queries x 32 keys), dP_j = dO_j . V^T,
// P_j = sigma, dS_j = dP_j * P(1-P), dV^T (d x 32 keys) += dO_j^T . P_j,
// dK^T += Q_j^T . dS_j.  Each workgroup owns its rows of dK and dV: one
// writer per row, no atomics.
// LDS: Q and dO in 3 stages each (tile j: transposing reads for dK, dV;
// tile j+1: scores; tile j+2: loading).  Per 16-row chunk the transposing
// reads are issued before the VALU block that computes P and dS, so their
// latency is covered; the next tile's S and dP follow, with the fragments of
// each K-step read one step ahead.
// ---------------------------------------------------------------------------
// softmax: lse2 and delta of each inner tile's rows, 3 stages
template <int D, bool SOFTMAX>
constexpr int dkdv_row_floats() { return SOFTMAX ? 6 * DkdvCfg<D>::BQ : 4; }

// The dK/dV work of block vb of schedule S (a kernel of its own, or the dK/dV
// part of the fused backward launch); lds: six stages of BQ x D elements,
// rowv: dkdv_row_floats<D, SOFTMAX>() floats.
template <int D, bool SPLIT, bool SOFTMAX, bool DB>
__device__ __forceinline__ void dkdv_body(const Ring& lds, float* __restrict__ rowv, int vb,
                                          const uint16_t* __restrict__ Q, const uint16_t* __restrict__ K,
                                          const uint16_t* __restrict__ V, const uint16_t* __restrict__ dO,
                                          uint16_t* __restrict__ dK, uint16_t* __restrict__ dV,
                                          const float* __restrict__ LSE, const float* __restrict__ DELTA,
                                          float* __restrict__ DBIAS, const SeqTable& T, const Sched& S) {
  constexpr int BKV = 128, BQ = DkdvCfg<D>::BQ, NMB = BQ / 32, NC = BQ / 16;

  if (vb >= S.compute_blocks) {
    zero_padded_rows<D>(T, S, vb, dK, 4, dV, 5, DB ? DBIAS : nullptr);
    return;
  }
  Item it;
  if (!find_item(T, S, vb, it)) return;
  constexpr bool PRE = !SPLIT && !SOFTMAX;  // fast precision: prescaled scores (sigmoid_pre)
  const int n = it.n;
  const int tid = threadIdx.x, lane = tid & 63, l32 = lane & 31, hf = lane >> 5;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const float c2 = item_c2(S, it);
  const float sarg = PRE ? item_bias_factor(S, it, c2) : c2;
  const TrFrag<D> tr(lane);
  const FragAddr<D> fa(l32, hf);
  const TileDma<BQ, D> dma_q(w, lane, S.sl[0]), dma_g(w, lane, S.sl[3]);
  auto Qb = [&](int i) { return lds.p[i]; };
  auto Gb = [&](int i) { return lds.p[3 + i]; };
  const Slice qs(slice_base(Q, S, it.bh, 0), n, S.sl[0]), ks(slice_base(K, S, it.bh, 1), n, S.sl[1]),
      vs(slice_base(V, S, it.bh, 2), n, S.sl[2]), gs(slice_base(dO, S, it.bh, 3), n, S.sl[3]);
  const int nq = (n + BQ - 1) / BQ;
  // causal: query tiles before this key tile's first key see none of it
  const int j0 = S.causal ? causal_first_inner(it.tile, BKV, BQ) : 0;
  const int k0w = it.tile * BKV + 32 * w;  // this wave's first key
  // softmax: wave 0 streams lse2, wave 1 delta (one value per lane and row)
  const RowDma<BQ> rdma(SOFTMAX && w < 2 ? (w == 0 ? LSE : DELTA) + (size_t)it.bh * S.Lmax : nullptr, n, lane);
  auto Rb = [&](int i) { return rowv + (2 * i + (w & 1)) * BQ; };
  auto row_load = [&](int row0, int i) {
    if constexpr (SOFTMAX)
      if (w < 2) rdma.load(row0, Rb(i));
  };
  // the first tiles load while the fragments below are read
  dma_q.load(qs, j0 * BQ, Qb(0));
  dma_g.load(gs, j0 * BQ, Gb(0));
  dma_q.load(qs, (j0 + 1) * BQ, Qb(1));
  dma_g.load(gs, (j0 + 1) * BQ, Gb(1));
  row_load(j0 * BQ, 0);
  row_load((j0 + 1) * BQ, 1);

  const int krow = it.tile * BKV + 32 * w + l32;
  e16x8 kf[D / 16], vf[D / 16];
  if (PRE) load_bfrag_scaled<D>(kf, ks, krow, hf, score_c1<D>());
  else load_bfrag<D>(kf, ks, krow, hf);
  load_bfrag<D>(vf, vs, krow, hf);
  f32x16 dk[D / 32], dv[D / 32];
#pragma unroll
  for (int i = 0; i < D / 32; ++i) {
    dk[i] = (f32x16){};
    dv[i] = (f32x16){};
  }

  vm_drain();
  __syncthreads();
  float dsum = 0.0f;  // with DB: sum of this lane's dS values (its key column)
  if constexpr (DkdvCfg<D>::ROLL) {
    // S and dP of the current query tile as two 32-row blocks.  Block 0 is
    // ready when a step starts; block 1 is computed during the step's first
    // two chunks (while the VALU works on block 0), and block 0 of the next
    // tile during the last two, with each chunk's A fragments read at its
    // start: every chunk mixes score products, sigma and dS on the VALU, and
    // the previous chunk's dV and dK products.
    static_assert(NMB == 2 && NC == 4, "two 32-row blocks, four 16-row chunks");
    constexpr int KS = D / 32;  // score K-steps per chunk
    f32x16 sc[2], gc[2];
    sc[0] = (f32x16){};
    gc[0] = (f32x16){};
    score_block<D>(sc[0], Qb(0), kf, 0, fa);
    score_block<D>(gc[0], Gb(0), vf, 0, fa);
    auto step = [&](auto phase, int jr) {
      const int j = j0 + jr;  // inner (query) tile
      constexpr int P = decltype(phase)::value;
      constexpr int kc = P % 3, k1 = (P + 1) % 3, k2 = (P + 2) % 3;
      dma_q.load(qs, (j + 2) * BQ, Qb(k2));
      dma_g.load(gs, (j + 2) * BQ, Gb(k2));
      row_load((j + 2) * BQ, k2);
      const uint16_t* Qn = Qb(k1);
      const uint16_t* Gn = Gb(k1);
      const uint16_t* Qt = Qb(kc);
      const uint16_t* Gt = Gb(kc);
      if (S.causal && j * BQ < k0w + 31) mask_causal_block(sc[0], j * BQ, krow, hf, masked_score<PRE>());
      e16x8 dh[NC], dl[NC], ph[NC], pl[NC];
      e16x8 ag[2][D / 32], aq[2][D / 32];
#pragma unroll
      for (int c = 0; c < NC; ++c) {
        // score products of this chunk: block 1 of tile j (c < 2) or block 0
        // of tile j+1 (c >= 2), K-steps KS*(c%2) ..
        const uint16_t* Qs = c < 2 ? Qt : Qn;
        const uint16_t* Gs = c < 2 ? Gt : Gn;
        const int mb = c < 2 ? 1 : 0;
        f32x16& st = sc[c < 2 ? 1 : 0];
        f32x16& gt = gc[c < 2 ? 1 : 0];
        read_value_frags<D>(ag[c & 1], tr, Gt, c);
        read_value_frags<D>(aq[c & 1], tr, Qt, c);
        e16x8 fs[KS], fg[KS];
#pragma unroll
        for (int k = 0; k < KS; ++k) {
          fs[k] = fa.read(Qs, mb, KS * (c & 1) + k);
          fg[k] = fa.read(Gs, mb, KS * (c & 1) + k);
        }
        sched_fence();
        if (c == 2 && S.causal && j * BQ + 32 < k0w + 31)
          mask_causal_block(sc[1], j * BQ + 32, krow, hf, masked_score<PRE>());
        if constexpr (SOFTMAX) {
          const float* lt = rowv + 2 * kc * BQ;  // lse2 of stage kc; delta follows
          const int r0 = 16 * c + 4 * hf;
          const f32x8 lse8 = cat8(*(const f32x4*)(lt + r0), *(const f32x4*)(lt + r0 + 8));
          const f32x8 dlt8 = cat8(*(const f32x4*)(lt + BQ + r0), *(const f32x4*)(lt + BQ + r0 + 8));
          dsoftmax_chunk_row<D, SPLIT>(sc, gc, c, lse8, dlt8, dh[c], dl[c], ph[c], pl[c]);
        } else {
          dsigmoid_chunk<D, SPLIT, PRE, true, DB>(sc, gc, c, sarg, dh[c], dl[c], ph[c], pl[c], &dsum);
        }
        if ((c & 1) == 0) {
          st = (f32x16){};
          gt = (f32x16){};
        }
#pragma unroll
        for (int k = 0; k < KS; ++k) {
          st = mfma(fs[k], kf[KS * (c & 1) + k], st);
          gt = mfma(fg[k], vf[KS * (c & 1) + k], gt);
        }
        if (c > 0) {
          value_chunk_pre<D, SPLIT>(dv, ag[(c - 1) & 1], ph[c - 1], pl[c - 1]);
          value_chunk_pre<D, SPLIT>(dk, aq[(c - 1) & 1], dh[c - 1], dl[c - 1]);
        }
        sched_fence();
      }
      value_chunk_pre<D, SPLIT>(dv, ag[(NC - 1) & 1], ph[NC - 1], pl[NC - 1]);
      value_chunk_pre<D, SPLIT>(dk, aq[(NC - 1) & 1], dh[NC - 1], dl[NC - 1]);
      vm_drain();
      __syncthreads();
    };
    run_steps(nq - j0, step);
  } else {
  f32x16 sA[NMB], dA[NMB], sB[NMB], dB[NMB];
  zero2(sA);
  zero2(dA);
  score_steps<D>(sA, Qb(0), kf, 0, D / 16, fa);
  score_steps<D>(dA, Gb(0), vf, 0, D / 16, fa);

  auto step = [&](auto phase, int jr) {
    const int j = j0 + jr;  // inner (query) tile
    constexpr int P = decltype(phase)::value;
    constexpr int kc = P % 3, k1 = (P + 1) % 3, k2 = (P + 2) % 3;
    f32x16(&cs)[NMB] = pick<P>(sA, sB);
    f32x16(&cd)[NMB] = pick<P>(dA, dB);
    f32x16(&ns)[NMB] = pick<P + 1>(sA, sB);
    f32x16(&nd)[NMB] = pick<P + 1>(dA, dB);
    dma_q.load(qs, (j + 2) * BQ, Qb(k2));
    dma_g.load(gs, (j + 2) * BQ, Gb(k2));
    row_load((j + 2) * BQ, k2);
    if (S.causal && j * BQ < k0w + 31) mask_causal_rows(cs, j * BQ, krow, hf, masked_score<PRE>());
    const uint16_t* Qn = Qb(k1);
    const uint16_t* Gn = Gb(k1);
    const uint16_t* Qt = Qb(kc);
    const uint16_t* Gt = Gb(kc);
    zero2(ns);
    zero2(nd);
    e16x8 dh[NC], dl[NC], ph[NC], pl[NC];
    {
      // Per chunk: issue the transposing reads of dO^T and Q^T, evaluate
      // P and dS on the VALU while they land, with the previous chunk's
      // dV and dK products interleaved into that VALU work.
      e16x8 ag[2][D / 32], aq[2][D / 32];
#pragma unroll
      for (int c = 0; c < NC; ++c) {
        read_value_frags<D>(ag[c & 1], tr, Gt, c);
        read_value_frags<D>(aq[c & 1], tr, Qt, c);
        sched_fence();
        if constexpr (SOFTMAX) {
          const float* lt = rowv + 2 * kc * BQ;  // lse2 of stage kc; delta follows
          const int r0 = 16 * c + 4 * hf;
          const f32x8 lse8 = cat8(*(const f32x4*)(lt + r0), *(const f32x4*)(lt + r0 + 8));
          const f32x8 dlt8 = cat8(*(const f32x4*)(lt + BQ + r0), *(const f32x4*)(lt + BQ + r0 + 8));
          dsoftmax_chunk_row<D, SPLIT>(cs, cd, c, lse8, dlt8, dh[c], dl[c], ph[c], pl[c]);
        } else {
          dsigmoid_chunk<D, SPLIT, PRE, true, DB>(cs, cd, c, sarg, dh[c], dl[c], ph[c], pl[c], &dsum);
        }
        if (c > 0) {
          value_chunk_pre<D, SPLIT>(dv, ag[(c - 1) & 1], ph[c - 1], pl[c - 1]);
          value_chunk_pre<D, SPLIT>(dk, aq[(c - 1) & 1], dh[c - 1], dl[c - 1]);
          // the previous chunk's products spread through this chunk's VALU work
          constexpr int nm = 2 * (D / 32) * (SPLIT ? 2 : 1);
          interleave<nm, 64 / nm>();
        }
        sched_fence();
      }
      value_chunk_pre<D, SPLIT>(dv, ag[(NC - 1) & 1], ph[NC - 1], pl[NC - 1]);
      value_chunk_pre<D, SPLIT>(dk, aq[(NC - 1) & 1], dh[NC - 1], dl[NC - 1]);
      score_pipelined<D>(ns, Qn, kf, fa);
      score_pipelined<D>(nd, Gn, vf, fa);
    }
    vm_drain();
    __syncthreads();
  };
  run_steps(nq - j0, step);
  }

  if constexpr (DB) {
    dsum += __shfl_xor(dsum, 32);  // the other half of the column's query rows
    if (krow < n && hf == 0) DBIAS[(size_t)it.bh * S.Lmax + krow] = dsum;
  }
  if (krow < n) {
    const float scale = S.out_scale;
    uint16_t* dstk = slice_base(dK, S, it.bh, 4) + (size_t)krow * S.sl[4];
    uint16_t* dstv = slice_base(dV, S, it.bh, 5) + (size_t)krow * S.sl[5];
#pragma unroll
    for (int db = 0; db < D / 32; ++db)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        store4(dstk + 32 * db + 8 * i + 4 * hf, dk[db], i, scale);
        store4(dstv + 32 * db + 8 * i + 4 * hf, dv[db], i, 1.0f);
      }
  }
}

template <int D, bool SPLIT, bool SOFTMAX = false, bool DB = false>
__global__ __launch_bounds__(kThreads, DkdvCfg<D>::OCC) void dkdv_kernel(
    const uint16_t* __restrict__ Q, const uint16_t* __restrict__ K, const uint16_t* __restrict__ V,
    const uint16_t* __restrict__ dO, uint16_t* __restrict__ dK, uint16_t* __restrict__ dV,
    const float* __restrict__ LSE, const float* __restrict__ DELTA, float* __restrict__ DBIAS, const SeqTable T,
    const Sched S) {
  SIGATTN_RING(lds, 6, DkdvCfg<D>::BQ * D, D == 64);  // Q0 Q1 Q2 G0 G1 G2
  __shared__ __align__(16) float rowv[dkdv_row_floats<D, SOFTMAX>()];
  dkdv_body<D, SPLIT, SOFTMAX, DB>(lds, rowv, (int)blockIdx.x, Q, K, V, dO, dK, dV, LSE, DELTA, DBIAS, T, S);
}

// ---------------------------------------------------------------------------
// Fused backward: one launch runs the dK/dV work (blocks 0 .. dq_off-1, in
// the dK/dV schedule's order: its items longest first, then its zero fill)
// and the dQ work (blocks dq_off .., the same for dQ).  The two parts share
// nothing but the launch: the dQ items fill the CUs that the dK/dV items
// leave idle towards their end, and one launch's fixed cost is saved.  Each
// workgroup takes one role, so LDS is the larger of the two layouts.
// ---------------------------------------------------------------------------
template <int D, bool SPLIT, bool SOFTMAX = false, bool DB = false>
__global__ __launch_bounds__(kThreads, DqCfg<D>::OCC < DkdvCfg<D>::OCC ? DqCfg<D>::OCC : DkdvCfg<D>::OCC) void
bwd_kernel(const uint16_t* __restrict__ Q, const uint16_t* __restrict__ K, const uint16_t* __restrict__ V,
           const uint16_t* __restrict__ dO, uint16_t* __restrict__ dQ, uint16_t* __restrict__ dK,
           uint16_t* __restrict__ dV, const float* __restrict__ LSE, const float* __restrict__ DELTA,
           float* __restrict__ DBIAS, const BwdSched P) {
  // the two roles use the same stages: dQ items K0 K1 K2 V0 V1, dK/dV items
  // Q0 Q1 Q2 G0 G1 G2
  static_assert(kInner == DkdvCfg<D>::BQ, "one stage size for both roles");
  SIGATTN_RING(lds, 6, kInner * D, D == 64);
  __shared__ __align__(16) float rowv[dkdv_row_floats<D, SOFTMAX>()];
  const int b = (int)blockIdx.x;
  if (b < P.dq_off)
    dkdv_body<D, SPLIT, SOFTMAX, DB>(lds, rowv, b, Q, K, V, dO, dK, dV, LSE, DELTA, DBIAS, P.T, P.kv);
  else
    dq_body<D, SPLIT, SOFTMAX>(lds, b - P.dq_off, Q, K, V, dO, dQ, LSE, DELTA, P.T, P.dq);
}

// ---------------------------------------------------------------------------
// Backward of short sequences, one workgroup per (sequence, head): Lmax <= R
// with R = 128 (4 waves) or 256 (8 waves); sigmoid, fast precision, no mask,
// head dim 64; optionally with the bias-gradient rows.  The two-kernel split of the pages (§2C) recomputes S and dP
// on each side; for long sequences that costs 2/5 more matrix work but keeps
// every workgroup's output private.  When one workgroup holds a whole
// (sequence, head), it owns all of its dQ, dK and dV rows, so the split buys
// nothing: this kernel computes S, dP and dS once.
// Wave w owns keys 32w .. 32w+31.  Phase 1 (as the dK/dV kernel, 64-query
// halves j): S = Q K^T and dP = dO V^T with the key as the lane's column,
// dS = dP sigma (1 - sigma), dV^T += dO^T P, dK^T += Q^T dS; each dS chunk is
// also stored to LDS as dS^T (keys x the 128 queries of the half's pair).
// Phase 2, after each pair of halves: dQ^T += K^T dS^T over all R keys for
// the pair's 128 queries, as eight 32-query x 32-column blocks spread over
// the waves (wave w: query block w % 4, column blocks w / 4 .. in steps of
// R / 128), both operands read from LDS by transposing reads.  At R = 256,
// halves past the sequence's last row skip their work (the workgroup's n is
// uniform), and so, with phase 2 over those keys, do the waves of the second
// 128-key tile when the sequence ends in the first.
// The dS^T buffer keeps each key row's 4-query (8-byte) groups in order up
// to an XOR of the group index by Y(r) = (r % 4) * 8 + (r / 2) % 8.  An 8-byte
// LDS store serves 16 lanes per cycle over 32 four-byte banks (128 bytes), a
// transposing read 32 lanes over 64 banks (measured: SQ_LDS_BANK_CONFLICT).
// The phase-1 stores (16 consecutive keys, one group) then hit 16 distinct
// groups modulo 16, and the phase-2 reads (4 keys x 8 aligned groups) 32
// distinct groups: no bank conflicts either way.
// LDS: Q, dO, K (R rows each) and the dS^T of one pair (R x 128): 80 KB at
// R = 128 (two workgroups per CU), 160 KB at R = 256 (one of eight waves).
// Rows of dQ, dK and dV from n_b to Lmax - 1 are written as 0 here.
// ---------------------------------------------------------------------------
__device__ __forceinline__ int ds_group(int r, int g) { return g ^ (((r & 3) << 3) | ((r >> 1) & 7)); }

// Rows n .. Lmax-1 of a slice as 0 (16-byte stores, all NT threads).
template <int D, int NT>
__device__ __forceinline__ void zero_rows(uint16_t* p, int rs, int n, int lmax) {
  const u32x4 z = {0u, 0u, 0u, 0u};
  for (int c = (int)threadIdx.x; c < (lmax - n) * (D / 8); c += NT)
    *(u32x4*)(p + (size_t)(n + c / (D / 8)) * rs + 8 * (c % (D / 8))) = z;
}

template <int R> struct SmallCfg {
  static constexpr int NW = R / 32;    // waves
  static constexpr int NT = 64 * NW;   // threads
  static constexpr int OCC = R == 128 ? 2 : 1;  // workgroups per CU the LDS allows
};

// DB: also the bias-gradient rows (per key, the sum of its dS column over the
// valid queries), as the dK/dV kernel writes them.
template <int D, int R, bool DB>
__global__ __launch_bounds__(SmallCfg<R>::NT, SmallCfg<R>::OCC) void bwd_small_kernel(
    const uint16_t* __restrict__ Q, const uint16_t* __restrict__ K, const uint16_t* __restrict__ V,
    const uint16_t* __restrict__ dO, uint16_t* __restrict__ dQ, uint16_t* __restrict__ dK, uint16_t* __restrict__ dV,
    float* __restrict__ DBIAS, const SeqTable T, const Sched S, const int64_t dq_sb, const int64_t dq_sh,
    const int32_t dq_sl) {
  static_assert(D == 64, "head dim 64");
  static_assert(R == 128 || R == 256, "one or two 128-row tiles");
  constexpr int NW = SmallCfg<R>::NW, NT = SmallCfg<R>::NT, PQ = 128;  // queries per pair
  constexpr int DBW = 8 / NW;  // phase-2 column blocks per wave
  __shared__ __align__(16) uint16_t qt[R * D], gt[R * D], kt[R * D], dst[R * PQ];

  const int s = (int)blockIdx.x / S.H, h = (int)blockIdx.x - s * S.H;
  Item it;
  it.s = s;
  it.n = table_n(T, s);
  it.bh = (T.b_base + s) * S.H + h;
  it.tile = 0;
  const int n = it.n;
  uint16_t* const dqp = dQ + (size_t)(T.b_base + s) * dq_sb + (size_t)h * dq_sh;
  uint16_t* const dkp = slice_base(dK, S, it.bh, 4);
  uint16_t* const dvp = slice_base(dV, S, it.bh, 5);
  if (n == 0) {
    zero_rows<D, NT>(dqp, dq_sl, 0, S.Lmax);
    zero_rows<D, NT>(dkp, S.sl[4], 0, S.Lmax);
    zero_rows<D, NT>(dvp, S.sl[5], 0, S.Lmax);
    if (DB)
      for (int r = (int)threadIdx.x; r < S.Lmax; r += NT) DBIAS[(size_t)it.bh * S.Lmax + r] = 0.0f;
    return;
  }
  const int tid = threadIdx.x, lane = tid & 63, l32 = lane & 31, hf = lane >> 5;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const Slice qs(slice_base(Q, S, it.bh, 0), n, S.sl[0]), ks(slice_base(K, S, it.bh, 1), n, S.sl[1]),
      vs(slice_base(V, S, it.bh, 2), n, S.sl[2]), gs(slice_base(dO, S, it.bh, 3), n, S.sl[3]);
  {
    const TileDma<R, D, NW> dma_q(w, lane, S.sl[0]), dma_g(w, lane, S.sl[3]), dma_k(w, lane, S.sl[1]);
    dma_q.load(qs, 0, qt);
    dma_g.load(gs, 0, gt);
    dma_k.load(ks, 0, kt);
  }
  const int krow = 32 * w + l32;
  // Waves of the second 128-key tile skip their work when the sequence ends
  // in the first (their dS^T rows are then not read).
  const bool keys = R == 128 || w < 4 || n > 128;
  e16x8 kf[D / 16], vf[D / 16];
  load_bfrag_scaled<D>(kf, ks, krow, hf, score_c1<D>());
  load_bfrag<D>(vf, vs, krow, hf);
  const float m = item_bias_factor(S, it, item_c2(S, it));
  const TrFrag<D> tr(lane);
  const FragAddr<D> fa(l32, hf);
  f32x16 dk[D / 32], dv[D / 32];
#pragma unroll
  for (int i = 0; i < D / 32; ++i) {
    dk[i] = (f32x16){};
    dv[i] = (f32x16){};
  }
  float dsum = 0.0f;  // with DB: sum of this lane's dS values (its key column)
  // phase 2: this wave's query block and the B-fragment offsets of its dS^T
  // reads: rows (keys) 16cc + 4hf + j/4 (+ 8), queries 32qb + 16gq + 4(j%4)
  // .. +3 (lane j of each 16, gq = lane / 16 % 2): the key order of TrFrag's
  // reads of K.  Y(16cc + x) = Y(x).
  const int qb = w & 3, db0 = DBW == 2 ? 0 : w >> 2;
  const int j16 = lane & 15, gq = (lane >> 4) & 1;
  const int rl = 4 * hf + (j16 >> 2), grp = 8 * qb + 4 * gq + (j16 & 3);
  int boff[2];  // first / second read
#pragma unroll
  for (int hh = 0; hh < 2; ++hh) boff[hh] = (rl + 8 * hh) * PQ + 4 * ds_group(rl + 8 * hh, grp);
  // TrFrag offsets of this wave's K^T column blocks (selected, not indexed:
  // db0 is a run-time value)
  int koff[DBW][2];
#pragma unroll
  for (int i = 0; i < DBW; ++i)
#pragma unroll
    for (int hh = 0; hh < 2; ++hh)
      koff[i][hh] = DBW == 2 ? tr.off[i][hh] : (db0 ? tr.off[1][hh] : tr.off[0][hh]);
  vm_drain();
  __syncthreads();

#pragma unroll
  for (int j = 0; j < R / 64; ++j) {
    if (keys && (R == 128 || 64 * j < n)) {
      const uint16_t* Qj = qt + 64 * j * D;
      const uint16_t* Gj = gt + 64 * j * D;
      f32x16 sc[2], gc[2];
      zero2(sc);
      zero2(gc);
      score_pipelined<D>(sc, Qj, kf, fa);
      score_pipelined<D>(gc, Gj, vf, fa);
      e16x8 dh[4], dl[4], ph[4], pl[4];
      e16x8 ag[2][D / 32], aq[2][D / 32];
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        read_value_frags<D>(ag[c & 1], tr, Gj, c);
        read_value_frags<D>(aq[c & 1], tr, Qj, c);
        sched_fence();
        dsigmoid_chunk<D, false, true, true, DB>(sc, gc, c, m, dh[c], dl[c], ph[c], pl[c], &dsum);
        // dS^T row: this lane's key; queries 64(j % 2) + 16c + 4hf + {0..3}
        // and + 8 of the pair (groups 16(j % 2) + 4c + hf, + 2)
        const u32x4 pk = as_u32x4(dh[c]);
        const int g0 = 16 * (j & 1) + 4 * c + hf;
        *(uint2*)(dst + krow * PQ + 4 * ds_group(krow, g0)) = (uint2){pk[0], pk[1]};
        *(uint2*)(dst + krow * PQ + 4 * ds_group(krow, g0 + 2)) = (uint2){pk[2], pk[3]};
        if (c > 0) {
          value_chunk_pre<D, false>(dv, ag[(c - 1) & 1], ph[c - 1], pl[c - 1]);
          value_chunk_pre<D, false>(dk, aq[(c - 1) & 1], dh[c - 1], dl[c - 1]);
          interleave<2 * (D / 32), 64 / (2 * (D / 32))>();
        }
        sched_fence();
      }
      value_chunk_pre<D, false>(dv, ag[1], ph[3], pl[3]);
      value_chunk_pre<D, false>(dk, aq[1], dh[3], dl[3]);
    }
    if (j == R / 64 - 1) {  // dK, dV complete
      if constexpr (DB) {
        dsum += __shfl_xor(dsum, 32);  // the other half of the column's query rows
        if (hf == 0 && krow < S.Lmax) DBIAS[(size_t)it.bh * S.Lmax + krow] = krow < n ? dsum : 0.0f;
      }
      const float scale = S.out_scale;
      if (krow < n) {
        uint16_t* rk = dkp + (size_t)krow * S.sl[4];
        uint16_t* rv = dvp + (size_t)krow * S.sl[5];
#pragma unroll
        for (int db = 0; db < D / 32; ++db)
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            store4(rk + 32 * db + 8 * i + 4 * hf, dk[db], i, scale);
            store4(rv + 32 * db + 8 * i + 4 * hf, dv[db], i, 1.0f);
          }
      } else if (krow < S.Lmax) {
        uint16_t* rk = dkp + (size_t)krow * S.sl[4];
        uint16_t* rv = dvp + (size_t)krow * S.sl[5];
#pragma unroll
        for (int i = 0; i < D / 8; ++i) {
          *(uint2*)(rk + 8 * i + 4 * hf) = (uint2){0u, 0u};
          *(uint2*)(rv + 8 * i + 4 * hf) = (uint2){0u, 0u};
        }
      }
    }
    if (j % 2 == 0) continue;
    // Phase 2 for the pair p = j / 2: queries PQ p + 32 qb + l32.
    const int p = j / 2;
    __syncthreads();  // the pair's dS^T is complete
    const int qrow = PQ * p + 32 * qb + l32;
    if (PQ * p < n) {
      f32x16 acc[DBW];
#pragma unroll
      for (int i = 0; i < DBW; ++i) acc[i] = (f32x16){};
#pragma unroll
      for (int cc = 0; cc < R / 16; ++cc) {
        if (cc < 8 || n > 128) {
          const bf16x4 lo = lds_tr4(dst + 16 * cc * PQ + boff[0]);
          const bf16x4 hi = lds_tr4(dst + 16 * cc * PQ + boff[1]);
          const e16x8 b = __builtin_bit_cast(e16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
#pragma unroll
          for (int i = 0; i < DBW; ++i) {
            const bf16x4 alo = lds_tr4(kt + 16 * cc * D + koff[i][0]);
            const bf16x4 ahi = lds_tr4(kt + 16 * cc * D + koff[i][1]);
            const e16x8 a = __builtin_bit_cast(e16x8, __builtin_shufflevector(alo, ahi, 0, 1, 2, 3, 4, 5, 6, 7));
            acc[i] = mfma(a, b, acc[i]);
          }
        }
      }
      if (qrow < n) {
        uint16_t* rq = dqp + (size_t)qrow * dq_sl;
#pragma unroll
        for (int i = 0; i < DBW; ++i)
#pragma unroll
          for (int r4 = 0; r4 < 4; ++r4) store4(rq + 32 * (db0 + i) + 8 * r4 + 4 * hf, acc[i], r4, S.out_scale);
      }
    }
    if (qrow >= n && qrow < S.Lmax) {
      uint16_t* rq = dqp + (size_t)qrow * dq_sl;
#pragma unroll
      for (int i = 0; i < DBW; ++i)
#pragma unroll
        for (int r4 = 0; r4 < 4; ++r4) *(uint2*)(rq + 32 * (db0 + i) + 8 * r4 + 4 * hf) = (uint2){0u, 0u};
    }
    if (j + 1 < R / 64) __syncthreads();  // phase-2 reads done before the next pair's stores
  }
}

// delta = rowsum(dO * O) per row for the softmax backward (0 on padded
// rows); one thread per row, fp32 accumulation of the 16-bit products.
template <int D>
__global__ __launch_bounds__(256) void softmax_prep_kernel(const uint16_t* __restrict__ O,
                                                           const uint16_t* __restrict__ dO,
                                                           float* __restrict__ DELTA, const PrepArgs A) {
  const int64_t gid = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (gid >= (int64_t)A.nb * A.H * A.Lmax) return;
  const int i = (int)(gid % A.Lmax);
  const int bhl = (int)(gid / A.Lmax);
  const int bl = bhl / A.H, h = bhl - bl * A.H, b = A.b0 + bl;
  float acc = 0.0f;
  if (i < A.n[bl]) {
    const uint16_t* po = O + (size_t)b * A.sb[0] + (size_t)h * A.sh[0] + (size_t)i * A.sl[0];
    const uint16_t* pg = dO + (size_t)b * A.sb[1] + (size_t)h * A.sh[1] + (size_t)i * A.sl[1];
#pragma unroll
    for (int c = 0; c < D / 8; ++c) {
      const f32x8 x = to_f32x8(as_e16x8(*(const u32x4*)(po + 8 * c)));
      const f32x8 y = to_f32x8(as_e16x8(*(const u32x4*)(pg + 8 * c)));
#pragma unroll
      for (int t = 0; t < 8; ++t) acc = __builtin_fmaf(x[t], y[t], acc);
    }
  }
  DELTA[((size_t)b * A.H + h) * A.Lmax + i] = acc;
}

template <int D, bool SPLIT>
hipError_t launch_fwd_t(const Launch& L, const void* q, const void* k, const void* v, void* o, hipStream_t st) {
  hipLaunchKernelGGL((fwd_kernel<D, SPLIT>), dim3(L.blocks), dim3(kThreads), 0, st, (const uint16_t*)q,
                     (const uint16_t*)k, (const uint16_t*)v, (uint16_t*)o, L.T, L.sched);
  return hipGetLastError();
}

template <int D, bool SPLIT>
hipError_t launch_dq_t(const Launch& L, const void* q, const void* k, const void* v, const void* g, void* dq,
                       hipStream_t st) {
  hipLaunchKernelGGL((dq_kernel<D, SPLIT>), dim3(L.blocks), dim3(kThreads), 0, st, (const uint16_t*)q,
                     (const uint16_t*)k, (const uint16_t*)v, (const uint16_t*)g, (uint16_t*)dq, (const float*)nullptr,
                     (const float*)nullptr, L.T, L.sched);
  return hipGetLastError();
}

template <int D, bool SPLIT>
hipError_t launch_dkdv_t(const Launch& L, const void* q, const void* k, const void* v, const void* g, void* dk,
                         void* dv, float* dbias, hipStream_t st) {
  if (dbias)
    hipLaunchKernelGGL((dkdv_kernel<D, SPLIT, false, true>), dim3(L.blocks), dim3(kThreads), 0, st,
                       (const uint16_t*)q, (const uint16_t*)k, (const uint16_t*)v, (const uint16_t*)g, (uint16_t*)dk,
                       (uint16_t*)dv, (const float*)nullptr, (const float*)nullptr, dbias, L.T, L.sched);
  else
    hipLaunchKernelGGL((dkdv_kernel<D, SPLIT>), dim3(L.blocks), dim3(kThreads), 0, st, (const uint16_t*)q,
                       (const uint16_t*)k, (const uint16_t*)v, (const uint16_t*)g, (uint16_t*)dk, (uint16_t*)dv,
                       (const float*)nullptr, (const float*)nullptr, (float*)nullptr, L.T, L.sched);
  return hipGetLastError();
}

template <int D, bool SPLIT, bool SOFTMAX, bool DB>
hipError_t launch_bwd_fused_t(const BwdSched& P, int32_t blocks, const void* q, const void* k, const void* v,
                              const void* g, void* dq, void* dk, void* dv, const float* lse, const float* delta,
                              float* dbias, hipStream_t st) {
  hipLaunchKernelGGL((bwd_kernel<D, SPLIT, SOFTMAX, DB>), dim3(blocks), dim3(kThreads), 0, st, (const uint16_t*)q,
                     (const uint16_t*)k, (const uint16_t*)v, (const uint16_t*)g, (uint16_t*)dq, (uint16_t*)dk,
                     (uint16_t*)dv, lse, delta, dbias, P);
  return hipGetLastError();
}

template <int D, bool SPLIT>
hipError_t launch_bwd_fused_d(const BwdSched& P, int32_t blocks, const void* q, const void* k, const void* v,
                              const void* g, void* dq, void* dk, void* dv, const float* lse, const float* delta,
                              float* dbias, hipStream_t st) {
  if (lse) return launch_bwd_fused_t<D, SPLIT, true, false>(P, blocks, q, k, v, g, dq, dk, dv, lse, delta, dbias, st);
  if (dbias) return launch_bwd_fused_t<D, SPLIT, false, true>(P, blocks, q, k, v, g, dq, dk, dv, lse, delta, dbias, st);
  return launch_bwd_fused_t<D, SPLIT, false, false>(P, blocks, q, k, v, g, dq, dk, dv, lse, delta, dbias, st);
}

template <int R, bool DB>
void launch_small_r(int64_t blocks, const Launch& L, const void* q, const void* k, const void* v, const void* g,
                    void* dq, void* dk, void* dv, float* dbias, int64_t dq_sb, int64_t dq_sh, int32_t dq_sl,
                    hipStream_t st) {
  hipLaunchKernelGGL((bwd_small_kernel<64, R, DB>), dim3((unsigned)blocks), dim3(SmallCfg<R>::NT), 0, st,
                     (const uint16_t*)q, (const uint16_t*)k, (const uint16_t*)v, (const uint16_t*)g, (uint16_t*)dq,
                     (uint16_t*)dk, (uint16_t*)dv, dbias, L.T, L.sched, dq_sb, dq_sh, dq_sl);
}

hipError_t launch_bwd_small_t(const Launch& L, const void* q, const void* k, const void* v, const void* g, void* dq,
                              void* dk, void* dv, float* dbias, int64_t dq_sb, int64_t dq_sh, int32_t dq_sl,
                              hipStream_t st) {
  const int64_t blocks = (int64_t)L.T.nseq * L.sched.H;
  if (L.sched.Lmax > 256 || blocks <= 0 || blocks > INT32_MAX) return hipErrorInvalidValue;
  if (L.sched.Lmax <= 128) {
    if (dbias) launch_small_r<128, true>(blocks, L, q, k, v, g, dq, dk, dv, dbias, dq_sb, dq_sh, dq_sl, st);
    else launch_small_r<128, false>(blocks, L, q, k, v, g, dq, dk, dv, dbias, dq_sb, dq_sh, dq_sl, st);
  } else {
    if (dbias) launch_small_r<256, true>(blocks, L, q, k, v, g, dq, dk, dv, dbias, dq_sb, dq_sh, dq_sl, st);
    else launch_small_r<256, false>(blocks, L, q, k, v, g, dq, dk, dv, dbias, dq_sb, dq_sh, dq_sl, st);
  }
  return hipGetLastError();
}

// db[h] = sum over sequences b and rows j of dbias[b, h, j]: one workgroup of
// 1024 threads per head, each thread summing a fixed strided subset (16-byte
// loads when the rows are 16-byte aligned), then a fixed-order tree: the
// result does not depend on timing.
constexpr int kBiasGradThreads = 1024;
__global__ __launch_bounds__(kBiasGradThreads) void bias_grad_kernel(const float* __restrict__ dbias,
                                                                     float* __restrict__ db, int32_t B, int32_t H,
                                                                     int32_t Lmax) {
  __shared__ float part[kBiasGradThreads];
  const int h = (int)blockIdx.x, tid = (int)threadIdx.x;
  float acc = 0.0f;
  if (Lmax % 4 == 0) {
    const int32_t n4 = Lmax / 4;
#pragma unroll 4
    for (int32_t b = 0; b < B; ++b) {
      const f32x4* row = (const f32x4*)(dbias + ((size_t)b * H + h) * Lmax);
      for (int32_t j = tid; j < n4; j += kBiasGradThreads) {
        const f32x4 x = row[j];
        acc += (x[0] + x[1]) + (x[2] + x[3]);
      }
    }
  } else {
    for (int32_t b = 0; b < B; ++b) {
      const float* row = dbias + ((size_t)b * H + h) * Lmax;
      for (int32_t j = tid; j < Lmax; j += kBiasGradThreads) acc += row[j];
    }
  }
  part[tid] = acc;
  __syncthreads();
#pragma unroll
  for (int s = kBiasGradThreads / 2; s > 0; s >>= 1) {
    if (tid < s) part[tid] += part[tid + s];
    __syncthreads();
  }
  if (tid == 0) db[h] = part[0];
}

template <int D, bool SPLIT>
hipError_t launch_softmax_fwd_t(const Launch& L, const void* q, const void* k, const void* v, void* o, float* lse,
                                hipStream_t st) {
  hipLaunchKernelGGL((fwd_softmax_kernel<D, SPLIT>), dim3(L.blocks), dim3(kThreads), 0, st, (const uint16_t*)q,
                     (const uint16_t*)k, (const uint16_t*)v, (uint16_t*)o, lse, L.T, L.sched);
  return hipGetLastError();
}

template <int D, bool SPLIT>
hipError_t launch_softmax_dq_t(const Launch& L, const void* q, const void* k, const void* v, const void* g,
                               const float* lse, const float* delta, void* dq, hipStream_t st) {
  hipLaunchKernelGGL((dq_kernel<D, SPLIT, true>), dim3(L.blocks), dim3(kThreads), 0, st, (const uint16_t*)q,
                     (const uint16_t*)k, (const uint16_t*)v, (const uint16_t*)g, (uint16_t*)dq, lse, delta, L.T, L.sched);
  return hipGetLastError();
}

template <int D, bool SPLIT>
hipError_t launch_softmax_dkdv_t(const Launch& L, const void* q, const void* k, const void* v, const void* g,
                                 const float* lse, const float* delta, void* dk, void* dv, hipStream_t st) {
  hipLaunchKernelGGL((dkdv_kernel<D, SPLIT, true>), dim3(L.blocks), dim3(kThreads), 0, st, (const uint16_t*)q,
                     (const uint16_t*)k, (const uint16_t*)v, (const uint16_t*)g, (uint16_t*)dk, (uint16_t*)dv, lse,
                     delta, (float*)nullptr, L.T, L.sched);
  return hipGetLastError();
}

template <int D>
hipError_t launch_softmax_prep_t(const PrepArgs& A, const void* o, const void* g, float* delta, hipStream_t st) {
  const int64_t rows = (int64_t)A.nb * A.H * A.Lmax;
  hipLaunchKernelGGL((softmax_prep_kernel<D>), dim3((unsigned)((rows + 255) / 256)), dim3(256), 0, st,
                     (const uint16_t*)o, (const uint16_t*)g, delta, A);
  return hipGetLastError();
}

}  // namespace kern

using kern::launch_fwd_t;
using kern::launch_dq_t;
using kern::launch_dkdv_t;

hipError_t launch_fwd(int d, bool split, const Launch& L, const void* q, const void* k, const void* v, void* o,
                      hipStream_t st) {
  if (d == 64) return split ? launch_fwd_t<64, true>(L, q, k, v, o, st) : launch_fwd_t<64, false>(L, q, k, v, o, st);
  return split ? launch_fwd_t<128, true>(L, q, k, v, o, st) : launch_fwd_t<128, false>(L, q, k, v, o, st);
}

hipError_t launch_bwd_dq(int d, bool split, const Launch& L, const void* q, const void* k, const void* v,
                         const void* g, void* dq, hipStream_t st) {
  if (d == 64)
    return split ? launch_dq_t<64, true>(L, q, k, v, g, dq, st) : launch_dq_t<64, false>(L, q, k, v, g, dq, st);
  return split ? launch_dq_t<128, true>(L, q, k, v, g, dq, st) : launch_dq_t<128, false>(L, q, k, v, g, dq, st);
}

hipError_t launch_bwd_dkdv(int d, bool split, const Launch& L, const void* q, const void* k, const void* v,
                           const void* g, void* dk, void* dv, float* dbias, hipStream_t st) {
  if (d == 64)
    return split ? launch_dkdv_t<64, true>(L, q, k, v, g, dk, dv, dbias, st)
                 : launch_dkdv_t<64, false>(L, q, k, v, g, dk, dv, dbias, st);
  return split ? launch_dkdv_t<128, true>(L, q, k, v, g, dk, dv, dbias, st)
               : launch_dkdv_t<128, false>(L, q, k, v, g, dk, dv, dbias, st);
}

hipError_t launch_bwd_fused(int d, bool split, const BwdSched& P, int32_t blocks, const void* q, const void* k,
                            const void* v, const void* g, void* dq, void* dk, void* dv, const float* lse2,
                            const float* delta, float* dbias, hipStream_t st) {
  if (d != 64) return hipErrorInvalidValue;  // d = 128 runs the two launches (see DqCfg)
  return split ? kern::launch_bwd_fused_d<64, true>(P, blocks, q, k, v, g, dq, dk, dv, lse2, delta, dbias, st)
               : kern::launch_bwd_fused_d<64, false>(P, blocks, q, k, v, g, dq, dk, dv, lse2, delta, dbias, st);
}

hipError_t launch_bwd_small(const Launch& L, const void* q, const void* k, const void* v, const void* g, void* dq,
                            void* dk, void* dv, float* dbias, int64_t dq_sb, int64_t dq_sh, int32_t dq_sl,
                            hipStream_t st) {
  return kern::launch_bwd_small_t(L, q, k, v, g, dq, dk, dv, dbias, dq_sb, dq_sh, dq_sl, st);
}

hipError_t launch_bias_grad(int32_t B, int32_t H, int32_t Lmax, const float* dbias, float* db, hipStream_t st) {
  hipLaunchKernelGGL(kern::bias_grad_kernel, dim3((unsigned)H), dim3(kern::kBiasGradThreads), 0, st, dbias, db, B,
                     H, Lmax);
  return hipGetLastError();
}

hipError_t launch_softmax_fwd(int d, bool split, const Launch& L, const void* q, const void* k, const void* v,
                              void* o, float* lse, hipStream_t st) {
  if (d == 64)
    return split ? kern::launch_softmax_fwd_t<64, true>(L, q, k, v, o, lse, st)
                 : kern::launch_softmax_fwd_t<64, false>(L, q, k, v, o, lse, st);
  return split ? kern::launch_softmax_fwd_t<128, true>(L, q, k, v, o, lse, st)
               : kern::launch_softmax_fwd_t<128, false>(L, q, k, v, o, lse, st);
}

hipError_t launch_softmax_dq(int d, bool split, const Launch& L, const void* q, const void* k, const void* v,
                             const void* g, const float* lse, const float* delta, void* dq, hipStream_t st) {
  if (d == 64)
    return split ? kern::launch_softmax_dq_t<64, true>(L, q, k, v, g, lse, delta, dq, st)
                 : kern::launch_softmax_dq_t<64, false>(L, q, k, v, g, lse, delta, dq, st);
  return split ? kern::launch_softmax_dq_t<128, true>(L, q, k, v, g, lse, delta, dq, st)
               : kern::launch_softmax_dq_t<128, false>(L, q, k, v, g, lse, delta, dq, st);
}

hipError_t launch_softmax_dkdv(int d, bool split, const Launch& L, const void* q, const void* k, const void* v,
                               const void* g, const float* lse, const float* delta, void* dk, void* dv,
                               hipStream_t st) {
  if (d == 64)
    return split ? kern::launch_softmax_dkdv_t<64, true>(L, q, k, v, g, lse, delta, dk, dv, st)
                 : kern::launch_softmax_dkdv_t<64, false>(L, q, k, v, g, lse, delta, dk, dv, st);
  return split ? kern::launch_softmax_dkdv_t<128, true>(L, q, k, v, g, lse, delta, dk, dv, st)
               : kern::launch_softmax_dkdv_t<128, false>(L, q, k, v, g, lse, delta, dk, dv, st);
}

hipError_t launch_softmax_prep(int d, const PrepArgs& A, const void* o, const void* g, float* delta,
                               hipStream_t st) {
  return d == 64 ? kern::launch_softmax_prep_t<64>(A, o, g, delta, st)
                 : kern::launch_softmax_prep_t<128>(A, o, g, delta, st);
}

}  // namespace SIGATTN_ELT
}  // namespace sigattn
