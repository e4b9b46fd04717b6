// Sigmoid attention kernels for gfx950: fused forward, backward-dQ,
// backward-dK/dV, and the padded-row zero fill.
//
// Method: "Better Models, Faster Training: Sigmoid Attention for single-cell
// Foundation Models", technical summary §2A (O = sigma(Q K^T / sqrt(d) + b) V,
// b = -log n), §2B (sigma' = sigma (1 - sigma), diagonal Jacobian) and §2C
// (fused forward, backward split into a dQ kernel and a dK/dV kernel so no
// atomics are needed, activations recomputed, fully padded blocks skipped).
//
// Design for MI355X (not a translation of the pages' Triton/H100 kernel):
// * one 256-thread workgroup (4 waves of 64) per output tile; each wave owns
//   32 output rows, so every product is a 32x32x16 bf16 MFMA;
// * the streamed tile (K/V in the forward and dQ kernels, Q/dO in the dK/dV
//   kernel) goes global -> registers -> LDS, double-buffered, with the next
//   tile's global loads in flight while the current one is multiplied: one
//   barrier per inner step;
// * tiles feeding an MFMA A operand along the contraction index are written
//   to LDS transposed (see device_common.h for the permuted row order), so
//   the score product's output registers are directly the B operand of the
//   second product: P never leaves registers and is never stored;
// * rows at or beyond n_b are zero-filled on load, never read, so no mask is
//   applied to P: a zero K row gives a finite score and a zero V (or dO, Q)
//   row contributes nothing;
// * with no row normaliser (§2A), partial products need no running max or
//   rescale, and the inner tiles may be visited in any order;
// * padded output rows are written as 0 by trailing workgroups of the same
//   launch (dispatched last, they fill the tail), so each call is one launch.
#include "device_common.h"
#include "launch.h"
#include "plan.h"

namespace sigattn {

namespace {

constexpr int kThreads = 256;

// ---------------------------------------------------------------------------
// Forward.  Item = (b, h, 128-query tile).  Inner loop: 64-key tiles.
// Per wave and key tile: S^T (64 keys x 32 queries) = K . Q^T, P = sigma,
// O^T (d x 32 queries) += V^T . P^T.
// ---------------------------------------------------------------------------
template <int D, bool SPLIT>
__global__ __launch_bounds__(kThreads, 2) void fwd_kernel(const uint16_t* __restrict__ Q,
                                                          const uint16_t* __restrict__ K,
                                                          const uint16_t* __restrict__ V,
                                                          uint16_t* __restrict__ O, const Sched S) {
  constexpr int BQ = 128, BK = 64;
  constexpr int KS = D + 8;   // K tile row stride (elements); +16 B keeps 16-B reads conflict-free
  constexpr int VS = BK + 8;  // V^T tile row stride
  constexpr int KE = BK * KS, VE = D * VS, STAGE = KE + VE;
  __shared__ __align__(16) uint16_t lds[2 * STAGE];

  if ((int)blockIdx.x >= S.compute_blocks) {
    zero_padded_rows<D>(S, O, nullptr);
    return;
  }
  Item it;
  if (!find_item(S, it)) return;
  const int n = it.n;
  const size_t base = (size_t)it.bh * S.Lmax * D;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6, l32 = lane & 31, hf = lane >> 5;
  const float c1 = S.c1, c2 = it.c2;

  const int qrow = it.tile * BQ + 32 * w + l32;
  bf16x8 qf[D / 16];
#pragma unroll
  for (int s = 0; s < D / 16; ++s) {
    const u32x4 z = {0u, 0u, 0u, 0u};
    qf[s] = as_bf16x8(qrow < n ? *(const u32x4*)(Q + base + (size_t)qrow * D + 16 * s + 8 * hf) : z);
  }

  f32x16 acc[D / 32];
#pragma unroll
  for (int i = 0; i < D / 32; ++i) acc[i] = (f32x16){};

  const int nk = (n + BK - 1) / BK;
  TileRegs<BK, D> kr, vr;
  kr.load(K + base, 0, n, tid);
  vr.load(V + base, 0, n, tid);
  kr.template store_rows<KS>(lds, tid);
  vr.template store_cols<VS>(lds + KE, tid);
  __syncthreads();

  for (int kt = 0; kt < nk; ++kt) {
    const uint16_t* Ks = lds + (kt & 1) * STAGE;
    const uint16_t* Vt = Ks + KE;
    if (kt + 1 < nk) {
      kr.load(K + base, (kt + 1) * BK, n, tid);
      vr.load(V + base, (kt + 1) * BK, n, tid);
    }
    f32x16 st[2] = {(f32x16){}, (f32x16){}};
#pragma unroll
    for (int s = 0; s < D / 16; ++s) {
#pragma unroll
      for (int mb = 0; mb < 2; ++mb)
        st[mb] = mfma(lds_frag(Ks + (32 * mb + l32) * KS + 16 * s + 8 * hf), qf[s], st[mb]);
    }
    bf16x8 ph[4], pl[4];
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      f32x8 p = chunk8(st[c >> 1], c & 1);
#pragma unroll
      for (int t = 0; t < 8; ++t) p[t] = sigmoid2(p[t], c1, c2);
      ph[c] = to_bf16x8(p);
      if (SPLIT) pl[c] = to_bf16x8(p - to_f32x8(ph[c]));
    }
#pragma unroll
    for (int c = 0; c < 4; ++c) {
#pragma unroll
      for (int db = 0; db < D / 32; ++db) {
        const bf16x8 a = lds_frag(Vt + (32 * db + l32) * VS + 16 * c + 8 * hf);
        acc[db] = mfma(a, ph[c], acc[db]);
        if (SPLIT) acc[db] = mfma(a, pl[c], acc[db]);
      }
    }
    if (kt + 1 < nk) {
      uint16_t* nxt = lds + ((kt + 1) & 1) * STAGE;
      kr.template store_rows<KS>(nxt, tid);
      vr.template store_cols<VS>(nxt + KE, tid);
    }
    __syncthreads();
  }

  if (qrow < n) {
    uint16_t* dst = O + base + (size_t)qrow * D;
#pragma unroll
    for (int db = 0; db < D / 32; ++db) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        f32x8 v8;
#pragma unroll
        for (int t = 0; t < 4; ++t) { v8[t] = acc[db][4 * i + t]; v8[4 + t] = 0.0f; }
        const u32x4 packed = as_u32x4(to_bf16x8(v8));
        uint2 out = {packed[0], packed[1]};
        *(uint2*)(dst + 32 * db + 8 * i + 4 * hf) = out;
      }
    }
  }
}

// ---------------------------------------------------------------------------
// Backward, dQ.  Item = (b, h, 128-query tile).  Inner loop: 64-key tiles.
// Per wave and key tile: S^T = K . Q^T, dP^T = V . dO^T, dS^T = dP^T * P(1-P),
// dQ^T (d x 32 queries) += K^T . dS^T.  dQ = dQ^T^T / sqrt(d).
// ---------------------------------------------------------------------------
template <int D, bool SPLIT>
__global__ __launch_bounds__(kThreads, (D == 64 ? 2 : 1)) void dq_kernel(
    const uint16_t* __restrict__ Q, const uint16_t* __restrict__ K, const uint16_t* __restrict__ V,
    const uint16_t* __restrict__ dO, uint16_t* __restrict__ dQ, const Sched S) {
  constexpr int BQ = 128, BK = 64;
  constexpr int RS = D + 8;   // row-major K and V tiles
  constexpr int TS = BK + 8;  // transposed K tile
  constexpr int KE = BK * RS, TE = D * TS, STAGE = 2 * KE + TE;
  __shared__ __align__(16) uint16_t lds[2 * STAGE];

  if ((int)blockIdx.x >= S.compute_blocks) {
    zero_padded_rows<D>(S, dQ, nullptr);
    return;
  }
  Item it;
  if (!find_item(S, it)) return;
  const int n = it.n;
  const size_t base = (size_t)it.bh * S.Lmax * D;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6, l32 = lane & 31, hf = lane >> 5;
  const float c1 = S.c1, c2 = it.c2;

  const int qrow = it.tile * BQ + 32 * w + l32;
  bf16x8 qf[D / 16], gf[D / 16];
#pragma unroll
  for (int s = 0; s < D / 16; ++s) {
    const u32x4 z = {0u, 0u, 0u, 0u};
    const size_t off = base + (size_t)qrow * D + 16 * s + 8 * hf;
    qf[s] = as_bf16x8(qrow < n ? *(const u32x4*)(Q + off) : z);
    gf[s] = as_bf16x8(qrow < n ? *(const u32x4*)(dO + off) : z);
  }

  f32x16 acc[D / 32];
#pragma unroll
  for (int i = 0; i < D / 32; ++i) acc[i] = (f32x16){};

  const int nk = (n + BK - 1) / BK;
  TileRegs<BK, D> kr, vr;
  kr.load(K + base, 0, n, tid);
  vr.load(V + base, 0, n, tid);
  kr.template store_rows<RS>(lds, tid);
  vr.template store_rows<RS>(lds + KE, tid);
  kr.template store_cols<TS>(lds + 2 * KE, tid);
  __syncthreads();

  for (int kt = 0; kt < nk; ++kt) {
    const uint16_t* Ks = lds + (kt & 1) * STAGE;
    const uint16_t* Vs = Ks + KE;
    const uint16_t* Kt = Ks + 2 * KE;
    if (kt + 1 < nk) {
      kr.load(K + base, (kt + 1) * BK, n, tid);
      vr.load(V + base, (kt + 1) * BK, n, tid);
    }
    f32x16 st[2] = {(f32x16){}, (f32x16){}}, dpt[2] = {(f32x16){}, (f32x16){}};
#pragma unroll
    for (int s = 0; s < D / 16; ++s) {
#pragma unroll
      for (int mb = 0; mb < 2; ++mb) {
        st[mb] = mfma(lds_frag(Ks + (32 * mb + l32) * RS + 16 * s + 8 * hf), qf[s], st[mb]);
        dpt[mb] = mfma(lds_frag(Vs + (32 * mb + l32) * RS + 16 * s + 8 * hf), gf[s], dpt[mb]);
      }
    }
    bf16x8 dh[4], dl[4];
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      const f32x8 sv = chunk8(st[c >> 1], c & 1), dv = chunk8(dpt[c >> 1], c & 1);
      f32x8 ds;
#pragma unroll
      for (int t = 0; t < 8; ++t) {
        const float p = sigmoid2(sv[t], c1, c2);
        ds[t] = dv[t] * __builtin_fmaf(-p, p, p);  // dP * p (1 - p)
      }
      dh[c] = to_bf16x8(ds);
      if (SPLIT) dl[c] = to_bf16x8(ds - to_f32x8(dh[c]));
    }
#pragma unroll
    for (int c = 0; c < 4; ++c) {
#pragma unroll
      for (int db = 0; db < D / 32; ++db) {
        const bf16x8 a = lds_frag(Kt + (32 * db + l32) * TS + 16 * c + 8 * hf);
        acc[db] = mfma(a, dh[c], acc[db]);
        if (SPLIT) acc[db] = mfma(a, dl[c], acc[db]);
      }
    }
    if (kt + 1 < nk) {
      uint16_t* nxt = lds + ((kt + 1) & 1) * STAGE;
      kr.template store_rows<RS>(nxt, tid);
      vr.template store_rows<RS>(nxt + KE, tid);
      kr.template store_cols<TS>(nxt + 2 * KE, tid);
    }
    __syncthreads();
  }

  if (qrow < n) {
    const float sc = S.out_scale;
    uint16_t* dst = dQ + base + (size_t)qrow * D;
#pragma unroll
    for (int db = 0; db < D / 32; ++db) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        f32x8 v8;
#pragma unroll
        for (int t = 0; t < 4; ++t) { v8[t] = sc * acc[db][4 * i + t]; v8[4 + t] = 0.0f; }
        const u32x4 packed = as_u32x4(to_bf16x8(v8));
        uint2 out = {packed[0], packed[1]};
        *(uint2*)(dst + 32 * db + 8 * i + 4 * hf) = out;
      }
    }
  }
}

// ---------------------------------------------------------------------------
// Backward, dK/dV.  Item = (b, h, 128-key tile).  Inner loop: 64-query tiles.
// Per wave (32 keys) and query tile: S = Q . K^T (64 queries x 32 keys),
// dP = dO . V^T, P = sigma, dS = dP * P(1-P),
// dV^T (d x 32 keys) += dO^T . P,  dK^T += Q^T . dS.  dK = dK^T^T / sqrt(d).
// Each workgroup owns its rows of dK and dV: one writer per row, no atomics.
// ---------------------------------------------------------------------------
template <int D, bool SPLIT>
__global__ __launch_bounds__(kThreads, (D == 64 ? 2 : 1)) void dkdv_kernel(
    const uint16_t* __restrict__ Q, const uint16_t* __restrict__ K, const uint16_t* __restrict__ V,
    const uint16_t* __restrict__ dO, uint16_t* __restrict__ dK, uint16_t* __restrict__ dV,
    const Sched S) {
  constexpr int BKV = 128, BQ = 64;
  constexpr int RS = D + 8;   // row-major Q and dO tiles
  constexpr int TS = BQ + 8;  // transposed Q and dO tiles
  constexpr int RE = BQ * RS, TE = D * TS, STAGE = 2 * RE + 2 * TE;
  __shared__ __align__(16) uint16_t lds[2 * STAGE];

  if ((int)blockIdx.x >= S.compute_blocks) {
    zero_padded_rows<D>(S, dK, dV);
    return;
  }
  Item it;
  if (!find_item(S, it)) return;
  const int n = it.n;
  const size_t base = (size_t)it.bh * S.Lmax * D;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6, l32 = lane & 31, hf = lane >> 5;
  const float c1 = S.c1, c2 = it.c2;

  const int krow = it.tile * BKV + 32 * w + l32;
  bf16x8 kf[D / 16], vf[D / 16];
#pragma unroll
  for (int s = 0; s < D / 16; ++s) {
    const u32x4 z = {0u, 0u, 0u, 0u};
    const size_t off = base + (size_t)krow * D + 16 * s + 8 * hf;
    kf[s] = as_bf16x8(krow < n ? *(const u32x4*)(K + off) : z);
    vf[s] = as_bf16x8(krow < n ? *(const u32x4*)(V + off) : z);
  }

  f32x16 dk[D / 32], dv[D / 32];
#pragma unroll
  for (int i = 0; i < D / 32; ++i) { dk[i] = (f32x16){}; dv[i] = (f32x16){}; }

  const int nq = (n + BQ - 1) / BQ;
  TileRegs<BQ, D> qr, gr;
  qr.load(Q + base, 0, n, tid);
  gr.load(dO + base, 0, n, tid);
  qr.template store_rows<RS>(lds, tid);
  gr.template store_rows<RS>(lds + RE, tid);
  qr.template store_cols<TS>(lds + 2 * RE, tid);
  gr.template store_cols<TS>(lds + 2 * RE + TE, tid);
  __syncthreads();

  for (int qt = 0; qt < nq; ++qt) {
    const uint16_t* Qs = lds + (qt & 1) * STAGE;
    const uint16_t* Gs = Qs + RE;
    const uint16_t* Qt = Qs + 2 * RE;
    const uint16_t* Gt = Qt + TE;
    if (qt + 1 < nq) {
      qr.load(Q + base, (qt + 1) * BQ, n, tid);
      gr.load(dO + base, (qt + 1) * BQ, n, tid);
    }
    f32x16 sc[2] = {(f32x16){}, (f32x16){}}, dp[2] = {(f32x16){}, (f32x16){}};
#pragma unroll
    for (int s = 0; s < D / 16; ++s) {
#pragma unroll
      for (int mb = 0; mb < 2; ++mb) {
        sc[mb] = mfma(lds_frag(Qs + (32 * mb + l32) * RS + 16 * s + 8 * hf), kf[s], sc[mb]);
        dp[mb] = mfma(lds_frag(Gs + (32 * mb + l32) * RS + 16 * s + 8 * hf), vf[s], dp[mb]);
      }
    }
    bf16x8 ph[4], pl[4], dh[4], dl[4];
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      const f32x8 sv = chunk8(sc[c >> 1], c & 1), gv = chunk8(dp[c >> 1], c & 1);
      f32x8 p8, ds;
#pragma unroll
      for (int t = 0; t < 8; ++t) {
        const float p = sigmoid2(sv[t], c1, c2);
        p8[t] = p;
        ds[t] = gv[t] * __builtin_fmaf(-p, p, p);
      }
      ph[c] = to_bf16x8(p8);
      dh[c] = to_bf16x8(ds);
      if (SPLIT) {
        pl[c] = to_bf16x8(p8 - to_f32x8(ph[c]));
        dl[c] = to_bf16x8(ds - to_f32x8(dh[c]));
      }
    }
#pragma unroll
    for (int c = 0; c < 4; ++c) {
#pragma unroll
      for (int db = 0; db < D / 32; ++db) {
        const bf16x8 ag = lds_frag(Gt + (32 * db + l32) * TS + 16 * c + 8 * hf);
        dv[db] = mfma(ag, ph[c], dv[db]);
        if (SPLIT) dv[db] = mfma(ag, pl[c], dv[db]);
        const bf16x8 aq = lds_frag(Qt + (32 * db + l32) * TS + 16 * c + 8 * hf);
        dk[db] = mfma(aq, dh[c], dk[db]);
        if (SPLIT) dk[db] = mfma(aq, dl[c], dk[db]);
      }
    }
    if (qt + 1 < nq) {
      uint16_t* nxt = lds + ((qt + 1) & 1) * STAGE;
      qr.template store_rows<RS>(nxt, tid);
      gr.template store_rows<RS>(nxt + RE, tid);
      qr.template store_cols<TS>(nxt + 2 * RE, tid);
      gr.template store_cols<TS>(nxt + 2 * RE + TE, tid);
    }
    __syncthreads();
  }

  if (krow < n) {
    const float sc = S.out_scale;
    uint16_t* dstk = dK + base + (size_t)krow * D;
    uint16_t* dstv = dV + base + (size_t)krow * D;
#pragma unroll
    for (int db = 0; db < D / 32; ++db) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        f32x8 k8, v8;
#pragma unroll
        for (int t = 0; t < 4; ++t) {
          k8[t] = sc * dk[db][4 * i + t];
          v8[t] = dv[db][4 * i + t];
          k8[4 + t] = 0.0f;
          v8[4 + t] = 0.0f;
        }
        const u32x4 pk = as_u32x4(to_bf16x8(k8)), pv = as_u32x4(to_bf16x8(v8));
        *(uint2*)(dstk + 32 * db + 8 * i + 4 * hf) = (uint2){pk[0], pk[1]};
        *(uint2*)(dstv + 32 * db + 8 * i + 4 * hf) = (uint2){pv[0], pv[1]};
      }
    }
  }
}

template <int D, bool SPLIT>
hipError_t launch_fwd_t(const Launch& L, const void* q, const void* k, const void* v, void* o, hipStream_t st) {
  hipLaunchKernelGGL((fwd_kernel<D, SPLIT>), dim3(L.blocks), dim3(kThreads), 0, st, (const uint16_t*)q,
                     (const uint16_t*)k, (const uint16_t*)v, (uint16_t*)o, L.sched);
  return hipGetLastError();
}

template <int D, bool SPLIT>
hipError_t launch_dq_t(const Launch& L, const void* q, const void* k, const void* v, const void* g, void* dq,
                       hipStream_t st) {
  hipLaunchKernelGGL((dq_kernel<D, SPLIT>), dim3(L.blocks), dim3(kThreads), 0, st, (const uint16_t*)q,
                     (const uint16_t*)k, (const uint16_t*)v, (const uint16_t*)g, (uint16_t*)dq, L.sched);
  return hipGetLastError();
}

template <int D, bool SPLIT>
hipError_t launch_dkdv_t(const Launch& L, const void* q, const void* k, const void* v, const void* g, void* dk,
                         void* dv, hipStream_t st) {
  hipLaunchKernelGGL((dkdv_kernel<D, SPLIT>), dim3(L.blocks), dim3(kThreads), 0, st, (const uint16_t*)q,
                     (const uint16_t*)k, (const uint16_t*)v, (const uint16_t*)g, (uint16_t*)dk, (uint16_t*)dv,
                     L.sched);
  return hipGetLastError();
}

}  // namespace

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
                           const void* g, void* dk, void* dv, hipStream_t st) {
  if (d == 64)
    return split ? launch_dkdv_t<64, true>(L, q, k, v, g, dk, dv, st)
                 : launch_dkdv_t<64, false>(L, q, k, v, g, dk, dv, st);
  return split ? launch_dkdv_t<128, true>(L, q, k, v, g, dk, dv, st)
               : launch_dkdv_t<128, false>(L, q, k, v, g, dk, dv, st);
}

}  // namespace sigattn
