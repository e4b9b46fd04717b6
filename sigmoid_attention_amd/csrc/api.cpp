// C-ABI entry points of libsigattn: validation, schedule, launches.
// Every check runs on the host before anything is enqueued, so an error
// return has no side effect.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstdint>
#include <vector>

#include "../../include/sigattn.h"
#include "launch.h"
#include "plan.h"

namespace {

using sigattn::Launch;

constexpr int32_t kFwdOuter = 128, kFwdInner = 64;    // query tile, key tile
constexpr int32_t kDqOuter = 128, kDqInner = 64;      // query tile, key tile
constexpr int32_t kDkdvOuter = 128, kDkdvInner = 64;  // key tile, query tile

sigattn_status tile_rows(int32_t pass, int32_t* outer, int32_t* inner) {
  switch (pass) {
    case SIGATTN_PASS_FWD: *outer = kFwdOuter; *inner = kFwdInner; return SIGATTN_OK;
    case SIGATTN_PASS_BWD_DQ: *outer = kDqOuter; *inner = kDqInner; return SIGATTN_OK;
    case SIGATTN_PASS_BWD_DKDV: *outer = kDkdvOuter; *inner = kDkdvInner; return SIGATTN_OK;
    default: return SIGATTN_ERR_PASS;
  }
}

// Whether the call's tensors are fp16 (else bf16): picks the kernel build.
bool f16(const sigattn_args* a) { return a->dtype == SIGATTN_DTYPE_F16; }

// Shape, lengths, bias, precision, mask and element type (no pointers).
constexpr int64_t kLmaxSlack = 256;  // rows a tile may reach past Lmax, with margin

sigattn_status check_args(const sigattn_args* a) {
  if (!a) return SIGATTN_ERR_NULL;
  if (a->B < 1 || a->H < 1 || a->Lmax < 1 || (a->d != 64 && a->d != 128)) return SIGATTN_ERR_SHAPE;
  // Element count must fit comfortably in 62 bits; B * H must fit the
  // schedule's 32-bit head index; byte offsets within one (sequence, head)
  // slice, up to one tile past Lmax, must fit the kernels' 32-bit buffer
  // offsets (Lmax <= 8,388,351 at d = 128, 16,776,959 at d = 64).
  const double elems = (double)a->B * a->H * a->Lmax * a->d;
  if (elems > 4.0e18 || (int64_t)a->B * a->H > INT32_MAX) return SIGATTN_ERR_SHAPE;
  if (((int64_t)a->Lmax + kLmaxSlack) * a->d * 2 > INT32_MAX) return SIGATTN_ERR_SHAPE;
  if (!a->seqlens) return SIGATTN_ERR_NULL;
  for (int32_t b = 0; b < a->B; ++b)
    if (a->seqlens[b] < 0 || a->seqlens[b] > a->Lmax) return SIGATTN_ERR_SEQLEN;
  switch (a->bias_mode) {
    case SIGATTN_BIAS_NEG_LOG_SEQLEN: break;
    case SIGATTN_BIAS_NEG_LOG_N:
      if (!std::isfinite(a->bias_arg) || !(a->bias_arg > 0.0f)) return SIGATTN_ERR_BIAS;
      break;
    case SIGATTN_BIAS_CONST:
      if (!std::isfinite(a->bias_arg)) return SIGATTN_ERR_BIAS;
      break;
    case SIGATTN_BIAS_PER_HEAD:
      if (!a->head_bias) return SIGATTN_ERR_NULL;
      if ((uintptr_t)a->head_bias % 4) return SIGATTN_ERR_ALIGN;
      break;
    default: return SIGATTN_ERR_BIAS;
  }
  if (a->precision != SIGATTN_PREC_FAST && a->precision != SIGATTN_PREC_SPLIT) return SIGATTN_ERR_PRECISION;
  if (a->mask != SIGATTN_MASK_NONE && a->mask != SIGATTN_MASK_CAUSAL) return SIGATTN_ERR_MASK;
  if (a->dtype != SIGATTN_DTYPE_BF16 && a->dtype != SIGATTN_DTYPE_F16) return SIGATTN_ERR_DTYPE;
  return SIGATTN_OK;
}

// One tensor argument: address and element strides of its [B, H, Lmax, d] view.
struct View {
  uintptr_t p;
  int64_t sb, sh, sl;
};

// Contiguous [B, H, Lmax, d] unless args->strides says otherwise.
// idx: which args->strides entry each of the n tensors uses (null: entry i).
std::vector<View> views(const sigattn_args* a, const void* const* t, int n, const int* idx = nullptr) {
  std::vector<View> v(n);
  for (int i = 0; i < n; ++i) {
    v[i].p = (uintptr_t)t[i];
    if (a->strides) {
      const sigattn_strides& s = a->strides[idx ? idx[i] : i];
      v[i].sb = s.b;
      v[i].sh = s.h;
      v[i].sl = s.l;
    } else {
      v[i].sl = a->d;
      v[i].sh = (int64_t)a->Lmax * a->d;
      v[i].sb = (int64_t)a->H * a->Lmax * a->d;
    }
  }
  return v;
}

// Dimensions (extent > 1) of a view, inner run of d elements included, sorted
// by stride.
struct Dim {
  int64_t e, s;
};

std::vector<Dim> dims(const sigattn_args* a, const View& v) {
  std::vector<Dim> d = {{a->d, 1}};
  if (a->B > 1) d.push_back({a->B, v.sb});
  if (a->H > 1) d.push_back({a->H, v.sh});
  if (a->Lmax > 1) d.push_back({a->Lmax, v.sl});
  std::sort(d.begin(), d.end(), [](const Dim& x, const Dim& y) { return x.s < y.s; });
  return d;
}

// Distinct elements at distinct addresses: each stride at least the extent of
// the dimensions below it (sufficient, and exact for the usual layouts).
bool injective(const sigattn_args* a, const View& v) {
  const std::vector<Dim> d = dims(a, v);
  if (d[0].s < 1) return false;  // a broadcast (zero-stride) dimension
  for (size_t k = 1; k < d.size(); ++k)
    if (d[k].s < d[k - 1].s * d[k - 1].e) return false;
  return true;
}

// Byte range [lo, hi) a view can touch.
void span(const sigattn_args* a, const View& v, uintptr_t& lo, uintptr_t& hi) {
  const int64_t last = (int64_t)(a->B - 1) * v.sb + (int64_t)(a->H - 1) * v.sh + (int64_t)(a->Lmax - 1) * v.sl;
  lo = v.p;
  hi = v.p + 2 * (uintptr_t)(last + a->d);
}

// Whether two views may share an address.  Disjoint address ranges never do.
// Two injective views with the same strides whose footprint repeats with the
// period of their first non-contiguous stride (all outer strides multiples of
// it) occupy residue windows [0, R) and [delta, delta + R) modulo that period,
// R being the contiguous run; they are disjoint when those windows are.
bool may_overlap(const sigattn_args* a, const View& x, const View& y) {
  uintptr_t xl, xh, yl, yh;
  span(a, x, xl, xh);
  span(a, y, yl, yh);
  if (xh <= yl || yh <= xl) return false;
  if (x.sb != y.sb || x.sh != y.sh || x.sl != y.sl || !injective(a, x)) return true;
  std::vector<Dim> d = dims(a, x);
  int64_t run = d[0].e;  // contiguous elements from the start of a run
  size_t k = 1;
  while (k < d.size() && d[k].s == run) run *= d[k++].e;
  if (k == d.size()) return true;  // one contiguous block: ranges already overlap
  const int64_t period = d[k].s;
  for (size_t m = k + 1; m < d.size(); ++m)
    if (d[m].s % period) return true;
  const int64_t delta_bytes = (int64_t)(y.p - x.p);
  if (delta_bytes % 2) return true;
  int64_t r = (delta_bytes / 2) % period;
  if (r < 0) r += period;
  return !(r >= run && r <= period - run);
}

// Null, alignment, stride and aliasing checks.  Inputs may alias one another;
// an output may overlap neither an input nor another output.
sigattn_status check_ptrs(const sigattn_args* a, const void* const* in, int nin, void* const* out, int nout) {
  for (int i = 0; i < nin; ++i)
    if (!in[i]) return SIGATTN_ERR_NULL;
  for (int i = 0; i < nout; ++i)
    if (!out[i]) return SIGATTN_ERR_NULL;
  for (int i = 0; i < nin; ++i)
    if ((uintptr_t)in[i] % 16) return SIGATTN_ERR_ALIGN;
  for (int i = 0; i < nout; ++i)
    if ((uintptr_t)out[i] % 16) return SIGATTN_ERR_ALIGN;
  std::vector<const void*> all(in, in + nin);
  for (int i = 0; i < nout; ++i) all.push_back(out[i]);
  const std::vector<View> v = views(a, all.data(), nin + nout);
  for (int i = 0; i < nin + nout; ++i) {
    const View& t = v[i];
    if (t.sb < 0 || t.sh < 0 || t.sl < 0 || t.sb % 8 || t.sh % 8 || t.sl % 8 || t.sl < a->d)
      return SIGATTN_ERR_STRIDE;
    if (((int64_t)a->Lmax + kLmaxSlack) * t.sl * 2 > INT32_MAX) return SIGATTN_ERR_STRIDE;
    if (i >= nin && !injective(a, t)) return SIGATTN_ERR_STRIDE;
  }
  for (int i = nin; i < nin + nout; ++i)
    for (int j = 0; j < i; ++j)
      if (may_overlap(a, v[i], v[j])) return SIGATTN_ERR_ALIAS;
  return SIGATTN_OK;
}

// The per-head bias values are read while the outputs are written: they may
// overlap inputs but no output (tensors t[nt_in..nt-1], row arrays r[0..nr-1]).
sigattn_status check_head_bias(const sigattn_args* a, const void* const* t, int nt, int nt_in,
                               const void* const* r = nullptr, int nr = 0) {
  if (a->bias_mode != SIGATTN_BIAS_PER_HEAD) return SIGATTN_OK;
  const uintptr_t lo = (uintptr_t)a->head_bias, hi = lo + 4 * (uintptr_t)a->H;
  const std::vector<View> v = views(a, t, nt);
  for (int j = nt_in; j < nt; ++j) {
    uintptr_t tl, th;
    span(a, v[j], tl, th);
    if (lo < th && tl < hi) return SIGATTN_ERR_ALIAS;
  }
  const uintptr_t bytes = (uintptr_t)a->B * a->H * a->Lmax * 4;
  for (int j = 0; j < nr; ++j)
    if (lo < (uintptr_t)r[j] + bytes && (uintptr_t)r[j] < hi) return SIGATTN_ERR_ALIAS;
  return SIGATTN_OK;
}

// fp32 [B, H, Lmax] per-row arrays of the softmax path: null, alignment, and
// no overlap between an output (row array or tensor) and anything else.
sigattn_status check_rows(const sigattn_args* a, const void* const* t, int nt, int nt_in, const void* const* r,
                          int nr, int nr_in) {
  for (int i = 0; i < nr; ++i) {
    if (!r[i]) return SIGATTN_ERR_NULL;
    if ((uintptr_t)r[i] % 16) return SIGATTN_ERR_ALIGN;
  }
  const uintptr_t bytes = (uintptr_t)a->B * a->H * a->Lmax * 4;
  const std::vector<View> v = views(a, t, nt);
  for (int i = 0; i < nr; ++i) {
    const uintptr_t lo = (uintptr_t)r[i], hi = lo + bytes;
    for (int j = 0; j < nr; ++j)
      if (j != i && (i >= nr_in || j >= nr_in) && lo < (uintptr_t)r[j] + bytes && (uintptr_t)r[j] < hi)
        return SIGATTN_ERR_ALIAS;
    for (int j = 0; j < nt; ++j) {
      if (i < nr_in && j < nt_in) continue;  // input against input
      uintptr_t tl, th;
      span(a, v[j], tl, th);
      if (lo < th && tl < hi) return SIGATTN_ERR_ALIAS;
    }
  }
  return SIGATTN_OK;
}

// Strides of the call's tensor arguments, in argument order, into the schedule.
void set_strides(const sigattn_args* a, const void* const* t, int n, Launch& L, const int* idx = nullptr) {
  const std::vector<View> v = views(a, t, n, idx);
  for (int i = 0; i < n; ++i) {
    L.sched.sb[i] = v[i].sb;
    L.sched.sh[i] = v[i].sh;
    L.sched.sl[i] = (int32_t)v[i].sl;
  }
}

sigattn::PlanInput plan_input(const sigattn_args* a, int32_t pass) {
  sigattn::PlanInput in;
  in.B = a->B;
  in.H = a->H;
  in.Lmax = a->Lmax;
  in.d = a->d;
  in.seqlens = a->seqlens;
  tile_rows(pass, &in.outer_rows, &in.inner_rows);
  in.bias_mode = a->bias_mode;
  in.bias_arg = a->bias_arg;
  in.causal = a->mask == SIGATTN_MASK_CAUSAL;
  in.outer_is_key = pass == SIGATTN_PASS_BWD_DKDV;
  return in;
}

template <class F>
sigattn_status run(const sigattn_args* a, int32_t pass, const void* const* t, int n, F&& launch_one) {
  std::vector<Launch> plan = sigattn::build_plan(plan_input(a, pass), nullptr);
  (void)hipGetLastError();  // start from a clean per-thread error state
  for (Launch& L : plan) {
    set_strides(a, t, n, L);
    L.sched.head_bias = a->bias_mode == SIGATTN_BIAS_PER_HEAD ? a->head_bias : nullptr;
    if (launch_one(L) != hipSuccess) return SIGATTN_ERR_HIP;
  }
  return SIGATTN_OK;
}

// Whether the backward of both sides runs as one fused launch: at head dim 64
// when each side's schedule is one launch (all but batches beyond one
// launch's length table).  At head dim 128 the dK/dV kernel runs one wave per
// SIMD and the dQ kernel two, so they run as their own launches.
bool fused_bwd(int32_t d, size_t dkdv_launches, size_t dq_launches) {
  return d == 64 && dkdv_launches == 1 && dq_launches == 1;
}

// Whether the sigmoid backward runs as the short-sequence kernel
// (launch_bwd_small, one workgroup per (sequence, head)): head dim 64, fast
// precision, no mask, every sequence within 256 rows.
constexpr int32_t kSmallBwdRows = 256;
bool small_bwd(const sigattn_args* a, bool softmax) {
  return a->d == 64 && a->precision == SIGATTN_PREC_FAST && a->mask != SIGATTN_MASK_CAUSAL && !softmax &&
         a->Lmax <= kSmallBwdRows;
}

// The backward of both sides: one fused launch (fused_bwd), the dK/dV
// blocks first; otherwise the dK/dV launches run, then the dQ launches.
// t: q, k, v, dout, dq, dk, dv (args->strides order).
// lse2/delta: the softmax path; dbias: the sigmoid bias-gradient rows.
sigattn_status run_bwd(const sigattn_args* a, const void* const* t, const float* lse2, const float* delta,
                       float* dbias) {
  static const int kDq[] = {0, 1, 2, 3, 4}, kKv[] = {0, 1, 2, 3, 5, 6};
  const void* tq[] = {t[0], t[1], t[2], t[3], t[4]};
  const void* tkv[] = {t[0], t[1], t[2], t[3], t[5], t[6]};
  std::vector<Launch> pk = sigattn::build_plan(plan_input(a, SIGATTN_PASS_BWD_DKDV), nullptr);
  std::vector<Launch> pq = sigattn::build_plan(plan_input(a, SIGATTN_PASS_BWD_DQ), nullptr);
  const float* hb = a->bias_mode == SIGATTN_BIAS_PER_HEAD ? a->head_bias : nullptr;
  for (Launch& L : pk) {
    set_strides(a, tkv, 6, L, kKv);
    L.sched.head_bias = hb;
  }
  for (Launch& L : pq) {
    set_strides(a, tq, 5, L, kDq);
    L.sched.head_bias = hb;
  }
  const bool split = a->precision == SIGATTN_PREC_SPLIT;
  const hipStream_t st = (hipStream_t)a->stream;
  const auto impl_fused = f16(a) ? sigattn::f16::launch_bwd_fused : sigattn::bf16::launch_bwd_fused;
  (void)hipGetLastError();
  if (small_bwd(a, lse2 != nullptr)) {
    const View vq = views(a, tq, 5, kDq)[4];
    for (const Launch& L : pk)
      if ((f16(a) ? sigattn::f16::launch_bwd_small : sigattn::bf16::launch_bwd_small)(
              L, t[0], t[1], t[2], t[3], const_cast<void*>(t[4]), const_cast<void*>(t[5]), const_cast<void*>(t[6]),
              dbias, vq.sb, vq.sh, (int32_t)vq.sl, st) != hipSuccess)
        return SIGATTN_ERR_HIP;
    return SIGATTN_OK;
  }
  if (fused_bwd(a->d, pk.size(), pq.size()) && pk[0].T.b_base == pq[0].T.b_base && pk[0].T.nseq == pq[0].T.nseq) {
    sigattn::BwdSched P;  // 14.5 KB, copied into the launch's kernel arguments
    P.T = pk[0].T;
    P.kv = pk[0].sched;
    P.dq = pq[0].sched;
    P.dq_off = (pk[0].blocks + 7) / 8 * 8;
    const int32_t blocks = P.dq_off + pq[0].blocks;
    return impl_fused(a->d, split, P, blocks, t[0], t[1], t[2], t[3], const_cast<void*>(t[4]),
                      const_cast<void*>(t[5]), const_cast<void*>(t[6]), lse2, delta, dbias, st) == hipSuccess
               ? SIGATTN_OK
               : SIGATTN_ERR_HIP;
  }
  for (const Launch& L : pk) {
    const hipError_t e =
        lse2 ? (f16(a) ? sigattn::f16::launch_softmax_dkdv : sigattn::bf16::launch_softmax_dkdv)(
                   a->d, split, L, t[0], t[1], t[2], t[3], lse2, delta, const_cast<void*>(t[5]),
                   const_cast<void*>(t[6]), st)
             : (f16(a) ? sigattn::f16::launch_bwd_dkdv : sigattn::bf16::launch_bwd_dkdv)(
                   a->d, split, L, t[0], t[1], t[2], t[3], const_cast<void*>(t[5]), const_cast<void*>(t[6]), dbias,
                   st);
    if (e != hipSuccess) return SIGATTN_ERR_HIP;
  }
  for (const Launch& L : pq) {
    const hipError_t e =
        lse2 ? (f16(a) ? sigattn::f16::launch_softmax_dq : sigattn::bf16::launch_softmax_dq)(
                   a->d, split, L, t[0], t[1], t[2], t[3], lse2, delta, const_cast<void*>(t[4]), st)
             : (f16(a) ? sigattn::f16::launch_bwd_dq : sigattn::bf16::launch_bwd_dq)(
                   a->d, split, L, t[0], t[1], t[2], t[3], const_cast<void*>(t[4]), st);
    if (e != hipSuccess) return SIGATTN_ERR_HIP;
  }
  return SIGATTN_OK;
}

}  // namespace

extern "C" {

sigattn_status sigattn_fwd(const sigattn_args* a, const void* q, const void* k, const void* v, void* o) {
  sigattn_status s = check_args(a);
  if (s != SIGATTN_OK) return s;
  const void* in[] = {q, k, v};
  void* out[] = {o};
  if ((s = check_ptrs(a, in, 3, out, 1)) != SIGATTN_OK) return s;
  const bool split = a->precision == SIGATTN_PREC_SPLIT;
  const void* t[] = {q, k, v, o};
  if ((s = check_head_bias(a, t, 4, 3)) != SIGATTN_OK) return s;
  return run(a, SIGATTN_PASS_FWD, t, 4, [&](const Launch& L) {
    return (f16(a) ? sigattn::f16::launch_fwd : sigattn::bf16::launch_fwd)(a->d, split, L, q, k, v, o, (hipStream_t)a->stream);
  });
}

sigattn_status sigattn_bwd_dq(const sigattn_args* a, const void* q, const void* k, const void* v, const void* dout,
                              void* dq) {
  sigattn_status s = check_args(a);
  if (s != SIGATTN_OK) return s;
  const void* in[] = {q, k, v, dout};
  void* out[] = {dq};
  if ((s = check_ptrs(a, in, 4, out, 1)) != SIGATTN_OK) return s;
  const bool split = a->precision == SIGATTN_PREC_SPLIT;
  const void* t[] = {q, k, v, dout, dq};
  if ((s = check_head_bias(a, t, 5, 4)) != SIGATTN_OK) return s;
  return run(a, SIGATTN_PASS_BWD_DQ, t, 5, [&](const Launch& L) {
    return (f16(a) ? sigattn::f16::launch_bwd_dq : sigattn::bf16::launch_bwd_dq)(a->d, split, L, q, k, v, dout, dq, (hipStream_t)a->stream);
  });
}

sigattn_status sigattn_bwd_dkdv(const sigattn_args* a, const void* q, const void* k, const void* v,
                                const void* dout, void* dk, void* dv) {
  sigattn_status s = check_args(a);
  if (s != SIGATTN_OK) return s;
  const void* in[] = {q, k, v, dout};
  void* out[] = {dk, dv};
  if ((s = check_ptrs(a, in, 4, out, 2)) != SIGATTN_OK) return s;
  const bool split = a->precision == SIGATTN_PREC_SPLIT;
  const void* t[] = {q, k, v, dout, dk, dv};
  if ((s = check_head_bias(a, t, 6, 4)) != SIGATTN_OK) return s;
  return run(a, SIGATTN_PASS_BWD_DKDV, t, 6, [&](const Launch& L) {
    return (f16(a) ? sigattn::f16::launch_bwd_dkdv : sigattn::bf16::launch_bwd_dkdv)(a->d, split, L, q, k, v, dout, dk, dv, nullptr, (hipStream_t)a->stream);
  });
}

sigattn_status sigattn_bwd_dkdv_dbias(const sigattn_args* a, const void* q, const void* k, const void* v,
                                      const void* dout, void* dk, void* dv, float* dbias) {
  sigattn_status s = check_args(a);
  if (s != SIGATTN_OK) return s;
  const void* in[] = {q, k, v, dout};
  void* out[] = {dk, dv};
  if ((s = check_ptrs(a, in, 4, out, 2)) != SIGATTN_OK) return s;
  const void* t[] = {q, k, v, dout, dk, dv};
  const void* r[] = {dbias};
  if ((s = check_rows(a, t, 6, 4, r, 1, 0)) != SIGATTN_OK) return s;
  if ((s = check_head_bias(a, t, 6, 4, r, 1)) != SIGATTN_OK) return s;
  const bool split = a->precision == SIGATTN_PREC_SPLIT;
  return run(a, SIGATTN_PASS_BWD_DKDV, t, 6, [&](const Launch& L) {
    return (f16(a) ? sigattn::f16::launch_bwd_dkdv : sigattn::bf16::launch_bwd_dkdv)(a->d, split, L, q, k, v, dout, dk, dv, dbias, (hipStream_t)a->stream);
  });
}

sigattn_status sigattn_bwd(const sigattn_args* a, const void* q, const void* k, const void* v, const void* dout,
                           void* dq, void* dk, void* dv, float* dbias) {
  sigattn_status s = check_args(a);
  if (s != SIGATTN_OK) return s;
  const void* in[] = {q, k, v, dout};
  void* out[] = {dq, dk, dv};
  if ((s = check_ptrs(a, in, 4, out, 3)) != SIGATTN_OK) return s;
  const void* t[] = {q, k, v, dout, dq, dk, dv};
  const void* r[] = {dbias};
  const int nr = dbias ? 1 : 0;
  if (nr && (s = check_rows(a, t, 7, 4, r, 1, 0)) != SIGATTN_OK) return s;
  if ((s = check_head_bias(a, t, 7, 4, r, nr)) != SIGATTN_OK) return s;
  return run_bwd(a, t, nullptr, nullptr, dbias);
}

sigattn_status sigattn_softmax_bwd(const sigattn_args* a, const void* q, const void* k, const void* v,
                                   const void* dout, const float* lse2, const float* delta, void* dq, void* dk,
                                   void* dv) {
  sigattn_status s = check_args(a);
  if (s != SIGATTN_OK) return s;
  const void* in[] = {q, k, v, dout};
  void* out[] = {dq, dk, dv};
  if ((s = check_ptrs(a, in, 4, out, 3)) != SIGATTN_OK) return s;
  const void* t[] = {q, k, v, dout, dq, dk, dv};
  const void* r[] = {lse2, delta};
  if ((s = check_rows(a, t, 7, 4, r, 2, 2)) != SIGATTN_OK) return s;
  return run_bwd(a, t, lse2, delta, nullptr);
}

sigattn_status sigattn_bias_grad(const sigattn_args* a, const float* dbias, float* db) {
  sigattn_status s = check_args(a);
  if (s != SIGATTN_OK) return s;
  if (!dbias || !db) return SIGATTN_ERR_NULL;
  if ((uintptr_t)dbias % 16 || (uintptr_t)db % 4) return SIGATTN_ERR_ALIGN;
  const uintptr_t rl = (uintptr_t)dbias, rh = rl + (uintptr_t)a->B * a->H * a->Lmax * 4;
  const uintptr_t ol = (uintptr_t)db, oh = ol + 4 * (uintptr_t)a->H;
  if (ol < rh && rl < oh) return SIGATTN_ERR_ALIAS;
  (void)hipGetLastError();
  if (sigattn::bf16::launch_bias_grad(a->B, a->H, a->Lmax, dbias, db, (hipStream_t)a->stream) != hipSuccess)
    return SIGATTN_ERR_HIP;
  return SIGATTN_OK;
}

sigattn_status sigattn_validate(const sigattn_args* a, int32_t pass, const void* const* t) {
  int32_t o, i;
  if (pass != SIGATTN_PASS_BWD && tile_rows(pass, &o, &i) != SIGATTN_OK) return SIGATTN_ERR_PASS;
  sigattn_status s = check_args(a);
  if (s != SIGATTN_OK) return s;
  if (!t) return SIGATTN_ERR_NULL;
  const int nin = pass == SIGATTN_PASS_FWD ? 3 : 4;
  const int nout = pass == SIGATTN_PASS_BWD ? 3 : pass == SIGATTN_PASS_BWD_DKDV ? 2 : 1;
  void* out[3] = {const_cast<void*>(t[nin]), nout >= 2 ? const_cast<void*>(t[nin + 1]) : nullptr,
                  nout == 3 ? const_cast<void*>(t[nin + 2]) : nullptr};
  if ((s = check_ptrs(a, t, nin, out, nout)) != SIGATTN_OK) return s;
  return check_head_bias(a, t, nin + nout, nin);
}

sigattn_status sigattn_softmax_fwd(const sigattn_args* a, const void* q, const void* k, const void* v, void* o,
                                   float* lse2) {
  sigattn_status s = check_args(a);
  if (s != SIGATTN_OK) return s;
  const void* in[] = {q, k, v};
  void* out[] = {o};
  if ((s = check_ptrs(a, in, 3, out, 1)) != SIGATTN_OK) return s;
  const void* t[] = {q, k, v, o};
  const void* r[] = {lse2};
  if ((s = check_rows(a, t, 4, 3, r, 1, 0)) != SIGATTN_OK) return s;
  const bool split = a->precision == SIGATTN_PREC_SPLIT;
  return run(a, SIGATTN_PASS_FWD, t, 4, [&](const Launch& L) {
    return (f16(a) ? sigattn::f16::launch_softmax_fwd : sigattn::bf16::launch_softmax_fwd)(a->d, split, L, q, k, v, o, lse2, (hipStream_t)a->stream);
  });
}

sigattn_status sigattn_softmax_bwd_prep(const sigattn_args* a, const void* o, const void* dout, float* delta) {
  sigattn_status s = check_args(a);
  if (s != SIGATTN_OK) return s;
  const void* t[] = {o, dout};
  for (const void* p : t) {
    if (!p) return SIGATTN_ERR_NULL;
    if ((uintptr_t)p % 16) return SIGATTN_ERR_ALIGN;
  }
  const std::vector<View> v = views(a, t, 2);
  for (const View& x : v)
    if (x.sb < 0 || x.sh < 0 || x.sl < 0 || x.sb % 8 || x.sh % 8 || x.sl % 8 || x.sl < a->d) return SIGATTN_ERR_STRIDE;
  const void* r[] = {delta};
  if ((s = check_rows(a, t, 2, 2, r, 1, 0)) != SIGATTN_OK) return s;
  (void)hipGetLastError();
  sigattn::PrepArgs A;
  A.H = a->H;
  A.Lmax = a->Lmax;
  for (int i = 0; i < 2; ++i) {
    A.sb[i] = v[i].sb;
    A.sh[i] = v[i].sh;
    A.sl[i] = (int32_t)v[i].sl;
  }
  for (int32_t b0 = 0; b0 < a->B; b0 += sigattn::kPrepSeqs) {
    A.b0 = b0;
    A.nb = std::min(a->B - b0, sigattn::kPrepSeqs);
    for (int32_t i = 0; i < A.nb; ++i) A.n[i] = a->seqlens[b0 + i];
    if ((f16(a) ? sigattn::f16::launch_softmax_prep : sigattn::bf16::launch_softmax_prep)(a->d, A, o, dout, delta, (hipStream_t)a->stream) != hipSuccess)
      return SIGATTN_ERR_HIP;
  }
  return SIGATTN_OK;
}

sigattn_status sigattn_softmax_bwd_dq(const sigattn_args* a, const void* q, const void* k, const void* v,
                                      const void* dout, const float* lse2, const float* delta, void* dq) {
  sigattn_status s = check_args(a);
  if (s != SIGATTN_OK) return s;
  const void* in[] = {q, k, v, dout};
  void* out[] = {dq};
  if ((s = check_ptrs(a, in, 4, out, 1)) != SIGATTN_OK) return s;
  const void* t[] = {q, k, v, dout, dq};
  const void* r[] = {lse2, delta};
  if ((s = check_rows(a, t, 5, 4, r, 2, 2)) != SIGATTN_OK) return s;
  const bool split = a->precision == SIGATTN_PREC_SPLIT;
  return run(a, SIGATTN_PASS_BWD_DQ, t, 5, [&](const Launch& L) {
    return (f16(a) ? sigattn::f16::launch_softmax_dq : sigattn::bf16::launch_softmax_dq)(a->d, split, L, q, k, v, dout, lse2, delta, dq, (hipStream_t)a->stream);
  });
}

sigattn_status sigattn_softmax_bwd_dkdv(const sigattn_args* a, const void* q, const void* k, const void* v,
                                        const void* dout, const float* lse2, const float* delta, void* dk,
                                        void* dv) {
  sigattn_status s = check_args(a);
  if (s != SIGATTN_OK) return s;
  const void* in[] = {q, k, v, dout};
  void* out[] = {dk, dv};
  if ((s = check_ptrs(a, in, 4, out, 2)) != SIGATTN_OK) return s;
  const void* t[] = {q, k, v, dout, dk, dv};
  const void* r[] = {lse2, delta};
  if ((s = check_rows(a, t, 6, 4, r, 2, 2)) != SIGATTN_OK) return s;
  const bool split = a->precision == SIGATTN_PREC_SPLIT;
  return run(a, SIGATTN_PASS_BWD_DKDV, t, 6, [&](const Launch& L) {
    return (f16(a) ? sigattn::f16::launch_softmax_dkdv : sigattn::bf16::launch_softmax_dkdv)(a->d, split, L, q, k, v, dout, lse2, delta, dk, dv,
                                        (hipStream_t)a->stream);
  });
}

sigattn_status sigattn_probe_mfma(int32_t blocks, int32_t iters, float* out, uint64_t* clocks, void* stream) {
  if (!out || !clocks) return SIGATTN_ERR_NULL;
  if ((uintptr_t)out % 4 || (uintptr_t)clocks % 8) return SIGATTN_ERR_ALIGN;
  if (blocks < 1 || blocks > 65536 || iters < 1) return SIGATTN_ERR_SHAPE;
  const uintptr_t ol = (uintptr_t)out, oh = ol + (uintptr_t)blocks * 1024 * 4;
  const uintptr_t cl = (uintptr_t)clocks, ch = cl + 16;
  if (ol < ch && cl < oh) return SIGATTN_ERR_ALIAS;
  (void)hipGetLastError();
  if (sigattn::launch_mfma_probe(blocks, iters, out, (unsigned long long*)clocks, (hipStream_t)stream) !=
      hipSuccess)
    return SIGATTN_ERR_HIP;
  return SIGATTN_OK;
}

const char* sigattn_status_str(sigattn_status s) {
  switch (s) {
    case SIGATTN_OK: return "ok";
    case SIGATTN_ERR_NULL: return "null pointer (args, tensor, seqlens or per-head bias)";
    case SIGATTN_ERR_SHAPE: return "bad shape: B, H, Lmax must be >= 1 and d must be 64 or 128";
    case SIGATTN_ERR_SEQLEN: return "a valid length lies outside [0, Lmax]";
    case SIGATTN_ERR_ALIGN: return "a pointer is misaligned (tensors 16 bytes, per-head bias values 4 bytes)";
    case SIGATTN_ERR_ALIAS: return "an output overlaps an input, another output or the per-head bias values";
    case SIGATTN_ERR_BIAS: return "bad bias: unknown mode, non-finite argument, or n <= 0 for a fixed-n bias";
    case SIGATTN_ERR_PRECISION: return "unknown precision mode";
    case SIGATTN_ERR_HIP: return "HIP kernel launch failed";
    case SIGATTN_ERR_PASS: return "unknown pass";
    case SIGATTN_ERR_MASK: return "unknown mask mode";
    case SIGATTN_ERR_DTYPE: return "unknown element type (bf16 or fp16)";
    case SIGATTN_ERR_STRIDE:
      return "bad strides: negative, not a multiple of 8, row stride below d or too large, or an output "
             "that maps two elements to one address";
  }
  return "unknown status";
}

sigattn_status sigattn_plan_stats(const sigattn_args* a, int32_t pass, int64_t* work_items, int64_t* tile_pairs,
                                  int32_t* launches) {
  int32_t o, i;
  if (pass != SIGATTN_PASS_BWD && tile_rows(pass, &o, &i) != SIGATTN_OK) return SIGATTN_ERR_PASS;
  const sigattn_status s = check_args(a);
  if (s != SIGATTN_OK) return s;
  if (pass == SIGATTN_PASS_BWD) {  // both sides; one launch when run_bwd fuses them
    sigattn::PlanStats sk, sq;
    const size_t lk = sigattn::build_plan(plan_input(a, SIGATTN_PASS_BWD_DKDV), &sk).size();
    const size_t lq = sigattn::build_plan(plan_input(a, SIGATTN_PASS_BWD_DQ), &sq).size();
    if (work_items) *work_items = sk.items + sq.items;
    if (tile_pairs) *tile_pairs = sk.pairs + sq.pairs;
    if (launches)
      *launches = small_bwd(a, false) ? (int32_t)lk : fused_bwd(a->d, lk, lq) ? 1 : (int32_t)(lk + lq);
    return SIGATTN_OK;
  }
  sigattn::PlanStats st;
  const std::vector<Launch> plan = sigattn::build_plan(plan_input(a, pass), &st);
  if (work_items) *work_items = st.items;
  if (tile_pairs) *tile_pairs = st.pairs;
  if (launches) *launches = (int32_t)plan.size();
  return SIGATTN_OK;
}

sigattn_status sigattn_tile_shape(int32_t pass, int32_t d, int32_t* outer_rows, int32_t* inner_rows) {
  int32_t o, i;
  if (tile_rows(pass, &o, &i) != SIGATTN_OK) return SIGATTN_ERR_PASS;
  if (d != 64 && d != 128) return SIGATTN_ERR_SHAPE;
  if (outer_rows) *outer_rows = o;
  if (inner_rows) *inner_rows = i;
  return SIGATTN_OK;
}

}  // extern "C"
