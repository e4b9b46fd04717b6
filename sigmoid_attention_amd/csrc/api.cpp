// C-ABI entry points of libsigattn: validation, schedule, launches.
// Every check runs on the host before anything is enqueued, so an error
// return has no side effect.
#include <hip/hip_runtime.h>

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

// Shape, lengths, bias and precision (no pointers).
constexpr int64_t kLmaxSlack = 256;  // rows a tile may reach past Lmax, with margin

sigattn_status check_args(const sigattn_args* a) {
  if (!a) return SIGATTN_ERR_NULL;
  if (a->B < 1 || a->H < 1 || a->Lmax < 1 || (a->d != 64 && a->d != 128)) return SIGATTN_ERR_SHAPE;
  // Element count must fit comfortably in 62 bits; B * H must fit the
  // schedule's 32-bit head index; byte offsets within one (sequence, head)
  // slice, up to one tile past Lmax, must fit the kernels' 32-bit buffer
  // offsets (Lmax <= 4,194,048 at d = 128, 8,388,352 at d = 64).
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
    default: return SIGATTN_ERR_BIAS;
  }
  if (a->precision != SIGATTN_PREC_FAST && a->precision != SIGATTN_PREC_SPLIT) return SIGATTN_ERR_PRECISION;
  return SIGATTN_OK;
}

struct Span {
  uintptr_t lo, hi;
};

bool overlaps(Span x, Span y) { return x.lo < y.hi && y.lo < x.hi; }

// Null, alignment and aliasing checks.  Inputs may alias one another; an
// output may overlap neither an input nor another output.
sigattn_status check_ptrs(const sigattn_args* a, const void* const* in, int nin, void* const* out, int nout) {
  for (int i = 0; i < nin; ++i)
    if (!in[i]) return SIGATTN_ERR_NULL;
  for (int i = 0; i < nout; ++i)
    if (!out[i]) return SIGATTN_ERR_NULL;
  for (int i = 0; i < nin; ++i)
    if ((uintptr_t)in[i] % 16) return SIGATTN_ERR_ALIGN;
  for (int i = 0; i < nout; ++i)
    if ((uintptr_t)out[i] % 16) return SIGATTN_ERR_ALIGN;
  const uintptr_t bytes = (uintptr_t)a->B * a->H * a->Lmax * a->d * 2;
  for (int i = 0; i < nout; ++i) {
    const Span o = {(uintptr_t)out[i], (uintptr_t)out[i] + bytes};
    for (int j = 0; j < nin; ++j)
      if (overlaps(o, {(uintptr_t)in[j], (uintptr_t)in[j] + bytes})) return SIGATTN_ERR_ALIAS;
    for (int j = i + 1; j < nout; ++j)
      if (overlaps(o, {(uintptr_t)out[j], (uintptr_t)out[j] + bytes})) return SIGATTN_ERR_ALIAS;
  }
  return SIGATTN_OK;
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
  return in;
}

template <class F>
sigattn_status run(const sigattn_args* a, int32_t pass, F&& launch_one) {
  const std::vector<Launch> plan = sigattn::build_plan(plan_input(a, pass), nullptr);
  (void)hipGetLastError();  // start from a clean per-thread error state
  for (const Launch& L : plan)
    if (launch_one(L) != hipSuccess) return SIGATTN_ERR_HIP;
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
  return run(a, SIGATTN_PASS_FWD, [&](const Launch& L) {
    return sigattn::launch_fwd(a->d, split, L, q, k, v, o, (hipStream_t)a->stream);
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
  return run(a, SIGATTN_PASS_BWD_DQ, [&](const Launch& L) {
    return sigattn::launch_bwd_dq(a->d, split, L, q, k, v, dout, dq, (hipStream_t)a->stream);
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
  return run(a, SIGATTN_PASS_BWD_DKDV, [&](const Launch& L) {
    return sigattn::launch_bwd_dkdv(a->d, split, L, q, k, v, dout, dk, dv, (hipStream_t)a->stream);
  });
}

const char* sigattn_status_str(sigattn_status s) {
  switch (s) {
    case SIGATTN_OK: return "ok";
    case SIGATTN_ERR_NULL: return "null pointer (args, tensor or seqlens)";
    case SIGATTN_ERR_SHAPE: return "bad shape: B, H, Lmax must be >= 1 and d must be 64 or 128";
    case SIGATTN_ERR_SEQLEN: return "a valid length lies outside [0, Lmax]";
    case SIGATTN_ERR_ALIGN: return "a tensor pointer is not 16-byte aligned";
    case SIGATTN_ERR_ALIAS: return "an output overlaps an input or another output";
    case SIGATTN_ERR_BIAS: return "bad bias: unknown mode, non-finite argument, or n <= 0 for a fixed-n bias";
    case SIGATTN_ERR_PRECISION: return "unknown precision mode";
    case SIGATTN_ERR_HIP: return "HIP kernel launch failed";
    case SIGATTN_ERR_PASS: return "unknown pass";
  }
  return "unknown status";
}

sigattn_status sigattn_plan_stats(const sigattn_args* a, int32_t pass, int64_t* work_items, int64_t* tile_pairs,
                                  int32_t* launches) {
  int32_t o, i;
  if (tile_rows(pass, &o, &i) != SIGATTN_OK) return SIGATTN_ERR_PASS;
  const sigattn_status s = check_args(a);
  if (s != SIGATTN_OK) return s;
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
