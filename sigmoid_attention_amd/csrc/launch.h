// Kernel launchers (defined in kernels.hip).  Each enqueues one launch on
// `st` and returns hipGetLastError().  Shapes have been validated by the caller.
#pragma once

#include <hip/hip_runtime.h>

#include "plan.h"

namespace sigattn {

hipError_t launch_fwd(int d, bool split, const Launch& L, const void* q, const void* k, const void* v, void* o,
                      hipStream_t st);
hipError_t launch_bwd_dq(int d, bool split, const Launch& L, const void* q, const void* k, const void* v,
                         const void* g, void* dq, hipStream_t st);
// dbias: null, or fp32 [B, H, Lmax] per-key sums of dX (the bias gradient).
hipError_t launch_bwd_dkdv(int d, bool split, const Launch& L, const void* q, const void* k, const void* v,
                           const void* g, void* dk, void* dv, float* dbias, hipStream_t st);
// db[h] = sum over b, j of dbias[b, h, j].
hipError_t launch_bias_grad(int32_t B, int32_t H, int32_t Lmax, const float* dbias, float* db, hipStream_t st);

// Softmax attention (comparison path): lse2 and delta are fp32 [B, H, Lmax].
hipError_t launch_softmax_fwd(int d, bool split, const Launch& L, const void* q, const void* k, const void* v,
                              void* o, float* lse2, hipStream_t st);
hipError_t launch_softmax_dq(int d, bool split, const Launch& L, const void* q, const void* k, const void* v,
                             const void* g, const float* lse2, const float* delta, void* dq, hipStream_t st);
hipError_t launch_softmax_dkdv(int d, bool split, const Launch& L, const void* q, const void* k, const void* v,
                               const void* g, const float* lse2, const float* delta, void* dk, void* dv,
                               hipStream_t st);

// delta = rowsum(dO * O) for sequences b0 .. b0+nb-1 (nb <= kPrepSeqs).
constexpr int kPrepSeqs = 256;
struct PrepArgs {
  int32_t H, Lmax, b0, nb;
  int32_t n[kPrepSeqs];
  int64_t sb[2], sh[2];  // strides of O (0) and dO (1)
  int32_t sl[2];
};
hipError_t launch_softmax_prep(int d, const PrepArgs& A, const void* o, const void* g, float* delta, hipStream_t st);

}  // namespace sigattn
