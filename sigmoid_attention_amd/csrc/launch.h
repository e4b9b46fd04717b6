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
hipError_t launch_bwd_dkdv(int d, bool split, const Launch& L, const void* q, const void* k, const void* v,
                           const void* g, void* dk, void* dv, hipStream_t st);

}  // namespace sigattn
