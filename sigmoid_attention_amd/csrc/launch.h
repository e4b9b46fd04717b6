// Kernel launchers (defined in kernels.hip, compiled once per element type:
// sigattn::bf16 for bf16 tensors, sigattn::f16 for fp16 tensors).
#pragma once

#include <hip/hip_runtime.h>

#include "plan.h"

namespace sigattn {

// Arguments of the softmax delta pass: sequences b0 .. b0+nb-1.
constexpr int kPrepSeqs = 256;
struct PrepArgs {
  int32_t H, Lmax, b0, nb;
  int32_t n[kPrepSeqs];
  int64_t sb[2], sh[2];  // strides of O (0) and dO (1)
  int32_t sl[2];
};

// Measurement helper: `blocks` x 1024 threads of back-to-back bf16 MFMAs
// (probe.hip).
hipError_t launch_mfma_probe(int32_t blocks, int32_t iters, float* out, unsigned long long* clocks, hipStream_t st);

namespace bf16 {
#include "launch_decls.inc"
}  // namespace bf16

namespace f16 {
#include "launch_decls.inc"
}  // namespace f16

}  // namespace sigattn
