// Measurement helper, not part of the method: the sustained rate of the bf16
// 32x32x16 MFMA that every attention kernel here uses, and the shader clock
// while it runs, so a measured rate can be set beside the published peak.
#include <hip/hip_runtime.h>

#include "device_common.h"
#include "launch.h"

namespace sigattn {
namespace {

// 1024 threads per block (4 waves per SIMD), each wave running kProbeChains
// independent accumulation chains on register operands; every thread stores
// its sum so nothing is removed.  clocks[0] = shader-clock ticks (s_memtime),
// clocks[1] = 100 MHz ticks (s_memrealtime) over the loop of block 0, wave 0.
constexpr int kProbeThreads = 1024, kProbeChains = 4;
__global__ __launch_bounds__(kProbeThreads) void mfma_probe_kernel(int32_t iters, float* __restrict__ out,
                                                                   unsigned long long* __restrict__ clocks) {
  using namespace sigattn::bf16;
  const int tid = (int)threadIdx.x;
  f32x8 x;
#pragma unroll
  for (int t = 0; t < 8; ++t) x[t] = 1.0f / (float)(tid + t + 1);
  const e16x8 a = to_e16x8(x), b = to_e16x8(x * 0.5f);
  f32x16 c[kProbeChains];
#pragma unroll
  for (int j = 0; j < kProbeChains; ++j) c[j] = (f32x16){};
  const unsigned long long t0 = __builtin_amdgcn_s_memtime(), r0 = __builtin_amdgcn_s_memrealtime();
  for (int32_t i = 0; i < iters; ++i) {
#pragma unroll
    for (int j = 0; j < kProbeChains; ++j) c[j] = mfma(a, b, c[j]);
  }
  const unsigned long long t1 = __builtin_amdgcn_s_memtime(), r1 = __builtin_amdgcn_s_memrealtime();
  float s = 0.0f;
#pragma unroll
  for (int j = 0; j < kProbeChains; ++j)
#pragma unroll
    for (int r = 0; r < 16; ++r) s += c[j][r];
  out[(size_t)blockIdx.x * kProbeThreads + tid] = s;
  if (blockIdx.x == 0 && tid == 0) {
    clocks[0] = t1 - t0;
    clocks[1] = r1 - r0;
  }
}

}  // namespace

hipError_t launch_mfma_probe(int32_t blocks, int32_t iters, float* out, unsigned long long* clocks, hipStream_t st) {
  hipLaunchKernelGGL(mfma_probe_kernel, dim3((unsigned)blocks), dim3(kProbeThreads), 0, st, iters, out, clocks);
  return hipGetLastError();
}

}  // namespace sigattn
