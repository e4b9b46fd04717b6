// Device helpers shared by the sigmoid attention kernels (gfx950 / CDNA4).
//
// Matrix products use v_mfma_f32_32x32x16_bf16 (bf16 inputs, fp32
// accumulate).  Its register layout, per 64-lane wave, with l32 = lane % 32
// and hf = lane / 32:
//   A (32 x 16, M x K): lane holds row l32, K-slots 8*hf .. 8*hf+7
//   B (16 x 32, K x N): lane holds column l32, K-slots 8*hf .. 8*hf+7
//   C (32 x 32):        lane holds column l32; register r is row
//                       8*(r/4) + 4*hf + (r%4)
// Every product below is arranged so that the operand read from LDS is A and
// the operand held in registers is B, and so that the C layout of the score
// product S^T (keys x queries) feeds the B operand of the second product
// directly: for a 16-wide K-chunk c the lane's eight C values
// r = 8*(c%2) .. 8*(c%2)+7 of block c/2 are the rows
//   16c + 4*hf + {0,1,2,3}  and  16c + 8 + 4*hf + {0,1,2,3}.
// The contraction order inside a chunk does not matter as long as the A
// operand uses the same order, so tiles that feed A along that index are
// stored transposed in LDS with the rows of each 16-chunk permuted as
//   [0-3, 8-11, 4-7, 12-15]  (quads 1 and 2 swapped)
// which makes each lane's eight A values one contiguous 16-byte read.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "plan.h"

namespace sigattn {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x8 __attribute__((ext_vector_type(8)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ f32x16 mfma(bf16x8 a, bf16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ bf16x8 as_bf16x8(u32x4 v) { return __builtin_bit_cast(bf16x8, v); }
__device__ __forceinline__ u32x4 as_u32x4(bf16x8 v) { return __builtin_bit_cast(u32x4, v); }

// sigma(x) with x = s * score + b, in base 2: t = c1 * score + c2 where
// c1 = -log2(e)/sqrt(d), c2 = -b*log2(e); sigma = 1/(1 + 2^t).  This is the
// identity sigma(x) = 1/(1 + e^-x) evaluated with the hardware base-2
// exponential (v_exp_f32) and reciprocal (v_rcp_f32), each about 1 ulp.  For
// t -> +inf, 2^t = inf and the reciprocal gives 0; for t -> -inf it gives 1;
// no NaN arises from finite scores.
__device__ __forceinline__ float sigmoid2(float score, float c1, float c2) {
  return __builtin_amdgcn_rcpf(1.0f + __builtin_amdgcn_exp2f(__builtin_fmaf(score, c1, c2)));
}

// Round 8 floats to bf16 (round-to-nearest-even, v_cvt_pk_bf16_f32).
__device__ __forceinline__ bf16x8 to_bf16x8(f32x8 x) { return __builtin_convertvector(x, bf16x8); }

// Widen bf16 back to float exactly (bits << 16).
__device__ __forceinline__ f32x8 to_f32x8(bf16x8 x) { return __builtin_convertvector(x, f32x8); }

// Position of row r (0..63, or any multiple-of-16 range) inside a transposed
// tile: quads 1 and 2 of every 16-row chunk trade places.
__device__ __forceinline__ int perm_pos(int r) {
  const int q4 = (r >> 2) & 3;
  const int pq = ((q4 & 1) << 1) | (q4 >> 1);
  return (r & ~15) | (pq << 2) | (r & 3);
}

// The eight values of C register block `blk` that form K-chunk `half` (0/1).
__device__ __forceinline__ f32x8 chunk8(const f32x16& c, int half) {
  f32x8 r;
#pragma unroll
  for (int t = 0; t < 8; ++t) r[t] = c[8 * half + t];
  return r;
}

// A global tile of ROWS x D bf16 rows (row stride D elements) staged through
// registers.  Thread `tid` (0..255) owns NP row pairs (2kp, 2kp+1) of one
// 8-column group each: pair index p = tid + 256*i, kp = p / (D/8),
// col8 = p % (D/8).  Eight consecutive lanes read one full 2*D-byte row, so
// global loads are coalesced 16-byte vectors.  Rows at or beyond `valid` are
// zero-filled and never read from memory (so padding garbage, even NaN/Inf,
// cannot reach the products).
template <int ROWS, int D>
struct TileRegs {
  static constexpr int NP = ROWS * D / (16 * 256);
  static_assert(NP >= 1 && ROWS * D == NP * 16 * 256, "tile must split evenly over 256 threads");
  u32x4 r0[NP], r1[NP];

  __device__ __forceinline__ void load(const uint16_t* __restrict__ src, int row0, int valid, int tid) {
#pragma unroll
    for (int i = 0; i < NP; ++i) {
      const int p = tid + 256 * i;
      const int kp = p / (D / 8), col8 = p % (D / 8);
      const int ra = row0 + 2 * kp, rb = ra + 1;
      const u32x4 z = {0u, 0u, 0u, 0u};
      r0[i] = ra < valid ? *(const u32x4*)(src + (size_t)ra * D + 8 * col8) : z;
      r1[i] = rb < valid ? *(const u32x4*)(src + (size_t)rb * D + 8 * col8) : z;
    }
  }

  // Row-major copy: lds[row * STRIDE + col].
  template <int STRIDE>
  __device__ __forceinline__ void store_rows(uint16_t* lds, int tid) const {
#pragma unroll
    for (int i = 0; i < NP; ++i) {
      const int p = tid + 256 * i;
      const int kp = p / (D / 8), col8 = p % (D / 8);
      *(u32x4*)(lds + (2 * kp) * STRIDE + 8 * col8) = r0[i];
      *(u32x4*)(lds + (2 * kp + 1) * STRIDE + 8 * col8) = r1[i];
    }
  }

  // Transposed copy with permuted row order: lds[col * STRIDE + perm_pos(row)].
  // Rows 2kp and 2kp+1 stay adjacent (quads are 4-aligned), so each column
  // element pair is one 4-byte store.
  template <int STRIDE>
  __device__ __forceinline__ void store_cols(uint16_t* lds, int tid) const {
#pragma unroll
    for (int i = 0; i < NP; ++i) {
      const int p = tid + 256 * i;
      const int kp = p / (D / 8), col8 = p % (D / 8);
      const int pos = perm_pos(2 * kp);
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const uint32_t a = r0[i][e >> 1], b = r1[i][e >> 1];
        const uint32_t word = (e & 1) ? ((a >> 16) | (b & 0xffff0000u)) : ((a & 0xffffu) | (b << 16));
        *(uint32_t*)(lds + (8 * col8 + e) * STRIDE + pos) = word;
      }
    }
  }
};

// 16-byte LDS read of an A fragment.
__device__ __forceinline__ bf16x8 lds_frag(const uint16_t* p) { return as_bf16x8(*(const u32x4*)p); }

// Trailing workgroups (blockIdx.x >= compute_blocks) write the padded rows
// n_b..Lmax-1 of one or two outputs as 0 with 16-byte stores; the compute
// workgroups store valid rows only, so no row has two writers.
template <int D>
__device__ __forceinline__ void zero_padded_rows(const Sched& S, uint16_t* __restrict__ o1,
                                                 uint16_t* __restrict__ o2) {
  const int zb = (int)blockIdx.x - S.compute_blocks;
  const int bhl = zb / kZeroSplit, part = zb % kZeroSplit;
  const int bl = bhl / S.H;
  if (bl >= S.zero_nseq) return;
  const int n = S.zero_n[bl];
  const size_t head = (size_t)S.zero_b0 * S.H + bhl;
  const size_t begin = (head * S.Lmax + n) * D;
  const size_t chunks = (size_t)(S.Lmax - n) * (D / 8);
  const u32x4 z = {0u, 0u, 0u, 0u};
  for (size_t c = (size_t)part * blockDim.x + threadIdx.x; c < chunks; c += (size_t)kZeroSplit * blockDim.x) {
    *(u32x4*)(o1 + begin + 8 * c) = z;
    if (o2) *(u32x4*)(o2 + begin + 8 * c) = z;
  }
}

// Work item of this workgroup (see plan.h); false for idle blocks.  The
// result is uniform across the workgroup.
__device__ __forceinline__ bool find_item(const Sched& S, Item& it) {
  return decode_item(S, (int32_t)(blockIdx.x & 7), (int32_t)(blockIdx.x >> 3), it);
}

}  // namespace sigattn
