// Device helpers shared by the sigmoid attention kernels (gfx950 / CDNA4).
//
// Element type.  The tensors hold 16-bit floats: bf16, or fp16 when the
// kernels are compiled with SIGATTN_FP16.  The library compiles the kernels
// once for each; every definition lives in the namespace sigattn::bf16 or
// sigattn::f16 accordingly, so the two builds link side by side.
//
// Matrix products use v_mfma_f32_32x32x16_bf16 (or _f16; 16-bit inputs, fp32
// accumulate).  Its register layout, per 64-lane wave, with l32 = lane % 32
// and hf = lane / 32:
//   A (32 x 16, M x K): lane holds row l32, K-slots 8*hf .. 8*hf+7
//   B (16 x 32, K x N): lane holds column l32, K-slots 8*hf .. 8*hf+7
//   C (32 x 32):        lane holds column l32; register r is row
//                       8*(r/4) + 4*hf + (r%4)
// Every product below is arranged so that the operand read from LDS is A and
// the operand held in registers is B, and so that the C layout of the score
// product (e.g. S^T, keys x queries) feeds the B operand of the second product
// directly: for a 16-wide K-chunk c the lane's eight C values
// r = 8*(c%2) .. 8*(c%2)+7 of block c/2 are the rows
//   16c + 4*hf + {0,1,2,3}  and  16c + 8 + 4*hf + {0,1,2,3}.
// The contraction order inside a chunk does not matter as long as the A
// operand uses the same order; the A operand of the second product is read
// with transposing LDS reads (see TrFrag) in exactly that order.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

#include "plan.h"

#if defined(SIGATTN_FP16)
#define SIGATTN_ELT f16
#else
#define SIGATTN_ELT bf16
#endif

namespace sigattn {
namespace SIGATTN_ELT {

#if defined(SIGATTN_FP16)
typedef _Float16 e16x8 __attribute__((ext_vector_type(8)));
#else
typedef __bf16 e16x8 __attribute__((ext_vector_type(8)));
#endif
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x8 __attribute__((ext_vector_type(8)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ f32x16 mfma(e16x8 a, e16x8 b, f32x16 c) {
#if defined(SIGATTN_FP16)
  return __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, c, 0, 0, 0);
#else
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
#endif
}

__device__ __forceinline__ e16x8 as_e16x8(u32x4 v) { return __builtin_bit_cast(e16x8, v); }
__device__ __forceinline__ u32x4 as_u32x4(e16x8 v) { return __builtin_bit_cast(u32x4, v); }

// sigma(x) with x = s * score + b, in base 2: t = c1 * score + c2 where
// c1 = -log2(e)/sqrt(d), c2 = -b*log2(e); sigma = 1/(1 + 2^t).  This is the
// identity sigma(x) = 1/(1 + e^-x) evaluated with the hardware base-2
// exponential (v_exp_f32) and reciprocal (v_rcp_f32), each about 1 ulp.  For
// t -> +inf, 2^t = inf and the reciprocal gives 0; for t -> -inf it gives 1;
// no NaN arises from finite scores.
// The score scale c1 for head dim D, a compile-time literal (so the scale
// and bias take one VOP2 fmamk instruction per score).
template <int D>
__device__ __forceinline__ constexpr float score_c1() {
  static_assert(D == 64 || D == 128, "head dim");
  return (float)(-1.4426950408889634074 / (D == 64 ? 8.0 : 11.313708498984760390));
}

__device__ __forceinline__ float sigmoid2(float score, float c1, float c2) {
  return __builtin_amdgcn_rcpf(1.0f + __builtin_amdgcn_exp2f(__builtin_fmaf(score, c1, c2)));
}

// Fast precision folds c1 into the operand a wave holds in registers for its
// whole item (rounded to the element type once per item), so the score
// product yields u = c1 * score directly, and the bias enters as the factor
// m = 2^c2 (e^-b): sigma = 1/(1 + 2^u * m), three VALU instructions per score
// (exp, fma, rcp) where sigmoid2 needs four.  For u -> +inf the fma gives inf
// and the reciprocal 0; for u -> -inf it gives 1; m is finite and positive, so
// no NaN arises.  c2 is clamped to +-126 so that m stays a normal float: that
// changes sigma only where |b| > 87, and there by less than 2^-126 e^|score|.
__device__ __forceinline__ float sigmoid_pre(float u, float m) {
  return __builtin_amdgcn_rcpf(__builtin_fmaf(__builtin_amdgcn_exp2f(u), m, 1.0f));
}

__device__ __forceinline__ float bias_factor(float c2) {
  return __builtin_amdgcn_exp2f(__builtin_fminf(__builtin_fmaxf(c2, -126.0f), 126.0f));
}

// Round 8 floats to the element type (round-to-nearest-even,
// v_cvt_pk_bf16_f32 / v_cvt_pk_f16_f32).
__device__ __forceinline__ e16x8 to_e16x8(f32x8 x) { return __builtin_convertvector(x, e16x8); }

// Widen back to float exactly.
__device__ __forceinline__ f32x8 to_f32x8(e16x8 x) { return __builtin_convertvector(x, f32x8); }

// The low part of split precision: the remainder x - hi, rounded, where hi is
// x rounded (to_e16x8(x)).  hi is widened from its packed registers (one VALU
// instruction per value); the empty asm keeps the compiler from seeing that
// hi came from x, since it would then round every value of x a second time,
// one at a time, to widen it (two instructions per value).
__device__ __forceinline__ e16x8 split_lo(const f32x8& x, e16x8 hi) {
  u32x4 w = as_u32x4(hi);
  asm("" : "+v"(w));
  return to_e16x8(x - to_f32x8(as_e16x8(w)));
}

// The eight values of C register block `blk` that form K-chunk `half` (0/1).
__device__ __forceinline__ f32x8 chunk8(const f32x16& c, int half) {
  f32x8 r;
#pragma unroll
  for (int t = 0; t < 8; ++t) r[t] = c[8 * half + t];
  return r;
}

// ---------------------------------------------------------------------------
// LDS tile layout.  A tile holds ROWS rows of D 16-bit values (keys or queries
// by d).  Row r keeps its D/8 16-byte groups in order up to an XOR of the
// group index by X(r):
//     slot(r, g) = r * D/8 + (g ^ X(r))        (16-byte slots)
//     D = 64:  X(r) = ((r >> 1) & 1) << 2 | ((r >> 2) & 3)
//     D = 128: X(r) = (r & 3) << 2 | ((r >> 2) & 3)
// The same copy serves both operand shapes the products need:
// * 16-byte fragment reads (A operand, rows = tile rows, K-slots along d):
//   the 16 lanes a 64-bank LDS serves per cycle read 16 consecutive rows at
//   one group, and X is a bijection on those rows (within each row parity for
//   D = 64), so all 64 banks are hit once;
// * transposing reads (ds_read_b64_tr_b16; A operand, rows = d, K-slots along
//   the tile rows): 32 lanes read 4 consecutive rows x 4 aligned groups, and X
//   sends the 4 rows to disjoint group sets.
// Both were measured conflict-free (SQ_LDS_BANK_CONFLICT = 0) on MI355X.
// Each row's groups stay contiguous, so a tile is filled by direct
// global -> LDS loads in which 8 consecutive lanes read one row.
// ---------------------------------------------------------------------------
template <int D>
__device__ __forceinline__ int tile_xor(int r) {
  if (D == 64) return (((r >> 1) & 1) << 2) | ((r >> 2) & 3);
  return ((r & 3) << 2) | ((r >> 2) & 3);
}

template <int D>
__device__ __forceinline__ int tile_slot(int r, int g) {
  return r * (D / 8) + (g ^ tile_xor<D>(r));
}

// Range-checked view of one (sequence, head) slice: rows 0..n-1 of D 16-bit
// values, row r at element r * rs.  Loads go through a raw buffer resource
// whose size is n * rs * 2 bytes, so a load at or beyond row n returns zeros
// without touching memory: padded rows are zero-filled by the hardware, with
// no VALU masking and no branch, and garbage (even NaN/Inf) in padded rows
// cannot reach a product.  Offsets are 32-bit: the API bounds
// (Lmax + 256) * rs * 2 below 2^31.
struct Slice {
  __amdgpu_buffer_rsrc_t rsrc;
  const uint16_t* base;
  int n, rs;
  __device__ __forceinline__ Slice(const uint16_t* base_, int n_, int row_stride)
      : rsrc(__builtin_amdgcn_make_buffer_rsrc((void*)base_, 0, n_ * row_stride * 2, 0x00020000)),
        base(base_), n(n_), rs(row_stride) {}
  // 16 bytes at element offset `elem` (a multiple of 8).
  __device__ __forceinline__ u32x4 load16(int elem) const {
    return __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rsrc, elem * 2, 0, 0));
  }
  // The same range check for rows row0.. (row0 wave-uniform): a resource whose
  // base is row row0, so per-lane offsets within a tile stay loop-invariant.
  __device__ __forceinline__ __amdgpu_buffer_rsrc_t from_row(int row0) const {
    const int rows = n > row0 ? n - row0 : 0;
    return __builtin_amdgcn_make_buffer_rsrc((void*)(base + (size_t)row0 * rs), 0, rows * rs * 2, 0x00020000);
  }
};

// Start of the (sequence, head) slice of tensor argument t of a launch.
template <class T>
__device__ __forceinline__ T* slice_base(T* p, const Sched& S, int bh, int t) {
  const int b = bh / S.H, h = bh - b * S.H;
  return p + (size_t)b * S.sb[t] + (size_t)h * S.sh[t];
}

typedef __attribute__((address_space(3))) void lds_void;

// Direct global -> LDS loading of a ROWS x D tile (buffer_load_dwordx4 ... lds).
// Each of the NW waves issues NI instructions per tile; instruction i of wave w
// fills the 1 KB block b = NW*i + w of the tile, lane L writing slot 64b + L.
// The per-lane source offset inverts the tile layout, so the 8 lanes of one
// row read that row's 128 contiguous bytes (coalesced).  Completion is
// tracked by vmcnt: wait (vm_drain) before the barrier that publishes a tile.
template <int ROWS, int D, int NW = 4>
struct TileDma {
  static constexpr int NI = ROWS * D * 2 / (NW * 1024);
  static_assert(NI >= 1 && NI * NW * 1024 == ROWS * D * 2, "tile must split into 1 KB blocks over the waves");
  int src[NI];  // byte offset within the tile's rows (row stride row_stride)
  int dst[NI];  // element offset of this wave's block within the tile (wave-uniform)
  __device__ __forceinline__ TileDma(int wave, int lane, int row_stride) {
#pragma unroll
    for (int i = 0; i < NI; ++i) {
      const int blk = NW * i + wave;
      const int t = 64 * blk + lane;  // 16-byte slot filled by this lane
      const int r = t / (D / 8);
      const int g = (t % (D / 8)) ^ tile_xor<D>(r);
      src[i] = 2 * (r * row_stride + 8 * g);
      dst[i] = 512 * blk;
    }
  }
  // Tile rows row0 .. row0+ROWS-1 of `s` into `tile` (rows >= n read as zeros).
  // The builtin is compiled in the device pass only: seen by the host pass,
  // it makes clang drop the host stubs of the kernels that use it.
  __device__ __forceinline__ void load(const Slice& s, int row0, uint16_t* tile) const {
#if defined(__HIP_DEVICE_COMPILE__)
    const __amdgpu_buffer_rsrc_t r = s.from_row(row0);
#pragma unroll
    for (int i = 0; i < NI; ++i)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_void*)(tile + dst[i]), 16, src[i], 0, 0, 0);
#endif
  }
};

// Direct global -> LDS loading of a per-row fp32 array (one value per row):
// lane L loads row row0 + L, so one 64-lane instruction fills 64 rows.  Rows
// >= n read as 0.  The LDS destination must be wave-uniform.
template <int ROWS>
struct RowDma {
  static_assert(ROWS == 64, "one 64-lane instruction per tile");
  const float* base;
  int n, off;
  __device__ __forceinline__ RowDma(const float* base_, int n_, int lane) : base(base_), n(n_), off(4 * lane) {}
  __device__ __forceinline__ void load(int row0, float* dst) const {
#if defined(__HIP_DEVICE_COMPILE__)
    const int rows = n > row0 ? n - row0 : 0;
    const __amdgpu_buffer_rsrc_t r =
        __builtin_amdgcn_make_buffer_rsrc((void*)(base + row0), 0, rows * 4, 0x00020000);
    __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_void*)dst, 4, off, 0, 0, 0);
#endif
  }
};

__device__ __forceinline__ f32x8 cat8(f32x4 a, f32x4 b) { return __builtin_shufflevector(a, b, 0, 1, 2, 3, 4, 5, 6, 7); }

// Wait until this wave's outstanding global loads (including LDS DMA) landed.
__device__ __forceinline__ void vm_drain() { __builtin_amdgcn_s_waitcnt(0); }

// B-operand fragments of one row of a slice (this lane's row), K-slots along
// d: 16s + 8hf .. +7.  Rows >= n read as zero.
template <int D>
__device__ __forceinline__ void load_bfrag(e16x8 (&f)[D / 16], const Slice& src, int row, int hf) {
#pragma unroll
  for (int s = 0; s < D / 16; ++s) f[s] = as_e16x8(src.load16(row * src.rs + 16 * s + 8 * hf));
}

// The same fragments multiplied by `scale` and rounded back to the element
// type (round-to-nearest-even): the operand of the fast-precision score
// product (see sigmoid_pre).
template <int D>
__device__ __forceinline__ void load_bfrag_scaled(e16x8 (&f)[D / 16], const Slice& src, int row, int hf,
                                                  float scale) {
  load_bfrag<D>(f, src, row, hf);
#pragma unroll
  for (int s = 0; s < D / 16; ++s) f[s] = to_e16x8(to_f32x8(f[s]) * scale);
}

typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));

// Transposing 8-byte LDS read (ds_read_b64_tr_b16): a move of 16-bit lanes,
// the same for either element type (the bf16 form of the builtin is used and
// the result reinterpreted).
__device__ __forceinline__ bf16x4 lds_tr4(const uint16_t* p) {
  typedef __attribute__((address_space(3))) bf16x4 lds_bf16x4;
  return __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4*)(p));
}

// A fragment for rows = head-dim index d, K-slots = tile rows, read with
// transposing reads.  For the MFMA of output block db (d = 32db .. 32db+31)
// and K-chunk c (tile rows 16c .. 16c+15 in the order of the score registers):
//   first read: rows 16c + 4*hf + {0..3}, second read: rows 16c + 8 + 4*hf + {0..3}.
// Source lane j (of each 16) addresses row 16c + 4hf + j/4 (+8) at columns
// 32db + 16gq + 4(j%4) .. +3; destination lane i then holds column
// 32db + 16gq + i of those four rows.
// X(r) depends on bits 0..3 of r only, so the address of row 16c + x is that
// of row x plus 16c full rows: the lane offsets are computed once (off) and
// the chunk, tile and stage enter as compile-time immediates.
template <int D>
struct TrFrag {
  int off[D / 32][2];  // element offsets of rows 4hf + j/4 (+8) for block db
  __device__ __forceinline__ TrFrag(int lane) {
    const int j = lane & 15, gq = (lane >> 4) & 1, hf = lane >> 5;
    const int row_lane = 4 * hf + (j >> 2);
    const int chunk = 4 * gq + (j & 3);  // this lane's 4-column chunk within a 32-column block
#pragma unroll
    for (int db = 0; db < D / 32; ++db)
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const int ch = 8 * db + chunk;
        off[db][h] = 8 * tile_slot<D>(row_lane + 8 * h, ch >> 1) + 4 * (ch & 1);
      }
  }
  __device__ __forceinline__ e16x8 read(const uint16_t* tile, int db, int c) const {
    const bf16x4 lo = lds_tr4(tile + 16 * c * D + off[db][0]);
    const bf16x4 hi = lds_tr4(tile + 16 * c * D + off[db][1]);
    return __builtin_bit_cast(e16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
  }
};

// A fragment (rows = tile rows 32mb .. 32mb+31, K-slots = head dim
// 16s + 8hf .. +7) with a 16-byte read.  As above, the lane offsets of rows
// l32 are computed once and the row block enters as an immediate.
template <int D>
struct FragAddr {
  int off[D / 16];
  __device__ __forceinline__ FragAddr(int l32, int hf) {
#pragma unroll
    for (int s = 0; s < D / 16; ++s) off[s] = 8 * tile_slot<D>(l32, 2 * s + hf);
  }
  __device__ __forceinline__ e16x8 read(const uint16_t* tile, int mb, int s) const {
    return as_e16x8(*(const u32x4*)(tile + 32 * mb * D + off[s]));
  }
};

// Trailing workgroups (blockIdx.x >= compute_blocks) write the padded rows
// n_b..Lmax-1 of one or two outputs (tensor arguments t1, t2) as 0 with
// 16-byte stores; the compute workgroups store valid rows only, so no row has
// two writers.
// vb: the workgroup's block index within this schedule's part of the grid.
template <int D>
__device__ __forceinline__ void zero_padded_rows(const SeqTable& T, const Sched& S, int vb,
                                                 uint16_t* __restrict__ o1, int t1, uint16_t* __restrict__ o2,
                                                 int t2, float* __restrict__ rows = nullptr) {
  const int zb = vb - S.compute_blocks;
  const int split = S.zero_split;
  const int shl = zb / split, part = zb - shl * split;
  const int sl = shl / S.H;
  if (sl >= S.zero_nseq) return;
  const int n = table_n(T, sl);
  const int bh = (T.b_base + sl) * S.H + (shl - sl * S.H);
  uint16_t* p1 = slice_base(o1, S, bh, t1);
  uint16_t* p2 = o2 ? slice_base(o2, S, bh, t2) : nullptr;
  const int rs1 = S.sl[t1], rs2 = o2 ? S.sl[t2] : 0;
  const int chunks = (S.Lmax - n) * (D / 8);
  const u32x4 z = {0u, 0u, 0u, 0u};
  for (int c = part * (int)blockDim.x + (int)threadIdx.x; c < chunks; c += split * (int)blockDim.x) {
    const int row = n + c / (D / 8), col = 8 * (c % (D / 8));
    *(u32x4*)(p1 + (size_t)row * rs1 + col) = z;
    if (o2) *(u32x4*)(p2 + (size_t)row * rs2 + col) = z;
  }
  // a per-row fp32 output, contiguous [B, H, Lmax] (the softmax lse2)
  if (rows)
    for (int row = n + part * (int)blockDim.x + (int)threadIdx.x; row < S.Lmax; row += split * (int)blockDim.x)
      rows[(size_t)bh * S.Lmax + row] = 0.0f;
}

// -b log2(e) for the item's (sequence, head): log2(n) for b = -ln n, the
// schedule's constant, or from the per-head values in device memory (a
// uniform scalar load).
__device__ __forceinline__ float item_c2(const Sched& S, const Item& it) {
  if (S.bias_kind == 0) return __builtin_amdgcn_logf((float)it.n);
  if (S.bias_kind == 1) return S.c2_const;
  return -1.4426950408889634f * S.head_bias[it.bh % S.H];
}

// The bias factor m = 2^c2 = e^-b of the prescaled sigmoid (sigmoid_pre): for
// b = -ln n exactly n.
__device__ __forceinline__ float item_bias_factor(const Sched& S, const Item& it, float c2) {
  return S.bias_kind == 0 ? (float)it.n : bias_factor(c2);
}

// The work item of block vb (list x = vb % 8, position j = vb / 8), as the
// host's decode_item computes it, or false for an idle block; uniform across
// the workgroup.  The piece comes from a binary search over the list's first
// positions.  In a piece of several short sequences (at most 64) the search
// for the sequence is spread over the wave instead of walked: one lane per
// sequence reads its length, the lanes' item counts are summed up to each
// lane, and the first lane whose sum passes the item's offset names the
// sequence: one round of independent loads where the walk chained up to
// eight, which cost 13-16 % of the time of a batch of 4096 sequences of 128.
__device__ __forceinline__ bool find_item(const SeqTable& T, const Sched& S, int vb, Item& it) {
  const int32_t x = vb & 7, j = vb >> 3;
  if (j >= S.xcd_items[x]) return false;
  const int32_t lane = (int32_t)(threadIdx.x & 63);
  int32_t lo = S.xcd_begin[x], hi = S.xcd_begin[x + 1] - 1;
  while (lo < hi) {  // last piece whose first list position is <= j
    const int32_t mid = (lo + hi + 1) >> 1;
    if (S.item0[mid] <= j) lo = mid;
    else hi = mid - 1;
  }
  const int32_t ns = S.ns[lo], nh = S.nh[lo];
  int32_t s = S.s0[lo], nt = S.nt[lo], t0 = S.t0[lo], r = j - S.item0[lo];
  if (ns > 1) {
    const int32_t q = s + (lane < ns ? lane : ns - 1);  // a sequence of the piece
    int32_t nq;
    if (T.wide) nq = (int32_t)T.n32[q];
    else nq = (int32_t)T.n16[q];
    const int32_t tiles = lane < ns ? (nq + S.outer_rows - 1) / S.outer_rows : 0;
    const int32_t cnt = nh * tiles;
    // items of sequences s .. s + lane: each bit plane of cnt as a ballot,
    // counted over the lanes up to this one (as many planes as the largest
    // count has bits)
    const uint64_t upto = lane == 63 ? ~0ull : (2ull << lane) - 1;
    int32_t incl = 0;
    for (int b = 0;; ++b) {
      const uint64_t plane = __ballot((cnt >> b) & 1);
      if (__ballot((cnt >> b) != 0) == 0) break;
      incl += __popcll(plane & upto) << b;
    }
    const uint64_t m = __ballot(lane < ns && incl > r);
    const int32_t k = __builtin_amdgcn_readfirstlane(m ? __ffsll((long long)m) - 1 : ns - 1);
    r -= __builtin_amdgcn_readfirstlane(__shfl(incl - cnt, k, 64));
    nt = __builtin_amdgcn_readfirstlane(__shfl(tiles, k, 64));
    s += k;
    t0 = 0;
  }
  const int32_t hoff = r / nt;
  it.s = s;
  it.n = ns > 1 ? table_n(T, s) : S.n1[lo];
  it.bh = (T.b_base + s) * S.H + S.h0[lo] + hoff;
  it.tile = t0 + (r - hoff * nt);
  return true;
}

}  // namespace SIGATTN_ELT
}  // namespace sigattn
