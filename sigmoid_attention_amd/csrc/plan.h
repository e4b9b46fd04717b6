// Host-side tile schedule for the sigmoid attention kernels.
//
// The pages' kernel skips blocks that are entirely padding on the query side
// and on the key side ("Better Models, Faster Training", summary §2C, native
// padding support).  Here that becomes a schedule: for each (sequence, head)
// with n_b > 0 only the ceil(n_b / T_outer) output tiles exist as work items,
// and each item loops over ceil(n_b / T_inner) inner tiles.  Padded tiles
// never appear.
//
// The schedule travels to the GPU in the kernel-argument block (no device
// allocation).  Its layout is made for MI355X: 256 CUs in 8 XCDs, each with a
// private L2, and workgroup i dispatched to XCD i mod 8.  Work is cut into
// pieces (a run of consecutive tiles of one (sequence, head)), the pieces are
// assigned to XCDs by longest-processing-time-first so every XCD gets about the
// same number of tile pairs, and all pieces of one XCD sit in one list: the
// items of one (sequence, head) then run on one XCD and share its L2 copy of
// that head's K/V (or Q/dO).  Within an XCD list the pieces are in decreasing
// cost, so long items start first.
#pragma once

#include <cstddef>
#include <cstdint>
#include <vector>

namespace sigattn {

constexpr int kXcds = 8;
// Pieces per launch (seven 4-byte arrays of kMaxPieces: 2.7 KB of kernel
// arguments per schedule).
constexpr int kMaxPieces = 96;
// Sequences per launch: their lengths travel in a table of 16-bit values
// (8 KB), or of 32-bit values for Lmax > 65535 (then half as many).  One
// table serves both schedules of the fused backward, whose kernel-argument
// block (BwdSched) is then 14.5 KB; the largest block the kernels take must
// stay within kKernargBudget, the size checked to launch on MI355X with
// ROCm 7 (static_assert below the structures).
constexpr int kMaxSeqs = 4096;
constexpr int kMaxSeqsWide = 2048;
// Sequences one piece may span (bounds the decode's scan over them).
constexpr int kPieceSeqs = 64;

// Lengths of the sequences b_base .. b_base + nseq - 1 of one launch.  The
// table is 16-byte aligned so that the kernels read it in 16-byte words.
struct alignas(16) SeqTable {
  int32_t b_base;
  int32_t nseq;
  int32_t wide;  // 1: the lengths are 32-bit (Lmax > 65535)
  int32_t pad_;
  union {
    uint16_t n16[kMaxSeqs];
    uint32_t n32[kMaxSeqsWide];
  };
};

// Kernel-argument block of one pass.  Plain data; copied by value into every
// launch together with the launch's SeqTable.
struct Sched {
  int32_t H;
  int32_t Lmax;
  int32_t outer_rows;            // rows per output tile (work item)
  float out_scale;               // 1 / sqrt(d) (gradient epilogues)
  int32_t xcd_begin[kXcds + 1];  // piece range of each XCD list
  int32_t xcd_items[kXcds];      // work items in each XCD list
  // Piece p covers the launch-local sequences s0 .. s0+ns-1 (indices into the
  // SeqTable) and heads h0 .. h0+nh-1; with ns = 1, outer tiles t0 .. t0+nt-1
  // of that sequence (items head-major, tile fastest); with ns > 1, every
  // outer tile of each sequence (items sequence-major, then head, then tile).
  int32_t s0[kMaxPieces];
  int32_t ns[kMaxPieces];
  int32_t h0[kMaxPieces];
  int32_t nh[kMaxPieces];
  int32_t t0[kMaxPieces];
  int32_t nt[kMaxPieces];
  int32_t item0[kMaxPieces];     // first list position (within its XCD list) of the piece
  int32_t n1[kMaxPieces];        // length of the piece's sequence when ns = 1 (saves a table read)
  // The bias term c2 = -b log2(e) of an item: from the sequence length
  // (bias_kind 0: b = -ln n, c2 = log2 n), the constant c2_const (1), or the
  // per-head values at head_bias (2).
  int32_t bias_kind;
  float c2_const;
  // Padded rows n_b..Lmax-1 of the outputs are written as 0 by trailing
  // workgroups: block compute_blocks + (s * H + h) * zero_split + part clears
  // part `part` of those rows of table sequence s, head h.
  int32_t compute_blocks;        // 8 * max(xcd_items)
  int32_t zero_nseq;             // table sequences zero-filled by this launch (0 or the table's nseq)
  int32_t zero_split;            // workgroups per (sequence, head) of the zero fill
  int32_t causal;                // causal mask (see PlanInput)
  const float* head_bias;        // device: one bias per head (bias_kind 2), or null
  // Element strides (sequence, head, row) of each tensor argument of the
  // launch, in argument order; the head dimension is contiguous.
  int64_t sb[6];
  int64_t sh[6];
  int32_t sl[6];
};

// Callable from kernels and from host-side checks of the schedule.
#if defined(__HIPCC__)
#define SIGATTN_HD __host__ __device__
#else
#define SIGATTN_HD
#endif

inline SIGATTN_HD int32_t table_n(const SeqTable& T, int32_t s) { return T.wide ? (int32_t)T.n32[s] : (int32_t)T.n16[s]; }

// One work item: outer tile `tile` of head bh = b * H + h, b = T.b_base + s.
struct Item {
  int32_t bh, n, tile, s;
};

// The item of list position j in XCD list x, or false for an idle block
// (j beyond the list).  Workgroup i runs x = i % 8, j = i / 8.
inline SIGATTN_HD bool decode_item(const SeqTable& T, const Sched& S, int32_t x, int32_t j, Item& it) {
  if (j >= S.xcd_items[x]) return false;
  int32_t lo = S.xcd_begin[x], hi = S.xcd_begin[x + 1] - 1;
  while (lo < hi) {  // last piece whose first list position is <= j
    const int32_t mid = (lo + hi + 1) >> 1;
    if (S.item0[mid] <= j) lo = mid;
    else hi = mid - 1;
  }
  int32_t i = j - S.item0[lo];
  int32_t s = S.s0[lo], nt = S.nt[lo], t0 = S.t0[lo];
  if (S.ns[lo] > 1) {  // walk the piece's sequences (at most kPieceSeqs)
    const int32_t send = s + S.ns[lo] - 1;
    for (;; ++s) {
      nt = (table_n(T, s) + S.outer_rows - 1) / S.outer_rows;
      const int32_t cnt = S.nh[lo] * nt;
      if (i < cnt || s == send) break;
      i -= cnt;
    }
    t0 = 0;
  }
  const int32_t hoff = i / nt;
  it.s = s;
  it.n = S.ns[lo] > 1 ? table_n(T, s) : S.n1[lo];
  it.bh = (T.b_base + s) * S.H + S.h0[lo] + hoff;
  it.tile = t0 + (i - hoff * nt);
  return true;
}

struct Launch {
  SeqTable T;
  Sched sched;
  int32_t blocks;  // grid size: compute blocks + zero-fill blocks
};

// The fused backward launch: the dK/dV schedule's blocks first, then the dQ
// schedule's from block dq_off (a multiple of 8, so that each part's block
// index keeps its XCD; blocks between the two parts are idle).  Both
// schedules cover the sequences of the one table.
struct BwdSched {
  SeqTable T;
  Sched kv;
  Sched dq;
  int32_t dq_off;
};

// Kernel-argument bytes a launch may carry (blocks of 16 KB were checked on
// MI355X); the fused backward's ten pointers come before its BwdSched.
constexpr size_t kKernargBudget = 16384;
static_assert(sizeof(BwdSched) + 10 * sizeof(void*) <= kKernargBudget, "fused backward arguments exceed the budget");
static_assert(sizeof(SeqTable) + sizeof(Sched) + 10 * sizeof(void*) <= kKernargBudget,
              "single-pass arguments exceed the budget");

struct PlanInput {
  int32_t B, H, Lmax, d;
  const int32_t* seqlens;
  int32_t outer_rows;  // rows per output tile (one work item)
  int32_t inner_rows;  // rows per inner-loop tile
  int32_t bias_mode;
  float bias_arg;
  int32_t causal = 0;        // query i sees keys 0..i only
  int32_t outer_is_key = 0;  // outer tiles are key tiles (the dK/dV pass)
};

// Inner tiles visited by the item of outer tile t of a sequence of length n:
// all of them, or with a causal mask only those on the visible side of the
// diagonal (the kernels use the same bounds).
inline SIGATTN_HD int32_t causal_first_inner(int32_t t, int32_t outer_rows, int32_t inner_rows) {
  return t * outer_rows / inner_rows;  // first query tile that can see key tile t
}
inline SIGATTN_HD int32_t causal_inner_end(int32_t t, int32_t outer_rows, int32_t inner_rows) {
  return ((t + 1) * outer_rows + inner_rows - 1) / inner_rows;  // key tiles up to query tile t's last row
}

struct PlanStats {
  int64_t items = 0;
  int64_t pairs = 0;
};

// Builds the launches: the compute work (if any n_b > 0) and the zero fill of
// padded rows (if any n_b < Lmax).  Empty when there is neither.
std::vector<Launch> build_plan(const PlanInput& in, PlanStats* stats);

// The bias b for a sequence of valid length n (n >= 1) in double precision.
double bias_value(int32_t n, int32_t mode, float arg);

}  // namespace sigattn
