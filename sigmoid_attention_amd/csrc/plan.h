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

#include <cstdint>
#include <vector>

namespace sigattn {

constexpr int kXcds = 8;
// Pieces per launch and sequences zero-filled per launch: six 4-byte arrays of
// kMaxPieces, one of kZeroSeqs and a small header keep the kernel-argument
// block near 3.4 KB, under the 4 KB limit.
constexpr int kMaxPieces = 96;
constexpr int kZeroSeqs = 256;
// Workgroups that share the zero fill of one (sequence, head).
constexpr int kZeroSplit = 4;

// Kernel-argument block.  Plain data; copied by value into every launch.
struct Sched {
  int32_t H;
  int32_t Lmax;
  float out_scale;               // 1 / sqrt(d) (gradient epilogues)
  int32_t xcd_begin[kXcds + 1];  // piece range of each XCD list
  int32_t xcd_items[kXcds];      // work items in each XCD list
  // A piece is nh consecutive heads h0..h0+nh-1 of one sequence b times nt
  // consecutive outer tiles t0..t0+nt-1; its items are enumerated head-major.
  int32_t bh0[kMaxPieces];       // b * H + h0
  int32_t n[kMaxPieces];         // valid length n_b
  int32_t item0[kMaxPieces];     // first list position (within its XCD list) of the piece
  int32_t t0[kMaxPieces];        // first outer tile of the piece
  int32_t nt[kMaxPieces];        // outer tiles per head in the piece
  float c2[kMaxPieces];          // -bias * log2(e)
  // Padded rows n_b..Lmax-1 of the outputs are written as 0 by trailing
  // workgroups: block compute_blocks + (bl * H + h) * kZeroSplit + part clears
  // part `part` of those rows of sequence zero_b0 + bl, head h.
  int32_t compute_blocks;        // 8 * max(xcd_items)
  int32_t zero_b0;               // first sequence zero-filled by this launch
  int32_t zero_nseq;             // sequences zero-filled by this launch (0: none)
  int32_t zero_n[kZeroSeqs];     // their valid lengths
  int32_t causal;                // causal mask (see PlanInput)
  const float* head_bias;        // device: one bias per head (replaces c2), or null
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

// One work item: outer tile `tile` of head bh = b * H + h.
struct Item {
  int32_t bh, n, tile;
  float c2;
};

// The item of list position j in XCD list x, or false for an idle block
// (j beyond the list).  Workgroup i runs x = i % 8, j = i / 8.
inline SIGATTN_HD bool decode_item(const Sched& S, int32_t x, int32_t j, Item& it) {
  if (j >= S.xcd_items[x]) return false;
  int32_t lo = S.xcd_begin[x], hi = S.xcd_begin[x + 1] - 1;
  while (lo < hi) {  // last piece whose first list position is <= j
    const int32_t mid = (lo + hi + 1) >> 1;
    if (S.item0[mid] <= j) lo = mid;
    else hi = mid - 1;
  }
  const int32_t i = j - S.item0[lo];
  const int32_t nt = S.nt[lo];
  const int32_t hoff = i / nt;
  it.bh = S.bh0[lo] + hoff;
  it.tile = S.t0[lo] + (i - hoff * nt);
  it.n = S.n[lo];
  it.c2 = S.c2[lo];
  return true;
}

struct Launch {
  Sched sched;
  int32_t blocks;  // grid size: compute blocks + zero-fill blocks
};

// The fused backward launch: the dK/dV schedule's blocks first, then the dQ
// schedule's from block dq_off (a multiple of 8, so that each part's block
// index keeps its XCD; blocks between the two parts are idle).
struct BwdSched {
  Sched kv;
  Sched dq;
  int32_t dq_off;
};

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
