// Host-side tile schedule: which output tiles exist, how they are grouped into
// pieces, which XCD list each piece goes to, and which sequences each launch
// covers.  Pure C++; no HIP calls.
#include "plan.h"

#include <algorithm>
#include <cmath>
#include <cstring>

namespace sigattn {

namespace {

struct Piece {
  int32_t s0, ns, h0, nh, t0, nt;  // see Sched; s0 is launch-local
  int64_t item_cost;               // inner tiles of the piece's longest item
  int64_t total;                   // inner tiles over all its items
  int64_t items;                   // work items
};

int32_t ceil_div(int32_t a, int32_t b) { return (a + b - 1) / b; }

// Inner tiles visited by item t (outer tile t) of a sequence of length n.
int64_t item_inner(const PlanInput& in, int32_t n, int32_t t) {
  const int32_t inner = ceil_div(n, in.inner_rows);
  if (!in.causal) return inner;
  if (in.outer_is_key) return std::max(0, inner - causal_first_inner(t, in.outer_rows, in.inner_rows));
  return std::min(inner, causal_inner_end(t, in.outer_rows, in.inner_rows));
}

// Tiles t0 .. t0+nt-1 of nh heads of one sequence (launch-local index s).
Piece seq_piece(const PlanInput& in, int32_t s, int32_t n, int32_t h0, int32_t nh, int32_t t0, int32_t nt) {
  int64_t sum = 0, mx = 0;
  for (int32_t t = t0; t < t0 + nt; ++t) {
    const int64_t c = item_inner(in, n, t);
    sum += c;
    mx = std::max(mx, c);
  }
  return {s, 1, h0, nh, t0, nt, mx, sum * nh, (int64_t)nt * nh};
}

// Pieces of at most about `target` tile pairs over the sequences
// [b_lo, b_hi), cut evenly: runs of consecutive short sequences (all heads,
// at most kPieceSeqs sequences), whole sequences, runs of heads, or runs of
// tiles of one head.
std::vector<Piece> make_pieces(const PlanInput& in, int32_t b_lo, int32_t b_hi, int64_t target) {
  std::vector<Piece> pieces;
  Piece group{};
  bool open = false;
  auto close = [&]() {
    if (!open) return;
    if (group.ns == 1) {  // a group of one is a plain whole-sequence piece
      const int32_t n = in.seqlens[b_lo + group.s0];
      pieces.push_back(seq_piece(in, group.s0, n, 0, in.H, 0, ceil_div(n, in.outer_rows)));
    } else {
      pieces.push_back(group);
    }
    open = false;
  };
  for (int32_t b = b_lo; b < b_hi; ++b) {
    const int32_t n = in.seqlens[b];
    if (n <= 0) continue;  // no items; inside a group it is skipped by the decode
    const int32_t s = b - b_lo;
    const int32_t items = ceil_div(n, in.outer_rows);
    const Piece one = seq_piece(in, s, n, 0, 1, 0, items);
    const int64_t whole = one.total * in.H;
    if (whole <= target) {
      if (open && (group.total + whole > target || s - group.s0 + 1 > kPieceSeqs)) close();
      if (!open) {
        group = {s, 0, 0, in.H, 0, 0, 0, 0, 0};
        open = true;
      }
      group.ns = s - group.s0 + 1;
      group.total += whole;
      group.items += (int64_t)items * in.H;
      group.item_cost = std::max(group.item_cost, one.item_cost);
      continue;
    }
    close();
    if (one.total <= target) {
      const int32_t parts = (int32_t)((whole + target - 1) / target);
      const int32_t k = ceil_div(in.H, parts);
      for (int32_t h = 0; h < in.H; h += k) pieces.push_back(seq_piece(in, s, n, h, std::min(k, in.H - h), 0, items));
    } else {
      const int32_t parts = (int32_t)std::min<int64_t>(items, (one.total + target - 1) / target);
      const int32_t m = ceil_div(items, parts);
      for (int32_t h = 0; h < in.H; ++h)
        for (int32_t t = 0; t < items; t += m) pieces.push_back(seq_piece(in, s, n, h, 1, t, std::min(m, items - t)));
    }
  }
  close();
  return pieces;
}

// Pieces for the sequences [b_lo, b_hi) that fit one launch, cut as finely as
// the piece limit allows (about 1/64 of the work each, else 1/32 .. 1/8), or
// an empty optional when even the coarsest cut needs more than kMaxPieces.
bool plan_pieces(const PlanInput& in, int32_t b_lo, int32_t b_hi, std::vector<Piece>& out) {
  int64_t total = 0;
  for (int32_t b = b_lo; b < b_hi; ++b)
    if (in.seqlens[b] > 0) total += seq_piece(in, 0, in.seqlens[b], 0, in.H, 0, ceil_div(in.seqlens[b], in.outer_rows)).total;
  out.clear();
  if (total == 0) return true;
  // No piece larger than about 1/64 of the launch's work (1/8 of one XCD's
  // share): longest-first assignment then evens out the 8 XCD lists to within
  // a few percent on ragged batches.  If that needs more pieces than one
  // launch holds, cut coarser (1/32, 1/16, 1/8).
  for (int64_t parts_per_xcd = 8; parts_per_xcd >= 1; parts_per_xcd /= 2) {
    out = make_pieces(in, b_lo, b_hi, std::max<int64_t>(1, (total + parts_per_xcd * kXcds - 1) / (parts_per_xcd * kXcds)));
    if (out.size() <= (size_t)kMaxPieces) return true;
  }
  return false;
}

// One launch over the sequences [b_lo, b_hi) with the given pieces.
Launch make_launch(const PlanInput& in, int32_t b_lo, int32_t b_hi, std::vector<Piece> pieces) {
  const double log2e = 1.4426950408889634;
  Launch L;
  std::memset(&L, 0, sizeof(L));
  L.T.b_base = b_lo;
  L.T.nseq = b_hi - b_lo;
  L.T.wide = in.Lmax > 65535;
  for (int32_t s = 0; s < L.T.nseq; ++s) {
    if (L.T.wide) L.T.n32[s] = (uint32_t)in.seqlens[b_lo + s];
    else L.T.n16[s] = (uint16_t)in.seqlens[b_lo + s];
  }
  Sched& S = L.sched;
  S.H = in.H;
  S.Lmax = in.Lmax;
  S.outer_rows = in.outer_rows;
  S.out_scale = (float)(1.0 / std::sqrt((double)in.d));
  S.causal = in.causal;
  S.bias_kind = in.bias_mode == 0 ? 0 : in.bias_mode == 3 ? 2 : 1;
  S.c2_const = S.bias_kind == 1 ? (float)(-bias_value(1, in.bias_mode, in.bias_arg) * log2e) : 0.0f;

  // Longest first (ties: lower sequence, head, tile first, so plans are deterministic).
  std::stable_sort(pieces.begin(), pieces.end(), [](const Piece& a, const Piece& b) { return a.total > b.total; });
  // Longest-processing-time-first over the 8 XCD lists.
  std::vector<std::vector<Piece>> lists(kXcds);
  int64_t load[kXcds] = {0};
  for (const Piece& pc : pieces) {
    int best = 0;
    for (int x = 1; x < kXcds; ++x)
      if (load[x] < load[best]) best = x;
    lists[best].push_back(pc);
    load[best] += pc.total;
  }
  int32_t g = 0, max_items = 0;
  for (int x = 0; x < kXcds; ++x) {
    // Within a list, items with the most inner tiles start first.
    std::stable_sort(lists[x].begin(), lists[x].end(),
                     [](const Piece& a, const Piece& b) { return a.item_cost > b.item_cost; });
    S.xcd_begin[x] = g;
    int32_t item = 0;
    for (const Piece& pc : lists[x]) {
      S.s0[g] = pc.s0;
      S.ns[g] = pc.ns;
      S.h0[g] = pc.h0;
      S.nh[g] = pc.nh;
      S.t0[g] = pc.t0;
      S.nt[g] = pc.nt;
      S.item0[g] = item;
      S.n1[g] = pc.ns == 1 ? in.seqlens[b_lo + pc.s0] : 0;
      item += (int32_t)pc.items;
      ++g;
    }
    S.xcd_items[x] = item;
    max_items = std::max(max_items, item);
  }
  S.xcd_begin[kXcds] = g;
  S.compute_blocks = kXcds * max_items;
  L.blocks = S.compute_blocks;
  bool pad = false;
  for (int32_t b = b_lo; b < b_hi; ++b) pad |= in.seqlens[b] < in.Lmax;
  if (pad) {
    S.zero_nseq = L.T.nseq;
    S.zero_split = (int64_t)L.T.nseq * in.H <= 2048 ? 4 : 1;
    L.blocks += S.zero_nseq * in.H * S.zero_split;
  }
  return L;
}

// Launches for the sequences [b_lo, b_hi): one if its pieces fit, else the
// two halves in turn.
void plan_range(const PlanInput& in, int32_t b_lo, int32_t b_hi, std::vector<Launch>& out) {
  std::vector<Piece> pieces;
  if (b_hi - b_lo > 1 && !plan_pieces(in, b_lo, b_hi, pieces)) {
    const int32_t mid = b_lo + (b_hi - b_lo) / 2;
    plan_range(in, b_lo, mid, out);
    plan_range(in, mid, b_hi, out);
    return;
  }
  if (b_hi - b_lo == 1) plan_pieces(in, b_lo, b_hi, pieces);  // one sequence always fits
  bool pad = false;
  for (int32_t b = b_lo; b < b_hi; ++b) pad |= in.seqlens[b] < in.Lmax;
  if (pieces.empty() && !pad) return;  // nothing to compute or clear
  out.push_back(make_launch(in, b_lo, b_hi, std::move(pieces)));
}

}  // namespace

double bias_value(int32_t n, int32_t mode, float arg) {
  // Summary §2A: b = -log(n).  Mode 0 reads n as the sequence's valid length.
  if (mode == 0) return -std::log((double)n);
  if (mode == 1) return -std::log((double)arg);
  if (mode == 3) return 0.0;  // per-head values: the kernels read them from device memory
  return (double)arg;
}

std::vector<Launch> build_plan(const PlanInput& in, PlanStats* stats) {
  if (stats) {
    int64_t items = 0, pairs = 0;
    for (int32_t b = 0; b < in.B; ++b) {
      const int32_t n = in.seqlens[b];
      if (n <= 0) continue;
      const Piece p = seq_piece(in, 0, n, 0, in.H, 0, ceil_div(n, in.outer_rows));
      items += p.items;
      pairs += p.total;
    }
    stats->items = items;
    stats->pairs = pairs;
  }
  // Sequences per launch: what one length table holds.
  const int32_t cap = in.Lmax > 65535 ? kMaxSeqsWide : kMaxSeqs;
  std::vector<Launch> launches;
  for (int32_t b0 = 0; b0 < in.B; b0 += cap) plan_range(in, b0, std::min(in.B, b0 + cap), launches);
  return launches;
}

}  // namespace sigattn
