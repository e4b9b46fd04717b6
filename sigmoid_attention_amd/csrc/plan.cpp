// Host-side tile schedule: which output tiles exist, how they are grouped into
// pieces, and which XCD list each piece goes to.  Pure C++; no HIP calls.
#include "plan.h"

#include <algorithm>
#include <cmath>
#include <cstring>

namespace sigattn {

namespace {

struct Piece {
  int32_t b, h0, nh, t0, nt;
  int32_t n;
  int64_t item_cost;   // inner tiles of the piece's longest item
  int64_t total;       // inner tiles over all its items
  int64_t cost() const { return total; }
};

int32_t ceil_div(int32_t a, int32_t b) { return (a + b - 1) / b; }

// Inner tiles visited by item t (outer tile t) of a sequence of length n.
int64_t item_inner(const PlanInput& in, int32_t n, int32_t t) {
  const int32_t inner = ceil_div(n, in.inner_rows);
  if (!in.causal) return inner;
  if (in.outer_is_key) return std::max(0, inner - causal_first_inner(t, in.outer_rows, in.inner_rows));
  return std::min(inner, causal_inner_end(t, in.outer_rows, in.inner_rows));
}

Piece make_piece(const PlanInput& in, int32_t b, int32_t h0, int32_t nh, int32_t t0, int32_t nt, int32_t n) {
  int64_t sum = 0, mx = 0;
  for (int32_t t = t0; t < t0 + nt; ++t) {
    const int64_t c = item_inner(in, n, t);
    sum += c;
    mx = std::max(mx, c);
  }
  return {b, h0, nh, t0, nt, n, mx, sum * nh};
}

// Pieces of at most about `target` tile pairs, cut evenly: whole sequences
// (all heads) when small, else runs of heads, else runs of tiles of one head.
std::vector<Piece> make_pieces(const PlanInput& in, int64_t target) {
  std::vector<Piece> pieces;
  for (int32_t b = 0; b < in.B; ++b) {
    const int32_t n = in.seqlens[b];
    if (n <= 0) continue;
    const int32_t items = ceil_div(n, in.outer_rows);
    const int64_t head_cost = make_piece(in, b, 0, 1, 0, items, n).total;
    if (head_cost * in.H <= target) {
      pieces.push_back(make_piece(in, b, 0, in.H, 0, items, n));
    } else if (head_cost <= target) {
      const int32_t parts = (int32_t)((head_cost * in.H + target - 1) / target);
      const int32_t k = ceil_div(in.H, parts);
      for (int32_t h = 0; h < in.H; h += k) pieces.push_back(make_piece(in, b, h, std::min(k, in.H - h), 0, items, n));
    } else {
      const int32_t parts = (int32_t)std::min<int64_t>(items, (head_cost + target - 1) / target);
      const int32_t m = ceil_div(items, parts);
      for (int32_t h = 0; h < in.H; ++h)
        for (int32_t t = 0; t < items; t += m) pieces.push_back(make_piece(in, b, h, 1, t, std::min(m, items - t), n));
    }
  }
  return pieces;
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
  const double log2e = 1.4426950408889634;
  std::vector<Piece> pieces;
  int64_t total_cost = 0, total_items = 0;
  for (int32_t b = 0; b < in.B; ++b) {
    const int32_t n = in.seqlens[b];
    if (n <= 0) continue;
    const int32_t items = ceil_div(n, in.outer_rows);
    total_items += (int64_t)items * in.H;
    total_cost += make_piece(in, b, 0, in.H, 0, items, n).total;
  }
  if (stats) {
    stats->items = total_items;
    stats->pairs = total_cost;
  }

  // Cut work so that no piece is larger than about 1/64 of the total (1/8 of
  // one XCD's share): longest-first assignment then evens out the 8 XCD lists
  // to within a few percent on ragged batches.  If that needs more pieces than
  // one launch holds, cut coarser (1/32, 1/16, 1/8) before resorting to
  // several launches.
  for (int64_t parts_per_xcd = 8; parts_per_xcd >= 1; parts_per_xcd /= 2) {
    pieces = make_pieces(in, std::max<int64_t>(1, (total_cost + parts_per_xcd * kXcds - 1) / (parts_per_xcd * kXcds)));
    if (pieces.size() <= (size_t)kMaxPieces) break;
  }
  // Longest first (ties: lower sequence, head, tile first, so plans are deterministic).
  std::stable_sort(pieces.begin(), pieces.end(), [](const Piece& a, const Piece& b) {
    return a.cost() > b.cost();
  });

  // Zero-fill chunks: sequences [256c, 256c + 256) that have padding.
  std::vector<int32_t> zero_chunks;
  for (int32_t b0 = 0; b0 < in.B; b0 += kZeroSeqs) {
    bool any = false;
    for (int32_t b = b0; b < std::min(in.B, b0 + kZeroSeqs); ++b) any |= in.seqlens[b] < in.Lmax;
    if (any) zero_chunks.push_back(b0);
  }
  const size_t piece_chunks = (pieces.size() + kMaxPieces - 1) / kMaxPieces;
  const size_t nlaunch = std::max(piece_chunks, zero_chunks.size());

  std::vector<Launch> launches;
  for (size_t li = 0; li < nlaunch; ++li) {
    const size_t p0 = std::min(pieces.size(), li * kMaxPieces);
    const size_t p1 = std::min(pieces.size(), p0 + kMaxPieces);
    // Longest-processing-time-first over the 8 XCD lists.
    std::vector<std::vector<Piece>> lists(kXcds);
    int64_t load[kXcds] = {0};
    for (size_t p = p0; p < p1; ++p) {
      int best = 0;
      for (int x = 1; x < kXcds; ++x)
        if (load[x] < load[best]) best = x;
      lists[best].push_back(pieces[p]);
      load[best] += pieces[p].cost();
    }
    Launch L;
    std::memset(&L.sched, 0, sizeof(L.sched));
    L.sched.H = in.H;
    L.sched.Lmax = in.Lmax;
    L.sched.out_scale = (float)(1.0 / std::sqrt((double)in.d));
    L.sched.causal = in.causal;
    int32_t g = 0, max_items = 0;
    for (int x = 0; x < kXcds; ++x) {
      // Within a list, items with the most inner tiles start first.
      std::stable_sort(lists[x].begin(), lists[x].end(), [](const Piece& a, const Piece& b) {
        return a.item_cost > b.item_cost;
      });
      L.sched.xcd_begin[x] = g;
      int32_t item = 0;
      for (const Piece& pc : lists[x]) {
        L.sched.bh0[g] = pc.b * in.H + pc.h0;
        L.sched.n[g] = pc.n;
        L.sched.item0[g] = item;
        L.sched.t0[g] = pc.t0;
        L.sched.nt[g] = pc.nt;
        L.sched.c2[g] = (float)(-bias_value(pc.n, in.bias_mode, in.bias_arg) * log2e);
        item += pc.nh * pc.nt;
        ++g;
      }
      L.sched.xcd_items[x] = item;
      max_items = std::max(max_items, item);
    }
    L.sched.xcd_begin[kXcds] = g;
    L.sched.compute_blocks = kXcds * max_items;
    L.blocks = L.sched.compute_blocks;
    if (li < zero_chunks.size()) {
      const int32_t b0 = zero_chunks[li];
      L.sched.zero_b0 = b0;
      L.sched.zero_nseq = std::min(kZeroSeqs, in.B - b0);
      for (int32_t i = 0; i < L.sched.zero_nseq; ++i) L.sched.zero_n[i] = in.seqlens[b0 + i];
      L.blocks += L.sched.zero_nseq * in.H * kZeroSplit;
    }
    launches.push_back(L);
  }
  return launches;
}

}  // namespace sigattn
