// Host-only check of the tile schedule: builds the plan for the lengths given
// on the command line and walks every workgroup of every launch through the
// same decode_item() the kernels use.  Verifies that each non-padded output
// tile is visited exactly once and that no fully padded tile appears; prints
// a one-line JSON summary.  Also checks that every sequence with padding is
// zero-filled by exactly one launch, that each launch's length table holds
// its sequences, and that no piece spans more sequences than allowed.
//
// usage: plan_harness B H Lmax d outer_rows inner_rows n_0 ... n_{B-1}
#include <cstdio>
#include <cstdlib>
#include <map>
#include <utility>
#include <vector>

#include "plan.h"

int main(int argc, char** argv) {
  if (argc < 7) return 2;
  sigattn::PlanInput in;
  in.B = atoi(argv[1]);
  in.H = atoi(argv[2]);
  in.Lmax = atoi(argv[3]);
  in.d = atoi(argv[4]);
  in.outer_rows = atoi(argv[5]);
  in.inner_rows = atoi(argv[6]);
  in.bias_mode = 0;
  in.bias_arg = 0.0f;
  if (argc != 7 + in.B) return 2;
  std::vector<int32_t> lens(in.B);
  for (int b = 0; b < in.B; ++b) lens[b] = atoi(argv[7 + b]);
  in.seqlens = lens.data();

  sigattn::PlanStats st;
  const std::vector<sigattn::Launch> plan = sigattn::build_plan(in, &st);
  std::map<std::pair<int, int>, int> seen;
  std::vector<int> zeroed(in.B, 0);
  long long blocks = 0, idle = 0, bad = 0, pairs = 0;
  double worst_imbalance = 0.0;
  int max_piece_seqs = 0;
  for (const auto& L : plan) {
    if (L.sched.compute_blocks % sigattn::kXcds) ++bad;
    if (L.blocks != L.sched.compute_blocks + L.sched.zero_nseq * in.H * L.sched.zero_split) ++bad;
    // the length table holds this launch's sequences exactly
    const int cap = L.T.wide ? sigattn::kMaxSeqsWide : sigattn::kMaxSeqs;
    if (L.T.nseq < 1 || L.T.nseq > cap || L.T.b_base < 0 || L.T.b_base + L.T.nseq > in.B) ++bad;
    else
      for (int32_t s = 0; s < L.T.nseq; ++s)
        if (sigattn::table_n(L.T, s) != lens[L.T.b_base + s]) ++bad;
    if (L.sched.zero_nseq != 0 && L.sched.zero_nseq != L.T.nseq) ++bad;
    for (int32_t i = 0; i < L.sched.zero_nseq; ++i) zeroed[L.T.b_base + i]++;
    for (int32_t p = 0; p < L.sched.xcd_begin[sigattn::kXcds]; ++p) {
      if (L.sched.ns[p] < 1 || L.sched.ns[p] > sigattn::kPieceSeqs || L.sched.s0[p] < 0 ||
          L.sched.s0[p] + L.sched.ns[p] > L.T.nseq)
        ++bad;
      max_piece_seqs = L.sched.ns[p] > max_piece_seqs ? L.sched.ns[p] : max_piece_seqs;
    }
    long long xload[sigattn::kXcds] = {0};
    for (int32_t i = 0; i < L.sched.compute_blocks; ++i) {
      sigattn::Item it;
      ++blocks;
      if (!sigattn::decode_item(L.T, L.sched, i % sigattn::kXcds, i / sigattn::kXcds, it)) {
        ++idle;
        continue;
      }
      const int b = it.bh / in.H;
      const int ntiles = (lens[b] + in.outer_rows - 1) / in.outer_rows;
      if (b < 0 || b >= in.B || b != L.T.b_base + it.s || it.n != lens[b] || it.tile < 0 || it.tile >= ntiles) ++bad;
      seen[{it.bh, it.tile}]++;
      const long long inner = (lens[b] + in.inner_rows - 1) / in.inner_rows;
      pairs += inner;
      xload[i % sigattn::kXcds] += inner;
    }
    long long mx = 0, sum = 0;
    for (int x = 0; x < sigattn::kXcds; ++x) {
      mx = xload[x] > mx ? xload[x] : mx;
      sum += xload[x];
    }
    if (sum > 0) {
      const double imb = (double)mx * sigattn::kXcds / (double)sum - 1.0;
      worst_imbalance = imb > worst_imbalance ? imb : worst_imbalance;
    }
  }
  long long expect = 0, dup = 0, missing = 0;
  for (int b = 0; b < in.B; ++b) {
    const int ntiles = (lens[b] + in.outer_rows - 1) / in.outer_rows;
    for (int h = 0; h < in.H; ++h)
      for (int t = 0; t < ntiles; ++t) {
        ++expect;
        auto itr = seen.find({b * in.H + h, t});
        if (itr == seen.end()) ++missing;
        else if (itr->second != 1) ++dup;
      }
  }
  const long long extra = (long long)seen.size() - (expect - missing);
  long long zero_bad = 0;
  for (int b = 0; b < in.B; ++b)
    if (lens[b] < in.Lmax ? zeroed[b] != 1 : zeroed[b] > 1) ++zero_bad;
  printf("{\"launches\": %zu, \"blocks\": %lld, \"idle\": %lld, \"items\": %lld, \"expect\": %lld, "
         "\"missing\": %lld, \"dup\": %lld, \"extra\": %lld, \"bad\": %lld, \"pairs\": %lld, "
         "\"stats_items\": %lld, \"stats_pairs\": %lld, \"xcd_imbalance\": %.4f, \"zero_bad\": %lld, "
         "\"max_piece_seqs\": %d}\n",
         plan.size(), blocks, idle, blocks - idle, expect, missing, dup, extra, bad, pairs, (long long)st.items,
         (long long)st.pairs, worst_imbalance, zero_bad, max_piece_seqs);
  return 0;
}
