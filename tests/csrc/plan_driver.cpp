// Test driver for the host planner (built with g++ and sanitizers by the
// CPU test suite).  Reads one problem from stdin as whitespace-separated
// integers:
//   n_users n_cand n_q H with_self bm bn grid_slots min_chunk allow_split single_pass xcd_bins group_span span_tail
//   user_offsets[n_users+1] cand_to_user[n_cand]
// and prints "rc <status>", then "plan <n_items> <grid> <n_groups> <n_slots>",
// "bins <n_bins> <bin_off[0..kMaxBins]>", "perm <cand_perm...>", and one "item"
// line per work item (all 12 fields).
#include <cstdio>
#include <iostream>
#include <string>
#include <vector>

#include "ikbo_plan.h"

int main() {
  int32_t n_users, n_cand, n_q, H, with_self, bm, bn, grid_slots, min_chunk, allow_split, single_pass, xcd_bins,
      group_span, span_tail;
  if (!(std::cin >> n_users >> n_cand >> n_q >> H >> with_self >> bm >> bn >> grid_slots >> min_chunk >>
        allow_split >> single_pass >> xcd_bins >> group_span >> span_tail))
    return 2;
  std::vector<int32_t> offs(static_cast<size_t>(n_users) + 1), c2u(n_cand);
  for (auto& x : offs) std::cin >> x;
  for (auto& x : c2u) std::cin >> x;
  ikbo::PlanParams p;
  p.bm = bm;
  p.bn = bn;
  p.grid_slots = grid_slots;
  p.min_chunk = min_chunk;
  p.allow_split = allow_split != 0;
  p.single_pass = single_pass != 0;
  p.xcd_bins = xcd_bins;
  p.group_span = group_span;
  p.span_tail = span_tail;
  ikbo::HostPlan hp;
  std::string err;
  const int rc = ikbo::build_plan(offs.data(), c2u.data(), n_users, n_cand, n_q, H, with_self != 0, p, &hp, &err);
  std::printf("rc %d\n", rc);
  if (rc != 0) return 0;
  std::printf("plan %zu %d %d %d\n", hp.items.size(), hp.grid, hp.n_groups, hp.n_slots);
  std::printf("bins %d", hp.n_bins);
  for (int b = 0; b <= ikbo::kMaxBins; ++b) std::printf(" %d", hp.bin_off[b]);
  std::printf("\n");
  std::printf("perm");
  for (int32_t x : hp.cand_perm) std::printf(" %d", x);
  std::printf("\n");
  for (const auto& it : hp.items)
    std::printf("item %d %d %d %d %d %d %d %d %d %d %d %d\n", it.kv_base, it.row_base, it.row0, it.nrows, it.k0,
                it.k1, it.h, it.kind, it.grp, it.chunk, it.nchunk, it.slot0);
  return 0;
}
