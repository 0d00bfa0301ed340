// Host-side grouping and work-list construction (see ikbo_plan.h).
#include "ikbo_plan.h"

#include <algorithm>
#include <cstdio>
#include <limits>
#include <numeric>

namespace ikbo {

namespace {

void set_err(std::string* err, const char* msg) {
  if (err) *err = msg;
}

int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }

}  // namespace

int check_offsets(const int32_t* user_offsets, int32_t n_users, std::string* err) {
  if (n_users < 0) {
    set_err(err, "n_users must be >= 0");
    return kErrInvalidArg;
  }
  if (!user_offsets) {
    set_err(err, "user_offsets is null");
    return kErrInvalidArg;
  }
  if (user_offsets[0] != 0) {
    set_err(err, "user_offsets[0] must be 0");
    return kErrBadOffsets;
  }
  for (int32_t u = 0; u < n_users; ++u) {
    if (user_offsets[u + 1] < user_offsets[u]) {
      set_err(err, "user_offsets must be non-decreasing");
      return kErrBadOffsets;
    }
  }
  return kOk;
}

int group_csr(const int32_t* cand_to_user, int32_t n_cand, int32_t n_users, int32_t n_q,
              int32_t bm, int32_t* counts, int32_t* cand_offsets, int32_t* cand_perm,
              std::vector<int32_t>* tiles, int64_t* n_tiles, std::string* err,
              std::vector<int32_t>* cursor_buf) {
  if (n_cand < 0 || n_users < 0 || n_q < 1 || bm < 1) {
    set_err(err, "group_csr: n_cand, n_users >= 0 and n_q, bm >= 1 required");
    return kErrInvalidArg;
  }
  if (n_cand > 0 && n_users == 0) {
    set_err(err, "candidates present but n_users == 0");
    return kErrBadMapping;
  }
  if (static_cast<int64_t>(n_cand) * n_q > std::numeric_limits<int32_t>::max()) {
    set_err(err, "n_cand * n_q overflows int32");
    return kErrInvalidArg;
  }
  for (int32_t u = 0; u < n_users; ++u) counts[u] = 0;
  for (int32_t c = 0; c < n_cand; ++c) {
    const int32_t u = cand_to_user[c];
    if (u < 0 || u >= n_users) {
      set_err(err, "cand_to_user entry outside [0, n_users)");
      return kErrBadMapping;
    }
    ++counts[u];
  }
  cand_offsets[0] = 0;
  for (int32_t u = 0; u < n_users; ++u) cand_offsets[u + 1] = cand_offsets[u] + counts[u];
  // Counting sort; scanning candidates in index order keeps it stable.
  std::vector<int32_t> local;
  std::vector<int32_t>& cursor = cursor_buf ? *cursor_buf : local;
  cursor.assign(cand_offsets, cand_offsets + n_users);
  for (int32_t c = 0; c < n_cand; ++c) cand_perm[cursor[cand_to_user[c]]++] = c;
  int64_t t = 0;
  if (tiles) tiles->clear();
  for (int32_t u = 0; u < n_users; ++u) {
    const int64_t rows = static_cast<int64_t>(counts[u]) * n_q;
    for (int64_t r0 = 0; r0 < rows; r0 += bm, ++t) {
      if (tiles) {
        tiles->push_back(u);
        tiles->push_back(static_cast<int32_t>(r0));
        tiles->push_back(static_cast<int32_t>(std::min<int64_t>(bm, rows - r0)));
      }
    }
  }
  if (n_tiles) *n_tiles = t;
  return kOk;
}

namespace {

// Reorders a longest-first item list into XCD bins (see HostPlan::bin_off):
// (user, head) groups by decreasing total cost, each into the least loaded bin;
// within a bin the items keep their longest-first order, or with group_span
// come in spans of that many groups of the bin, in that same group order
// (items of a span longest first), so the workgroups of one XCD share the K/V
// of a few groups at a time.  Only for plans whose grid is a multiple of the bin count and which
// give workgroups more than one item (in a single-pass plan every workgroup
// runs one item whatever its bin).
void assign_bins(const int32_t* user_offsets, int32_t n_users, int32_t H, const PlanParams& p, HostPlan* out) {
  out->n_bins = 0;
  const int32_t nb = p.xcd_bins;
  const int64_t n = static_cast<int64_t>(out->items.size());
  if (nb <= 1 || nb > kMaxBins || out->grid < nb || out->grid % nb != 0 || n <= out->grid) return;
  // group of an item: user * H + head (the user is found from its K/V base).
  std::vector<int64_t>& cost = out->group_cost;
  std::vector<int32_t>& bin = out->group_bin;
  const int64_t n_groups = static_cast<int64_t>(n_users) * H;
  cost.assign(n_groups, 0);
  auto group_of = [&](const WorkItem& it) {
    const int32_t u = static_cast<int32_t>(
        std::upper_bound(user_offsets, user_offsets + n_users + 1, it.kv_base) - user_offsets - 1);
    // users with zero keys share their K/V base with the next user; the item's
    // key range is empty then and any of them is as good
    return static_cast<int64_t>(std::min(std::max(u, 0), n_users - 1)) * H + it.h;
  };
  std::vector<int32_t>& gid = out->cursor;  // reused as per-item group ids
  gid.resize(n);
  for (int64_t i = 0; i < n; ++i) {
    const WorkItem& it = out->items[i];
    const int64_t g = group_of(it);
    gid[i] = static_cast<int32_t>(g);
    cost[g] += (it.k1 - it.k0) + p.overhead;
  }
  // groups by decreasing cost (ties by index), then each to the least loaded bin
  std::vector<uint64_t>& ord = out->keys;
  ord.clear();
  for (int64_t g = 0; g < n_groups; ++g)
    if (cost[g] > 0) ord.push_back((static_cast<uint64_t>(0xffffffffull - std::min<int64_t>(cost[g], 0xffffffffll)) << 32) |
                                   static_cast<uint64_t>(g));
  std::sort(ord.begin(), ord.end());
  int64_t load[kMaxBins] = {};
  bin.assign(n_groups, 0);
  for (uint64_t k : ord) {
    const int64_t g = static_cast<int64_t>(k & 0xffffffffull);
    int b = 0;
    for (int j = 1; j < nb; ++j)
      if (load[j] < load[b]) b = j;
    bin[g] = b;
    load[b] += cost[g];
  }
  std::vector<WorkItem>& tmp = out->unsorted;
  tmp.resize(n);
  if (p.group_span > 0) {
    // stable counting sort of the items by the span their group falls in
    // within its bin, short items (span_tail) and groups without cost
    // (possible only with overhead 0) last; the stable partition by bin below
    // keeps that order inside each bin
    const int64_t nr = static_cast<int64_t>(ord.size()) + 1;
    std::vector<int64_t>& start = out->lens;  // reused as per-span start positions
    start.assign(nr + 1, 0);
    std::vector<int64_t>& rank = out->group_cost;  // cost is no longer needed
    rank.assign(n_groups, nr - 1);
    int64_t seen[kMaxBins] = {};  // groups of each bin placed so far
    for (int64_t r = 0; r + 1 < nr; ++r) {
      const int64_t g = static_cast<int64_t>(ord[r] & 0xffffffffull);
      rank[g] = seen[bin[g]]++ / p.group_span;
    }
    auto bucket = [&](int64_t i) {
      const WorkItem& it = out->items[i];
      return it.k1 - it.k0 <= p.span_tail ? nr - 1 : rank[gid[i]];
    };
    for (int64_t i = 0; i < n; ++i) ++start[bucket(i) + 1];
    for (int64_t r = 0; r < nr; ++r) start[r + 1] += start[r];
    for (int64_t i = 0; i < n; ++i) tmp[start[bucket(i)]++] = out->items[i];
    out->items.swap(tmp);
    for (int64_t i = 0; i < n; ++i) gid[i] = static_cast<int32_t>(group_of(out->items[i]));
  }
  // stable partition of the items by bin
  int32_t cnt[kMaxBins + 1] = {};
  for (int64_t i = 0; i < n; ++i) ++cnt[bin[gid[i]] + 1];
  for (int b = 0; b < nb; ++b) cnt[b + 1] += cnt[b];
  for (int b = 0; b <= nb; ++b) out->bin_off[b] = cnt[b];
  for (int64_t i = 0; i < n; ++i) tmp[cnt[bin[gid[i]]]++] = out->items[i];
  out->items.swap(tmp);
  out->n_bins = nb;
}

}  // namespace

int build_plan(const int32_t* user_offsets, const int32_t* cand_to_user, int32_t n_users,
               int32_t n_cand, int32_t n_q, int32_t H, bool with_self, const PlanParams& p,
               HostPlan* out, std::string* err) {
  if (H < 1 || n_q < 1 || n_cand < 0 || p.bm < 1 || p.bn < 1 || p.grid_slots < 1 || p.max_chunks < 1 ||
      p.max_chunks > kMaxSplit) {
    set_err(err, "invalid sizes (H, n_q >= 1, n_cand >= 0 required)");
    return kErrInvalidArg;
  }
  if (with_self && n_q != 1) {
    set_err(err, "fused self + target attention needs n_q == 1");
    return kErrInvalidArg;
  }
  int rc = check_offsets(user_offsets, n_users, err);
  if (rc != kOk) return rc;
  out->n_bins = 0;
  out->counts.resize(n_users);
  out->cand_offsets.resize(static_cast<size_t>(n_users) + 1);
  out->cand_perm.resize(n_cand);
  rc = group_csr(cand_to_user, n_cand, n_users, n_q, p.bm, out->counts.data(), out->cand_offsets.data(),
                 out->cand_perm.data(), nullptr, &out->n_target_tiles, err, &out->cursor);
  if (rc != kOk) return rc;

  // 1. Total cost of the unsplit items: one per (user, head, row tile), target
  //    then self.  Row tiles of one (user, head) share its K/V and are built
  //    adjacently.
  int64_t total = 0, n_base = 0;
  out->n_self_tiles = 0;
  for (int32_t u = 0; u < n_users; ++u) {
    const int64_t L = user_offsets[u + 1] - user_offsets[u];
    const int64_t tiles_t = ceil_div(static_cast<int64_t>(out->counts[u]) * n_q, p.bm);
    total += H * tiles_t * (L + p.overhead);
    n_base += H * tiles_t;
    if (with_self && L > 0) {
      const int64_t tiles_s = ceil_div(L, p.bm);
      out->n_self_tiles += tiles_s;
      n_base += H * tiles_s;
      for (int64_t r0 = 0; r0 < L; r0 += p.bm) total += H * (std::min<int64_t>(r0 + p.bm, L) + p.overhead);
    }
  }
  // 2. Split long key ranges when there are too few items to fill the grid:
  //    chunk lengths are multiples of bn; the kernel merges chunk partials by
  //    log-sum-exp in chunk order, so results do not depend on the schedule.
  //    By cost: ranges longer than 1.5x the average load per workgroup are cut
  //    into chunks of about that load.  Single pass: every workgroup runs one
  //    item, so the longest item sets the time; the chunk length is the
  //    shortest multiple of bn (at least min_chunk) whose item count fits the
  //    grid, found by bisection.
  const int64_t target = std::max<int64_t>(p.min_chunk, ceil_div(total, p.grid_slots));
  auto chunks_of = [&](int64_t len, int64_t c) {  // chunks of a range of len keys for chunk length c
    const int64_t floor_len = ceil_div(ceil_div(len, p.max_chunks), p.bn) * p.bn;
    return std::max<int64_t>(1, ceil_div(len, std::max(c, floor_len)));
  };
  int64_t single_len = 0;  // 0: split by cost
  if (p.allow_split && p.single_pass && n_base < p.grid_slots) {
    // lengths of the unsplit items, in the order they are built below
    std::vector<int64_t>& lens = out->lens;
    lens.clear();
    int64_t max_len = 0;
    for (int32_t u = 0; u < n_users; ++u) {
      const int64_t L = user_offsets[u + 1] - user_offsets[u];
      const int64_t tiles_t = ceil_div(static_cast<int64_t>(out->counts[u]) * n_q, p.bm);
      for (int64_t k = 0; k < H * tiles_t; ++k) lens.push_back(L);
      if (with_self)
        for (int64_t r0 = 0; r0 < L; r0 += p.bm)
          for (int32_t h = 0; h < H; ++h) lens.push_back(std::min<int64_t>(r0 + p.bm, L));
      max_len = std::max(max_len, L);
    }
    auto count = [&](int64_t c) {
      int64_t n = 0;
      for (int64_t len : lens) n += len > 0 ? chunks_of(len, c) : 1;
      return n;
    };
    int64_t lo = std::max<int64_t>(p.bn, ceil_div(p.min_chunk, p.bn) * p.bn);
    int64_t hi = std::max<int64_t>(lo, ceil_div(max_len, p.bn) * p.bn);
    if (count(hi) <= p.grid_slots) {
      while (lo < hi) {  // smallest multiple of bn in [lo, hi] with count <= grid_slots
        const int64_t mid = (lo / p.bn + (hi / p.bn - lo / p.bn) / 2) * p.bn;
        if (count(mid) <= p.grid_slots)
          hi = mid;
        else
          lo = mid + p.bn;
      }
      single_len = hi;
    }
  }
  out->n_groups = 0;
  out->n_slots = 0;
  out->groups.clear();
  const int64_t cap = p.launch_grid > 0 ? p.launch_grid : p.grid_slots;

  // Chunks the rule below cuts a key range of len keys into.
  auto n_chunks = [&](int64_t len) -> int64_t {
    if (single_len > 0 && len > 0) {
      const int64_t nc = chunks_of(len, single_len);
      return ceil_div(len, ceil_div(ceil_div(len, nc), p.bn) * p.bn);
    }
    if (single_len == 0 && p.allow_split && len > target + target / 2) {
      const int64_t nc = std::min<int64_t>(ceil_div(len, target), p.max_chunks);
      return ceil_div(len, ceil_div(ceil_div(len, nc), p.bn) * p.bn);
    }
    return 1;
  };
  bool split_any = false;
  for (int32_t u = 0; u < n_users && !split_any; ++u)
    split_any = out->counts[u] > 0 && n_chunks(user_offsets[u + 1] - user_offsets[u]) > 1;
  if (!with_self && !split_any) {
    // Every item of a user then costs that user's key length, so longest first
    // with ties in construction order is: users by decreasing length (ties by
    // index), each user's items in construction order.  Same list as the
    // general path below, without sorting the items.
    std::vector<uint64_t>& ord = out->keys;
    ord.resize(n_users);
    for (int32_t u = 0; u < n_users; ++u)
      ord[u] = (static_cast<uint64_t>(0xffffffffu - static_cast<uint32_t>(user_offsets[u + 1] - user_offsets[u])) << 32) |
               static_cast<uint32_t>(u);
    std::sort(ord.begin(), ord.end());
    std::vector<WorkItem>& fast = out->items;
    fast.clear();
    for (int32_t k = 0; k < n_users; ++k) {
      const int32_t u = static_cast<int32_t>(ord[k] & 0xffffffffu);
      const int32_t L = user_offsets[u + 1] - user_offsets[u];
      const int64_t rows = static_cast<int64_t>(out->counts[u]) * n_q;
      for (int32_t h = 0; h < H; ++h)
        for (int64_t r0 = 0; r0 < rows; r0 += p.bm)
          fast.push_back(WorkItem{user_offsets[u], out->cand_offsets[u], static_cast<int32_t>(r0),
                                  static_cast<int32_t>(std::min<int64_t>(p.bm, rows - r0)), 0, L, h, kKindTarget, -1,
                                  0, 1, 0});
    }
    out->grid = static_cast<int32_t>(std::min<int64_t>(fast.size(), cap));
    assign_bins(user_offsets, n_users, H, p, out);
    return kOk;
  }

  std::vector<WorkItem>& items = out->unsorted;
  items.clear();
  items.reserve(static_cast<size_t>(n_base) * 2);
  auto emit = [&](WorkItem it) {
    const int64_t len = it.k1 - it.k0;
    int64_t nchunk = 1, clen = len;
    if (single_len > 0 && len > 0) {
      nchunk = chunks_of(len, single_len);
      clen = ceil_div(ceil_div(len, nchunk), p.bn) * p.bn;
      nchunk = ceil_div(len, clen);
    } else if (single_len == 0 && p.allow_split && len > target + target / 2) {
      nchunk = std::min<int64_t>(ceil_div(len, target), p.max_chunks);
      clen = ceil_div(ceil_div(len, nchunk), p.bn) * p.bn;
      nchunk = ceil_div(len, clen);
    }
    if (nchunk <= 1) {
      items.push_back(it);
      return;
    }
    const int32_t g = out->n_groups++;
    const int32_t slot0 = g * kMaxSplit;
    out->n_slots = out->n_groups * kMaxSplit;
    out->groups.push_back(MergeItem{it.row_base, it.row0, it.nrows, it.h, it.kind, slot0,
                                    static_cast<int32_t>(nchunk), 0});
    const int32_t k0 = it.k0, k1 = it.k1;
    for (int64_t c = 0; c < nchunk; ++c) {
      it.k0 = static_cast<int32_t>(k0 + c * clen);
      it.k1 = static_cast<int32_t>(std::min<int64_t>(k1, k0 + (c + 1) * clen));
      it.grp = g;
      it.chunk = static_cast<int32_t>(c);
      it.nchunk = static_cast<int32_t>(nchunk);
      it.slot0 = slot0;
      items.push_back(it);
    }
  };
  for (int32_t u = 0; u < n_users; ++u) {
    const int32_t L = user_offsets[u + 1] - user_offsets[u];
    const int64_t rows = static_cast<int64_t>(out->counts[u]) * n_q;
    for (int32_t h = 0; h < H; ++h) {
      for (int64_t r0 = 0; r0 < rows; r0 += p.bm) {
        emit(WorkItem{user_offsets[u], out->cand_offsets[u], static_cast<int32_t>(r0),
                      static_cast<int32_t>(std::min<int64_t>(p.bm, rows - r0)), 0, L, h, kKindTarget, -1, 0, 1, 0});
      }
    }
    if (with_self) {
      for (int32_t h = 0; h < H; ++h) {
        for (int64_t r0 = 0; r0 < L; r0 += p.bm) {
          const int32_t nr = static_cast<int32_t>(std::min<int64_t>(p.bm, L - r0));
          // causal: no row of the tile sees past the tile's last token
          emit(WorkItem{user_offsets[u], user_offsets[u], static_cast<int32_t>(r0), nr, 0,
                        static_cast<int32_t>(r0) + nr, h, kKindSelf, -1, 0, 1, 0});
        }
      }
    }
  }
  // 3. Longest first; equal costs keep construction order, so tiles of one
  //    (user, head) stay adjacent and land on one XCD (the kernel maps
  //    neighbouring logical workgroups to the same XCD).
  const size_t n = items.size();
  std::vector<uint64_t>& keys = out->keys;
  int64_t max_cost = 0;
  for (size_t i = 0; i < n; ++i) max_cost = std::max<int64_t>(max_cost, items[i].k1 - items[i].k0);
  if (max_cost < 65536) {
    // Stable LSD radix sort on (65535 - cost), two 8-bit digits.
    keys.resize(2 * n);
    uint64_t* a = keys.data();
    uint64_t* b = a + n;
    for (size_t i = 0; i < n; ++i)
      a[i] = (static_cast<uint64_t>(65535 - (items[i].k1 - items[i].k0)) << 32) | static_cast<uint64_t>(i);
    for (int shift = 32; shift <= 40; shift += 8) {
      uint32_t cnt[257] = {0};
      for (size_t i = 0; i < n; ++i) ++cnt[((a[i] >> shift) & 255u) + 1];
      for (int k = 0; k < 256; ++k) cnt[k + 1] += cnt[k];
      for (size_t i = 0; i < n; ++i) b[cnt[(a[i] >> shift) & 255u]++] = a[i];
      std::swap(a, b);
    }
    out->items.resize(n);
    for (size_t i = 0; i < n; ++i) out->items[i] = items[a[i] & 0xffffffffull];
  } else {
    keys.resize(n);
    for (size_t i = 0; i < n; ++i) {
      const uint64_t cost = static_cast<uint64_t>(items[i].k1 - items[i].k0);
      keys[i] = ((0xffffffffull - cost) << 32) | static_cast<uint64_t>(i);
    }
    std::sort(keys.begin(), keys.end());
    out->items.resize(n);
    for (size_t i = 0; i < n; ++i) out->items[i] = items[keys[i] & 0xffffffffull];
  }
  out->grid = static_cast<int32_t>(std::min<int64_t>(out->items.size(), cap));
  assign_bins(user_offsets, n_users, H, p, out);
  return kOk;
}

}  // namespace ikbo
