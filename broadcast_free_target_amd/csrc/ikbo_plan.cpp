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
              std::vector<int32_t>* tiles, int64_t* n_tiles, std::string* err) {
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
  std::vector<int32_t> cursor(cand_offsets, cand_offsets + n_users);
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

int build_plan(const int32_t* user_offsets, const int32_t* cand_to_user, int32_t n_users,
               int32_t n_cand, int32_t n_q, int32_t H, bool with_self, const PlanParams& p,
               HostPlan* out, std::string* err) {
  if (H < 1 || n_q < 1 || n_cand < 0 || p.bm < 1 || p.bn < 1 || p.grid_slots < 1) {
    set_err(err, "invalid sizes (H, n_q >= 1, n_cand >= 0 required)");
    return kErrInvalidArg;
  }
  if (with_self && n_q != 1) {
    set_err(err, "fused self + target attention needs n_q == 1");
    return kErrInvalidArg;
  }
  int rc = check_offsets(user_offsets, n_users, err);
  if (rc != kOk) return rc;
  out->counts.assign(n_users, 0);
  out->cand_offsets.assign(static_cast<size_t>(n_users) + 1, 0);
  out->cand_perm.assign(n_cand, 0);
  rc = group_csr(cand_to_user, n_cand, n_users, n_q, p.bm, out->counts.data(),
                 out->cand_offsets.data(), out->cand_perm.data(), nullptr, &out->n_target_tiles,
                 err);
  if (rc != kOk) return rc;

  // 1. Unsplit items: one per (user, head, row tile), target then self.  Row
  //    tiles of one (user, head) share its K/V, so they are built adjacently.
  struct Proto {
    WorkItem it;
    int64_t order;  // construction order, the deterministic tie-break
  };
  std::vector<Proto> base;
  int64_t order = 0;
  out->n_self_tiles = 0;
  for (int32_t u = 0; u < n_users; ++u) {
    const int32_t L = user_offsets[u + 1] - user_offsets[u];
    const int64_t rows = static_cast<int64_t>(out->counts[u]) * n_q;
    for (int32_t h = 0; h < H; ++h) {
      for (int64_t r0 = 0; r0 < rows; r0 += p.bm) {
        WorkItem it{};
        it.kv_base = user_offsets[u];
        it.row_base = out->cand_offsets[u];
        it.row0 = static_cast<int32_t>(r0);
        it.nrows = static_cast<int32_t>(std::min<int64_t>(p.bm, rows - r0));
        it.k0 = 0;
        it.k1 = L;
        it.h = h;
        it.kind = kKindTarget;
        it.grp = -1;
        it.chunk = 0;
        it.nchunk = 1;
        it.slot0 = 0;
        base.push_back({it, order++});
      }
    }
    if (with_self) {
      out->n_self_tiles += ceil_div(L, p.bm);
      for (int32_t h = 0; h < H; ++h) {
        for (int64_t r0 = 0; r0 < L; r0 += p.bm) {
          WorkItem it{};
          it.kv_base = user_offsets[u];
          it.row_base = user_offsets[u];
          it.row0 = static_cast<int32_t>(r0);
          it.nrows = static_cast<int32_t>(std::min<int64_t>(p.bm, L - r0));
          it.k0 = 0;
          it.k1 = it.row0 + it.nrows;  // causal: no row sees past its own token
          it.h = h;
          it.kind = kKindSelf;
          it.grp = -1;
          it.chunk = 0;
          it.nchunk = 1;
          it.slot0 = 0;
          base.push_back({it, order++});
        }
      }
    }
  }

  // 2. Split long key ranges when there are too few items to fill the grid.
  //    Chunk lengths are multiples of bn; the kernel merges chunk partials by
  //    log-sum-exp in chunk order, so results do not depend on the schedule.
  int64_t total = 0;
  for (const auto& b : base) total += (b.it.k1 - b.it.k0) + p.overhead;
  const int64_t target = std::max<int64_t>(p.min_chunk, ceil_div(total, p.grid_slots));
  std::vector<Proto> items;
  items.reserve(base.size());
  out->n_groups = 0;
  out->n_slots = 0;
  out->groups.clear();
  for (const auto& b : base) {
    const int64_t len = b.it.k1 - b.it.k0;
    int64_t nchunk = 1;
    if (p.allow_split && len > target + target / 2) nchunk = ceil_div(len, target);
    if (nchunk > 1) {
      const int64_t clen = ceil_div(ceil_div(len, nchunk), p.bn) * p.bn;
      nchunk = ceil_div(len, clen);
      if (nchunk > 1) {
        const int32_t g = out->n_groups++;
        const int32_t slot0 = out->n_slots;
        out->n_slots += static_cast<int32_t>(nchunk);
        out->groups.push_back(MergeItem{b.it.row_base, b.it.row0, b.it.nrows, b.it.h, b.it.kind, slot0,
                                        static_cast<int32_t>(nchunk), 0});
        for (int64_t c = 0; c < nchunk; ++c) {
          Proto q = b;
          q.it.k0 = static_cast<int32_t>(b.it.k0 + c * clen);
          q.it.k1 = static_cast<int32_t>(std::min<int64_t>(b.it.k1, b.it.k0 + (c + 1) * clen));
          q.it.grp = g;
          q.it.chunk = static_cast<int32_t>(c);
          q.it.nchunk = static_cast<int32_t>(nchunk);
          q.it.slot0 = slot0;
          q.order = b.order * 65536 + c;
          items.push_back(q);
        }
        continue;
      }
    }
    Proto q = b;
    q.order = b.order * 65536;
    items.push_back(q);
  }

  // 3. Longest first; equal costs keep construction order, so tiles of one
  //    (user, head) stay adjacent and land on one XCD (the kernel maps
  //    neighbouring logical workgroups to the same XCD).
  std::stable_sort(items.begin(), items.end(), [](const Proto& a, const Proto& b) {
    const int64_t ca = a.it.k1 - a.it.k0, cb = b.it.k1 - b.it.k0;
    if (ca != cb) return ca > cb;
    return a.order < b.order;
  });
  out->items.resize(items.size());
  for (size_t i = 0; i < items.size(); ++i) out->items[i] = items[i].it;
  const int64_t cap = p.launch_grid > 0 ? p.launch_grid : p.grid_slots;
  out->grid = static_cast<int32_t>(std::min<int64_t>(items.size(), cap));
  return kOk;
}

}  // namespace ikbo
