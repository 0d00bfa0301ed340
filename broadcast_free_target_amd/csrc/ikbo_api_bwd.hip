// C ABI of libikbo.so, target-attention backward (declared in include/ikbo.h):
// host grouping and work lists, workspaces and the dQ / merge / dK-dV launches.
// All device work is stream-ordered; the work lists are read by the kernels in
// place from pinned host memory.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <limits>
#include <map>
#include <mutex>
#include <new>
#include <string>
#include <utility>
#include <vector>

#include "ikbo.h"
#include "ikbo_api_common.h"
#include "ikbo_bwd.h"
#include "ikbo_plan.h"

using namespace ikbo_host;

namespace {

using ikbo::HostPlan;
using ikbo::PlanParams;
using ikbo::WorkItem;

// Target-attention backward: the work lists of the last calls (pinned buffers
// handed out in turn by the ring; the kernels read them in place) and the
// sorted-row workspace.
struct Bwd {
  int device = -1;
  PinnedRing ring;
  int n_cu = 0;
  DevBuf ws;              // qrow [R + pad] int32, then lse and dd [H][R + pad] fp32
  DevBuf ws_dq, ws_rec;   // split dQ partials and their row records
  DevBuf ws_rows;         // Q and dO rows in user-sorted order, per head (zeroed padding)
  HostPlan hp;            // dQ work items (the forward's planner) and the CSR grouping
  std::vector<WorkItem> items_b;
  std::vector<WorkItem> tmp;        // scratch of the XCD interleave
  std::vector<int64_t> gcost;
  std::vector<int32_t> gbin;
  int64_t n_items_a = 0, n_items_b = 0, n_groups = 0;
  int64_t n_real_a = 0, n_real_b = 0;  // items before the interleave's padding
  TimedEvents timed;      // per timed call: dQ kernel start/end, dK/dV kernel start/end
  ~Bwd() {
    timed.release();
    ring.release();
    ws.release();
    ws_dq.release();
    ws_rec.release();
    ws_rows.release();
  }
};

// Reorders a longest-first list of one-workgroup-per-item launches so that all
// items of one (user, head) run on one XCD and every XCD still gets a
// longest-first, balanced share: the dispatcher places workgroup b on XCD
// b % 8 and starts an XCD's workgroups in order of b.  (user, head) groups go to
// 8 bins, largest total cost first, each into the least loaded bin; position
// 8 j + x then holds bin x's j-th item, and the list is padded with empty items
// (no keys, no rows: a workgroup that writes nothing) to 8 times the largest
// bin.  cost(item) estimates an item's time.
template <typename Cost>
void xcd_interleave(std::vector<WorkItem>* items, const int32_t* offs, int32_t n_users, int32_t H, Cost cost,
                    std::vector<WorkItem>* tmp, std::vector<int64_t>* gcost, std::vector<int32_t>* gbin) {
  constexpr int kBins = 8;
  const size_t n = items->size();
  if (n < 2 * kBins || n_users < 1) return;
  auto group_of = [&](const WorkItem& it) {
    const int32_t u = static_cast<int32_t>(std::upper_bound(offs, offs + n_users + 1, it.kv_base) - offs - 1);
    return static_cast<int64_t>(std::min(std::max(u, 0), n_users - 1)) * H + it.h;
  };
  const int64_t n_groups = static_cast<int64_t>(n_users) * H;
  gcost->assign(n_groups, 0);
  for (const WorkItem& it : *items) (*gcost)[group_of(it)] += cost(it);
  std::vector<std::pair<int64_t, int64_t>> ord;
  ord.reserve(n_groups);
  for (int64_t g = 0; g < n_groups; ++g)
    if ((*gcost)[g] > 0) ord.emplace_back(-(*gcost)[g], g);
  std::sort(ord.begin(), ord.end());
  int64_t load[kBins] = {};
  gbin->assign(n_groups, 0);
  for (const auto& o : ord) {
    int b = 0;
    for (int j = 1; j < kBins; ++j)
      if (load[j] < load[b]) b = j;
    (*gbin)[o.second] = b;
    load[b] -= o.first;
  }
  size_t cnt[kBins] = {};
  for (const WorkItem& it : *items) ++cnt[(*gbin)[group_of(it)]];
  const size_t per = *std::max_element(cnt, cnt + kBins);
  WorkItem empty{};
  empty.grp = -1;
  empty.nchunk = 1;
  tmp->assign(per * kBins, empty);
  size_t next[kBins] = {};
  for (const WorkItem& it : *items) {  // longest first within each bin, as in the input
    const int b = (*gbin)[group_of(it)];
    (*tmp)[next[b]++ * kBins + b] = it;
  }
  items->swap(*tmp);
}

}  // namespace

extern "C" {

int ikbo_bwd_create(void** bwd) {
  try {
    if (!bwd) return fail(IKBO_ERR_INVALID_ARG, "bwd is null");
    *bwd = nullptr;
    Bwd* b = new (std::nothrow) Bwd();
    if (!b) return fail(IKBO_ERR_NOMEM, "bwd allocation");
    hipError_t e = hipGetDevice(&b->device);
    if (e == hipSuccess) e = hipDeviceGetAttribute(&b->n_cu, hipDeviceAttributeMultiprocessorCount, b->device);
    if (e != hipSuccess) {
      delete b;
      return fail_hip(e, "bwd create");
    }
    if (int rc = b->ring.init(); rc != IKBO_OK) {
      delete b;
      return rc;
    }
    *bwd = b;
    return IKBO_OK;
  } catch (...) {
    return fail(IKBO_ERR_NOMEM, "unexpected host error");
  }
}

int ikbo_attn_bwd(void* bwd, const int32_t* user_offsets, const int32_t* cand_to_user, int32_t n_users, int32_t n_cand,
                  int32_t n_q, int32_t H, int32_t d, float scale, const void* q_cand, const void* k_user,
                  const void* v_user, const void* out, const void* dout, void* dq_cand, void* dk_user, void* dv_user,
                  const float* lse, void* stream_) {
  try {
    if (!bwd) return fail(IKBO_ERR_INVALID_ARG, "bwd is null");
    Bwd* b = static_cast<Bwd*>(bwd);
    hipStream_t stream = static_cast<hipStream_t>(stream_);
    int dev = -1;
    IKBO_HIP(hipGetDevice(&dev));
    if (dev != b->device) return fail(IKBO_ERR_INVALID_ARG, "bwd belongs to another device");
    if (n_users < 0 || n_cand < 0 || n_q < 1 || H < 1) return fail(IKBO_ERR_INVALID_ARG, "n_users, n_cand >= 0 and n_q, H >= 1 required");
    if (d != ikbo::kBwdHeadDim) return fail(IKBO_ERR_UNSUPPORTED, "the backward takes head dim 128");
    if (!user_offsets || (n_cand > 0 && !cand_to_user)) return fail(IKBO_ERR_INVALID_ARG, "null mapping array");
    std::string err;
    int rc = ikbo::check_offsets(user_offsets, n_users, &err);
    if (rc != ikbo::kOk) return fail(rc, err);
    const int64_t T = n_users > 0 ? user_offsets[n_users] : 0;
    // dQ items: the forward's work list (row tiles of every user and head, long
    // key ranges split into chunks, longest first) and its CSR grouping.
    PlanParams pp;
    pp.bm = ikbo::kBwdRowsA;
    pp.bn = ikbo::kBwdKeysA;
    pp.grid_slots = std::max(1, 2 * b->n_cu);
    pp.min_chunk = 256;
    pp.allow_split = static_cast<int64_t>(n_cand) * n_q < ikbo::kBwdMaxSplitRows && !env_int("IKBO_NO_SPLIT", 0);
    rc = ikbo::build_plan(user_offsets, cand_to_user, n_users, n_cand, n_q, H, false, pp, &b->hp, &err);
    if (rc != ikbo::kOk) return fail(rc, err);
    const int64_t R = static_cast<int64_t>(n_cand) * n_q;
    if (R == 0 && T == 0) return IKBO_OK;  // nothing to write
    const size_t qb = static_cast<size_t>(R) * H * d * 2, kb = static_cast<size_t>(T) * H * d * 2;
    if (n_cand > 0 && (!q_cand || !out || !dout || !dq_cand)) return fail(IKBO_ERR_INVALID_ARG, "null query-side tensor");
    if (T > 0 && (!k_user || !v_user || !dk_user || !dv_user)) return fail(IKBO_ERR_INVALID_ARG, "null key-side tensor");
    // With no keys at all (T = 0) the dQ kernel still runs: its items have empty
    // key ranges and write zero query-gradient rows.
    const uintptr_t align_or = reinterpret_cast<uintptr_t>(q_cand) | reinterpret_cast<uintptr_t>(k_user) |
                               reinterpret_cast<uintptr_t>(v_user) | reinterpret_cast<uintptr_t>(out) |
                               reinterpret_cast<uintptr_t>(dout) | reinterpret_cast<uintptr_t>(dq_cand) |
                               reinterpret_cast<uintptr_t>(dk_user) | reinterpret_cast<uintptr_t>(dv_user);
    if (align_or & 15) return fail(IKBO_ERR_INVALID_ARG, "tensor pointers must be 16-byte aligned");
    if (reinterpret_cast<uintptr_t>(lse) & 3) return fail(IKBO_ERR_INVALID_ARG, "lse must be 4-byte aligned");
    const void* ins[6] = {q_cand, k_user, v_user, out, dout, lse};
    const size_t in_sz[6] = {qb, kb, kb, qb, qb, lse ? static_cast<size_t>(R) * H * sizeof(float) : 0};
    void* outs[3] = {dq_cand, dk_user, dv_user};
    const size_t out_sz[3] = {qb, kb, kb};
    for (int i = 0; i < 3; ++i) {
      if (out_sz[i] == 0) continue;
      for (int j = 0; j < 6; ++j)
        if (in_sz[j] && overlaps(outs[i], out_sz[i], ins[j], in_sz[j])) return fail(IKBO_ERR_INVALID_ARG, "a gradient aliases an input");
      for (int j = i + 1; j < 3; ++j)
        if (out_sz[j] && overlaps(outs[i], out_sz[i], outs[j], out_sz[j])) return fail(IKBO_ERR_INVALID_ARG, "gradients overlap");
    }
    // dK/dV items: every kBwdKeysB keys of every user and head, most rows first.
    b->items_b.clear();
    for (int32_t u = 0; u < n_users; ++u) {
      const int32_t L = user_offsets[u + 1] - user_offsets[u];
      for (int32_t h = 0; h < H; ++h)
        for (int32_t k0 = 0; k0 < L; k0 += ikbo::kBwdKeysB) {
          WorkItem w{};
          w.kv_base = user_offsets[u];
          w.row_base = b->hp.cand_offsets[u];
          w.row0 = 0;
          w.nrows = b->hp.counts[u] * n_q;
          w.k0 = k0;
          w.k1 = std::min(L, k0 + ikbo::kBwdKeysB);
          w.h = h;
          w.grp = -1;
          b->items_b.push_back(w);
        }
    }
    std::stable_sort(b->items_b.begin(), b->items_b.end(),
                     [](const WorkItem& x, const WorkItem& y) { return x.nrows > y.nrows; });
    // Items of one (user, head) share its K/V (dQ: row tiles) or its sorted
    // Q/dO rows (dK/dV: key blocks): keep them on one XCD's L2.
    b->n_real_a = static_cast<int64_t>(b->hp.items.size());
    b->n_real_b = static_cast<int64_t>(b->items_b.size());
    if (env_int("IKBO_XCD_BINS", 8) > 1) {
      xcd_interleave(&b->hp.items, user_offsets, n_users, H,
                     [](const WorkItem& it) { return static_cast<int64_t>(it.k1 - it.k0) + 128; }, &b->tmp, &b->gcost,
                     &b->gbin);
      xcd_interleave(&b->items_b, user_offsets, n_users, H,
                     [](const WorkItem& it) { return static_cast<int64_t>(it.nrows + 64) * (it.k1 - it.k0); }, &b->tmp,
                     &b->gcost, &b->gbin);
    }
    const int64_t na = static_cast<int64_t>(b->hp.items.size()), nb = static_cast<int64_t>(b->items_b.size());
    if (na > std::numeric_limits<int32_t>::max() || nb > std::numeric_limits<int32_t>::max() ||
        R + ikbo::kBwdPad > std::numeric_limits<int32_t>::max())
      return fail(IKBO_ERR_INVALID_ARG, "problem too large");
    b->n_items_a = na;
    b->n_items_b = nb;
    b->n_groups = b->hp.n_groups;
    // workspace
    const size_t rp = static_cast<size_t>(R + ikbo::kBwdPad);
    if ((rc = b->ws.ensure(rp * 4 * (1 + 2 * static_cast<size_t>(H)), false)) != IKBO_OK) return rc;
    // Sorted Q and dO copies, zero-filled when allocated: the padding rows the
    // dK/dV kernel may read hold zeros or rows of an earlier call, finite either way.
    const size_t rows_bytes = static_cast<size_t>(H) * rp * ikbo::kBwdHeadDim * 2;
    if ((rc = b->ws_rows.ensure(2 * rows_bytes, true)) != IKBO_OK) return rc;
    const size_t slot_rows = static_cast<size_t>(b->hp.n_slots) * ikbo::kBwdRowsA;
    if (slot_rows > 0 && ((rc = b->ws_dq.ensure(slot_rows * ikbo::kBwdHeadDim * 4, false)) != IKBO_OK ||
                          (rc = b->ws_rec.ensure(slot_rows * 16, false)) != IKBO_OK))
      return rc;
    // work lists into the next pinned buffer, once its last reader is done
    const size_t items_bytes = static_cast<size_t>(na + nb) * sizeof(WorkItem);
    const size_t bytes = items_bytes + static_cast<size_t>(std::max(n_cand, 1)) * 4;
    int si = 0;
    if ((rc = b->ring.acquire(bytes, &si)) != IKBO_OK) return rc;
    char* base = static_cast<char*>(b->ring.buf[si].ptr);
    std::memcpy(base, b->hp.items.data(), static_cast<size_t>(na) * sizeof(WorkItem));
    std::memcpy(base + na * sizeof(WorkItem), b->items_b.data(), static_cast<size_t>(nb) * sizeof(WorkItem));
    if (n_cand > 0) std::memcpy(base + items_bytes, b->hp.cand_perm.data(), static_cast<size_t>(n_cand) * 4);
    hipEvent_t* te = nullptr;
    if ((rc = b->timed.next(&te, true)) != IKBO_OK) return rc;
    ikbo::BwdParams p{};
    p.q = q_cand;
    p.k = k_user;
    p.v = v_user;
    p.o = out;
    p.dout = dout;
    p.dq = dq_cand;
    p.dk = dk_user;
    p.dv = dv_user;
    p.cand_perm = reinterpret_cast<const int32_t*>(base + items_bytes);
    p.lse_in = lse;
    p.qrow = static_cast<int32_t*>(b->ws.ptr);
    p.lse = reinterpret_cast<float*>(p.qrow + rp);
    p.dd = p.lse + rp * H;
    p.qs = static_cast<uint16_t*>(b->ws_rows.ptr);
    p.dos = p.qs + rows_bytes / 2;
    p.ws_dq = static_cast<float*>(b->ws_dq.ptr);
    p.ws_rec = static_cast<float*>(b->ws_rec.ptr);
    p.rows_total = static_cast<int32_t>(R);
    p.H = H;
    p.n_q = n_q;
    p.scale = scale;
    p.scale_log2 = scale * 1.4426950408889634f;
    p.items = reinterpret_cast<const WorkItem*>(base);
    // timing: the dQ span runs from the dQ kernel's start to the merge's end
    hipEvent_t ev_dq[2] = {te ? te[0] : nullptr, te && b->n_groups == 0 ? te[1] : nullptr};
    if ((rc = b->ring.on_stream(stream)) != IKBO_OK) return rc;  // before anything is enqueued
    hipError_t e = ikbo::launch_bwd_dq(p, static_cast<int>(na), stream, te ? ev_dq : nullptr);
    if (e != hipSuccess) return fail_hip(e, "dQ launch");
    e = ikbo::launch_bwd_merge(p, static_cast<int>(b->n_groups), stream, te ? te[1] : nullptr);
    if (e != hipSuccess) return fail_hip(e, "dQ merge launch");
    p.items = reinterpret_cast<const WorkItem*>(base) + na;
    e = ikbo::launch_bwd_dkv(p, static_cast<int>(nb), stream, te ? te + 2 : nullptr);
    if (e != hipSuccess) return fail_hip(e, "dK/dV launch");
    return b->ring.launched(si, stream);
  } catch (...) {
    return fail(IKBO_ERR_NOMEM, "unexpected host error");
  }
}

int ikbo_bwd_info(void* bwd, int64_t* info, int32_t n_info) {
  if (!bwd || !info || n_info < 0) return fail(IKBO_ERR_INVALID_ARG, "null argument");
  Bwd* b = static_cast<Bwd*>(bwd);
  const int64_t v[3] = {b->n_real_a, b->n_real_b, b->n_groups};
  for (int i = 0; i < std::min<int32_t>(n_info, 3); ++i) info[i] = v[i];
  return IKBO_OK;
}

int ikbo_bwd_timing(void* bwd, int32_t enable) {
  if (!bwd) return fail(IKBO_ERR_INVALID_ARG, "bwd is null");
  return static_cast<Bwd*>(bwd)->timed.enable(enable != 0);
}

int ikbo_bwd_timing_read(void* bwd, float* dq_ms, float* dkv_ms, int32_t max_n, int32_t* n) {
  if (!bwd || !n || max_n < 0 || (max_n > 0 && (!dq_ms || !dkv_ms))) return fail(IKBO_ERR_INVALID_ARG, "null argument");
  Bwd* b = static_cast<Bwd*>(bwd);
  const std::vector<hipEvent_t>& ev = b->timed.ev;
  const int m = std::min<int>(b->timed.n, max_n);
  for (int i = 0; i < m; ++i) {
    IKBO_HIP(hipEventSynchronize(ev[4 * i + 1]));
    IKBO_HIP(hipEventElapsedTime(&dq_ms[i], ev[4 * i], ev[4 * i + 1]));
    IKBO_HIP(hipEventSynchronize(ev[4 * i + 3]));
    IKBO_HIP(hipEventElapsedTime(&dkv_ms[i], ev[4 * i + 2], ev[4 * i + 3]));
  }
  *n = m;
  return IKBO_OK;
}

void ikbo_bwd_destroy(void* bwd) {
  if (!bwd) return;
  Bwd* b = static_cast<Bwd*>(bwd);
  int cur = -1;
  if (hipGetDevice(&cur) == hipSuccess) {
    (void)hipSetDevice(b->device);
    (void)hipDeviceSynchronize();
    (void)hipSetDevice(cur);
  }
  delete b;
}

}  // extern "C"

