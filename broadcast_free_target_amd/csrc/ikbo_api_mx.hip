// C ABI of libikbo.so, MXFP8 target attention (declared in include/ikbo.h):
// per-call grouping and work lists from host mapping arrays, the per-item
// V-scale block range, workspaces, and the MXFP8 kernel and split-merge
// launches.  All device work is stream-ordered; the work lists are read by the
// kernel in place from pinned host memory.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstdint>
#include <cstring>
#include <limits>
#include <new>
#include <string>
#include <vector>

#include "ikbo.h"
#include "ikbo_api_common.h"
#include "ikbo_kernels.h"
#include "ikbo_mx.h"
#include "ikbo_plan.h"

using namespace ikbo_host;

namespace {

using ikbo::HostPlan;
using ikbo::PlanParams;
using ikbo::WorkItem;

// MXFP8 attention: the work lists of the last calls (pinned buffers handed
// out in turn by the ring) and the split partials.
struct Mx {
  int device = -1;
  int n_cu = 0;
  PinnedRing ring;
  DevBuf ws_o, ws_rec;
  HostPlan hp;
  std::vector<int32_t> vblk;  // per item: first and last V-scale block
  TimedEvents timed;  // per timed call: kernel start/end, merge start/end; flag: merged
  ~Mx() {
    timed.release();
    ring.release();
    ws_o.release();
    ws_rec.release();
  }
};

}  // namespace

extern "C" {

int ikbo_mx_create(void** mx) {
  try {
    if (!mx) return fail(IKBO_ERR_INVALID_ARG, "mx is null");
    *mx = nullptr;
    Mx* m = new (std::nothrow) Mx();
    if (!m) return fail(IKBO_ERR_NOMEM, "mx allocation");
    hipError_t e = hipGetDevice(&m->device);
    if (e == hipSuccess) e = hipDeviceGetAttribute(&m->n_cu, hipDeviceAttributeMultiprocessorCount, m->device);
    if (e != hipSuccess) {
      delete m;
      return fail_hip(e, "mx create");
    }
    if (int rc = m->ring.init(); rc != IKBO_OK) {
      delete m;
      return rc;
    }
    *mx = m;
    return IKBO_OK;
  } catch (...) {
    return fail(IKBO_ERR_NOMEM, "unexpected host error");
  }
}

int ikbo_attn_fwd_mxfp8(void* mx, const int32_t* user_offsets, const int32_t* cand_to_user, int32_t n_users,
                        int32_t n_cand, int32_t n_q, int32_t H, int32_t d, float scale, const void* q_codes,
                        const void* q_scales, const void* k_codes, const void* k_scales, const void* v_codes,
                        const void* v_scales, void* out, void* stream_) {
  try {
    if (!mx) return fail(IKBO_ERR_INVALID_ARG, "mx is null");
    Mx* m = static_cast<Mx*>(mx);
    hipStream_t stream = static_cast<hipStream_t>(stream_);
    int dev = -1;
    IKBO_HIP(hipGetDevice(&dev));
    if (dev != m->device) return fail(IKBO_ERR_INVALID_ARG, "mx belongs to another device");
    if (n_users < 0 || n_cand < 0 || n_q < 1 || H < 1) return fail(IKBO_ERR_INVALID_ARG, "n_users, n_cand >= 0 and n_q, H >= 1 required");
    if (d != ikbo::kMxHeadDim) return fail(IKBO_ERR_UNSUPPORTED, "MXFP8 attention takes head dim 128");
    if (!std::isfinite(scale)) return fail(IKBO_ERR_INVALID_ARG, "scale must be finite");
    if (!user_offsets || (n_cand > 0 && !cand_to_user)) return fail(IKBO_ERR_INVALID_ARG, "null mapping array");
    std::string err;
    int rc = ikbo::check_offsets(user_offsets, n_users, &err);
    if (rc != ikbo::kOk) return fail(rc, err);
    // Small requests: one workgroup per CU, each with a longer key range (fewer
    // split partials to merge), when every item then fits one pass; otherwise
    // two resident workgroups per CU.  IKBO_SPLIT_SLOTS fixes the slot count.
    PlanParams pp;
    pp.bm = ikbo::kMxRows;
    pp.bn = ikbo::kMxKeys;
    const int forced_slots = env_int("IKBO_SPLIT_SLOTS", 0);
    pp.grid_slots = forced_slots > 0 ? forced_slots : std::max(1, m->n_cu);
    pp.min_chunk = std::max(pp.bn, env_int("IKBO_MIN_CHUNK", 256) / pp.bn * pp.bn);
    pp.launch_grid = std::max(0, env_int("IKBO_GRID_WGS", 0));
    pp.allow_split = !env_int("IKBO_NO_SPLIT", 0);
    rc = ikbo::build_plan(user_offsets, cand_to_user, n_users, n_cand, n_q, H, false, pp, &m->hp, &err);
    if (rc != ikbo::kOk) return fail(rc, err);
    if (forced_slots <= 0 && m->hp.items.size() > static_cast<size_t>(pp.grid_slots)) {
      pp.grid_slots = std::max(1, 2 * m->n_cu);
      rc = ikbo::build_plan(user_offsets, cand_to_user, n_users, n_cand, n_q, H, false, pp, &m->hp, &err);
      if (rc != ikbo::kOk) return fail(rc, err);
    }
    if (n_cand == 0) return IKBO_OK;
    const int64_t T = user_offsets[n_users];
    const int64_t R = static_cast<int64_t>(n_cand) * n_q;
    const size_t qb = static_cast<size_t>(R) * H * d, kb = static_cast<size_t>(T) * H * d;
    const size_t qsb = qb / ikbo::kMxBlock, ksb = kb / ikbo::kMxBlock;
    int64_t nvb = 0;
    for (int32_t u = 0; u < n_users; ++u)
      nvb += (user_offsets[u + 1] - user_offsets[u] + ikbo::kMxBlock - 1) / ikbo::kMxBlock;
    const size_t vsb = static_cast<size_t>(nvb) * H * d;
    if (!q_codes || !q_scales || !out) return fail(IKBO_ERR_INVALID_ARG, "null query-side tensor");
    if (T > 0 && (!k_codes || !k_scales || !v_codes || !v_scales)) return fail(IKBO_ERR_INVALID_ARG, "null key-side tensor");
    const uintptr_t a16 = reinterpret_cast<uintptr_t>(q_codes) | reinterpret_cast<uintptr_t>(k_codes) |
                          reinterpret_cast<uintptr_t>(v_codes) | reinterpret_cast<uintptr_t>(out);
    const uintptr_t a4 = reinterpret_cast<uintptr_t>(q_scales) | reinterpret_cast<uintptr_t>(k_scales) |
                         reinterpret_cast<uintptr_t>(v_scales);
    if ((a16 & 15) || (a4 & 3))
      return fail(IKBO_ERR_INVALID_ARG, "codes and out must be 16-byte aligned, scales 4-byte aligned");
    const size_t out_bytes = static_cast<size_t>(R) * H * d * 2;
    const void* ins[6] = {q_codes, q_scales, k_codes, k_scales, v_codes, v_scales};
    const size_t in_sz[6] = {qb, qsb, kb, ksb, kb, vsb};
    for (int i = 0; i < 6; ++i)
      if (overlaps(out, out_bytes, ins[i], in_sz[i])) return fail(IKBO_ERR_INVALID_ARG, "out aliases an input");
    const int64_t n_items = static_cast<int64_t>(m->hp.items.size());
    if (n_items > std::numeric_limits<int32_t>::max() || kb > static_cast<size_t>(std::numeric_limits<int64_t>::max() / 2))
      return fail(IKBO_ERR_INVALID_ARG, "problem too large");

    // V-scale block range of every item: blocks of its user start at the
    // user's first block; the item reads blocks k0 / 32 .. ceil(k1 / 32) - 1.
    std::vector<int64_t> vbo(static_cast<size_t>(n_users) + 1, 0);
    for (int32_t u = 0; u < n_users; ++u)
      vbo[u + 1] = vbo[u] + (user_offsets[u + 1] - user_offsets[u] + ikbo::kMxBlock - 1) / ikbo::kMxBlock;
    m->vblk.resize(static_cast<size_t>(2 * n_items));
    for (int64_t i = 0; i < n_items; ++i) {
      const WorkItem& it = m->hp.items[i];
      // users with equal offsets (empty users in between) share their first block
      const int32_t u = static_cast<int32_t>(std::upper_bound(user_offsets, user_offsets + n_users, it.kv_base) -
                                             user_offsets) - 1;
      const int64_t b0 = vbo[std::max(u, 0)];
      m->vblk[2 * i] = static_cast<int32_t>(b0 + it.k0 / ikbo::kMxBlock);
      m->vblk[2 * i + 1] = static_cast<int32_t>(b0 + (it.k1 + ikbo::kMxBlock - 1) / ikbo::kMxBlock - 1);
    }
    const size_t slot_rows = static_cast<size_t>(m->hp.n_slots) * ikbo::kMxRows;
    if (slot_rows > 0 && ((rc = m->ws_o.ensure(slot_rows * ikbo::kMxHeadDim * 4, false)) != IKBO_OK ||
                          (rc = m->ws_rec.ensure(slot_rows * 16, false)) != IKBO_OK))
      return rc;

    // work list, candidate order and block ranges into the next pinned buffer
    const size_t items_bytes = static_cast<size_t>(n_items) * sizeof(WorkItem);
    const size_t perm_at = (items_bytes + 255) & ~size_t(255);
    const size_t vblk_at = perm_at + ((static_cast<size_t>(n_cand) * 4 + 255) & ~size_t(255));
    const size_t bytes = vblk_at + static_cast<size_t>(2 * n_items) * 4 + 256;
    int si = 0;
    if ((rc = m->ring.acquire(bytes, &si)) != IKBO_OK) return rc;
    char* base = static_cast<char*>(m->ring.buf[si].ptr);
    std::memcpy(base, m->hp.items.data(), items_bytes);
    std::memcpy(base + perm_at, m->hp.cand_perm.data(), static_cast<size_t>(n_cand) * 4);
    std::memcpy(base + vblk_at, m->vblk.data(), static_cast<size_t>(2 * n_items) * 4);

    hipEvent_t* te = nullptr;
    if ((rc = m->timed.next(&te, m->hp.n_groups > 0)) != IKBO_OK) return rc;
    ikbo::MxParams p{};
    p.q = static_cast<const uint8_t*>(q_codes);
    p.qs = static_cast<const uint8_t*>(q_scales);
    p.k = static_cast<const uint8_t*>(k_codes);
    p.ks = static_cast<const uint8_t*>(k_scales);
    p.v = static_cast<const uint8_t*>(v_codes);
    p.vs = static_cast<const uint8_t*>(v_scales);
    p.cand_perm = reinterpret_cast<const int32_t*>(base + perm_at);
    p.items = reinterpret_cast<const WorkItem*>(base);
    p.vblk = reinterpret_cast<const int32_t*>(base + vblk_at);
    p.n_items = static_cast<int32_t>(n_items);
    p.H = H;
    p.n_q = n_q;
    p.scale_log2 = static_cast<float>(static_cast<double>(scale) * 1.4426950408889634);
    p.out = out;
    p.ws_o = static_cast<float*>(m->ws_o.ptr);
    p.ws_rec = static_cast<float*>(m->ws_rec.ptr);
    if ((rc = m->ring.on_stream(stream)) != IKBO_OK) return rc;  // before anything is enqueued
    hipError_t e = ikbo::launch_mx(p, m->hp.grid, stream, te);
    if (e != hipSuccess) return fail_hip(e, "MXFP8 kernel launch");
    if (m->hp.n_groups > 0) {
      ikbo::AttnParams ap{};
      ap.out_cand = out;
      ap.H = H;
      ap.n_q = n_q;
      ap.ws_o = p.ws_o;
      ap.ws_rec = p.ws_rec;
      e = ikbo::launch_merge(ap, m->hp.n_groups, ikbo::kMxHeadDim, false, stream, te ? te + 2 : nullptr);
      if (e != hipSuccess) return fail_hip(e, "merge launch");
    }
    return m->ring.launched(si, stream);
  } catch (...) {
    return fail(IKBO_ERR_NOMEM, "unexpected host error");
  }
}

int ikbo_mx_info(void* mx, int64_t* info, int32_t n_info) {
  if (!mx || !info || n_info < 3) return fail(IKBO_ERR_INVALID_ARG, "mx and info[3] required");
  const Mx* m = static_cast<const Mx*>(mx);
  info[0] = static_cast<int64_t>(m->hp.items.size());
  info[1] = m->hp.n_groups;
  info[2] = m->hp.grid;
  return IKBO_OK;
}

int ikbo_mx_timing(void* mx, int32_t enable) {
  if (!mx) return fail(IKBO_ERR_INVALID_ARG, "mx is null");
  return static_cast<Mx*>(mx)->timed.enable(enable != 0);
}

int ikbo_mx_timing_read(void* mx, float* attn_ms, float* merge_ms, int32_t max_n, int32_t* n) {
  if (!mx || !n || max_n < 0 || (max_n > 0 && (!attn_ms || !merge_ms)))
    return fail(IKBO_ERR_INVALID_ARG, "null argument");
  Mx* m = static_cast<Mx*>(mx);
  const std::vector<hipEvent_t>& ev = m->timed.ev;
  const int cnt = std::min(m->timed.n, max_n);
  for (int i = 0; i < cnt; ++i) {
    IKBO_HIP(hipEventSynchronize(ev[4 * i + 1]));
    IKBO_HIP(hipEventElapsedTime(&attn_ms[i], ev[4 * i], ev[4 * i + 1]));
    merge_ms[i] = 0.0f;
    if (m->timed.flag[i]) {
      IKBO_HIP(hipEventSynchronize(ev[4 * i + 3]));
      IKBO_HIP(hipEventElapsedTime(&merge_ms[i], ev[4 * i + 2], ev[4 * i + 3]));
    }
  }
  *n = cnt;
  return IKBO_OK;
}

void ikbo_mx_destroy(void* mx) {
  if (!mx) return;
  Mx* m = static_cast<Mx*>(mx);
  int cur = -1;
  if (hipGetDevice(&cur) == hipSuccess) {
    (void)hipSetDevice(m->device);
    (void)hipDeviceSynchronize();
    (void)hipSetDevice(cur);
  }
  delete m;
}

}  // extern "C"
