// C ABI of libikbo.so (declared in include/ikbo.h).
//
// Host responsibilities: argument checks, the host grouping pass and work
// list (ikbo_plan.cpp), workspaces, uploads and launches.  All device work is
// stream-ordered; the only host-device synchronisations are the ones the
// header documents (copying a device-resident mapping to the host).
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
#include "ikbo_api_attn.h"
#include "ikbo_api_common.h"
#include "ikbo_kernels.h"
#include "ikbo_plan.h"

namespace ikbo_host {
thread_local std::string g_last_error;

using ikbo::HostPlan;
using ikbo::PlanParams;
using ikbo::WorkItem;

// Depth of the bf16 kernel's HBM -> LDS ring (IKBO_STAGES overrides; 2, 3 or 4).
int bf16_stages() {
  const int s = env_int("IKBO_STAGES", ikbo::kBf16DefaultStages);
  return (s == 2 || s == 3 || s == 4) ? s : ikbo::kBf16DefaultStages;
}

// bf16 kernel variants: the eight-wave kernel (one per CU, two waves per
// SIMD) and the 4-wave kernel (two resident per CU).  By default a build plans
// for the eight-wave kernel and keeps it when every workgroup gets at most one
// item; otherwise it plans again for the 4-wave kernel, whose two independent
// workgroups per CU keep the SIMDs busier over many items.  IKBO_KERNEL =
// w8 | w4 forces a variant; w4r is the 4-wave kernel visiting each item's key
// tiles last to first (the reverse-order variant of the TLX attention post's
// persistent kernel).  The variant codes are in ikbo_api_attn.h.
int bf16_variant() {
  const char* s = std::getenv("IKBO_KERNEL");
  if (s && std::strcmp(s, "w4r") == 0) return kVariantW4R;
  if (s && std::strcmp(s, "w4") == 0) return kVariantW4;
  if (s && std::strcmp(s, "w8") == 0) return kVariantW8;
  return kVariantAuto;
}

PlanParams params_for(int n_cu, int32_t dtype, int variant) {
  PlanParams pp;
  if (dtype == IKBO_DTYPE_BF16 && variant != kVariantW4 && variant != kVariantW4R) {
    // one resident workgroup per CU; the 8-wave kernel's chunks are whole ring stages
    pp.bm = ikbo::kBf16TileRows;
    pp.bn = (variant == kVariantW8 ? 2 : 1) * ikbo::kBf16TileKeys;
    pp.grid_slots = std::max(1, n_cu);
    pp.min_chunk = 256;
    pp.allow_split = true;
    pp.single_pass = true;
  } else if (dtype == IKBO_DTYPE_BF16) {
    pp.bm = ikbo::kBf16TileRows;
    pp.bn = ikbo::kBf16TileKeys;
    pp.xcd_bins = env_int("IKBO_XCD_BINS", ikbo::kMaxBins);  // 0 or 1: no bins
    pp.grid_slots = std::max(1, n_cu * (bf16_stages() == 2 ? 2 : 1));
    pp.min_chunk = 256;
    pp.allow_split = true;
  } else {
    pp.bm = ikbo::kF32TileRows;
    pp.bn = ikbo::kF32TileKeys;
    pp.grid_slots = std::max(1, n_cu * 4);
    pp.allow_split = false;
  }
  // Test and tuning overrides.  IKBO_GRID_WGS changes only the launched grid;
  // IKBO_SPLIT_SLOTS and IKBO_MIN_CHUNK change how key ranges are split.
  pp.grid_slots = std::max(1, env_int("IKBO_SPLIT_SLOTS", pp.grid_slots));
  pp.launch_grid = std::max(0, env_int("IKBO_GRID_WGS", 0));
  pp.min_chunk = std::max(pp.bn, env_int("IKBO_MIN_CHUNK", pp.min_chunk));
  if (env_int("IKBO_NO_SPLIT", 0)) pp.allow_split = false;
  return pp;
}

int check_dims(int32_t n_users, int32_t n_cand, int32_t n_q, int32_t H, int32_t d, int32_t dtype) {
  if (n_users < 0 || n_cand < 0) return fail(IKBO_ERR_INVALID_ARG, "n_users and n_cand must be >= 0");
  if (H < 1) return fail(IKBO_ERR_INVALID_ARG, "H must be >= 1");
  if (n_q < 1) return fail(IKBO_ERR_INVALID_ARG, "n_q must be >= 1");
  if (dtype != IKBO_DTYPE_BF16 && dtype != IKBO_DTYPE_F32) return fail(IKBO_ERR_UNSUPPORTED, "dtype");
  if (d != 32 && d != 64 && d != 128) return fail(IKBO_ERR_UNSUPPORTED, "head dim must be 32, 64 or 128");
  if (n_cand > 0 && n_users == 0) return fail(IKBO_ERR_BAD_MAPPING, "candidates present but n_users == 0");
  return IKBO_OK;
}

// Plans one request: validation, grouping and the work list for the eight-wave
// kernel, or, when that plan needs more items than there are CUs, for the
// 4-wave kernel.  allow_split = false keeps every key range whole.
int plan_request(int n_cu, const int32_t* offs, const int32_t* c2u, int32_t n_users, int32_t n_cand, int32_t n_q,
                 int32_t H, int32_t d, int32_t dtype, int32_t with_self, bool allow_split, bool queued, HostPlan* hp,
                 int* variant_out) {
  int rc = check_dims(n_users, n_cand, n_q, H, d, dtype);
  if (rc != IKBO_OK) return rc;
  if (!offs || (n_cand > 0 && !c2u)) return fail(IKBO_ERR_INVALID_ARG, "null host mapping");
  std::string err;
  // Split partials name their output row as row * H + h in an int32.
  const int64_t out_units = std::max<int64_t>(static_cast<int64_t>(n_cand) * n_q, with_self ? offs[n_users] : 0) * H;
  const bool split_ok = allow_split && out_units < std::numeric_limits<int32_t>::max();
  const int forced = bf16_variant();
  int variant = forced == kVariantAuto ? kVariantW8 : forced;
  auto params = [&](int v) {
    PlanParams pp = params_for(n_cu, dtype, v);
    if (!split_ok) pp.allow_split = false;
    if (queued) {
      // Causal self rows re-read growing prefixes of their (user, head)'s K/V:
      // a bin works through its groups four at a time, so those prefixes stay
      // in its XCD's L2 (fused self + target request: read traffic 211 -> 146
      // MB per launch), and items of at most 256 keys wait for the end of the
      // bin, which then still ends on its shortest items.
      const bool spans = with_self != 0;
      pp.group_span = std::max(0, env_int("IKBO_GROUP_SPAN", spans ? 4 : 0));
      pp.span_tail = std::max(0, env_int("IKBO_SPAN_TAIL", spans ? 256 : 0));
    }
    return pp;
  };
  PlanParams pp = params(variant);
  rc = ikbo::build_plan(offs, c2u, n_users, n_cand, n_q, H, with_self != 0, pp, hp, &err);
  if (rc != ikbo::kOk) return fail(rc, err);
  if (dtype == IKBO_DTYPE_BF16 && forced == kVariantAuto && hp->items.size() > static_cast<size_t>(n_cu)) {
    variant = kVariantW4;
    pp = params(variant);
    rc = ikbo::build_plan(offs, c2u, n_users, n_cand, n_q, H, with_self != 0, pp, hp, &err);
    if (rc != ikbo::kOk) return fail(rc, err);
  }
  *variant_out = variant;
  return IKBO_OK;
}

// Checks the tensors of one launch against the sizes the plan touches: null
// pointers, outputs overlapping inputs or each other, 16-byte alignment.
int check_tensors(int32_t dtype, int32_t n_cand, int32_t n_q, int32_t H, int32_t d, int64_t total_len,
                  int32_t with_self, const void* q_cand, const void* q_user, const void* k, const void* v,
                  const void* out_cand, const void* out_user) {
  const size_t es = elem_size(dtype);
  const size_t row = static_cast<size_t>(H) * d * es;
  const size_t cand_bytes = static_cast<size_t>(n_cand) * n_q * row;
  const size_t kv_bytes = static_cast<size_t>(total_len) * row;
  const bool has_target = n_cand > 0;
  const bool has_self = with_self && total_len > 0;
  if (has_target && (!q_cand || !out_cand)) return fail(IKBO_ERR_INVALID_ARG, "null q_cand or out");
  if ((has_target || has_self) && total_len > 0 && (!k || !v)) return fail(IKBO_ERR_INVALID_ARG, "null k or v");
  if (has_self && (!q_user || !out_user)) return fail(IKBO_ERR_INVALID_ARG, "null q_user or out_user");
  const void* ins[4] = {q_cand, k, v, q_user};
  const size_t in_sz[4] = {cand_bytes, kv_bytes, kv_bytes, has_self ? kv_bytes : 0};
  for (int i = 0; i < 4; ++i) {
    if (has_target && overlaps(out_cand, cand_bytes, ins[i], in_sz[i]))
      return fail(IKBO_ERR_INVALID_ARG, "out_cand aliases an input");
    if (has_self && overlaps(out_user, kv_bytes, ins[i], in_sz[i]))
      return fail(IKBO_ERR_INVALID_ARG, "out_user aliases an input");
  }
  if (has_target && has_self && overlaps(out_cand, cand_bytes, out_user, kv_bytes))
    return fail(IKBO_ERR_INVALID_ARG, "out_cand and out_user overlap");
  const uintptr_t align_or = reinterpret_cast<uintptr_t>(q_cand) | reinterpret_cast<uintptr_t>(k) |
                             reinterpret_cast<uintptr_t>(v) | reinterpret_cast<uintptr_t>(out_cand) |
                             reinterpret_cast<uintptr_t>(q_user) | reinterpret_cast<uintptr_t>(out_user);
  if (align_or & 15) return fail(IKBO_ERR_INVALID_ARG, "tensor pointers must be 16-byte aligned");
  return IKBO_OK;
}

// Enqueues the attention kernel the plan chose and, for split key ranges, the
// merge.  te: optional events (attention start/end, merge start/end).
int launch_kernels(ikbo::AttnParams& ap, int32_t dtype, int variant, int d, int stages, const HostPlan& hp,
                   hipStream_t stream, hipEvent_t* te) {
  hipError_t e;
  if (dtype != IKBO_DTYPE_BF16)
    e = ikbo::launch_attn_f32(ap, d, hp.grid, stream, te);
  else if (variant == kVariantW8)
    e = ikbo::launch_attn_bf16_w8(ap, d, hp.grid, stream, te);
  else {
    ap.kv_reverse = variant == kVariantW4R ? 1 : 0;
    e = ikbo::launch_attn_bf16(ap, d, stages, hp.grid, stream, te);
  }
  if (e != hipSuccess) return fail_hip(e, "kernel launch");
  if (hp.n_groups > 0) {
    e = ikbo::launch_merge(ap, hp.n_groups, d, true, stream, te ? te + 2 : nullptr);
    if (e != hipSuccess) return fail_hip(e, "merge launch");
  }
  return IKBO_OK;
}

}  // namespace ikbo_host

using namespace ikbo_host;

namespace {

struct Plan {
  int device = -1;
  int n_cu = 0;
  // last build
  bool built = false;
  int32_t n_users = 0, n_cand = 0, n_q = 1, H = 0, d = 0, dtype = IKBO_DTYPE_BF16, with_self = 0;
  int32_t stages = 2;  // bf16 kernel ring depth chosen at build time
  int32_t variant = 0;  // bf16 kernel: kVariantW8, kVariantW4 or kVariantW4R
  int64_t total_len = 0;
  HostPlan hp;
  // device copies of the work list
  DevBuf d_items, d_ws_o, d_ws_rec;  // d_items: device copy of the plan buffer (copy mode)
  DevBuf d_queue;                     // the 4-wave kernel's per-bin item counters (zeroed once)
  bool static_deal = false;           // IKBO_STATIC_DEAL=1 at build: deal items statically instead
  // Pinned plan buffers, handed out in turn by the ring.  With in-place reads
  // (the default) the kernels read the work list from them; otherwise
  // (IKBO_PLAN_UPLOAD=copy) a copy to the device buffers above reads them.
  bool read_in_place = true;
  PinnedRing ring;
  std::mutex mu;  // held by the entry points that use a library-owned plan, for the whole call
  int cur_stage = 0;
  const WorkItem* k_items = nullptr;            // what the kernels read
  const int32_t* k_perm = nullptr;
  // optional kernel timing (measurement)
  TimedEvents timed;                            // flag: the launch had a merge kernel
  bool tracing = false;
  DevBuf d_trace;                               // [items, 6] uint64 per-item records
  // pinned landing area for device-resident mappings (synchronous entry points)
  PinnedBuf d2h;

  ~Plan() {
    timed.release();
    ring.release();
    d2h.release();
    d_items.release();
    d_ws_o.release();
    d_ws_rec.release();
    d_queue.release();
    d_trace.release();
  }
};

int plan_init(Plan* p) {
  IKBO_HIP(hipGetDevice(&p->device));
  hipDeviceProp_t prop;
  IKBO_HIP(hipGetDeviceProperties(&prop, p->device));
  p->n_cu = prop.multiProcessorCount;
  int rc = p->ring.init();
  if (rc != IKBO_OK) return rc;
  if ((rc = p->d_queue.ensure(2 * ikbo::kMaxBins * sizeof(int32_t), true)) != IKBO_OK) return rc;
  const char* up = std::getenv("IKBO_PLAN_UPLOAD");
  p->read_in_place = !(up && std::strcmp(up, "copy") == 0);
  return IKBO_OK;
}

int build_and_upload(Plan* p, const int32_t* offs, const int32_t* c2u, int32_t n_users, int32_t n_cand,
                     int32_t n_q, int32_t H, int32_t d, int32_t dtype, int32_t with_self, hipStream_t stream) {
  int dev = -1;
  IKBO_HIP(hipGetDevice(&dev));
  if (dev != p->device) return fail(IKBO_ERR_INVALID_ARG, "plan belongs to another device");
  // Build into the plan's own storage (reused across builds); until this plan build
  // completes the plan cannot be launched.
  p->built = false;
  HostPlan& hp = p->hp;
  int variant = kVariantW8;
  const bool static_deal = env_int("IKBO_STATIC_DEAL", 0) != 0;
  int rc = plan_request(p->n_cu, offs, c2u, n_users, n_cand, n_q, H, d, dtype, with_self, true, !static_deal, &hp,
                        &variant);
  if (rc != IKBO_OK) return rc;

  const int tile_rows = dtype == IKBO_DTYPE_BF16 ? ikbo::kBf16TileRows : ikbo::kF32TileRows;
  const size_t items_bytes = hp.items.size() * sizeof(WorkItem);
  const size_t perm_bytes = hp.cand_perm.size() * sizeof(int32_t);
  if ((rc = p->d_ws_o.ensure(static_cast<size_t>(hp.n_slots) * tile_rows * d * sizeof(float), false)) != IKBO_OK)
    return rc;
  if ((rc = p->d_ws_rec.ensure(static_cast<size_t>(hp.n_slots) * tile_rows * 4 * sizeof(float), false)) != IKBO_OK)
    return rc;

  // Write the work list into the next pinned buffer whose last reader has finished.
  const size_t a0 = 0, a1 = (items_bytes + 255) & ~size_t(255), a2 = a1 + ((perm_bytes + 255) & ~size_t(255));
  int s = 0;
  if ((rc = p->ring.acquire(a2 + 256, &s)) != IKBO_OK) return rc;
  char* hb = static_cast<char*>(p->ring.buf[s].ptr);
  if (items_bytes) std::memcpy(hb + a0, hp.items.data(), items_bytes);
  if (perm_bytes) std::memcpy(hb + a1, hp.cand_perm.data(), perm_bytes);
  if (p->read_in_place) {
    char* db = static_cast<char*>(p->ring.buf[s].dev);
    p->k_items = reinterpret_cast<const WorkItem*>(db + a0);
    p->k_perm = reinterpret_cast<const int32_t*>(db + a1);
  } else {
    if ((rc = p->d_items.ensure(a2 + 256, false)) != IKBO_OK) return rc;
    if ((rc = p->ring.on_stream(stream)) != IKBO_OK) return rc;
    IKBO_HIP(hipMemcpyAsync(p->d_items.ptr, hb, a2, hipMemcpyHostToDevice, stream));
    if ((rc = p->ring.launched(s, stream)) != IKBO_OK) return rc;  // the copy reads the buffer
    char* db = static_cast<char*>(p->d_items.ptr);
    p->k_items = reinterpret_cast<const WorkItem*>(db + a0);
    p->k_perm = reinterpret_cast<const int32_t*>(db + a1);
  }
  p->cur_stage = s;

  p->n_users = n_users;
  p->n_cand = n_cand;
  p->n_q = n_q;
  p->H = H;
  p->d = d;
  p->dtype = dtype;
  p->with_self = with_self;
  p->stages = bf16_stages();
  p->variant = variant;
  p->static_deal = static_deal;
  p->total_len = offs[n_users];
  p->built = true;
  return IKBO_OK;
}


int launch_planned(Plan* p, const void* q_cand, const void* q_user, const void* k, const void* v, float scale,
                   void* out_cand, void* out_user, hipStream_t stream, float* lse = nullptr) {
  if (!p->built) return fail(IKBO_ERR_INVALID_ARG, "plan has not been built");
  int dev = -1;
  IKBO_HIP(hipGetDevice(&dev));
  if (dev != p->device) return fail(IKBO_ERR_INVALID_ARG, "plan belongs to another device");
  if (!std::isfinite(scale)) return fail(IKBO_ERR_INVALID_ARG, "scale must be finite");
  int rc = check_tensors(p->dtype, p->n_cand, p->n_q, p->H, p->d, p->total_len, p->with_self, q_cand, q_user, k, v,
                         out_cand, out_user);
  if (rc != IKBO_OK) return rc;
  if (lse) {
    if (p->dtype != IKBO_DTYPE_BF16 || p->with_self)
      return fail(IKBO_ERR_UNSUPPORTED, "the log-sum-exp output needs a bf16 plan without self rows");
    const size_t es = elem_size(p->dtype);
    const size_t cand_bytes = static_cast<size_t>(p->n_cand) * p->n_q * p->H * p->d * es;
    const size_t kv_bytes = static_cast<size_t>(p->total_len) * p->H * p->d * es;
    const size_t lse_bytes = static_cast<size_t>(p->n_cand) * p->n_q * p->H * sizeof(float);
    if (reinterpret_cast<uintptr_t>(lse) & 3) return fail(IKBO_ERR_INVALID_ARG, "lse must be 4-byte aligned");
    if (overlaps(lse, lse_bytes, q_cand, cand_bytes) || overlaps(lse, lse_bytes, k, kv_bytes) ||
        overlaps(lse, lse_bytes, v, kv_bytes) || overlaps(lse, lse_bytes, out_cand, cand_bytes))
      return fail(IKBO_ERR_INVALID_ARG, "lse overlaps another tensor");
  }
  if (p->hp.items.empty()) return IKBO_OK;

  ikbo::AttnParams ap{};
  ap.lse = lse;
  ap.q_cand = q_cand;
  ap.q_user = q_user;
  ap.k = k;
  ap.v = v;
  ap.out_cand = out_cand;
  ap.out_user = out_user;
  ap.cand_perm = p->k_perm;
  ap.items = p->k_items;
  ap.n_items = static_cast<int32_t>(p->hp.items.size());
  ap.H = p->H;
  ap.n_q = p->n_q;
  ap.scale_log2 = static_cast<float>(static_cast<double>(scale) * 1.4426950408889634);
  ap.ws_o = static_cast<float*>(p->d_ws_o.ptr);
  ap.ws_rec = static_cast<float*>(p->d_ws_rec.ptr);
  ap.n_bins = p->hp.n_bins;
  for (int b = 0; b <= ikbo::kMaxBins; ++b) ap.bin_off[b] = p->hp.bin_off[b];
  // the queue only where workgroups take several items (a one-pass plan gives
  // each one item; its workgroups would only meet on the counters at the end)
  const bool multi_pass = p->hp.items.size() > static_cast<size_t>(p->hp.grid);
  ap.queue = p->static_deal || !multi_pass ? nullptr : static_cast<int32_t*>(p->d_queue.ptr);
  ap.trace = nullptr;
  if (p->tracing && p->dtype == IKBO_DTYPE_BF16) {
    if ((rc = p->d_trace.ensure(p->hp.items.size() * 6 * sizeof(uint64_t), false)) != IKBO_OK) return rc;
    ap.trace = static_cast<uint64_t*>(p->d_trace.ptr);
  }
  if ((rc = p->ring.on_stream(stream)) != IKBO_OK) return rc;  // before anything is enqueued
  hipEvent_t* te = nullptr;  // attention start/end, merge start/end (stamped by the dispatches)
  if ((rc = p->timed.next(&te, p->hp.n_groups > 0)) != IKBO_OK) return rc;
  if ((rc = launch_kernels(ap, p->dtype, p->variant, p->d, p->stages, p->hp, stream, te)) != IKBO_OK) return rc;
  if (p->read_in_place) {
    // The pinned work list of this plan build stays in use until these kernels end.
    if ((rc = p->ring.launched(p->cur_stage, stream)) != IKBO_OK) return rc;
  }
  return IKBO_OK;
}

// Library-owned plans for the entry points that take device-resident mappings,
// one per (device, stream).
std::mutex g_cache_mu;
std::map<std::pair<int, void*>, Plan*> g_plan_cache;

int cached_plan(hipStream_t stream, int slot, Plan** out) {
  int dev = -1;
  IKBO_HIP(hipGetDevice(&dev));
  std::lock_guard<std::mutex> lock(g_cache_mu);
  auto key = std::make_pair(dev * 4 + slot, static_cast<void*>(stream));
  auto it = g_plan_cache.find(key);
  if (it != g_plan_cache.end()) {
    *out = it->second;
    return IKBO_OK;
  }
  Plan* p = new (std::nothrow) Plan();
  if (!p) return fail(IKBO_ERR_NOMEM, "plan allocation");
  int rc = plan_init(p);
  if (rc != IKBO_OK) {
    delete p;
    return rc;
  }
  g_plan_cache[key] = p;
  *out = p;
  return IKBO_OK;
}

// Copies a device-resident mapping to pinned host memory and waits for it.
int fetch_mapping(Plan* p, const int32_t* offs_dev, const int32_t* c2u_dev, int32_t n_users, int32_t n_cand,
                  hipStream_t stream, const int32_t** offs_host, const int32_t** c2u_host) {
  if (!offs_dev || (n_cand > 0 && !c2u_dev)) return fail(IKBO_ERR_INVALID_ARG, "null user_offsets or cand_to_user");
  const size_t ob = (static_cast<size_t>(n_users) + 1) * sizeof(int32_t);
  const size_t cb = static_cast<size_t>(n_cand) * sizeof(int32_t);
  int rc = p->d2h.ensure(ob + cb + 16);
  if (rc != IKBO_OK) return rc;
  char* hb = static_cast<char*>(p->d2h.ptr);
  IKBO_HIP(hipMemcpyAsync(hb, offs_dev, ob, hipMemcpyDeviceToHost, stream));
  if (cb) IKBO_HIP(hipMemcpyAsync(hb + ob, c2u_dev, cb, hipMemcpyDeviceToHost, stream));
  IKBO_HIP(hipStreamSynchronize(stream));
  *offs_host = reinterpret_cast<const int32_t*>(hb);
  *c2u_host = reinterpret_cast<const int32_t*>(hb + ob);
  return IKBO_OK;
}

int attn_device_mapping(const void* q_cand, const void* q_user, const void* k, const void* v, const int32_t* offs,
                        const int32_t* c2u, int32_t n_users, int32_t n_cand, int32_t n_q, int32_t H, int32_t d,
                        float scale, int32_t dtype, int32_t with_self, void* out_cand, void* out_user,
                        void* stream_) {
  hipStream_t stream = static_cast<hipStream_t>(stream_);
  int rc = check_dims(n_users, n_cand, n_q, H, d, dtype);
  if (rc != IKBO_OK) return rc;
  if (n_cand == 0 && !with_self) return IKBO_OK;
  Plan* p = nullptr;
  if ((rc = cached_plan(stream, 0, &p)) != IKBO_OK) return rc;
  std::lock_guard<std::mutex> plan_lock(p->mu);
  const int32_t *ho = nullptr, *hc = nullptr;
  if ((rc = fetch_mapping(p, offs, c2u, n_users, n_cand, stream, &ho, &hc)) != IKBO_OK) return rc;
  if ((rc = build_and_upload(p, ho, hc, n_users, n_cand, n_q, H, d, dtype, with_self, stream)) != IKBO_OK) return rc;
  return launch_planned(p, q_cand, q_user, k, v, scale, out_cand, out_user, stream);
}

// Broadcast buffers of the materialised comparator, per device.
struct BcastWs {
  DevBuf kb, vb, meta;
  PinnedBuf host_meta;
};
std::mutex g_bcast_mu;
std::map<int, BcastWs*> g_bcast;

}  // namespace

extern "C" {

int ikbo_version(void) { return 100; }

const char* ikbo_last_error(void) { return g_last_error.c_str(); }

int ikbo_group_csr(const int32_t* cand_to_user_host, int32_t n_cand, int32_t n_users, int32_t n_q, int32_t bm,
                   int32_t* counts, int32_t* cand_offsets, int32_t* cand_perm, int32_t* tiles, int32_t max_tiles,
                   int32_t* n_tiles) {
  try {
    if ((n_cand > 0 && (!cand_to_user_host || !cand_perm)) || !cand_offsets || (n_users > 0 && !counts) ||
        !n_tiles || (max_tiles > 0 && !tiles) || max_tiles < 0)
      return fail(IKBO_ERR_INVALID_ARG, "null pointer or negative max_tiles");
    std::vector<int32_t> tv;
    std::string err;
    int64_t nt = 0;
    int rc = ikbo::group_csr(cand_to_user_host, n_cand, n_users, n_q, bm, counts, cand_offsets, cand_perm, &tv, &nt,
                             &err);
    if (rc != ikbo::kOk) return fail(rc, err);
    if (nt > std::numeric_limits<int32_t>::max()) return fail(IKBO_ERR_INVALID_ARG, "too many tiles");
    *n_tiles = static_cast<int32_t>(nt);
    if (nt > max_tiles) return fail(IKBO_ERR_INVALID_ARG, "max_tiles too small (n_tiles holds the size needed)");
    if (nt) std::memcpy(tiles, tv.data(), tv.size() * sizeof(int32_t));
    return IKBO_OK;
  } catch (const std::bad_alloc&) {
    return fail(IKBO_ERR_NOMEM, "host allocation");
  } catch (...) {
    return fail(IKBO_ERR_INVALID_ARG, "unexpected host error");
  }
}

int ikbo_plan_create(const int32_t* user_offsets_host, const int32_t* cand_to_user_host, int32_t n_users,
                     int32_t n_cand, int32_t n_q, int32_t H, int32_t d, int32_t dtype, int32_t with_self, void* stream,
                     void** plan) {
  if (!plan) return fail(IKBO_ERR_INVALID_ARG, "plan is null");
  *plan = nullptr;
  try {
    Plan* p = new (std::nothrow) Plan();
    if (!p) return fail(IKBO_ERR_NOMEM, "plan allocation");
    int rc = plan_init(p);
    if (rc == IKBO_OK)
      rc = build_and_upload(p, user_offsets_host, cand_to_user_host, n_users, n_cand, n_q, H, d, dtype, with_self,
                            static_cast<hipStream_t>(stream));
    if (rc != IKBO_OK) {
      delete p;
      return rc;
    }
    *plan = p;
    return IKBO_OK;
  } catch (const std::bad_alloc&) {
    return fail(IKBO_ERR_NOMEM, "host allocation");
  } catch (...) {
    return fail(IKBO_ERR_INVALID_ARG, "unexpected host error");
  }
}

int ikbo_plan_build(void* plan, const int32_t* user_offsets_host, const int32_t* cand_to_user_host, int32_t n_users,
                    int32_t n_cand, int32_t n_q, int32_t H, int32_t d, int32_t dtype, int32_t with_self,
                    void* stream) {
  if (!plan) return fail(IKBO_ERR_INVALID_ARG, "plan is null");
  try {
    return build_and_upload(static_cast<Plan*>(plan), user_offsets_host, cand_to_user_host, n_users, n_cand, n_q, H,
                            d, dtype, with_self, static_cast<hipStream_t>(stream));
  } catch (const std::bad_alloc&) {
    return fail(IKBO_ERR_NOMEM, "host allocation");
  } catch (...) {
    return fail(IKBO_ERR_INVALID_ARG, "unexpected host error");
  }
}

int ikbo_attn_fwd_planned(void* plan, const void* q_cand, const void* q_user, const void* k_user,
                          const void* v_user, float scale, void* out_cand, void* out_user, void* stream) {
  if (!plan) return fail(IKBO_ERR_INVALID_ARG, "plan is null");
  return launch_planned(static_cast<Plan*>(plan), q_cand, q_user, k_user, v_user, scale, out_cand, out_user,
                        static_cast<hipStream_t>(stream));
}

int ikbo_attn_fwd_hostmap(void* plan, const int32_t* user_offsets_host, const int32_t* cand_to_user_host,
                          int32_t n_users, int32_t n_cand, int32_t n_q, int32_t H, int32_t d, int32_t dtype,
                          int32_t with_self, const void* q_cand, const void* q_user, const void* k_user,
                          const void* v_user, float scale, void* out_cand, void* out_user, void* stream) {
  if (!plan) return fail(IKBO_ERR_INVALID_ARG, "plan is null");
  try {
    Plan* p = static_cast<Plan*>(plan);
    hipStream_t st = static_cast<hipStream_t>(stream);
    if (!std::isfinite(scale)) return fail(IKBO_ERR_INVALID_ARG, "scale must be finite");
    // The tensor checks need the request's sizes: run them before the build so
    // that an error leaves the plan's previous build in place.
    int rc = check_dims(n_users, n_cand, n_q, H, d, dtype);
    if (rc != IKBO_OK) return rc;
    if (!user_offsets_host) return fail(IKBO_ERR_INVALID_ARG, "null host mapping");
    std::string err;
    if ((rc = ikbo::check_offsets(user_offsets_host, n_users, &err)) != ikbo::kOk) return fail(rc, err);
    if ((rc = check_tensors(dtype, n_cand, n_q, H, d, user_offsets_host[n_users], with_self, q_cand, q_user, k_user,
                            v_user, out_cand, out_user)) != IKBO_OK)
      return rc;
    if ((rc = build_and_upload(p, user_offsets_host, cand_to_user_host, n_users, n_cand, n_q, H, d, dtype, with_self,
                               st)) != IKBO_OK)
      return rc;
    return launch_planned(p, q_cand, q_user, k_user, v_user, scale, out_cand, out_user, st);
  } catch (const std::bad_alloc&) {
    return fail(IKBO_ERR_NOMEM, "host allocation");
  } catch (...) {
    return fail(IKBO_ERR_INVALID_ARG, "unexpected host error");
  }
}

int ikbo_attn_fwd_train(void* plan, const void* q_cand, const void* k_user, const void* v_user, float scale,
                        void* out_cand, float* lse, void* stream) {
  if (!plan) return fail(IKBO_ERR_INVALID_ARG, "plan is null");
  Plan* p = static_cast<Plan*>(plan);
  if (p->built && p->n_cand > 0 && !lse) return fail(IKBO_ERR_INVALID_ARG, "lse is null");
  return launch_planned(p, q_cand, nullptr, k_user, v_user, scale, out_cand, nullptr,
                        static_cast<hipStream_t>(stream), lse);
}

void ikbo_plan_destroy(void* plan) {
  if (!plan) return;
  Plan* p = static_cast<Plan*>(plan);
  int cur = -1;
  if (hipGetDevice(&cur) == hipSuccess && p->device >= 0) {
    (void)hipSetDevice(p->device);
    (void)hipDeviceSynchronize();
    (void)hipSetDevice(cur);
  }
  delete p;
}

int ikbo_plan_info(void* plan, int64_t* info, int32_t n_info) {
  if (!plan || !info || n_info < 1) return fail(IKBO_ERR_INVALID_ARG, "null plan or info");
  const Plan* p = static_cast<const Plan*>(plan);
  // kernel: 0 fp32, 1 bf16 eight-wave, 2 bf16 4-wave, 4 bf16 4-wave with key
  // tiles in reverse order (3 is no longer used)
  const int64_t kernel = p->dtype != IKBO_DTYPE_BF16 ? 0
                         : p->variant == kVariantW8  ? 1
                         : p->variant == kVariantW4R ? 4
                                                     : 2;
  const int64_t v[9] = {static_cast<int64_t>(p->hp.items.size()),
                        p->hp.grid,
                        p->hp.n_groups,
                        p->hp.n_slots,
                        static_cast<int64_t>(p->hp.n_slots) *
                            (p->dtype == IKBO_DTYPE_BF16 ? ikbo::kBf16TileRows : ikbo::kF32TileRows) * (p->d + 4) * 4,
                        p->hp.n_target_tiles,
                        p->hp.n_self_tiles,
                        p->n_cu,
                        kernel};
  for (int i = 0; i < n_info && i < 9; ++i) info[i] = v[i];
  return IKBO_OK;
}

int ikbo_plan_timing(void* plan, int32_t enable) {
  if (!plan) return fail(IKBO_ERR_INVALID_ARG, "plan is null");
  return static_cast<Plan*>(plan)->timed.enable(enable != 0);
}

int ikbo_plan_timing_read(void* plan, float* attn_ms, float* merge_ms, int32_t max_n, int32_t* n) {
  if (!plan || !n || max_n < 0 || (max_n > 0 && (!attn_ms || !merge_ms)))
    return fail(IKBO_ERR_INVALID_ARG, "null argument");
  Plan* p = static_cast<Plan*>(plan);
  const std::vector<hipEvent_t>& ev = p->timed.ev;
  const int m = std::min<int>(p->timed.n, max_n);
  for (int i = 0; i < m; ++i) {
    IKBO_HIP(hipEventSynchronize(ev[4 * i + 1]));
    IKBO_HIP(hipEventElapsedTime(&attn_ms[i], ev[4 * i], ev[4 * i + 1]));
    merge_ms[i] = 0.0f;
    if (p->timed.flag[i]) {
      IKBO_HIP(hipEventSynchronize(ev[4 * i + 3]));
      IKBO_HIP(hipEventElapsedTime(&merge_ms[i], ev[4 * i + 2], ev[4 * i + 3]));
    }
  }
  *n = m;
  return IKBO_OK;
}

int ikbo_plan_trace(void* plan, int32_t enable) {
  if (!plan) return fail(IKBO_ERR_INVALID_ARG, "plan is null");
  static_cast<Plan*>(plan)->tracing = enable != 0;
  return IKBO_OK;
}

int ikbo_plan_trace_read(void* plan, int64_t* records, int32_t max_items, int32_t* n_items) {
  if (!plan || !n_items || max_items < 0 || (max_items > 0 && !records))
    return fail(IKBO_ERR_INVALID_ARG, "null argument");
  Plan* p = static_cast<Plan*>(plan);
  const int n = std::min<int>(max_items, static_cast<int>(p->hp.items.size()));
  *n_items = 0;
  if (!p->d_trace.ptr || n == 0) return IKBO_OK;
  IKBO_HIP(hipDeviceSynchronize());
  IKBO_HIP(hipMemcpy(records, p->d_trace.ptr, static_cast<size_t>(n) * 6 * sizeof(uint64_t), hipMemcpyDeviceToHost));
  *n_items = n;
  return IKBO_OK;
}

int ikbo_attn_fwd(const void* q_cand, const void* k_user, const void* v_user, const int32_t* user_offsets,
                  const int32_t* cand_to_user, int32_t n_users, int32_t n_cand, int32_t H, int32_t d, float scale,
                  void* out, void* stream) {
  try {
    return attn_device_mapping(q_cand, nullptr, k_user, v_user, user_offsets, cand_to_user, n_users, n_cand, 1, H, d,
                               scale, IKBO_DTYPE_BF16, 0, out, nullptr, stream);
  } catch (...) {
    return fail(IKBO_ERR_NOMEM, "unexpected host error");
  }
}

int ikbo_attn_fwd_f32(const void* q_cand, const void* k_user, const void* v_user, const int32_t* user_offsets,
                      const int32_t* cand_to_user, int32_t n_users, int32_t n_cand, int32_t H, int32_t d, float scale,
                      void* out, void* stream) {
  try {
    return attn_device_mapping(q_cand, nullptr, k_user, v_user, user_offsets, cand_to_user, n_users, n_cand, 1, H, d,
                               scale, IKBO_DTYPE_F32, 0, out, nullptr, stream);
  } catch (...) {
    return fail(IKBO_ERR_NOMEM, "unexpected host error");
  }
}

int ikbo_attn_fwd_mt(const void* q_cand, const void* k_user, const void* v_user, const int32_t* user_offsets,
                     const int32_t* cand_to_user, int32_t n_users, int32_t n_cand, int32_t H, int32_t d, float scale,
                     void* out, void* stream, int32_t n_q, int32_t dtype) {
  try {
    return attn_device_mapping(q_cand, nullptr, k_user, v_user, user_offsets, cand_to_user, n_users, n_cand, n_q, H,
                               d, scale, dtype, 0, out, nullptr, stream);
  } catch (...) {
    return fail(IKBO_ERR_NOMEM, "unexpected host error");
  }
}

int ikbo_attn_fwd_ex(const void* q_cand, const void* k_user, const void* v_user, const int32_t* user_offsets,
                     const int32_t* cand_to_user, int32_t n_users, int32_t n_cand, int32_t n_q, int32_t H, int32_t d,
                     float scale, int32_t dtype, void* out, void* stream) {
  try {
    return attn_device_mapping(q_cand, nullptr, k_user, v_user, user_offsets, cand_to_user, n_users, n_cand, n_q, H,
                               d, scale, dtype, 0, out, nullptr, stream);
  } catch (...) {
    return fail(IKBO_ERR_NOMEM, "unexpected host error");
  }
}

int ikbo_self_target_fwd(const void* q_user, const void* q_cand, const void* k_user, const void* v_user,
                         const int32_t* user_offsets, const int32_t* cand_to_user, int32_t n_users, int32_t n_cand,
                         int32_t H, int32_t d, float scale, int32_t dtype, void* out_user, void* out_cand,
                         void* stream) {
  try {
    return attn_device_mapping(q_cand, q_user, k_user, v_user, user_offsets, cand_to_user, n_users, n_cand, 1, H, d,
                               scale, dtype, 1, out_cand, out_user, stream);
  } catch (...) {
    return fail(IKBO_ERR_NOMEM, "unexpected host error");
  }
}

int ikbo_attn_fwd_materialized(const void* q_cand, const void* k_user, const void* v_user,
                               const int32_t* user_offsets, const int32_t* cand_to_user, int32_t n_users,
                               int32_t n_cand, int32_t H, int32_t d, float scale, void* out, void* stream_,
                               int32_t n_q, int32_t dtype) {
  try {
    hipStream_t stream = static_cast<hipStream_t>(stream_);
    int rc = check_dims(n_users, n_cand, n_q, H, d, dtype);
    if (rc != IKBO_OK) return rc;
    if (n_cand == 0) return IKBO_OK;
    if (!q_cand || !out || !k_user || !v_user) return fail(IKBO_ERR_INVALID_ARG, "null tensor pointer");
    Plan* p = nullptr;
    if ((rc = cached_plan(stream, 1, &p)) != IKBO_OK) return rc;
    std::lock_guard<std::mutex> plan_lock(p->mu);
    const int32_t *ho = nullptr, *hc = nullptr;
    if ((rc = fetch_mapping(p, user_offsets, cand_to_user, n_users, n_cand, stream, &ho, &hc)) != IKBO_OK) return rc;
    std::string err;
    if ((rc = ikbo::check_offsets(ho, n_users, &err)) != ikbo::kOk) return fail(rc, err);
    for (int32_t c = 0; c < n_cand; ++c)
      if (hc[c] < 0 || hc[c] >= n_users) return fail(IKBO_ERR_BAD_MAPPING, "cand_to_user entry outside [0, n_users)");
    // Copy the mapping out of the pinned landing area (the plan build below reuses the plan's buffers).
    std::vector<int32_t> offs(ho, ho + n_users + 1), c2u(hc, hc + n_cand);

    const size_t es = elem_size(dtype);
    const int64_t row_bytes = static_cast<int64_t>(H) * d * static_cast<int64_t>(es);
    const double max_gb = std::max(0.001, std::atof(std::getenv("IKBO_BCAST_MAX_GB") ? std::getenv("IKBO_BCAST_MAX_GB")
                                                                                        : "32"));
    const int64_t max_bytes = static_cast<int64_t>(max_gb * 1e9);
    int dev = -1;
    IKBO_HIP(hipGetDevice(&dev));
    BcastWs* ws = nullptr;
    {
      std::lock_guard<std::mutex> lock(g_bcast_mu);
      auto it = g_bcast.find(dev);
      if (it == g_bcast.end()) it = g_bcast.emplace(dev, new BcastWs()).first;
      ws = it->second;
    }
    const char* qc = static_cast<const char*>(q_cand);
    char* oc = static_cast<char*>(out);
    const int64_t cand_row_bytes = static_cast<int64_t>(n_q) * row_bytes;
    int32_t c0 = 0;
    while (c0 < n_cand) {
      // Candidates [c0, c1): the broadcast copy (K and V) must fit in max_bytes.
      int32_t c1 = c0;
      int64_t rows = 0;
      while (c1 < n_cand && c1 - c0 < 65535) {
        const int64_t L = offs[c2u[c1] + 1] - offs[c2u[c1]];
        if (c1 > c0 && 2 * (rows + L) * row_bytes > max_bytes) break;
        rows += L;
        ++c1;
      }
      if (rows > std::numeric_limits<int32_t>::max()) return fail(IKBO_ERR_INVALID_ARG, "broadcast chunk too large");
      const int32_t n = c1 - c0;
      if ((rc = ws->kb.ensure(static_cast<size_t>(std::max<int64_t>(rows, 1)) * row_bytes, false)) != IKBO_OK)
        return rc;
      if ((rc = ws->vb.ensure(static_cast<size_t>(std::max<int64_t>(rows, 1)) * row_bytes, false)) != IKBO_OK)
        return rc;
      // Per-candidate copy descriptors and the identity mapping of the broadcast problem.
      const size_t meta_bytes = static_cast<size_t>(n) * (8 + 8 + 4);
      if ((rc = ws->meta.ensure(meta_bytes + 64, false)) != IKBO_OK) return rc;
      if ((rc = ws->host_meta.ensure(meta_bytes + 64)) != IKBO_OK) return rc;
      int64_t* src = static_cast<int64_t*>(ws->host_meta.ptr);
      int64_t* dst = src + n;
      int32_t* len = reinterpret_cast<int32_t*>(dst + n);
      std::vector<int32_t> offs_b(static_cast<size_t>(n) + 1, 0), c2u_b(n);
      int32_t max_len = 0;
      for (int32_t i = 0; i < n; ++i) {
        const int32_t u = c2u[c0 + i];
        src[i] = offs[u];
        len[i] = offs[u + 1] - offs[u];
        dst[i] = offs_b[i];
        offs_b[i + 1] = offs_b[i] + len[i];
        c2u_b[i] = i;
        max_len = std::max(max_len, len[i]);
      }
      char* dmeta = static_cast<char*>(ws->meta.ptr);
      IKBO_HIP(hipMemcpyAsync(dmeta, src, meta_bytes, hipMemcpyHostToDevice, stream));
      hipError_t e = ikbo::launch_bcast_copy(k_user, v_user, ws->kb.ptr, ws->vb.ptr,
                                             reinterpret_cast<const int64_t*>(dmeta),
                                             reinterpret_cast<const int64_t*>(dmeta) + n,
                                             reinterpret_cast<const int32_t*>(dmeta + 16 * static_cast<size_t>(n)), n,
                                             row_bytes, max_len, stream);
      if (e != hipSuccess) return fail_hip(e, "broadcast copy launch");
      if ((rc = build_and_upload(p, offs_b.data(), c2u_b.data(), n, n, n_q, H, d, dtype, 0, stream)) != IKBO_OK)
        return rc;
      if ((rc = launch_planned(p, qc + c0 * cand_row_bytes, nullptr, ws->kb.ptr, ws->vb.ptr, scale,
                               oc + c0 * cand_row_bytes, nullptr, stream)) != IKBO_OK)
        return rc;
      c0 = c1;
      // The pinned descriptors and broadcast buffers are reused by the next chunk.
      if (c0 < n_cand) IKBO_HIP(hipStreamSynchronize(stream));
    }
    return IKBO_OK;
  } catch (const std::bad_alloc&) {
    return fail(IKBO_ERR_NOMEM, "host allocation");
  } catch (...) {
    return fail(IKBO_ERR_INVALID_ARG, "unexpected host error");
  }
}

}  // extern "C"
