// C ABI of libikbo.so: the allocation-free variant of the multi-target
// attention call (declared in include/ikbo.h).  It runs the same planner and
// kernels as ikbo_attn_fwd_mt, with every byte of kernel scratch in one
// file-scope device array of fixed size.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstdint>
#include <cstring>
#include <mutex>
#include <new>
#include <string>
#include <vector>

#include "ikbo.h"
#include "ikbo_api_attn.h"
#include "ikbo_api_common.h"
#include "ikbo_kernels.h"
#include "ikbo_plan.h"

using namespace ikbo_host;

namespace {

using ikbo::HostPlan;
using ikbo::WorkItem;

// The kernels' scratch memory -- split-KV partials and row records, then the
// work list and candidate order -- lives in one file-scope device array of
// fixed size instead of plan-owned allocations.  Each device holds its own
// copy for the life of the process; host code reaches it only through the
// address hipGetSymbolAddress returns for the current device (the array's
// name is a host-side stand-in, not a device address).  Host-side planning
// storage is reserved once, at the first call, for the largest request the
// scratch admits, so no later call allocates, on the host or the device.

constexpr size_t kNaPartialBytes = size_t(48) << 20;  // split partials: O and row records
constexpr size_t kNaListBytes = size_t(16) << 20;     // work items, then the candidate order
constexpr size_t kNaScratchBytes = kNaPartialBytes + kNaListBytes;
constexpr int32_t kNaMaxUsers = 1 << 16;
constexpr int32_t kNaMaxCand = 1 << 20;
constexpr int64_t kNaMaxItems = 1 << 17;
constexpr int kNaMaxDevices = 64;
static_assert(kNaMaxItems * sizeof(WorkItem) + size_t(kNaMaxCand) * 4 + 512 <= kNaListBytes, "work-list region");

static __device__ __align__(256) unsigned char scratch[kNaScratchBytes];

struct NoAlloc {
  std::mutex mu;                      // one call at a time per process (host staging is shared)
  void* ptr[kNaMaxDevices] = {};      // scratch address on each device, once taken
  int n_cu[kNaMaxDevices] = {};       // compute units of each device
  bool reserved = false;
  HostPlan hp;
  std::vector<int32_t> map_host;      // the mapping copied from the device: offsets, then cand_to_user
  std::vector<char> list_host;        // the work list and candidate order, staged for the copy
};
NoAlloc g_na;

// The scratch address and compute-unit count of the current device, taken
// once per device with that device current.
int na_scratch(void** out, int* n_cu) {
  int dev = -1;
  IKBO_HIP(hipGetDevice(&dev));
  if (dev < 0 || dev >= kNaMaxDevices) return fail(IKBO_ERR_UNSUPPORTED, "device index beyond the scratch table");
  if (!g_na.ptr[dev]) {
    void* ptr = nullptr;
    hipError_t e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return fail_hip(e, "hipGetSymbolAddress(scratch)");
    if (!ptr) return fail(IKBO_ERR_HIP, "hipGetSymbolAddress(scratch) returned null");
    int cu = 0;
    IKBO_HIP(hipDeviceGetAttribute(&cu, hipDeviceAttributeMultiprocessorCount, dev));
    g_na.n_cu[dev] = std::max(cu, 1);
    g_na.ptr[dev] = ptr;
  }
  *out = g_na.ptr[dev];
  *n_cu = g_na.n_cu[dev];
  return IKBO_OK;
}

// Host storage for the largest admitted request, reserved once.
void na_reserve() {
  if (g_na.reserved) return;
  HostPlan& hp = g_na.hp;
  hp.counts.reserve(kNaMaxUsers);
  hp.cand_offsets.reserve(kNaMaxUsers + 1);
  hp.cursor.reserve(kNaMaxItems);  // also the per-item group ids of the XCD bins
  hp.group_cost.reserve(kNaMaxItems);  // (user, head) groups: H * n_users <= the item limit
  hp.group_bin.reserve(kNaMaxItems);
  hp.cand_perm.reserve(kNaMaxCand);
  hp.items.reserve(kNaMaxItems);
  hp.unsorted.reserve(2 * kNaMaxItems);
  hp.groups.reserve(kNaMaxItems);
  hp.keys.reserve(2 * kNaMaxItems);
  hp.lens.reserve(kNaMaxItems);
  g_na.map_host.resize(static_cast<size_t>(kNaMaxUsers) + 1 + kNaMaxCand);
  g_na.list_host.resize(kNaListBytes);
  g_na.reserved = true;
}

int attn_noalloc(const void* q_cand, const void* k, const void* v, const int32_t* offs_dev, const int32_t* c2u_dev,
                 int32_t n_users, int32_t n_cand, int32_t n_q, int32_t H, int32_t d, float scale, int32_t dtype,
                 void* out, hipStream_t stream) {
  int rc = check_dims(n_users, n_cand, n_q, H, d, dtype);
  if (rc != IKBO_OK) return rc;
  if (n_cand == 0) return IKBO_OK;
  if (!std::isfinite(scale)) return fail(IKBO_ERR_INVALID_ARG, "scale must be finite");
  if (!offs_dev || !c2u_dev) return fail(IKBO_ERR_INVALID_ARG, "null user_offsets or cand_to_user");
  if (n_users > kNaMaxUsers || n_cand > kNaMaxCand)
    return fail(IKBO_ERR_INVALID_ARG, "request exceeds the allocation-free limits (65536 users, 1048576 candidates)");
  // Items before splitting: at most one per (head, row tile); row tiles of all
  // users are at most rows / 128 + n_users.  Splitting multiplies by at most
  // kMaxSplit and is only allowed when that bound fits.
  const int32_t tile_rows = dtype == IKBO_DTYPE_BF16 ? ikbo::kBf16TileRows : ikbo::kF32TileRows;
  const int64_t base_items = static_cast<int64_t>(H) * ((static_cast<int64_t>(n_cand) * n_q) / tile_rows + 1 + n_users);
  if (base_items > kNaMaxItems)
    return fail(IKBO_ERR_INVALID_ARG, "request exceeds the allocation-free work-list limit (131072 items)");
  const bool split_fits = base_items * ikbo::kMaxSplit <= kNaMaxItems;

  std::lock_guard<std::mutex> lock(g_na.mu);
  void* scr = nullptr;
  int n_cu = 1;
  if ((rc = na_scratch(&scr, &n_cu)) != IKBO_OK) return rc;
  na_reserve();
  // The mapping, from the device: one copy each into host staging, then wait.
  // The wait also orders this call after every earlier one on the stream, whose
  // kernels read the scratch this call is about to overwrite.
  int32_t* ho = g_na.map_host.data();
  int32_t* hc = ho + n_users + 1;
  IKBO_HIP(hipMemcpyAsync(ho, offs_dev, (static_cast<size_t>(n_users) + 1) * 4, hipMemcpyDeviceToHost, stream));
  IKBO_HIP(hipMemcpyAsync(hc, c2u_dev, static_cast<size_t>(n_cand) * 4, hipMemcpyDeviceToHost, stream));
  IKBO_HIP(hipStreamSynchronize(stream));
  HostPlan& hp = g_na.hp;
  int variant = kVariantW8;
  if ((rc = plan_request(n_cu, ho, hc, n_users, n_cand, n_q, H, d, dtype, 0, split_fits, false, &hp, &variant)) !=
      IKBO_OK)
    return rc;
  const int64_t total_len = ho[n_users];
  const size_t o_bytes = static_cast<size_t>(hp.n_slots) * tile_rows * d * sizeof(float);
  const size_t rec_at = (o_bytes + 255) & ~size_t(255);
  if (rec_at + static_cast<size_t>(hp.n_slots) * tile_rows * 4 * sizeof(float) > kNaPartialBytes) {
    // The split partials would not fit: plan again with whole key ranges.
    if ((rc = plan_request(n_cu, ho, hc, n_users, n_cand, n_q, H, d, dtype, 0, false, false, &hp, &variant)) !=
        IKBO_OK)
      return rc;
  }
  if ((rc = check_tensors(dtype, n_cand, n_q, H, d, total_len, 0, q_cand, nullptr, k, v, out, nullptr)) != IKBO_OK)
    return rc;
  if (hp.items.empty()) return IKBO_OK;
  const size_t items_bytes = hp.items.size() * sizeof(WorkItem);
  const size_t perm_at = (items_bytes + 255) & ~size_t(255);
  const size_t list_bytes = perm_at + hp.cand_perm.size() * sizeof(int32_t);
  if (hp.items.size() > static_cast<size_t>(kNaMaxItems) || list_bytes > kNaListBytes)
    return fail(IKBO_ERR_INVALID_ARG, "work list exceeds the allocation-free scratch");
  char* lh = g_na.list_host.data();
  std::memcpy(lh, hp.items.data(), items_bytes);
  std::memcpy(lh + perm_at, hp.cand_perm.data(), hp.cand_perm.size() * sizeof(int32_t));
  char* part = static_cast<char*>(scr);
  char* list = part + kNaPartialBytes;
  IKBO_HIP(hipMemcpyAsync(list, lh, list_bytes, hipMemcpyHostToDevice, stream));

  ikbo::AttnParams ap{};
  ap.q_cand = q_cand;
  ap.k = k;
  ap.v = v;
  ap.out_cand = out;
  ap.cand_perm = reinterpret_cast<const int32_t*>(list + perm_at);
  ap.items = reinterpret_cast<const WorkItem*>(list);
  ap.n_items = static_cast<int32_t>(hp.items.size());
  ap.H = H;
  ap.n_q = n_q;
  ap.scale_log2 = static_cast<float>(static_cast<double>(scale) * 1.4426950408889634);
  ap.ws_o = reinterpret_cast<float*>(part);
  ap.ws_rec = reinterpret_cast<float*>(part + (hp.n_slots > 0 ? rec_at : 0));
  ap.n_bins = hp.n_bins;
  for (int b = 0; b <= ikbo::kMaxBins; ++b) ap.bin_off[b] = hp.bin_off[b];
  ap.trace = nullptr;
  return launch_kernels(ap, dtype, variant, d, bf16_stages(), hp, stream, nullptr);
}

}  // namespace

extern "C" {

int ikbo_attn_fwd_mt_noalloc(const void* q_cand, const void* k_user, const void* v_user,
                             const int32_t* user_offsets, const int32_t* cand_to_user, int32_t n_users,
                             int32_t n_cand, int32_t H, int32_t d, float scale, void* out, void* stream, int32_t n_q,
                             int32_t dtype) {
  try {
    return attn_noalloc(q_cand, k_user, v_user, user_offsets, cand_to_user, n_users, n_cand, n_q, H, d, scale, dtype,
                        out, static_cast<hipStream_t>(stream));
  } catch (const std::bad_alloc&) {
    return fail(IKBO_ERR_NOMEM, "host allocation");
  } catch (...) {
    return fail(IKBO_ERR_INVALID_ARG, "unexpected host error");
  }
}

}  // extern "C"
