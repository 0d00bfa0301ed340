// C ABI of libikbo.so, linear compression (declared in include/ikbo.h): W
// packing, the user / vendor / item GEMM launches and their workspaces.  All
// device work is stream-ordered; no call synchronises with the host except
// ikbo_lce_errors and the timing reads.
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
#include "ikbo_lce.h"

using namespace ikbo_host;

namespace {

// IKBO linear compression: packed W blocks, the user-result workspace and the
// mapping error counter, bound to one device.
struct Lce {
  int device = -1;
  bool nested = false;  // created for three levels (user -> vendor -> item)
  int32_t M = 0, K_u = 0, K_v = 0, K_c = 0, M_pad = 0, K_u_pad = 0, K_v_pad = 0, K_c_pad = 0;
  DevBuf wu, wv, wc, y, yv, errors, order;
  TimedEvents timed;  // per timed call: upper levels start/end, item GEMM start/end; flag: upper ran
  ~Lce() {
    timed.release();
    wu.release();
    wv.release();
    wc.release();
    y.release();
    yv.release();
    errors.release();
    order.release();
  }
};



int lce_create(void** lce, const void* w, int32_t M, int32_t K_u, int32_t K_v, int32_t K_c, int32_t ldw, bool nested,
               void* stream_) {
  if (!lce) return fail(IKBO_ERR_INVALID_ARG, "lce is null");
  *lce = nullptr;
  if (!w) return fail(IKBO_ERR_INVALID_ARG, "w is null");
  if (M < 1 || K_u < 0 || K_v < 0 || K_c < 0 || K_u + K_v + K_c < 1)
    return fail(IKBO_ERR_INVALID_ARG, "M >= 1, K blocks >= 0 and a positive total K required");
  if (ldw < K_u + K_v + K_c) return fail(IKBO_ERR_INVALID_ARG, "ldw must be >= the total K");
  if (static_cast<int64_t>(M) * ldw > std::numeric_limits<int32_t>::max()) return fail(IKBO_ERR_INVALID_ARG, "W too large");
  Lce* l = new (std::nothrow) Lce();
  if (!l) return fail(IKBO_ERR_NOMEM, "lce allocation");
  hipError_t e = hipGetDevice(&l->device);
  if (e != hipSuccess) {
    delete l;
    return fail_hip(e, "hipGetDevice");
  }
  l->nested = nested;
  l->M = M;
  l->K_u = K_u;
  l->K_v = K_v;
  l->K_c = K_c;
  l->M_pad = round_up(M, ikbo::kLceTileM);
  l->K_u_pad = round_up(K_u, ikbo::kLceTileK);
  l->K_v_pad = round_up(K_v, ikbo::kLceTileK);
  l->K_c_pad = round_up(K_c, ikbo::kLceTileK);
  int rc;
  if ((rc = l->wu.ensure(static_cast<size_t>(l->M_pad) * std::max(l->K_u_pad, 1) * 2, false)) != IKBO_OK ||
      (rc = l->wv.ensure(static_cast<size_t>(l->M_pad) * std::max(l->K_v_pad, 1) * 2, false)) != IKBO_OK ||
      (rc = l->wc.ensure(static_cast<size_t>(l->M_pad) * std::max(l->K_c_pad, 1) * 2, false)) != IKBO_OK ||
      (rc = l->errors.ensure(sizeof(int32_t), true)) != IKBO_OK) {
    delete l;
    return rc;
  }
  e = ikbo::launch_lce_pack(w, M, ldw, K_u, K_v, K_c, l->M_pad, l->K_u_pad, l->K_v_pad, l->K_c_pad, l->wu.ptr,
                            l->wv.ptr, l->wc.ptr, static_cast<hipStream_t>(stream_));
  if (e != hipSuccess) {
    delete l;
    return fail_hip(e, "pack launch");
  }
  *lce = l;
  return IKBO_OK;
}

// One level's GEMM: y_out (mode 0) or out (mode 1) for `batches` elements of x,
// with the parent level's results y_in added through map.
hipError_t lce_level(const Lce* l, const void* wblk, int32_t K_pad, const void* x, int32_t K, int32_t N,
                     int32_t n_tiles, const float* y_in, const int32_t* map, int32_t n_parent, float* y_out,
                     void* out, const int32_t* order, int mode, int32_t batches, hipStream_t stream, hipEvent_t* ev) {
  ikbo::LceParams p{};
  p.w = wblk;
  p.ldw = std::max(K_pad, 1);
  p.x = x;
  p.K = K;
  p.N = N;
  p.M = l->M;
  p.m_tiles = l->M_pad / ikbo::kLceTileM;
  p.n_tiles = n_tiles;
  p.y_in = y_in;
  p.map = map;
  p.n_parent = n_parent;
  p.y_out = y_out;
  p.out = out;
  p.errors = static_cast<int32_t*>(l->errors.ptr);
  p.order = order;
  return ikbo::launch_lce_gemm(p, mode, batches, stream, ev);
}

hipEvent_t* lce_timing_slot(Lce* l, bool upper) {
  hipEvent_t* te = nullptr;
  return l->timed.next(&te, upper) == IKBO_OK ? te : nullptr;
}

// Checks shared by the two forward calls: device, sizes, N, grid limits.
int lce_check(const Lce* l, int32_t n_parents_max, int32_t n_cand, int32_t N, int64_t* n_tiles_out) {
  int dev = -1;
  IKBO_HIP(hipGetDevice(&dev));
  if (dev != l->device) return fail(IKBO_ERR_INVALID_ARG, "lce belongs to another device");
  if (N < ikbo::kLceAlignN || N % ikbo::kLceAlignN != 0)
    return fail(IKBO_ERR_UNSUPPORTED, "N must be a positive multiple of 128");
  const int32_t n_tiles = (N + ikbo::kLceTileN - 1) / ikbo::kLceTileN;
  const int64_t per = static_cast<int64_t>(l->M_pad / ikbo::kLceTileM) * n_tiles;
  if (static_cast<int64_t>(std::max(n_parents_max, n_cand)) * per > std::numeric_limits<int32_t>::max() ||
      static_cast<int64_t>(std::max(n_parents_max, n_cand)) * l->M * N > std::numeric_limits<int32_t>::max() * 8LL)
    return fail(IKBO_ERR_INVALID_ARG, "problem too large");
  *n_tiles_out = n_tiles;
  return IKBO_OK;
}

}  // namespace

extern "C" {

int ikbo_lce_create(void** lce, const void* w, int32_t M, int32_t K_u, int32_t K_c, int32_t ldw, void* stream_) {
  try {
    return lce_create(lce, w, M, K_u, 0, K_c, ldw, false, stream_);
  } catch (...) {
    return fail(IKBO_ERR_NOMEM, "unexpected host error");
  }
}

int ikbo_lce3_create(void** lce, const void* w, int32_t M, int32_t K_u, int32_t K_v, int32_t K_c, int32_t ldw,
                     void* stream_) {
  try {
    return lce_create(lce, w, M, K_u, K_v, K_c, ldw, true, stream_);
  } catch (...) {
    return fail(IKBO_ERR_NOMEM, "unexpected host error");
  }
}

int ikbo_lce_fwd(void* lce, const void* x_user, const void* x_cand, const int32_t* cand_to_user, int32_t n_users,
                 int32_t n_cand, int32_t N, void* out, void* stream_) {
  try {
    if (!lce) return fail(IKBO_ERR_INVALID_ARG, "lce is null");
    Lce* l = static_cast<Lce*>(lce);
    if (l->nested) return fail(IKBO_ERR_INVALID_ARG, "a three-level handle takes ikbo_lce3_fwd");
    hipStream_t stream = static_cast<hipStream_t>(stream_);
    if (n_users < 0 || n_cand < 0) return fail(IKBO_ERR_INVALID_ARG, "n_users and n_cand must be >= 0");
    int64_t n_tiles = 0;
    int rc = lce_check(l, n_users, n_cand, N, &n_tiles);
    if (rc != IKBO_OK) return rc;
    if (n_cand == 0) return IKBO_OK;
    if (n_users == 0) return fail(IKBO_ERR_BAD_MAPPING, "candidates present but n_users == 0");
    if (!out || !cand_to_user || (l->K_c > 0 && !x_cand) || (l->K_u > 0 && !x_user))
      return fail(IKBO_ERR_INVALID_ARG, "null tensor pointer");
    const uintptr_t align_or = reinterpret_cast<uintptr_t>(x_user) | reinterpret_cast<uintptr_t>(x_cand) |
                               reinterpret_cast<uintptr_t>(out);
    if (align_or & 15) return fail(IKBO_ERR_INVALID_ARG, "tensor pointers must be 16-byte aligned");
    const size_t out_bytes = static_cast<size_t>(n_cand) * l->M * N * 2;
    if (overlaps(out, out_bytes, x_user, static_cast<size_t>(n_users) * l->K_u * N * 2) ||
        overlaps(out, out_bytes, x_cand, static_cast<size_t>(n_cand) * l->K_c * N * 2) ||
        overlaps(out, out_bytes, cand_to_user, static_cast<size_t>(n_cand) * 4))
      return fail(IKBO_ERR_INVALID_ARG, "out aliases an input");
    const int64_t per = static_cast<int64_t>(l->M_pad / ikbo::kLceTileM) * n_tiles;
    if (l->K_u > 0 && (rc = l->y.ensure(static_cast<size_t>(n_users) * per * ikbo::kLceYTileFloats * 4, false)) != IKBO_OK)
      return rc;
    if ((rc = l->order.ensure(static_cast<size_t>(n_cand) * 4, false)) != IKBO_OK) return rc;
    hipError_t e = ikbo::launch_lce_order(cand_to_user, n_cand, n_users, static_cast<int32_t*>(l->order.ptr), stream);
    if (e != hipSuccess) return fail_hip(e, "candidate ordering launch");
    hipEvent_t* te = lce_timing_slot(l, l->K_u > 0);
    float* yu = l->K_u > 0 ? static_cast<float*>(l->y.ptr) : nullptr;
    if (l->K_u > 0) {  // user GEMM at the user batch
      e = lce_level(l, l->wu.ptr, l->K_u_pad, x_user, l->K_u, N, static_cast<int32_t>(n_tiles), nullptr, nullptr, 0, yu,
                    nullptr, nullptr, 0, n_users, stream, te);
      if (e != hipSuccess) return fail_hip(e, "user GEMM launch");
    }
    // candidate GEMM with the gathered user result added in the epilogue
    e = lce_level(l, l->wc.ptr, l->K_c_pad, x_cand, l->K_c, N, static_cast<int32_t>(n_tiles), yu, cand_to_user, n_users,
                  nullptr, out, static_cast<const int32_t*>(l->order.ptr), 1, n_cand, stream, te ? te + 2 : nullptr);
    if (e != hipSuccess) return fail_hip(e, "candidate GEMM launch");
    return IKBO_OK;
  } catch (...) {
    return fail(IKBO_ERR_NOMEM, "unexpected host error");
  }
}

int ikbo_lce3_fwd(void* lce, const void* x_user, const void* x_vendor, const void* x_cand,
                  const int32_t* vendor_to_user, const int32_t* cand_to_vendor, int32_t n_users, int32_t n_vendors,
                  int32_t n_cand, int32_t N, void* out, void* stream_) {
  try {
    if (!lce) return fail(IKBO_ERR_INVALID_ARG, "lce is null");
    Lce* l = static_cast<Lce*>(lce);
    if (!l->nested) return fail(IKBO_ERR_INVALID_ARG, "a two-level handle takes ikbo_lce_fwd");
    hipStream_t stream = static_cast<hipStream_t>(stream_);
    if (n_users < 0 || n_vendors < 0 || n_cand < 0) return fail(IKBO_ERR_INVALID_ARG, "counts must be >= 0");
    int64_t n_tiles = 0;
    int rc = lce_check(l, std::max(n_users, n_vendors), n_cand, N, &n_tiles);
    if (rc != IKBO_OK) return rc;
    if (n_cand == 0) return IKBO_OK;
    if (n_vendors == 0 || n_users == 0) return fail(IKBO_ERR_BAD_MAPPING, "items present but no vendors or users");
    if (!out || !cand_to_vendor || !vendor_to_user || (l->K_c > 0 && !x_cand) || (l->K_v > 0 && !x_vendor) ||
        (l->K_u > 0 && !x_user))
      return fail(IKBO_ERR_INVALID_ARG, "null tensor pointer");
    const uintptr_t align_or = reinterpret_cast<uintptr_t>(x_user) | reinterpret_cast<uintptr_t>(x_vendor) |
                               reinterpret_cast<uintptr_t>(x_cand) | reinterpret_cast<uintptr_t>(out);
    if (align_or & 15) return fail(IKBO_ERR_INVALID_ARG, "tensor pointers must be 16-byte aligned");
    const size_t out_bytes = static_cast<size_t>(n_cand) * l->M * N * 2;
    if (overlaps(out, out_bytes, x_user, static_cast<size_t>(n_users) * l->K_u * N * 2) ||
        overlaps(out, out_bytes, x_vendor, static_cast<size_t>(n_vendors) * l->K_v * N * 2) ||
        overlaps(out, out_bytes, x_cand, static_cast<size_t>(n_cand) * l->K_c * N * 2) ||
        overlaps(out, out_bytes, cand_to_vendor, static_cast<size_t>(n_cand) * 4) ||
        overlaps(out, out_bytes, vendor_to_user, static_cast<size_t>(n_vendors) * 4))
      return fail(IKBO_ERR_INVALID_ARG, "out aliases an input");
    const int64_t per = static_cast<int64_t>(l->M_pad / ikbo::kLceTileM) * n_tiles;
    if ((l->K_u > 0 && (rc = l->y.ensure(static_cast<size_t>(n_users) * per * ikbo::kLceYTileFloats * 4, false)) != IKBO_OK) ||
        (rc = l->yv.ensure(static_cast<size_t>(n_vendors) * per * ikbo::kLceYTileFloats * 4, false)) != IKBO_OK ||
        (rc = l->order.ensure(static_cast<size_t>(n_cand) * 4, false)) != IKBO_OK)
      return rc;
    hipError_t e = ikbo::launch_lce_order(cand_to_vendor, n_cand, n_vendors, static_cast<int32_t*>(l->order.ptr), stream);
    if (e != hipSuccess) return fail_hip(e, "item ordering launch");
    hipEvent_t* te = lce_timing_slot(l, true);
    hipEvent_t ev_upper[2] = {te ? te[0] : nullptr, nullptr};
    float* yu = l->K_u > 0 ? static_cast<float*>(l->y.ptr) : nullptr;
    if (l->K_u > 0) {  // users
      e = lce_level(l, l->wu.ptr, l->K_u_pad, x_user, l->K_u, N, static_cast<int32_t>(n_tiles), nullptr, nullptr, 0, yu,
                    nullptr, nullptr, 0, n_users, stream, te ? ev_upper : nullptr);
      if (e != hipSuccess) return fail_hip(e, "user GEMM launch");
    }
    // vendors, each with its user's result added; the vendor GEMM runs even when
    // K_v = 0 (it then forwards the user result to the vendor batch)
    hipEvent_t ev_v[2] = {te && l->K_u == 0 ? te[0] : nullptr, te ? te[1] : nullptr};
    e = lce_level(l, l->wv.ptr, l->K_v_pad, x_vendor, l->K_v, N, static_cast<int32_t>(n_tiles), yu, vendor_to_user,
                  n_users, static_cast<float*>(l->yv.ptr), nullptr, nullptr, 0, n_vendors, stream, te ? ev_v : nullptr);
    if (e != hipSuccess) return fail_hip(e, "vendor GEMM launch");
    // items, each with its vendor's result added
    e = lce_level(l, l->wc.ptr, l->K_c_pad, x_cand, l->K_c, N, static_cast<int32_t>(n_tiles),
                  static_cast<const float*>(l->yv.ptr), cand_to_vendor, n_vendors, nullptr, out,
                  static_cast<const int32_t*>(l->order.ptr), 1, n_cand, stream, te ? te + 2 : nullptr);
    if (e != hipSuccess) return fail_hip(e, "item GEMM launch");
    return IKBO_OK;
  } catch (...) {
    return fail(IKBO_ERR_NOMEM, "unexpected host error");
  }
}

int ikbo_lce_errors(void* lce, int64_t* count) {
  if (!lce || !count) return fail(IKBO_ERR_INVALID_ARG, "null argument");
  Lce* l = static_cast<Lce*>(lce);
  int cur = -1;
  IKBO_HIP(hipGetDevice(&cur));
  if (cur != l->device) return fail(IKBO_ERR_INVALID_ARG, "lce belongs to another device");
  IKBO_HIP(hipDeviceSynchronize());
  int32_t v = 0;
  IKBO_HIP(hipMemcpy(&v, l->errors.ptr, sizeof(v), hipMemcpyDeviceToHost));
  IKBO_HIP(hipMemset(l->errors.ptr, 0, sizeof(int32_t)));
  *count = v;
  return IKBO_OK;
}

int ikbo_lce_timing(void* lce, int32_t enable) {
  if (!lce) return fail(IKBO_ERR_INVALID_ARG, "lce is null");
  return static_cast<Lce*>(lce)->timed.enable(enable != 0);
}

int ikbo_lce_timing_read(void* lce, float* user_ms, float* cand_ms, int32_t max_n, int32_t* n) {
  if (!lce || !n || max_n < 0 || (max_n > 0 && (!user_ms || !cand_ms))) return fail(IKBO_ERR_INVALID_ARG, "null argument");
  Lce* l = static_cast<Lce*>(lce);
  const std::vector<hipEvent_t>& ev = l->timed.ev;
  const int m = std::min<int>(l->timed.n, max_n);
  for (int i = 0; i < m; ++i) {
    user_ms[i] = 0.0f;
    if (l->timed.flag[i]) {
      IKBO_HIP(hipEventSynchronize(ev[4 * i + 1]));
      IKBO_HIP(hipEventElapsedTime(&user_ms[i], ev[4 * i], ev[4 * i + 1]));
    }
    IKBO_HIP(hipEventSynchronize(ev[4 * i + 3]));
    IKBO_HIP(hipEventElapsedTime(&cand_ms[i], ev[4 * i + 2], ev[4 * i + 3]));
  }
  *n = m;
  return IKBO_OK;
}

void ikbo_lce_destroy(void* lce) {
  if (!lce) return;
  Lce* l = static_cast<Lce*>(lce);
  int cur = -1;
  if (hipGetDevice(&cur) == hipSuccess) {
    (void)hipSetDevice(l->device);
    (void)hipDeviceSynchronize();
    (void)hipSetDevice(cur);
  }
  delete l;
}

}  // extern "C"
