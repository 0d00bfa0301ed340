// Launch interface of the IKBO target-attention backward kernels (host side).
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>

#include "ikbo_plan.h"

namespace ikbo {

constexpr int kBwdHeadDim = 128;   // head dimension the backward kernels take
constexpr int kBwdRowsA = 128;     // query rows per dQ workgroup (4 waves x 32)
constexpr int kBwdKeysA = 64;      // keys per K/V tile of the dQ kernel
constexpr int kBwdKeysB = 128;     // keys per dK/dV workgroup (4 waves x 32)
constexpr int kBwdRowsB = 64;      // query rows per tile of the dK/dV kernel
constexpr int kBwdPad = 2 * kBwdRowsB;  // padding entries after the sorted-row arrays (the
                                        // dK/dV kernel reads up to two tiles past a user's rows)

struct BwdParams {
  const void* q;        // q_cand [C, n_q, H, d] bf16
  const void* k;        // k_user [T, H, d]
  const void* v;        // v_user [T, H, d]
  const void* o;        // forward output, like q
  const void* dout;     // output gradient, like q
  void* dq;             // like q
  void* dk;             // like k
  void* dv;             // like v
  const WorkItem* items;      // dQ items (row tiles) or dK/dV items (key tiles)
  const int32_t* cand_perm;   // candidates grouped by user (CSR order)
  // Per query row in user-sorted order (sorted row = cand_offsets[u] * n_q + r),
  // written by the dQ kernel and read by the dK/dV kernel; each array has
  // kBwdPad entries of padding at the end.
  int32_t* qrow;        // [R + pad] row index cand * n_q + query
  float* lse;           // [H][R + pad] base-2 log-sum-exp of the row's scores
  float* dd;            // [H][R + pad] rowsum(dO * O)
  int32_t rows_total;   // R = n_cand * n_q
  int32_t H;
  int32_t n_q;
  float scale;          // softmax scale
  float scale_log2;     // scale * log2(e)
};

// dQ (and the per-row log-sum-exp and D): one workgroup per item
// (kv_base, row_base = cand_offsets[u], row0, nrows <= kBwdRowsA, k0 = 0, k1 = L_u, h).
hipError_t launch_bwd_dq(const BwdParams& p, int n_items, hipStream_t stream, hipEvent_t* ev = nullptr);
// dK and dV: one workgroup per item (kv_base, row_base, row0 = 0, nrows = all
// rows of the user, [k0, k1) <= kBwdKeysB keys, h).
hipError_t launch_bwd_dkv(const BwdParams& p, int n_items, hipStream_t stream, hipEvent_t* ev = nullptr);

}  // namespace ikbo
