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
  // Split dQ items (grp >= 0) leave partials in slots: per slot 128 rows x d
  // fp32 dQ against the chunk's own log-sum-exp, and per row one 16-byte record
  // {lse_c, D, output unit qrow * H + h (or -1: no row), srow | nchunk << 27}.
  float* ws_dq;
  float* ws_rec;
  // Q and dO rows in user-sorted order, per head: [H][R + pad][d] bf16, written by
  // the dQ kernel, read by the dK/dV kernel as contiguous row tiles.  The
  // padding rows are zero (never written).
  uint16_t* qs;
  uint16_t* dos;
  // Optional: the forward's natural-log log-sum-exp per (row, head), [C, n_q, H]
  // fp32.  Given, the dQ kernel skips its log-sum-exp pass over the keys, every
  // key chunk of a split row uses the row's whole-range value, and the merge
  // sums the chunks' partials; null, the dQ kernel recomputes it.
  const float* lse_in;
  int32_t rows_total;   // R = n_cand * n_q
  int32_t H;
  int32_t n_q;
  float scale;          // softmax scale
  float scale_log2;     // scale * log2(e)
};

// dQ (and the per-row log-sum-exp and D): one workgroup per item
// (kv_base, row_base = cand_offsets[u], row0, nrows <= kBwdRowsA, key range
// [k0, k1), h, split group grp or -1, chunk, nchunk, slot0), the forward's
// work items.  ev (optional): ev[0] is stamped at the kernel's start, ev[1] at
// its end unless null.
hipError_t launch_bwd_dq(const BwdParams& p, int n_items, hipStream_t stream, hipEvent_t* ev = nullptr);
// Folds the split dQ partials of groups 0 .. n_groups-1 and writes dQ and the
// rows' log-sum-exp, D and row index.  ev_stop (optional) is stamped at its end.
hipError_t launch_bwd_merge(const BwdParams& p, int n_groups, hipStream_t stream, hipEvent_t ev_stop = nullptr);
// Largest sorted-row index the split records can hold (srow < 2^27).
constexpr int64_t kBwdMaxSplitRows = int64_t(1) << 27;
// dK and dV: one workgroup per item (kv_base, row_base, row0 = 0, nrows = all
// rows of the user, [k0, k1) <= kBwdKeysB keys, h).
hipError_t launch_bwd_dkv(const BwdParams& p, int n_items, hipStream_t stream, hipEvent_t* ev = nullptr);

}  // namespace ikbo
