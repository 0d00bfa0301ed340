// Launch interface of the IKBO device kernels (host side).
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>

#include "ikbo_plan.h"

namespace ikbo {

// Rows per workgroup tile and keys per K/V tile of the bf16 MFMA kernel.
constexpr int kBf16TileRows = 128;
constexpr int kBf16TileKeys = 64;
constexpr int kBf16DefaultStages = 2;
// Rows per tile of the fp32 kernel (one thread per row) and keys per tile.
constexpr int kF32TileRows = 64;
constexpr int kF32TileKeys = 32;

struct AttnParams {
  const void* q_cand;     // [n_cand, n_q, H, d]
  const void* q_user;     // [total_len, H, d] or null
  const void* k;          // [total_len, H, d]
  const void* v;          // [total_len, H, d]
  void* out_cand;         // [n_cand, n_q, H, d]
  void* out_user;         // [total_len, H, d] or null
  const int32_t* cand_perm;
  const WorkItem* items;
  int32_t n_items;
  int32_t H;
  int32_t n_q;
  float scale_log2;       // scale * log2(e): scores are kept in base 2
  void* ws_o;             // split partials: [slots, tile_rows, d] unnormalised O, fp16 with
                          // per-half-row power-of-two scales (bf16 kernels) or fp32 (MXFP8)
  float* ws_rec;          // split partials: [slots, tile_rows, 4] row records: running max m,
                          // running sum l, output unit (row * H + h, -1: no row) and a tag,
                          // the last two as int32 bits: nchunk | kind << 4 | c0 << 8 | c1 << 16
                          // (c_h: the half-row scale codes; 0 for fp32 partials)
  float* lse;             // optional (bf16 kernels, target rows): [n_cand, n_q, H] natural-log
                          // log-sum-exp of each row's scaled scores, or null
  uint64_t* trace;        // optional: [n_items, 6] per-item records (bf16 kernel), or null
  int32_t kv_reverse;     // 4-wave bf16 kernel: 1 = visit each item's key tiles last to first
  int32_t n_bins;         // 4-wave bf16 kernel: XCD bins of the work list (0: none), see HostPlan
  int32_t bin_off[kMaxBins + 1];
  int32_t* queue;         // 4-wave bf16 kernel: [2 * kMaxBins] per-bin next-item and finished-workgroup
                          // counters, zero before a launch and left zero by it (the last workgroup
                          // of a bin resets them); null: items dealt statically
};

// stages: depth of the HBM -> LDS ring (2, 3 or 4); 2 stages allow two
// resident workgroups per CU, 3-4 stages one.  ev (optional): two events the
// dispatch stamps at the kernel's start and end.
hipError_t launch_attn_bf16(const AttnParams& p, int d, int stages, int grid, hipStream_t stream,
                            hipEvent_t* ev = nullptr);
// Eight-wave variant (two waves per SIMD, key tiles alternating between the
// two wave halves, one resident workgroup per CU).  Work items are the same;
// key chunks should be multiples of 2 * kBf16TileKeys to keep both halves busy.
hipError_t launch_attn_bf16_w8(const AttnParams& p, int d, int grid, hipStream_t stream, hipEvent_t* ev = nullptr);
hipError_t launch_attn_f32(const AttnParams& p, int d, int grid, hipStream_t stream, hipEvent_t* ev = nullptr);
// Merges the split-KV partials of groups 0 .. n_groups-1 into the bf16 outputs.
// half_partials: the bf16 kernels' fp16 partials (any d); else fp32 partials
// (the MXFP8 kernel's, d = 128).
hipError_t launch_merge(const AttnParams& p, int n_groups, int d, bool half_partials, hipStream_t stream,
                        hipEvent_t* ev = nullptr);

// Materialised broadcast: for each of n local candidates, copy `len[c]` rows of
// `row_bytes` bytes from k/v at src_row[c] to kb/vb at dst_row[c].
hipError_t launch_bcast_copy(const void* k, const void* v, void* kb, void* vb,
                             const int64_t* src_row, const int64_t* dst_row, const int32_t* len,
                             int32_t n, int64_t row_bytes, int32_t max_len, hipStream_t stream);

}  // namespace ikbo
