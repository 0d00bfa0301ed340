// Launch interface of the MXFP8 IKBO target-attention kernel (host side).
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>

#include "ikbo_plan.h"

namespace ikbo {

constexpr int kMxHeadDim = 128;  // head dimension the MXFP8 kernel takes
constexpr int kMxRows = 128;     // query rows per work item (4 waves x 32)
constexpr int kMxKeys = 64;      // keys per K/V tile; chunk boundaries align to it
constexpr int kMxBlock = 32;     // elements per MX scale block

struct MxParams {
  const uint8_t* q;       // E4M3 codes [C, n_q, H, 128]
  const uint8_t* qs;      // E8M0 scales [C, n_q, H, 4]
  const uint8_t* k;       // E4M3 codes [T, H, 128]
  const uint8_t* ks;      // E8M0 scales [T, H, 4]
  const uint8_t* v;       // E4M3 codes [T, H, 128]
  const uint8_t* vs;      // E8M0 scales [NVB, H, 128]: 32-key blocks from each user's first key
  const int32_t* cand_perm;
  const WorkItem* items;
  const int32_t* vblk;    // per item: {V-scale block of its first key, last V-scale block it may read}
  int32_t n_items;
  int32_t H;
  int32_t n_q;
  float scale_log2;       // scale * log2(e)
  void* out;              // bf16 [C, n_q, H, 128]
  // Split items leave unnormalised O rows and row records in the layout the
  // bf16 path's merge kernel folds (slots of kMxRows rows x 128 fp32, one
  // 16-byte record per row).
  float* ws_o;
  float* ws_rec;
};

// One 4-wave workgroup per item at a time, persistent over the item list
// (boustrophedon deal, XCD-aware ids).  ev (optional): stamped at the
// kernel's start and end.
hipError_t launch_mx(const MxParams& p, int grid, hipStream_t stream, hipEvent_t* ev = nullptr);

}  // namespace ikbo
