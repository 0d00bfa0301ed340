// Host-side steps of the attention entry points shared by the source files of
// libikbo.so that launch the attention kernels: argument checks, planning a
// request and enqueuing the kernels the plan chose.  Defined in ikbo_api.hip.
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>

#include "ikbo_kernels.h"
#include "ikbo_plan.h"

namespace ikbo_host {

// bf16 kernel variants (ikbo_plan_info reports them as kernel codes 1, 2, 4).
enum { kVariantW8 = 1, kVariantW4 = 2, kVariantAuto = 3, kVariantW4R = 4 };

// Depth of the bf16 4-wave kernel's HBM -> LDS ring.
int bf16_stages();

// Sizes and dtype of one request (status code, message set on failure).
int check_dims(int32_t n_users, int32_t n_cand, int32_t n_q, int32_t H, int32_t d, int32_t dtype);

// Validates and plans one request from host mapping arrays into *hp: the
// eight-wave kernel's plan, or the 4-wave kernel's when the former needs more
// items than the device has CUs.  allow_split = false keeps key ranges whole.
// queued: the launch deals items from the per-bin work queue, so each XCD bin
// may list its items group by group (a static deal needs them longest first).
int plan_request(int n_cu, const int32_t* offs, const int32_t* c2u, int32_t n_users, int32_t n_cand, int32_t n_q,
                 int32_t H, int32_t d, int32_t dtype, int32_t with_self, bool allow_split, bool queued,
                 ikbo::HostPlan* hp, int* variant_out);

// Null, aliasing and alignment checks of one launch's tensors.
int check_tensors(int32_t dtype, int32_t n_cand, int32_t n_q, int32_t H, int32_t d, int64_t total_len,
                  int32_t with_self, const void* q_cand, const void* q_user, const void* k, const void* v,
                  const void* out_cand, const void* out_user);

// Enqueues the planned attention kernel and, for split key ranges, the merge.
int launch_kernels(ikbo::AttnParams& ap, int32_t dtype, int variant, int d, int stages, const ikbo::HostPlan& hp,
                   hipStream_t stream, hipEvent_t* te);

}  // namespace ikbo_host
