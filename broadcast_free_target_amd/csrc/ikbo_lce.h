// Launch interface of the IKBO linear-compression kernels (host side).
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>

namespace ikbo {

// Output tile of one workgroup and the K rows of one ring stage.
constexpr int kLceTileM = 128;
constexpr int kLceTileN = 128;
constexpr int kLceTileK = 64;

struct LceParams {
  const void* w;               // packed W block [m_tiles * 128, ldw] bf16, zero padded
  int32_t ldw;                 // row stride of the packed block (K padded to 64)
  const void* x;               // [batches, K, N] bf16
  int32_t K, N, M;             // unpadded K of this block, N (multiple of 128), M
  int32_t m_tiles, n_tiles;    // ceil(M / 128), N / 128
  float* y;                    // user results [n_users, M, N] fp32 (written by mode 0, read by mode 1; may be null in mode 1)
  void* out;                   // mode 1: [batches, M, N] bf16
  const int32_t* cand_to_user; // mode 1: [batches]
  int32_t n_users;
  int32_t* errors;             // mode 1: count of mapping entries outside [0, n_users)
};

hipError_t launch_lce_pack(const void* w, int M, int ldw, int K_u, int K_c, int M_pad, int K_u_pad, int K_c_pad,
                           void* wu, void* wc, hipStream_t stream);
// mode 0: y[b] = W . x[b] (fp32); mode 1: out[b] = bf16(W . x[b] + y[cand_to_user[b]]).
hipError_t launch_lce_gemm(const LceParams& p, int mode, int batches, hipStream_t stream, hipEvent_t* ev = nullptr);

}  // namespace ikbo
