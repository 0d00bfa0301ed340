// Launch interface of the IKBO linear-compression kernels (host side).
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>

namespace ikbo {

// Output tile of one workgroup and the K rows of one ring stage.
constexpr int kLceTileM = 256;
constexpr int kLceTileN = 256;
constexpr int kLceTileK = 32;
// Floats of user results per output tile.
constexpr int kLceYTileFloats = kLceTileM * kLceTileN;
// N must be a multiple of this (a tile's second 128 columns may lie past N).
constexpr int kLceAlignN = 128;

struct LceParams {
  const void* w;               // packed W block [m_tiles * kLceTileM, ldw] bf16, zero padded
  int32_t ldw;                 // row stride of the packed block (K padded to kLceTileK)
  const void* x;               // [batches, K, N] bf16
  int32_t K, N, M;             // unpadded K of this block, N (multiple of kLceAlignN), M
  int32_t m_tiles, n_tiles;    // ceil(M / kLceTileM), ceil(N / kLceTileN)
  // Results of the parent level (fp32, tile by tile in accumulator order,
  // kLceYTileFloats per (parent, m tile, n tile)), added to every batch element
  // through map, or null; map entries outside [0, n_parent) give zero results
  // and are counted in errors.
  const float* y_in;
  const int32_t* map;          // [batches] batch element -> parent, or null
  int32_t n_parent;
  float* y_out;                // mode 0: this level's results, same layout as y_in
  void* out;                   // mode 1: [batches, M, N] bf16
  int32_t* errors;             // count of batch elements with an out-of-range map entry
  const int32_t* order;        // batches processed in this order ([batches], a permutation), or null
};

// W (M x ldw; columns: user [0, K_u), vendor [K_u, K_u + K_v), item after) into
// zero-padded blocks [M_pad, K_x_pad]; wv may be null when K_v = 0.
hipError_t launch_lce_pack(const void* w, int M, int ldw, int K_u, int K_v, int K_c, int M_pad, int K_u_pad,
                           int K_v_pad, int K_c_pad, void* wu, void* wv, void* wc, hipStream_t stream);
// Users at most the ordering kernel groups (more: identity order).
constexpr int kLceOrderMaxUsers = 8192;
// order[0 .. n_cand) = the candidates grouped by user (users ascending, entries
// outside [0, n_users) last; the order within a user is unspecified).  One
// workgroup; the order only decides which tiles run together.
hipError_t launch_lce_order(const int32_t* cand_to_user, int32_t n_cand, int32_t n_users, int32_t* order,
                            hipStream_t stream);
// mode 0: y_out[b] = W . x[b] (+ y_in[map[b]]), fp32 in accumulator order;
// mode 1: out[b] = bf16(W . x[b] + y_in[map[b]]) (y_in may be null).
hipError_t launch_lce_gemm(const LceParams& p, int mode, int batches, hipStream_t stream, hipEvent_t* ev = nullptr);

}  // namespace ikbo
