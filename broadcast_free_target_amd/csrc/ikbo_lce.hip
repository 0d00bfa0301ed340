// IKBO linear compression kernels for gfx950 (MI355X, CDNA4).
//
// What is computed (IKBO blog, section 2.1, Fig. 2; section 2.3, Fig. 3): the
// linear compression multiplies one learned matrix W (M x K) with every
// candidate's K input embeddings of width N.  The K embeddings are a user block
// (K_u rows, the same for every candidate of a user) followed by a candidate
// block (K_c rows).  Split W along K into W_u (M x K_u) and W_c (M x K_c):
//   user GEMM       y_u = W_u . x_user[u]                 once per user, fp32
//   candidate GEMM  out_b = W_c . x_cand[b] + y_{u(b)}     the user result is
//                   gathered through the mapping in the epilogue and added in
//                   registers, so neither the broadcast input nor a broadcast
//                   intermediate is ever written.
//
// One kernel serves both GEMMs: a workgroup of 4 wave64 computes a 128 x 128
// tile of one batch element's M x N output.  W rows come from a zero-padded
// packed copy (K padded to a multiple of the 64-row stage, M to a multiple of
// 128: the padding of section 2.2, done once when W is packed); x rows past K
// load row K-1 again (finite data times a zero W column).  K and x tiles move
// HBM -> LDS with global_load_lds_dwordx4 through a 2-stage ring; two
// workgroups share a CU.  MFMA v_mfma_f32_32x32x16_bf16: the W fragment is a
// row-major 16-byte LDS read, the x fragment (8 consecutive k of one column)
// comes from two ds_read_b64_tr_b16 on the natural [k][n] tile.
#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cstdint>

#include "ikbo_device.h"
#include "ikbo_lce.h"

namespace ikbo {
namespace {

using namespace dev;

constexpr int kTM = kLceTileM;   // output rows per workgroup
constexpr int kTN = kLceTileN;   // output columns per workgroup
constexpr int kTK = kLceTileK;   // K rows per ring stage
constexpr int kNT = 256;         // 4 wave64
constexpr int kStages = 2;

constexpr int kAChunks = kTK / 8;           // 16-byte chunks per W tile row (8)
constexpr int kBChunks = kTN / 8;           // 16-byte chunks per x tile row (16)
constexpr int kAElems = kTM * kTK;          // W tile elements
constexpr int kBElems = kTK * kTN;          // x tile elements
constexpr int kStageElems = kAElems + kBElems;
constexpr int kALoads = kTM * kAChunks / kNT;  // 16-byte copies per thread per stage
constexpr int kBLoads = kTK * kBChunks / kNT;
static_assert(kALoads * kNT == kTM * kAChunks && kBLoads * kNT == kTK * kBChunks, "tile shapes");

// W tile: 128-byte rows.  The chunk XOR takes 8 values over each pair of rows,
// so 16 consecutive rows (one 16-lane read group) hit 16 distinct
// (row parity, chunk) slots of a 256-byte bank line.
__device__ __forceinline__ int swz8(int row) { return (row >> 1) & 7; }
__device__ __forceinline__ int a_off(int row, int chunk) { return (row * kAChunks + (chunk ^ swz8(row))) * 8; }
// x tile: 256-byte rows, the attention kernels' swizzle.
__device__ __forceinline__ int b_off(int row, int chunk) { return (row * kBChunks + (chunk ^ swz(row))) * 8; }

// MODE 0: y[batch] = acc (fp32 store).  MODE 1: out[batch] = bf16(acc + y[user(batch)]).
template <int MODE>
__global__ __launch_bounds__(kNT, 2) void ikbo_lce_gemm_kernel(LceParams P) {
  __shared__ __attribute__((aligned(16))) uint16_t smem[kStages * kStageElems];

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int n = lane & 31, g = lane >> 5;
  const int kq = lane & 15, half = (lane >> 4) & 1;
  const int wm = wave & 1, wn = wave >> 1;  // this wave's 64 x 64 quadrant

  // Tile of this workgroup: neighbouring logical ids share an XCD and take the
  // M tiles of one (batch, column tile), which read the same x tile.
  const int L = logical_wg();
  const int mt = L % P.m_tiles;
  const int nt = (L / P.m_tiles) % P.n_tiles;
  const int batch = L / (P.m_tiles * P.n_tiles);
  const int m0 = mt * kTM, n0 = nt * kTN;

  int user = 0;
  bool bad = false;
  if (MODE == 1) {
    user = P.cand_to_user[batch];
    bad = user < 0 || user >= P.n_users;
  }

  const uint16_t* __restrict__ Wp = static_cast<const uint16_t*>(P.w) + static_cast<int64_t>(m0) * P.ldw;
  const uint16_t* __restrict__ Xp =
      static_cast<const uint16_t*>(P.x) + static_cast<int64_t>(batch) * P.K * P.N + n0;

  // Loader mapping: unit u of a tile lands at LDS unit u (row u / chunks, chunk
  // position u % chunks, holding the swizzled global chunk).
  int a_row[kALoads], a_chk[kALoads], b_row[kBLoads], b_chk[kBLoads];
#pragma unroll
  for (int r = 0; r < kALoads; ++r) {
    const int u = tid + kNT * r;
    a_row[r] = u / kAChunks;
    a_chk[r] = (u % kAChunks) ^ swz8(a_row[r]);
  }
#pragma unroll
  for (int r = 0; r < kBLoads; ++r) {
    const int u = tid + kNT * r;
    b_row[r] = u / kBChunks;
    b_chk[r] = (u % kBChunks) ^ swz(b_row[r]);
  }
  const uint32_t lds_base = lds_address(smem);
  const int wave_u = __builtin_amdgcn_readfirstlane(wave);
  const int nstages = (P.K + kTK - 1) / kTK;

  auto issue = [&](int s) {
    const uint32_t st = lds_base + static_cast<uint32_t>((s % kStages) * kStageElems * 2);
    const int k0 = s * kTK;
#pragma unroll
    for (int r = 0; r < kALoads; ++r)
      copy16_to_lds(Wp + static_cast<int64_t>(a_row[r]) * P.ldw + k0 + a_chk[r] * 8,
                    st + static_cast<uint32_t>((kNT * r + 64 * wave_u) * 16));
#pragma unroll
    for (int r = 0; r < kBLoads; ++r) {
      const int k = min(k0 + b_row[r], P.K - 1);
      copy16_to_lds(Xp + static_cast<int64_t>(k) * P.N + b_chk[r] * 8,
                    st + static_cast<uint32_t>((kAElems + (kNT * r + 64 * wave_u) * 8) * 2));
    }
  };

  f32x16_t acc[2][2];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j) acc[i][j] = f32x16_t{};

  // Waves whose 64 rows all lie past M do the loads and barriers but no MFMAs.
  const bool wave_live = m0 + wm * 64 < P.M;
  if (nstages > 0) issue(0);
  for (int s = 0; s < nstages; ++s) {
    wait_vmcnt<0>();
    __syncthreads();  // stage s is in LDS for every thread; stage s-1 is free
    if (s + 1 < nstages) issue(s + 1);
    if (wave_live) {
      const uint16_t* At = smem + (s % kStages) * kStageElems;
      const uint16_t* Bt = At + kAElems;
#pragma unroll
      for (int ks = 0; ks < kTK / 16; ++ks) {
        u32x4_t a[2];
#pragma unroll
        for (int mb = 0; mb < 2; ++mb)
          a[mb] = *reinterpret_cast<const u32x4_t*>(At + a_off(wm * 64 + mb * 32 + n, ks * 2 + g));
        bf16x8_t b[2];
#pragma unroll
        for (int nb = 0; nb < 2; ++nb) {
          // lane kq of each 16-lane group points at x[r][c]: the transposed read
          // returns x[r0 .. r0+3][column of this lane]; two reads give k = g*8 + 0..7.
          const int col = wn * 64 + nb * 32 + half * 16 + 4 * (kq & 3);
          const int r0 = ks * 16 + g * 8 + (kq >> 2);
          const i16x4_t lo =
              __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4_t*)(Bt + b_off(r0, col >> 3) + (col & 4)));
          const i16x4_t hi =
              __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4_t*)(Bt + b_off(r0 + 4, col >> 3) + (col & 4)));
          b[nb] = __builtin_bit_cast(bf16x8_t, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
        }
#pragma unroll
        for (int mb = 0; mb < 2; ++mb)
#pragma unroll
          for (int nb = 0; nb < 2; ++nb)
            acc[mb][nb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(a[mb]), b[nb], acc[mb][nb], 0, 0, 0);
      }
    }
  }

  // Epilogue.  Lane value v of block (mb, nb) is row wm*64 + mb*32 + (v/4)*8 +
  // g*4 + v%4 and column wn*64 + nb*32 + n of the tile.
  if (MODE == 1 && bad) {
    if (tid == 0) atomicAdd(P.errors, 1);
  }
#pragma unroll
  for (int mb = 0; mb < 2; ++mb) {
#pragma unroll
    for (int v = 0; v < 16; ++v) {
      const int m = m0 + wm * 64 + mb * 32 + (v >> 2) * 8 + g * 4 + (v & 3);
      if (m >= P.M) continue;
#pragma unroll
      for (int nb = 0; nb < 2; ++nb) {
        const int col = n0 + wn * 64 + nb * 32 + n;
        const int64_t o = (static_cast<int64_t>(batch) * P.M + m) * P.N + col;
        if (MODE == 0) {
          P.y[o] = acc[mb][nb][v];
        } else {
          float val = 0.0f;
          if (!bad) {
            val = acc[mb][nb][v];
            if (P.y) val += P.y[(static_cast<int64_t>(user) * P.M + m) * P.N + col];
          }
          static_cast<__bf16*>(P.out)[o] = static_cast<__bf16>(val);
        }
      }
    }
  }
}

// W (M x ldw, user columns [0, K_u), candidate columns [K_u, K_u + K_c)) into
// the two zero-padded blocks [M_pad, K_u_pad] and [M_pad, K_c_pad].
__global__ __launch_bounds__(256) void ikbo_lce_pack_kernel(const uint16_t* __restrict__ w, int M, int ldw, int K_u,
                                                           int K_c, int M_pad, int K_u_pad, int K_c_pad,
                                                           uint16_t* __restrict__ wu, uint16_t* __restrict__ wc) {
  const int64_t total = static_cast<int64_t>(M_pad) * (K_u_pad + K_c_pad);
  for (int64_t i = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x; i < total;
       i += static_cast<int64_t>(gridDim.x) * blockDim.x) {
    const int m = static_cast<int>(i / (K_u_pad + K_c_pad));
    const int k = static_cast<int>(i % (K_u_pad + K_c_pad));
    if (k < K_u_pad) {
      wu[static_cast<int64_t>(m) * K_u_pad + k] = (m < M && k < K_u) ? w[static_cast<int64_t>(m) * ldw + k] : 0;
    } else {
      const int kc = k - K_u_pad;
      wc[static_cast<int64_t>(m) * K_c_pad + kc] =
          (m < M && kc < K_c) ? w[static_cast<int64_t>(m) * ldw + K_u + kc] : 0;
    }
  }
}

}  // namespace

hipError_t launch_lce_pack(const void* w, int M, int ldw, int K_u, int K_c, int M_pad, int K_u_pad, int K_c_pad,
                           void* wu, void* wc, hipStream_t stream) {
  const int64_t total = static_cast<int64_t>(M_pad) * (K_u_pad + K_c_pad);
  if (total <= 0) return hipSuccess;
  const int grid = static_cast<int>(std::min<int64_t>(4096, (total + 255) / 256));
  hipLaunchKernelGGL(ikbo_lce_pack_kernel, dim3(grid), dim3(256), 0, stream, static_cast<const uint16_t*>(w), M,
                     ldw, K_u, K_c, M_pad, K_u_pad, K_c_pad, static_cast<uint16_t*>(wu), static_cast<uint16_t*>(wc));
  return hipGetLastError();
}

hipError_t launch_lce_gemm(const LceParams& p, int mode, int batches, hipStream_t stream, hipEvent_t* ev) {
  const int64_t grid = static_cast<int64_t>(batches) * p.m_tiles * p.n_tiles;
  if (grid <= 0) return hipSuccess;
  if (grid > 0x7fffffff) return hipErrorInvalidValue;
  const dim3 g(static_cast<unsigned>(grid));
  if (mode == 0) {
    if (ev)
      hipExtLaunchKernelGGL(ikbo_lce_gemm_kernel<0>, g, dim3(kNT), 0, stream, ev[0], ev[1], 0, p);
    else
      hipLaunchKernelGGL(ikbo_lce_gemm_kernel<0>, g, dim3(kNT), 0, stream, p);
  } else {
    if (ev)
      hipExtLaunchKernelGGL(ikbo_lce_gemm_kernel<1>, g, dim3(kNT), 0, stream, ev[0], ev[1], 0, p);
    else
      hipLaunchKernelGGL(ikbo_lce_gemm_kernel<1>, g, dim3(kNT), 0, stream, p);
  }
  return hipGetLastError();
}

}  // namespace ikbo
