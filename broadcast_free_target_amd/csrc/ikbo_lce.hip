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
// One kernel serves both GEMMs.  A workgroup of 8 wave64 (one per CU) computes
// a 256 x 256 tile of one batch element's M x N output, transposed: the MFMA
// forms out^T = x^T . W^T, so each lane's accumulator holds 4 consecutive
// output columns and the epilogue moves 8-byte bf16 stores and 16-byte fp32
// user-result loads.  Each wave owns 128 rows x 64 columns (4 x 2 blocks of
// v_mfma_f32_32x32x16_bf16).  W rows come from a zero-padded packed copy (K
// padded to a multiple of the 32-row stage, M to a multiple of 256: the padding
// of section 2.2, done once when W is packed); x rows past K load row K-1 again
// (finite data times a zero W column).  W and x tiles move HBM -> LDS with
// global_load_lds_dwordx4 through a 4-stage ring (128 KB), so up to three
// stages are in flight while one is multiplied.  The x fragment (8 consecutive
// k of one column) comes from two ds_read_b64_tr_b16 on the natural [k][n]
// tile; the W fragment is a row-major 16-byte LDS read.  32-row or 32-column
// blocks that lie wholly past M or N skip their MFMAs; the two waves sharing a
// SIMD take rows 0-127 and 128-255 of the tile, so a ragged M tail idles half
// of each SIMD's waves rather than whole SIMDs.
#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cstdint>
#include <type_traits>

#include "ikbo_device.h"
#include "ikbo_lce.h"

namespace ikbo {
namespace {

using namespace dev;

constexpr int kTM = kLceTileM;   // output rows (M) per workgroup
constexpr int kTN = kLceTileN;   // output columns (N) per workgroup
constexpr int kTK = kLceTileK;   // K rows per ring stage
#ifndef IKBO_LCE_WAVES_N
#define IKBO_LCE_WAVES_N 4
#endif
constexpr int kWavesM = 2;                       // waves along M (128 rows each)
constexpr int kWavesN = IKBO_LCE_WAVES_N;        // waves along N
constexpr int kNT = 64 * kWavesM * kWavesN;      // threads per workgroup
constexpr int kMB = kTM / (32 * kWavesM);        // 32-row blocks per wave (4)
constexpr int kNB = kTN / (32 * kWavesN);        // 32-column blocks per wave
constexpr int kWR = 32 * kMB, kWC = 32 * kNB;    // rows and columns per wave
#ifndef IKBO_LCE_STAGES
#define IKBO_LCE_STAGES 4
#endif
constexpr int kStages = IKBO_LCE_STAGES;

constexpr int kWChunks = kTK / 8;           // 16-byte chunks per W tile row (4)
constexpr int kXChunks = kTN / 8;           // 16-byte chunks per x tile row (32)
constexpr int kWElems = kTM * kTK;          // W tile elements
constexpr int kXElems = kTK * kTN;          // x tile elements
constexpr int kStageElems = kWElems + kXElems;
constexpr int kWLoads = kTM * kWChunks / kNT;  // 16-byte copies per thread per stage
constexpr int kXLoads = kTK * kXChunks / kNT;
static_assert(kWLoads * kNT == kTM * kWChunks && kXLoads * kNT == kTK * kXChunks, "tile shapes");
static_assert(kStages >= 3 && kStages <= 5 && kStages * kStageElems * 2 <= 160 * 1024, "LDS ring");
static_assert(kTM * kTN <= kStages * kStageElems, "the output tile is staged in the ring");

// W tile: 64-byte rows, four to a 256-byte bank line.  A 16-lane read group
// takes one chunk of 16 consecutive rows; XOR-ing the chunk with bits 2-3 of the
// row puts the four rows that share a line position on four distinct chunks.
__device__ __forceinline__ int w_off(int row, int chunk) { return (row * kWChunks + (chunk ^ ((row >> 2) & 3))) * 8; }
// x tile: 512-byte rows.  A transposed read covers 4 consecutive rows x 64
// bytes; XOR-ing the chunk with (row & 3) << 2 moves those 4 windows onto the 4
// quarters of a 256-byte bank line.
__device__ __forceinline__ int x_off(int row, int chunk) { return (row * kXChunks + (chunk ^ ((row & 3) << 2))) * 8; }

// Level results of tile (index, mt, nt), wave `wave`: kNB * kMB blocks of
// 4 x 64 lanes x 4 floats, in accumulator order (block (nb, mb), quarter q,
// lane) so that the writer and the reader move whole 1 KB requests.
__device__ __forceinline__ const f32x4_t* y_tile(const float* y, const LceParams& P, int index, int mt, int nt,
                                                 int wave) {
  const int64_t tile = (static_cast<int64_t>(index) * P.m_tiles + mt) * P.n_tiles + nt;
  return reinterpret_cast<const f32x4_t*>(y) + (tile * (kNT / 64) + wave) * (kNB * kMB * 4 * 64);
}

// MODE 0: y_out[batch] = acc (+ y_in[map[batch]]), fp32 in accumulator order.
// MODE 1: out[batch] = bf16(acc + y_in[map[batch]]), row-major.
template <int MODE>
__global__ __launch_bounds__(kNT, 1) void ikbo_lce_gemm_kernel(LceParams P) {
  __shared__ __attribute__((aligned(16))) uint16_t smem[kStages * kStageElems];

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int n = lane & 31, g = lane >> 5;
  const int kq = lane & 15, half = (lane >> 4) & 1;
  const int wm = wave / kWavesN, wn = wave % kWavesN;  // rows wm*kWR.., columns wn*kWC..

  // Tile of this workgroup: neighbouring logical ids share an XCD and take the
  // M tiles of one (batch, column tile), which read the same x tile.  Candidates
  // run grouped by user, so the tiles an XCD holds at once mostly read the same
  // user result from its L2.
  const int L = logical_wg();
  const int mt = L % P.m_tiles;
  const int nt = (L / P.m_tiles) % P.n_tiles;
  const int slot = L / (P.m_tiles * P.n_tiles);
  const int batch = P.order ? P.order[slot] : slot;
  const int m0 = mt * kTM, n0 = nt * kTN;

  int parent = 0;
  bool bad = false;
  if (P.map) {
    parent = P.map[batch];
    bad = parent < 0 || parent >= P.n_parent;
  }

  const uint16_t* __restrict__ Wp = static_cast<const uint16_t*>(P.w) + static_cast<int64_t>(m0) * P.ldw;
  const uint16_t* __restrict__ Xp = static_cast<const uint16_t*>(P.x) + static_cast<int64_t>(batch) * P.K * P.N;

  // Loader mapping: copy unit u of a tile lands at LDS unit u (row u / chunks,
  // position u % chunks) and holds the chunk that the swizzle puts there.
  // x columns past N (a 128-column tail) load an in-range column instead.
  int w_row[kWLoads], w_chk[kWLoads], x_row[kXLoads], x_col[kXLoads];
#pragma unroll
  for (int r = 0; r < kWLoads; ++r) {
    const int u = tid + kNT * r;
    w_row[r] = u / kWChunks;
    w_chk[r] = (u % kWChunks) ^ ((w_row[r] >> 2) & 3);
  }
#pragma unroll
  for (int r = 0; r < kXLoads; ++r) {
    const int u = tid + kNT * r;
    x_row[r] = u / kXChunks;
    x_col[r] = min(n0 + ((u % kXChunks) ^ ((x_row[r] & 3) << 2)) * 8, P.N - 8);
  }
  const uint32_t lds_base = lds_address(smem);
  const int wave_u = __builtin_amdgcn_readfirstlane(wave);
  const int nstages = (P.K + kTK - 1) / kTK;

  auto issue = [&](int s) {
    const uint32_t st = lds_base + static_cast<uint32_t>((s % kStages) * kStageElems * 2);
    const int k0 = s * kTK;
#pragma unroll
    for (int r = 0; r < kWLoads; ++r)
      copy16_to_lds(Wp + static_cast<int64_t>(w_row[r]) * P.ldw + k0 + w_chk[r] * 8,
                    st + static_cast<uint32_t>((kNT * r + 64 * wave_u) * 16));
#pragma unroll
    for (int r = 0; r < kXLoads; ++r) {
      const int k = min(k0 + x_row[r], P.K - 1);
      copy16_to_lds(Xp + static_cast<int64_t>(k) * P.N + x_col[r],
                    st + static_cast<uint32_t>(kWElems * 2 + (kNT * r + 64 * wave_u) * 16));
    }
  };

  // Waits until at most `ahead` stages' copies are outstanding.
  auto wait_stage = [&](int ahead) {
    constexpr int kL = kWLoads + kXLoads;
    static_assert(kL * (kStages - 2) < 64, "vmcnt range");
    if (kStages > 4 && ahead >= 3)
      wait_vmcnt<kL * (kStages > 4 ? 3 : 0)>();
    else if (ahead >= 2)
      wait_vmcnt<2 * kL>();
    else if (ahead == 1)
      wait_vmcnt<kL>();
    else
      wait_vmcnt<0>();
  };

  // Live 32-row blocks of this wave (0..4) and live 32-column blocks (0..2).
  const int m_live = max(0, min(kMB, (P.M - m0 - wm * kWR + 31) / 32));
  const int n_live = max(0, min(kNB, (P.N - n0 - wn * kWC) / 32));
  const bool full = m_live == kMB && n_live == kNB;

  // Accumulators.  Lane value v of block (nb, mb) is output row (M index)
  // m0 + wm*128 + mb*32 + n and column n0 + wn*64 + nb*32 + (v/4)*8 + g*4 + v%4.
  // A level with a parent starts from the parent's result, loaded while the
  // first ring stages are in flight.  One full wait then covers those loads
  // and the first stages: the compiler, which does not see the ring copies,
  // would otherwise guard the accumulators with a wait for every load in
  // flight at each ring step.
  f32x16_t acc[kNB][kMB];
  for (int s = 0; s < min(nstages, kStages - 1); ++s) issue(s);
  // Level results are kept in accumulator order (see the MODE 0 store), so
  // each 16-byte lane load is part of one contiguous 1 KB request.
  const f32x4_t* yt = (P.y_in && !bad) ? y_tile(P.y_in, P, parent, mt, nt, wave) : nullptr;
#pragma unroll
  for (int nb = 0; nb < kNB; ++nb)
#pragma unroll
    for (int mb = 0; mb < kMB; ++mb) {
      if (yt) {
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const f32x4_t t = yt[((nb * kMB + mb) * 4 + q) * 64 + lane];
          acc[nb][mb][q * 4 + 0] = t[0];
          acc[nb][mb][q * 4 + 1] = t[1];
          acc[nb][mb][q * 4 + 2] = t[2];
          acc[nb][mb][q * 4 + 3] = t[3];
        }
      } else {
        acc[nb][mb] = f32x16_t{};
      }
    }

  // Fragments of one k16 step: W^T for the wave's 4 row blocks, x^T for its 2
  // column blocks.
  struct Frag {
    u32x4_t w[kMB];
    bf16x8_t x[kNB];
  };
  auto read_frag = [&](int s, int ks, Frag& f) {
    const uint16_t* Wt = smem + (s % kStages) * kStageElems;
    const uint16_t* Xt = Wt + kWElems;
#pragma unroll
    for (int mb = 0; mb < kMB; ++mb)
      f.w[mb] = *reinterpret_cast<const u32x4_t*>(Wt + w_off(wm * kWR + mb * 32 + n, ks * 2 + g));
#pragma unroll
    for (int nb = 0; nb < kNB; ++nb) {
      // lane kq of each 16-lane group points at x[r][c]: the transposed read
      // returns x[r0 .. r0+3][column of this lane]; two reads give k = g*8 + 0..7.
      const int col = wn * kWC + nb * 32 + half * 16 + 4 * (kq & 3);
      const int r0 = ks * 16 + g * 8 + (kq >> 2);
      const i16x4_t lo =
          __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4_t*)(Xt + x_off(r0, col >> 3) + (col & 4)));
      const i16x4_t hi =
          __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4_t*)(Xt + x_off(r0 + 4, col >> 3) + (col & 4)));
      f.x[nb] = __builtin_bit_cast(bf16x8_t, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
    }
  };
  auto mma = [&](const Frag& f, auto full_tag) {
    constexpr bool kFull = decltype(full_tag)::value;
#pragma unroll
    for (int nb = 0; nb < kNB; ++nb)
#pragma unroll
      for (int mb = 0; mb < kMB; ++mb)
        if (kFull || (nb < n_live && mb < m_live))
          acc[nb][mb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(f.x[nb], as_bf16x8(f.w[mb]), acc[nb][mb], 0, 0, 0);
  };
  auto mma_live = [&](const Frag& f) {
    if (full)
      mma(f, std::true_type{});
    else if (m_live > 0 && n_live > 0)
      mma(f, std::false_type{});
  };

  // Ring: stage s lives in slot s % 4 and holds two k16 steps.  The second
  // step's fragments are read before the barrier that publishes stage s+1 and
  // multiplied after it, so the MFMA pipe stays fed while the first fragments of
  // stage s+1 come out of LDS.  Behind that barrier every wave has finished its
  // reads of slot s (the barrier waits for LDS reads), which then takes stage
  // s+4; stages s+2 and s+3 stay in flight meanwhile.
  wait_vmcnt<0>();
  __syncthreads();
  if (kStages - 1 < nstages) issue(kStages - 1);
  Frag f0, f1;
  if (nstages > 0) read_frag(0, 0, f0);
  for (int s = 0; s < nstages; ++s) {
    read_frag(s, 1, f1);
    mma_live(f0);
    if (s + 1 < nstages) {
      wait_stage(min(nstages - 2 - s, kStages - 2));  // issued stages after s+1
      __syncthreads();
      if (s + kStages < nstages) issue(s + kStages);
      read_frag(s + 1, 0, f0);
    }
    mma_live(f1);
  }

  if (bad && mt == 0 && nt == 0 && tid == 0) atomicAdd(P.errors, 1);  // once per batch element
  if (MODE == 0) {
    // Level results, fp32, in accumulator order: the whole tile, blocks past M
    // or N included (they hold zeros), lane-contiguous 16-byte stores.
    f32x4_t* yt = const_cast<f32x4_t*>(y_tile(P.y_out, P, batch, mt, nt, wave));
#pragma unroll
    for (int nb = 0; nb < kNB; ++nb)
#pragma unroll
      for (int mb = 0; mb < kMB; ++mb)
#pragma unroll
        for (int q = 0; q < 4; ++q)
          yt[((nb * kMB + mb) * 4 + q) * 64 + lane] =
              bad ? f32x4_t{}
                  : f32x4_t{acc[nb][mb][q * 4 + 0], acc[nb][mb][q * 4 + 1], acc[nb][mb][q * 4 + 2],
                            acc[nb][mb][q * 4 + 3]};
    return;
  }

  // Candidate outputs, bf16, staged through the (now idle) ring as a
  // [256][256] tile so that each output row leaves as 512 contiguous bytes.
  // The tile is kept in 8-byte units (4 columns), unit index XOR (row & 31):
  // the 32 rows one ds_write_b64 covers then land on 32 distinct units, and a
  // 16-byte read of an aligned unit pair stays one pair (halves swapped when
  // bit 0 of the XOR is set).
  __syncthreads();  // every wave is done with the last ring stage
  uint16_t* const tile = smem;
#pragma unroll
  for (int nb = 0; nb < kNB; ++nb) {
    if (nb >= n_live) continue;
#pragma unroll
    for (int mb = 0; mb < kMB; ++mb) {
      if (mb >= m_live) continue;
      const int row = wm * kWR + mb * 32 + n;
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int unit = wn * (kWC / 4) + nb * 8 + q * 2 + g;
        const u32x2_t v = bad ? u32x2_t{0u, 0u}
                              : pack4_bf16(acc[nb][mb][q * 4 + 0], acc[nb][mb][q * 4 + 1], acc[nb][mb][q * 4 + 2],
                                           acc[nb][mb][q * 4 + 3]);
        *reinterpret_cast<u32x2_t*>(tile + row * kTN + (unit ^ (row & 31)) * 4) = v;
      }
    }
  }
  __syncthreads();
  const int pr = tid & 31;  // unit pair (8 columns) of this thread within a row
#pragma unroll 4
  for (int r = tid >> 5; r < kTM; r += kNT / 32) {
    const int m = m0 + r, col = n0 + pr * 8;
    if (m >= P.M || col >= P.N) continue;
    const int x = r & 31;
    u32x4_t v = *reinterpret_cast<const u32x4_t*>(tile + r * kTN + (pr ^ (x >> 1)) * 8);
    if (x & 1) v = u32x4_t{v[2], v[3], v[0], v[1]};
    *reinterpret_cast<u32x4_t*>(static_cast<uint16_t*>(P.out) + (static_cast<int64_t>(batch) * P.M + m) * P.N + col) =
        v;
  }
}

// Counting sort of the candidates by user in one workgroup: counts in LDS,
// an exclusive scan, then a scatter through per-user cursors.
constexpr int kOrderThreads = 1024;
__global__ __launch_bounds__(kOrderThreads) void ikbo_lce_order_kernel(const int32_t* __restrict__ c2u, int n_cand,
                                                                       int n_users, int32_t* __restrict__ order) {
  __shared__ int cnt[kLceOrderMaxUsers + 1];
  __shared__ int part[kOrderThreads];
  const int tid = threadIdx.x;
  if (n_users > kLceOrderMaxUsers) {
    for (int c = tid; c < n_cand; c += kOrderThreads) order[c] = c;
    return;
  }
  const int nb = n_users + 1;  // bucket n_users takes out-of-range entries
  for (int i = tid; i < nb; i += kOrderThreads) cnt[i] = 0;
  __syncthreads();
  for (int c = tid; c < n_cand; c += kOrderThreads) {
    const int u = c2u[c];
    atomicAdd(&cnt[(u < 0 || u >= n_users) ? n_users : u], 1);
  }
  __syncthreads();
  // exclusive scan: each thread owns a contiguous run of buckets
  const int run = (nb + kOrderThreads - 1) / kOrderThreads;
  const int b0 = min(nb, tid * run), b1 = min(nb, b0 + run);
  int sum = 0;
  for (int i = b0; i < b1; ++i) sum += cnt[i];
  part[tid] = sum;
  __syncthreads();
  for (int off = 1; off < kOrderThreads; off <<= 1) {
    const int v = tid >= off ? part[tid - off] : 0;
    __syncthreads();
    part[tid] += v;
    __syncthreads();
  }
  int base = part[tid] - sum;
  for (int i = b0; i < b1; ++i) {
    const int c = cnt[i];
    cnt[i] = base;
    base += c;
  }
  __syncthreads();
  for (int c = tid; c < n_cand; c += kOrderThreads) {
    const int u = c2u[c];
    order[atomicAdd(&cnt[(u < 0 || u >= n_users) ? n_users : u], 1)] = c;
  }
}

// W (M x ldw; user columns [0, K_u), vendor columns [K_u, K_u + K_v), item
// columns after) into the zero-padded blocks [M_pad, K_u_pad], [M_pad, K_v_pad]
// and [M_pad, K_c_pad].
__global__ __launch_bounds__(256) void ikbo_lce_pack_kernel(const uint16_t* __restrict__ w, int M, int ldw, int K_u,
                                                           int K_v, int K_c, int M_pad, int K_u_pad, int K_v_pad,
                                                           int K_c_pad, uint16_t* __restrict__ wu,
                                                           uint16_t* __restrict__ wv, uint16_t* __restrict__ wc) {
  const int row_len = K_u_pad + K_v_pad + K_c_pad;
  const int64_t total = static_cast<int64_t>(M_pad) * row_len;
  for (int64_t i = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x; i < total;
       i += static_cast<int64_t>(gridDim.x) * blockDim.x) {
    const int m = static_cast<int>(i / row_len);
    const int k = static_cast<int>(i % row_len);
    if (k < K_u_pad) {
      wu[static_cast<int64_t>(m) * K_u_pad + k] = (m < M && k < K_u) ? w[static_cast<int64_t>(m) * ldw + k] : 0;
    } else if (k < K_u_pad + K_v_pad) {
      const int kv = k - K_u_pad;
      wv[static_cast<int64_t>(m) * K_v_pad + kv] =
          (m < M && kv < K_v) ? w[static_cast<int64_t>(m) * ldw + K_u + kv] : 0;
    } else {
      const int kc = k - K_u_pad - K_v_pad;
      wc[static_cast<int64_t>(m) * K_c_pad + kc] =
          (m < M && kc < K_c) ? w[static_cast<int64_t>(m) * ldw + K_u + K_v + kc] : 0;
    }
  }
}

}  // namespace

hipError_t launch_lce_pack(const void* w, int M, int ldw, int K_u, int K_v, int K_c, int M_pad, int K_u_pad,
                           int K_v_pad, int K_c_pad, void* wu, void* wv, void* wc, hipStream_t stream) {
  const int64_t total = static_cast<int64_t>(M_pad) * (K_u_pad + K_v_pad + K_c_pad);
  if (total <= 0) return hipSuccess;
  const int grid = static_cast<int>(std::min<int64_t>(4096, (total + 255) / 256));
  hipLaunchKernelGGL(ikbo_lce_pack_kernel, dim3(grid), dim3(256), 0, stream, static_cast<const uint16_t*>(w), M,
                     ldw, K_u, K_v, K_c, M_pad, K_u_pad, K_v_pad, K_c_pad, static_cast<uint16_t*>(wu),
                     static_cast<uint16_t*>(wv), static_cast<uint16_t*>(wc));
  return hipGetLastError();
}

hipError_t launch_lce_order(const int32_t* cand_to_user, int32_t n_cand, int32_t n_users, int32_t* order,
                            hipStream_t stream) {
  if (n_cand <= 0) return hipSuccess;
  hipLaunchKernelGGL(ikbo_lce_order_kernel, dim3(1), dim3(kOrderThreads), 0, stream, cand_to_user, n_cand, n_users,
                     order);
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
