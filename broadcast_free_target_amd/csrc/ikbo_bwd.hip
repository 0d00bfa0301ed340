// IKBO target-attention backward kernels for gfx950 (MI355X, CDNA4).
//
// What is computed: the gradient of IKBO target attention (IKBO blog, section
// 3.1, Fig. 10; section 1.2 notes the same kernels serve training when
// candidates outnumber users).  Each candidate's query rows attend over its
// user's K/V; the K/V is never copied per candidate, so the gradient of a
// user's K/V is the sum over all its candidates' rows.  With scores
// z = scale * q k^T, P = softmax(z), D = rowsum(dO * O) and dS = P * (dO V^T - D):
//   dQ = scale * dS K,   dK_u = scale * sum_rows dS^T q,   dV_u = sum_rows P^T dO.
// P is recomputed from the scores and a per-row log-sum-exp (AI-infra guide,
// section 4.6.3); there are two kernels, one per loop order (same section, and
// the TLX jagged-attention post, section 2.2: the dK/dV pass loops over K/V
// blocks outside and query rows inside, from a host-built tile list):
//
//   dQ kernel   one workgroup (4 wave64 x 32 rows) per CSR row tile of one
//               (user, head).  Pass 1 streams the user's K tiles and forms each
//               row's base-2 log-sum-exp; pass 2 streams K and V, rebuilds
//               P^T = exp2(S^T - lse), dP^T = V dO^T and dS^T, and accumulates
//               dQ^T = K^T dS^T.  It also writes, per row in user-sorted order,
//               the row index, the log-sum-exp and D for the second kernel.
//   dK/dV kernel  one workgroup (4 wave64 x 32 keys) per 128 keys of one
//               (user, head); K and V fragments stay in registers while the
//               user's candidate rows stream through LDS in 64-row tiles:
//               S = Q K^T, P, dP = dO V^T, dS, then dV^T += dO^T P and
//               dK^T += Q^T dS.  The sum over the user's candidates happens in
//               the accumulators: no atomics, results independent of schedule.
//
// MFMA v_mfma_f32_32x32x16_bf16 throughout.  Products that contract over d
// take the tile operand as a row-major 16-byte LDS read and the other from
// registers; products that contract over keys (dQ) or rows (dK, dV) take the
// accumulator of the previous product directly as the B operand (its 16
// values per lane, in the accumulator's own order) and read the matching rows
// of the tile with ds_read_b64_tr_b16 in the same order.
#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>

#include <cstdint>

#include "ikbo_bwd.h"
#include "ikbo_device.h"

namespace ikbo {
namespace {

using namespace dev;

constexpr int D = kBwdHeadDim;
constexpr int kCH = D / 8;    // 16-byte chunks per row
constexpr int kKS = D / 16;   // MFMA k-steps over d
constexpr int kDB = D / 32;   // 32-wide blocks of d
constexpr int kNT = 256;      // 4 wave64
constexpr float kNegInf = -__builtin_huge_valf();
static_assert(kCH == 16, "the tile swizzle assumes 256-byte rows");

// [rows][D] bf16 tile with 256-byte rows, chunk XOR swz(row): conflict-free for
// the 16-byte row reads and for the transposed 4-row reads.
__device__ __forceinline__ int t_off(int row, int chunk) { return (row * kCH + (chunk ^ swz(row))) * 8; }

__device__ __forceinline__ u32x4_t ld16(const uint16_t* p) { return *reinterpret_cast<const u32x4_t*>(p); }

__device__ __forceinline__ float dot8(u32x4_t a, u32x4_t b) {
  float s = 0.0f;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const uint32_t x = a[i], y = b[i];
    s += __builtin_bit_cast(float, x << 16) * __builtin_bit_cast(float, y << 16);
    s += __builtin_bit_cast(float, x & 0xffff0000u) * __builtin_bit_cast(float, y & 0xffff0000u);
  }
  return s;
}

// B operand from accumulator values base .. base+7 (rounded to bf16).
__device__ __forceinline__ bf16x8_t pack8(const f32x16_t& x, int base) {
  u32x4_t r;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const float lo = x[base + 2 * i], hi = x[base + 2 * i + 1];
    r[i] = bf16_bits(lo) | (bf16_bits(hi) << 16);
  }
  return as_bf16x8(r);
}

// A operand of a product that contracts over tile rows, matching a B operand
// taken from accumulator values v = 8*j0 .. 8*j0+7 of a 32-row block: those
// values belong to rows K0..K0+3 and K0+8..K0+11 with K0 = block + 16*j0 + 4*g.
// Lane kq of each 16-lane group points at (K0 + kq/4, D0 + 4*(kq%4)) and
// receives T[K0..K0+3][D0 + kq].
__device__ __forceinline__ bf16x8_t tr_rows(const uint16_t* T, int K0, int D0, int kq) {
  const int row = K0 + (kq >> 2), col = D0 + 4 * (kq & 3);
  const i16x4_t lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4_t*)(T + t_off(row, col >> 3) + (col & 4)));
  const i16x4_t hi =
      __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4_t*)(T + t_off(row + 8, col >> 3) + (col & 4)));
  return __builtin_bit_cast(bf16x8_t, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
}

// Two 32x32 blocks of T[rows 0..63] . B^T where B is one row per lane in
// registers (bf[ks] = its d values 16*ks + 8*g .. +7): result block kb holds
// row kb*32 + (v/4)*8 + 4*g + v%4 of T against the lane's own register row n.
__device__ __forceinline__ void tile_products(const uint16_t* T, const u32x4_t (&bf)[kKS], f32x16_t (&s)[2], int n,
                                              int g) {
#pragma unroll
  for (int kb = 0; kb < 2; ++kb) {
    s[kb] = f32x16_t{};
#pragma unroll
    for (int ks = 0; ks < kKS; ++ks)
      s[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(ld16(T + t_off(kb * 32 + n, ks * 2 + g))),
                                                      as_bf16x8(bf[ks]), s[kb], 0, 0, 0);
  }
}

// ---------------------------------------------------------------------------
// dQ kernel
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(kNT, 2) void ikbo_bwd_dq_kernel(BwdParams P) {
  constexpr int KT = kBwdKeysA;          // keys per tile
  constexpr int TE = KT * D;             // elements per K or V tile
  constexpr int LPT = KT * kCH / kNT;    // copies per thread per tile
  static_assert(LPT * kNT == KT * kCH, "tile shape");
  __shared__ __attribute__((aligned(16))) uint16_t smem[2 * 2 * TE];  // 2 stages x (K, V)

  const WorkItem it = P.items[blockIdx.x];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int n = lane & 31, g = lane >> 5, kq = lane & 15, half = (lane >> 4) & 1;
  const int wave_u = __builtin_amdgcn_readfirstlane(wave);
  const int L = it.k1 - it.k0;
  const int64_t rs = static_cast<int64_t>(P.H) * D;
  const int rloc = wave * 32 + n;
  const bool row_ok = rloc < it.nrows;
  const bool wave_live = wave * 32 < it.nrows;
  const int r = it.row0 + rloc;
  int64_t qrow = 0;
  if (row_ok) {
    const int cand = P.cand_perm[it.row_base + r / P.n_q];
    qrow = static_cast<int64_t>(cand) * P.n_q + r % P.n_q;
  }
  const int64_t qoff = qrow * rs + static_cast<int64_t>(it.h) * D;

  // This lane's row of Q and dO as B operands (d = 16*ks + 8*g .. +7), and D.
  u32x4_t qf[kKS], df[kKS];
  float dsum = 0.0f;
#pragma unroll
  for (int ks = 0; ks < kKS; ++ks) {
    if (row_ok) {
      const int64_t e = qoff + ks * 16 + g * 8;
      qf[ks] = ld16(static_cast<const uint16_t*>(P.q) + e);
      df[ks] = ld16(static_cast<const uint16_t*>(P.dout) + e);
      dsum += dot8(df[ks], ld16(static_cast<const uint16_t*>(P.o) + e));
    } else {
      qf[ks] = u32x4_t{0u, 0u, 0u, 0u};
      df[ks] = u32x4_t{0u, 0u, 0u, 0u};
    }
  }
  dsum += __shfl_xor(dsum, 32);
  // The row loads are complete before the ring starts, so the compiler has no
  // load of its own to wait for inside the loops.
  wait_vmcnt<0>();

  const uint32_t lds_base = lds_address(smem);
  const uint16_t* kg = static_cast<const uint16_t*>(P.k) + static_cast<int64_t>(it.kv_base) * rs + it.h * D;
  const uint16_t* vg = static_cast<const uint16_t*>(P.v) + static_cast<int64_t>(it.kv_base) * rs + it.h * D;
  const int ntiles = (L + KT - 1) / KT;
  auto issue = [&](int t, bool with_v) {
    const uint32_t st = lds_base + static_cast<uint32_t>((t & 1) * 2 * TE * 2);
#pragma unroll
    for (int c = 0; c < LPT; ++c) {
      const int u = tid + kNT * c;
      const int key = u / kCH, pos = u % kCH;
      const int64_t go = static_cast<int64_t>(min(t * KT + key, L - 1)) * rs + (pos ^ swz(key)) * 8;
      const uint32_t dst = st + static_cast<uint32_t>((kNT * c + 64 * wave_u) * 16);
      copy16_to_lds(kg + go, dst);
      if (with_v) copy16_to_lds(vg + go, dst + TE * 2);
    }
  };
  const float c2 = P.scale_log2;

  // Pass 1: base-2 log-sum-exp of each row over the user's keys.
  float m = kNegInf, l = 0.0f;
  if (ntiles > 0) issue(0, false);
  for (int t = 0; t < ntiles; ++t) {
    if (t + 1 < ntiles) {
      issue(t + 1, false);
      wait_vmcnt<LPT>();
    } else {
      wait_vmcnt<0>();
    }
    __syncthreads();
    if (wave_live) {
      const uint16_t* Kt = smem + (t & 1) * 2 * TE;
      f32x16_t s[2];
      tile_products(Kt, qf, s, n, g);
      float mx = kNegInf;
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int v = 0; v < 16; ++v) {
          const int key = t * KT + kb * 32 + (v >> 2) * 8 + g * 4 + (v & 3);
          const float x = key < L ? s[kb][v] * c2 : kNegInf;
          s[kb][v] = x;
          mx = fmaxf(mx, x);
        }
      mx = fmaxf(mx, __shfl_xor(mx, 32));
      const float mn = fmaxf(m, mx);  // finite: every tile holds a key of the user
      float sum = 0.0f;
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int v = 0; v < 16; ++v) sum += exp2f(s[kb][v] - mn);
      sum += __shfl_xor(sum, 32);
      l = l * exp2f(m - mn) + sum;
      m = mn;
    }
    __syncthreads();
  }
  const float lse = L > 0 ? m + log2f(l) : 0.0f;

  // Pass 2: dQ^T += K^T dS^T.
  f32x16_t dqa[kDB];
#pragma unroll
  for (int db = 0; db < kDB; ++db) dqa[db] = f32x16_t{};
  if (ntiles > 0) issue(0, true);
  for (int t = 0; t < ntiles; ++t) {
    if (t + 1 < ntiles) {
      issue(t + 1, true);
      wait_vmcnt<2 * LPT>();
    } else {
      wait_vmcnt<0>();
    }
    __syncthreads();
    if (wave_live) {
      const uint16_t* Kt = smem + (t & 1) * 2 * TE;
      const uint16_t* Vt = Kt + TE;
      f32x16_t s[2], dp[2];
      tile_products(Kt, qf, s, n, g);   // S^T: keys x this lane's row
      tile_products(Vt, df, dp, n, g);  // dP^T
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int v = 0; v < 16; ++v) {
          const int key = t * KT + kb * 32 + (v >> 2) * 8 + g * 4 + (v & 3);
          const float p = key < L ? exp2f(s[kb][v] * c2 - lse) : 0.0f;
          s[kb][v] = p * (dp[kb][v] - dsum);  // dS^T
        }
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int j0 = 0; j0 < 2; ++j0) {
          const bf16x8_t b = pack8(s[kb], j0 * 8);
#pragma unroll
          for (int db = 0; db < kDB; ++db)
            dqa[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
                tr_rows(Kt, kb * 32 + j0 * 16 + g * 4, db * 32 + half * 16, kq), b, dqa[db], 0, 0, 0);
        }
    }
    __syncthreads();
  }

  // dQ^T block db: lane value v is d = db*32 + (v/4)*8 + 4*g + v%4 of row n.
  if (row_ok) {
    uint16_t* dq = static_cast<uint16_t*>(P.dq) + qoff;
#pragma unroll
    for (int db = 0; db < kDB; ++db)
#pragma unroll
      for (int q4 = 0; q4 < 4; ++q4)
        *reinterpret_cast<u32x2_t*>(dq + db * 32 + q4 * 8 + g * 4) =
            pack4_bf16(P.scale * dqa[db][q4 * 4 + 0], P.scale * dqa[db][q4 * 4 + 1], P.scale * dqa[db][q4 * 4 + 2],
                       P.scale * dqa[db][q4 * 4 + 3]);
    if (g == 0) {
      const int64_t srow = static_cast<int64_t>(it.row_base) * P.n_q + r;
      const int64_t hb = static_cast<int64_t>(it.h) * (P.rows_total + kBwdPad);
      P.lse[hb + srow] = lse;
      P.dd[hb + srow] = dsum;
      if (it.h == 0) P.qrow[srow] = static_cast<int32_t>(qrow);
    }
  }
}

// ---------------------------------------------------------------------------
// dK / dV kernel
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(kNT, 1) void ikbo_bwd_dkv_kernel(BwdParams P) {
  constexpr int RT = kBwdRowsB;          // rows per tile
  constexpr int TE = RT * D;             // elements per Q or dO tile
  constexpr int LPT = RT * kCH / kNT;    // copies per thread per tile and tensor
  constexpr int META = 4 * RT;           // per stage: lse[RT], dd[RT], next tile's row ids[RT], spare[RT]
  constexpr int STAGE = 2 * TE * 2 + META * 4;  // bytes
  static_assert(LPT * kNT == RT * kCH && RT == 64, "tile shape");
  __shared__ __attribute__((aligned(16))) uint8_t smem[2 * STAGE];
  __shared__ int32_t first_rows[RT];

  const WorkItem it = P.items[blockIdx.x];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int n = lane & 31, g = lane >> 5, kq = lane & 15, half = (lane >> 4) & 1;
  const int wave_u = __builtin_amdgcn_readfirstlane(wave);
  const int64_t rs = static_cast<int64_t>(P.H) * D;
  const int nrows = it.nrows;
  const int ntiles = (nrows + RT - 1) / RT;
  const int64_t srow0 = static_cast<int64_t>(it.row_base) * P.n_q;
  const int64_t hb = static_cast<int64_t>(it.h) * (P.rows_total + kBwdPad);
  const int key = it.k0 + wave * 32 + n;
  const bool key_ok = key < it.k1;
  const bool wave_live = it.k0 + wave * 32 < it.k1;
  const int64_t koff = (static_cast<int64_t>(it.kv_base) + key) * rs + static_cast<int64_t>(it.h) * D;

  // This lane's key row of K and V as B operands (d = 16*ks + 8*g .. +7).
  u32x4_t kf[kKS], vf[kKS];
#pragma unroll
  for (int ks = 0; ks < kKS; ++ks) {
    if (key_ok) {
      kf[ks] = ld16(static_cast<const uint16_t*>(P.k) + koff + ks * 16 + g * 8);
      vf[ks] = ld16(static_cast<const uint16_t*>(P.v) + koff + ks * 16 + g * 8);
    } else {
      kf[ks] = u32x4_t{0u, 0u, 0u, 0u};
      vf[ks] = u32x4_t{0u, 0u, 0u, 0u};
    }
  }
  if (ntiles > 0 && tid < RT) first_rows[tid] = P.qrow[srow0 + min(tid, nrows - 1)];
  wait_vmcnt<0>();
  __syncthreads();

  const uint32_t lds_base = lds_address(smem);
  const uint16_t* qg = static_cast<const uint16_t*>(P.q) + static_cast<int64_t>(it.h) * D;
  const uint16_t* dg = static_cast<const uint16_t*>(P.dout) + static_cast<int64_t>(it.h) * D;
  // Stage t: the Q and dO rows of tile t (gathered by row id), then one copy by
  // wave 0 of tile t's log-sum-exp and D and of tile t+1's row ids.
  auto issue = [&](int t, const int32_t* rows) {
    const uint32_t st = lds_base + static_cast<uint32_t>((t & 1) * STAGE);
#pragma unroll
    for (int c = 0; c < LPT; ++c) {
      const int u = tid + kNT * c;
      const int row = u / kCH, pos = u % kCH;
      const int qr = t * RT + row < nrows ? rows[row] : rows[0];
      const int64_t go = static_cast<int64_t>(qr) * rs + (pos ^ swz(row)) * 8;
      const uint32_t dst = st + static_cast<uint32_t>((kNT * c + 64 * wave_u) * 16);
      copy16_to_lds(qg + go, dst);
      copy16_to_lds(dg + go, dst + TE * 2);
    }
    if (wave_u == 0) {
      const int part = lane >> 4, j = lane & 15;
      const int64_t at = srow0 + static_cast<int64_t>(t) * RT + 4 * j;
      const void* src = part == 0   ? static_cast<const void*>(P.lse + hb + at)
                        : part == 1 ? static_cast<const void*>(P.dd + hb + at)
                        : part == 2 ? static_cast<const void*>(P.qrow + at + RT)
                                    : static_cast<const void*>(P.lse + hb + srow0);
      copy16_to_lds(src, st + 2 * TE * 2);
    }
  };

  f32x16_t dka[kDB], dva[kDB];
#pragma unroll
  for (int db = 0; db < kDB; ++db) {
    dka[db] = f32x16_t{};
    dva[db] = f32x16_t{};
  }
  const float c2 = P.scale_log2;
  if (ntiles > 0) issue(0, first_rows);
  for (int t = 0; t < ntiles; ++t) {
    const uint8_t* slot = smem + (t & 1) * STAGE;
    wait_vmcnt<0>();
    __syncthreads();  // tile t and tile t+1's row ids are in LDS
    if (t + 1 < ntiles) issue(t + 1, reinterpret_cast<const int32_t*>(slot + 2 * TE * 2) + 2 * RT);
    if (wave_live) {
      const uint16_t* Qt = reinterpret_cast<const uint16_t*>(slot);
      const uint16_t* Dt = Qt + TE;
      const float* lse_t = reinterpret_cast<const float*>(slot + 2 * TE * 2);
      const float* dd_t = lse_t + RT;
      f32x16_t s[2], dp[2];
      tile_products(Qt, kf, s, n, g);   // S: rows x this lane's key
      tile_products(Dt, vf, dp, n, g);  // dP
#pragma unroll
      for (int rb = 0; rb < 2; ++rb)
#pragma unroll
        for (int q4 = 0; q4 < 4; ++q4) {
          const int rbase = rb * 32 + q4 * 8 + g * 4;
          const f32x4_t l4 = *reinterpret_cast<const f32x4_t*>(lse_t + rbase);
          const f32x4_t d4 = *reinterpret_cast<const f32x4_t*>(dd_t + rbase);
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const bool ok = t * RT + rbase + i < nrows;
            // rows past the user's count read padding: both products are forced to 0
            const float p = ok ? exp2f(s[rb][q4 * 4 + i] * c2 - l4[i]) : 0.0f;
            s[rb][q4 * 4 + i] = p;
            dp[rb][q4 * 4 + i] = ok ? p * (dp[rb][q4 * 4 + i] - d4[i]) : 0.0f;  // dS
          }
        }
#pragma unroll
      for (int rb = 0; rb < 2; ++rb)
#pragma unroll
        for (int j0 = 0; j0 < 2; ++j0) {
          const bf16x8_t bp = pack8(s[rb], j0 * 8);
          const bf16x8_t bs = pack8(dp[rb], j0 * 8);
          const int K0 = rb * 32 + j0 * 16 + g * 4;
#pragma unroll
          for (int db = 0; db < kDB; ++db) {
            dva[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(tr_rows(Dt, K0, db * 32 + half * 16, kq), bp, dva[db],
                                                              0, 0, 0);
            dka[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(tr_rows(Qt, K0, db * 32 + half * 16, kq), bs, dka[db],
                                                              0, 0, 0);
          }
        }
    }
    __syncthreads();  // every wave is done with this slot before it is refilled
  }

  // dK^T / dV^T block db: lane value v is d = db*32 + (v/4)*8 + 4*g + v%4 of key n.
  if (key_ok) {
    uint16_t* dk = static_cast<uint16_t*>(P.dk) + koff;
    uint16_t* dv = static_cast<uint16_t*>(P.dv) + koff;
#pragma unroll
    for (int db = 0; db < kDB; ++db)
#pragma unroll
      for (int q4 = 0; q4 < 4; ++q4) {
        const int d0 = db * 32 + q4 * 8 + g * 4;
        *reinterpret_cast<u32x2_t*>(dk + d0) =
            pack4_bf16(P.scale * dka[db][q4 * 4 + 0], P.scale * dka[db][q4 * 4 + 1], P.scale * dka[db][q4 * 4 + 2],
                       P.scale * dka[db][q4 * 4 + 3]);
        *reinterpret_cast<u32x2_t*>(dv + d0) =
            pack4_bf16(dva[db][q4 * 4 + 0], dva[db][q4 * 4 + 1], dva[db][q4 * 4 + 2], dva[db][q4 * 4 + 3]);
      }
  }
}

}  // namespace

hipError_t launch_bwd_dq(const BwdParams& p, int n_items, hipStream_t stream, hipEvent_t* ev) {
  if (n_items <= 0) return hipSuccess;
  if (ev)
    hipExtLaunchKernelGGL(ikbo_bwd_dq_kernel, dim3(n_items), dim3(kNT), 0, stream, ev[0], ev[1], 0, p);
  else
    hipLaunchKernelGGL(ikbo_bwd_dq_kernel, dim3(n_items), dim3(kNT), 0, stream, p);
  return hipGetLastError();
}

hipError_t launch_bwd_dkv(const BwdParams& p, int n_items, hipStream_t stream, hipEvent_t* ev) {
  if (n_items <= 0) return hipSuccess;
  if (ev)
    hipExtLaunchKernelGGL(ikbo_bwd_dkv_kernel, dim3(n_items), dim3(kNT), 0, stream, ev[0], ev[1], 0, p);
  else
    hipLaunchKernelGGL(ikbo_bwd_dkv_kernel, dim3(n_items), dim3(kNT), 0, stream, p);
  return hipGetLastError();
}

}  // namespace ikbo
