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
//               (user, head) and key chunk (long key ranges are split as in
//               the forward).  Pass 1 streams the chunk's K tiles and forms each
//               row's base-2 log-sum-exp over the chunk; pass 2 streams K and
//               V, rebuilds P^T = exp2(S^T - lse), dP^T = V dO^T and dS^T, and
//               accumulates dQ^T = K^T dS^T.  D = rowsum(dO * O) needs no keys,
//               so every chunk has it.  An unsplit item writes dQ and, per row
//               in user-sorted order, the row index, the log-sum-exp and D for
//               the second kernel; a split item leaves its dQ and log-sum-exp
//               in a slot and the merge kernel combines the chunks,
//                   lse = log2 sum_c 2^lse_c,  dQ = scale * sum_c 2^(lse_c - lse) dQ_c,
//               in chunk order (the log-sum-exp merge of the AI-infra guide,
//               section 4.6.4, applied to gradients), then writes the same rows.
//   dK/dV kernel  one workgroup per 128 keys of one (user, head), 8 wave64 in
//               two roles over the same keys: K (and V) fragments stay in
//               registers while the user's candidate rows stream through LDS
//               in 64-row tiles; one role forms S = Q K^T and P and accumulates
//               dV^T += dO^T P, the other forms S, dP = dO V^T and dS and
//               accumulates dK^T += Q^T dS.  The sum over the user's candidates
//               happens in the accumulators: no atomics, results independent
//               of schedule.
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
#include <type_traits>

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

#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"
// One 4-byte-per-lane HBM -> LDS copy (global_load_lds_dword, saddr form):
// lane l's 4 bytes from sbase + voff_bytes land at LDS byte lds_byte + 4*l.
__device__ __forceinline__ void copy4_to_lds_s(const void* sbase, uint32_t voff_bytes, uint32_t lds_byte) {
  asm volatile("s_mov_b32 m0, %2\n\tglobal_load_lds_dword %0, %1" ::"v"(voff_bytes), "s"(sbase), "s"(lds_byte)
               : "memory", "m0");
}
#pragma clang diagnostic pop

// B operand from accumulator values base .. base+7 (rounded to bf16, nearest
// even; one v_cvt_pk_bf16_f32 per pair).
__device__ __forceinline__ bf16x8_t pack8(const f32x16_t& x, int base) {
  bf16x8_t r;
#pragma unroll
  for (int i = 0; i < 8; ++i) r[i] = static_cast<__bf16>(x[base + i]);
  return r;
}

// 2^x with the hardware instruction (no denormal range handling: softmax
// weights below 2^-126 flush to zero).
__device__ __forceinline__ float exp2_hw(float x) { return __builtin_amdgcn_exp2f(x); }

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
  const int L = it.k1 - it.k0;  // keys of this item, from it.k0
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
  // Sorted copies of the rows for the dK/dV kernel (one chunk per row writes).
  const int64_t srow = static_cast<int64_t>(it.row_base) * P.n_q + r;
  if (row_ok && (it.grp < 0 || it.chunk == 0)) {
    const int64_t so = (static_cast<int64_t>(it.h) * (P.rows_total + kBwdPad) + srow) * D + g * 8;
#pragma unroll
    for (int ks = 0; ks < kKS; ++ks) {
      *reinterpret_cast<u32x4_t*>(P.qs + so + ks * 16) = qf[ks];
      *reinterpret_cast<u32x4_t*>(P.dos + so + ks * 16) = df[ks];
    }
  }
  // The row loads are complete before the ring starts, so the compiler has no
  // load of its own to wait for inside the loops.
  wait_vmcnt<0>();

  const uint32_t lds_base = lds_address(smem);
  const uint16_t* kg =
      static_cast<const uint16_t*>(P.k) + (static_cast<int64_t>(it.kv_base) + it.k0) * rs + it.h * D;
  const uint16_t* vg =
      static_cast<const uint16_t*>(P.v) + (static_cast<int64_t>(it.kv_base) + it.k0) * rs + it.h * D;
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

  // Pass 1: base-2 log-sum-exp of each row over the user's keys (skipped when
  // the forward's value is given: natural log, converted to base 2).
  float m = kNegInf, l = 0.0f;
  const bool given = P.lse_in != nullptr;
  const int ntiles1 = given ? 0 : ntiles;
  if (ntiles1 > 0) issue(0, false);
  for (int t = 0; t < ntiles1; ++t) {
    if (t + 1 < ntiles1) {
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
        for (int v = 0; v < 16; ++v) sum += exp2_hw(s[kb][v] - mn);
      sum += __shfl_xor(sum, 32);
      l = l * exp2_hw(m - mn) + sum;
      m = mn;
    }
    __syncthreads();
  }
  const float lse = given ? (row_ok && L > 0 ? P.lse_in[qrow * P.H + it.h] * 1.4426950408889634f : 0.0f)
                          : (L > 0 ? m + log2f(l) : 0.0f);

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
    if ((t + 1) * KT > L) {
      // The item's last tile: its keys past the range hold copies of the last
      // key.  Their K rows are zeroed here, so whatever dS they get adds
      // nothing to dQ = dS K (dS is finite: P and dP come from finite rows),
      // and the products below take no per-value mask.
      uint16_t* Kw = smem + (t & 1) * 2 * TE;
      const int dead = KT - (L - t * KT);  // rows lim .. KT-1, 16 chunks of 16 bytes each
      for (int u = tid; u < dead * kCH; u += kNT)
        *reinterpret_cast<u32x4_t*>(Kw + (KT - dead) * D + u * 8) = u32x4_t{0u, 0u, 0u, 0u};
      __syncthreads();
    }
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
          const float p = exp2_hw(s[kb][v] * c2 - lse);
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
  if (it.grp >= 0) {
    // split: the unscaled partial against this chunk's log-sum-exp, one record per tile row
    const int64_t slot_row = (static_cast<int64_t>(it.slot0) + it.chunk) * kBwdRowsA + rloc;
    if (row_ok) {
      float* pd = P.ws_dq + slot_row * D;
#pragma unroll
      for (int db = 0; db < kDB; ++db)
#pragma unroll
        for (int q4 = 0; q4 < 4; ++q4)
          *reinterpret_cast<f32x4_t*>(pd + db * 32 + q4 * 8 + g * 4) =
              f32x4_t{dqa[db][q4 * 4 + 0], dqa[db][q4 * 4 + 1], dqa[db][q4 * 4 + 2], dqa[db][q4 * 4 + 3]};
    }
    if (g == 0) {
      const int unit = row_ok ? static_cast<int>(qrow * P.H + it.h) : -1;
      const int tag = row_ok ? static_cast<int>(srow | (static_cast<int64_t>(it.nchunk) << 27)) : 0;
      *reinterpret_cast<f32x4_t*>(P.ws_rec + slot_row * 4) =
          f32x4_t{lse, dsum, __builtin_bit_cast(float, unit), __builtin_bit_cast(float, tag)};
    }
    return;
  }
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
      const int64_t hb = static_cast<int64_t>(it.h) * (P.rows_total + kBwdPad);
      P.lse[hb + srow] = lse;
      P.dd[hb + srow] = dsum;
      if (it.h == 0) P.qrow[srow] = static_cast<int32_t>(qrow);
    }
  }
}

// ---------------------------------------------------------------------------
// merge of split dQ partials: block (group, 8 rows); thread -> (row, 4 d)
// ---------------------------------------------------------------------------
// dQ = scale * sum_c 2^(m_c - lse) dQ_c with lse = log2 sum_c 2^(m_c) over the
// group's N chunks, in chunk order.  Straight-line over exactly N chunks: with
// the loads guarded chunk by chunk the compiler waits between them.
template <int N>
__device__ __forceinline__ f32x4_t merge_dq(const f32x4_t (&rec)[kMaxSplit], const float* ws_dq, int64_t slot0,
                                            int r, int d0, float* lse_out) {
  f32x4_t o[N];
#pragma unroll
  for (int ch = 0; ch < N; ++ch)
    o[ch] = *reinterpret_cast<const f32x4_t*>(ws_dq + ((slot0 + ch) * kBwdRowsA + r) * D + d0);
  float mx = rec[0][0];
#pragma unroll
  for (int ch = 1; ch < N; ++ch) mx = fmaxf(mx, rec[ch][0]);
  float sum = 0.0f;
#pragma unroll
  for (int ch = 0; ch < N; ++ch) sum += exp2f(rec[ch][0] - mx);
  const float lse = mx + log2f(sum);
  f32x4_t acc = f32x4_t{0, 0, 0, 0};
#pragma unroll
  for (int ch = 0; ch < N; ++ch) acc += o[ch] * exp2f(rec[ch][0] - lse);
  *lse_out = lse;
  return acc;
}

__global__ __launch_bounds__(256) void ikbo_bwd_merge_kernel(BwdParams P) {
  constexpr int TPR = D / 4;      // threads per row
  constexpr int RPB = 256 / TPR;  // rows per block
  const int r = blockIdx.y * RPB + threadIdx.x / TPR;
  const int d0 = (threadIdx.x % TPR) * 4;
  const int64_t slot0 = static_cast<int64_t>(blockIdx.x) * kMaxSplit;
  // Records of every slot of the group at once (slots past nchunk are stale and
  // ignored), then the partials of the live chunks.
  f32x4_t rec[kMaxSplit];
#pragma unroll
  for (int ch = 0; ch < kMaxSplit; ++ch)
    rec[ch] = *reinterpret_cast<const f32x4_t*>(P.ws_rec + ((slot0 + ch) * kBwdRowsA + r) * 4);
  // Fields are copied out of the vector before the bit cast (clang reads a bit
  // cast of a vector element as a cast of element 0).
  const float unit_f = rec[0][2], tag_f = rec[0][3];
  const int unit = __builtin_bit_cast(int, unit_f);
  const int tag = __builtin_bit_cast(int, tag_f);
  if (unit < 0) return;
  const int nchunk = tag >> 27;
  const int64_t srow = tag & ((1 << 27) - 1);
  float lse = 0.0f;
  f32x4_t acc;
  if (P.lse_in) {  // every chunk used the row's whole-range log-sum-exp: the partials add up
    lse = rec[0][0];
    acc = f32x4_t{0, 0, 0, 0};
    for (int ch = 0; ch < nchunk; ++ch)
      acc += *reinterpret_cast<const f32x4_t*>(P.ws_dq + ((slot0 + ch) * kBwdRowsA + r) * D + d0);
  } else switch (nchunk) {
    case 1: acc = merge_dq<1>(rec, P.ws_dq, slot0, r, d0, &lse); break;
    case 2: acc = merge_dq<2>(rec, P.ws_dq, slot0, r, d0, &lse); break;
    case 3: acc = merge_dq<3>(rec, P.ws_dq, slot0, r, d0, &lse); break;
    case 4: acc = merge_dq<4>(rec, P.ws_dq, slot0, r, d0, &lse); break;
    case 5: acc = merge_dq<5>(rec, P.ws_dq, slot0, r, d0, &lse); break;
    case 6: acc = merge_dq<6>(rec, P.ws_dq, slot0, r, d0, &lse); break;
    case 7: acc = merge_dq<7>(rec, P.ws_dq, slot0, r, d0, &lse); break;
    default: acc = merge_dq<8>(rec, P.ws_dq, slot0, r, d0, &lse); break;
  }
  acc *= P.scale;
  *reinterpret_cast<u32x2_t*>(static_cast<uint16_t*>(P.dq) + static_cast<int64_t>(unit) * D + d0) =
      pack4_bf16(acc[0], acc[1], acc[2], acc[3]);
  if (d0 == 0) {
    const int h = unit % P.H;
    const int64_t hb = static_cast<int64_t>(h) * (P.rows_total + kBwdPad);
    P.lse[hb + srow] = lse;
    P.dd[hb + srow] = rec[0][1];
    if (h == 0) P.qrow[srow] = unit / P.H;
  }
}

// ---------------------------------------------------------------------------
// dK / dV kernel
// ---------------------------------------------------------------------------
// Lane constants of the tile read offsets (elements), from which each read's
// offset takes one XOR and one shift-add.  Row reads (16 bytes of row
// kb*32 + n, chunk 2 ks + g): the swizzle only sees the row's low four bits,
// and (2 ks + g) ^ swz(n) = 2 ks ^ t with t = g ^ swz(n).  Transposed reads
// (tr_rows at K0 = R16 + 4 g, a multiple of 16 plus the lane's 4 g, and
// D0 = 32 db + 16 half): the lane's rows are R16 + r and R16 + r + 8 with
// r = 4 g + kq / 4 < 8, its chunk is 4 db + c with c = 2 half + (kq % 4) / 2 < 4,
// so chunk ^ swz(row) = 4 db ^ (c ^ swz(row)).  Sixteen per-lane offsets
// otherwise stay live across the tile loop and push the kernel past the
// register file (the spill reloads then wait on every ring copy in flight).
struct LaneOffs {
  int nb;        // n * 128
  int t;         // g ^ swz(n)
  int rb;        // r * 128 + 4 (kq % 2)
  int ta, tb;    // c ^ swz(r), c ^ swz(r + 8)
  __device__ __forceinline__ LaneOffs(int n, int g, int kq, int half) {
    const int r = 4 * g + (kq >> 2), c = 2 * half + ((kq & 3) >> 1);
    nb = n * kCH * 8;
    t = g ^ swz(n);
    rb = r * kCH * 8 + 4 * (kq & 1);
    ta = c ^ swz(r);
    tb = c ^ swz(r + 8);
  }
  // Fresh copies the compiler cannot hoist out of a loop: the offsets built
  // from them are recomputed where they are used instead of held.
  __device__ __forceinline__ LaneOffs opaque() const {
    LaneOffs o = *this;
    asm volatile("" : "+v"(o.nb), "+v"(o.t), "+v"(o.rb), "+v"(o.ta), "+v"(o.tb));
    return o;
  }
  // t_off(kb * 32 + n, 2 ks + g)
  __device__ __forceinline__ int row(int kb, int ks) const { return kb * 32 * kCH * 8 + nb + (((2 * ks) ^ t) << 3); }
  // tr_rows(T, R16 + 4 g, 32 db + 16 half, kq) as two offsets
  __device__ __forceinline__ int tr_lo(int r16, int db) const { return r16 * kCH * 8 + rb + (((4 * db) ^ ta) << 3); }
  __device__ __forceinline__ int tr_hi(int r16, int db) const {
    return (r16 + 8) * kCH * 8 + rb + (((4 * db) ^ tb) << 3);
  }
};

__device__ __forceinline__ bf16x8_t tr_rows_at(const uint16_t* T, int lo_off, int hi_off) {
  const i16x4_t lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4_t*)(T + lo_off));
  const i16x4_t hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4_t*)(T + hi_off));
  return __builtin_bit_cast(bf16x8_t, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
}

// Eight waves in two roles over the same 128 keys and the same staged rows:
// waves 0-3 form S and P and accumulate dV, waves 4-7 form dP meanwhile, take
// P of the same keys through LDS, form dS and accumulate dK (64 MFMAs per tile
// and SIMD, S formed once).  Waves w and w+4 share a SIMD, so each SIMD holds
// one wave of each role and the softmax work of one overlaps the products of
// the other; each role fits two waves per SIMD.
constexpr int kNT8 = 512;
__global__ __launch_bounds__(kNT8, 1) void ikbo_bwd_dkv_kernel(BwdParams P) {
  constexpr int RT = kBwdRowsB;          // rows per tile
  constexpr int TE = RT * D;             // elements per Q or dO tile
  constexpr int LPT = RT * kCH / kNT8;   // copies per thread per tile and tensor
  constexpr int NST = 3;                 // ring stages: two tiles in flight while one is used
  constexpr int META = 4 * RT * 4;       // bytes per stage: lse[RT], dd[RT], then 512 spare bytes (alignment)
  constexpr int STAGE = 2 * TE * 2 + META;
  constexpr int L0 = 2 * LPT;            // copies per stage of waves 1-7; wave 0 adds two
  static_assert(LPT * kNT8 == RT * kCH && RT == 64 && META >= 2 * RT * 4, "tile shape; lse and D of the tile's rows");
  __shared__ __attribute__((aligned(16))) uint8_t smem[NST * STAGE];
  // P of the current tile, [key block][row block][value quad][lane]: written by
  // the dV wave of each 32-key block, read by the dK wave of the same keys in
  // the same lane layout.
  __shared__ f32x4_t pshare[4 * 2 * 4 * 64];

  const WorkItem it = P.items[blockIdx.x];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int n = lane & 31, g = lane >> 5, kq = lane & 15, half = (lane >> 4) & 1;
  const int wave_u = __builtin_amdgcn_readfirstlane(wave);
  const bool dk_role = wave_u >= 4;       // wave-uniform
  const int kw = wave & 3;                // this wave's 32 keys
  const int64_t rs = static_cast<int64_t>(P.H) * D;
  const int nrows = it.nrows;
  const int ntiles = (nrows + RT - 1) / RT;
  const int64_t hrow0 = static_cast<int64_t>(it.h) * (P.rows_total + kBwdPad) + static_cast<int64_t>(it.row_base) * P.n_q;
  const int key = it.k0 + kw * 32 + n;
  const bool key_ok = key < it.k1;
  const bool wave_live = it.k0 + kw * 32 < it.k1;
  const int64_t koff = (static_cast<int64_t>(it.kv_base) + key) * rs + static_cast<int64_t>(it.h) * D;

  // This lane's key row of K (dV role, for S) or of V (dK role, for dP) as B operands.
  u32x4_t kf[kKS], vf[kKS];
#pragma unroll
  for (int ks = 0; ks < kKS; ++ks) {
    kf[ks] = key_ok && !dk_role ? ld16(static_cast<const uint16_t*>(P.k) + koff + ks * 16 + g * 8)
                                : u32x4_t{0u, 0u, 0u, 0u};
    vf[ks] = key_ok && dk_role ? ld16(static_cast<const uint16_t*>(P.v) + koff + ks * 16 + g * 8)
                               : u32x4_t{0u, 0u, 0u, 0u};
  }
  wait_vmcnt<0>();

  const uint32_t lds_base = lds_address(smem);
  // Stage t: rows t*RT .. t*RT + RT-1 of the user's sorted Q and dO (contiguous;
  // rows past the user's count belong to the next user or to the zeroed
  // padding), then one copy by wave 0 of those rows' log-sum-exp and D.
  // Copies from a scalar base (the stage's first row) plus per-lane byte
  // offsets, fixed per thread: no per-lane 64-bit address is held across the
  // loop.
  uint32_t ld_off[LPT];
#pragma unroll
  for (int c = 0; c < LPT; ++c) {
    const int u = tid + kNT8 * c;
    const int row = u / kCH, pos = u % kCH;
    ld_off[c] = static_cast<uint32_t>((row * D + (pos ^ swz(row)) * 8) * 2);
  }
  auto issue = [&](int t) {
    const uint32_t st = lds_base + static_cast<uint32_t>((t % NST) * STAGE);
    const int64_t r0 = hrow0 + static_cast<int64_t>(t) * RT;
    const uint16_t* qb = P.qs + r0 * D;
    const uint16_t* db = P.dos + r0 * D;
#pragma unroll
    for (int c = 0; c < LPT; ++c) {
      const uint32_t dst = st + static_cast<uint32_t>((kNT8 * c + 64 * wave_u) * 16);
      copy16_to_lds_s(qb, ld_off[c], dst);
      copy16_to_lds_s(db, ld_off[c], dst + TE * 2);
    }
    if (wave_u == 0) {
      // the tile rows' log-sum-exp and D, 4 bytes per lane each
      copy4_to_lds_s(P.lse + r0, static_cast<uint32_t>(4 * lane), st + 2 * TE * 2);
      copy4_to_lds_s(P.dd + r0, static_cast<uint32_t>(4 * lane), st + 2 * TE * 2 + RT * 4);
    }
  };
  // Waits until stage t has landed: `ahead` later stages may stay in flight.
  auto wait_stage = [&](int ahead) {
    if (wave_u == 0) {
      if (ahead >= 1) wait_vmcnt<L0 + 2>();
      else wait_vmcnt<0>();
    } else {
      if (ahead >= 1) wait_vmcnt<L0>();
      else wait_vmcnt<0>();
    }
  };
  static_assert(NST == 3, "wait_stage covers one stage in flight behind the awaited one");

  const LaneOffs lane_offs(n, g, kq, half);
  f32x16_t acc[kDB];  // dV^T (waves 0-3) or dK^T (waves 4-7)
#pragma unroll
  for (int db = 0; db < kDB; ++db) acc[db] = f32x16_t{};
  const float c2 = P.scale_log2;
  for (int t = 0; t < min(ntiles, NST - 1); ++t) issue(t);
  // One copy of the tile loop per role (the role is fixed per wave), so that
  // each loop keeps its accumulators in registers of its own: a loop shared
  // by both roles had the register allocator copy all 64 accumulator values
  // at the end of every dK tile to match the dV branch's registers.
  auto tiles = [&](auto role) {
  constexpr bool DK = decltype(role)::value;
  for (int t = 0; t < ntiles; ++t) {
    wait_stage(min(ntiles - 1 - t, NST - 2));
    __syncthreads();  // tile t is in LDS; every wave is done with tile t-1's slot
    if (t + NST - 1 < ntiles) issue(t + NST - 1);
    uint8_t* slot = smem + (t % NST) * STAGE;
    if ((t + 1) * RT > nrows) {
      // The user's last tile: its rows past the count belong to the next user
      // or to the padding.  Their staged log-sum-exp becomes +inf, so their
      // weight exp2(s c - lse) is exactly 0 (s c is finite) and so is
      // dS = P (dP - D): the products below take no per-value mask.
      if (tid < RT && tid >= nrows - t * RT) reinterpret_cast<float*>(slot + 2 * TE * 2)[tid] = __builtin_huge_valf();
      __syncthreads();
    }
    const LaneOffs lo = lane_offs.opaque();
    const uint16_t* Qt = reinterpret_cast<const uint16_t*>(slot);
    const uint16_t* Dt = Qt + TE;
    const float* lse_t = reinterpret_cast<const float*>(slot + 2 * TE * 2);
    const float* dd_t = lse_t + RT;
    // dV waves: S, then P (also handed to the dK wave of the same keys through
    // LDS); dK waves: dP, formed meanwhile.
    f32x16_t x[2];
    if (wave_live) {
      if constexpr (DK) {
#pragma unroll
        for (int rb = 0; rb < 2; ++rb) {
          x[rb] = f32x16_t{};
#pragma unroll
          for (int ks = 0; ks < kKS; ++ks)
            x[rb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(ld16(Dt + lo.row(rb, ks))), as_bf16x8(vf[ks]),
                                                            x[rb], 0, 0, 0);
        }
      } else {
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) {
          x[kb] = f32x16_t{};
#pragma unroll
          for (int ks = 0; ks < kKS; ++ks)
            x[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(ld16(Qt + lo.row(kb, ks))), as_bf16x8(kf[ks]),
                                                            x[kb], 0, 0, 0);
        }
#pragma unroll
        for (int rb = 0; rb < 2; ++rb)
#pragma unroll
          for (int q4 = 0; q4 < 4; ++q4) {
            const int rbase = rb * 32 + q4 * 8 + g * 4;
            const f32x4_t l4 = *reinterpret_cast<const f32x4_t*>(lse_t + rbase);
#pragma unroll
            for (int i = 0; i < 4; ++i) x[rb][q4 * 4 + i] = exp2_hw(x[rb][q4 * 4 + i] * c2 - l4[i]);  // P
            pshare[((kw * 2 + rb) * 4 + q4) * 64 + lane] =
                f32x4_t{x[rb][q4 * 4 + 0], x[rb][q4 * 4 + 1], x[rb][q4 * 4 + 2], x[rb][q4 * 4 + 3]};
          }
      }
    }
    __syncthreads();  // every live key block's P is in LDS
    if (wave_live) {
      if constexpr (DK) {
#pragma unroll
        for (int rb = 0; rb < 2; ++rb) {
#pragma unroll
          for (int q4 = 0; q4 < 4; ++q4) {
            const int rbase = rb * 32 + q4 * 8 + g * 4;
            const f32x4_t d4 = *reinterpret_cast<const f32x4_t*>(dd_t + rbase);
            const f32x4_t p4 = pshare[((kw * 2 + rb) * 4 + q4) * 64 + lane];
#pragma unroll
            for (int i = 0; i < 4; ++i) x[rb][q4 * 4 + i] = p4[i] * (x[rb][q4 * 4 + i] - d4[i]);  // dS
          }
#pragma unroll
          for (int j0 = 0; j0 < 2; ++j0) {
            const bf16x8_t bs = pack8(x[rb], j0 * 8);
            const int r16 = rb * 32 + j0 * 16;
#pragma unroll
            for (int db = 0; db < kDB; ++db)
              acc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(tr_rows_at(Qt, lo.tr_lo(r16, db), lo.tr_hi(r16, db)),
                                                                bs, acc[db], 0, 0, 0);
          }
        }
      } else {
#pragma unroll
        for (int rb = 0; rb < 2; ++rb)
#pragma unroll
          for (int j0 = 0; j0 < 2; ++j0) {
            const bf16x8_t bp = pack8(x[rb], j0 * 8);
            const int r16 = rb * 32 + j0 * 16;
#pragma unroll
            for (int db = 0; db < kDB; ++db)
              acc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(tr_rows_at(Dt, lo.tr_lo(r16, db), lo.tr_hi(r16, db)),
                                                                bp, acc[db], 0, 0, 0);
          }
      }
    }
  }
  };
  if (dk_role)
    tiles(std::true_type{});
  else
    tiles(std::false_type{});

  // dK^T / dV^T block db: lane value v is d = db*32 + (v/4)*8 + 4*g + v%4 of key n.
  if (key_ok) {
    uint16_t* dst = static_cast<uint16_t*>(dk_role ? P.dk : P.dv) + koff;
    const float f = dk_role ? P.scale : 1.0f;
#pragma unroll
    for (int db = 0; db < kDB; ++db)
#pragma unroll
      for (int q4 = 0; q4 < 4; ++q4)
        *reinterpret_cast<u32x2_t*>(dst + db * 32 + q4 * 8 + g * 4) =
            pack4_bf16(f * acc[db][q4 * 4 + 0], f * acc[db][q4 * 4 + 1], f * acc[db][q4 * 4 + 2],
                       f * acc[db][q4 * 4 + 3]);
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

hipError_t launch_bwd_merge(const BwdParams& p, int n_groups, hipStream_t stream, hipEvent_t ev_stop) {
  if (n_groups <= 0) return hipSuccess;
  const dim3 grid(static_cast<unsigned>(n_groups), kBwdRowsA / (256 / (D / 4)));
  if (ev_stop)
    hipExtLaunchKernelGGL(ikbo_bwd_merge_kernel, grid, dim3(256), 0, stream, nullptr, ev_stop, 0, p);
  else
    hipLaunchKernelGGL(ikbo_bwd_merge_kernel, grid, dim3(256), 0, stream, p);
  return hipGetLastError();
}

hipError_t launch_bwd_dkv(const BwdParams& p, int n_items, hipStream_t stream, hipEvent_t* ev) {
  if (n_items <= 0) return hipSuccess;
  if (ev)
    hipExtLaunchKernelGGL(ikbo_bwd_dkv_kernel, dim3(n_items), dim3(kNT8), 0, stream, ev[0], ev[1], 0, p);
  else
    hipLaunchKernelGGL(ikbo_bwd_dkv_kernel, dim3(n_items), dim3(kNT8), 0, stream, p);
  return hipGetLastError();
}

}  // namespace ikbo
