// IKBO target attention kernels for gfx950 (MI355X, CDNA4).
//
// What is computed (IKBO blog, section 3.1, Fig. 10 right): every candidate
// row attends over the K/V of the user the mapping names; the user's K/V is
// read from its packed location and never copied per candidate.  Rows of one
// user are grouped on the host into tiles; a workgroup streams the user's K/V
// once per tile through LDS and every row of the tile reuses each K/V tile.
//
// bf16 kernel, one workgroup = 4 wave64s = 128 rows (32 rows per wave):
//   * S^T = K . Q^T with v_mfma_f32_32x32x16_bf16.  Keys are the MFMA M
//     dimension and query rows the N dimension, so each lane owns one query
//     row: the row max and row sum of the online softmax reduce inside the
//     lane plus one exchange with the lane 32 apart.
//   * O^T = V^T . P^T with the same instruction: P^T is the lane's own
//     probabilities (no re-layout), V^T comes from a transposed LDS copy.
//   * K rows enter the A operand in an order that swaps bits 2 and 3 of the
//     row index; then the 8 probabilities a lane feeds to one PV step belong
//     to 8 consecutive keys, and the V^T operand is one 16-byte LDS read.
//   * Online softmax (AI-infra guide, section 4.6.1): running max m, running
//     sum l, O rescaled by exp2(m_old - m_new); scores carry the log2(e)
//     factor so exp2 is used.  Only the last, partial K/V tile and tiles on
//     the causal diagonal run the masked variant (loop peeling, TLX jagged
//     attention post, "loop peeling").
//   * Keys past the user's end are zero-filled in LDS, never loaded.
//   * Persistent launch: items arrive longest-first; logical workgroup w
//     takes the items of a boustrophedon deal.  Logical ids are mapped so that
//     neighbouring ids run on one XCD (workgroups are dealt to the 8 XCDs
//     round-robin), keeping row tiles of one (user, head) on one L2.
//   * Split key ranges write unnormalised partials (O, m, l); the last
//     workgroup of a group to arrive merges all chunks in chunk order
//     (log-sum-exp merge, AI-infra guide section 4.6.4), so the result does
//     not depend on arrival order.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cstdint>

#include "ikbo_kernels.h"

namespace ikbo {
namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));

constexpr int kBM = kBf16TileRows;  // rows per workgroup
constexpr int kBN = kBf16TileKeys;  // keys per K/V tile
constexpr int kThreads = 256;       // 4 wave64
constexpr float kNegInf = -__builtin_inff();

template <int D>
struct Smem {
  static constexpr int kStride = D + 8;    // K tile row stride, bf16 elements (pad: bank spread)
  static constexpr int vStride = kBN + 8;  // V^T tile row stride
  static constexpr int kElems = kBN * kStride;
  static constexpr int vElems = D * vStride;
  static constexpr int stage = kElems + vElems;
};

__device__ __forceinline__ bf16x8_t as_bf16x8(u32x4_t x) { return __builtin_bit_cast(bf16x8_t, x); }

__device__ __forceinline__ uint32_t bf16_bits(float f) {
  return static_cast<uint32_t>(__builtin_bit_cast(uint16_t, static_cast<__bf16>(f)));
}

__device__ __forceinline__ u32x2_t pack4_bf16(float a, float b, float c, float d) {
  u32x2_t r;
  r.x = bf16_bits(a) | (bf16_bits(b) << 16);
  r.y = bf16_bits(c) | (bf16_bits(d) << 16);
  return r;
}

// Row of the A operand that carries key `m` of a 32-key block: bits 2 and 3 swapped.
__device__ __forceinline__ int swap_bits23(int m) {
  return (m & ~12) | ((m & 4) << 1) | ((m & 8) >> 1);
}

__device__ __forceinline__ float exp2_fast(float x) { return __builtin_amdgcn_exp2f(x); }

// Item position of logical workgroup w in a given pass of the boustrophedon
// deal (same rule as ikbo::zigzag_position on the host).
__device__ __forceinline__ int64_t deal_position(int64_t pass, int w, int grid) {
  return pass * grid + ((pass & 1) ? (grid - 1 - w) : w);
}

// Logical workgroup id: ids w and w+1 share an XCD when the grid is a multiple of 8.
__device__ __forceinline__ int logical_wg() {
  const int G = gridDim.x, b = blockIdx.x;
  return (G & 7) ? b : (b & 7) * (G >> 3) + (b >> 3);
}

// ---------------------------------------------------------------------------
// bf16 MFMA kernel
// ---------------------------------------------------------------------------

// One K/V tile for one wave: S^T, online softmax update, O^T += V^T P^T.
template <int D, bool MASK>
__device__ __forceinline__ void tile_step(const uint16_t* __restrict__ Ks,
                                          const uint16_t* __restrict__ Vt,
                                          const u32x4_t (&qf)[D / 16], f32x16_t (&oacc)[D / 32],
                                          float& m_run, float& l_run, int key_base, int key_end,
                                          bool causal, int row_tok, float c, int n, int g) {
  using S = Smem<D>;
  f32x16_t s[2];
#pragma unroll
  for (int b = 0; b < 2; ++b) {
    s[b] = f32x16_t{};
    const uint16_t* kr = Ks + (b * 32 + swap_bits23(n)) * S::kStride + g * 8;
#pragma unroll
    for (int st = 0; st < D / 16; ++st) {
      const u32x4_t a = *reinterpret_cast<const u32x4_t*>(kr + st * 16);
      s[b] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(a), as_bf16x8(qf[st]), s[b], 0, 0, 0);
    }
  }
  // Lane value i of block b holds key  b*32 + (i/8)*16 + g*8 + i%8  of row n.
  float mx = kNegInf;
#pragma unroll
  for (int b = 0; b < 2; ++b) {
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      float x = s[b][i] * c;
      if (MASK) {
        const int key = key_base + b * 32 + (i >> 3) * 16 + g * 8 + (i & 7);
        const bool ok = key < key_end && (!causal || key <= row_tok);
        x = ok ? x : kNegInf;
      }
      s[b][i] = x;
      mx = fmaxf(mx, x);
    }
  }
  mx = fmaxf(mx, __shfl_xor(mx, 32));
  const float m_new = fmaxf(m_run, mx);
  const float m_use = (m_new == kNegInf) ? 0.0f : m_new;  // a row with no live key yet
  const float alpha = exp2_fast(m_run - m_use);
  float rs = 0.0f;
#pragma unroll
  for (int b = 0; b < 2; ++b) {
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const float p = exp2_fast(s[b][i] - m_use);
      s[b][i] = p;
      rs += p;
    }
  }
  rs += __shfl_xor(rs, 32);
  l_run = l_run * alpha + rs;
  m_run = m_new;
#pragma unroll
  for (int mb = 0; mb < D / 32; ++mb) oacc[mb] *= alpha;

  bf16x8_t pb[2][2];
#pragma unroll
  for (int b = 0; b < 2; ++b)
#pragma unroll
    for (int s2 = 0; s2 < 2; ++s2)
#pragma unroll
      for (int j = 0; j < 8; ++j) pb[b][s2][j] = static_cast<__bf16>(s[b][s2 * 8 + j]);

#pragma unroll
  for (int mb = 0; mb < D / 32; ++mb) {
    const uint16_t* vr = Vt + (mb * 32 + n) * S::vStride + g * 8;
#pragma unroll
    for (int b = 0; b < 2; ++b) {
#pragma unroll
      for (int s2 = 0; s2 < 2; ++s2) {
        const u32x4_t a = *reinterpret_cast<const u32x4_t*>(vr + b * 32 + s2 * 16);
        oacc[mb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(a), pb[b][s2], oacc[mb], 0, 0, 0);
      }
    }
  }
}

template <int D>
__global__ __launch_bounds__(kThreads, 2) void ikbo_attn_bf16_kernel(AttnParams P) {
  using S = Smem<D>;
  __shared__ __attribute__((aligned(16))) uint16_t smem[2 * S::stage];
  __shared__ int s_last;

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int n = lane & 31, g = lane >> 5;
  const int r_w = wave * 32 + n;  // this lane's row within the tile

  // Loader mapping: thread -> (16-byte column chunk, group of KPT consecutive keys).
  constexpr int CH = D / 8;
  constexpr int KPT = kBN * CH / kThreads;
  static_assert(KPT >= 1 && KPT <= 4 && kBN * CH == KPT * kThreads, "loader shape");
  const int lc = tid % CH, lq = tid / CH;

  const uint16_t* __restrict__ Kg = static_cast<const uint16_t*>(P.k);
  const uint16_t* __restrict__ Vg = static_cast<const uint16_t*>(P.v);
  const int64_t row_stride = static_cast<int64_t>(P.H) * D;  // elements between consecutive tokens

  const int G = gridDim.x;
  const int w = logical_wg();
  for (int64_t pass = 0;; ++pass) {
    const int64_t pos = deal_position(pass, w, G);
    if (pos >= P.n_items) break;
    const WorkItem it = P.items[pos];
    const bool causal = it.kind == kKindSelf;

    // ---- query fragment (B operand of S^T): row r_w, 16 bytes per MFMA K-step
    int64_t qrow = -1;
    if (r_w < it.nrows) {
      const int r = it.row0 + r_w;
      if (!causal) {
        const int cand = P.cand_perm[it.row_base + r / P.n_q];
        qrow = static_cast<int64_t>(cand) * P.n_q + r % P.n_q;
      } else {
        qrow = static_cast<int64_t>(it.row_base) + r;
      }
    }
    u32x4_t qf[D / 16];
    {
      const uint16_t* qb = static_cast<const uint16_t*>(causal ? P.q_user : P.q_cand);
      const uint16_t* qp = qb + (qrow < 0 ? 0 : (qrow * P.H + it.h) * D) + g * 8;
#pragma unroll
      for (int st = 0; st < D / 16; ++st)
        qf[st] = (qrow < 0) ? u32x4_t{0, 0, 0, 0} : *reinterpret_cast<const u32x4_t*>(qp + st * 16);
    }

    f32x16_t oacc[D / 32];
#pragma unroll
    for (int mb = 0; mb < D / 32; ++mb) oacc[mb] = f32x16_t{};
    float m_run = kNegInf, l_run = 0.0f;

    const int nkv = it.k1 - it.k0;
    const int ntiles = (nkv + kBN - 1) / kBN;
    const uint16_t* kbase = Kg + (static_cast<int64_t>(it.kv_base) + it.k0) * row_stride + it.h * D + lc * 8;
    const uint16_t* vbase = Vg + (static_cast<int64_t>(it.kv_base) + it.k0) * row_stride + it.h * D + lc * 8;
    u32x4_t kreg[KPT], vreg[KPT];

    auto gload = [&](int t) {
#pragma unroll
      for (int i = 0; i < KPT; ++i) {
        const int key = t * kBN + lq * KPT + i;  // relative to k0
        if (key < nkv) {
          kreg[i] = *reinterpret_cast<const u32x4_t*>(kbase + key * row_stride);
          vreg[i] = *reinterpret_cast<const u32x4_t*>(vbase + key * row_stride);
        } else {
          kreg[i] = u32x4_t{0, 0, 0, 0};
          vreg[i] = u32x4_t{0, 0, 0, 0};
        }
      }
    };
    auto lstore = [&](int buf) {
      uint16_t* Ks = smem + buf * S::stage;
      uint16_t* Vt = Ks + S::kElems;
#pragma unroll
      for (int i = 0; i < KPT; ++i)
        *reinterpret_cast<u32x4_t*>(Ks + (lq * KPT + i) * S::kStride + lc * 8) = kreg[i];
      // Transposed V: column element e of the chunk becomes row lc*8+e; the KPT keys are contiguous.
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        uint32_t h16[KPT];
#pragma unroll
        for (int i = 0; i < KPT; ++i) h16[i] = (vreg[i][e >> 1] >> ((e & 1) * 16)) & 0xffffu;
        uint16_t* dst = Vt + (lc * 8 + e) * S::vStride + lq * KPT;
        if constexpr (KPT == 4) {
          *reinterpret_cast<u32x2_t*>(dst) = u32x2_t{h16[0] | (h16[1] << 16), h16[2] | (h16[3] << 16)};
        } else if constexpr (KPT == 2) {
          *reinterpret_cast<uint32_t*>(dst) = h16[0] | (h16[1] << 16);
        } else {
          *dst = static_cast<uint16_t>(h16[0]);
        }
      }
    };

    const bool wave_has_rows = wave * 32 < it.nrows;
    const int row_tok = it.row0 + r_w;                   // token index (self rows)
    const int wave_last_tok = it.row0 + wave * 32 + 31;  // largest token of this wave's rows
    const float c = P.scale_log2;

    if (ntiles > 0) {
      gload(0);
      lstore(0);
    }
    __syncthreads();
    for (int t = 0; t < ntiles; ++t) {
      if (t + 1 < ntiles) gload(t + 1);
      const int key_base = it.k0 + t * kBN;  // first key of this tile, user-relative
      const bool skip = !wave_has_rows || (causal && key_base > wave_last_tok);
      if (!skip) {
        const uint16_t* Ks = smem + (t & 1) * S::stage;
        const uint16_t* Vt = Ks + S::kElems;
        const bool need_mask = (key_base + kBN > it.k1) || (causal && key_base + kBN - 1 > it.row0 + wave * 32);
        if (need_mask)
          tile_step<D, true>(Ks, Vt, qf, oacc, m_run, l_run, key_base, it.k1, causal, row_tok, c, n, g);
        else
          tile_step<D, false>(Ks, Vt, qf, oacc, m_run, l_run, key_base, it.k1, causal, row_tok, c, n, g);
      }
      if (t + 1 < ntiles) lstore((t + 1) & 1);
      __syncthreads();
    }

    // ---- epilogue
    // Lane holds O^T rows d = mb*32 + (i/4)*8 + g*4 + i%4 of query row r_w.
    if (it.grp < 0) {
      if (qrow >= 0) {
        uint16_t* ob = static_cast<uint16_t*>(causal ? P.out_user : P.out_cand);
        uint16_t* op = ob + (qrow * P.H + it.h) * D + g * 4;
        const float inv = l_run > 0.0f ? 1.0f / l_run : 0.0f;
#pragma unroll
        for (int mb = 0; mb < D / 32; ++mb)
#pragma unroll
          for (int i4 = 0; i4 < 4; ++i4)
            *reinterpret_cast<u32x2_t*>(op + mb * 32 + i4 * 8) =
                pack4_bf16(oacc[mb][i4 * 4 + 0] * inv, oacc[mb][i4 * 4 + 1] * inv,
                           oacc[mb][i4 * 4 + 2] * inv, oacc[mb][i4 * 4 + 3] * inv);
      }
    } else {
      const int64_t slot = static_cast<int64_t>(it.slot0) + it.chunk;
      if (r_w < it.nrows) {
        float* wo = P.ws_o + (slot * kBM + r_w) * D + g * 4;
#pragma unroll
        for (int mb = 0; mb < D / 32; ++mb)
#pragma unroll
          for (int i4 = 0; i4 < 4; ++i4)
            *reinterpret_cast<f32x4_t*>(wo + mb * 32 + i4 * 8) =
                f32x4_t{oacc[mb][i4 * 4 + 0], oacc[mb][i4 * 4 + 1], oacc[mb][i4 * 4 + 2], oacc[mb][i4 * 4 + 3]};
        if (g == 0) {
          P.ws_ml[(slot * kBM + r_w) * 2 + 0] = m_run;
          P.ws_ml[(slot * kBM + r_w) * 2 + 1] = l_run;
        }
      }
      __threadfence();  // release this workgroup's partials device-wide
      __syncthreads();
      if (tid == 0) {
        const int prev = atomicAdd(P.counters + it.grp, 1);
        const int last = prev == it.nchunk - 1;
        if (last) atomicExch(P.counters + it.grp, 0);  // ready for the next launch
        s_last = last;
      }
      __syncthreads();
      if (s_last) {
        __threadfence();  // acquire the other chunks' partials
        const int64_t s0 = it.slot0;
        constexpr int D4 = D / 4;
        for (int idx = tid; idx < it.nrows * D4; idx += kThreads) {
          const int r = idx / D4, d4 = idx % D4;
          float mmax = kNegInf;
          for (int ch = 0; ch < it.nchunk; ++ch) mmax = fmaxf(mmax, P.ws_ml[((s0 + ch) * kBM + r) * 2]);
          const float mu = (mmax == kNegInf) ? 0.0f : mmax;
          float lsum = 0.0f;
          f32x4_t acc = f32x4_t{0, 0, 0, 0};
          for (int ch = 0; ch < it.nchunk; ++ch) {
            const float wgt = exp2_fast(P.ws_ml[((s0 + ch) * kBM + r) * 2] - mu);
            lsum += wgt * P.ws_ml[((s0 + ch) * kBM + r) * 2 + 1];
            const f32x4_t o = *reinterpret_cast<const f32x4_t*>(P.ws_o + ((s0 + ch) * kBM + r) * D + d4 * 4);
            acc += wgt * o;
          }
          const float inv = lsum > 0.0f ? 1.0f / lsum : 0.0f;
          const int rr = it.row0 + r;
          int64_t orow;
          if (!causal) {
            const int cand = P.cand_perm[it.row_base + rr / P.n_q];
            orow = static_cast<int64_t>(cand) * P.n_q + rr % P.n_q;
          } else {
            orow = static_cast<int64_t>(it.row_base) + rr;
          }
          uint16_t* ob = static_cast<uint16_t*>(causal ? P.out_user : P.out_cand);
          *reinterpret_cast<u32x2_t*>(ob + (orow * P.H + it.h) * D + d4 * 4) =
              pack4_bf16(acc[0] * inv, acc[1] * inv, acc[2] * inv, acc[3] * inv);
        }
      }
      __syncthreads();
    }
  }
}

// ---------------------------------------------------------------------------
// fp32 kernel: one thread per row, K/V tiles broadcast from LDS, VALU math.
// ---------------------------------------------------------------------------

template <int D>
__global__ __launch_bounds__(64) void ikbo_attn_f32_kernel(AttnParams P) {
  constexpr int TK = kF32TileKeys;
  __shared__ __attribute__((aligned(16))) float Ks[TK][D];
  __shared__ __attribute__((aligned(16))) float Vs[TK][D];
  const float* __restrict__ Kg = static_cast<const float*>(P.k);
  const float* __restrict__ Vg = static_cast<const float*>(P.v);
  const int t = threadIdx.x;
  const int64_t row_stride = static_cast<int64_t>(P.H) * D;
  const float c = P.scale_log2;

  for (int64_t pos = blockIdx.x; pos < P.n_items; pos += gridDim.x) {
    const WorkItem it = P.items[pos];
    const bool causal = it.kind == kKindSelf;
    int64_t qrow = -1;
    if (t < it.nrows) {
      const int r = it.row0 + t;
      if (!causal) {
        const int cand = P.cand_perm[it.row_base + r / P.n_q];
        qrow = static_cast<int64_t>(cand) * P.n_q + r % P.n_q;
      } else {
        qrow = static_cast<int64_t>(it.row_base) + r;
      }
    }
    float q[D], o[D];
    {
      const float* qb = static_cast<const float*>(causal ? P.q_user : P.q_cand);
#pragma unroll
      for (int e = 0; e < D; ++e) {
        q[e] = qrow < 0 ? 0.0f : qb[(qrow * P.H + it.h) * D + e];
        o[e] = 0.0f;
      }
    }
    float m_run = kNegInf, l_run = 0.0f;
    const int row_tok = it.row0 + t;
    const int nkv = it.k1 - it.k0;
    const float* kb = Kg + (static_cast<int64_t>(it.kv_base) + it.k0) * row_stride + it.h * D;
    const float* vb = Vg + (static_cast<int64_t>(it.kv_base) + it.k0) * row_stride + it.h * D;
    for (int kt = 0; kt < nkv; kt += TK) {
      __syncthreads();
      for (int idx = t; idx < TK * (D / 4); idx += 64) {
        const int key = idx / (D / 4), c4 = idx % (D / 4);
        f32x4_t kv = f32x4_t{0, 0, 0, 0}, vv = f32x4_t{0, 0, 0, 0};
        if (kt + key < nkv) {
          kv = *reinterpret_cast<const f32x4_t*>(kb + (kt + key) * row_stride + c4 * 4);
          vv = *reinterpret_cast<const f32x4_t*>(vb + (kt + key) * row_stride + c4 * 4);
        }
        *reinterpret_cast<f32x4_t*>(&Ks[key][c4 * 4]) = kv;
        *reinterpret_cast<f32x4_t*>(&Vs[key][c4 * 4]) = vv;
      }
      __syncthreads();
      float s[TK];
      float mx = kNegInf;
#pragma unroll
      for (int j = 0; j < TK; ++j) {
        float acc = 0.0f;
#pragma unroll
        for (int e = 0; e < D; ++e) acc = fmaf(q[e], Ks[j][e], acc);
        const int key = it.k0 + kt + j;
        const bool ok = (kt + j < nkv) && (!causal || key <= row_tok);
        s[j] = ok ? acc * c : kNegInf;
        mx = fmaxf(mx, s[j]);
      }
      const float m_new = fmaxf(m_run, mx);
      const float m_use = (m_new == kNegInf) ? 0.0f : m_new;
      const float alpha = exp2_fast(m_run - m_use);
      float rs = 0.0f;
#pragma unroll
      for (int j = 0; j < TK; ++j) {
        s[j] = exp2_fast(s[j] - m_use);
        rs += s[j];
      }
      l_run = l_run * alpha + rs;
      m_run = m_new;
#pragma unroll
      for (int e = 0; e < D; ++e) o[e] *= alpha;
#pragma unroll
      for (int j = 0; j < TK; ++j)
#pragma unroll
        for (int e = 0; e < D; ++e) o[e] = fmaf(s[j], Vs[j][e], o[e]);
    }
    if (qrow >= 0) {
      float* ob = static_cast<float*>(causal ? P.out_user : P.out_cand);
      const float inv = l_run > 0.0f ? 1.0f / l_run : 0.0f;
#pragma unroll
      for (int e = 0; e < D; e += 4)
        *reinterpret_cast<f32x4_t*>(ob + (qrow * P.H + it.h) * D + e) =
            f32x4_t{o[e] * inv, o[e + 1] * inv, o[e + 2] * inv, o[e + 3] * inv};
    }
  }
}

// ---------------------------------------------------------------------------
// Materialised broadcast (comparator): per-candidate copies of the user K/V.
// ---------------------------------------------------------------------------

__global__ __launch_bounds__(256) void ikbo_bcast_copy_kernel(const u32x4_t* __restrict__ k,
                                                              const u32x4_t* __restrict__ v,
                                                              u32x4_t* __restrict__ kb,
                                                              u32x4_t* __restrict__ vb,
                                                              const int64_t* __restrict__ src_row,
                                                              const int64_t* __restrict__ dst_row,
                                                              const int32_t* __restrict__ len,
                                                              int64_t vecs_per_row) {
  const int cidx = blockIdx.y;
  const int64_t nvec = static_cast<int64_t>(len[cidx]) * vecs_per_row;
  const int64_t s0 = src_row[cidx] * vecs_per_row, d0 = dst_row[cidx] * vecs_per_row;
  for (int64_t i = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x; i < nvec;
       i += static_cast<int64_t>(gridDim.x) * blockDim.x) {
    kb[d0 + i] = k[s0 + i];
    vb[d0 + i] = v[s0 + i];
  }
}

}  // namespace

hipError_t launch_attn_bf16(const AttnParams& p, int d, int grid, hipStream_t stream) {
  if (grid <= 0 || p.n_items <= 0) return hipSuccess;
  switch (d) {
    case 128: hipLaunchKernelGGL(ikbo_attn_bf16_kernel<128>, dim3(grid), dim3(kThreads), 0, stream, p); break;
    case 64: hipLaunchKernelGGL(ikbo_attn_bf16_kernel<64>, dim3(grid), dim3(kThreads), 0, stream, p); break;
    case 32: hipLaunchKernelGGL(ikbo_attn_bf16_kernel<32>, dim3(grid), dim3(kThreads), 0, stream, p); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t launch_attn_f32(const AttnParams& p, int d, int grid, hipStream_t stream) {
  if (grid <= 0 || p.n_items <= 0) return hipSuccess;
  switch (d) {
    case 128: hipLaunchKernelGGL(ikbo_attn_f32_kernel<128>, dim3(grid), dim3(64), 0, stream, p); break;
    case 64: hipLaunchKernelGGL(ikbo_attn_f32_kernel<64>, dim3(grid), dim3(64), 0, stream, p); break;
    case 32: hipLaunchKernelGGL(ikbo_attn_f32_kernel<32>, dim3(grid), dim3(64), 0, stream, p); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t launch_bcast_copy(const void* k, const void* v, void* kb, void* vb, const int64_t* src_row,
                             const int64_t* dst_row, const int32_t* len, int32_t n, int64_t row_bytes,
                             int32_t max_len, hipStream_t stream) {
  if (n <= 0 || max_len <= 0) return hipSuccess;
  if (row_bytes % 16 != 0 || n > 65535) return hipErrorInvalidValue;
  const int64_t vecs = row_bytes / 16;
  const int64_t per_cand = static_cast<int64_t>(max_len) * vecs;
  const int gx = static_cast<int>(std::min<int64_t>(64, (per_cand + 255) / 256));
  hipLaunchKernelGGL(ikbo_bcast_copy_kernel, dim3(gx, n), dim3(256), 0, stream,
                     static_cast<const u32x4_t*>(k), static_cast<const u32x4_t*>(v), static_cast<u32x4_t*>(kb),
                     static_cast<u32x4_t*>(vb), src_row, dst_row, len, vecs);
  return hipGetLastError();
}

}  // namespace ikbo
