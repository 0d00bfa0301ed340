// IKBO target attention kernels for gfx950 (MI355X, CDNA4).
//
// What is computed (IKBO blog, section 3.1, Fig. 10 right): every candidate
// row attends over the K/V of the user the mapping names; the user's K/V is
// read from its packed location and never copied per candidate.  Rows of one
// user are grouped on the host into tiles; a workgroup streams the user's K/V
// once per tile through LDS and every row of the tile reuses each K/V tile.
//
// bf16 kernel, one workgroup = 4 wave64s = 128 rows (32 rows per wave):
//   * K/V tiles of 64 keys move HBM -> LDS with global_load_lds_dwordx4
//     (no register staging) through a ring of NST stages, so up to NST-1
//     tiles are in flight while one is being computed (with two stages, the
//     two-per-CU variant copies K one tile ahead of V and forms the next
//     tile's scores during the current tile's exponentials).  Each tile is stored
//     in natural [key][d] order with its 16-byte chunks XOR-swizzled per row
//     (bank-conflict-free reads).  Keys past the user's end load the user's
//     last key again (finite data) and are masked to -inf in the scores.
//   * S^T = K . Q^T with v_mfma_f32_32x32x16_bf16: keys are the MFMA M
//     dimension and query rows the N dimension, so each lane owns one query
//     row; the online-softmax row max and row sum reduce inside the lane plus
//     one exchange with the lane 32 apart.
//   * O^T = V^T . P^T with the same instruction: P^T is the lane's own
//     probabilities (no re-layout).  The V^T operand is read with
//     ds_read_b64_tr_b16, which hands each lane 4 consecutive keys of one
//     d column out of the natural-layout tile; two such reads make one
//     8-key MFMA operand whose key order matches the probabilities' order.
//   * Online softmax (AI-infra guide, section 4.6.1): running max m, running
//     sum l, O rescaled by exp2(m_old - m_new); scores carry the log2(e)
//     factor so exp2 is used.  Only the last, partial K/V tile and tiles on
//     the causal diagonal run the masked variant (loop peeling, TLX jagged
//     attention post, "loop peeling").
//   * Persistent launch: items arrive longest-first; logical workgroup w
//     takes the items of a boustrophedon deal.  Logical ids are mapped so that
//     neighbouring ids run on one XCD (workgroups are dealt to the 8 XCDs
//     round-robin), keeping row tiles of one (user, head) on one L2.
//   * Split key ranges write unnormalised partials (O, m, l); a second,
//     wide kernel merges each group's chunks in chunk order (the
//     log-sum-exp merge of the AI-infra guide, section 4.6.4), so the result
//     does not depend on the schedule and no workgroup waits on another.
#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cstdint>
#include <type_traits>

#include "ikbo_device.h"
#include "ikbo_kernels.h"

namespace ikbo {
namespace {

using namespace dev;


constexpr int kBM = kBf16TileRows;  // rows per workgroup
constexpr int kBN = kBf16TileKeys;  // keys per K/V tile
constexpr int kThreads = 256;       // 4 wave64
constexpr float kNegInf = -__builtin_inff();

// One K or V tile in LDS: kBN rows of D bf16, 16-byte chunks swizzled per row.
template <int D>
struct Tile {
  static constexpr int NCH = D / 8;                 // 16-byte chunks per row
  static constexpr int elems = kBN * D;             // one K or V tile
  static constexpr int stage = 2 * elems;           // K tile then V tile
  static constexpr int loads = kBN * NCH / kThreads;  // 16-byte loads per thread per tile
  static_assert(loads >= 1 && loads * kThreads == kBN * NCH, "tile shape");
};


template <int D>
__device__ __forceinline__ int tile_off(int row, int chunk) {
  return (row * Tile<D>::NCH + (chunk ^ (swz(row) & (Tile<D>::NCH - 1)))) * 8;
}


__device__ __forceinline__ float exp2_fast(float x) { return __builtin_amdgcn_exp2f(x); }

// Natural-log log-sum-exp of a row from its base-2 reference m and sum l
// (l = sum_j 2^(x_j - m)); -inf for a row without keys.
__device__ __forceinline__ float row_lse(float m, float l) {
  return l > 0.0f ? (m + __log2f(l)) * 0.69314718055994531f : kNegInf;
}

// Split partials of the bf16 kernels: per row and chunk, the unnormalised O in
// fp16, each half-row (d < D/2, d >= D/2) scaled by its own power of two, and
// a 16-byte row record {m, l, output unit (-1 when the tile row is empty),
// tag}.  tag = nchunk | kind << 4 | c0 << 8 | c1 << 16, where c_h is the
// biased fp32 exponent field of the half-row's largest |O|: the stored value
// is O * 2^(141 - c_h), whose largest magnitude then lies in [2^14, 2^15)
// (fp16's top binade; a half-row of zeros stores zeros), and the merge
// multiplies back by 2^(c_h - 141), exactly.  (The MXFP8 kernel's partials
// stay fp32, with tag = nchunk.)
__device__ __forceinline__ int half_code(float maxabs) {
  return static_cast<int>((__builtin_bit_cast(uint32_t, maxabs) >> 23) & 255u);
}
__device__ __forceinline__ int split_tag(const WorkItem& it, int c0, int c1) {
  return it.nchunk | (it.kind << 4) | (c0 << 8) | (c1 << 16);
}
__device__ __forceinline__ f32x4_t split_record(float m, float l, int64_t qrow, const WorkItem& it, int H, int tag) {
  const int unit = qrow < 0 ? -1 : static_cast<int>(qrow * H + it.h);
  return f32x4_t{m, l, __builtin_bit_cast(float, unit), __builtin_bit_cast(float, tag)};
}
// Four values times 2^(141 - code), rounded to fp16 (nearest even), packed.
__device__ __forceinline__ u32x2_t pack4_f16_scaled(float a, float b, float c, float d, int code) {
  typedef _Float16 f16x4_t __attribute__((ext_vector_type(4)));
  const int e = 141 - code;
  const f16x4_t v = {static_cast<_Float16>(__builtin_ldexpf(a, e)), static_cast<_Float16>(__builtin_ldexpf(b, e)),
                     static_cast<_Float16>(__builtin_ldexpf(c, e)), static_cast<_Float16>(__builtin_ldexpf(d, e))};
  return __builtin_bit_cast(u32x2_t, v);
}

// Chunk weights of one row of a split group: w_c = 2^(m_c - M) / L with
// M = max_c m_c and L = sum_c 2^(m_c - M) l_c, so that O = sum_c w_c O_c (the
// log-sum-exp merge of Flash-Decoding's split-KV partials, AI-infra guide,
// section 4.6.4).
// Contraction off: every build rounds the merge alike.
__device__ __forceinline__ void chunk_weights(const float* m, const float* l, int nchunk, float* w) {
#pragma clang fp contract(off)
  float M = kNegInf;
#pragma unroll
  for (int c = 0; c < kMaxSplit; ++c)
    if (c < nchunk) M = fmaxf(M, m[c]);
  const float mu = (M == kNegInf) ? 0.0f : M;
  float e[kMaxSplit];
  float L = 0.0f;
#pragma unroll
  for (int c = 0; c < kMaxSplit; ++c) {
    e[c] = c < nchunk ? exp2_fast(m[c] - mu) : 0.0f;
    if (c < nchunk) L = L + e[c] * l[c];
  }
  const float inv = L > 0.0f ? 1.0f / L : 0.0f;
#pragma unroll
  for (int c = 0; c < kMaxSplit; ++c) w[c] = e[c] * inv;
}

// sum_c w_c O_c over one 4-column slice, in chunk order, packed to bf16.
template <int N>
__device__ __forceinline__ u32x2_t weigh_slice(const float* w, const f32x4_t* o) {
#pragma clang fp contract(off)
  f32x4_t acc = o[0] * w[0];
#pragma unroll
  for (int c = 1; c < N; ++c) acc = acc + o[c] * w[c];
  return pack4_bf16(acc[0], acc[1], acc[2], acc[3]);
}


// {x[l], x[l ^ 32]} for every lane l, via v_permlane32_swap: with both
// operands holding x, the first comes back with the lower half's values in
// both halves and the second with the upper half's, so a symmetric op of the
// two is the pair's reduction.  Written as assembly: the compiler's model of
// the swap builtin treats its two results as equal and folds the op.  The
// s_nop pairs give the wait states around a VALU write read by the swap.  Not
// volatile: it is a pure function of x, so the scheduler may move it (and
// memory operations across it).
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"
__device__ __forceinline__ void swap_halves(float x, float& a, float& b) {
  asm("s_nop 1\n\tv_permlane32_swap_b32 %0, %1\n\ts_nop 1" : "=v"(a), "=v"(b) : "0"(x), "1"(x));
}
#pragma clang diagnostic pop
__device__ __forceinline__ float pair_max(float x) {
  float a, b;
  swap_halves(x, a, b);
  return fmaxf(a, b);
}
__device__ __forceinline__ float pair_sum(float x) {
  float a, b;
  swap_halves(x, a, b);
  return a + b;
}



// Optional per-item trace (a measurement aid): 100 MHz real-time stamps and the
// hardware placement of the workgroup.  s_getreg reads HW_ID (CU, SE) and
// XCC_ID; s_memrealtime reads the device's constant-rate clock.
__device__ __forceinline__ uint64_t now_ticks() { return __builtin_amdgcn_s_memrealtime(); }
__device__ __forceinline__ uint32_t hw_place() {
  const uint32_t hw = __builtin_amdgcn_s_getreg((31 << 11) | 4);   // HW_ID
  const uint32_t xcc = __builtin_amdgcn_s_getreg((31 << 11) | 20); // XCC_ID
  return ((xcc & 15u) << 16) | ((hw >> 8) & 0xffffu);               // xcc | se/sh/cu bits
}

// Item position of logical workgroup w in a given pass of the boustrophedon
// deal (same rule as ikbo::zigzag_position on the host).
__device__ __forceinline__ int64_t deal_position(int64_t pass, int w, int grid) {
  return pass * grid + ((pass & 1) ? (grid - 1 - w) : w);
}


// ---------------------------------------------------------------------------
// bf16 MFMA kernel
// ---------------------------------------------------------------------------

// One K/V tile for one wave in three parts: S^T = K Q^T (qk_tile), the online
// softmax update that turns S into the bf16 P^T operands (softmax_tile), and
// O^T += V^T P^T (pv_tile).  tile_step runs the three in a row.

// Per-lane LDS element offsets of the tile reads, computed once per kernel:
// koff[st] for the K fragment of K-step st of rows 0..31 (rows 32..63 add
// 32 * D), voff[2 mb + h] for the transposed V reads of O^T block mb of the
// tile's first K-step (h = 1: the read eight keys further; later K-steps add
// whole rows).
template <int D>
struct TileOffsets {
  int koff[D / 16];
  int voff[D / 16];
  __device__ __forceinline__ explicit TileOffsets(int lane) {
    const int n = lane & 31, g = lane >> 5, kq = lane & 15, half = (lane >> 4) & 1;
#pragma unroll
    for (int st = 0; st < D / 16; ++st) koff[st] = tile_off<D>(n, st * 2 + g);
#pragma unroll
    for (int mb = 0; mb < D / 32; ++mb) {
      const int col = mb * 32 + half * 16 + 4 * (kq & 3);
      const int r0 = g * 4 + (kq >> 2);
      voff[2 * mb] = tile_off<D>(r0, col >> 3) + (col & 4);
      voff[2 * mb + 1] = tile_off<D>(r0 + 8, col >> 3) + (col & 4);
    }
  }
};

// S^T of the tile's two 32-key blocks for this lane's query row.
template <int D>
__device__ __forceinline__ void qk_tile(const uint16_t* __restrict__ Ks, const u32x4_t (&qf)[D / 16],
                                        f32x16_t (&s)[2], const TileOffsets<D>& to) {
#pragma unroll
  for (int b = 0; b < 2; ++b) {
    u32x4_t a[D / 16];
#pragma unroll
    for (int st = 0; st < D / 16; ++st)
      a[st] = *reinterpret_cast<const u32x4_t*>(Ks + b * 32 * D + to.koff[st]);
    s[b] = f32x16_t{};
#pragma unroll
    for (int st = 0; st < D / 16; ++st)
      s[b] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(a[st]), as_bf16x8(qf[st]), s[b], 0, 0, 0);
  }
  // Issue order: K fragments three ahead of the MFMAs that use them (the
  // scheduler would otherwise put each read right before its MFMA and wait on
  // it, leaving the matrix cores idle for a whole LDS latency per MFMA).
  __builtin_amdgcn_sched_group_barrier(0x100, 3, 0);
#pragma unroll
  for (int k = 0; k < D / 8 - 3; ++k) {
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
    __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
  }
  __builtin_amdgcn_sched_group_barrier(0x008, 3, 0);
}

// Kernel-side softmax scale in base 2.  A zero scale is replaced by a tiny
// one: every weight is then 2^(tiny * s - tiny * max s) = 1.0f exactly, as
// with a zero scale, while masked keys (scores set to -inf or +inf, see
// mask_scores) still get weight 0 instead of 0 * inf = NaN.
__device__ __forceinline__ float kernel_scale(float scale_log2) {
  return scale_log2 != 0.0f ? scale_log2 : 1e-30f;
}

// Masks one tile's scores: lane value i of block b holds key
// key_base + g*4 + off(b, i) of query row n, off(b, i) = b*32 + (i/4)*8 + i%4;
// keys past key_end and, for causal rows, keys after the row's own token get a
// score whose scaled value is -inf (weight 0).  Keys grow with off, so one bound
// per lane decides every value; off is a constant of the unrolled code.
__device__ __forceinline__ void mask_scores(f32x16_t (&s)[2], int key_base, int key_end, bool causal, int row_tok,
                                            float c, int lane) {
  const int kb = key_base + (lane >> 5) * 4;
  const int lim = causal ? min(key_end, row_tok + 1) - kb : key_end - kb;
  const float fill = c > 0.0f ? kNegInf : -kNegInf;
#pragma unroll
  for (int b = 0; b < 2; ++b)
#pragma unroll
    for (int i = 0; i < 16; ++i)
      if (!(b * 32 + (i >> 2) * 8 + (i & 3) < lim)) s[b][i] = fill;
}

// Largest scaled score of each row in one tile (scores already masked), over
// both lanes of the row; -inf when every key is masked.
__device__ __forceinline__ float tile_max(const f32x16_t (&s)[2], float c) {
  float mx;
  if (c >= 0.0f) {
    mx = kNegInf;
#pragma unroll
    for (int b = 0; b < 2; ++b)
#pragma unroll
      for (int i = 0; i < 16; ++i) mx = fmaxf(mx, s[b][i]);
  } else {
    mx = -kNegInf;
#pragma unroll
    for (int b = 0; b < 2; ++b)
#pragma unroll
      for (int i = 0; i < 16; ++i) mx = fminf(mx, s[b][i]);
  }
  float m_tile = mx * c;
  if (!(m_tile == m_tile)) m_tile = kNegInf;
  return pair_max(m_tile);
}

// Lazy reference update of the online softmax for a tile with row max m_tile:
// the reference m_ref only moves when the row max exceeds it by more than 8 (a
// factor 256 in p), so most tiles skip the O rescale.  O and l always share
// one reference, so the final O / l is unchanged.  Returns the reference the
// tile's weights are taken against: p = exp2(c*s - m_ref), c != 0.
template <int D>
__device__ __forceinline__ float ref_update(float m_tile, f32x16_t (&oacc)[D / 32], float& m_run, float& l_run) {
  const bool need = m_tile > m_run + 8.0f;
  if (__any(need)) {
    const float m_new = need ? m_tile : m_run;
    const float alpha = exp2_fast(m_run - m_new);  // 0 when m_run was -inf
    l_run *= alpha;
#pragma unroll
    for (int mb = 0; mb < D / 32; ++mb) oacc[mb] *= alpha;
    m_run = m_new;
  }
  return (m_run == kNegInf) ? 0.0f : m_run;  // a row with no live key yet
}

// First half of the online softmax of one tile: row max and reference update.
template <int D>
__device__ __forceinline__ float softmax_ref(const f32x16_t (&s)[2], f32x16_t (&oacc)[D / 32], float& m_run,
                                             float& l_run, float c) {
  return ref_update<D>(tile_max(s, c), oacc, m_run, l_run);
}

// Second half: the weights, their row sum and the bf16 P^T operands pb[b][s2]
// of the PV K-steps.
__device__ __forceinline__ void softmax_exp(f32x16_t (&s)[2], float m_use, float c, float& l_run,
                                            bf16x8_t (&pb)[2][2]) {
  float rs = 0.0f;
#pragma unroll
  for (int b = 0; b < 2; ++b) {
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const float p = exp2_fast(fmaf(s[b][i], c, -m_use));
      s[b][i] = p;
      rs += p;
    }
  }
  l_run += pair_sum(rs);

  // P^T operand of K-step (b, s2): the lane's values i = 8*s2 .. 8*s2+7, i.e. keys
  // b*32 + 16*s2 + {g*4 + 0..3, 8 + g*4 + 0..3}.
#pragma unroll
  for (int b = 0; b < 2; ++b)
#pragma unroll
    for (int s2 = 0; s2 < 2; ++s2)
#pragma unroll
      for (int j = 0; j < 8; ++j) pb[b][s2][j] = static_cast<__bf16>(s[b][s2 * 8 + j]);
}

// Online softmax of one tile: both halves.
template <int D>
__device__ __forceinline__ void softmax_tile(f32x16_t (&s)[2], f32x16_t (&oacc)[D / 32], float& m_run,
                                             float& l_run, float c, bf16x8_t (&pb)[2][2]) {
  const float m_use = softmax_ref<D>(s, oacc, m_run, l_run, c);
  softmax_exp(s, m_use, c, l_run, pb);
}

// V^T operand of PV MFMA j of the tile (see pv_tile): lane k of each 16-lane
// group points at V[K0 + k/4][D0 + 4*(k%4)]; the transposed read returns
// V[K0 .. K0+3][D0 + k] to lane k.
template <int D>
__device__ __forceinline__ i16x8_t v_operand(const uint16_t* __restrict__ Vs, int j, const TileOffsets<D>& to) {
  constexpr int NMB = D / 32;
  const int bs = j / NMB, mb = j % NMB;
  const int rows = (bs >> 1) * 32 + 16 * (bs & 1);  // first key of K-step bs
  const i16x4_t va = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4_t*)(Vs + rows * D + to.voff[2 * mb]));
  const i16x4_t vb = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4_t*)(Vs + rows * D + to.voff[2 * mb + 1]));
  return __builtin_shufflevector(va, vb, 0, 1, 2, 3, 4, 5, 6, 7);
}

// Operands of the first kPvPre<D> PV MFMAs (of 4 * D / 32), read before the
// softmax so their LDS latency passes under its VALU work.
template <int D>
constexpr int kPvPre = D >= 64 ? 4 : 2;

// O^T += V^T P^T over the tile.  MFMA j is K-step (b, s2) = j / (D/32) of O^T
// block mb = j % (D/32): blocks alternate, so consecutive MFMAs are
// independent.  The operands of MFMAs 0 .. kPvPre<D>-1 arrive in vpre; every
// later one is read kPvPre<D> MFMAs ahead.
template <int D, int PRE>
__device__ __forceinline__ void pv_tile(const uint16_t* __restrict__ Vs, const bf16x8_t (&pb)[2][2],
                                        f32x16_t (&oacc)[D / 32], const TileOffsets<D>& to,
                                        const i16x8_t (&vpre)[PRE > 0 ? PRE : 1]) {
  constexpr int NMB = D / 32, NJ = 4 * NMB;
  static_assert(NJ > PRE, "more PV MFMAs than prefetched operands");
  i16x8_t vf[NJ];
#pragma unroll
  for (int j = 0; j < NJ; ++j) vf[j] = j < PRE ? vpre[j] : v_operand<D>(Vs, j, to);
#pragma unroll
  for (int j = 0; j < NJ; ++j) {
    const int bs = j / NMB, mb = j % NMB;
    oacc[mb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, vf[j]), pb[bs >> 1][bs & 1],
                                                      oacc[mb], 0, 0, 0);
  }
  if constexpr (PRE > 0) {
#pragma unroll
    for (int k = 0; k < NJ - PRE; ++k) {
      __builtin_amdgcn_sched_group_barrier(0x100, 2, 1);
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 1);
    }
    __builtin_amdgcn_sched_group_barrier(0x008, PRE, 1);
  } else {  // reads two MFMAs ahead
    __builtin_amdgcn_sched_group_barrier(0x100, 4, 1);
#pragma unroll
    for (int k = 0; k < NJ - 2; ++k) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 1);
      __builtin_amdgcn_sched_group_barrier(0x100, 2, 1);
    }
    __builtin_amdgcn_sched_group_barrier(0x008, 2, 1);
  }
}

// One tile, computed in order: S, mask, softmax, PV.
template <int D, bool MASK>
__device__ __forceinline__ void tile_step(const uint16_t* __restrict__ Ks, const uint16_t* __restrict__ Vs,
                                          const u32x4_t (&qf)[D / 16], f32x16_t (&oacc)[D / 32],
                                          float& m_run, float& l_run, int key_base, int key_end,
                                          bool causal, int row_tok, float c, int lane, const TileOffsets<D>& to) {
  f32x16_t s[2];
  qk_tile<D>(Ks, qf, s, to);
  if (MASK) mask_scores(s, key_base, key_end, causal, row_tok, c, lane);
  bf16x8_t pb[2][2];
  softmax_tile<D>(s, oacc, m_run, l_run, c, pb);
  const i16x8_t none[1] = {};
  pv_tile<D, 0>(Vs, pb, oacc, to, none);
}

// One tile of the K-ahead loop of the two-per-CU kernel: the softmax and PV of
// tile t, whose scores s were computed during tile t-1.  With NEXT, the S MFMAs
// of tile t+1 (into sn, from the K tile at Kn) are interleaved with tile t's
// exponentials: the matrix cores work on the next scores while the VALU forms
// this tile's weights, inside one wave.
template <int D, bool MASK, bool NEXT>
__device__ __forceinline__ void tile_step_ahead(const uint16_t* __restrict__ Kn, const uint16_t* __restrict__ Vs,
                                                const u32x4_t (&qf)[D / 16], f32x16_t (&s)[2], f32x16_t (&sn)[2],
                                                f32x16_t (&oacc)[D / 32], float& m_run, float& l_run, int key_base,
                                                int key_end, bool causal, int row_tok, float c, int lane,
                                                const TileOffsets<D>& to) {
  if (MASK) mask_scores(s, key_base, key_end, causal, row_tok, c, lane);
  const float m_use = softmax_ref<D>(s, oacc, m_run, l_run, c);
  constexpr int PRE = kPvPre<D>;
  bf16x8_t pb[2][2];
  i16x8_t vpre[PRE];
  if constexpr (NEXT) {
    constexpr int NS = D / 16;  // MFMA K-steps per 32-key block
    u32x4_t a[2][NS];
#pragma unroll
    for (int b = 0; b < 2; ++b)
#pragma unroll
      for (int st = 0; st < NS; ++st) a[b][st] = *reinterpret_cast<const u32x4_t*>(Kn + b * 32 * D + to.koff[st]);
#pragma unroll
    for (int b = 0; b < 2; ++b) {
      sn[b] = f32x16_t{};
#pragma unroll
      for (int st = 0; st < NS; ++st)
        sn[b] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(a[b][st]), as_bf16x8(qf[st]), sn[b], 0, 0, 0);
    }
    softmax_exp(s, m_use, c, l_run, pb);
#pragma unroll
    for (int j = 0; j < PRE; ++j) vpre[j] = v_operand<D>(Vs, j, to);
    // K fragments three ahead of their MFMAs; between consecutive MFMAs a
    // share of the exponential phase's VALU work (about 112 instructions).
    constexpr int NM = 2 * NS, kVal = 112 / NM;
    __builtin_amdgcn_sched_group_barrier(0x100, 3, 0);
#pragma unroll
    for (int j = 0; j < NM; ++j) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      if (j < NM - 3) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
      __builtin_amdgcn_sched_group_barrier(0x402, kVal, 0);
    }
    __builtin_amdgcn_sched_barrier(0);
  } else {
    softmax_exp(s, m_use, c, l_run, pb);
#pragma unroll
    for (int j = 0; j < PRE; ++j) vpre[j] = v_operand<D>(Vs, j, to);
    __builtin_amdgcn_sched_barrier(0);
  }
  __builtin_amdgcn_s_setprio(1);
  pv_tile<D, PRE>(Vs, pb, oacc, to, vpre);
  __builtin_amdgcn_s_setprio(0);
}

template <int D, int NST>
__global__ __launch_bounds__(kThreads, (NST <= 2 ? 2 : 1)) void ikbo_attn_bf16_kernel(AttnParams P) {
  using T = Tile<D>;
  __shared__ __attribute__((aligned(16))) uint16_t smem[NST * T::stage];

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int n = lane & 31, g = lane >> 5;
  const int r_w = wave * 32 + n;  // this lane's row within the tile

  const uint16_t* __restrict__ Kg = static_cast<const uint16_t*>(P.k);
  const uint16_t* __restrict__ Vg = static_cast<const uint16_t*>(P.v);
  const int64_t row_stride = static_cast<int64_t>(P.H) * D;  // elements between consecutive tokens

  // Loader mapping: 16-byte unit u = tid + 256*r of a tile lands at LDS unit u;
  // it holds row u / NCH and (swizzled) chunk u % NCH.
  int ld_row[T::loads], ld_chunk[T::loads];
  uint32_t ld_off[T::loads];  // byte offset of the copy within a whole tile
#pragma unroll
  for (int r = 0; r < T::loads; ++r) {
    const int u = tid + kThreads * r;
    ld_row[r] = u / T::NCH;
    ld_chunk[r] = (u % T::NCH) ^ (swz(ld_row[r]) & (T::NCH - 1));
    ld_off[r] = static_cast<uint32_t>((ld_row[r] * row_stride + ld_chunk[r] * 8) * 2);
  }
  // Whole tiles are copied from a scalar tile base plus these offsets when a
  // tile's byte span fits 32 bits (always, short of ~8M elements per key row).
  const bool whole_fast = static_cast<int64_t>(kBN) * row_stride * 2 < (int64_t{1} << 31);

  const uint32_t lds_base = lds_address(smem);
  const int wave_u = __builtin_amdgcn_readfirstlane(wave);
  const TileOffsets<D> to(lane);

  // The items this workgroup takes from: its XCD's bin (workgroup i runs on
  // XCD i % 8, as the i / 8-th of that XCD's workgroups), or the whole list.
  // Without a queue the workgroups deal the bin boustrophedon-style.  With one,
  // workgroup w starts with item w and then takes the bin's next untaken item
  // (list order, longest first) whenever it finishes one; it asks for it while
  // computing its current item's last tile, so the counter's latency hides
  // behind that tile.
  const int wid = logical_wg();
  int w = wid, G = gridDim.x, x = 0;
  int64_t first = 0, end = P.n_items;
  if (P.n_bins > 1) {
    x = blockIdx.x % P.n_bins;
    w = blockIdx.x / P.n_bins;
    G = gridDim.x / P.n_bins;
    first = P.bin_off[x];
    end = P.bin_off[x + 1];
  }
  __shared__ int32_t q_next;
  int32_t* const queue = P.queue;
  int64_t pos = first + (queue ? w : deal_position(0, w, G));
  for (int64_t pass = 0;; ++pass) {
    if (pos >= end) break;
    const WorkItem it = P.items[pos];
    int32_t q_mine = 0;  // with a queue: this workgroup's next item (thread 0)
    const bool causal = it.kind == kKindSelf;
    uint64_t t_start = 0, t_ready = 0, t_loop = 0;
    if (P.trace) t_start = now_ticks();

    f32x16_t oacc[D / 32];
#pragma unroll
    for (int mb = 0; mb < D / 32; ++mb) oacc[mb] = f32x16_t{};
    float m_run = kNegInf, l_run = 0.0f;

    const int nkv = it.k1 - it.k0;
    const int ntiles = (nkv + kBN - 1) / kBN;
    const uint16_t* kbase = Kg + (static_cast<int64_t>(it.kv_base) + it.k0) * row_stride + it.h * D;
    const uint16_t* vbase = Vg + (static_cast<int64_t>(it.kv_base) + it.k0) * row_stride + it.h * D;

    // Issue the HBM -> LDS copies of the t-th tile visited into stage t % NST.
    // Tiles are visited first to last, or last to first with kv_reverse (the
    // masked partial tile then comes first; the result differs only in the
    // order of the fp32 sums).
    auto tile_of = [&](int t) { return P.kv_reverse ? ntiles - 1 - t : t; };
    auto issue = [&](int t) {
      const uint32_t st = lds_base + static_cast<uint32_t>((t % NST) * T::stage * 2);
      const int tt = tile_of(t);
      if (whole_fast && (tt + 1) * kBN <= nkv) {
        const uint16_t* kt = kbase + static_cast<int64_t>(tt) * kBN * row_stride;
        const uint16_t* vt = vbase + static_cast<int64_t>(tt) * kBN * row_stride;
#pragma unroll
        for (int r = 0; r < T::loads; ++r) {
          const uint32_t dk = st + static_cast<uint32_t>((kThreads * r + 64 * wave_u) * 16);
          copy16_to_lds_s(kt, ld_off[r], dk);
          copy16_to_lds_s(vt, ld_off[r], dk + static_cast<uint32_t>(T::elems * 2));
        }
        return;
      }
#pragma unroll
      for (int r = 0; r < T::loads; ++r) {
        const int key = min(tt * kBN + ld_row[r], nkv - 1);
        const int64_t off = key * row_stride + ld_chunk[r] * 8;
        const uint32_t dk = st + static_cast<uint32_t>((kThreads * r + 64 * wave_u) * 16);
        copy16_to_lds(kbase + off, dk);
        copy16_to_lds(vbase + off, dk + static_cast<uint32_t>(T::elems * 2));
      }
    };
    // One K or V tile (base kbase or vbase) of the t-th tile visited, to the
    // LDS byte address dst (the K-ahead ring of the two-per-CU kernel).
    auto issue_one = [&](int t, uint32_t dst, const uint16_t* base) {
      const int tt = tile_of(t);
      if (whole_fast && (tt + 1) * kBN <= nkv) {
        const uint16_t* bt = base + static_cast<int64_t>(tt) * kBN * row_stride;
#pragma unroll
        for (int r = 0; r < T::loads; ++r)
          copy16_to_lds_s(bt, ld_off[r], dst + static_cast<uint32_t>((kThreads * r + 64 * wave_u) * 16));
        return;
      }
#pragma unroll
      for (int r = 0; r < T::loads; ++r) {
        const int key = min(tt * kBN + ld_row[r], nkv - 1);
        copy16_to_lds(base + key * row_stride + ld_chunk[r] * 8,
                      dst + static_cast<uint32_t>((kThreads * r + 64 * wave_u) * 16));
      }
    };
    constexpr uint32_t kStageBytes = T::stage * 2, kTileBytes = T::elems * 2;

    const bool wave_has_rows = wave * 32 < it.nrows;
    const int row_tok = it.row0 + r_w;                   // token index (self rows)
    const int wave_last_tok = it.row0 + wave * 32 + 31;  // largest token of this wave's rows
    const float c = kernel_scale(P.scale_log2);

    // The ring's first copies depend only on the item: issue them before the
    // candidate gather, so their latency overlaps the cand_perm -> Q chain.
    if constexpr (NST == 2) {
      // K-ahead ring: stage s holds K tile t and V tile t' with t = t' + 1 once
      // the loop runs; the prologue brings K(0), V(0) and K(1).
      if (ntiles > 0) {
        issue_one(0, lds_base, kbase);
        issue_one(0, lds_base + kTileBytes, vbase);
      }
      if (ntiles > 1) issue_one(1, lds_base + kStageBytes, kbase);
    } else {
#pragma unroll
      for (int t = 0; t < NST - 1; ++t)
        if (t < ntiles) issue(t);
    }

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

    // The query fragment must be resident before the loop: the compiler then
    // has no load of its own outstanding inside the loop and adds no wait
    // there (its wait here also covers the prologue copies just issued).
#pragma unroll
    for (int st = 0; st < D / 16; ++st) asm volatile("" ::"v"(qf[st]));
    if (P.trace) t_ready = now_ticks();
    // Tile t's keys lie past every row of this wave (causal) or the wave has no rows.
    auto skip_of = [&](int t) {
      return !wave_has_rows || (causal && it.k0 + tile_of(t) * kBN > wave_last_tok);
    };
    if constexpr (NST == 2) {
      // K-ahead loop.  At the top of tile t, K(t+1) and V(t) are resident (both
      // copied during tile t-1) and every wave is done with tile t-1, so K(t+2)
      // goes to the slot of K(t) (read during tile t-1) and V(t+1) to that of
      // V(t-1).  S(t) was computed during tile t-1; tile t computes S(t+1)
      // alongside its own exponentials.  Unrolled by two so that the ring slots and
      // the two score buffers are compile-time choices.
      f32x16_t sa[2], sb[2];
      wait_vmcnt<0>();
      __syncthreads();
      if (ntiles > 0 && !skip_of(0)) qk_tile<D>(smem, qf, sa, to);
      auto body = [&](int t, auto par, f32x16_t (&sc)[2], f32x16_t (&sn)[2]) {
        constexpr int p = decltype(par)::value;
        wait_vmcnt<0>();
        __syncthreads();
        if (t + 2 < ntiles) issue_one(t + 2, lds_base + p * kStageBytes, kbase);
        if (t + 1 < ntiles) issue_one(t + 1, lds_base + (p ^ 1) * kStageBytes + kTileBytes, vbase);
        if (queue && tid == 0 && t == ntiles - 1) q_mine = G + atomicAdd(&queue[x], 1);
        const int key_base = it.k0 + tile_of(t) * kBN;
        const bool next = t + 1 < ntiles && !skip_of(t + 1);
        const uint16_t* Kn = smem + (p ^ 1) * T::stage;
        const uint16_t* Vs = smem + p * T::stage + T::elems;
        if (!skip_of(t)) {
          const bool need_mask =
              (key_base + kBN > it.k1) || (causal && key_base + kBN - 1 > it.row0 + wave * 32);
          if (next) {
            if (need_mask)
              tile_step_ahead<D, true, true>(Kn, Vs, qf, sc, sn, oacc, m_run, l_run, key_base, it.k1, causal,
                                             row_tok, c, lane, to);
            else
              tile_step_ahead<D, false, true>(Kn, Vs, qf, sc, sn, oacc, m_run, l_run, key_base, it.k1, causal,
                                              row_tok, c, lane, to);
          } else {
            if (need_mask)
              tile_step_ahead<D, true, false>(Kn, Vs, qf, sc, sn, oacc, m_run, l_run, key_base, it.k1, causal,
                                              row_tok, c, lane, to);
            else
              tile_step_ahead<D, false, false>(Kn, Vs, qf, sc, sn, oacc, m_run, l_run, key_base, it.k1, causal,
                                               row_tok, c, lane, to);
          }
        } else if (next) {
          qk_tile<D>(Kn, qf, sn, to);
        }
      };
      for (int t = 0; t < ntiles; t += 2) {
        body(t, std::integral_constant<int, 0>{}, sa, sb);
        if (t + 1 < ntiles) body(t + 1, std::integral_constant<int, 1>{}, sb, sa);
      }
    } else
    for (int t = 0; t < ntiles; ++t) {
      // Wait for this thread's copies of tile t: later tiles may stay in flight.
      const int after = min(NST - 2, ntiles - 1 - t);
      if (after <= 0) {
        wait_vmcnt<0>();
      } else if (after == 1) {
        wait_vmcnt<2 * T::loads>();
      } else {
        wait_vmcnt<(NST >= 4 ? 2 : 1) * 2 * T::loads>();
      }
      __syncthreads();  // every thread's copies of tile t are in LDS; stage (t-1) % NST is free
      if (t + NST - 1 < ntiles) issue(t + NST - 1);
      if (queue && tid == 0 && t == ntiles - 1) q_mine = G + atomicAdd(&queue[x], 1);
      const int key_base = it.k0 + tile_of(t) * kBN;  // first key of this tile, user-relative
      if (!skip_of(t)) {
        const uint16_t* Ks = smem + (t % NST) * T::stage;
        const uint16_t* Vs = Ks + T::elems;
        const bool need_mask = (key_base + kBN > it.k1) || (causal && key_base + kBN - 1 > it.row0 + wave * 32);
        if (need_mask)
          tile_step<D, true>(Ks, Vs, qf, oacc, m_run, l_run, key_base, it.k1, causal, row_tok, c, lane,
                                          to);
        else
          tile_step<D, false>(Ks, Vs, qf, oacc, m_run, l_run, key_base, it.k1, causal, row_tok, c,
                                           lane, to);
      }
    }
    __syncthreads();  // all stages free before the next item's copies
    if (queue && tid == 0 && ntiles == 0) q_mine = G + atomicAdd(&queue[x], 1);  // an item without keys
    if (P.trace) t_loop = now_ticks();

    // ---- epilogue
    // Lane holds O^T rows d = mb*32 + (i/4)*8 + g*4 + i%4 of query row r_w.
    if (it.grp < 0) {
      if (qrow >= 0) {
        if (P.lse && !causal && g == 0) P.lse[qrow * P.H + it.h] = row_lse(m_run, l_run);
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
      // value i of block mb is column mb*32 + (i/4)*8 + g*4 + i%4: in half-row 1
      // when mb*32 + (i/4)*8 >= D/2 (the lane part never crosses it)
      auto upper = [](int mb, int i) { return mb * 32 + (i / 4) * 8 >= D / 2; };
      float mx0 = 0.0f, mx1 = 0.0f;
#pragma unroll
      for (int mb = 0; mb < D / 32; ++mb)
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          if (upper(mb, i)) mx1 = fmaxf(mx1, __builtin_fabsf(oacc[mb][i]));
          else mx0 = fmaxf(mx0, __builtin_fabsf(oacc[mb][i]));
        }
      const int c0 = half_code(pair_max(mx0)), c1 = half_code(pair_max(mx1));
      if (r_w < it.nrows) {
        uint16_t* wo = static_cast<uint16_t*>(P.ws_o) + (slot * kBM + r_w) * D + g * 4;
#pragma unroll
        for (int mb = 0; mb < D / 32; ++mb)
#pragma unroll
          for (int i4 = 0; i4 < 4; ++i4)
            *reinterpret_cast<u32x2_t*>(wo + mb * 32 + i4 * 8) =
                pack4_f16_scaled(oacc[mb][i4 * 4 + 0], oacc[mb][i4 * 4 + 1], oacc[mb][i4 * 4 + 2],
                                 oacc[mb][i4 * 4 + 3], upper(mb, i4 * 4) ? c1 : c0);
      }
      if (g == 0)  // every tile row gets a record; empty rows are marked
        *reinterpret_cast<f32x4_t*>(P.ws_rec + (slot * kBM + r_w) * 4) =
            split_record(m_run, l_run, qrow, it, P.H, split_tag(it, c0, c1));
    }
    wait_vmcnt<0>();  // epilogue stores retire before the next item's copies are counted
    if (P.trace && tid == 0) {
      uint64_t* tr = P.trace + pos * 6;
      tr[0] = (static_cast<uint64_t>(wid) << 32) | hw_place();
      tr[1] = t_start;
      tr[2] = t_ready;
      tr[3] = t_loop;
      tr[4] = now_ticks();
      tr[5] = static_cast<uint64_t>(ntiles);
    }
    if (queue) {
      if (tid == 0) q_next = q_mine;
      __syncthreads();
      pos = first + q_next;
    } else {
      pos = first + deal_position(pass + 1, w, G);
    }
  }
  if (queue && tid == 0) {
    // Every workgroup of the bin is done taking items (its last answer, or its
    // first item, was past the bin's end); the last one to get here leaves
    // both counters at zero for the next launch.
    if (atomicAdd(&queue[kMaxBins + x], 1) == G - 1) {
      atomicExch(&queue[x], 0);
      atomicExch(&queue[kMaxBins + x], 0);
    }
  }
}

// ---------------------------------------------------------------------------
// bf16 MFMA kernel, two waves per SIMD: 8 wave64 = two key halves x 4 row blocks
// ---------------------------------------------------------------------------
//
// Waves w and w + 4 own the same 32 rows (row block w % 4).  Each ring stage
// holds two consecutive K/V tiles; wave half kh = w / 4 computes the tile
// 2 s + kh of stage s, so the two waves on a SIMD alternate MFMA and softmax
// work of different tiles.  After the key loop the halves exchange half of
// their O columns through LDS and each merges the (O, m, l) of both halves for
// the columns it owns (the split-softmax merge, AI-infra guide, section
// 4.6.4), then writes them.

template <int D>
struct Step {
  static constexpr int NCH = D / 8;                     // 16-byte chunks per row
  static constexpr int tile = kBN * D;                  // elements of one K (or V) tile
  static constexpr int stage = 4 * tile;                // K tile 0, K tile 1, V tile 0, V tile 1
  static constexpr int threads = 512;
  static constexpr int loads = 2 * kBN * NCH / threads; // 16-byte copies per thread per stage (K; V again)
  static constexpr int nv = D / 2;                      // O values per lane
  static constexpr int hv = nv / 2;                     // O values per lane one half owns
  static_assert(loads >= 1 && loads * threads == 2 * kBN * NCH, "stage shape");
};

// Merge the partner half's (O, m, l) into this wave's own values v in
// [V0, V0 + hv) and write them: the final bf16 rows, or the split partial
// (write_rec: this lane also writes its half's part of the row's record).
template <int D, int V0>
__device__ __forceinline__ void finish_half(const AttnParams& P, const WorkItem& it, f32x16_t (&oacc)[D / 32],
                                            float m_run, float l_run, const float* __restrict__ xo,
                                            float pm, float pl, int64_t qrow, bool causal, int r_w, int lane,
                                            bool write_rec) {
  constexpr int HV = Step<D>::hv;
  const int g = lane >> 5;
  const float M = fmaxf(m_run, pm);
  const float mu = (M == kNegInf) ? 0.0f : M;
  const float fa = exp2_fast(m_run - mu), fb = exp2_fast(pm - mu);
  const float L = l_run * fa + pl * fb;
#pragma unroll
  for (int j = 0; j < HV; ++j) {
    const int v = V0 + j;
    oacc[v / 16][v % 16] = oacc[v / 16][v % 16] * fa + xo[j * 64] * fb;
  }
  if (it.grp < 0) {
    if (qrow >= 0) {
      if (P.lse && !causal && V0 == 0 && g == 0) P.lse[qrow * P.H + it.h] = row_lse(M, L);
      uint16_t* ob = static_cast<uint16_t*>(causal ? P.out_user : P.out_cand);
      uint16_t* op = ob + (qrow * P.H + it.h) * D + g * 4;
      const float inv = L > 0.0f ? 1.0f / L : 0.0f;
#pragma unroll
      for (int j = 0; j < HV; j += 4) {
        const int v = V0 + j, mb = v / 16, i = v % 16;
        *reinterpret_cast<u32x2_t*>(op + mb * 32 + (i / 4) * 8) =
            pack4_bf16(oacc[mb][i] * inv, oacc[mb][i + 1] * inv, oacc[mb][i + 2] * inv, oacc[mb][i + 3] * inv);
      }
    }
  } else {
    // This wave's values v = V0 .. V0+HV-1 (column (v/16)*32 + ((v%16)/4)*8 +
    // g*4 + v%4) all lie in half-row V0 / HV (d < D/2 or d >= D/2); the other
    // half-row's wave writes that half's exponent into the record.
    const int64_t slot = static_cast<int64_t>(it.slot0) + it.chunk;
    float mx = 0.0f;
#pragma unroll
    for (int j = 0; j < HV; ++j) mx = fmaxf(mx, __builtin_fabsf(oacc[(V0 + j) / 16][(V0 + j) % 16]));
    const int code = half_code(pair_max(mx));
    if (r_w < it.nrows) {
      uint16_t* wo = static_cast<uint16_t*>(P.ws_o) + (slot * kBM + r_w) * D + g * 4;
#pragma unroll
      for (int j = 0; j < HV; j += 4) {
        const int v = V0 + j, mb = v / 16, i = v % 16;
        *reinterpret_cast<u32x2_t*>(wo + mb * 32 + (i / 4) * 8) =
            pack4_f16_scaled(oacc[mb][i], oacc[mb][i + 1], oacc[mb][i + 2], oacc[mb][i + 3], code);
      }
    }
    // every tile row gets a record (empty rows are marked): m, l, unit and the
    // tag's low half from half-row 0's wave, the tag's high half (c1) from
    // half-row 1's: separate bytes, no overlap
    float* rec = P.ws_rec + (slot * kBM + r_w) * 4;
    if (write_rec) {
      if (V0 == 0) {
        const f32x4_t r = split_record(M, L, qrow, it, P.H, 0);
        rec[0] = r[0];
        rec[1] = r[1];
        rec[2] = r[2];
        reinterpret_cast<uint16_t*>(rec + 3)[0] = static_cast<uint16_t>(split_tag(it, code, 0) & 0xffff);
      } else {
        reinterpret_cast<uint16_t*>(rec + 3)[1] = static_cast<uint16_t>(code);
      }
    }
  }
}

template <int D, int NST>
__global__ __launch_bounds__(512, 1) void ikbo_attn_bf16_w8_kernel(AttnParams P) {
  using S = Step<D>;
  constexpr int NT = S::threads;
  __shared__ __attribute__((aligned(16))) uint16_t smem[NST * S::stage];
  static_assert(NST * S::stage * 2 >= (8 * S::hv * 64 + 8 * 64 * 2) * 4, "exchange area fits in the ring");

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int n = lane & 31;
  const int rb = wave & 3, kh = wave >> 2;
  const int r_w = rb * 32 + n;  // this lane's row within the tile

  const uint16_t* __restrict__ Kg = static_cast<const uint16_t*>(P.k);
  const uint16_t* __restrict__ Vg = static_cast<const uint16_t*>(P.v);
  const int64_t row_stride = static_cast<int64_t>(P.H) * D;

  // Loader mapping: 16-byte unit u = tid + 512*r of a stage's K half lands at
  // LDS unit u; it holds key row u / NCH (0..127: two tiles) and, swizzled,
  // chunk u % NCH.  The V half mirrors it.
  int ld_row[S::loads], ld_chunk[S::loads];
  uint32_t ld_off[S::loads];  // byte offset of the copy within a whole stage
#pragma unroll
  for (int r = 0; r < S::loads; ++r) {
    const int u = tid + NT * r;
    ld_row[r] = u / S::NCH;
    ld_chunk[r] = (u % S::NCH) ^ (swz(ld_row[r]) & (S::NCH - 1));
    ld_off[r] = static_cast<uint32_t>((ld_row[r] * row_stride + ld_chunk[r] * 8) * 2);
  }
  const bool whole_fast = static_cast<int64_t>(2 * kBN) * row_stride * 2 < (int64_t{1} << 31);

  const uint32_t lds_base = lds_address(smem);
  const int wave_u = __builtin_amdgcn_readfirstlane(wave);
  const TileOffsets<D> to(lane);

  // The items this workgroup deals from: its XCD's bin (workgroup i runs on
  // XCD i % 8, as the i / 8-th of that XCD's workgroups), or the whole list.
  const int wid = logical_wg();
  int w = wid, G = gridDim.x;
  int64_t first = 0, end = P.n_items;
  if (P.n_bins > 1) {
    const int x = blockIdx.x % P.n_bins;
    w = blockIdx.x / P.n_bins;
    G = gridDim.x / P.n_bins;
    first = P.bin_off[x];
    end = P.bin_off[x + 1];
  }
  for (int64_t pass = 0;; ++pass) {
    const int64_t pos = first + deal_position(pass, w, G);
    if (pos >= end) break;
    const WorkItem it = P.items[pos];
    const bool causal = it.kind == kKindSelf;
    uint64_t t_start = 0, t_ready = 0, t_loop = 0;
    if (P.trace) t_start = now_ticks();

    f32x16_t oacc[D / 32];
#pragma unroll
    for (int mb = 0; mb < D / 32; ++mb) oacc[mb] = f32x16_t{};
    float m_run = kNegInf, l_run = 0.0f;

    const int nkv = it.k1 - it.k0;
    const int ntiles = (nkv + kBN - 1) / kBN;
    const int nsteps = (ntiles + 1) / 2;
    const uint16_t* kbase = Kg + (static_cast<int64_t>(it.kv_base) + it.k0) * row_stride + it.h * D;
    const uint16_t* vbase = Vg + (static_cast<int64_t>(it.kv_base) + it.k0) * row_stride + it.h * D;

    // Issue the HBM -> LDS copies of tiles 2s and 2s+1 into stage s % NST.
    // Keys past the range load the last key again (in bounds, masked later).
    auto issue = [&](int st_idx) {
      const uint32_t st = lds_base + static_cast<uint32_t>((st_idx % NST) * S::stage * 2);
      if (whole_fast && (st_idx + 1) * 2 * kBN <= nkv) {
        const uint16_t* kt = kbase + static_cast<int64_t>(st_idx) * 2 * kBN * row_stride;
        const uint16_t* vt = vbase + static_cast<int64_t>(st_idx) * 2 * kBN * row_stride;
#pragma unroll
        for (int r = 0; r < S::loads; ++r) {
          const uint32_t dk = st + static_cast<uint32_t>((NT * r + 64 * wave_u) * 16);
          copy16_to_lds_s(kt, ld_off[r], dk);
          copy16_to_lds_s(vt, ld_off[r], dk + static_cast<uint32_t>(2 * S::tile * 2));
        }
        return;
      }
#pragma unroll
      for (int r = 0; r < S::loads; ++r) {
        const int key = min(st_idx * 2 * kBN + ld_row[r], nkv - 1);
        const int64_t off = key * row_stride + ld_chunk[r] * 8;
        const uint32_t dk = st + static_cast<uint32_t>((NT * r + 64 * wave_u) * 16);
        copy16_to_lds(kbase + off, dk);
        copy16_to_lds(vbase + off, dk + static_cast<uint32_t>(2 * S::tile * 2));
      }
    };

    const bool wave_has_rows = rb * 32 < it.nrows;
    const int row_tok = it.row0 + r_w;
    const int wave_last_tok = it.row0 + rb * 32 + 31;
    const float c = kernel_scale(P.scale_log2);

#pragma unroll
    for (int s = 0; s < NST - 1; ++s)
      if (s < nsteps) issue(s);

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
      const int g = lane >> 5;
      const uint16_t* qb = static_cast<const uint16_t*>(causal ? P.q_user : P.q_cand);
      const uint16_t* qp = qb + (qrow < 0 ? 0 : (qrow * P.H + it.h) * D) + g * 8;
#pragma unroll
      for (int st = 0; st < D / 16; ++st)
        qf[st] = (qrow < 0) ? u32x4_t{0, 0, 0, 0} : *reinterpret_cast<const u32x4_t*>(qp + st * 16);
    }
#pragma unroll
    for (int st = 0; st < D / 16; ++st) asm volatile("" ::"v"(qf[st]));
    if (P.trace) t_ready = now_ticks();

    for (int s = 0; s < nsteps; ++s) {
      const int after = min(NST - 2, nsteps - 1 - s);
      if (after <= 0) {
        wait_vmcnt<0>();
      } else if (after == 1) {
        wait_vmcnt<2 * S::loads>();
      } else {
        wait_vmcnt<(NST >= 4 ? 2 : 1) * 2 * S::loads>();
      }
      __syncthreads();  // stage s is in LDS for every thread; stage (s-1) % NST is free
      if (s + NST - 1 < nsteps) issue(s + NST - 1);
      const int t = 2 * s + kh;
      const int key_base = it.k0 + t * kBN;
      const bool skip = t >= ntiles || !wave_has_rows || (causal && key_base > wave_last_tok);
      if (!skip) {
        const uint16_t* Ks = smem + (s % NST) * S::stage + kh * S::tile;
        const uint16_t* Vs = smem + (s % NST) * S::stage + 2 * S::tile + kh * S::tile;
        const bool need_mask = (key_base + kBN > it.k1) || (causal && key_base + kBN - 1 > it.row0 + rb * 32);
        if (need_mask)
          tile_step<D, true>(Ks, Vs, qf, oacc, m_run, l_run, key_base, it.k1, causal, row_tok, c, lane,
                                       to);
        else
          tile_step<D, false>(Ks, Vs, qf, oacc, m_run, l_run, key_base, it.k1, causal, row_tok, c,
                                        lane, to);
      }
    }
    __syncthreads();  // every ring read is done: the ring becomes the exchange area
    if (P.trace) t_loop = now_ticks();

    // ---- exchange: half 0 keeps O values [0, hv), half 1 keeps [hv, nv).
    // Each wave stores the values its partner keeps, lane-major (conflict free).
    float* xbuf = reinterpret_cast<float*>(smem);
    float* mlbuf = xbuf + 8 * S::hv * 64;
    {
      float* mine = xbuf + wave * S::hv * 64 + lane;
      if (kh == 0) {
#pragma unroll
        for (int j = 0; j < S::hv; ++j) mine[j * 64] = oacc[(S::hv + j) / 16][(S::hv + j) % 16];
      } else {
#pragma unroll
        for (int j = 0; j < S::hv; ++j) mine[j * 64] = oacc[j / 16][j % 16];
      }
      mlbuf[(wave * 64 + lane) * 2 + 0] = m_run;
      mlbuf[(wave * 64 + lane) * 2 + 1] = l_run;
    }
    __syncthreads();
    {
      const int partner = wave ^ 4;
      const float* xo = xbuf + partner * S::hv * 64 + lane;
      const float pm = mlbuf[(partner * 64 + lane) * 2 + 0];
      const float pl = mlbuf[(partner * 64 + lane) * 2 + 1];
      const bool write_rec = (lane >> 5) == 0;  // one lane per row in each half
      if (kh == 0)
        finish_half<D, 0>(P, it, oacc, m_run, l_run, xo, pm, pl, qrow, causal, r_w, lane, write_rec);
      else
        finish_half<D, S::hv>(P, it, oacc, m_run, l_run, xo, pm, pl, qrow, causal, r_w, lane, write_rec);
    }
    wait_vmcnt<0>();  // epilogue stores retire before the next item's copies are counted
    __syncthreads();  // the exchange area is read before the next item's copies overwrite it
    if (P.trace && tid == 0) {
      uint64_t* tr = P.trace + pos * 6;
      tr[0] = (static_cast<uint64_t>(wid) << 32) | hw_place();
      tr[1] = t_start;
      tr[2] = t_ready;
      tr[3] = t_loop;
      tr[4] = now_ticks();
      tr[5] = static_cast<uint64_t>(ntiles);
    }
  }
}

// ---------------------------------------------------------------------------
// split-KV merge: block (group, row block); thread -> (row, 4 d)
// ---------------------------------------------------------------------------
//
// Everything the merge needs comes from the partials' row records: the chunk
// count, the output row and the kind.  A thread loads the records of all
// kMaxSplit slots of its group at once (slots past nchunk hold stale records
// and are ignored), then one 16-byte slice of O per chunk, computes its row's
// chunk weights and sums the weighted slices in chunk order.

template <int D, bool HALF>
__global__ __launch_bounds__(256) void ikbo_merge_kernel(AttnParams P) {
  constexpr int TPR = D / 4;      // threads per row
  constexpr int RPB = 256 / TPR;  // rows per block
  const int r = blockIdx.y * RPB + threadIdx.x / TPR;
  const int d0 = (threadIdx.x % TPR) * 4;
  const int64_t slot0 = static_cast<int64_t>(blockIdx.x) * kMaxSplit;
  f32x4_t rec[kMaxSplit];
#pragma unroll
  for (int ch = 0; ch < kMaxSplit; ++ch)
    rec[ch] = *reinterpret_cast<const f32x4_t*>(P.ws_rec + ((slot0 + ch) * kBM + r) * 4);
  // The fields are copied out of the vector before the bit cast: clang reads a
  // bit cast of a vector element as a cast of element 0.
  const float unit_f = rec[0][2], tag_f = rec[0][3];
  const int unit = __builtin_bit_cast(int, unit_f);
  const int tag = __builtin_bit_cast(int, tag_f);
  const int nchunk = tag & 15, kind = (tag >> 4) & 1;
  if (unit < 0) return;  // no row here
  f32x4_t o[kMaxSplit];
#pragma unroll
  for (int ch = 0; ch < kMaxSplit; ++ch) {
    const int64_t at = ((slot0 + ch) * kBM + r) * D + d0;
    if constexpr (HALF) {
      typedef _Float16 f16x4_t __attribute__((ext_vector_type(4)));
      // this slice's half-row exponent, from the chunk's own record
      const float ct = rec[ch][3];
      const int e = ((__builtin_bit_cast(int, ct) >> (d0 < D / 2 ? 8 : 16)) & 255) - 141;
      const f16x4_t x = ch < nchunk ? *reinterpret_cast<const f16x4_t*>(static_cast<const uint16_t*>(P.ws_o) + at)
                                    : f16x4_t{0, 0, 0, 0};
      o[ch] = f32x4_t{__builtin_ldexpf(static_cast<float>(x[0]), e), __builtin_ldexpf(static_cast<float>(x[1]), e),
                      __builtin_ldexpf(static_cast<float>(x[2]), e), __builtin_ldexpf(static_cast<float>(x[3]), e)};
    } else {
      o[ch] = ch < nchunk ? *reinterpret_cast<const f32x4_t*>(static_cast<const float*>(P.ws_o) + at)
                          : f32x4_t{0, 0, 0, 0};
    }
  }
  float m[kMaxSplit], l[kMaxSplit], w[kMaxSplit];
#pragma unroll
  for (int ch = 0; ch < kMaxSplit; ++ch) {
    m[ch] = ch < nchunk ? rec[ch][0] : kNegInf;
    l[ch] = ch < nchunk ? rec[ch][1] : 0.0f;
  }
  chunk_weights(m, l, nchunk, w);
  u32x2_t packed;
  switch (nchunk) {  // straight-line sums over exactly nchunk slices
    case 1: packed = weigh_slice<1>(w, o); break;
    case 2: packed = weigh_slice<2>(w, o); break;
    case 3: packed = weigh_slice<3>(w, o); break;
    case 4: packed = weigh_slice<4>(w, o); break;
    case 5: packed = weigh_slice<5>(w, o); break;
    case 6: packed = weigh_slice<6>(w, o); break;
    case 7: packed = weigh_slice<7>(w, o); break;
    default: packed = weigh_slice<8>(w, o); break;
  }
  uint16_t* ob = static_cast<uint16_t*>(kind == kKindSelf ? P.out_user : P.out_cand);
  *reinterpret_cast<u32x2_t*>(ob + static_cast<int64_t>(unit) * D + d0) = packed;
  if (P.lse && d0 == 0 && kind == kKindTarget) {
    // the row's log-sum-exp over all chunks: 2^M sum_c 2^(m_c - M) l_c
    float M = kNegInf;
#pragma unroll
    for (int ch = 0; ch < kMaxSplit; ++ch) M = fmaxf(M, m[ch]);
    const float mu = (M == kNegInf) ? 0.0f : M;
    float L = 0.0f;
#pragma unroll
    for (int ch = 0; ch < kMaxSplit; ++ch) L += ch < nchunk ? exp2_fast(m[ch] - mu) * l[ch] : 0.0f;
    P.lse[unit] = row_lse(mu, L);
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

// With ev != nullptr, ev[0] / ev[1] are stamped by the dispatch itself at the
// kernel's start and end (hipExtLaunchKernelGGL), for timing.
#define IKBO_LAUNCH(KERNEL, GRID, BLOCK, ...)                                              \
  do {                                                                                    \
    if (ev)                                                                               \
      hipExtLaunchKernelGGL(KERNEL, GRID, BLOCK, 0, stream, ev[0], ev[1], 0, __VA_ARGS__); \
    else                                                                                  \
      hipLaunchKernelGGL(KERNEL, GRID, BLOCK, 0, stream, __VA_ARGS__);                    \
  } while (0)

hipError_t launch_attn_bf16(const AttnParams& p, int d, int stages, int grid, hipStream_t stream,
                            hipEvent_t* ev) {
  if (grid <= 0 || p.n_items <= 0) return hipSuccess;
#define IKBO_LAUNCH_BF16(DD, SS) IKBO_LAUNCH((ikbo_attn_bf16_kernel<DD, SS>), dim3(grid), dim3(kThreads), p)
  if (stages == 2) {
    switch (d) {
      case 128: IKBO_LAUNCH_BF16(128, 2); break;
      case 64: IKBO_LAUNCH_BF16(64, 2); break;
      case 32: IKBO_LAUNCH_BF16(32, 2); break;
      default: return hipErrorInvalidValue;
    }
  } else if (stages == 3) {
    switch (d) {
      case 128: IKBO_LAUNCH_BF16(128, 3); break;
      case 64: IKBO_LAUNCH_BF16(64, 3); break;
      case 32: IKBO_LAUNCH_BF16(32, 3); break;
      default: return hipErrorInvalidValue;
    }
  } else if (stages == 4) {
    switch (d) {
      case 128: IKBO_LAUNCH_BF16(128, 4); break;
      case 64: IKBO_LAUNCH_BF16(64, 4); break;
      case 32: IKBO_LAUNCH_BF16(32, 4); break;
      default: return hipErrorInvalidValue;
    }
  } else {
    return hipErrorInvalidValue;
  }
#undef IKBO_LAUNCH_BF16
  return hipGetLastError();
}

hipError_t launch_attn_bf16_w8(const AttnParams& p, int d, int grid, hipStream_t stream, hipEvent_t* ev) {
  if (grid <= 0 || p.n_items <= 0) return hipSuccess;
  switch (d) {
    case 128: IKBO_LAUNCH((ikbo_attn_bf16_w8_kernel<128, 2>), dim3(grid), dim3(512), p); break;
    case 64: IKBO_LAUNCH((ikbo_attn_bf16_w8_kernel<64, 2>), dim3(grid), dim3(512), p); break;
    case 32: IKBO_LAUNCH((ikbo_attn_bf16_w8_kernel<32, 2>), dim3(grid), dim3(512), p); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t launch_merge(const AttnParams& p, int n_groups, int d, bool half_partials, hipStream_t stream,
                        hipEvent_t* ev) {
  if (n_groups <= 0) return hipSuccess;
  const dim3 grid(n_groups, kBM / (256 / (d / 4)));
  if (half_partials) {
    switch (d) {
      case 128: IKBO_LAUNCH((ikbo_merge_kernel<128, true>), grid, dim3(256), p); break;
      case 64: IKBO_LAUNCH((ikbo_merge_kernel<64, true>), grid, dim3(256), p); break;
      case 32: IKBO_LAUNCH((ikbo_merge_kernel<32, true>), grid, dim3(256), p); break;
      default: return hipErrorInvalidValue;
    }
  } else {
    if (d != 128) return hipErrorInvalidValue;
    IKBO_LAUNCH((ikbo_merge_kernel<128, false>), grid, dim3(256), p);
  }
  return hipGetLastError();
}

hipError_t launch_attn_f32(const AttnParams& p, int d, int grid, hipStream_t stream, hipEvent_t* ev) {
  if (grid <= 0 || p.n_items <= 0) return hipSuccess;
  switch (d) {
    case 128: IKBO_LAUNCH(ikbo_attn_f32_kernel<128>, dim3(grid), dim3(64), p); break;
    case 64: IKBO_LAUNCH(ikbo_attn_f32_kernel<64>, dim3(grid), dim3(64), p); break;
    case 32: IKBO_LAUNCH(ikbo_attn_f32_kernel<32>, dim3(grid), dim3(64), p); break;
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
