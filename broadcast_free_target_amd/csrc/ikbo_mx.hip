// MXFP8 IKBO target attention for gfx950 (TLX attention post, section 3, the
// low-precision variant; IKBO blog, section 3.1, Fig. 10): Q, K and V arrive
// as E4M3 codes with one E8M0 scale per 32 elements along each product's
// contraction, both products run on the block-scaled FP8 matrix instruction
// v_mfma_scale_f32_32x32x64_f8f6f4, and the softmax weights are quantized to
// E4M3 on the fly with their own per-32-key scales.
//
// Lane layout of the scaled instruction (32 x 32 output, 64-deep contraction,
// 32 bytes per lane and operand): lane l holds row l % 32 of A (column l % 32
// of B); its bytes 0-15 belong to contraction block 0 and bytes 16-31 to block
// 1, each block being bytes 0-15 (or 16-31) of lanes i and i + 32.  The scale
// of row i's block c is the byte the opsel selects in lane i + 32c's scale
// register.  Which contraction index a byte stands for is free as long as A
// and B agree, so:
//   * S^T = K . Q^T over d: lane half g holds d chunks g and 2 + g (16 bytes
//     each) of its key (A) or query row (B) for d 0..63, chunks 4 + g and
//     6 + g for d 64..127; scale block c is d-block c (0..3).
//   * O^T = V^T . P^T over keys: the S accumulator leaves lane (row n, half g)
//     with keys kk(b, v) = 32b + 8(v/4) + 4g + v%4 of block b; byte v of block
//     b of the P operand is that key, and the V^T operand is gathered in the
//     same key order with ds_read_b64_tr_b8.  Scale block b is the tile's key
//     block b, which is a V-scale block (tiles start on 64-key boundaries of
//     the user's sequence).
#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>

#include <cstdint>
#include <type_traits>

#include "ikbo_device.h"
#include "ikbo_mx.h"

namespace ikbo {
namespace {

using namespace dev;

constexpr int kT = 256;  // 4 wave64
constexpr int kNst = 4;  // HBM -> LDS ring depth
constexpr float kNegInf = -__builtin_inff();
constexpr float kLazyRef = 8.0f;  // headroom of the softmax reference (log2 units)

// One ring stage: K tile [64 keys][128 B], V tile [64][128 B] (16-byte
// chunks swizzled per key, mx_swz), K scales [64 keys][4 B], V scales [2 blocks][128 B],
// and a spare area the scale copies of waves 2-3 land in (every wave issues the
// same number of copies, so one vmcnt wait fits all).
constexpr int kStK = 0, kStV = 8192, kStKS = 16384, kStVS = 16640, kStSpare = 16896, kStBytes = 17408;
constexpr int kCopies = 5;  // copies per thread per stage: 2 K, 2 V, 1 scale

typedef int v8i __attribute__((ext_vector_type(8)));
typedef int v4i __attribute__((ext_vector_type(4)));
typedef int v2i __attribute__((ext_vector_type(2)));
typedef __attribute__((address_space(3))) v2i lds_v2i;

// 16-byte chunk swizzle of a key row: bits 1, 3 and 2 of the key become bits
// 1, 2 and 0 of the XOR.  Over 16 consecutive keys (a K fragment read) the
// even keys, and the odd ones, get 8 distinct values; over the 8 keys of one
// transposed V read (8(r/4) + 4g + r%4, read as column chunks 2mb and 2mb + 1
// by the two 16-lane groups of a half) the even keys, and the odd ones, get
// values that differ in bits 1-2, so the chunk pair stays on distinct banks.
__device__ __forceinline__ int mx_swz(int key) { return (((key >> 1) & 1) << 1) | (((key >> 3) & 1) << 2) | ((key >> 2) & 1); }

#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"
// One 4-byte-per-lane HBM -> LDS copy (global_load_lds_dword): lane l's 4
// bytes land at lds_byte + 4*l.
__device__ __forceinline__ void copy4_to_lds(const void* src, uint32_t lds_byte) {
  asm volatile("s_mov_b32 m0, %1\n\tglobal_load_lds_dword %0, off" ::"v"(src), "s"(lds_byte) : "memory", "m0");
}
#pragma clang diagnostic pop

__device__ __forceinline__ float half_max(float x) { return fmaxf(x, __shfl_xor(x, 32)); }
__device__ __forceinline__ float half_sum(float x) {
  const float y = __shfl_xor(x, 32);
  return (threadIdx.x & 32) ? y + x : x + y;  // same operand order in both lanes of a pair
}

__device__ __forceinline__ int64_t deal_position(int64_t pass, int w, int grid) {
  return pass * grid + ((pass & 1) ? (grid - 1 - w) : w);
}

// Exponent of P's block scale: the smallest e with amax <= 448 * 2^e (read
// from amax's exponent and mantissa bits), or a value below -100 when the
// block is dropped (amax < 2^-100, including 0).
__device__ __forceinline__ int p_block_exp(float amax) {
  const uint32_t b = __builtin_bit_cast(uint32_t, amax);
  const int top = static_cast<int>((b >> 23) & 0xFF) - 127;  // amax = 1.m * 2^top (normal amax)
  return top - 8 + ((b & 0x7FFFFF) > 0x600000 ? 1 : 0);
}

// One tile's online softmax (base 2, integer reference m) and P quantization,
// for lane (row n, half g) holding scores s[b][v] of keys kk(b, v).
//  * Block maxima are taken on the scores oriented by the scale's sign
//    (NEG: the scale is negative), since fl(c * s) is monotone in s; when the
//    tile maximum of x = c * s passes m by more than kLazyRef, m rises to the
//    next integer at or above it and O and l are rescaled by an exact power
//    of two.
//  * A block's largest weight is exp2(fma(s*, c, -m)) for its largest score s*,
//    bit for bit the weight of that key, and gives the block's scale 2^e.
//  * The scaled weights y = exp2(fma(s, c, -(m + e))) are rounded to E4M3 by
//    the hardware conversion (nearest, ties to even; y <= 448 up to one
//    rounding) and packed in value order; l gains 2^e * sum(y).
//  * MASK: keys at or past kv_left (the item's last tile) get weight 0.
// The block's 32 keys live in lanes n and n + 32 (half_max pairs them).
template <bool NEG, bool MASK>
__device__ __forceinline__ void softmax_quant(const f32x16_t (&s)[2], float c, int kv_left, int g, float& m_run,
                                              float& l_run, f32x16_t (&oacc)[4], v8i& pf, int& psc) {
  auto live = [&](int b, int v) { return !MASK || 32 * b + 8 * (v >> 2) + 4 * g + (v & 3) < kv_left; };
  float smax[2], xb[2];
#pragma unroll
  for (int b = 0; b < 2; ++b) {
    float mx = kNegInf;
#pragma unroll
    for (int v = 0; v < 16; ++v) mx = fmaxf(mx, live(b, v) ? (NEG ? -s[b][v] : s[b][v]) : kNegInf);
    smax[b] = half_max(mx);
    smax[b] = NEG ? -smax[b] : smax[b];  // the block's largest-weight score (+-inf if the block is empty)
    xb[b] = (smax[b] == kNegInf || smax[b] == -kNegInf) ? kNegInf : smax[b] * c;
  }
  // The reference stays put while the row's maximum exceeds it by at most
  // kLazyRef (weights up to 2^kLazyRef): every block's scale follows the
  // weights by the same power of two, so the codes and the output do not
  // change.  When a row passes that, its reference rises to the next integer
  // at or above its maximum; the wave skips the rescale when no row rises
  // (rows that do not rise multiply by exactly 1).
  const float tmax = fmaxf(xb[0], xb[1]);
  const bool rise = m_run == kNegInf || tmax > m_run + kLazyRef;
  if (__any(rise)) {
    const float m_new = rise ? __builtin_ceilf(tmax) : m_run;
    const float alpha = m_new == m_run    ? 1.0f
                        : m_run == kNegInf ? 0.0f
                                           : __builtin_ldexpf(1.0f, static_cast<int>(m_run - m_new));
#pragma unroll
    for (int mb = 0; mb < 4; ++mb) oacc[mb] *= alpha;
    l_run *= alpha;
    m_run = m_new;
  }
  int pw[8], e[2];
#pragma unroll
  for (int b = 0; b < 2; ++b) {
    const float amax = xb[b] == kNegInf ? 0.0f : __builtin_amdgcn_exp2f(__builtin_fmaf(smax[b], c, -m_run));
    if (amax >= 0x1p-100f) {
      e[b] = p_block_exp(amax);
      const float bias = -(m_run + static_cast<float>(e[b]));
      float sum = 0.0f;
#pragma unroll
      for (int k = 0; k < 4; ++k) {  // four weights at a time: computed, summed, converted
        float y[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int v = 4 * k + i;
          y[i] = live(b, v) ? __builtin_amdgcn_exp2f(__builtin_fmaf(s[b][v], c, bias)) : 0.0f;
          sum += y[i];
        }
        const int lo = __builtin_amdgcn_cvt_pk_fp8_f32(y[0], y[1], 0, false);
        pw[4 * b + k] = __builtin_amdgcn_cvt_pk_fp8_f32(y[2], y[3], lo, true);
      }
      l_run += __builtin_ldexpf(sum, e[b]);
    } else {  // dropped block: no weight (the largest is below 2^-100)
      e[b] = 0;
      pw[4 * b] = pw[4 * b + 1] = pw[4 * b + 2] = pw[4 * b + 3] = 0;
    }
  }
  psc = (g == 0 ? e[0] : e[1]) + 127;
  pf = v8i{pw[0], pw[1], pw[2], pw[3], pw[4], pw[5], pw[6], pw[7]};
}

template <bool NEG>
__global__ __launch_bounds__(kT, 2) void ikbo_attn_mx_kernel(MxParams P) {
  __shared__ __attribute__((aligned(16))) uint8_t smem[kNst * kStBytes];

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int n = lane & 31, g = lane >> 5;
  const int r_w = wave * 32 + n;  // this lane's row within the tile
  const int wave_u = __builtin_amdgcn_readfirstlane(wave);
  const int64_t krow = static_cast<int64_t>(P.H) * 128;  // bytes between consecutive tokens
  const uint32_t lds_base = lds_address(smem);

  // Loader mapping: 16-byte unit u = tid + 256 r of a K (V) tile lands at LDS
  // unit u, which holds key u / 8 and chunk (u % 8) ^ swizzle(key).
  int ld_key[2], ld_chunk[2];
#pragma unroll
  for (int r = 0; r < 2; ++r) {
    const int u = tid + kT * r;
    ld_key[r] = u >> 3;
    ld_chunk[r] = (u & 7) ^ mx_swz(ld_key[r]);
  }
  // Transposed V reads: lane (2r + h) of each 16-lane group points at key row r
  // of the read, byte half h of the group's 16-column chunk.
  const int tr_r = (lane & 15) >> 1, tr_h = lane & 1, tr_grp = (lane >> 4) & 1;
  // Per-lane LDS byte offsets of the tile reads, computed once: the swizzle
  // only sees key bits 1-3, so it is a lane constant and the block (K: 32
  // keys) or read (V: 16 keys) index only adds an immediate.
  //   K fragment i (chunk 2i + g) of key 32b + n:  koffs[i] + 4096 b
  //   V^T read rd of column block mb, key 16 rd + kl with
  //   kl = 8 (tr_r / 4) + 4 g + tr_r % 4:          voffs[mb] + 2048 rd
  int koffs[4], voffs[4];
  {
    const int swk = mx_swz(n);
    const int kl = 8 * (tr_r >> 2) + 4 * g + (tr_r & 3);
    const int swv = mx_swz(kl);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      koffs[i] = n * 128 + (((2 * i + g) ^ swk) << 4);
      voffs[i] = kl * 128 + (((2 * i + tr_grp) ^ swv) << 4) + 8 * tr_h;
    }
  }

  const int G = gridDim.x;
  const int wg = logical_wg();
  for (int64_t pass = 0;; ++pass) {
    const int64_t pos = deal_position(pass, wg, G);
    if (pos >= P.n_items) break;
    const WorkItem it = P.items[pos];
    const int vb0 = P.vblk[2 * pos], vlast = P.vblk[2 * pos + 1];

    f32x16_t oacc[4];
#pragma unroll
    for (int mb = 0; mb < 4; ++mb) oacc[mb] = f32x16_t{};
    float m_run = kNegInf, l_run = 0.0f;

    const int nkv = it.k1 - it.k0;
    const int ntiles = (nkv + kMxKeys - 1) / kMxKeys;
    const int64_t tok0 = static_cast<int64_t>(it.kv_base) + it.k0;
    const uint8_t* kbase = P.k + tok0 * krow + it.h * 128;
    const uint8_t* vbase = P.v + tok0 * krow + it.h * 128;
    const uint8_t* ksbase = P.ks + tok0 * P.H * 4 + it.h * 4;
    const uint8_t* vsbase = P.vs + static_cast<int64_t>(it.h) * 128;

    // Copies of tile t into stage t % kNst.  Keys past the range load the last
    // key again (in bounds, masked later); V-scale blocks past the item's last
    // block load that block again.
    auto issue = [&](int t) {
      const uint32_t st = lds_base + static_cast<uint32_t>((t % kNst) * kStBytes);
#pragma unroll
      for (int r = 0; r < 2; ++r) {
        const int key = min(t * kMxKeys + ld_key[r], nkv - 1);
        const int64_t off = key * krow + ld_chunk[r] * 16;
        const uint32_t d = static_cast<uint32_t>((kT * r + 64 * wave_u) * 16);
        copy16_to_lds(kbase + off, st + kStK + d);
        copy16_to_lds(vbase + off, st + kStV + d);
      }
      if (wave_u == 1) {
        const int blk = min(vb0 + 2 * t + (lane >> 5), vlast);
        copy4_to_lds(vsbase + static_cast<int64_t>(blk) * krow + (lane & 31) * 4, st + kStVS);
      } else {
        const int key = min(t * kMxKeys + lane, nkv - 1);
        const uint32_t dst = wave_u == 0 ? kStKS : kStSpare + (wave_u == 2 ? 0 : 256);
        copy4_to_lds(ksbase + static_cast<int64_t>(key) * P.H * 4, st + dst);
      }
    };

#pragma unroll
    for (int t = 0; t < kNst - 1; ++t)
      if (t < ntiles) issue(t);

    // ---- query fragment (B operand of S^T): chunks g, 2+g, 4+g, 6+g of the row
    int64_t qrow = -1;
    if (r_w < it.nrows) {
      const int r = it.row0 + r_w;
      const int cand = P.cand_perm[it.row_base + r / P.n_q];
      qrow = static_cast<int64_t>(cand) * P.n_q + r % P.n_q;
    }
    u32x4_t qf[4];
    uint32_t qsc = 0x7F7F7F7Fu;
    {
      const uint8_t* qp = P.q + (qrow < 0 ? 0 : (qrow * P.H + it.h) * 128);
#pragma unroll
      for (int i = 0; i < 4; ++i)
        qf[i] = (qrow < 0) ? u32x4_t{0, 0, 0, 0} : *reinterpret_cast<const u32x4_t*>(qp + (2 * i + g) * 16);
      if (qrow >= 0) qsc = *reinterpret_cast<const uint32_t*>(P.qs + (qrow * P.H + it.h) * 4) >> (8 * g);
    }
    // Resident before the loop, so the compiler adds no wait inside it.
#pragma unroll
    for (int i = 0; i < 4; ++i) asm volatile("" ::"v"(qf[i]));
    asm volatile("" ::"v"(qsc));
    const v8i qa = {static_cast<int>(qf[0][0]), static_cast<int>(qf[0][1]), static_cast<int>(qf[0][2]),
                    static_cast<int>(qf[0][3]), static_cast<int>(qf[1][0]), static_cast<int>(qf[1][1]),
                    static_cast<int>(qf[1][2]), static_cast<int>(qf[1][3])};
    const v8i qb = {static_cast<int>(qf[2][0]), static_cast<int>(qf[2][1]), static_cast<int>(qf[2][2]),
                    static_cast<int>(qf[2][3]), static_cast<int>(qf[3][0]), static_cast<int>(qf[3][1]),
                    static_cast<int>(qf[3][2]), static_cast<int>(qf[3][3])};
    const bool wave_has_rows = wave * 32 < it.nrows;
    const float c = P.scale_log2;

    // Tile t: wait for its copies, then the barrier that also frees stage
    // (t - 1) % kNst for the copies of tile t + kNst - 1.
    auto advance = [&](int t) {
      const int after = min(kNst - 2, ntiles - 1 - t);
      if (after <= 0)
        wait_vmcnt<0>();
      else if (after == 1)
        wait_vmcnt<kCopies>();
      else
        wait_vmcnt<2 * kCopies>();
      __syncthreads();  // tile t is in LDS for every thread; stage (t-1) % kNst is free
      if (t + kNst - 1 < ntiles) issue(t + kNst - 1);
    };
    auto compute = [&](int t, auto mask_tag) {
      constexpr bool MASK = decltype(mask_tag)::value;
      const uint8_t* st = smem + (t % kNst) * kStBytes;
      const int kv_left = nkv - t * kMxKeys;  // keys of this tile inside the range (may exceed 64)
      // ---- S^T = K . Q^T, two 32-key blocks (raised priority while the
      // MFMAs issue: the other resident workgroup's wave on this SIMD
      // fills the matrix cores' busy cycles with its softmax)
      f32x16_t s[2];
      __builtin_amdgcn_s_setprio(1);
#pragma unroll
      for (int b = 0; b < 2; ++b) {
        const int key = 32 * b + n;
        const uint8_t* kt = st + kStK + 4096 * b;
        const v4i k0 = *reinterpret_cast<const v4i*>(kt + koffs[0]);
        const v4i k1 = *reinterpret_cast<const v4i*>(kt + koffs[1]);
        const v4i k2 = *reinterpret_cast<const v4i*>(kt + koffs[2]);
        const v4i k3 = *reinterpret_cast<const v4i*>(kt + koffs[3]);
        const uint32_t ksc = *reinterpret_cast<const uint32_t*>(st + kStKS + key * 4) >> (8 * g);
        // the 32-byte operands as concatenations, so the loads can land in place
        const v8i ka = __builtin_shufflevector(k0, k1, 0, 1, 2, 3, 4, 5, 6, 7);
        const v8i kb = __builtin_shufflevector(k2, k3, 0, 1, 2, 3, 4, 5, 6, 7);
        f32x16_t acc = f32x16_t{};
        acc = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(ka, qa, acc, 0, 0, 0, static_cast<int>(ksc), 0,
                                                              static_cast<int>(qsc));
        acc = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(kb, qb, acc, 0, 0, 2, static_cast<int>(ksc), 2,
                                                              static_cast<int>(qsc));
        s[b] = acc;
      }

      __builtin_amdgcn_s_setprio(0);
      // ---- online softmax and P quantization
      v8i pf;
      int psc;
      softmax_quant<NEG, MASK>(s, c, kv_left, g, m_run, l_run, oacc, pf, psc);
      __builtin_amdgcn_s_setprio(1);

      // ---- O^T += V^T . P^T, four 32-column blocks
#pragma unroll
      for (int mb = 0; mb < 4; ++mb) {
        // bytes 8rd .. 8rd+7 of the operand: keys of value indices j = 8rd + r
        // (block j / 16), key 32 (j / 16) + 8 ((j % 16) / 4) + 4 g + j % 4 = 16 rd + kl
        v2i w[4];
#pragma unroll
        for (int rd = 0; rd < 4; ++rd)
          w[rd] = __builtin_amdgcn_ds_read_tr8_b64_v2i32((lds_v2i*)(st + kStV + voffs[mb] + 2048 * rd));
        const int vsc = st[kStVS + 128 * g + 32 * mb + n];
        const v8i vf = __builtin_shufflevector(__builtin_shufflevector(w[0], w[1], 0, 1, 2, 3),
                                               __builtin_shufflevector(w[2], w[3], 0, 1, 2, 3), 0, 1, 2, 3, 4, 5, 6, 7);
        oacc[mb] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(vf, pf, oacc[mb], 0, 0, 0, vsc, 0, psc);
      }
      __builtin_amdgcn_s_setprio(0);
    };
    // Only the last tile can hold keys past the range: the loop runs unmasked
    // and the last tile separately.
    for (int t = 0; t + 1 < ntiles; ++t) {
      advance(t);
      if (wave_has_rows) compute(t, std::false_type{});
    }
    if (ntiles > 0) {
      advance(ntiles - 1);
      if (wave_has_rows) compute(ntiles - 1, std::true_type{});
    }
    __syncthreads();  // every stage read before the next item's copies

    // ---- epilogue: lane holds O^T rows d = 32mb + 8(v/4) + 4g + v%4 of row r_w
    const float l_tot = half_sum(l_run);
    if (it.grp < 0) {
      if (qrow >= 0) {
        uint16_t* op = static_cast<uint16_t*>(P.out) + (qrow * P.H + it.h) * 128 + g * 4;
        const float inv = l_tot > 0.0f ? 1.0f / l_tot : 0.0f;
#pragma unroll
        for (int mb = 0; mb < 4; ++mb)
#pragma unroll
          for (int i4 = 0; i4 < 4; ++i4)
            *reinterpret_cast<u32x2_t*>(op + mb * 32 + i4 * 8) =
                pack4_bf16(oacc[mb][4 * i4 + 0] * inv, oacc[mb][4 * i4 + 1] * inv, oacc[mb][4 * i4 + 2] * inv,
                           oacc[mb][4 * i4 + 3] * inv);
      }
    } else {
      const int64_t slot = static_cast<int64_t>(it.slot0) + it.chunk;
      if (r_w < it.nrows) {
        float* wo = P.ws_o + (slot * kMxRows + r_w) * 128 + g * 4;
#pragma unroll
        for (int mb = 0; mb < 4; ++mb)
#pragma unroll
          for (int i4 = 0; i4 < 4; ++i4)
            *reinterpret_cast<f32x4_t*>(wo + mb * 32 + i4 * 8) = f32x4_t{
                oacc[mb][4 * i4 + 0], oacc[mb][4 * i4 + 1], oacc[mb][4 * i4 + 2], oacc[mb][4 * i4 + 3]};
      }
      if (g == 0) {  // every tile row gets a record; empty rows are marked
        const int unit = qrow < 0 ? -1 : static_cast<int>(qrow * P.H + it.h);
        *reinterpret_cast<f32x4_t*>(P.ws_rec + (slot * kMxRows + r_w) * 4) =
            f32x4_t{m_run, l_tot, __builtin_bit_cast(float, unit), __builtin_bit_cast(float, it.nchunk)};
      }
    }
    wait_vmcnt<0>();  // epilogue stores retire before the next item's copies are counted
  }
}

}  // namespace

hipError_t launch_mx(const MxParams& p, int grid, hipStream_t stream, hipEvent_t* ev) {
  if (grid <= 0 || p.n_items <= 0) return hipSuccess;
  auto kernel = p.scale_log2 < 0.0f ? ikbo_attn_mx_kernel<true> : ikbo_attn_mx_kernel<false>;
  if (ev)
    hipExtLaunchKernelGGL(kernel, dim3(grid), dim3(kT), 0, stream, ev[0], ev[1], 0, p);
  else
    hipLaunchKernelGGL(kernel, dim3(grid), dim3(kT), 0, stream, p);
  return hipGetLastError();
}

}  // namespace ikbo
