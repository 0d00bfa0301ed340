"""fp64 CPU oracle for MXFP8 IKBO target attention -- TEST INFRASTRUCTURE ONLY.

Only the test suite, the package smoke check and the benchmark's CPU-baseline
leg may import or call this module; the product path never routes through it
and shares no code with it.

What it computes, and where the pages say so:

* The TLX attention post (section 3, the low-precision variant) describes a
  micro-scaled FP8 attention: both matrix products take FP8 E4M3 data with one
  E8M0 scale per block of elements along the contraction, and the softmax
  output P is quantized to FP8 on the fly, with its own block scales, before
  the P.V product.  Applied to IKBO target attention (IKBO blog, section 3.1,
  Fig. 10), each candidate's query attends over its user's keys and values,
  and the oracle builds that user's K/V copy for every candidate explicitly.
* Number formats (the OCP FP8 and microscaling conventions the post names):
  E4M3 has a sign, 4 exponent bits with bias 7 and 3 mantissa bits, no
  infinities, and S.1111.111 as NaN (largest finite value 448); exponent field
  0 holds subnormals m/8 * 2^-6.  E8M0 is an unsigned biased exponent: code s
  means 2^(s - 127); 255 is NaN.  A block is 32 consecutive elements along the
  contraction.

Readings where the pages leave a step open (also listed in the design notes):

* Blocks.  Q and K carry one scale per 32 consecutive head-dimension entries
  (q_scales [C, n_q, H, d/32], k_scales [T, H, d/32]).  V is contracted over
  keys, so its blocks run along each user's sequence: 32 consecutive keys of
  one user, starting at the user's first key, share one scale per head and
  column (v_scales [NVB, H, d], user u's blocks from v_block_offsets(offs)[u],
  the last one partial).
* Softmax in base 2 with an integer reference: x = scale * log2(e) * (q . k),
  m = ceil(max_j x_j), p_j = 2^(x_j - m).  Any integer m gives the same output
  (every quantization step below is invariant under powers of two; only which
  blocks fall below the 2^-100 drop threshold, relative to the row maximum,
  moves), so a kernel may keep a running integer reference, let it lag the
  running maximum by a few units (weights above 1), and rescale by exact
  powers of two; pinned for references above and below ceil(max x).
* P's block scale: the smallest power of two 2^e with max|p| <= 448 * 2^e over
  the block's 32 keys (blocks aligned like V's); each p_j / 2^e is rounded to
  E4M3 (nearest, ties to even) and multiplied back.  A block whose maximum is
  below 2^-100 is dropped (its quantized weights are zero).  This rule never
  saturates.
* The row sum l = sum_j p_j is taken before quantization, and
  O = sum_j P^_j v^_j / l.  A user with no keys gives zero rows.
"""

from __future__ import annotations

import math

import numpy as np

__all__ = ["e4m3_decode", "e8m0_decode", "e4m3_round", "p_block_exponent", "v_block_offsets", "dequantize_rows",
           "dequantize_v", "target_attention_mxfp8"]

E4M3_MAX = 448.0
P_BLOCK = 32
P_DROP = 2.0 ** -100
LOG2E = 1.4426950408889634


def e4m3_decode(codes) -> np.ndarray:
    """Value of each E4M3 code (NaN for the two NaN codes), fp64."""
    c = np.asarray(codes, dtype=np.int64)
    sign = np.where((c >> 7) & 1, -1.0, 1.0)
    exp = (c >> 3) & 0xF
    man = (c & 7).astype(np.float64)
    mag = np.where(exp == 0, man / 8.0 * 2.0 ** -6, (1.0 + man / 8.0) * np.exp2(exp.astype(np.float64) - 7.0))
    val = sign * mag
    return np.where((c & 0x7F) == 0x7F, np.nan, val)


def e8m0_decode(codes) -> np.ndarray:
    """2^(s - 127) for each E8M0 code s (NaN for 255), fp64."""
    s = np.asarray(codes, dtype=np.int64)
    return np.where(s == 255, np.nan, np.exp2(s.astype(np.float64) - 127.0))


def e4m3_round(x) -> np.ndarray:
    """Nearest E4M3 value (ties to even), magnitudes above 448 clamped to 448."""
    x = np.asarray(x, dtype=np.float64)
    a = np.minimum(np.abs(x), E4M3_MAX)
    _, ex = np.frexp(a)                                  # a = f * 2^ex, f in [0.5, 1)
    binade = np.clip(ex - 1, -6, 8)                      # floor(log2 a); subnormals share binade -6
    step = np.exp2(binade.astype(np.float64) - 3.0)      # 3 mantissa bits
    q = np.round(a / step) * step                        # a / step is exact; np.round ties to even
    return np.copysign(q, x)


def p_block_exponent(amax: float):
    """Exponent e of P's block scale: the smallest e with amax <= 448 * 2^e, or
    None when the block is dropped (amax below 2^-100)."""
    if not amax >= P_DROP:
        return None
    f, ex = math.frexp(amax)           # amax = f * 2^ex, f in [0.5, 1)
    mant, top = 2.0 * f, ex - 1        # amax = mant * 2^top, mant in [1, 2)
    return top - 8 if mant <= 1.75 else top - 7


def v_block_offsets(user_offsets) -> np.ndarray:
    """First V-scale block of each user (exclusive scan of ceil(L_u / 32)), [U + 1]."""
    offs = np.asarray(user_offsets, dtype=np.int64)
    nblk = (offs[1:] - offs[:-1] + P_BLOCK - 1) // P_BLOCK
    return np.concatenate([[0], np.cumsum(nblk)]).astype(np.int64)


def dequantize_rows(codes, scales) -> np.ndarray:
    """Q or K: codes [..., d] with one scale per 32 entries of the last axis."""
    v = e4m3_decode(codes)
    s = e8m0_decode(scales)
    return v * np.repeat(s, P_BLOCK, axis=-1)


def dequantize_v(v_codes, v_scales, user_offsets) -> np.ndarray:
    """V [T, H, d]: token t of user u uses block v_block_offsets[u] + (t - offs[u]) // 32."""
    offs = np.asarray(user_offsets, dtype=np.int64)
    vb = v_block_offsets(offs)
    v = e4m3_decode(v_codes)
    s = e8m0_decode(v_scales)
    out = np.empty_like(v)
    for u in range(len(offs) - 1):
        a, b = int(offs[u]), int(offs[u + 1])
        t = np.arange(a, b)
        out[a:b] = v[a:b] * s[vb[u] + (t - a) // P_BLOCK]
    return out


def _quantize_p(p: np.ndarray) -> np.ndarray:
    """P's on-the-fly quantization over blocks of 32 keys from the user's first key."""
    q = np.zeros_like(p)
    for j0 in range(0, p.shape[0], P_BLOCK):
        blk = p[j0:j0 + P_BLOCK]
        e = p_block_exponent(float(blk.max()))
        if e is None:
            continue
        q[j0:j0 + P_BLOCK] = e4m3_round(blk / 2.0 ** e) * 2.0 ** e
    return q


def target_attention_mxfp8(q_codes, q_scales, k_codes, k_scales, v_codes, v_scales, user_offsets, cand_to_user,
                           scale, m_shift: int = 0) -> np.ndarray:
    """MXFP8 IKBO target attention, fp64.  q_codes [C, n_q, H, d], q_scales
    [C, n_q, H, d/32], k_codes [T, H, d], k_scales [T, H, d/32], v_codes
    [T, H, d], v_scales [NVB, H, d] (uint8 codes); returns [C, n_q, H, d].
    m_shift adds an integer to the softmax reference (the output must not
    change)."""
    offs = np.asarray(user_offsets, dtype=np.int64)
    c2u = np.asarray(cand_to_user, dtype=np.int64)
    q = dequantize_rows(q_codes, q_scales)
    k = dequantize_rows(k_codes, k_scales)
    v = dequantize_v(v_codes, v_scales, offs)
    c_log2 = float(np.float32(scale)) * LOG2E
    C, n_q, H, d = q.shape
    out = np.zeros((C, n_q, H, d), dtype=np.float64)
    for c in range(C):
        u = int(c2u[c])
        a, b = int(offs[u]), int(offs[u + 1])
        if b == a:
            continue
        kc = k[a:b].copy()  # the broadcast copies this candidate would receive
        vc = v[a:b].copy()
        for r in range(n_q):
            for h in range(H):
                x = c_log2 * (kc[:, h, :] @ q[c, r, h, :])
                m = math.ceil(float(x.max())) + m_shift
                p = np.exp2(x - m)
                out[c, r, h, :] = (_quantize_p(p) @ vc[:, h, :]) / p.sum()
    return out
