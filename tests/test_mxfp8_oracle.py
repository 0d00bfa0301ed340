"""Pins of the MXFP8 attention oracle (CPU).

Sources: the TLX attention post (section 3, the low-precision variant: FP8
E4M3 data with E8M0 block scales for both products, P quantized on the fly
with block scales) applied to IKBO target attention (IKBO blog, section 3.1,
Fig. 10).  The number formats are pinned to torch's float8_e4m3fn (an
independent implementation of the same format); the attention is pinned by
scalar loops that round with a lookup over the format's value table, by
closed forms, by the exact invariance to the integer softmax reference, by a
rigorous error bound against unquantized attention on the same dequantized
inputs, and by planted mistakes that the loops reject.
"""

import math

import numpy as np
import pytest

from oracle import ikbo_oracle as O
from oracle import mxfp8_oracle as M
from workloads import make_mxfp8, make_mxfp8_custom

torch = pytest.importorskip("torch")


def _torch_decode(codes):
    return torch.from_numpy(np.asarray(codes, np.uint8).copy()).view(torch.float8_e4m3fn).double().numpy()


def _torch_round(x):
    return torch.from_numpy(np.asarray(x, np.float32)).to(torch.float8_e4m3fn).double().numpy()


def test_e4m3_decode_matches_torch_on_every_code():
    codes = np.arange(256, dtype=np.uint8)
    mine, ref = M.e4m3_decode(codes), _torch_decode(codes)
    assert np.array_equal(np.isnan(mine), np.isnan(ref))
    ok = ~np.isnan(ref)
    assert np.array_equal(mine[ok], ref[ok])
    assert np.nanmax(mine) == 448.0 and mine[1] == 2.0 ** -9


def test_e4m3_round_matches_torch_nearest_even():
    rng = np.random.default_rng(0)
    vals = _torch_decode(np.arange(0, 127, dtype=np.uint8))
    mids = (vals[:-1] + vals[1:]) / 2                     # exact ties (fp32-representable)
    x = np.concatenate([rng.uniform(-448, 448, 50000), rng.standard_normal(50000) * 2.0 ** -7,
                        mids, -mids, vals, [0.0, 448.0, -448.0]]).astype(np.float32)
    assert np.array_equal(M.e4m3_round(x), _torch_round(x))
    assert np.all(M.e4m3_round([449.0, 1e6, -2e4]) == [448.0, 448.0, -448.0])  # clamped, never NaN


def test_e8m0_decode():
    assert list(M.e8m0_decode([0, 126, 127, 128, 254])) == [2.0 ** -127, 0.5, 1.0, 2.0, 2.0 ** 127]
    assert np.isnan(M.e8m0_decode([255])[0])


def test_p_block_exponent_is_the_smallest_non_saturating_power():
    rng = np.random.default_rng(1)
    for a in np.concatenate([rng.uniform(0, 1, 2000), 2.0 ** rng.uniform(-90, 0, 2000), [1.0, 0.875, 0.8749999]]):
        e = M.p_block_exponent(float(a))
        assert a <= 448.0 * 2.0 ** e and a > 448.0 * 2.0 ** (e - 1)
        for k in (-5, 3):
            assert M.p_block_exponent(float(a) * 2.0 ** k) == e + k
    assert M.p_block_exponent(2.0 ** -101) is None and M.p_block_exponent(0.0) is None


# ---------------------------------------------------------------------------
# attention
# ---------------------------------------------------------------------------

_TABLE = None


def _round_by_table(y: float) -> float:
    """E4M3 rounding by search over the value table (ties to the even code)."""
    global _TABLE
    if _TABLE is None:
        codes = np.arange(0, 127)
        _TABLE = (codes, _torch_decode(codes.astype(np.uint8)))
    codes, vals = _TABLE
    a = min(abs(y), 448.0)
    dist = np.abs(vals - a)
    best = np.flatnonzero(dist == dist.min())
    pick = best[0] if len(best) == 1 else [b for b in best if codes[b] % 2 == 0][0]
    return math.copysign(float(vals[pick]), y)


def _brute_force(w, c, r, h, planted=None):
    """One output row by scalar loops over the pages' definitions."""
    offs = w.user_offsets
    u = int(w.cand_to_user[c])
    a, b = int(offs[u]), int(offs[u + 1])
    d = w.d
    if b == a:
        return np.zeros(d)
    dq = _torch_decode(w.q_codes[c, r, h])
    qv = [dq[i] * 2.0 ** (int(w.q_scales[c, r, h, i // 32]) - 127) for i in range(d)]
    xs = []
    for t in range(a, b):
        dk = _torch_decode(w.k_codes[t, h])
        kv = [dk[i] * 2.0 ** (int(w.k_scales[t, h, i // 32]) - 127) for i in range(d)]
        xs.append(float(np.float32(w.scale)) * M.LOG2E * math.fsum(qv[i] * kv[i] for i in range(d)))
    m = math.ceil(max(xs))
    p = [2.0 ** (x - m) for x in xs]
    ph = [0.0] * len(p)
    for j0 in range(0, len(p), 32):
        blk = p[j0:j0 + 32]
        amax = max(blk)
        if amax < 2.0 ** -100:
            continue
        if planted == "floor_scale_rule":  # the shared-exponent rule that saturates the top binade
            e = math.floor(math.log2(amax)) - 8
        else:
            e = math.ceil(math.log2(amax / 448.0))
            while amax > 448.0 * 2.0 ** e:  # guard the log's rounding
                e += 1
            while amax <= 448.0 * 2.0 ** (e - 1):
                e -= 1
        for j in range(j0, min(j0 + 32, len(p))):
            ph[j] = _round_by_table(p[j] / 2.0 ** e) * 2.0 ** e
    l = math.fsum(ph) if planted == "quantized_row_sum" else math.fsum(p)
    vbo = w.v_block_offsets
    out = np.zeros(d)
    for col in range(d):
        terms = []
        for j, t in enumerate(range(a, b)):
            blk = (t // 32) if planted == "global_v_blocks" else int(vbo[u]) + j // 32
            blk = min(blk, w.v_scales.shape[0] - 1)
            vv = _torch_decode(w.v_codes[t, h, col:col + 1])[0] * 2.0 ** (int(w.v_scales[blk, h, col]) - 127)
            terms.append(ph[j] * vv)
        out[col] = math.fsum(terms) / l
    return out


def _oracle(w, **kw):
    return M.target_attention_mxfp8(*w.arrays(), w.user_offsets, w.cand_to_user, w.scale, **kw)


def test_brute_force_scalar_loops_on_the_tiny_config():
    w = make_mxfp8("mx_tiny")
    got = _oracle(w)
    for c in range(w.n_cand):
        for r in range(w.n_q):
            for h in range(w.H):
                ref = _brute_force(w, c, r, h)
                np.testing.assert_allclose(got[c, r, h], ref, rtol=1e-12, atol=1e-12)


def test_invariant_to_the_integer_softmax_reference():
    """Moving the integer reference by k scales every p by 2^-k; the block
    scales follow and the codes do not change, so the output is the same up to
    the fp64 rounding of x - m (a rule that did not follow powers of two would
    move outputs by up to 2^-4 of |v|).  References below the maximum (weights
    up to 2^8) are what a kernel with a lagging reference uses."""
    w = make_mxfp8("mx_tiny")
    base = _oracle(w)
    for k in (-8, -3, 1, 3, 17):
        np.testing.assert_allclose(_oracle(w, m_shift=k), base, rtol=1e-12, atol=1e-14)


def test_error_bound_against_unquantized_attention():
    """P^_j = p_j (1 + d_j) with |d_j| <= 2^-4 for every weight above the block's
    subnormal range, so |O_mx - O| <= (2^-4 + tail) * max|v| per row, O being
    exact softmax attention on the same dequantized inputs."""
    w = make_mxfp8("mx_tiny")
    q = M.dequantize_rows(w.q_codes, w.q_scales)
    k = M.dequantize_rows(w.k_codes, w.k_scales)
    v = M.dequantize_v(w.v_codes, w.v_scales, w.user_offsets)
    exact = O.target_attention(q, k, v, w.user_offsets, w.cand_to_user, w.scale)
    got = _oracle(w)
    for c in range(w.n_cand):
        u = int(w.cand_to_user[c])
        a, b = int(w.user_offsets[u]), int(w.user_offsets[u + 1])
        if b == a:
            assert np.all(got[c] == 0)
            continue
        vmax = np.abs(v[a:b]).max(axis=(0, 2))  # per head
        nblk = (b - a + 31) // 32
        bound = (2.0 ** -4 + 1e-3 * nblk) * vmax
        err = np.abs(got[c] - exact[c]).max(axis=(0, 2))
        assert np.all(err <= bound), (c, err, bound)
    assert np.abs(got - exact).mean() < 2.0 ** -5 * np.abs(v).mean()  # mean E4M3 rounding is about a quarter ulp


def test_zero_scale_gives_the_mean_of_v():
    """scale 0: every x is 0, p = 1 exactly (representable), so the output is
    the plain mean of the user's dequantized values."""
    w = make_mxfp8_custom(7, (3, 40, 70), [0, 1, 2, 1], n_q=1, H=2)
    w.scale = np.float32(0.0)
    got = _oracle(w)
    v = M.dequantize_v(w.v_codes, w.v_scales, w.user_offsets)
    for c in range(w.n_cand):
        u = int(w.cand_to_user[c])
        a, b = int(w.user_offsets[u]), int(w.user_offsets[u + 1])
        np.testing.assert_allclose(got[c, 0], v[a:b].mean(axis=0), rtol=1e-13, atol=1e-15)


def test_single_key_user_is_a_scaled_copy_of_its_value():
    """One key: O = (P^ / p) v^ with P^ / p within 2^-4 of one, the same factor
    for every column."""
    w = make_mxfp8_custom(9, (1, 50), [0, 0, 1], n_q=2, H=2)
    got = _oracle(w)
    v = M.dequantize_v(w.v_codes, w.v_scales, w.user_offsets)
    for c in (0, 1):
        for r in range(2):
            for h in range(2):
                ratio = got[c, r, h] / v[0, h]
                assert np.allclose(ratio, ratio[0], rtol=1e-13) and abs(ratio[0] - 1.0) <= 2.0 ** -4


def test_v_blocks_belong_to_their_user():
    """Changing one V-scale block of user u changes only u's candidates, and
    only when u has a key in that block."""
    w = make_mxfp8("mx_tiny")
    base = _oracle(w)
    u = 4                                    # 70 keys: blocks vbo[4] .. vbo[4] + 2
    blk = int(w.v_block_offsets[u]) + 2
    w.v_scales = w.v_scales.copy()
    w.v_scales[blk] += 1
    got = _oracle(w)
    mine = w.cand_to_user == u
    assert np.all(got[~mine] == base[~mine])
    assert np.abs(got[mine] - base[mine]).max() > 0


def test_candidate_permutation_permutes_outputs():
    w = make_mxfp8("mx_tiny")
    base = _oracle(w)
    perm = np.random.default_rng(3).permutation(w.n_cand)
    w.cand_to_user = w.cand_to_user[perm]
    w.q_codes, w.q_scales = w.q_codes[perm], w.q_scales[perm]
    assert np.array_equal(_oracle(w), base[perm])


@pytest.mark.parametrize("mistake", ["global_v_blocks", "quantized_row_sum", "floor_scale_rule"])
def test_planted_mistakes_fail_the_brute_force(mistake):
    w = make_mxfp8("mx_tiny")
    got = _oracle(w)
    worst = 0.0
    for c in range(w.n_cand):
        u = int(w.cand_to_user[c])
        if w.lengths[u] < 2:
            continue
        for h in range(w.H):
            worst = max(worst, float(np.abs(_brute_force(w, c, 0, h, planted=mistake) - got[c, 0, h]).max()))
    assert worst > 1e-3, worst


def test_per_user_calls_assemble_the_whole_call():
    """Users do not interact: one call per user (its candidates, its key and
    value rows, its value-scale blocks, offsets [0, L]) placed back together
    gives the whole call's output bit for bit."""
    w = make_mxfp8("mx_tiny")
    whole = M.target_attention_mxfp8(*w.arrays(), w.user_offsets, w.cand_to_user, w.scale)
    vbo = M.v_block_offsets(w.user_offsets)
    out = np.zeros_like(whole)
    for u in range(w.n_users):
        cands = np.flatnonzero(w.cand_to_user == u)
        a, b = int(w.user_offsets[u]), int(w.user_offsets[u + 1])
        out[cands] = M.target_attention_mxfp8(w.q_codes[cands], w.q_scales[cands], w.k_codes[a:b],
                                              w.k_scales[a:b], w.v_codes[a:b], w.v_scales[vbo[u]:vbo[u + 1]],
                                              np.array([0, b - a], np.int32), np.zeros(len(cands), np.int32),
                                              w.scale)
    assert np.array_equal(out, whole)
