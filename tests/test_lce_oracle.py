"""Pins of the LCE oracle (CPU): brute force, the pages' equivalences, closed forms.

Sources: IKBO blog section 2.1 and Fig. 2 (the batched projection and its split
along K), section 2.2 and Proof 1 (zero padding of each decomposed K), App. 2
(the FLOP and byte counts behind the printed arithmetic intensity of 356).
"""

import math

import numpy as np
import pytest

from oracle import ikbo_oracle as O
from oracle import lce_oracle as L
from workloads import make_lce, make_lce_custom


def _vals(w):
    return w.values("w"), w.values("x_user"), w.values("x_cand"), w.cand_to_user


def test_brute_force_scalar_loops():
    w = make_lce_custom(7, 2, [1, 0, 1, 1], M=5, K_u=3, K_c=4, N=6)
    W, xu, xc, c2u = _vals(w)
    got = L.lce_baseline(W, xu, xc, c2u)
    for b in range(4):
        u = int(c2u[b])
        for m in range(5):
            for n in range(6):
                terms = [float(W[m, k]) * float(xu[u, k, n]) for k in range(3)]
                terms += [float(W[m, 3 + k]) * float(xc[b, k, n]) for k in range(4)]
                assert got[b, m, n] == pytest.approx(math.fsum(terms), rel=1e-13, abs=1e-13)


def test_brute_force_on_tiny_config_sample():
    w = make_lce("lce_tiny")
    W, xu, xc, c2u = _vals(w)
    got = L.lce_baseline(W, xu, xc, c2u)
    rng = np.random.default_rng(0)
    for _ in range(300):
        b, m, n = rng.integers(w.n_cand), rng.integers(w.M), rng.integers(w.N)
        u = int(c2u[b])
        ref = math.fsum([float(W[m, k]) * float(xu[u, k, n]) for k in range(w.K_u)] +
                        [float(W[m, w.K_u + k]) * float(xc[b, k, n]) for k in range(w.K_c)])
        assert got[b, m, n] == pytest.approx(ref, rel=1e-12, abs=1e-12)


def test_split_along_k_equals_the_batched_product():
    """Section 2.1: with W split into user and candidate columns, the user
    product at the user batch plus the candidate product equals the baseline."""
    w = make_lce("lce_tiny")
    W, xu, xc, c2u = _vals(w)
    base = L.lce_baseline(W, xu, xc, c2u)
    Wu, Wc = W[:, :w.K_u].astype(np.float64), W[:, w.K_u:].astype(np.float64)
    yu = np.einsum("mk,ukn->umn", Wu, xu.astype(np.float64))     # user batch only
    dec = np.einsum("mk,bkn->bmn", Wc, xc.astype(np.float64)) + yu[c2u]
    np.testing.assert_allclose(dec, base, rtol=1e-12, atol=1e-12)


def test_zero_padding_each_k_is_exact():
    """Section 2.2, Proof 1: zero-padding K_u and K_c to multiples of 8 leaves the
    product unchanged."""
    w = make_lce("lce_tiny")
    W, xu, xc, c2u = _vals(w)
    pu, pc = (-w.K_u) % 8, (-w.K_c) % 8
    assert pu and pc
    Wp = np.concatenate([W[:, :w.K_u], np.zeros((w.M, pu), np.float32), W[:, w.K_u:],
                         np.zeros((w.M, pc), np.float32)], axis=1)
    xup = np.concatenate([xu, np.zeros((w.n_users, pu, w.N), np.float32)], axis=1)
    xcp = np.concatenate([xc, np.zeros((w.n_cand, pc, w.N), np.float32)], axis=1)
    np.testing.assert_allclose(L.lce_baseline(Wp, xup, xcp, c2u), L.lce_baseline(W, xu, xc, c2u),
                               rtol=1e-13, atol=1e-13)


def test_identity_projection_returns_the_concatenation():
    U, B, K_u, K_c, N = 2, 3, 4, 3, 5
    w = make_lce_custom(9, U, [1, 1, 0], M=K_u + K_c, K_u=K_u, K_c=K_c, N=N)
    xu, xc = w.values("x_user"), w.values("x_cand")
    got = L.lce_baseline(np.eye(K_u + K_c), xu, xc, w.cand_to_user)
    for b in range(B):
        assert np.array_equal(got[b], np.concatenate([xu[w.cand_to_user[b]], xc[b]]).astype(np.float64))


def test_candidate_permutation_and_shared_inputs():
    w = make_lce("lce_tiny")
    W, xu, xc, c2u = _vals(w)
    base = L.lce_baseline(W, xu, xc, c2u)
    p = np.random.default_rng(3).permutation(w.n_cand)
    assert np.array_equal(L.lce_baseline(W, xu, xc[p], c2u[p]), base[p])
    # two candidates of one user with the same own embeddings get the same rows
    xc2 = xc.copy()
    same = np.where(c2u == c2u[0])[0]
    assert len(same) >= 2
    xc2[same[1]] = xc2[same[0]]
    out = L.lce_baseline(W, xu, xc2, c2u)
    assert np.array_equal(out[same[0]], out[same[1]])


@pytest.mark.parametrize("mistake", ["wrong_user", "no_user_block", "swapped_columns"])
def test_planted_mistakes_fail_the_brute_force(mistake):
    w = make_lce_custom(11, 3, [2, 0, 1, 2], M=4, K_u=3, K_c=2, N=3)
    W, xu, xc, c2u = _vals(w)
    W64, xu64, xc64 = W.astype(np.float64), xu.astype(np.float64), xc.astype(np.float64)
    bad = np.empty((4, 4, 3))
    for b in range(4):
        u = int(c2u[b])
        if mistake == "wrong_user":
            xb = np.concatenate([xu64[(u + 1) % 3], xc64[b]])
            bad[b] = W64 @ xb
        elif mistake == "no_user_block":
            bad[b] = W64[:, 3:] @ xc64[b]
        else:
            bad[b] = np.concatenate([W64[:, 2:], W64[:, :2]], axis=1) @ np.concatenate([xu64[u], xc64[b]])
    brute = np.empty((4, 4, 3))
    for b in range(4):
        for m in range(4):
            for n in range(3):
                brute[b, m, n] = math.fsum([W[m, k] * xu[c2u[b], k, n] for k in range(3)] +
                                           [W[m, 3 + k] * xc[b, k, n] for k in range(2)])
    np.testing.assert_allclose(L.lce_baseline(W, xu, xc, c2u), brute, rtol=1e-12, atol=1e-12)
    assert np.max(np.abs(bad - brute)) > 1e-3


def test_printed_arithmetic_intensity_and_user_side_saving():
    """App. 2: the batched product's intensity is about 356 FLOP/B at B=1024,
    M=433, K=2044, N=256; section 2.1: the user side shrinks by the ratio."""
    B, M, K, N = 1024, 433, 2044, 256
    ai = L.lce_flops_baseline(B, M, K, N) / L.lce_bytes_baseline(B, M, K, N)
    assert int(ai) == 356  # printed as about 356 (356.8 truncated)
    assert ai == pytest.approx(O.ai_gemm(B, M, K, N), rel=1e-12)
    K_u = K_c = 1022
    full_user = 2.0 * M * N * B * K_u
    ikbo_user = L.lce_flops_ikbo(B, 15, M, K_u, K_c, N) - 2.0 * M * N * B * K_c
    assert full_user / ikbo_user == pytest.approx(1024 / 15)


# ---- three levels: user -> vendor -> item (IKBO blog, conclusion) ----

from workloads import make_lce_nested, make_lce_nested_custom  # noqa: E402


def _nested_small(seed=31, K_v=4):
    v2u = np.array([1, 0, 1, 1, 0], np.int32)
    c2v = np.array([3, 0, 4, 4, 1, 2, 0], np.int32)
    return make_lce_nested_custom(seed, 2, v2u, c2v, M=5, K_u=3, K_v=K_v, K_c=2, N=6)


def _nested_vals(w):
    return (w.values("w"), w.values("x_user"), w.values("x_vendor"), w.values("x_cand"), w.vendor_to_user,
            w.cand_to_vendor)


def test_nested_brute_force_scalar_loops():
    w = _nested_small()
    W, xu, xv, xc, v2u, c2v = _nested_vals(w)
    got = L.lce_baseline_nested(W, xu, xv, xc, v2u, c2v)
    for b in range(w.n_cand):
        v = int(c2v[b])
        u = int(v2u[v])
        for m in range(w.M):
            for n in range(w.N):
                terms = [float(W[m, k]) * float(xu[u, k, n]) for k in range(w.K_u)]
                terms += [float(W[m, w.K_u + k]) * float(xv[v, k, n]) for k in range(w.K_v)]
                terms += [float(W[m, w.K_u + w.K_v + k]) * float(xc[b, k, n]) for k in range(w.K_c)]
                assert got[b, m, n] == pytest.approx(math.fsum(terms), rel=1e-13, abs=1e-13)


def test_nested_without_vendor_block_is_two_levels():
    w = _nested_small(K_v=0)
    W, xu, xv, xc, v2u, c2v = _nested_vals(w)
    got = L.lce_baseline_nested(W, xu, xv, xc, v2u, c2v)
    ref = L.lce_baseline(W, xu, xc, v2u[c2v])
    np.testing.assert_allclose(got, ref, rtol=1e-13, atol=1e-13)


def test_nested_decomposition_equals_the_batched_product():
    """Each level at its own batch, the parent's result added: users, then
    vendors (plus their user's result), then items (plus their vendor's)."""
    w = make_lce_nested("lce3_tiny")
    W, xu, xv, xc, v2u, c2v = (a.astype(np.float64) if a.dtype.kind == "f" else a for a in _nested_vals(w))
    base = L.lce_baseline_nested(W, xu, xv, xc, v2u, c2v)
    Wu, Wv, Wc = W[:, :w.K_u], W[:, w.K_u:w.K_u + w.K_v], W[:, w.K_u + w.K_v:]
    yu = np.einsum("mk,ukn->umn", Wu, xu)
    yv = np.einsum("mk,vkn->vmn", Wv, xv) + yu[v2u]
    dec = np.einsum("mk,bkn->bmn", Wc, xc) + yv[c2v]
    np.testing.assert_allclose(dec, base, rtol=1e-12, atol=1e-12)


def test_nested_relabelling_and_permutation():
    w = make_lce_nested("lce3_tiny")
    W, xu, xv, xc, v2u, c2v = _nested_vals(w)
    base = L.lce_baseline_nested(W, xu, xv, xc, v2u, c2v)
    rng = np.random.default_rng(4)
    pv = rng.permutation(w.n_vendors)           # new vendor id of old vendor i is inv[i]
    inv = np.argsort(pv)
    got = L.lce_baseline_nested(W, xu, xv[pv], xc, v2u[pv], inv[c2v])
    assert np.array_equal(got, base)
    pb = rng.permutation(w.n_cand)
    got = L.lce_baseline_nested(W, xu, xv, xc[pb], v2u, c2v[pb])
    assert np.array_equal(got, base[pb])


@pytest.mark.parametrize("mistake", ["item_index_as_vendor_user", "no_vendor_block", "wrong_vendor"])
def test_nested_planted_mistakes_fail_the_brute_force(mistake):
    w = _nested_small()
    W, xu, xv, xc, v2u, c2v = _nested_vals(w)
    bad = np.empty((w.n_cand, w.M, w.N))
    for b in range(w.n_cand):
        v = int(c2v[b])
        u = int(v2u[v]) if mistake != "item_index_as_vendor_user" else int(c2v[b]) % w.n_users
        blocks = [xu[u], xv[v], xc[b]]
        if mistake == "no_vendor_block":
            blocks[1] = np.zeros_like(xv[v])
        if mistake == "wrong_vendor":
            blocks[1] = xv[(v + 1) % w.n_vendors]
        bad[b] = W @ np.concatenate(blocks)
    ref = L.lce_baseline_nested(W, xu, xv, xc, v2u, c2v)
    assert np.abs(bad - ref).max() > 1e-3
