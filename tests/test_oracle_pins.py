"""Pins of the fp64 oracle against facts it does not compute itself.

Each test states the fact that pins it: brute-force scalar loops, closed forms,
invariances of softmax attention, torch's SDPA as an independent library
implementation, and the figures the IKBO blog prints for its roofline model.
None of these re-types the oracle's own formula.
"""

import math

import numpy as np
import pytest
import torch

from oracle import ikbo_oracle as O
from workloads import make_custom, make_workload

GOLDEN = __file__.rsplit("/", 1)[0] + "/golden/page_closed_forms.txt"


def _tiny(seed=7, lengths=(5, 9, 3), c2u=(2, 0, 1, 0, 2, 2), n_q=2, H=2, d=8, scale=None):
    rng = np.random.default_rng(seed)
    L = np.asarray(lengths)
    offs = np.concatenate([[0], np.cumsum(L)]).astype(np.int32)
    T = int(offs[-1])
    c2u = np.asarray(c2u, dtype=np.int32)
    q = rng.standard_normal((len(c2u), n_q, H, d))
    k = rng.standard_normal((T, H, d))
    v = rng.standard_normal((T, H, d))
    sc = np.float32(1.0 / math.sqrt(d)) if scale is None else np.float32(scale)
    return q, k, v, offs, c2u, sc


def _brute_force(q, k, v, offs, c2u, scale):
    """Scalar loops with Python floats and math.exp (the pages' definition, written out)."""
    C, n_q, H, d = q.shape
    sc = float(np.float32(scale))
    out = np.zeros((C, n_q, H, d))
    for c in range(C):
        u = int(c2u[c])
        lo, hi = int(offs[u]), int(offs[u + 1])
        for i in range(n_q):
            for h in range(H):
                if hi == lo:
                    continue
                s = []
                for j in range(lo, hi):
                    acc = 0.0
                    for e in range(d):
                        acc += float(q[c, i, h, e]) * float(k[j, h, e])
                    s.append(sc * acc)
                mx = max(s)
                w = [math.exp(x - mx) for x in s]
                tot = math.fsum(w)
                for e in range(d):
                    out[c, i, h, e] = math.fsum(w[jj] * float(v[j, h, e]) for jj, j in enumerate(range(lo, hi))) / tot
    return out


def _brute_force_self(q, k, v, offs, scale):
    T, H, d = q.shape
    sc = float(np.float32(scale))
    out = np.zeros((T, H, d))
    for u in range(len(offs) - 1):
        lo, hi = int(offs[u]), int(offs[u + 1])
        for t in range(hi - lo):
            for h in range(H):
                s = [sc * sum(float(q[lo + t, h, e]) * float(k[lo + j, h, e]) for e in range(d)) for j in range(t + 1)]
                mx = max(s)
                w = [math.exp(x - mx) for x in s]
                tot = math.fsum(w)
                for e in range(d):
                    out[lo + t, h, e] = math.fsum(w[j] * float(v[lo + j, h, e]) for j in range(t + 1)) / tot
    return out


# P1 -------------------------------------------------------------------------
@pytest.mark.parametrize("seed", [1, 2, 3])
def test_p1_brute_force_tiny(seed):
    q, k, v, offs, c2u, sc = _tiny(seed=seed)
    ref = _brute_force(q, k, v, offs, c2u, sc)
    got = O.target_attention(q, k, v, offs, c2u, sc)
    assert np.max(np.abs(got - ref)) <= 1e-12


def test_p1_brute_force_config1():
    w = make_workload("c1_tiny_f32")
    q, k, v = w.values("q_cand"), w.values("k_user"), w.values("v_user")
    ref = _brute_force(q, k, v, w.user_offsets, w.cand_to_user, w.scale)
    got = O.target_attention(q, k, v, w.user_offsets, w.cand_to_user, w.scale)
    assert np.max(np.abs(got - ref)) <= 1e-12


def test_p1_brute_force_self():
    q, k, v, offs, c2u, sc = _tiny(seed=11, lengths=(4, 7, 1, 3))
    qu = np.random.default_rng(5).standard_normal(k.shape)
    ref = _brute_force_self(qu, k, v, offs, sc)
    got = O.self_attention_causal(qu, k, v, offs, sc)
    assert np.max(np.abs(got - ref)) <= 1e-12


def test_rows_and_subset_agree_with_full():
    q, k, v, offs, c2u, sc = _tiny(seed=4)
    full = O.target_attention(q, k, v, offs, c2u, sc)
    rows = [(0, 1, 1), (3, 0, 0), (5, 1, 0)]
    got = O.target_attention_rows(q, k, v, offs, c2u, sc, rows)
    for n, (c, i, h) in enumerate(rows):
        # same definition on a narrower BLAS shape: equal up to summation order
        assert np.max(np.abs(got[n] - full[c, i, h])) <= 1e-14
    sub = O.target_attention(q, k, v, offs, c2u, sc, cands=[4, 1])
    assert np.array_equal(sub[0], full[4]) and np.array_equal(sub[1], full[1])
    qu = np.random.default_rng(9).standard_normal(k.shape)
    fs = O.self_attention_causal(qu, k, v, offs, sc)
    srows = [(0, 0, 0), (1, 8, 1), (2, 2, 0)]
    gs = O.self_attention_rows(qu, k, v, offs, sc, srows)
    for n, (u, t, h) in enumerate(srows):
        assert np.allclose(gs[n], fs[offs[u] + t, h], atol=1e-14, rtol=0)


# P2 -------------------------------------------------------------------------
def test_p2_constant_keys_give_mean_of_v():
    q, k, v, offs, c2u, sc = _tiny(seed=3)
    k[:] = k[0]  # every key identical
    got = O.target_attention(q, k, v, offs, c2u, sc)
    for c, u in enumerate(c2u):
        lo, hi = offs[u], offs[u + 1]
        assert np.max(np.abs(got[c] - v[lo:hi].mean(axis=0)[None])) <= 1e-14


# P3 -------------------------------------------------------------------------
def test_p3_single_key_returns_v0():
    q, k, v, offs, c2u, sc = _tiny(seed=5, lengths=(1, 1, 4), c2u=(0, 1, 1, 2, 0))
    got = O.target_attention(q, k, v, offs, c2u, sc)
    for c, u in enumerate(c2u):
        if offs[u + 1] - offs[u] == 1:
            assert np.array_equal(got[c], np.broadcast_to(v[offs[u]], got[c].shape))
    qu = np.random.default_rng(1).standard_normal(k.shape)
    so = O.self_attention_causal(qu, k, v, offs, sc)
    for u in range(3):
        assert np.array_equal(so[offs[u]], v[offs[u]])  # row t=0 sees only key 0


# P4 -------------------------------------------------------------------------
def test_p4_zero_scale_gives_mean():
    q, k, v, offs, c2u, _ = _tiny(seed=6)
    got = O.target_attention(q, k, v, offs, c2u, 0.0)
    for c, u in enumerate(c2u):
        assert np.max(np.abs(got[c] - v[offs[u]:offs[u + 1]].mean(axis=0)[None])) <= 1e-14


# P5 -------------------------------------------------------------------------
def test_p5_convex_combination_bounds():
    w = make_workload("c1_tiny_f32")
    q, k, v = w.values("q_cand"), w.values("k_user"), w.values("v_user")
    got = O.target_attention(q, k, v, w.user_offsets, w.cand_to_user, w.scale)
    for c, u in enumerate(w.cand_to_user):
        vs = v[w.user_offsets[u]:w.user_offsets[u + 1]].astype(np.float64)
        assert np.all(got[c] >= vs.min(axis=0)[None] - 1e-15)
        assert np.all(got[c] <= vs.max(axis=0)[None] + 1e-15)


# P6 -------------------------------------------------------------------------
def test_p6_candidate_permutation_invariance():
    q, k, v, offs, c2u, sc = _tiny(seed=8, c2u=(2, 0, 1, 0, 2, 2, 1, 0))
    perm = np.random.default_rng(0).permutation(len(c2u))
    a = O.target_attention(q, k, v, offs, c2u, sc)
    b = O.target_attention(q[perm], k, v, offs, c2u[perm], sc)
    assert np.array_equal(a[perm], b)


# P7 -------------------------------------------------------------------------
def test_p7_broadcast_equals_index_based():
    q, k, v, offs, c2u, sc = _tiny(seed=9, n_q=3)
    got = O.target_attention(q, k, v, offs, c2u, sc)
    # independent evaluation: gather by index, mask the jagged tail, einsum; no copies per candidate
    L = np.diff(offs)
    Lmax = int(L.max())
    idx = offs[c2u][:, None] + np.arange(Lmax)[None, :]
    valid = np.arange(Lmax)[None, :] < L[c2u][:, None]
    idx = np.where(valid, idx, 0)
    kb, vb = k[idx], v[idx]                                  # [C, Lmax, H, d] (gather)
    s = float(np.float32(sc)) * np.einsum("cihe,cjhe->chij", q, kb)
    s = np.where(valid[:, None, None, :], s, -np.inf)
    p = np.exp(s - s.max(-1, keepdims=True))
    p = p / p.sum(-1, keepdims=True)
    ref = np.einsum("chij,cjhe->cihe", p, vb)
    assert np.max(np.abs(got - ref)) <= 1e-15 * 10


# P8 -------------------------------------------------------------------------
def test_p8_duplicated_sequence_invariance():
    q, k, v, offs, c2u, sc = _tiny(seed=10)
    a = O.target_attention(q, k, v, offs, c2u, sc)
    ks, vs, L = [], [], []
    for u in range(len(offs) - 1):
        seg_k, seg_v = k[offs[u]:offs[u + 1]], v[offs[u]:offs[u + 1]]
        ks += [seg_k, seg_k]
        vs += [seg_v, seg_v]
        L.append(2 * (offs[u + 1] - offs[u]))
    offs2 = np.concatenate([[0], np.cumsum(L)]).astype(np.int32)
    b = O.target_attention(q, np.concatenate(ks), np.concatenate(vs), offs2, c2u, sc)
    assert np.max(np.abs(a - b)) <= 1e-14


# P9 -------------------------------------------------------------------------
def test_p9_key_shift_invariance():
    q, k, v, offs, c2u, sc = _tiny(seed=12)
    a = O.target_attention(q, k, v, offs, c2u, sc)
    delta = np.random.default_rng(3).standard_normal(k.shape[1:])  # same shift for every key (per head)
    b = O.target_attention(q, k + delta[None], v, offs, c2u, sc)
    assert np.max(np.abs(a - b)) <= 1e-12


# P10 ------------------------------------------------------------------------
def test_p10_v_affine_equivariance():
    q, k, v, offs, c2u, sc = _tiny(seed=13)
    rng = np.random.default_rng(4)
    A = rng.standard_normal((v.shape[-1], v.shape[-1]))
    bvec = rng.standard_normal(v.shape[-1])
    a = O.target_attention(q, k, v, offs, c2u, sc)
    b = O.target_attention(q, k, v @ A + bvec, offs, c2u, sc)
    assert np.max(np.abs(a @ A + bvec - b)) <= 1e-12


# P11 ------------------------------------------------------------------------
def test_p11_identity_mapping_equals_torch_sdpa():
    B, H, n_q, L, d = 5, 3, 4, 11, 16
    rng = np.random.default_rng(14)
    q = rng.standard_normal((B, n_q, H, d))
    k = rng.standard_normal((B * L, H, d))
    v = rng.standard_normal((B * L, H, d))
    offs = (np.arange(B + 1) * L).astype(np.int32)
    c2u = np.arange(B, dtype=np.int32)
    sc = np.float32(0.3)
    got = O.target_attention(q, k, v, offs, c2u, sc)
    tq = torch.from_numpy(q).permute(0, 2, 1, 3)                        # [B, H, n_q, d]
    tk = torch.from_numpy(k.reshape(B, L, H, d)).permute(0, 2, 1, 3)
    tv = torch.from_numpy(v.reshape(B, L, H, d)).permute(0, 2, 1, 3)
    ref = torch.nn.functional.scaled_dot_product_attention(tq, tk, tv, scale=float(sc))
    assert np.max(np.abs(got - ref.permute(0, 2, 1, 3).numpy())) <= 1e-12


def test_p11_self_causal_equals_torch_sdpa_causal():
    lengths = (6, 1, 13)
    rng = np.random.default_rng(15)
    offs = np.concatenate([[0], np.cumsum(lengths)]).astype(np.int32)
    H, d = 2, 8
    q = rng.standard_normal((offs[-1], H, d))
    k = rng.standard_normal((offs[-1], H, d))
    v = rng.standard_normal((offs[-1], H, d))
    sc = np.float32(0.25)
    got = O.self_attention_causal(q, k, v, offs, sc)
    for u in range(len(lengths)):
        lo, hi = offs[u], offs[u + 1]
        t = lambda x: torch.from_numpy(x[lo:hi]).permute(1, 0, 2)[None]  # noqa: E731
        ref = torch.nn.functional.scaled_dot_product_attention(t(q), t(k), t(v), is_causal=True, scale=float(sc))
        assert np.max(np.abs(got[lo:hi] - ref[0].permute(1, 0, 2).numpy())) <= 1e-12


# P12 ------------------------------------------------------------------------
def test_p12_two_key_closed_form():
    q, k, v, offs, c2u, sc = _tiny(seed=16, lengths=(2, 2), c2u=(0, 1, 1, 0))
    got = O.target_attention(q, k, v, offs, c2u, sc)
    s_ = float(np.float32(sc))
    for c, u in enumerate(c2u):
        j0, j1 = offs[u], offs[u] + 1
        for i in range(q.shape[1]):
            for h in range(q.shape[2]):
                s0 = s_ * float(q[c, i, h] @ k[j0, h])
                s1 = s_ * float(q[c, i, h] @ k[j1, h])
                sig = 1.0 / (1.0 + math.exp(-(s0 - s1)))
                ref = sig * v[j0, h] + (1.0 - sig) * v[j1, h]
                assert np.max(np.abs(got[c, i, h] - ref)) <= 1e-14


# zero-length users and empty inputs (readings where the pages are silent) --
def test_zero_length_user_gives_zero_rows():
    q, k, v, offs, c2u, sc = _tiny(seed=17, lengths=(3, 0, 4), c2u=(1, 0, 1, 2))
    got = O.target_attention(q, k, v, offs, c2u, sc)
    assert np.all(got[0] == 0) and np.all(got[2] == 0)
    assert np.all(np.isfinite(got))


def test_empty_candidate_batch():
    q, k, v, offs, _, sc = _tiny(seed=18)
    got = O.target_attention(q[:0], k, v, offs, np.zeros(0, np.int32), sc)
    assert got.shape == (0,) + q.shape[1:]


# P16 ------------------------------------------------------------------------
def test_p16_split_kv_merge_equals_unsplit():
    rng = np.random.default_rng(19)
    n_q, H, d, L = 3, 2, 16, 37
    q = rng.standard_normal((n_q, H, d)) * 3.0
    k = rng.standard_normal((L, H, d))
    v = rng.standard_normal((L, H, d))
    offs = np.array([0, L], np.int32)
    full = O.target_attention(q[None], k, v, offs, np.zeros(1, np.int32), 0.5)[0]
    for cuts in ([0, 37], [0, 10, 37], [0, 1, 2, 20, 36, 37]):
        parts = [O.chunk_partial(q, k[a:b], v[a:b], 0.5) for a, b in zip(cuts[:-1], cuts[1:])]
        o, lse = O.merge_partials(parts)
        assert np.max(np.abs(o - full)) <= 1e-14
        # the merged lse is the log of the full partition function
        s = 0.5 * np.einsum("ihe,jhe->hij", q, k)
        assert np.max(np.abs(lse - np.log(np.exp(s).sum(-1)))) <= 1e-12


# P14 (oracle side; the C++ grouping is compared in test_library_cpu.py) -----
@pytest.mark.parametrize("n_q,bm", [(1, 128), (4, 128), (1, 32), (3, 7)])
def test_p14_csr_invariants(n_q, bm):
    rng = np.random.default_rng(20)
    U, C = 9, 200
    c2u = rng.integers(0, U - 2, size=C).astype(np.int32)  # last two users empty
    g = O.group_csr(c2u, U, n_q, bm)
    counts, co, perm, tiles = g["counts"], g["cand_offsets"], g["cand_perm"], g["tiles"]
    assert counts.sum() == C and co[0] == 0 and co[-1] == C and np.all(np.diff(co) >= 0)
    assert np.array_equal(np.sort(perm), np.arange(C))
    assert np.all(np.diff(c2u[perm]) >= 0)
    for u in range(U):
        seg = perm[co[u]:co[u + 1]]
        assert np.all(np.diff(seg) > 0) and np.all(c2u[seg] == u)
    covered = {u: np.zeros(counts[u] * n_q, int) for u in range(U)}
    for u, r0, n in tiles:
        assert 1 <= n <= bm
        covered[u][r0:r0 + n] += 1
    assert all(np.all(c == 1) for c in covered.values())
    assert np.all(np.diff(tiles[:, 0]) >= 0)


def test_validate_rules():
    offs = np.array([0, 3, 5], np.int32)
    O.validate(offs, np.array([0, 1, 1], np.int32), 2, 2, 128)
    cases = [
        (dict(user_offsets=np.array([1, 3, 5])), "bad_offsets"),
        (dict(user_offsets=np.array([0, 3, 2])), "bad_offsets"),
        (dict(cand_to_user=np.array([0, 2])), "bad_mapping"),
        (dict(cand_to_user=np.array([-1])), "bad_mapping"),
        (dict(d=48), "unsupported"),
        (dict(H=0), "invalid_arg"),
    ]
    for kw, code in cases:
        args = dict(user_offsets=offs, cand_to_user=np.array([0, 1]), n_users=2, H=2, d=128)
        args.update(kw)
        with pytest.raises(O.OracleInputError) as e:
            O.validate(**args)
        assert e.value.code == code


# P15: the measurement model against the blog's printed figures --------------
def _golden():
    rows = {}
    for line in open(GOLDEN):
        if line.startswith("#") or not line.strip():
            continue
        name, val, tol, inputs, _where = [x.strip() for x in line.split("|")]
        kv = dict(x.split("=") for x in inputs.replace(",", " ").split() if "=" in x)
        rows[name] = (float(val), float(tol), kv)
    return rows


def test_p15_page_printed_closed_forms():
    g = _golden()
    val, tol, kv = g["h100_balance"]
    assert abs(O.machine_balance(float(kv["peak"]), float(kv["bw"])) - val) <= tol
    val, tol, kv = g["lce_gemm_ai"]
    assert abs(O.ai_gemm(int(kv["B"]), int(kv["M"]), int(kv["K"]), int(kv["N"]), 2) - val) <= tol
    val, tol, kv = g["attn_standard_ai"]
    assert abs(O.ai_standard(int(kv["n"]), int(kv["L"])) - val) <= tol
    val, tol, kv = g["attn_ikbo_ai"]
    assert abs(O.ai_ikbo(int(kv["n"]), int(kv["L"]), float(kv["ratio"])) - val) <= tol


def test_p15_byte_and_flop_model_reproduce_ai():
    # The bench's FLOP and byte model reduces to the printed AI for one user.
    n, L, R, d = 64, 1024, 70, 128
    f = O.flops_target([R], [L], n, 1, d)
    b = O.bytes_ikbo(R, n, L, 1, d, 2)
    assert abs(f / b - O.ai_ikbo(n, L, R)) < 1e-9
    f1 = O.flops_target([1], [L], n, 1, d)
    b1 = O.bytes_ikbo(1, n, L, 1, d, 2)
    assert abs(f1 / b1 - O.ai_standard(n, L)) < 1e-9


# Planted mistakes: each plausible bug in the oracle fails at least one pin --
_ORIG_BROADCAST = O._broadcast_user_kv


def _mutants():
    def wrong_user(k_user, v_user, user_offsets, u):
        return _ORIG_BROADCAST(k_user, v_user, user_offsets, (u + 1) % (len(user_offsets) - 1))

    def transposed_scores(q, kc, scale):
        return scale * np.matmul(np.transpose(q, (1, 0, 2)), np.transpose(kc[:, ::-1, :], (1, 2, 0)))

    def dropped_scale(q, kc, scale):
        return np.matmul(np.transpose(q, (1, 0, 2)), np.transpose(kc, (1, 2, 0)))

    def wrong_sign(q, kc, scale):
        return -scale * np.matmul(np.transpose(q, (1, 0, 2)), np.transpose(kc, (1, 2, 0)))

    def no_normalise(s):
        return np.exp(s - np.max(s, axis=-1, keepdims=True))

    def off_by_one_key(k_user, v_user, user_offsets, u):
        lo, hi = int(user_offsets[u]), int(user_offsets[u + 1])
        return (np.array(k_user[lo:max(lo, hi - 1)], dtype=np.float64),
                np.array(v_user[lo:max(lo, hi - 1)], dtype=np.float64))

    return {
        "wrong_user": ("_broadcast_user_kv", wrong_user),
        "transposed_heads": ("_scores", transposed_scores),
        "dropped_scale": ("_scores", dropped_scale),
        "wrong_sign": ("_scores", wrong_sign),
        "no_normalise": ("_softmax_rows", no_normalise),
        "off_by_one_key": ("_broadcast_user_kv", off_by_one_key),
    }


@pytest.mark.parametrize("name", list(_mutants()))
def test_planted_mistakes_are_caught(monkeypatch, name):
    attr, fn = _mutants()[name]
    monkeypatch.setattr(O, attr, fn)
    q, k, v, offs, c2u, sc = _tiny(seed=21, lengths=(5, 9, 3, 6), c2u=(2, 0, 1, 0, 3, 2), H=3)
    ref = _brute_force(q, k, v, offs, c2u, sc)
    got = O.target_attention(q, k, v, offs, c2u, sc)
    assert not np.allclose(got, ref, atol=1e-12, rtol=0), f"mutant {name} slipped past the brute-force pin"


# log-sum-exp of the rows (the statistic a training forward keeps) ------------
def _brute_force_lse(q, k, offs, c2u, scale):
    """log(sum_j exp(s_j)) with Python floats: math.fsum of exp(s_j - max) plus the max."""
    C, n_q, H, d = q.shape
    sc = float(np.float32(scale))
    out = np.full((C, n_q, H), -np.inf)
    for c in range(C):
        u = int(c2u[c])
        lo, hi = int(offs[u]), int(offs[u + 1])
        for i in range(n_q):
            for h in range(H):
                if hi == lo:
                    continue
                s = [sc * math.fsum(float(q[c, i, h, e]) * float(k[j, h, e]) for e in range(d)) for j in range(lo, hi)]
                mx = max(s)
                out[c, i, h] = mx + math.log(math.fsum(math.exp(x - mx) for x in s))
    return out


@pytest.mark.parametrize("seed", [1, 2])
def test_lse_brute_force(seed):
    q, k, v, offs, c2u, sc = _tiny(seed=seed, lengths=(5, 0, 3, 1), c2u=(2, 0, 1, 3, 0, 2))
    ref = _brute_force_lse(q, k, offs, c2u, sc)
    got = O.target_attention_lse(q, k, offs, c2u, sc)
    finite = np.isfinite(ref)
    assert np.array_equal(finite, np.isfinite(got)) and np.all(got[~finite] == -np.inf)
    assert np.max(np.abs(got[finite] - ref[finite])) <= 1e-12


def test_lse_equals_library_logsumexp_and_normalises_the_weights():
    """scipy's logsumexp of the score matrix, and exp(s - lse) sums to one."""
    from scipy.special import logsumexp
    q, k, v, offs, c2u, sc = _tiny(seed=9, lengths=(40, 7), c2u=(1, 0, 0, 1), n_q=3, H=2, d=16)
    got = O.target_attention_lse(q, k, offs, c2u, sc)
    for c in range(len(c2u)):
        lo, hi = int(offs[c2u[c]]), int(offs[c2u[c] + 1])
        for i in range(3):
            for h in range(2):
                s = float(sc) * (k[lo:hi, h] @ q[c, i, h])
                assert abs(got[c, i, h] - logsumexp(s)) <= 1e-12
                assert abs(np.exp(s - got[c, i, h]).sum() - 1.0) <= 1e-12


def test_lse_closed_forms():
    """Equal scores give s + log L; one key gives its score; scale 0 gives log L."""
    q, k, v, offs, c2u, sc = _tiny(seed=4, lengths=(6, 1), c2u=(0, 1, 0), n_q=1, H=1, d=8)
    k[0:6] = k[0]  # user 0: six equal keys
    got = O.target_attention_lse(q, k, offs, c2u, sc)
    s0 = float(sc) * float(q[0, 0, 0] @ k[0, 0])
    assert abs(got[0, 0, 0] - (s0 + math.log(6))) <= 1e-12
    s1 = float(sc) * float(q[1, 0, 0] @ k[6, 0])
    assert abs(got[1, 0, 0] - s1) <= 1e-14
    z = O.target_attention_lse(q, k, offs, c2u, 0.0)
    assert abs(z[2, 0, 0] - math.log(6)) <= 1e-14


def test_lse_planted_mistakes_fail_the_brute_force():
    """Base-2 in place of natural log, a dropped scale, and the row maximum in
    place of the log-sum-exp all leave the brute force."""
    q, k, v, offs, c2u, sc = _tiny(seed=3)
    ref = _brute_force_lse(q, k, offs, c2u, sc)
    good = O.target_attention_lse(q, k, offs, c2u, sc)
    assert np.max(np.abs(good - ref)) <= 1e-12
    base2 = good / math.log(2)
    unscaled = O.target_attention_lse(q, k, offs, c2u, 1.0)
    rowmax = np.empty_like(good)
    for c in range(len(c2u)):
        lo, hi = int(offs[c2u[c]]), int(offs[c2u[c] + 1])
        rowmax[c] = np.transpose(np.max(float(sc) * np.einsum("ihe,jhe->hij", q[c], k[lo:hi]), axis=-1), (1, 0))
    for bad in (base2, unscaled, rowmax):
        assert np.max(np.abs(bad - ref)) > 1e-3
