"""Pins of the backward oracle (CPU).

Sources: the forward is IKBO target attention (IKBO blog, section 3.1, Fig. 10:
attention over an explicit per-candidate copy of the user's K/V); its gradient
is pinned here without re-typing the backward formulas: central finite
differences of the forward oracle, torch autograd in fp64, closed forms that
follow from softmax rows summing to one, and the linearity of the reduction
over a user's candidates.  Planted mistakes are rejected by the finite
differences.
"""

import numpy as np
import pytest

from oracle import ikbo_bwd_oracle as B
from oracle import ikbo_oracle as O
from workloads import add_output_grad, make_bwd_workload, make_custom


def _case(seed=11, lengths=(1, 4, 7, 0, 5), cand=(2, 1, 3, 2, 0), n_q=2, H=2, d=32):
    c2u = np.random.default_rng(seed).permutation(np.repeat(np.arange(len(lengths)), cand)).astype(np.int32)
    w = make_custom(seed, lengths, c2u, n_q=n_q, H=H, d=d, dtype="f32", name="bwd_pin")
    add_output_grad(w, seed + 1)
    return w


def _inputs(w):
    return (w.values("q_cand").astype(np.float64), w.values("k_user").astype(np.float64),
            w.values("v_user").astype(np.float64), w.values("dout").astype(np.float64))


def _loss(q, k, v, g, w):
    out = O.target_attention(q, k, v, w.user_offsets, w.cand_to_user, w.scale)
    return float(np.sum(out * g))


def _fd_check(w, grads, n_samples=60, h=1e-6, tol=1e-7):
    """Central differences of sum(out * dout) against given gradients, on
    random entries of q, k and v.  Returns the largest absolute mismatch."""
    q, k, v, g = _inputs(w)
    rng = np.random.default_rng(3)
    worst = 0.0
    for which, (x, gx) in enumerate(zip((q, k, v), grads)):
        flat = x.reshape(-1)
        for idx in rng.choice(flat.size, size=min(n_samples, flat.size), replace=False):
            keep = flat[idx]
            flat[idx] = keep + h
            lp = _loss(q, k, v, g, w)
            flat[idx] = keep - h
            lm = _loss(q, k, v, g, w)
            flat[idx] = keep
            fd = (lp - lm) / (2 * h)
            worst = max(worst, abs(fd - gx.reshape(-1)[idx]))
    return worst


def test_finite_differences_of_the_forward_oracle():
    w = _case()
    q, k, v, g = _inputs(w)
    grads = B.target_attention_bwd(q, k, v, g, w.user_offsets, w.cand_to_user, w.scale)
    assert _fd_check(w, grads) < 1e-7


def test_torch_autograd_on_the_explicit_copy():
    torch = pytest.importorskip("torch")
    w = _case(seed=21, lengths=(3, 9, 1), cand=(3, 2, 2), n_q=3, H=3, d=32)
    q, k, v, g = _inputs(w)
    tq = torch.tensor(q, requires_grad=True)
    tk = torch.tensor(k, requires_grad=True)
    tv = torch.tensor(v, requires_grad=True)
    sc = float(np.float32(w.scale))
    outs = []
    for c in range(w.n_cand):
        u = int(w.cand_to_user[c])
        a, b = int(w.user_offsets[u]), int(w.user_offsets[u + 1])
        kc = tk[a:b].permute(1, 0, 2)             # [H, L, d], an indexed copy per candidate
        vc = tv[a:b].permute(1, 0, 2)
        qc = tq[c].permute(1, 0, 2)               # [H, n_q, d]
        p = torch.softmax(sc * qc @ kc.transpose(1, 2), dim=-1)
        outs.append((p @ vc).permute(1, 0, 2))
    out = torch.stack(outs)
    (out * torch.tensor(g)).sum().backward()
    dq, dk, dv = B.target_attention_bwd(q, k, v, g, w.user_offsets, w.cand_to_user, w.scale)
    np.testing.assert_allclose(dq, tq.grad.numpy(), rtol=1e-10, atol=1e-12)
    np.testing.assert_allclose(dk, tk.grad.numpy(), rtol=1e-10, atol=1e-12)
    np.testing.assert_allclose(dv, tv.grad.numpy(), rtol=1e-10, atol=1e-12)


def test_closed_forms_per_user():
    """Rows of P sum to one, so per user and head the value gradients sum to the
    output gradients of its candidates' rows and the key gradients sum to zero
    (shifting every key by the same vector leaves the output unchanged)."""
    w = _case(seed=31, lengths=(6, 2, 11), cand=(4, 1, 3), n_q=2, H=2, d=64)
    q, k, v, g = _inputs(w)
    _, dk, dv = B.target_attention_bwd(q, k, v, g, w.user_offsets, w.cand_to_user, w.scale)
    for u in range(w.n_users):
        a, b = int(w.user_offsets[u]), int(w.user_offsets[u + 1])
        mine = w.cand_to_user == u
        np.testing.assert_allclose(dv[a:b].sum(axis=0), g[mine].sum(axis=(0, 1)), atol=1e-12)
        np.testing.assert_allclose(dk[a:b].sum(axis=0), 0.0, atol=1e-12)


def test_single_key_user():
    """One key: the output is v_0 whatever the scores, so the query and key
    gradients vanish (up to the rounding of dP - D, two sums of the same
    products) and dv_0 collects every output gradient."""
    w = _case(seed=41, lengths=(1,), cand=(5,), n_q=3, H=2, d=32)
    q, k, v, g = _inputs(w)
    dq, dk, dv = B.target_attention_bwd(q, k, v, g, w.user_offsets, w.cand_to_user, w.scale)
    assert np.abs(dq).max() < 1e-12 and np.abs(dk).max() < 1e-12
    np.testing.assert_allclose(dv[0], g.sum(axis=(0, 1)), atol=1e-12)


def test_reduction_over_candidates_is_a_sum():
    """A user's key and value gradients for two candidates equal the sums of the
    gradients of two one-candidate requests; query gradients are per candidate."""
    w = _case(seed=51, lengths=(9,), cand=(2,), n_q=2, H=2, d=32)
    q, k, v, g = _inputs(w)
    both = B.target_attention_bwd(q, k, v, g, w.user_offsets, w.cand_to_user, w.scale)
    parts = [B.target_attention_bwd(q[[c]], k, v, g[[c]], w.user_offsets, np.zeros(1, np.int32), w.scale)
             for c in range(2)]
    np.testing.assert_allclose(both[1], parts[0][1] + parts[1][1], atol=1e-13)
    np.testing.assert_allclose(both[2], parts[0][2] + parts[1][2], atol=1e-13)
    np.testing.assert_allclose(both[0], np.concatenate([parts[0][0], parts[1][0]]), atol=1e-13)


def test_empty_users():
    """A user with no keys gives zero query gradients; a user with no candidates
    gives zero key and value gradients."""
    w = _case()  # user 3 has no keys, user 4 no candidates
    q, k, v, g = _inputs(w)
    dq, dk, dv = B.target_attention_bwd(q, k, v, g, w.user_offsets, w.cand_to_user, w.scale)
    assert np.all(dq[w.cand_to_user == 3] == 0.0)
    a, b = int(w.user_offsets[4]), int(w.user_offsets[5])
    assert b > a and np.all(dk[a:b] == 0.0) and np.all(dv[a:b] == 0.0)


def _planted(w, mistake):
    q, k, v, g = _inputs(w)
    sc = float(np.float32(w.scale))
    dq = np.zeros_like(q)
    dk = np.zeros_like(k)
    dv = np.zeros_like(v)
    for c in range(w.n_cand):
        u = int(w.cand_to_user[c])
        a, b = int(w.user_offsets[u]), int(w.user_offsets[u + 1])
        if b == a:
            continue
        for h in range(w.H):
            qc, kc, vc, do = q[c, :, h], k[a:b, h], v[a:b, h], g[c, :, h]
            s = sc * qc @ kc.T
            p = np.exp(s - s.max(1, keepdims=True))
            p /= p.sum(1, keepdims=True)
            dp = do @ vc.T
            dd = 0.0 if mistake == "no_D" else np.sum(do * (p @ vc), 1, keepdims=True)
            ds = p * (dp - dd)
            dq[c, :, h] = (1.0 if mistake == "unscaled_dq" else sc) * ds @ kc
            gk, gv = sc * ds.T @ qc, p.T @ do
            if mistake == "last_candidate_wins":
                dk[a:b, h], dv[a:b, h] = gk, gv
            else:
                dk[a:b, h] += gk
                dv[a:b, h] += gv
    return dq, dk, dv


@pytest.mark.parametrize("mistake", ["no_D", "unscaled_dq", "last_candidate_wins"])
def test_planted_mistakes_fail_the_finite_differences(mistake):
    w = _case()
    assert _fd_check(w, _planted(w, mistake)) > 1e-4
    assert _fd_check(w, _planted(w, "none")) < 1e-7


def test_flop_count_is_the_five_products():
    w = make_bwd_workload("c2_typical")
    per = sum(2 * w.n_q * L * w.d for L in (1,)) * 5  # S, dP, dV, dK, dQ: n_q x L x d each
    assert B.flops_target_bwd([1], [1], w.n_q, 1, w.d) == per
    total = B.flops_target_bwd(w.counts, w.lengths, w.n_q, w.H, w.d)
    assert total == pytest.approx(2.5 * w.flops()["target"])


def test_per_user_calls_assemble_the_whole_call():
    """Users do not interact: calling the oracle once per user (that user's
    key/value rows, offsets [0, L] and its candidates) and placing the results
    gives the whole call's gradients bit for bit (the same candidate order
    within each user, so the same sums in the same order)."""
    w = _case()
    q, k, v, do = w.values("q_cand"), w.values("k_user"), w.values("v_user"), w.values("dout")
    whole = B.target_attention_bwd(q, k, v, do, w.user_offsets, w.cand_to_user, w.scale)
    dq, dk, dv = (np.zeros_like(x) for x in whole)
    for u in range(w.n_users):
        cands = np.flatnonzero(w.cand_to_user == u)
        a, b = int(w.user_offsets[u]), int(w.user_offsets[u + 1])
        gq, gk, gv = B.target_attention_bwd(q[cands], k[a:b], v[a:b], do[cands], np.array([0, b - a], np.int32),
                                            np.zeros(len(cands), np.int32), w.scale)
        dq[cands], dk[a:b], dv[a:b] = gq, gk, gv
    for x, y in zip((dq, dk, dv), whole):
        assert np.array_equal(x, y)
