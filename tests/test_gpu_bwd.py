"""GPU parity of the target-attention backward (through the C ABI) against the
fp64 backward oracle.

The forward output the backward receives is the oracle's forward rounded to
bf16, so these tests do not depend on the forward kernels.  Tolerance: the
forward's bf16 bar, per gradient tensor, scaled by s = max(1, rms of the
oracle tensor): max |err| <= 2e-2 * s and mean |err| <= 2e-3 * s.  Each
gradient is a sum of bf16-rounded products (P and dS are rounded to bf16
before their products, as P is in the forward) plus a final bf16 rounding, so
its error grows with its own magnitude; a user's dV row sums the output
gradients of all its candidates' rows (rms 2-4 when a key takes all the
weight).
"""

import numpy as np
import pytest

from oracle import ikbo_bwd_oracle as B
from oracle import ikbo_oracle as O
from workloads import add_output_grad, f32_to_bf16_bits, make_bwd_workload, make_custom

from gpu_helpers import dev_tensor, oracle_in_chunks, say, to_f64

pytestmark = pytest.mark.gpu

MAX_REL = 2e-2
MEAN_REL = 2e-3


def _close(got, ref, what):
    assert got.shape == ref.shape
    assert np.all(np.isfinite(got)), f"{what}: non-finite"
    s = max(1.0, float(np.sqrt(np.mean(ref * ref)))) if ref.size else 1.0
    err = np.abs(got - ref)
    mx, mean = (float(err.max()), float(err.mean())) if err.size else (0.0, 0.0)
    say(f"  {what}: scale {s:.3g} max {mx:.3g} mean {mean:.3g}")
    assert mx <= MAX_REL * s and mean <= MEAN_REL * s, f"{what}: max {mx:.3g} mean {mean:.3g} scale {s:.3g}"


def _forward_out_bits(w):
    out = O.target_attention(w.values("q_cand"), w.values("k_user"), w.values("v_user"), w.user_offsets,
                             w.cand_to_user, w.scale)
    return f32_to_bf16_bits(out.astype(np.float32)).reshape(out.shape)


def _lse(w):
    """The oracle's row log-sum-exp as fp32 on the device (the statistic a
    training forward hands the backward), independent of the forward kernels."""
    q, k = w.values("q_cand"), w.values("k_user")
    ref = np.concatenate(oracle_in_chunks(
        lambda c: O.target_attention_lse(q, k, w.user_offsets, w.cand_to_user, w.scale, cands=c),
        range(w.n_cand)), axis=0)
    import torch
    return torch.from_numpy(ref.astype(np.float32)).cuda()


def _run(w, out_bits, bwd=None, lse=None):
    import torch
    import broadcast_free_target_amd as ikbo
    t = {n: dev_tensor(w.raw(n), "bf16") for n in ("q_cand", "k_user", "v_user", "dout")}
    out = dev_tensor(out_bits, "bf16")
    dq = torch.full_like(t["q_cand"], float("nan"))
    dk = torch.full_like(t["k_user"], float("nan"))
    dv = torch.full_like(t["v_user"], float("nan"))
    own = bwd is None
    h = ikbo.ikbo_bwd_create() if own else bwd
    try:
        ikbo.ikbo_attn_bwd(h, w.user_offsets, w.cand_to_user, w.n_users, w.n_cand, w.n_q, w.H, w.d, w.scale,
                           t["q_cand"], t["k_user"], t["v_user"], out, t["dout"], dq, dk, dv, lse=lse)
        torch.cuda.synchronize()
    finally:
        if own:
            ikbo.ikbo_bwd_destroy(h)
    return to_f64(dq), to_f64(dk), to_f64(dv)


def _oracle(w, out_bits=None):
    return B.target_attention_bwd(w.values("q_cand"), w.values("k_user"), w.values("v_user"), w.values("dout"),
                                  w.user_offsets, w.cand_to_user, w.scale)


def _custom(seed, lengths, counts, n_q=1, H=2):
    c2u = np.random.default_rng(seed).permutation(np.repeat(np.arange(len(lengths)), counts)).astype(np.int32)
    w = make_custom(seed, lengths, c2u, n_q=n_q, H=H, d=128, dtype="bf16", name=f"bwd{seed}")
    return add_output_grad(w, seed + 100)


CASES = [
    # lengths, candidates per user, n_q, H
    ((70, 1, 200, 129), (5, 2, 9, 3), 1, 2),
    ((64, 65, 127, 128, 300), (1, 64, 65, 129, 3), 1, 1),
    ((33, 0, 150, 7), (4, 3, 2, 0), 2, 3),
    ((500,), (200,), 3, 1),
]


@pytest.mark.parametrize("given_lse", [False, True])
@pytest.mark.parametrize("i", range(len(CASES)))
def test_bwd_edges(i, given_lse):
    lengths, counts, n_q, H = CASES[i]
    w = _custom(3300 + i, lengths, counts, n_q, H)
    say(f"case bwd {CASES[i]} given lse {given_lse}")
    got = _run(w, _forward_out_bits(w), lse=_lse(w) if given_lse else None)
    ref = _oracle(w)
    for g, r, name in zip(got, ref, ("dq", "dk", "dv")):
        _close(g, r, name)


def _oracle_by_user(w):
    """The backward oracle evaluated one user at a time: each call gets one
    user's key and value rows and that user's candidates (users do not interact,
    so the assembled result is the whole call's; pinned on the CPU), the calls
    running side by side in a thread pool."""
    q, k, v, do = w.values("q_cand"), w.values("k_user"), w.values("v_user"), w.values("dout")
    offs, c2u = w.user_offsets, w.cand_to_user

    def users(us):
        res = []
        for u in us:
            cands = np.flatnonzero(c2u == u)
            a, b = int(offs[u]), int(offs[u + 1])
            g = B.target_attention_bwd(q[cands], k[a:b], v[a:b], do[cands], np.array([0, b - a], np.int32),
                                       np.zeros(len(cands), np.int32), w.scale)
            res.append((u, cands, g))
        return res

    dq = np.zeros(q.shape)
    dk = np.zeros(k.shape)
    dv = np.zeros(v.shape)
    for part in oracle_in_chunks(users, range(w.n_users)):
        for u, cands, (gq, gk, gv) in part:
            a, b = int(offs[u]), int(offs[u + 1])
            dq[cands] = gq
            dk[a:b] = gk
            dv[a:b] = gv
    return dq, dk, dv


@pytest.mark.timeout(900)
def test_bwd_large_request_full():
    """The backward at the large request it is benchmarked on (10,000
    candidates over 150 users, 4 query tokens, 8 heads): every element of dq,
    dk and dv against the oracle."""
    w = make_bwd_workload("c4_large")
    say("case bwd c4_large (full tensors)")
    q, k, v = w.values("q_cand"), w.values("k_user"), w.values("v_user")

    def fwd(cands):
        return O.target_attention(q, k, v, w.user_offsets, w.cand_to_user, w.scale, cands=cands)

    out = np.concatenate(oracle_in_chunks(fwd, range(w.n_cand)), axis=0)
    out_bits = f32_to_bf16_bits(out.astype(np.float32)).reshape(out.shape)
    del out
    got = _run(w, out_bits)
    got_lse = _run(w, out_bits, lse=_lse(w))
    say("  gradients computed (recomputed and given log-sum-exp); oracle by user")
    ref = _oracle_by_user(w)
    for g, g2, r, name in zip(got, got_lse, ref, ("dq", "dk", "dv")):
        _close(g, r, name)
        _close(g2, r, name + " (given lse)")


def test_bwd_single_key_users():
    """One key: dq and dk vanish up to the rounding of dP - D; dv_0 sums dout."""
    w = _custom(3400, (1, 1, 40), (6, 3, 2), n_q=2, H=2)
    say("case bwd single key")
    dq, dk, dv = _run(w, _forward_out_bits(w))
    ref = _oracle(w)
    for u in (0, 1):
        mine = w.cand_to_user == u
        assert np.abs(dq[mine]).max() <= 1e-3
        k0 = int(w.user_offsets[u])
        assert np.abs(dk[k0]).max() <= 1e-3
        _close(dv[k0:k0 + 1], ref[2][k0:k0 + 1], f"dv user {u}")


@pytest.mark.parametrize("given_lse", [False, True])
def test_bwd_typical_request_full(given_lse):
    w = make_bwd_workload("c2_typical")
    say(f"case bwd c2_typical given lse {given_lse}")
    got = _run(w, _forward_out_bits(w), lse=_lse(w) if given_lse else None)
    ref = _oracle(w)
    for g, r, name in zip(got, ref, ("dq", "dk", "dv")):
        _close(g, r, name)


def test_bwd_no_keys_at_all():
    """Every user has zero keys but there are candidates: the forward output is
    the constant 0, so every query-gradient row must be written as zero (the
    prefilled value must not survive) and there is no key gradient to write."""
    import torch
    import broadcast_free_target_amd as ikbo
    w = _custom(3450, (0, 0, 0), (3, 2, 4), n_q=2, H=2)
    say("case bwd no keys at all")
    assert w.total_len == 0
    t = {n: dev_tensor(w.raw(n), "bf16") for n in ("q_cand", "dout")}
    out = torch.zeros_like(t["q_cand"])
    dq = torch.full_like(t["q_cand"], 7.0)
    empty = torch.empty((0, w.H, w.d), dtype=torch.bfloat16, device="cuda")
    h = ikbo.ikbo_bwd_create()
    try:
        ikbo.ikbo_attn_bwd(h, w.user_offsets, w.cand_to_user, w.n_users, w.n_cand, w.n_q, w.H, w.d, w.scale,
                           t["q_cand"], empty, empty, out, t["dout"], dq, torch.empty_like(empty),
                           torch.empty_like(empty))
        torch.cuda.synchronize()
    finally:
        ikbo.ikbo_bwd_destroy(h)
    ref_dq = _oracle(w)[0]
    assert np.all(ref_dq == 0.0)
    assert torch.count_nonzero(dq).item() == 0


def test_bwd_repeatable_and_handle_reuse():
    import broadcast_free_target_amd as ikbo
    w1 = _custom(3500, (90, 17, 300), (7, 1, 5), n_q=1, H=2)
    w2 = _custom(3501, (40, 260), (12, 30), n_q=2, H=2)
    say("case bwd repeat / alternate")
    o1, o2 = _forward_out_bits(w1), _forward_out_bits(w2)
    h = ikbo.ikbo_bwd_create()
    try:
        a = _run(w1, o1, h)
        b = _run(w2, o2, h)
        c = _run(w1, o1, h)
        d = _run(w2, o2, h)
    finally:
        ikbo.ikbo_bwd_destroy(h)
    for x, y in zip(a, c):
        assert np.array_equal(x, y)
    for x, y in zip(b, d):
        assert np.array_equal(x, y)
    for g, r, name in zip(b, _oracle(w2), ("dq", "dk", "dv")):
        _close(g, r, name)


def test_bwd_work_list_ring_unsynchronised_calls():
    """36 calls on one handle, two requests alternating, no synchronisation in
    between (more calls than the handle's pinned work-list buffers, across
    several periodic events): every call's gradients equal its request's first
    ones bit for bit."""
    import torch
    import broadcast_free_target_amd as ikbo
    ws = (_custom(3510, (90, 17, 300), (7, 1, 5), n_q=1, H=2), _custom(3511, (40, 260), (12, 30), n_q=2, H=2))
    say("case bwd work-list ring, 36 unsynchronised calls")
    ins = []
    for w in ws:
        t = {n: dev_tensor(w.raw(n), "bf16") for n in ("q_cand", "k_user", "v_user", "dout")}
        t["out"] = dev_tensor(_forward_out_bits(w), "bf16")
        ins.append(t)
    h = ikbo.ikbo_bwd_create()
    grads = []
    try:
        for i in range(36):
            w, t = ws[i % 2], ins[i % 2]
            g = [torch.full_like(t[n], float("nan")) for n in ("q_cand", "k_user", "v_user")]
            ikbo.ikbo_attn_bwd(h, w.user_offsets, w.cand_to_user, w.n_users, w.n_cand, w.n_q, w.H, w.d, w.scale,
                               t["q_cand"], t["k_user"], t["v_user"], t["out"], t["dout"], *g)
            grads.append(g)
        torch.cuda.synchronize()
    finally:
        ikbo.ikbo_bwd_destroy(h)
    for i, g in enumerate(grads):
        for x, y in zip(g, grads[i % 2]):
            assert torch.equal(x.view(torch.int16), y.view(torch.int16)), f"call {i}"
    for g, r, name in zip(grads[1], _oracle(ws[1]), ("dq", "dk", "dv")):
        _close(to_f64(g), r, name)


def test_bwd_errors():
    import torch
    import broadcast_free_target_amd as ikbo
    from broadcast_free_target_amd import IkboError
    w = _custom(3600, (30, 20), (3, 2), n_q=1, H=1)
    t = {n: dev_tensor(w.raw(n), "bf16") for n in ("q_cand", "k_user", "v_user", "dout")}
    out = dev_tensor(_forward_out_bits(w), "bf16")
    dq = torch.zeros_like(t["q_cand"])
    dk = torch.zeros_like(t["k_user"])
    dv = torch.zeros_like(t["v_user"])
    say("case bwd errors")
    h = ikbo.ikbo_bwd_create()
    try:
        args = [w.user_offsets, w.cand_to_user, w.n_users, w.n_cand, w.n_q, w.H, w.d, w.scale,
                t["q_cand"], t["k_user"], t["v_user"], out, t["dout"], dq, dk, dv]
        bad = list(args)
        bad[6] = 64
        with pytest.raises(IkboError):
            ikbo.ikbo_attn_bwd(h, *bad)
        bad = list(args)
        bad[14] = t["k_user"]  # dk aliases k
        with pytest.raises(IkboError):
            ikbo.ikbo_attn_bwd(h, *bad)
        bad = list(args)
        bad[1] = np.array([0, 2, 1, 0, 1], np.int32)
        with pytest.raises(IkboError):
            ikbo.ikbo_attn_bwd(h, *bad)
        bad = list(args)
        bad[0] = np.array([0, 30, 20], np.int32)
        with pytest.raises(IkboError):
            ikbo.ikbo_attn_bwd(h, *bad)
        torch.cuda.synchronize()
        assert torch.count_nonzero(dq).item() == 0 and torch.count_nonzero(dk).item() == 0
        # no candidates: every key gradient is zero
        ikbo.ikbo_attn_bwd(h, w.user_offsets, np.zeros(0, np.int32), w.n_users, 0, 1, 1, 128, w.scale, None,
                           t["k_user"], t["v_user"], None, None, None, dk.fill_(1.0), dv.fill_(1.0))
        torch.cuda.synchronize()
        assert torch.count_nonzero(dk).item() == 0 and torch.count_nonzero(dv).item() == 0
    finally:
        ikbo.ikbo_bwd_destroy(h)


@pytest.mark.parametrize("given_lse", [False, True])
@pytest.mark.parametrize("no_split", ["1", "0"])
def test_bwd_split_and_unsplit(no_split, given_lse, monkeypatch):
    """Long key ranges split into chunks (merged in chunk order) and the
    unsplit path both meet the bar, with the log-sum-exp recomputed or given;
    each is bitwise repeatable."""
    import broadcast_free_target_amd as ikbo
    monkeypatch.setenv("IKBO_NO_SPLIT", no_split)
    w = _custom(3700, (2048, 1500, 64, 900), (3, 40, 5, 1), n_q=2, H=2)
    say(f"case bwd split disabled={no_split} given lse {given_lse}")
    o = _forward_out_bits(w)
    lse = _lse(w) if given_lse else None
    h = ikbo.ikbo_bwd_create()
    try:
        a = _run(w, o, h, lse)
        groups = ikbo.ikbo_bwd_info(h)["dq_split_groups"]
        b = _run(w, o, h, lse)
    finally:
        ikbo.ikbo_bwd_destroy(h)
    assert (groups == 0) == (no_split == "1")
    for x, y in zip(a, b):
        assert np.array_equal(x, y)
    for g, r, name in zip(a, _oracle(w), ("dq", "dk", "dv")):
        _close(g, r, name)


def test_binding_rejects_bwd_tensors_that_do_not_fit():
    """A dK tensor one key row short and an fp32 dQ are refused by the binding
    (sizes from the host offsets) before anything is launched."""
    import torch
    import broadcast_free_target_amd as ikbo
    from broadcast_free_target_amd import IKBO_ERR_INVALID_ARG, IkboError
    w = _custom(3520, (40, 90), (3, 5))
    say("case bwd tensors that do not fit")
    t = {n: dev_tensor(w.raw(n), "bf16") for n in ("q_cand", "k_user", "v_user", "dout")}
    out = dev_tensor(_forward_out_bits(w), "bf16")
    dq = torch.full_like(t["q_cand"], 7.0)
    dk = torch.full_like(t["k_user"], 7.0)
    dv = torch.full_like(t["v_user"], 7.0)
    h = ikbo.ikbo_bwd_create()
    try:
        args = [w.user_offsets, w.cand_to_user, w.n_users, w.n_cand, w.n_q, w.H, w.d, w.scale,
                t["q_cand"], t["k_user"], t["v_user"], out, t["dout"]]
        with pytest.raises(IkboError) as e:
            ikbo.ikbo_attn_bwd(h, *args, dq, dk[:-1], dv)
        assert e.value.status == IKBO_ERR_INVALID_ARG and "dk_user" in str(e.value)
        with pytest.raises(IkboError) as e:
            ikbo.ikbo_attn_bwd(h, *args, dq.float(), dk, dv)
        assert e.value.status == IKBO_ERR_INVALID_ARG and "element size" in str(e.value)
        torch.cuda.synchronize()
        for g in (dq, dk, dv):
            assert torch.all(g.float() == 7.0)
    finally:
        ikbo.ikbo_bwd_destroy(h)

