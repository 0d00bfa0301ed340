"""GPU parity of MXFP8 target attention (through the C ABI) against the fp64
MXFP8 oracle.

The GPU and the oracle quantize P with the same rule; they differ by the
scores' accumulation rounding (the FP8 matrix instruction sums its exact
products with about 2^-14 relative error; measured) and the final bf16
rounding.  Where a weight p_j / 2^e lies within that uncertainty of an E4M3
rounding midpoint (or a block maximum of a scale boundary), the two sides may
legitimately round it differently: one E4M3 step, up to 1/8 of the weight.
Bar, per output tensor with s = max(1, rms of the oracle output): mean |err|
<= 2e-3 * s, and per element |err| <= 2e-2 * s + slack, where slack sums, over
the row's ambiguous weights only, that weight's possible step times |v_j| / l
(computed from the oracle's own p, with the scores' uncertainty bounded by
2^-12 of sum_d |q_d k_d|, several times the measured error).  Rows with no
ambiguous weight get no slack.
"""

import os

import numpy as np
import pytest

from oracle import mxfp8_oracle as M
from workloads import make_mxfp8, make_mxfp8_custom

from gpu_helpers import mx_user_oracle, oracle_in_processes, say

pytestmark = pytest.mark.gpu

MAX_REL = 2e-2
MEAN_REL = 2e-3


@pytest.fixture(autouse=True)
def _clean_env():
    keys = ("IKBO_NO_SPLIT", "IKBO_MIN_CHUNK", "IKBO_SPLIT_SLOTS", "IKBO_GRID_WGS")
    saved = {k: os.environ.get(k) for k in keys}
    yield
    for k, v in saved.items():
        if v is None:
            os.environ.pop(k, None)
        else:
            os.environ[k] = v


def _dev(w):
    import torch
    return [torch.from_numpy(np.ascontiguousarray(a)).cuda() for a in w.arrays()]


def _run(w, h=None, dev=None):
    import torch
    import broadcast_free_target_amd as ikbo
    dev = dev or _dev(w)
    out = torch.full((w.n_cand, w.n_q, w.H, w.d), float("nan"), dtype=torch.bfloat16, device="cuda")
    own = h is None
    h = ikbo.ikbo_mx_create() if own else h
    try:
        ikbo.ikbo_attn_fwd_mxfp8(h, w.user_offsets, w.cand_to_user, w.n_users, w.n_cand, w.n_q, w.H, w.d, w.scale,
                                 *dev, out)
        torch.cuda.synchronize()
    finally:
        if own:
            ikbo.ikbo_mx_destroy(h)
    return out.float().cpu().numpy().astype(np.float64)


def _oracle(w, cands=None):
    if cands is None:
        return M.target_attention_mxfp8(*w.arrays(), w.user_offsets, w.cand_to_user, w.scale)
    cands = np.asarray(cands)
    return M.target_attention_mxfp8(w.q_codes[cands], w.q_scales[cands], w.k_codes, w.k_scales, w.v_codes,
                                    w.v_scales, w.user_offsets, w.cand_to_user[cands], w.scale)


def _e4m3_step(y):
    """Spacing of the E4M3 grid at y >= 0 (3 mantissa bits, subnormal spacing 2^-9)."""
    _, ex = np.frexp(np.maximum(y, 2.0 ** -6))
    return np.exp2(ex - 1 - 3.0)


def _slack(w, cands=None):
    """Per output element, the change the ambiguous rounding decisions of its
    row could cause (see the module docstring)."""
    cands = np.arange(w.n_cand) if cands is None else np.asarray(cands)
    q = M.dequantize_rows(w.q_codes, w.q_scales)
    k = M.dequantize_rows(w.k_codes, w.k_scales)
    v = M.dequantize_v(w.v_codes, w.v_scales, w.user_offsets)
    c_log2 = float(np.float32(w.scale)) * M.LOG2E
    out = np.zeros((cands.size, w.n_q, w.H, w.d))
    for i, c in enumerate(cands):
        u = int(w.cand_to_user[c])
        a, b = int(w.user_offsets[u]), int(w.user_offsets[u + 1])
        if b == a:
            continue
        for r in range(w.n_q):
            for h in range(w.H):
                kk, qq, vv = k[a:b, h], q[c, r, h], v[a:b, h]
                x = c_log2 * (kk @ qq)
                dx = abs(c_log2) * 2.0 ** -12 * (np.abs(kk) @ np.abs(qq))
                p = np.exp2(x - np.ceil(x.max()))
                rp = np.log(2.0) * dx + 2.0 ** -20          # relative uncertainty of each p
                sl = np.zeros_like(p)
                for j0 in range(0, p.size, 32):
                    blk, rb = p[j0:j0 + 32], rp[j0:j0 + 32]
                    e = M.p_block_exponent(float(blk.max()))
                    if e is None:
                        continue
                    y = blk / 2.0 ** e
                    step = _e4m3_step(y)
                    frac = y / step - np.floor(y / step)                  # position within the step
                    near_mid = np.abs(frac - 0.5) * step <= y * rb
                    f, ex = np.frexp(blk.max())
                    rel = rb.max()
                    edge = abs(2 * f - 1.75) <= 2 * rel or (2 * f - 1.0) <= 2 * rel or (2.0 - 2 * f) <= 4 * rel
                    sl[j0:j0 + 32] = np.where(edge | near_mid, (2.0 if edge else 1.0) * step * 2.0 ** e, 0.0)
                if sl.any():
                    out[i, r, h] = (sl @ np.abs(vv)) / p.sum()
    return out


def _close(got, ref, what, slack=None):
    assert got.shape == ref.shape
    assert np.all(np.isfinite(got)), f"{what}: non-finite"
    s = max(1.0, float(np.sqrt(np.mean(ref * ref))))
    err = np.abs(got - ref)
    mx, mean = float(err.max()), float(err.mean())
    sl = np.zeros_like(err) if slack is None else slack
    over = err - MAX_REL * s - sl
    say(f"  {what}: scale {s:.3g} max {mx:.3g} mean {mean:.3g}; elements with slack {int((sl > 0).sum())}, "
        f"largest slack {float(sl.max()):.3g}, worst margin {float(over.max()):.3g}")
    assert mean <= MEAN_REL * s, f"{what}: mean {mean:.3g}"
    assert np.all(over <= 0), f"{what}: max {mx:.3g} beyond the bar plus the rounding-ambiguity slack"


def test_mx_tiny_full():
    """Users of 1, 31, 32, 33, 70, 0, 130 and 5 keys (partial V-scale blocks,
    an empty user, several tiles), n_q = 2, H = 2."""
    w = make_mxfp8("mx_tiny")
    say("case mx_tiny")
    got = _run(w)
    _close(got, _oracle(w), "mx_tiny", _slack(w))
    empty = w.cand_to_user == 5
    assert np.all(got[empty] == 0)


def test_mx_typical_request_full():
    w = make_mxfp8("mx_c2_typical")
    say("case mx_c2_typical")
    _close(_run(w), _oracle(w), "mx_c2_typical", _slack(w))


def test_mx_skewed_request_sampled():
    w = make_mxfp8("mx_c3_skewed")
    say("case mx_c3_skewed (sampled)")
    got = _run(w)
    rng = np.random.default_rng(5)
    short = np.flatnonzero(w.lengths[w.cand_to_user] <= 3)
    cands = np.unique(np.concatenate([rng.choice(w.n_cand, 40, replace=False), short]))
    _close(got[cands], _oracle(w, cands), "mx_c3_skewed sample", _slack(w, cands))


def _oracle_by_user(w, users):
    """The MXFP8 oracle evaluated one user at a time (that user's candidates,
    key and value rows and value-scale blocks; users do not interact, pinned on
    the CPU), in a pool of worker processes: the oracle's per-row loops are
    bound by the interpreter, not by numpy's kernels.  Returns the candidates
    of those users and their outputs."""
    vbo = M.v_block_offsets(w.user_offsets)
    args, sel = [], []
    for u in users:
        cands = np.flatnonzero(w.cand_to_user == u)
        a, b = int(w.user_offsets[u]), int(w.user_offsets[u + 1])
        args.append((w.q_codes[cands], w.q_scales[cands], w.k_codes[a:b], w.k_scales[a:b], w.v_codes[a:b],
                     w.v_scales[vbo[u]:vbo[u + 1]], w.scale))
        sel.append(cands)
    return np.concatenate(sel), np.concatenate(oracle_in_processes(mx_user_oracle, args), axis=0)


@pytest.mark.timeout(600)
def test_mx_large_request_whole_users():
    """The large request (10,000 candidates over 150 users, 4 query tokens, 8
    heads): every output element of 32 whole users (the shortest, the longest
    and 30 spread over the length order; about a fifth of the output) against
    the oracle.  The rounding-ambiguity slack is only computed for candidates
    with an element beyond the plain bar."""
    w = make_mxfp8("mx_c4_large")
    say("case mx_c4_large (32 whole users)")
    got = _run(w)
    order = np.argsort(w.lengths, kind="stable")
    users = order[np.unique(np.linspace(0, w.n_users - 1, 32).round().astype(int))]
    cands, ref = _oracle_by_user(w, users)
    got = got[cands]
    s = max(1.0, float(np.sqrt(np.mean(ref * ref))))
    over = np.flatnonzero((np.abs(got - ref) > MAX_REL * s).reshape(len(cands), -1).any(axis=1))
    slack = np.zeros_like(ref)
    if over.size:
        say(f"  {over.size} candidates beyond the plain bar; computing their slack")
        slack[over] = _slack(w, cands[over])
    _close(got, ref, f"mx_c4_large, {len(users)} users, {len(cands)} candidates", slack)


@pytest.mark.parametrize("mode", ["unsplit", "default", "many_chunks"])
def test_mx_split_modes(mode):
    """Long key ranges split into chunks and merged, or not split: each meets
    the bar and is bitwise repeatable."""
    if mode == "unsplit":
        os.environ["IKBO_NO_SPLIT"] = "1"
    elif mode == "many_chunks":
        os.environ["IKBO_MIN_CHUNK"] = "64"
        os.environ["IKBO_SPLIT_SLOTS"] = "4096"
    w = make_mxfp8_custom(4400, (4096, 1, 700, 2048, 129, 64), np.random.default_rng(44).permutation(
        np.repeat(np.arange(6), (150, 3, 1, 65, 129, 2))), n_q=1, H=2)
    import broadcast_free_target_amd as ikbo
    say(f"case mx split mode {mode}")
    h = ikbo.ikbo_mx_create()
    try:
        dev = _dev(w)
        a = _run(w, h, dev)
        groups = ikbo.ikbo_mx_info(h)["n_groups"]
        b = _run(w, h, dev)
    finally:
        ikbo.ikbo_mx_destroy(h)
    assert (groups == 0) == (mode == "unsplit")
    assert np.array_equal(a, b)
    _close(a, _oracle(w), f"split mode {mode}", _slack(w))


def test_mx_zero_scale_is_the_mean_of_v():
    """scale 0: p = 1 exactly for every key, so each output row is the mean of
    the user's dequantized values (up to fp32 accumulation and bf16 rounding)."""
    w = make_mxfp8_custom(4500, (3, 40, 70, 300), [0, 1, 2, 3, 1, 3], n_q=1, H=2)
    w.scale = np.float32(0.0)
    say("case mx zero scale")
    got = _run(w)
    v = M.dequantize_v(w.v_codes, w.v_scales, w.user_offsets)
    for c in range(w.n_cand):
        u = int(w.cand_to_user[c])
        a, b = int(w.user_offsets[u]), int(w.user_offsets[u + 1])
        mean = v[a:b].mean(axis=0)
        # bf16 rounding of the mean plus the accumulation rounding of sum |v| / L
        tol = 2.0 ** -8 * np.abs(mean) + 2.0 ** -12 * np.abs(v[a:b]).mean(axis=0) + 1e-6
        assert np.all(np.abs(got[c, 0] - mean) <= tol)


@pytest.mark.parametrize("scale", [-0.0883883, -1.5])
def test_mx_negative_scale(scale):
    """A negative softmax scale runs the kernel's other instance (block maxima
    on the negated scores)."""
    w = make_mxfp8_custom(4550, (1, 33, 70, 300, 1500), [0, 1, 2, 3, 4, 4, 2, 1, 3], n_q=2, H=2)
    w.scale = np.float32(scale)
    say(f"case mx negative scale {scale}")
    _close(_run(w), _oracle(w), f"scale {scale}", _slack(w))


def test_mx_handle_reuse_alternating_requests():
    import broadcast_free_target_amd as ikbo
    w1 = make_mxfp8_custom(4600, (90, 17, 300), [0, 1, 2, 2, 0, 1, 2], n_q=1, H=2)
    w2 = make_mxfp8_custom(4601, (40, 260), [1, 0, 1, 1], n_q=2, H=2)
    say("case mx handle reuse")
    h = ikbo.ikbo_mx_create()
    try:
        d1, d2 = _dev(w1), _dev(w2)
        a, b, c, d = _run(w1, h, d1), _run(w2, h, d2), _run(w1, h, d1), _run(w2, h, d2)
    finally:
        ikbo.ikbo_mx_destroy(h)
    assert np.array_equal(a, c) and np.array_equal(b, d)
    _close(b, _oracle(w2), "second request", _slack(w2))


def test_mx_work_list_ring_unsynchronised_calls():
    """40 calls on one handle, two requests alternating, no synchronisation in
    between: more calls than the handle has pinned work-list buffers, across
    several of its periodic events.  Every call's output equals its request's
    first one, so no buffer was rewritten while a queued kernel still read it."""
    import torch
    import broadcast_free_target_amd as ikbo
    w1 = make_mxfp8_custom(4610, (90, 17, 300), [0, 1, 2, 2, 0, 1, 2], n_q=1, H=2)
    w2 = make_mxfp8_custom(4611, (40, 260, 5), [1, 0, 1, 1, 2], n_q=2, H=2)
    say("case mx work-list ring, 40 unsynchronised calls")
    h = ikbo.ikbo_mx_create()
    try:
        d = (_dev(w1), _dev(w2))
        outs = []
        for i in range(40):
            w = (w1, w2)[i % 2]
            o = torch.full((w.n_cand, w.n_q, w.H, w.d), float("nan"), dtype=torch.bfloat16, device="cuda")
            ikbo.ikbo_attn_fwd_mxfp8(h, w.user_offsets, w.cand_to_user, w.n_users, w.n_cand, w.n_q, w.H, w.d,
                                     w.scale, *d[i % 2], o)
            outs.append(o)
        torch.cuda.synchronize()
    finally:
        ikbo.ikbo_mx_destroy(h)
    for i, o in enumerate(outs):
        assert torch.equal(o.view(torch.int16), outs[i % 2].view(torch.int16)), f"call {i}"
    _close(outs[1].float().cpu().numpy().astype(np.float64), _oracle(w2), "ring", _slack(w2))


def test_mx_errors():
    import torch
    import broadcast_free_target_amd as ikbo
    from broadcast_free_target_amd import IKBO_ERR_INVALID_ARG, IKBO_ERR_UNSUPPORTED, IkboError
    w = make_mxfp8_custom(4700, (30, 20), [0, 1, 1], n_q=1, H=1)
    dev = _dev(w)
    out = torch.zeros((w.n_cand, 1, 1, 128), dtype=torch.bfloat16, device="cuda")
    say("case mx errors")
    h = ikbo.ikbo_mx_create()
    try:
        args = [w.user_offsets, w.cand_to_user, w.n_users, w.n_cand, 1, 1, 128, w.scale]
        bad = list(args)
        bad[6] = 64
        with pytest.raises(IkboError) as e:
            ikbo.ikbo_attn_fwd_mxfp8(h, *bad, *dev, out)
        assert e.value.status == IKBO_ERR_UNSUPPORTED
        with pytest.raises(IkboError) as e:  # out aliases the key codes
            ikbo.ikbo_attn_fwd_mxfp8(h, *args, *dev, dev[2].view(torch.bfloat16).view(-1)[: out.numel()].view(out.shape))
        assert e.value.status == IKBO_ERR_INVALID_ARG
        with pytest.raises(IkboError) as e:  # misaligned key codes (raw pointer: the library's own check)
            ikbo.ikbo_attn_fwd_mxfp8(h, *args, dev[0], dev[1], dev[2].data_ptr() + 1, dev[3], dev[4], dev[5], out)
        assert e.value.status == IKBO_ERR_INVALID_ARG
        with pytest.raises(IkboError) as e:  # key codes one byte short (the binding's size check)
            ikbo.ikbo_attn_fwd_mxfp8(h, *args, dev[0], dev[1], dev[2].view(-1)[1:], dev[3], dev[4], dev[5], out)
        assert "bytes, the call needs" in str(e.value)
        with pytest.raises(IkboError):  # mapping out of range
            ikbo.ikbo_attn_fwd_mxfp8(h, w.user_offsets, np.array([0, 2, 1], np.int32), *args[2:], *dev, out)
        torch.cuda.synchronize()
        assert torch.count_nonzero(out).item() == 0
    finally:
        ikbo.ikbo_mx_destroy(h)


def test_binding_rejects_mx_tensors_that_do_not_fit():
    """V scales one block short (the count follows from the users' lengths) and
    a float32 output are refused by the binding before anything is launched."""
    import torch
    import broadcast_free_target_amd as ikbo
    from broadcast_free_target_amd import IKBO_ERR_INVALID_ARG, IkboError
    w = make_mxfp8_custom(4620, (30, 20), [0, 1, 1], n_q=1, H=1)
    dev = _dev(w)
    out = torch.zeros((w.n_cand, 1, 1, 128), dtype=torch.bfloat16, device="cuda")
    say("case mx tensors that do not fit")
    h = ikbo.ikbo_mx_create()
    try:
        args = [w.user_offsets, w.cand_to_user, w.n_users, w.n_cand, 1, 1, 128, w.scale]
        with pytest.raises(IkboError) as e:
            ikbo.ikbo_attn_fwd_mxfp8(h, *args, *dev[:5], dev[5][:-1], out)
        assert e.value.status == IKBO_ERR_INVALID_ARG and "v_scales" in str(e.value)
        with pytest.raises(IkboError) as e:
            ikbo.ikbo_attn_fwd_mxfp8(h, *args, *dev, out.float())
        assert e.value.status == IKBO_ERR_INVALID_ARG and "element size" in str(e.value)
        torch.cuda.synchronize()
        assert torch.count_nonzero(out).item() == 0
    finally:
        ikbo.ikbo_mx_destroy(h)

