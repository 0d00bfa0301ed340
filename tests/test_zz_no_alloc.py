"""The allocation-free attention call (ikbo_attn_fwd_mt_noalloc) against the
allocating one (ikbo_attn_fwd_mt) and the oracle, through the C ABI.

Two calls in a row share the library's fixed scratch, the second with a
smaller request, so a call that read partials or work items left by the
previous one would show.  Bar: bf16 max |err| <= 2e-2 and mean |err| <= 2e-3
against both references (fp32: 1e-4).
"""

import numpy as np
import pytest

from oracle import ikbo_oracle as O
from workloads import make_custom, make_workload

from gpu_helpers import assert_close, dtype_code, empty_out, say, to_f64, upload

pytestmark = pytest.mark.gpu


def _calls(w, out_na, out_ref):
    import broadcast_free_target_amd as ikbo
    dev = upload(w)
    args = (dev["q_cand"], dev["k_user"], dev["v_user"], dev["user_offsets"], dev["cand_to_user"], w.n_users,
            w.n_cand, w.H, w.d, w.scale)
    ikbo.ikbo_attn_fwd_mt_noalloc(*args, out_na, n_q=w.n_q, dtype=dtype_code(w.dtype))
    ikbo.ikbo_attn_fwd_mt(*args, out_ref, n_q=w.n_q, dtype=dtype_code(w.dtype))
    return dev


def _check(w, out_na, out_ref, what):
    import torch
    torch.cuda.synchronize()
    got, ref = to_f64(out_na), to_f64(out_ref)
    mx, mean = assert_close(got, ref, w.dtype, f"{what}: against ikbo_attn_fwd_mt")
    say(f"  {what}: against ikbo_attn_fwd_mt max {mx:.3g} mean {mean:.3g}")
    oracle = O.target_attention(w.values("q_cand"), w.values("k_user"), w.values("v_user"), w.user_offsets,
                                w.cand_to_user, w.scale)
    mx, mean = assert_close(got, oracle, w.dtype, f"{what}: against the oracle")
    say(f"  {what}: against the oracle max {mx:.3g} mean {mean:.3g}")


def test_two_calls_in_a_row_second_smaller():
    say("case no-alloc: typical request, then a smaller multi-query request")
    w1 = make_workload("c2_typical")
    c2u = np.random.default_rng(31).permutation(np.repeat(np.arange(4), (9, 1, 40, 3))).astype(np.int32)
    w2 = make_custom(3131, (700, 1, 129, 2048), c2u, n_q=2, H=3, d=128, dtype="bf16", name="na_small")
    a1, r1 = empty_out(w1.raw("q_cand").shape, "bf16"), empty_out(w1.raw("q_cand").shape, "bf16")
    a2, r2 = empty_out(w2.raw("q_cand").shape, "bf16"), empty_out(w2.raw("q_cand").shape, "bf16")
    _calls(w1, a1, r1)
    _calls(w2, a2, r2)
    _check(w1, a1, r1, "first call (typical request)")
    _check(w2, a2, r2, "second call (smaller request)")


def test_fp32_and_edge_requests_in_a_row():
    say("case no-alloc: edge bf16 request, then fp32, then a smaller bf16 one")
    c2u = np.random.default_rng(32).permutation(np.repeat(np.arange(4), (127, 2, 0, 129))).astype(np.int32)
    wa = make_custom(3232, (129, 0, 7, 300), c2u, n_q=1, H=3, d=64, dtype="bf16", name="na_edge")
    wb = make_workload("c1_tiny_f32")
    c2u = np.random.default_rng(33).permutation(np.repeat(np.arange(2), (3, 5))).astype(np.int32)
    wc = make_custom(3333, (33, 65), c2u, n_q=3, H=1, d=32, dtype="bf16", name="na_tiny")
    outs = []
    for w in (wa, wb, wc):
        a, r = empty_out(w.raw("q_cand").shape, w.dtype), empty_out(w.raw("q_cand").shape, w.dtype)
        _calls(w, a, r)
        outs.append((w, a, r))
    for w, a, r in outs:
        _check(w, a, r, w.name)
    got = to_f64(outs[0][1])
    for c in range(wa.n_cand):  # the zero-key user's candidates get zero rows
        if wa.lengths[wa.cand_to_user[c]] == 0:
            assert np.all(got[c] == 0)


def test_limits_are_refused_before_anything_runs():
    import torch
    import broadcast_free_target_amd as ikbo
    from broadcast_free_target_amd import IKBO_ERR_INVALID_ARG, IkboError
    say("case no-alloc: a request beyond the limits")
    n_users = 70000
    offs = torch.zeros(n_users + 1, dtype=torch.int32, device="cuda")
    c2u = torch.zeros(4, dtype=torch.int32, device="cuda")
    q = torch.zeros((4, 1, 2, 128), dtype=torch.bfloat16, device="cuda")
    kv = torch.zeros((1, 2, 128), dtype=torch.bfloat16, device="cuda")
    out = torch.full_like(q, 7.0)
    with pytest.raises(IkboError) as e:
        ikbo.ikbo_attn_fwd_mt_noalloc(q, kv, kv, offs, c2u, n_users, 4, 2, 128, 0.1, out)
    assert e.value.status == IKBO_ERR_INVALID_ARG and "limit" in str(e.value)
    torch.cuda.synchronize()
    assert torch.all(out.float() == 7.0)
