"""GPU parity of IKBO linear compression (through the C ABI) against the fp64 oracle.

Tolerance: bf16 inputs, fp32 accumulation, bf16 output -> max |err| <= 2e-2 and
mean |err| <= 2e-3 (outputs are O(1): W is drawn with standard deviation
1/sqrt(K)).  Bitwise: repeated calls, and a permutation of the candidates
permutes the output rows exactly.
"""

import numpy as np
import pytest

from oracle import lce_oracle as L
from workloads import make_lce, make_lce_custom

from gpu_helpers import assert_close, oracle_in_chunks, say

pytestmark = pytest.mark.gpu


def _dev(a):
    import torch
    return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).cuda().view(torch.bfloat16)


def _run(w, c2u=None, n_users=None, stream=None):
    import torch
    from broadcast_free_target_amd import ikbo_lce_create, ikbo_lce_destroy, ikbo_lce_errors, ikbo_lce_fwd
    c2u = w.cand_to_user if c2u is None else np.asarray(c2u, np.int32)
    U = w.n_users if n_users is None else n_users
    W = _dev(w.raw("w"))
    xu = _dev(w.raw("x_user")) if w.K_u > 0 else None
    xc = _dev(w.raw("x_cand")) if w.K_c > 0 else None
    m = torch.from_numpy(c2u.copy()).cuda()
    out = torch.full((len(c2u), w.M, w.N), float("nan"), dtype=torch.bfloat16, device="cuda")
    h = ikbo_lce_create(W, w.M, w.K_u, w.K_c)
    try:
        ikbo_lce_fwd(h, xu, xc, m, U, len(c2u), w.N, out)
        torch.cuda.synchronize()
        errs = ikbo_lce_errors(h)
    finally:
        ikbo_lce_destroy(h)
    return out.float().cpu().numpy().astype(np.float64), errs


def _oracle(w, cands=None):
    xc = w.values("x_cand")
    c2u = w.cand_to_user
    if cands is not None:
        xc, c2u = xc[cands], c2u[cands]
    return L.lce_baseline(w.values("w"), w.values("x_user"), xc, c2u)


def test_lce_tiny_full():
    w = make_lce("lce_tiny")
    say("case lce_tiny")
    got, errs = _run(w)
    assert errs == 0
    mx, mean = assert_close(got, _oracle(w), "bf16", "lce_tiny")
    say(f"  max {mx:.3g} mean {mean:.3g}")


@pytest.mark.timeout(600)
@pytest.mark.parametrize("name", ["lce_typical", "lce_ratio1000"])
def test_lce_full_size(name):
    """The pages' shape (B=1024, M=433, K=2044, N=256) and a ratio-1000 request;
    every output element against the oracle (evaluated in candidate chunks
    side by side)."""
    w = make_lce(name)
    say(f"case {name} B={w.n_cand} U={w.n_users}")
    got, errs = _run(w)
    assert errs == 0
    ref = np.concatenate(oracle_in_chunks(lambda c: _oracle(w, c), range(w.n_cand)), axis=0)
    mx, mean = assert_close(got, ref, "bf16", name)
    say(f"  whole tensor: max {mx:.3g} mean {mean:.3g}")


EDGE = [
    # users, candidates per user, M, K_u, K_c, N
    (3, (2, 1, 4), 37, 21, 11, 128),
    (2, (3, 2), 129, 65, 1, 256),
    (1, (5,), 433, 200, 130, 128),
    (2, (1, 3), 128, 0, 70, 128),      # no user block
    (2, (2, 2), 200, 50, 0, 384),      # no candidate block: out = the user result
    (4, (1, 1, 1, 1), 1, 1, 1, 128),
]


@pytest.mark.parametrize("i", range(len(EDGE)))
def test_lce_edges(i):
    U, cnt, M, K_u, K_c, N = EDGE[i]
    c2u = np.random.default_rng(70 + i).permutation(np.repeat(np.arange(U), cnt)).astype(np.int32)
    w = make_lce_custom(3000 + i, U, c2u, M, K_u, K_c, N, name=f"lce_edge{i}")
    say(f"case lce edge {EDGE[i]}")
    got, errs = _run(w)
    assert errs == 0
    assert_close(got, _oracle(w), "bf16", f"lce edge {i}")


def test_lce_out_of_range_mapping_gives_zero_rows_and_is_counted():
    w = make_lce_custom(3100, 2, [0, 1, 1, 0], M=40, K_u=10, K_c=9, N=128)
    c2u = np.array([0, 5, 1, -1], np.int32)
    say("case lce bad mapping")
    got, errs = _run(w, c2u=c2u)
    assert errs == 2
    assert np.all(got[1] == 0) and np.all(got[3] == 0)
    ref = L.lce_baseline(w.values("w"), w.values("x_user"), w.values("x_cand")[[0, 2]], c2u[[0, 2]])
    assert_close(got[[0, 2]], ref, "bf16", "lce valid rows")


def test_lce_bitwise_determinism_and_permutation():
    w = make_lce_custom(3200, 3, np.repeat(np.arange(3), [5, 2, 6]).astype(np.int32), M=150, K_u=90, K_c=70, N=256)
    say("case lce determinism / permutation")
    a, _ = _run(w)
    b, _ = _run(w)
    assert np.array_equal(a, b)
    p = np.random.default_rng(9).permutation(w.n_cand)
    w2 = make_lce_custom(3200, 3, w.cand_to_user[p], M=150, K_u=90, K_c=70, N=256)
    w2.tensors = dict(w.tensors)
    w2.tensors["x_cand"] = w.raw("x_cand")[p]
    c, _ = _run(w2)
    assert np.array_equal(c, a[p])


def test_lce_errors():
    import torch
    from broadcast_free_target_amd import IkboError, ikbo_lce_create, ikbo_lce_destroy, ikbo_lce_fwd
    w = make_lce("lce_tiny")
    W = _dev(w.raw("w"))
    say("case lce errors")
    with pytest.raises(IkboError):
        ikbo_lce_create(W, 0, 3, 3)
    with pytest.raises(IkboError):
        ikbo_lce_create(W, w.M, w.K_u, w.K_c, ldw=w.K - 1)
    h = ikbo_lce_create(W, w.M, w.K_u, w.K_c)
    try:
        xu, xc = _dev(w.raw("x_user")), _dev(w.raw("x_cand"))
        m = torch.from_numpy(w.cand_to_user.copy()).cuda()
        out = torch.zeros((w.n_cand, w.M, w.N), dtype=torch.bfloat16, device="cuda")
        with pytest.raises(IkboError):  # N not a multiple of 128
            ikbo_lce_fwd(h, xu, xc, m, w.n_users, w.n_cand, 100, out)
        with pytest.raises(IkboError):  # output aliases an input
            ikbo_lce_fwd(h, xu, xc, m, w.n_users, w.n_cand, w.N, xc)
        with pytest.raises(IkboError):  # candidates but no users
            ikbo_lce_fwd(h, xu, xc, m, 0, w.n_cand, w.N, out)
        ikbo_lce_fwd(h, xu, xc, m, w.n_users, 0, w.N, out)  # no candidates: no-op
        torch.cuda.synchronize()
        assert torch.count_nonzero(out).item() == 0
    finally:
        ikbo_lce_destroy(h)


# ---- three levels: user -> vendor -> item ----

from workloads import make_lce_nested, make_lce_nested_custom  # noqa: E402


def _run3(w, v2u=None, c2v=None, n_users=None, n_vendors=None):
    import torch
    from broadcast_free_target_amd import ikbo_lce3_create, ikbo_lce3_fwd, ikbo_lce_destroy, ikbo_lce_errors
    v2u = w.vendor_to_user if v2u is None else np.asarray(v2u, np.int32)
    c2v = w.cand_to_vendor if c2v is None else np.asarray(c2v, np.int32)
    U = w.n_users if n_users is None else n_users
    V = len(v2u) if n_vendors is None else n_vendors
    W = _dev(w.raw("w"))
    xu = _dev(w.raw("x_user")) if w.K_u > 0 else None
    xv = _dev(w.raw("x_vendor")) if w.K_v > 0 else None
    xc = _dev(w.raw("x_cand")) if w.K_c > 0 else None
    mv = torch.from_numpy(v2u.copy()).cuda()
    mc = torch.from_numpy(c2v.copy()).cuda()
    out = torch.full((len(c2v), w.M, w.N), float("nan"), dtype=torch.bfloat16, device="cuda")
    h = ikbo_lce3_create(W, w.M, w.K_u, w.K_v, w.K_c)
    try:
        ikbo_lce3_fwd(h, xu, xv, xc, mv, mc, U, V, len(c2v), w.N, out)
        torch.cuda.synchronize()
        errs = ikbo_lce_errors(h)
    finally:
        ikbo_lce_destroy(h)
    return out.float().cpu().numpy().astype(np.float64), errs


def _oracle3(w, cands=None):
    xc, c2v = w.values("x_cand"), w.cand_to_vendor
    if cands is not None:
        xc, c2v = xc[cands], c2v[cands]
    return L.lce_baseline_nested(w.values("w"), w.values("x_user"), w.values("x_vendor"), xc, w.vendor_to_user, c2v)


def test_lce3_tiny_full():
    w = make_lce_nested("lce3_tiny")
    say("case lce3_tiny")
    got, errs = _run3(w)
    assert errs == 0
    assert_close(got, _oracle3(w), "bf16", "lce3_tiny")


@pytest.mark.timeout(600)
def test_lce3_typical_full():
    w = make_lce_nested("lce3_typical")
    say(f"case lce3_typical U={w.n_users} V={w.n_vendors} B={w.n_cand}")
    got, errs = _run3(w)
    assert errs == 0
    ref = np.concatenate(oracle_in_chunks(lambda c: _oracle3(w, c), range(w.n_cand)), axis=0)
    mx, mean = assert_close(got, ref, "bf16", "lce3_typical")
    say(f"  whole tensor: max {mx:.3g} mean {mean:.3g}")


EDGE3 = [
    # users, vendor -> user, item -> vendor, M, K_u, K_v, K_c, N
    (2, [1, 0, 1], [2, 0, 0, 2, 1], 40, 10, 9, 8, 128),
    (3, [2, 2, 0, 0], [0, 3, 3, 0, 2], 129, 0, 70, 33, 256),    # no user block; user 1 has no vendor
    (2, [0, 1, 1], [2, 1, 1, 0, 0, 0], 64, 50, 0, 20, 128),     # no vendor block
    (2, [1, 0], [0, 1, 0], 33, 20, 15, 0, 384),                 # no item block
    (1, [0, 0, 0, 0], [3, 3, 1], 300, 65, 64, 1, 128),          # vendors 0 and 2 have no item
]


@pytest.mark.parametrize("i", range(len(EDGE3)))
def test_lce3_edges(i):
    U, v2u, c2v, M, K_u, K_v, K_c, N = EDGE3[i]
    w = make_lce_nested_custom(3800 + i, U, v2u, c2v, M, K_u, K_v, K_c, N, name=f"lce3_edge{i}")
    say(f"case lce3 edge {i}")
    got, errs = _run3(w)
    assert errs == 0
    assert_close(got, _oracle3(w), "bf16", f"lce3 edge {i}")


def test_lce3_out_of_range_entries():
    """A vendor with an out-of-range user contributes zeros (its own part and its
    user's); an item with an out-of-range vendor is written as zeros."""
    w = make_lce_nested_custom(3900, 2, [0, 1, 0], [0, 1, 2, 2], M=40, K_u=10, K_v=9, K_c=8, N=128)
    v2u = np.array([0, 7, 0], np.int32)     # vendor 1 names no user
    c2v = np.array([0, 1, 5, 2], np.int32)  # item 2 names no vendor
    say("case lce3 bad mappings")
    got, errs = _run3(w, v2u=v2u, c2v=c2v)
    assert errs == 2
    assert np.all(got[2] == 0)
    Wc = w.values("w")[:, w.K_u + w.K_v:].astype(np.float64)
    assert_close(got[1:2], (Wc @ w.values("x_cand")[1].astype(np.float64))[None], "bf16", "item of the bad vendor")
    ok = [0, 3]
    ref = L.lce_baseline_nested(w.values("w"), w.values("x_user"), w.values("x_vendor"), w.values("x_cand")[ok],
                                w.vendor_to_user, w.cand_to_vendor[ok])
    assert_close(got[ok], ref, "bf16", "valid items")


def test_lce3_handle_kinds():
    import torch
    from broadcast_free_target_amd import (IkboError, ikbo_lce3_create, ikbo_lce3_fwd, ikbo_lce_create,
                                           ikbo_lce_destroy, ikbo_lce_fwd)
    w = make_lce_nested("lce3_tiny")
    W = _dev(w.raw("w"))
    out = torch.zeros((w.n_cand, w.M, w.N), dtype=torch.bfloat16, device="cuda")
    m = torch.from_numpy(w.cand_to_vendor.copy()).cuda()
    say("case lce3 handle kinds")
    h3 = ikbo_lce3_create(W, w.M, w.K_u, w.K_v, w.K_c)
    h2 = ikbo_lce_create(W, w.M, w.K_u + w.K_v, w.K_c)
    try:
        with pytest.raises(IkboError):
            ikbo_lce_fwd(h3, _dev(w.raw("x_user")), _dev(w.raw("x_cand")), m, w.n_users, w.n_cand, w.N, out)
        with pytest.raises(IkboError):
            ikbo_lce3_fwd(h2, None, None, None, m, m, 1, 1, w.n_cand, w.N, out)
    finally:
        ikbo_lce_destroy(h3)
        ikbo_lce_destroy(h2)


def test_binding_rejects_lce_tensors_that_do_not_fit():
    """The binding compares each tensor with what the call touches (from the
    handle's M, K_u, K_c and the call's sizes): a candidate input one batch
    element short and an fp32 output are refused before anything is launched."""
    import torch
    from broadcast_free_target_amd import IKBO_ERR_INVALID_ARG, IkboError, ikbo_lce_create, ikbo_lce_destroy, ikbo_lce_fwd
    w = make_lce("lce_tiny")
    say("case lce tensors that do not fit")
    h = ikbo_lce_create(_dev(w.raw("w")), w.M, w.K_u, w.K_c)
    try:
        xu, xc = _dev(w.raw("x_user")), _dev(w.raw("x_cand"))
        m = torch.from_numpy(w.cand_to_user.copy()).cuda()
        out = torch.full((w.n_cand, w.M, w.N), 7.0, dtype=torch.bfloat16, device="cuda")
        with pytest.raises(IkboError) as e:
            ikbo_lce_fwd(h, xu, xc[:-1], m, w.n_users, w.n_cand, w.N, out)
        assert e.value.status == IKBO_ERR_INVALID_ARG and "x_cand" in str(e.value)
        with pytest.raises(IkboError) as e:
            ikbo_lce_fwd(h, xu, xc, m, w.n_users, w.n_cand, w.N, out.float())
        assert e.value.status == IKBO_ERR_INVALID_ARG and "element size" in str(e.value)
        torch.cuda.synchronize()
        assert torch.all(out.float() == 7.0)
    finally:
        ikbo_lce_destroy(h)

