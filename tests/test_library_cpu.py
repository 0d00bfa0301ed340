"""CPU-only checks of the library: exports, CSR grouping bit-exact against the
oracle through the C ABI, argument errors, and the work-list planner built
with AddressSanitizer/UBSan."""

import os
import re
import subprocess

import numpy as np
import pytest

from oracle import ikbo_oracle as O
from workloads import make_workload

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "ikbo.h")
CSRC = os.path.join(ROOT, "broadcast_free_target_amd", "csrc")


@pytest.fixture(scope="module")
def lib():
    from broadcast_free_target_amd import ikbo
    return ikbo.load_library()


def _declared_symbols():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(ikbo_[a-z0-9_]+)\s*\(", text)))


def test_header_symbols_exported(lib):
    from broadcast_free_target_amd import ikbo
    names = _declared_symbols()
    assert len(names) >= 12
    for n in names:
        assert hasattr(lib, n), f"{n} declared in ikbo.h but not exported"
    assert sorted(ikbo.SIGNATURES) == names, "binding and header disagree"
    assert lib.ikbo_version() >= 100


CSR_CASES = ["c1_tiny_f32", "c2_typical", "c3_skewed"]


@pytest.mark.parametrize("name", CSR_CASES)
@pytest.mark.parametrize("n_q,bm", [(1, 128), (4, 128), (1, 32), (3, 7)])
def test_csr_bit_exact_vs_oracle(name, n_q, bm):
    from broadcast_free_target_amd import ikbo_group_csr
    w = make_workload(name)
    got = ikbo_group_csr(w.cand_to_user, w.n_users, n_q, bm)
    ref = O.group_csr(w.cand_to_user, w.n_users, n_q, bm)
    for g, key in zip(got, ("counts", "cand_offsets", "cand_perm", "tiles")):
        assert g.dtype == np.int32
        assert np.array_equal(g, ref[key]), key


def test_csr_bit_exact_large_mappings():
    from broadcast_free_target_amd import ikbo_group_csr
    rng = np.random.default_rng(3)
    for U, C in [(150, 10000), (30, 2048), (1, 500), (1000, 999)]:
        c2u = rng.integers(0, U, size=C).astype(np.int32)
        for n_q in (1, 4):
            got = ikbo_group_csr(c2u, U, n_q, 128)
            ref = O.group_csr(c2u, U, n_q, 128)
            assert all(np.array_equal(a, ref[k]) for a, k in zip(got, ("counts", "cand_offsets", "cand_perm", "tiles")))


def test_csr_edge_cases():
    from broadcast_free_target_amd import ikbo_group_csr
    # no candidates
    counts, offs, perm, tiles = ikbo_group_csr(np.zeros(0, np.int32), 3, 1, 128)
    assert counts.tolist() == [0, 0, 0] and offs.tolist() == [0, 0, 0, 0] and perm.size == 0 and tiles.shape[0] == 0
    # users without candidates, sorted and reverse-sorted mappings
    for c2u in ([2, 2, 0, 0, 0], [0, 0, 0, 2, 2], [2, 0, 2, 0, 0]):
        c2u = np.array(c2u, np.int32)
        got = ikbo_group_csr(c2u, 4, 2, 3)
        ref = O.group_csr(c2u, 4, 2, 3)
        assert all(np.array_equal(a, ref[k]) for a, k in zip(got, ("counts", "cand_offsets", "cand_perm", "tiles")))


def test_csr_errors(lib):
    from broadcast_free_target_amd import IKBO_ERR_BAD_MAPPING, IkboError, ikbo_group_csr
    with pytest.raises(IkboError) as e:
        ikbo_group_csr(np.array([0, 3], np.int32), 3, 1, 128)
    assert e.value.status == IKBO_ERR_BAD_MAPPING
    with pytest.raises(IkboError) as e:
        ikbo_group_csr(np.array([-1], np.int32), 3, 1, 128)
    assert e.value.status == IKBO_ERR_BAD_MAPPING
    with pytest.raises(IkboError) as e:
        ikbo_group_csr(np.array([0], np.int32), 0, 1, 128)
    assert e.value.status == IKBO_ERR_BAD_MAPPING


# ---------------------------------------------------------------------------
# work-list planner (host C++, sanitizer build)
# ---------------------------------------------------------------------------

@pytest.fixture(scope="module")
def driver(tmp_path_factory):
    out = str(tmp_path_factory.mktemp("plan") / "plan_driver")
    cmd = ["g++", "-std=c++17", "-O1", "-g", "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
           "-I", CSRC, os.path.join(ROOT, "tests", "csrc", "plan_driver.cpp"), os.path.join(CSRC, "ikbo_plan.cpp"),
           "-o", out]
    subprocess.run(cmd, check=True)
    return out


def _run_driver(driver, offs, c2u, n_q=1, H=2, with_self=0, bm=128, bn=64, grid=512, min_chunk=256, split=1,
                single=0, bins=0, group_span=0, span_tail=0):
    nums = [len(offs) - 1, len(c2u), n_q, H, with_self, bm, bn, grid, min_chunk, split, single, bins, group_span,
            span_tail,
            *offs, *c2u]
    r = subprocess.run([driver], input=" ".join(map(str, nums)), capture_output=True, text=True, check=True,
                       env={**os.environ, "ASAN_OPTIONS": "detect_leaks=1"})
    lines = r.stdout.splitlines()
    rc = int(lines[0].split()[1])
    if rc != 0:
        return rc, None
    _, n_items, grid_, n_groups, n_slots = lines[1].split()
    bins = [int(x) for x in lines[2].split()[1:]]
    perm = np.array(lines[3].split()[1:], dtype=np.int64)
    items = np.array([l.split()[1:] for l in lines[4:]], dtype=np.int64).reshape(-1, 12)
    return 0, dict(n_items=int(n_items), grid=int(grid_), n_groups=int(n_groups), n_slots=int(n_slots),
                   perm=perm, items=items, n_bins=bins[0], bin_off=bins[1:bins[0] + 2] if bins[0] else [0, len(items)])


def _check_plan(plan, offs, c2u, n_q, H, with_self, bm, bn, grid_slots, group_span=0, span_tail=0):
    offs = np.asarray(offs, dtype=np.int64)
    c2u = np.asarray(c2u, dtype=np.int64)
    U = len(offs) - 1
    L = np.diff(offs)
    items = plan["items"]
    assert plan["n_items"] == len(items)
    assert plan["grid"] == min(len(items), grid_slots)
    counts = np.bincount(c2u, minlength=U)
    cand_offsets = np.concatenate([[0], np.cumsum(counts)])

    def user_of(kind, kb, rb):
        if kind == 0:
            us = [u for u in range(U) if offs[u] == kb and cand_offsets[u] == rb and counts[u] > 0]
        else:
            us = [u for u in range(U) if offs[u] == kb and L[u] > 0]
        assert len(us) == 1
        return us[0]

    # group the chunks of each (kind, user, head, row tile)
    tiles = {}
    for it in items:
        kb, rb, r0, nr, a, b, hh, kd, g, ch, nc, s0 = (int(x) for x in it)
        assert 1 <= nr <= bm and 0 <= a <= b and kd in (0, 1)
        if g >= 0:
            assert a % bn == 0 and nc >= 2
        else:
            assert nc == 1 and ch == 0
        u = user_of(kd, kb, rb)
        tiles.setdefault((kd, u, hh, r0, nr), []).append((a, b, g, ch, nc, s0))
    rows = {}
    for (kd, u, hh, r0, nr), chunks in tiles.items():
        chunks.sort()
        assert chunks[0][0] == 0
        for x, y in zip(chunks[:-1], chunks[1:]):
            assert x[1] == y[0]
        assert [c[3] for c in chunks] == list(range(len(chunks)))
        assert len({(c[2], c[4], c[5]) for c in chunks}) == 1
        expect_end = L[u] if kd == 0 else r0 + nr  # causal rows never see past their last token
        assert chunks[-1][1] == expect_end
        rows.setdefault((kd, u, hh), []).append((r0, nr))
    for u in range(U):
        for hh in range(H):
            t = sorted(rows.get((0, u, hh), []))
            assert sum(n for _, n in t) == counts[u] * n_q
            assert all(a + n == b for (a, n), (b, _) in zip(t[:-1], t[1:])) and (not t or t[0][0] == 0)
            s = sorted(rows.get((1, u, hh), []))
            assert sum(n for _, n in s) == (L[u] if with_self else 0)
    # split group g owns slots [8 g, 8 g + nchunk): disjoint, found from g alone
    groups = {}
    for it in items:
        if it[8] >= 0:
            groups.setdefault(int(it[8]), set()).add((int(it[11]), int(it[10])))
    assert all(len(v) == 1 for v in groups.values())
    assert sorted(groups) == list(range(plan["n_groups"])) and plan["n_slots"] == 8 * plan["n_groups"]
    for g, v in groups.items():
        s0, nc = next(iter(v))
        assert s0 == 8 * g and 2 <= nc <= 8
    # longest first within each XCD bin (the whole list when there are none);
    # equal costs keep construction order (user, then target before self, head,
    # row tile, chunk), so one user's tiles stay adjacent.  With group spans:
    # the bin's (user, head) groups by decreasing total cost (ties by
    # user * H + head) in spans of group_span groups, each span's items
    # contiguous and in that same order, then the items of at most span_tail
    # keys, longest first.
    off = plan["bin_off"]
    nb = max(plan["n_bins"], 1)
    assert off[0] == 0 and off[-1] == len(items) and len(off) == nb + 1 and np.all(np.diff(off) >= 0)
    cost = items[:, 5] - items[:, 4]
    key = [(int(it[0]), int(it[7]), int(it[1]) if it[7] == 0 else 0, int(it[6]), int(it[2]), int(it[4]))
           for it in items]
    grp = [user_of(int(it[7]), int(it[0]), int(it[1])) * H + int(it[6]) for it in items]
    gtot = {}
    for g, c in zip(grp, cost):
        gtot[g] = gtot.get(g, 0) + int(c) + 128
    for b in range(nb):
        if group_span and plan["n_bins"]:
            order = sorted(set(grp[off[b]:off[b + 1]]), key=lambda g: (-gtot[g], g))
            span = {g: k // group_span for k, g in enumerate(order)}
            sp = [len(order) if cost[i] <= span_tail else span[grp[i]] for i in range(off[b], off[b + 1])]
            assert sp == sorted(sp)  # spans in order, each span's items contiguous
            runs, a = [], off[b]
            for i in range(off[b] + 1, off[b + 1] + 1):
                if i == off[b + 1] or sp[i - off[b]] != sp[i - 1 - off[b]]:
                    runs.append((a, i))
                    a = i
        else:
            runs = [(off[b], off[b + 1])]
        for a, e in runs:
            assert np.all(np.diff(cost[a:e]) <= 0)
            for i in range(a, e - 1):
                if cost[i] == cost[i + 1]:
                    assert key[i] < key[i + 1], (i, key[i], key[i + 1])
    # the boustrophedon deal over each bin's workgroups (workgroup i serves bin
    # i % n_bins) gives every item to exactly one workgroup
    G = plan["grid"]
    assert G % nb == 0
    hits = np.zeros(len(items), int)
    for i in range(G):
        b, w, Gb = i % nb, i // nb, G // nb
        p = 0
        while True:
            pos = off[b] + p * Gb + ((Gb - 1 - w) if p & 1 else w)
            if pos >= off[b + 1]:
                break
            hits[pos] += 1
            p += 1
    assert np.all(hits == 1)
    if plan["n_bins"]:
        # every (user, head) -- all its tiles, both kinds, all chunks -- in one bin
        where = {}
        for b in range(nb):
            for it in items[off[b]:off[b + 1]]:
                u = user_of(int(it[7]), int(it[0]), int(it[1]))
                assert where.setdefault((u, int(it[6])), b) == b
        # greedy largest-first filling: no bin exceeds the mean load by more than
        # the largest (user, head) cost
        gcost = {}
        for it in items:
            u = user_of(int(it[7]), int(it[0]), int(it[1]))
            gcost[(u, int(it[6]))] = gcost.get((u, int(it[6])), 0) + int(it[5] - it[4]) + 128
        load = np.zeros(nb)
        for g, c in gcost.items():
            load[where[g]] += c
        assert load.max() <= load.mean() + max(gcost.values()) + 1e-9
    assert np.array_equal(plan["perm"], np.argsort(c2u, kind="stable"))


@pytest.mark.parametrize("name", ["c2_typical", "c3_skewed", "c5_fused"])
def test_planner_on_configs(driver, name):
    w = make_workload(name) if name != "c5_fused" else None
    if w is None:
        rng = np.random.Generator(np.random.PCG64(1005))
        L = rng.integers(256, 2048, size=30, endpoint=True)
        counts = rng.multinomial(2048, [1 / 30] * 30)
        c2u = rng.permutation(np.repeat(np.arange(30), counts)).astype(np.int32)
        offs = np.concatenate([[0], np.cumsum(L)]).astype(np.int32)
        n_q, H, with_self = 1, 4, 1
    else:
        offs, c2u, n_q, H, with_self = w.user_offsets, w.cand_to_user, w.n_q, w.H, 0
    for grid, min_chunk in [(512, 256), (64, 128), (8, 64), (1, 256)]:
        rc, plan = _run_driver(driver, offs, c2u, n_q=n_q, H=H, with_self=with_self, grid=grid, min_chunk=min_chunk)
        assert rc == 0
        _check_plan(plan, offs, c2u, n_q, H, with_self, 128, 64, grid)


@pytest.mark.parametrize("name", ["c3_skewed", "c4_large", "c5_fused"])
def test_planner_xcd_bins(driver, name):
    """Multi-pass plans with XCD bins: every invariant above, plus each (user,
    head) in one bin, each bin longest first and dealt over its own workgroups,
    and bin loads within one (user, head) of the mean."""
    if name == "c5_fused":
        rng = np.random.Generator(np.random.PCG64(1005))
        L = rng.integers(256, 2048, size=30, endpoint=True)
        counts = rng.multinomial(2048, [1 / 30] * 30)
        c2u = rng.permutation(np.repeat(np.arange(30), counts)).astype(np.int32)
        offs = np.concatenate([[0], np.cumsum(L)]).astype(np.int32)
        n_q, H, with_self = 1, 4, 1
    else:
        w = make_workload(name)
        offs, c2u, n_q, H, with_self = w.user_offsets, w.cand_to_user, w.n_q, w.H, 0
    for grid in (512, 64, 8):
        for span, tail in ((0, 0), (1, 0), (3, 0), (2, 256)):
            rc, plan = _run_driver(driver, offs, c2u, n_q=n_q, H=H, with_self=with_self, grid=grid, bins=8,
                                   group_span=span, span_tail=tail)
            assert rc == 0
            assert plan["n_bins"] == (8 if plan["n_items"] > plan["grid"] else 0)
            _check_plan(plan, offs, c2u, n_q, H, with_self, 128, 64, grid, group_span=span, span_tail=tail)
    # a grid that is not a multiple of the bin count keeps one list
    rc, plan = _run_driver(driver, offs, c2u, n_q=n_q, H=H, with_self=with_self, grid=37, bins=8)
    assert rc == 0 and plan["n_bins"] == 0
    _check_plan(plan, offs, c2u, n_q, H, with_self, 128, 64, 37)


def _single_pass_count(lens, c, bn, max_chunks=8):
    """Items the single-pass rule makes for chunk length c (mirrors its definition)."""
    n = 0
    for L in lens:
        if L == 0:
            n += 1
            continue
        floor_len = -(-(-(-L // max_chunks)) // bn) * bn
        n += -(-L // max(c, floor_len))
    return n


@pytest.mark.parametrize("name", ["c2_typical", "c3_skewed", "c5_fused"])
def test_planner_single_pass(driver, name):
    """Single pass (fewer unsplit items than workgroups): at most grid items, and
    the chunk length is the shortest multiple of bn (>= min_chunk) that fits;
    every plan invariant still holds."""
    if name == "c5_fused":
        rng = np.random.Generator(np.random.PCG64(1005))
        L = rng.integers(256, 2048, size=30, endpoint=True)
        counts = rng.multinomial(2048, [1 / 30] * 30)
        c2u = rng.permutation(np.repeat(np.arange(30), counts)).astype(np.int32)
        offs = np.concatenate([[0], np.cumsum(L)]).astype(np.int32)
        n_q, H, with_self = 1, 4, 1
    else:
        w = make_workload(name)
        offs, c2u, n_q, H, with_self = w.user_offsets, w.cand_to_user, w.n_q, w.H, 0
    bn, bm = 128, 128
    for grid, min_chunk in [(256, 256), (1024, 128), (64, 256)]:
        rc, plan = _run_driver(driver, offs, c2u, n_q=n_q, H=H, with_self=with_self, bm=bm, bn=bn, grid=grid,
                               min_chunk=min_chunk, single=1)
        assert rc == 0
        _check_plan(plan, offs, c2u, n_q, H, with_self, bm, bn, grid)
        Ls = np.diff(np.asarray(offs, dtype=np.int64))
        counts = np.bincount(np.asarray(c2u, dtype=np.int64), minlength=len(Ls))
        lens = []
        for u in range(len(Ls)):
            lens += [int(Ls[u])] * (H * (-(-int(counts[u]) * n_q // bm)))
            if with_self:
                lens += [min(r0 + bm, int(Ls[u])) for r0 in range(0, int(Ls[u]), bm) for _ in range(H)]
        items = plan["items"]
        if len(lens) >= grid:
            continue  # more unsplit items than workgroups: the cost rule applies (checked above)
        assert len(items) <= grid
        # the shortest admissible chunk length, searched independently
        lo = max(bn, -(-min_chunk // bn) * bn)
        c = lo
        while _single_pass_count(lens, c, bn) > grid:
            c += bn
        assert len(items) == _single_pass_count(lens, c, bn)
        ends = {}  # split group -> end of its key range
        for it in items:
            if it[8] >= 0:
                ends[int(it[8])] = max(ends.get(int(it[8]), 0), int(it[5]))
        for it in items:  # no chunk longer than the rule allows for its range
            if it[8] >= 0:
                L = ends[int(it[8])]
                floor_len = -(-(-(-L // 8)) // bn) * bn
                assert int(it[5]) - int(it[4]) <= max(c, floor_len)


def test_planner_edge_cases(driver):
    cases = [
        ([0, 0, 5, 5], [1, 1, 0, 2]),          # zero-length users holding candidates
        ([0, 1, 2], [0, 1, 1, 1, 0]),           # length-1 users
        ([0, 3000], list(range(1)) * 3),        # one long user, few rows: split
        ([0, 100, 200], []),                    # no candidates
    ]
    for offs, c2u in cases:
        for ws in (0, 1):
            rc, plan = _run_driver(driver, offs, c2u, n_q=2 if not ws else 1, H=3, with_self=ws)
            assert rc == 0
            _check_plan(plan, offs, c2u, 2 if not ws else 1, 3, ws, 128, 64, 512)
    rc, _ = _run_driver(driver, [1, 2], [0])
    assert rc == -2
    rc, _ = _run_driver(driver, [0, 2, 1], [0])
    assert rc == -2
    rc, _ = _run_driver(driver, [0, 2], [1])
    assert rc == -3


class _FakeDeviceTensor:
    """Stands in for a device tensor: the binding's size check reads only these."""

    def __init__(self, numel, elem, contiguous=True, cuda=True):
        self.is_cuda, self._n, self._e, self._c = cuda, numel, elem, contiguous
        self.dtype = f"{elem}-byte"

    def numel(self):
        return self._n

    def element_size(self):
        return self._e

    def is_contiguous(self):
        return self._c


def test_binding_rejects_buffers_smaller_than_the_call_touches():
    """The C ABI gets bare pointers, so the binding compares each tensor with
    the extent the call will read or write before anything is launched."""
    from broadcast_free_target_amd import IKBO_ERR_INVALID_ARG, IkboError
    from broadcast_free_target_amd.ikbo import _need
    _need(None, 100, "x")
    _need(12345, 100, "x")  # raw pointers are the caller's to size
    _need(_FakeDeviceTensor(50, 2), 100, "x", 2)
    cases = [(_FakeDeviceTensor(49, 2), 2, "bytes, the call needs"),
             (_FakeDeviceTensor(50, 4), 2, "element size"),       # an fp32 tensor where bf16 is expected
             (_FakeDeviceTensor(50, 2, contiguous=False), 2, "contiguous"),
             (_FakeDeviceTensor(50, 2, cuda=False), 2, "device tensor")]
    for t, elem, msg in cases:
        with pytest.raises(IkboError) as e:
            _need(t, 100, "x", elem)
        assert e.value.status == IKBO_ERR_INVALID_ARG and msg in str(e.value)


def test_binding_host_array_addresses():
    """Host mapping arrays go to the C side as addresses: contiguous int32 only,
    the array's own buffer (cached per array, never another array's)."""
    from broadcast_free_target_amd import IkboError
    from broadcast_free_target_amd.ikbo import _host_i32
    a = np.arange(10, dtype=np.int32)
    b = np.arange(10, dtype=np.int32)
    assert _host_i32(a) == a.ctypes.data and _host_i32(a) == a.ctypes.data
    assert _host_i32(b) == b.ctypes.data != a.ctypes.data
    assert _host_i32(np.zeros(0, np.int32)) is None
    for bad in (np.arange(10, dtype=np.int64), np.arange(20, dtype=np.int32)[::2]):
        with pytest.raises(IkboError):
            _host_i32(bad)
    for _ in range(20):  # more arrays than the cache keeps: each still maps to its own buffer
        c = np.arange(5, dtype=np.int32)
        assert _host_i32(c) == c.ctypes.data
