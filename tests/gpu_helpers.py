"""Helpers shared by the GPU tests: upload a workload, run the library, compare."""

from __future__ import annotations

import os
import sys

import numpy as np

BF16_MAX_ABS = 2e-2
BF16_MEAN_ABS = 2e-3
F32_MAX_ABS = 1e-4


def say(msg: str) -> None:
    print(msg, flush=True)
    sys.stdout.flush()


def dev_tensor(arr: np.ndarray, dtype: str):
    import torch
    if dtype == "bf16":
        t = torch.from_numpy(np.ascontiguousarray(arr).view(np.int16)).cuda().view(torch.bfloat16)
    else:
        t = torch.from_numpy(np.ascontiguousarray(arr, dtype=np.float32)).cuda()
    return t


def upload(w):
    import torch
    d = {name: dev_tensor(w.raw(name), w.dtype) for name in w.tensors}
    d["user_offsets"] = torch.from_numpy(w.user_offsets.copy()).cuda()
    d["cand_to_user"] = torch.from_numpy(w.cand_to_user.copy()).cuda()
    return d


def to_f64(t) -> np.ndarray:
    import torch
    return t.float().cpu().numpy().astype(np.float64) if t.dtype == torch.bfloat16 else t.cpu().numpy().astype(np.float64)


def empty_out(shape, dtype: str, fill=float("nan")):
    import torch
    tdt = torch.bfloat16 if dtype == "bf16" else torch.float32
    return torch.full(shape, fill, dtype=tdt, device="cuda")


def dtype_code(dtype: str) -> int:
    from broadcast_free_target_amd import IKBO_DTYPE_BF16, IKBO_DTYPE_F32
    return IKBO_DTYPE_BF16 if dtype == "bf16" else IKBO_DTYPE_F32


def assert_close(got: np.ndarray, ref: np.ndarray, dtype: str, what: str = ""):
    assert got.shape == ref.shape, (got.shape, ref.shape)
    assert np.all(np.isfinite(got)), f"{what}: non-finite output"
    err = np.abs(got - ref)
    mx = float(err.max()) if err.size else 0.0
    mean = float(err.mean()) if err.size else 0.0
    if dtype == "bf16":
        assert mx <= BF16_MAX_ABS and mean <= BF16_MEAN_ABS, f"{what}: max {mx:.3g} mean {mean:.3g}"
    else:
        assert mx <= F32_MAX_ABS, f"{what}: max {mx:.3g}"
    return mx, mean


def run_planned(w, dev, out_cand, out_user=None, stream=None):
    """Host grouping from host arrays + planned launch: the path bench.py times."""
    from broadcast_free_target_amd import (ikbo_attn_fwd_planned, ikbo_plan_create, ikbo_plan_destroy,
                                           ikbo_plan_info)
    plan = ikbo_plan_create(w.user_offsets, w.cand_to_user, w.n_users, w.n_cand, w.n_q, w.H, w.d,
                            dtype_code(w.dtype), 1 if out_user is not None else 0, stream)
    try:
        info = ikbo_plan_info(plan)
        ikbo_attn_fwd_planned(plan, dev["q_cand"], dev.get("q_user") if out_user is not None else None,
                              dev["k_user"], dev["v_user"], w.scale, out_cand, out_user, stream)
        import torch
        torch.cuda.synchronize()
    finally:
        ikbo_plan_destroy(plan)
    return info


def host_workers(cap: int = 16) -> int:
    """Threads for oracle evaluations: the cores this process may use, at most cap."""
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        n = os.cpu_count() or 1
    return max(1, min(cap, n))


def oracle_in_chunks(fn, items, workers=None):
    """Runs fn(chunk) over chunks of `items` in a thread pool, in order, with
    the BLAS pool of each call limited to one thread (numpy releases the
    interpreter lock in its copies and products, so the chunks run side by
    side).  fn is an oracle call on a subset; the results are returned as a
    list in chunk order."""
    from concurrent.futures import ThreadPoolExecutor
    from threadpoolctl import threadpool_limits
    workers = workers or host_workers()
    items = list(items)
    n_chunks = max(1, min(len(items), 8 * workers))
    chunks = [c for c in np.array_split(np.asarray(items), n_chunks) if len(c)]
    with threadpool_limits(1), ThreadPoolExecutor(workers) as ex:
        return list(ex.map(fn, chunks))


def oracle_in_processes(fn, arg_list, workers=None):
    """Runs fn(*args) for every args in arg_list in a pool of fresh worker
    processes (spawned: nothing of this process's GPU state is inherited;
    the workers never touch the GPU), for oracle code that is bound by the
    interpreter rather than by numpy's kernels.  fn must be importable at
    module level.  Results come back in order."""
    import multiprocessing
    from concurrent.futures import ProcessPoolExecutor
    workers = workers or host_workers()
    ctx = multiprocessing.get_context("spawn")
    with ProcessPoolExecutor(max_workers=workers, mp_context=ctx) as ex:
        return list(ex.map(_call_star, [(fn, a) for a in arg_list], chunksize=1))


def _call_star(fa):
    import os
    os.environ.setdefault("OMP_NUM_THREADS", "1")
    fn, args = fa
    return fn(*args)


def mx_user_oracle(q_codes, q_scales, k_codes, k_scales, v_codes, v_scales, scale):
    """The MXFP8 oracle on one user's request: its candidates' query codes and
    scales, its key and value rows and its value-scale blocks (offsets [0, L],
    every candidate mapped to user 0)."""
    import numpy as np
    from oracle import mxfp8_oracle as M
    L = k_codes.shape[0]
    return M.target_attention_mxfp8(q_codes, q_scales, k_codes, k_scales, v_codes, v_scales,
                                    np.array([0, L], np.int32), np.zeros(q_codes.shape[0], np.int32), scale)
