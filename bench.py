"""Benchmark of IKBO target attention on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--config c2_typical]

One step is the whole hot path for one request batch, one library call
(ikbo_attn_fwd_hostmap): validation, the host grouping pass and work list
built from the host copy of the candidate-to-user mapping (as an inference
runtime holds it) into pinned memory that the kernels read in place, the
persistent attention kernel and, when key ranges were split, the merge
kernel.  Inputs are resident in HBM before timing.
Rank 0 prints one JSON line (the contract fields plus ``roofline`` and
``cpu_baseline``).  Under ``extra`` it also carries cold-cache kernel times,
the host time of a plan build and of a launch, the end-to-end time of the
device-mapping entry point and the materialised-broadcast comparator's time.
"""

from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "IKBO attn BF16 TFLOP/s (+% MFMA peak) and HBM bytes vs materialized broadcast"
PEAK_HBM_GBS = 8000.0
PEAK_BF16_TFLOPS = 2500.0
PEAK_F32_TFLOPS = 157.3
# Attention kernel a plan runs (ikbo_plan_info "kernel"), by head dim.
KERNEL_NAMES = {0: "ikbo_attn_f32_kernel<{d}>", 1: "ikbo_attn_bf16_w8_kernel<{d}, 2>",
                2: "ikbo_attn_bf16_kernel<{d}, 2>",
                4: "ikbo_attn_bf16_kernel<{d}, 2>"}  # 4: the 4-wave kernel visiting key tiles in reverse
MERGE_KERNEL = "ikbo_merge_kernel<{d}, true>"

WORKLOAD_TEXT = {
    "c1_tiny_f32": "tiny fp32: 4 users, L~U[16,64], 20 candidates, n_q=1, H=2, d=32",
    "c2_typical": "typical request: 1024 candidates over 15 users (multinomial), L~U[256,2048], n_q=1, H=4, d=128, bf16",
    "c3_skewed": "skewed: 1023 candidates over 32 users (Zipf 1.2), L~U[1,4096] with two L=1 users, n_q=1, H=4, d=128, bf16",
    "c4_large": "large: 10000 candidates over 150 users, L~U[512,4096], n_q=4, H=8, d=128, bf16",
    "c5_fused": "fused self+target: 2048 candidates over 30 users, causal self over L~U[256,2048], H=4, d=128, bf16",
    "p_app11": "App. 11 shape: 32 users x 64 candidates, n_q=64, L=1024, H=2, d=128, bf16",
    "mx_c2_typical": "MXFP8 typical request: 1024 candidates over 15 users, L~U[256,2048], n_q=1, H=4, d=128, E4M3 codes with E8M0 scales per 32",
    "mx_c4_large": "MXFP8 large request: 10,000 candidates over 150 users, L~U[512,4096], n_q=4, H=8, d=128, E4M3 codes with E8M0 scales per 32",
    "bwd_c2_typical": "backward of the typical request: 1024 candidates over 15 users, L~U[256,2048], n_q=1, H=4, d=128, bf16",
    "bwd_c4_large": "backward of the large request: 10000 candidates over 150 users, L~U[512,4096], n_q=4, H=8, d=128, bf16",
    "lce3_typical": "three-level linear compression: 1024 items over 120 vendors over 15 users, M=433, K_u=682, K_v=K_c=681, N=256, bf16",
    "lce_typical": "linear compression: 1024 candidates over 15 users, M=433, K_u=K_c=1022, N=256, bf16",
    "lce_ratio1000": "linear compression: 2000 candidates over 2 users, M=433, K_u=K_c=1022, N=256, bf16",
}
LCE_METRIC = "IKBO linear compression BF16 TFLOP/s (executed work) and FLOPs vs materialized broadcast"
BWD_METRIC = "IKBO attn backward BF16 TFLOP/s (five products: S, dP, dV, dK, dQ)"
BWD_KERNELS = ("ikbo_bwd_dq_kernel", "ikbo_bwd_dkv_kernel")
MX_METRIC = "IKBO attn MXFP8 TFLOP/s (QK^T and PV on block-scaled FP8 MFMA)"
MX_KERNEL = "ikbo_attn_mx_kernel"
PEAK_FP8_TFLOPS = 5000.0
LCE_KERNEL = "ikbo_lce_gemm_kernel<1>"  # candidate GEMM with the broadcast-add epilogue


def algorithmic_counts(w):
    """FLOPs (FA convention, softmax not counted) and HBM bytes of one step."""
    L = w.lengths.astype(np.float64)
    cnt = w.counts.astype(np.float64)
    elem = 2 if w.dtype == "bf16" else 4
    flops = 4.0 * w.n_q * w.d * w.H * float(np.dot(cnt, L))
    rows = w.n_cand * w.n_q
    byts = elem * w.H * w.d * (2.0 * rows + 2.0 * w.total_len)  # Q read + O write, K + V once
    if w.with_self:
        flops += 4.0 * w.d * w.H * float(np.sum(L * (L + 1.0) / 2.0))
        byts += 2.0 * elem * w.H * w.d * w.total_len  # q_user read + out_user write
    bcast_len = float(np.dot(cnt, L))
    mat_bytes = elem * w.H * w.d * (2.0 * rows + 2.0 * w.total_len) + 2.0 * 2.0 * elem * w.H * w.d * bcast_len
    return flops, byts, mat_bytes


def lce_counts(w):
    """Algorithmic FLOPs and HBM bytes of one linear-compression call, per kernel.

    user GEMM:      2 M N U K_u flops; reads W_u, x_user, writes y (fp32)
    candidate GEMM: 2 M N B K_c flops; reads W_c, x_cand, y once per user, writes out
    baseline:       2 M N B (K_u + K_c) flops on the materialised concatenation
    """
    U, B, M, K_u, K_c, N = w.n_users, w.n_cand, w.M, w.K_u, w.K_c, w.N
    f_user = 2.0 * M * N * U * K_u
    f_cand = 2.0 * M * N * B * K_c
    b_user = 2.0 * (M * K_u + U * K_u * N) + 4.0 * U * M * N
    b_cand = 2.0 * (M * K_c + B * K_c * N + B * M * N) + 4.0 * U * M * N
    f_base = 2.0 * M * N * B * (K_u + K_c)
    b_base = 2.0 * (M * (K_u + K_c) + B * (K_u + K_c) * N + B * M * N)
    return f_user, f_cand, b_user, b_cand, f_base, b_base


def bwd_counts(w):
    """Algorithmic FLOPs and HBM bytes of one backward call, whole and per kernel.

    FLOPs: 2 per multiply-add, softmax not counted; per (candidate row, head,
    key) the five products S, dP, dV, dK, dQ take 2*d each.  The dQ kernel
    must form S, dP and dQ; the dK/dV kernel S, dP, dV and dK.
    Bytes (bf16): dQ kernel reads Q, O, dO, the forward's log-sum-exp and the
    user's K and V once per (user, head), writes dQ; dK/dV kernel reads K, V, Q
    and dO once, writes dK and dV (per-row statistics, 8 bytes per row and
    head, are counted too).
    """
    L = w.lengths.astype(np.float64)
    cnt = w.counts.astype(np.float64)
    per = 2.0 * w.d * w.H * w.n_q * float(np.dot(cnt, L))   # one product over all rows and keys
    rows = float(w.n_cand * w.n_q)
    act = 2.0 * w.H * w.d                                   # bytes of one row (all heads)
    kv_users = float(np.sum(L[cnt > 0]))                      # keys of users that have candidates
    b_dq = act * (4.0 * rows + 2.0 * kv_users) + 12.0 * rows * w.H  # + the given log-sum-exp read
    b_dkv = act * (2.0 * rows + 4.0 * w.total_len) + 8.0 * rows * w.H
    return 5.0 * per, 3.0 * per, 4.0 * per, b_dq, b_dkv


def kernel_source_hash(files=("ikbo_kernels.hip", "ikbo_kernels.h", "ikbo_device.h", "ikbo_plan.cpp",
                              "ikbo_plan.h", "ikbo_api.hip", "ikbo_api_common.h")):
    h = hashlib.sha256()
    for f in files:
        with open(os.path.join(ROOT, "broadcast_free_target_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


LCE_SOURCES = ("ikbo_lce.hip", "ikbo_lce.h", "ikbo_device.h", "ikbo_api_lce.hip", "ikbo_api_common.h")
MX_SOURCES = ("ikbo_mx.hip", "ikbo_mx.h", "ikbo_device.h", "ikbo_plan.cpp", "ikbo_plan.h", "ikbo_api_mx.hip",
              "ikbo_api_common.h")
BWD_SOURCES = ("ikbo_bwd.hip", "ikbo_bwd.h", "ikbo_device.h", "ikbo_plan.cpp", "ikbo_plan.h", "ikbo_api_bwd.hip",
               "ikbo_api_common.h")


def traffic_from_profiles(workload):
    """Per-launch HBM bytes from the committed rocprofv3 --pmc summary, if it
    was taken on the current kernel sources; else None."""
    lce = workload.startswith("lce")
    bwd = workload.startswith("bwd_")
    mx = workload.startswith("mx_")
    name = (f"ikbo_lce_gemm_{workload}_pmc.json" if lce else f"ikbo_bwd_{workload}_pmc.json" if bwd
            else f"ikbo_attn_mx_{workload}_pmc.json" if mx else f"ikbo_attn_bf16_{workload}_pmc.json")
    path = os.path.join(ROOT, "profiles", name)
    if not os.path.exists(path):
        return None
    try:
        with open(path) as fh:
            s = json.load(fh)
        want = (kernel_source_hash(LCE_SOURCES) if lce else kernel_source_hash(BWD_SOURCES) if bwd
                else kernel_source_hash(MX_SOURCES) if mx else kernel_source_hash())
        if s.get("kernel_source_hash") != want:
            return None
        if not (lce or bwd or mx) and "hbm_bytes_per_step_with_merge" in s:
            return float(s["hbm_bytes_per_step_with_merge"])  # attention kernel + merge, as the roofline
        return float(s["hbm_bytes_per_launch"])
    except Exception:
        return None


def materialized_traffic_from_profiles(workload):
    """HBM bytes of one materialised-broadcast step (copy kernel + attention)
    from the committed rocprofv3 --pmc summary of --materialized-only, if it was
    taken on the current kernel sources; else None."""
    path = os.path.join(ROOT, "profiles", f"ikbo_materialized_{workload}_pmc.json")
    if not os.path.exists(path):
        return None
    try:
        with open(path) as fh:
            s = json.load(fh)
        if s.get("kernel_source_hash") != kernel_source_hash():
            return None
        return float(s["hbm_bytes_per_step_with_merge"])
    except Exception:
        return None


def upload(w):
    import torch
    t = {}
    for name in w.tensors:
        a = np.ascontiguousarray(w.raw(name))
        if w.dtype == "bf16":
            t[name] = torch.from_numpy(a.view(np.int16)).cuda().view(torch.bfloat16)
        else:
            t[name] = torch.from_numpy(a).cuda()
    t["user_offsets"] = torch.from_numpy(w.user_offsets.copy()).cuda()
    t["cand_to_user"] = torch.from_numpy(w.cand_to_user.copy()).cuda()
    return t


def cpu_baseline(w, reps):
    """The fp64 oracle as it stands, timed on this host's cores."""
    from oracle import ikbo_oracle as O
    try:
        from threadpoolctl import threadpool_info
        threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:
        threads = 1
    q, k, v = w.values("q_cand"), w.values("k_user"), w.values("v_user")
    flops, _, _ = algorithmic_counts(w)
    times = []
    for _ in range(reps):
        t0 = time.perf_counter()
        O.target_attention(q, k, v, w.user_offsets, w.cand_to_user, w.scale)
        if w.with_self:
            O.self_attention_causal(w.values("q_user"), k, v, w.user_offsets, w.scale)
        times.append(time.perf_counter() - t0)
    t = float(np.median(times))
    return {"value": flops / t / 1e12, "unit": "TFLOP/s", "cores": int(threads), "kind": "oracle",
            "sample": f"whole {w.name} batch ({w.n_cand} candidates), fp64 numpy with explicit per-candidate "
                      f"K/V replication, median of {reps} runs of {t:.2f} s",
            "seconds": t, "cands_per_s": w.n_cand / t}


def cpu_baseline_lce(w, n_sample, reps):
    """The fp64 oracle (explicit per-candidate concatenation) on the first
    n_sample candidates; its time is scaled to the whole batch and the rate is
    counted in the same executed FLOPs as the GPU figure."""
    from oracle import lce_oracle as O
    try:
        from threadpoolctl import threadpool_info
        threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:
        threads = 1
    wv, xu, xc = w.values("w"), w.values("x_user"), w.values("x_cand")[:n_sample]
    c2u = w.cand_to_user[:n_sample]
    times = []
    for _ in range(reps):
        t0 = time.perf_counter()
        O.lce_baseline(wv, xu, xc, c2u)
        times.append(time.perf_counter() - t0)
    t = float(np.median(times))
    f_user, f_cand, _, _, _, _ = lce_counts(w)
    t_whole = t * w.n_cand / n_sample
    return {"value": (f_user + f_cand) / t_whole / 1e12, "unit": "TFLOP/s", "cores": int(threads), "kind": "oracle",
            "sample": f"first {n_sample} of {w.n_cand} candidates of {w.name}, fp64 numpy with explicit "
                      f"per-candidate concatenation, median of {reps} runs of {t:.2f} s, scaled to the whole batch "
                      f"and counted in the same executed FLOPs as the GPU value",
            "seconds_whole_batch": t_whole, "cands_per_s": w.n_cand / t_whole}


def cpu_baseline_bwd(w, n_sample, reps):
    """The fp64 backward oracle on the first n_sample candidates (all keys of
    their users), scaled to the whole batch by candidate count."""
    from oracle import ikbo_bwd_oracle as B
    try:
        from threadpoolctl import threadpool_info
        threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:
        threads = 1
    sel = np.arange(min(n_sample, w.n_cand))
    q, do = w.values("q_cand")[sel], w.values("dout")[sel]
    k, v = w.values("k_user"), w.values("v_user")
    times = []
    for _ in range(reps):
        t0 = time.perf_counter()
        B.target_attention_bwd(q, k, v, do, w.user_offsets, w.cand_to_user[sel], w.scale)
        times.append(time.perf_counter() - t0)
    t = float(np.median(times))
    flops = bwd_counts(w)[0]
    t_whole = t * w.n_cand / len(sel)
    return {"value": flops / t_whole / 1e12, "unit": "TFLOP/s", "cores": int(threads), "kind": "oracle",
            "sample": f"first {len(sel)} of {w.n_cand} candidates of {w.name}, fp64 numpy with explicit per-candidate "
                      f"K/V copies, median of {reps} runs of {t:.2f} s, scaled to the whole batch",
            "seconds_whole_batch": t_whole}


def main_bwd(args):
    """One step = one ikbo_attn_bwd call: host grouping and work lists from the
    host mapping, the dQ kernel and the dK/dV kernel.  The forward output and
    the rows' log-sum-exp it consumes are produced once, before timing, by the
    training forward (ikbo_attn_fwd_train), as a training step would."""
    import torch
    import broadcast_free_target_amd as ikbo
    from workloads import make_bwd_workload

    cfg = args.config[len("bwd_"):]
    w = make_bwd_workload(cfg)
    dev = upload(w)
    out = torch.empty_like(dev["q_cand"])
    lse = torch.empty((w.n_cand, w.n_q, w.H), dtype=torch.float32, device="cuda")
    stream = torch.cuda.current_stream()
    offs_h = np.ascontiguousarray(w.user_offsets, dtype=np.int32)
    c2u_h = np.ascontiguousarray(w.cand_to_user, dtype=np.int32)
    fplan = ikbo.ikbo_plan_create(offs_h, c2u_h, w.n_users, w.n_cand, w.n_q, w.H, w.d, ikbo.IKBO_DTYPE_BF16, 0, stream)
    ikbo.ikbo_attn_fwd_train(fplan, dev["q_cand"], dev["k_user"], dev["v_user"], w.scale, out, lse, stream)
    torch.cuda.synchronize()
    ikbo.ikbo_plan_destroy(fplan)
    dq = torch.empty_like(dev["q_cand"])
    dk = torch.empty_like(dev["k_user"])
    dv = torch.empty_like(dev["v_user"])
    h = ikbo.ikbo_bwd_create()
    given = [lse]

    def step():
        ikbo.ikbo_attn_bwd(h, offs_h, c2u_h, w.n_users, w.n_cand, w.n_q, w.H, w.d, w.scale, dev["q_cand"],
                           dev["k_user"], dev["v_user"], out, dev["dout"], dq, dk, dv, stream, lse=given[0])

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    K = args.steps
    t0 = time.perf_counter()
    for _ in range(K):
        step()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ikbo.ikbo_bwd_timing(h, True)
    for _ in range(K):
        step()
    torch.cuda.synchronize()
    dq_ms, dkv_ms = ikbo.ikbo_bwd_timing_read(h, K)
    ikbo.ikbo_bwd_timing(h, False)
    info = ikbo.ikbo_bwd_info(h)
    # the same calls with the log-sum-exp recomputed by the dQ kernel (for
    # comparison; not with --kernel-only, which profiles the timed calls alone)
    dq_re_ms = [float("nan")]
    if not args.kernel_only:
        given[0] = None
        ikbo.ikbo_bwd_timing(h, True)
        for _ in range(K):
            step()
        torch.cuda.synchronize()
        dq_re_ms, _ = ikbo.ikbo_bwd_timing_read(h, K)
        ikbo.ikbo_bwd_timing(h, False)
    ikbo.ikbo_bwd_destroy(h)
    a_ms, b_ms = float(np.mean(dq_ms)), float(np.mean(dkv_ms))

    f_all, f_dq, f_dkv, b_dq, b_dkv = bwd_counts(w)
    ms_per_step = wall * 1e3 / K
    value = f_all / (ms_per_step * 1e-3) / 1e12
    dom = 0 if a_ms >= b_ms else 1
    f_k, b_k, t_k = (f_dq, b_dq, a_ms) if dom == 0 else (f_dkv, b_dkv, b_ms)
    if f_k / b_k < PEAK_BF16_TFLOPS * 1e12 / (PEAK_HBM_GBS * 1e9):
        achieved = b_k / (t_k * 1e-3) / 1e9
        roof = {"bound": "hbm", "achieved": achieved, "peak": PEAK_HBM_GBS, "unit": "GB/s", "frac": achieved / PEAK_HBM_GBS}
    else:
        achieved = f_k / (t_k * 1e-3) / 1e12
        roof = {"bound": "mfma", "achieved": achieved, "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                "frac": achieved / PEAK_BF16_TFLOPS}
    roof["traffic"] = traffic_from_profiles(args.config)
    roof["kernel"] = BWD_KERNELS[dom]
    roof["kernel_avg_us"] = t_k * 1e3
    roof["algorithmic_bytes_per_launch"] = b_k
    roof["algorithmic_flops_per_launch"] = f_k
    extra = {
        "dq_kernel_us": a_ms * 1e3, "dkv_kernel_us": b_ms * 1e3,
        "dq_kernel_us_lse_recomputed": float(np.mean(dq_re_ms)) * 1e3,
        "dq_kernel_tflops": f_dq / (a_ms * 1e-3) / 1e12, "dkv_kernel_tflops": f_dkv / (b_ms * 1e-3) / 1e12,
        "dq_kernel_hbm_gbs": b_dq / (a_ms * 1e-3) / 1e9, "dkv_kernel_hbm_gbs": b_dkv / (b_ms * 1e-3) / 1e9,
        "kernels_tflops": f_all / ((a_ms + b_ms) * 1e-3) / 1e12,
        "work_items": info, "backward_flops": f_all, "forward_flops": w.flops()["target"],
    }
    result = {
        "metric": BWD_METRIC, "value": value, "unit": "TFLOP/s", "n_gpus": 1, "steps": K, "warmup": args.warmup,
        "ms_per_step": ms_per_step, "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic (seeded N(0,1) inputs and output gradient, jagged lengths and mappings drawn per config)",
        "config": {"workload": f"{args.config}: {WORKLOAD_TEXT[args.config]}", "n_cand": w.n_cand,
                   "n_users": w.n_users, "n_q": w.n_q, "H": w.H, "d": w.d, "total_len": w.total_len, "seed": w.seed},
        "roofline": roof, "cpu_baseline": None, "extra": extra,
    }
    if not args.no_cpu_baseline:
        result["cpu_baseline"] = cpu_baseline_bwd(w, 24 if w.n_cand > 2000 else 128, 3)
    print(json.dumps(result), flush=True)


def mx_counts(w):
    """FLOPs of the two products and the MXFP8 kernel's algorithmic bytes: K/V
    codes and scales once per (user, head), Q codes and scales, bf16 output."""
    f = 4.0 * w.n_q * w.d * w.H * float(np.dot(w.counts, w.lengths))
    nvb = int(w.v_block_offsets[-1])
    b = (2.0 * w.total_len * w.H * w.d + w.total_len * w.H * (w.d // 32) + nvb * w.H * w.d
         + w.n_cand * w.n_q * w.H * (w.d + w.d // 32) + 2.0 * w.n_cand * w.n_q * w.H * w.d)
    return f, b


def cpu_baseline_mx(w, n_sample, reps):
    """The fp64 MXFP8 oracle on the first n_sample candidates, scaled to the batch."""
    from oracle import mxfp8_oracle as M
    try:
        from threadpoolctl import threadpool_info
        threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:
        threads = 1
    sl = slice(0, n_sample)
    times = []
    for _ in range(reps):
        t0 = time.perf_counter()
        M.target_attention_mxfp8(w.q_codes[sl], w.q_scales[sl], w.k_codes, w.k_scales, w.v_codes, w.v_scales,
                                 w.user_offsets, w.cand_to_user[sl], w.scale)
        times.append(time.perf_counter() - t0)
    t = float(np.median(times))
    f_sample = 4.0 * w.n_q * w.d * w.H * float(w.lengths[w.cand_to_user[sl]].sum())
    return {"value": f_sample / t / 1e12, "unit": "TFLOP/s", "cores": int(threads), "kind": "oracle",
            "sample": f"first {n_sample} of {w.n_cand} candidates of {w.name}, fp64 numpy with an explicit K/V copy "
                      f"per candidate and P quantized per 32-key block, median of {reps} runs of {t:.2f} s",
            "seconds_whole_batch": t * w.n_cand / n_sample}


def main_mx(args):
    """One step = one ikbo_attn_fwd_mxfp8 call: host grouping and work lists from
    the host mapping, the MXFP8 kernel and (for split key ranges) the merge."""
    import torch
    import broadcast_free_target_amd as ikbo
    from workloads import make_mxfp8

    w = make_mxfp8(args.config)
    dev = [torch.from_numpy(np.ascontiguousarray(a)).cuda() for a in w.arrays()]
    out = torch.empty((w.n_cand, w.n_q, w.H, w.d), dtype=torch.bfloat16, device="cuda")
    offs_h = np.ascontiguousarray(w.user_offsets, dtype=np.int32)
    c2u_h = np.ascontiguousarray(w.cand_to_user, dtype=np.int32)
    stream = torch.cuda.current_stream()
    h = ikbo.ikbo_mx_create()

    def step():
        ikbo.ikbo_attn_fwd_mxfp8(h, offs_h, c2u_h, w.n_users, w.n_cand, w.n_q, w.H, w.d, w.scale, *dev, out, stream)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    K = args.steps
    t0 = time.perf_counter()
    for _ in range(K):
        step()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ikbo.ikbo_mx_timing(h, True)
    for _ in range(K):
        step()
    torch.cuda.synchronize()
    attn_ms, merge_ms = ikbo.ikbo_mx_timing_read(h, K)
    ikbo.ikbo_mx_timing(h, False)
    info = ikbo.ikbo_mx_info(h)
    ikbo.ikbo_mx_destroy(h)
    a_ms, m_ms = float(np.mean(attn_ms)), float(np.mean(merge_ms))
    f, b = mx_counts(w)
    ms_per_step = wall * 1e3 / K
    if f / b < PEAK_FP8_TFLOPS * 1e12 / (PEAK_HBM_GBS * 1e9):
        achieved = b / (a_ms * 1e-3) / 1e9
        roof = {"bound": "hbm", "achieved": achieved, "peak": PEAK_HBM_GBS, "unit": "GB/s", "frac": achieved / PEAK_HBM_GBS}
    else:
        achieved = f / (a_ms * 1e-3) / 1e12
        roof = {"bound": "mfma", "achieved": achieved, "peak": PEAK_FP8_TFLOPS, "unit": "TFLOP/s",
                "frac": achieved / PEAK_FP8_TFLOPS}
    roof["traffic"] = traffic_from_profiles(args.config)
    roof["kernel"] = MX_KERNEL
    roof["kernel_avg_us"] = a_ms * 1e3
    roof["merge_kernel_avg_us"] = m_ms * 1e3
    roof["algorithmic_bytes_per_launch"] = b
    roof["algorithmic_flops_per_launch"] = f
    extra = {"kernel_tflops": f / (a_ms * 1e-3) / 1e12, "kernel_frac_fp8_mfma_peak": f / (a_ms * 1e-3) / 1e12 / PEAK_FP8_TFLOPS,
             "kernel_hbm_gbs": b / (a_ms * 1e-3) / 1e9, "candidates_per_s": w.n_cand / (ms_per_step * 1e-3),
             "work_items": info}
    result = {
        "metric": MX_METRIC, "value": f / (ms_per_step * 1e-3) / 1e12, "unit": "TFLOP/s", "n_gpus": 1, "steps": K,
        "warmup": args.warmup, "ms_per_step": ms_per_step, "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "fp8 (E4M3 data, E8M0 block scales, fp32 accumulation)",
        "data": "synthetic (seeded MX codes with per-block scales, dequantized values ~N(0,1); jagged lengths and "
                "mappings of the bf16 configuration of the same name)",
        "config": {"workload": f"{args.config}: {WORKLOAD_TEXT[args.config]}", "n_cand": w.n_cand,
                   "n_users": w.n_users, "n_q": w.n_q, "H": w.H, "d": w.d, "total_len": w.total_len, "seed": w.seed},
        "roofline": roof, "cpu_baseline": None, "extra": extra,
    }
    if not args.no_cpu_baseline:
        result["cpu_baseline"] = cpu_baseline_mx(w, 8 if w.n_cand > 2000 else 256, 3)
    print(json.dumps(result), flush=True)


def lce3_counts(w):
    """Executed and baseline FLOPs of a three-level call, and the item GEMM's
    algorithmic FLOPs and bytes (W_c, x_cand, out, vendor results once per vendor)."""
    U, V, B, M, N = w.n_users, w.n_vendors, w.n_cand, w.M, w.N
    f_exec = 2.0 * M * N * (U * w.K_u + V * w.K_v + B * w.K_c)
    f_base = 2.0 * M * N * B * w.K
    f_item = 2.0 * M * N * B * w.K_c
    b_item = 2.0 * (M * w.K_c + B * w.K_c * N + B * M * N) + 4.0 * V * M * N
    return f_exec, f_base, f_item, b_item


def cpu_baseline_lce3(w, n_sample, reps):
    """The fp64 nested oracle (both broadcast copies explicit) on the first
    n_sample items, its time scaled to the whole batch, counted in executed FLOPs."""
    from oracle import lce_oracle as O
    try:
        from threadpoolctl import threadpool_info
        threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:
        threads = 1
    args = (w.values("w"), w.values("x_user"), w.values("x_vendor"), w.values("x_cand")[:n_sample],
            w.vendor_to_user, w.cand_to_vendor[:n_sample])
    times = []
    for _ in range(reps):
        t0 = time.perf_counter()
        O.lce_baseline_nested(*args)
        times.append(time.perf_counter() - t0)
    t = float(np.median(times))
    t_whole = t * w.n_cand / n_sample
    return {"value": lce3_counts(w)[0] / t_whole / 1e12, "unit": "TFLOP/s", "cores": int(threads), "kind": "oracle",
            "sample": f"first {n_sample} of {w.n_cand} items of {w.name}, fp64 numpy with both broadcast copies "
                      f"explicit, median of {reps} runs of {t:.2f} s, scaled to the whole batch and counted in "
                      f"the same executed FLOPs as the GPU value",
            "seconds_whole_batch": t_whole}


def main_lce3(args):
    """One step = one ikbo_lce3_fwd: item ordering, user, vendor and item GEMMs."""
    import torch
    import broadcast_free_target_amd as ikbo
    from workloads import make_lce_nested

    w = make_lce_nested(args.config)

    def dev(a):
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).cuda().view(torch.bfloat16)

    W, xu, xv, xc = dev(w.raw("w")), dev(w.raw("x_user")), dev(w.raw("x_vendor")), dev(w.raw("x_cand"))
    v2u = torch.from_numpy(w.vendor_to_user.copy()).cuda()
    c2v = torch.from_numpy(w.cand_to_vendor.copy()).cuda()
    out = torch.empty((w.n_cand, w.M, w.N), dtype=torch.bfloat16, device="cuda")
    stream = torch.cuda.current_stream()
    h = ikbo.ikbo_lce3_create(W, w.M, w.K_u, w.K_v, w.K_c, stream=stream)

    def step():
        ikbo.ikbo_lce3_fwd(h, xu, xv, xc, v2u, c2v, w.n_users, w.n_vendors, w.n_cand, w.N, out, stream)

    def materialized():
        hb = ikbo.ikbo_lce_create(W, w.M, 0, w.K, stream=stream)
        xfull = torch.empty((w.n_cand, w.K, w.N), dtype=torch.bfloat16, device="cuda")
        vi = c2v.long()
        ui = v2u.long()[vi]

        def copy():
            xfull[:, :w.K_u].copy_(xu.index_select(0, ui))
            xfull[:, w.K_u:w.K_u + w.K_v].copy_(xv.index_select(0, vi))
            xfull[:, w.K_u + w.K_v:].copy_(xc)

        def gemm():
            ikbo.ikbo_lce_fwd(hb, None, xfull, c2v, w.n_vendors, w.n_cand, w.N, out, stream)

        return hb, copy, gemm

    if args.materialized_only:
        hb, copy, gemm = materialized()
        for _ in range(args.steps):
            copy()
            gemm()
        torch.cuda.synchronize()
        ikbo.ikbo_lce_destroy(hb)
        ikbo.ikbo_lce_destroy(h)
        print(json.dumps({"materialized_launches": args.steps, "config": args.config}), flush=True)
        return
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    K = args.steps
    t0 = time.perf_counter()
    for _ in range(K):
        step()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ikbo.ikbo_lce_timing(h, True)
    for _ in range(K):
        step()
    torch.cuda.synchronize()
    upper_ms, item_ms = ikbo.ikbo_lce_timing_read(h, K)
    ikbo.ikbo_lce_timing(h, False)
    if ikbo.ikbo_lce_errors(h) != 0:
        raise RuntimeError("three-level linear compression reported out-of-range mappings")
    u_avg, c_avg = float(np.mean(upper_ms)), float(np.mean(item_ms))
    f_exec, f_base, f_item, b_item = lce3_counts(w)
    ms_per_step = wall * 1e3 / K
    ai = f_item / b_item
    if ai < PEAK_BF16_TFLOPS * 1e12 / (PEAK_HBM_GBS * 1e9):
        achieved = b_item / (c_avg * 1e-3) / 1e9
        roof = {"bound": "hbm", "achieved": achieved, "peak": PEAK_HBM_GBS, "unit": "GB/s", "frac": achieved / PEAK_HBM_GBS}
    else:
        achieved = f_item / (c_avg * 1e-3) / 1e12
        roof = {"bound": "mfma", "achieved": achieved, "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                "frac": achieved / PEAK_BF16_TFLOPS}
    roof["traffic"] = traffic_from_profiles(args.config)
    roof["kernel"] = LCE_KERNEL
    roof["kernel_avg_us"] = c_avg * 1e3
    roof["user_and_vendor_kernels_us"] = u_avg * 1e3
    roof["algorithmic_bytes_per_launch"] = b_item
    roof["algorithmic_flops_per_launch"] = f_item
    extra = {"executed_flops": f_exec, "baseline_flops": f_base, "flops_saved_frac": 1.0 - f_exec / f_base,
             "baseline_equivalent_tflops": f_base / (ms_per_step * 1e-3) / 1e12,
             "item_gemm_tflops": f_item / (c_avg * 1e-3) / 1e12, "items_per_s": w.n_cand / (ms_per_step * 1e-3)}
    if args.report:
        hb, copy, gemm = materialized()
        for _ in range(3):
            copy()
            gemm()
        torch.cuda.synchronize()
        t1 = time.perf_counter()
        for _ in range(20):
            copy()
            gemm()
        torch.cuda.synchronize()
        extra["materialized_step_us"] = (time.perf_counter() - t1) / 20 * 1e6
        extra["speedup_vs_materialized_step"] = extra["materialized_step_us"] / (ms_per_step * 1e3)
        ikbo.ikbo_lce_destroy(hb)
    ikbo.ikbo_lce_destroy(h)
    result = {
        "metric": LCE_METRIC, "value": f_exec / (ms_per_step * 1e-3) / 1e12, "unit": "TFLOP/s", "n_gpus": 1,
        "steps": K, "warmup": args.warmup, "ms_per_step": ms_per_step, "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic (seeded N(0,1) inputs, W scaled by 1/sqrt(K), multinomial user->vendor->item mappings)",
        "config": {"workload": f"{args.config}: {WORKLOAD_TEXT[args.config]}", "n_cand": w.n_cand,
                   "n_vendors": w.n_vendors, "n_users": w.n_users, "M": w.M, "K_u": w.K_u, "K_v": w.K_v,
                   "K_c": w.K_c, "N": w.N, "seed": w.seed},
        "roofline": roof, "cpu_baseline": None, "extra": extra,
    }
    if not args.no_cpu_baseline:
        result["cpu_baseline"] = cpu_baseline_lce3(w, 256, max(3, args.cpu_reps // 3))
    print(json.dumps(result), flush=True)


def main_lce(args):
    """One step = one ikbo_lce_fwd: user GEMM, then the candidate GEMM whose
    epilogue adds each candidate's user result."""
    import torch
    import broadcast_free_target_amd as ikbo
    from workloads import make_lce

    w = make_lce(args.config)

    def dev(a):
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).cuda().view(torch.bfloat16)

    W, xu, xc = dev(w.raw("w")), dev(w.raw("x_user")), dev(w.raw("x_cand"))
    c2u = torch.from_numpy(w.cand_to_user.copy()).cuda()
    out = torch.empty((w.n_cand, w.M, w.N), dtype=torch.bfloat16, device="cuda")
    stream = torch.cuda.current_stream()
    h = ikbo.ikbo_lce_create(W, w.M, w.K_u, w.K_c, stream=stream)

    def step():
        ikbo.ikbo_lce_fwd(h, xu, xc, c2u, w.n_users, w.n_cand, w.N, out, stream)

    def materialized():
        """The comparator: the broadcast copy (x_user[u(b)] next to x_cand[b]
        along K) and the same GEMM kernel on the full K, with no user block."""
        hb = ikbo.ikbo_lce_create(W, w.M, 0, w.K, stream=stream)
        xfull = torch.empty((w.n_cand, w.K, w.N), dtype=torch.bfloat16, device="cuda")
        idx = c2u.long()

        def copy():
            xfull[:, :w.K_u].copy_(xu.index_select(0, idx))
            xfull[:, w.K_u:].copy_(xc)

        def gemm():
            ikbo.ikbo_lce_fwd(hb, None, xfull, c2u, w.n_users, w.n_cand, w.N, out, stream)

        return hb, xfull, copy, gemm

    if args.materialized_only:
        hb, xfull, copy, gemm = materialized()
        for _ in range(args.steps):
            copy()
            gemm()
        torch.cuda.synchronize()
        ikbo.ikbo_lce_destroy(hb)
        ikbo.ikbo_lce_destroy(h)
        print(json.dumps({"materialized_launches": args.steps, "config": args.config}), flush=True)
        return

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    K = args.steps
    t0 = time.perf_counter()
    for _ in range(K):
        step()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ikbo.ikbo_lce_timing(h, True)
    for _ in range(K):
        step()
    torch.cuda.synchronize()
    user_ms, cand_ms = ikbo.ikbo_lce_timing_read(h, K)
    ikbo.ikbo_lce_timing(h, False)
    if ikbo.ikbo_lce_errors(h) != 0:
        raise RuntimeError("linear compression reported out-of-range candidate mappings")
    u_avg, c_avg = float(np.mean(user_ms)), float(np.mean(cand_ms))

    f_user, f_cand, b_user, b_cand, f_base, b_base = lce_counts(w)
    ms_per_step = wall * 1e3 / K
    value = (f_user + f_cand) / (ms_per_step * 1e-3) / 1e12
    ai = f_cand / b_cand
    if ai < PEAK_BF16_TFLOPS * 1e12 / (PEAK_HBM_GBS * 1e9):
        achieved = b_cand / (c_avg * 1e-3) / 1e9
        roof = {"bound": "hbm", "achieved": achieved, "peak": PEAK_HBM_GBS, "unit": "GB/s",
                "frac": achieved / PEAK_HBM_GBS}
    else:
        achieved = f_cand / (c_avg * 1e-3) / 1e12
        roof = {"bound": "mfma", "achieved": achieved, "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                "frac": achieved / PEAK_BF16_TFLOPS}
    roof["traffic"] = traffic_from_profiles(args.config)
    roof["kernel"] = LCE_KERNEL
    roof["kernel_avg_us"] = c_avg * 1e3
    roof["user_kernel_avg_us"] = u_avg * 1e3
    roof["algorithmic_bytes_per_launch"] = b_cand
    roof["algorithmic_flops_per_launch"] = f_cand
    extra = {
        "candidate_gemm_tflops": f_cand / (c_avg * 1e-3) / 1e12,
        "candidate_gemm_hbm_gbs": b_cand / (c_avg * 1e-3) / 1e9,
        "user_gemm_tflops": f_user / (u_avg * 1e-3) / 1e12 if u_avg > 0 else None,
        "arith_intensity_candidate_gemm": ai,
        "executed_flops": f_user + f_cand,
        "baseline_flops": f_base,
        "flops_saved_frac": 1.0 - (f_user + f_cand) / f_base,
        "baseline_equivalent_tflops": f_base / (ms_per_step * 1e-3) / 1e12,
        "algorithmic_bytes_ikbo": b_user + b_cand,
        "algorithmic_bytes_baseline": b_base,
        "cands_per_s": w.n_cand / (ms_per_step * 1e-3),
    }
    if args.report:
        hb, xfull, copy, gemm = materialized()
        for _ in range(3):
            copy()
            gemm()
        torch.cuda.synchronize()
        n_mat = 20
        t1 = time.perf_counter()
        for _ in range(n_mat):
            copy()
            gemm()
        torch.cuda.synchronize()
        extra["materialized_step_us"] = (time.perf_counter() - t1) / n_mat * 1e6
        ikbo.ikbo_lce_timing(hb, True)
        for _ in range(n_mat):
            gemm()
        torch.cuda.synchronize()
        _, mat_ms = ikbo.ikbo_lce_timing_read(hb, n_mat)
        ikbo.ikbo_lce_destroy(hb)
        extra["materialized_gemm_us"] = float(np.mean(mat_ms)) * 1e3
        extra["materialized_gemm_tflops"] = f_base / (float(np.mean(mat_ms)) * 1e-3) / 1e12
        extra["speedup_vs_materialized_step"] = extra["materialized_step_us"] / (ms_per_step * 1e3)
        del xfull
    ikbo.ikbo_lce_destroy(h)
    result = {
        "metric": LCE_METRIC,
        "value": value,
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": args.warmup,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded N(0,1) inputs, W scaled by 1/sqrt(K), multinomial candidate-to-user mapping)",
        "config": {"workload": f"{args.config}: {WORKLOAD_TEXT[args.config]}", "n_cand": w.n_cand,
                   "n_users": w.n_users, "M": w.M, "K_u": w.K_u, "K_c": w.K_c, "N": w.N, "seed": w.seed},
        "roofline": roof,
        "cpu_baseline": None,
        "extra": extra,
    }
    if not args.no_cpu_baseline:
        result["cpu_baseline"] = cpu_baseline_lce(w, 256, max(3, args.cpu_reps // 3))
    print(json.dumps(result), flush=True)


def _pmc_rows(path):
    """Per-dispatch counter values from a rocprofv3 --pmc run: {(dispatch, kernel): {counter: value}}.
    `path` is the output directory (searched for *counter_collection.csv) or the file."""
    import csv
    import glob
    files = [path] if os.path.isfile(path) else sorted(glob.glob(os.path.join(path, "**", "*counter_collection.csv"),
                                                                 recursive=True))
    if not files:
        raise FileNotFoundError(f"no counter_collection.csv under {path}")
    rows = {}
    for f in files:
        with open(f, newline="") as fh:
            for r in csv.DictReader(fh):
                key = (f, r.get("Dispatch_Id") or r.get("Correlation_Id"), r["Kernel_Name"])
                d = rows.setdefault(key, {})
                d[r["Counter_Name"]] = d.get(r["Counter_Name"], 0.0) + float(r["Counter_Value"])
    return rows


def _pmc_mean(rows, counter, match):
    """Mean of a counter (KiB) over the dispatches whose kernel name contains `match`."""
    vals = [d[counter] for (_, _, name), d in rows.items() if match in name and counter in d]
    return (float(np.mean(vals)), len(vals)) if vals else (0.0, 0)


def summarize_pmc(args):
    """HBM bytes per launch from two rocprofv3 --pmc runs (FETCH_SIZE, then
    WRITE_SIZE, KiB per dispatch) of the benchmark command, scaled by the same
    counters taken on a plain 1 GiB device-to-device copy (--copy-calibration),
    written as the JSON summary that the roofline's `traffic` field reads."""
    n = 1 << 30
    cf = _pmc_rows(args.copy_fetch)
    cw = _pmc_rows(args.copy_write)
    copy_f = max((d.get("FETCH_SIZE", 0.0) for d in cf.values()), default=0.0)
    copy_w = max((d.get("WRITE_SIZE", 0.0) for d in cw.values()), default=0.0)
    if copy_f <= 0 or copy_w <= 0:
        raise RuntimeError("copy calibration runs hold no FETCH_SIZE / WRITE_SIZE")
    f_scale, w_scale = n / (copy_f * 1024.0), n / (copy_w * 1024.0)
    fr, wr = _pmc_rows(args.fetch), _pmc_rows(args.write)
    kernels = [k.strip() for k in args.kernels.split(";") if k.strip()]
    out = {"workload": args.config, "kernel_source_hash": None, "commands": {
               "fetch": args.fetch_cmd, "write": "the same with --pmc WRITE_SIZE",
               "copy_calibration": "rocprofv3 --pmc FETCH_SIZE (then WRITE_SIZE) --output-format csv -d <dir> -o run "
                                   "-- python3 bench.py --copy-calibration --steps 5"},
           "copy_calibration": {"bytes": n, "fetch_kib_per_dispatch": copy_f, "fetch_scale": f_scale,
                                "write_kib_per_dispatch": copy_w, "write_scale": w_scale},
           "kernels": {}}
    total = 0.0
    for k in kernels:
        f, nf = _pmc_mean(fr, "FETCH_SIZE", k)
        w_, nw = _pmc_mean(wr, "WRITE_SIZE", k)
        rb, wb = f * 1024.0 * f_scale, w_ * 1024.0 * w_scale
        out["kernels"][k] = {"read_bytes": rb, "write_bytes": wb, "dispatches": [nf, nw]}
        total += rb + wb
    first = out["kernels"][kernels[0]]
    out["hbm_bytes_per_launch"] = first["read_bytes"] + first["write_bytes"]
    out["hbm_bytes_per_step_with_merge"] = total
    lce, bwd, mx = args.config.startswith("lce"), args.config.startswith("bwd_"), args.config.startswith("mx_")
    out["kernel_source_hash"] = (kernel_source_hash(LCE_SOURCES) if lce else kernel_source_hash(BWD_SOURCES) if bwd
                                 else kernel_source_hash(MX_SOURCES) if mx else kernel_source_hash())
    with open(args.out, "w") as fh:
        json.dump(out, fh, indent=1)
    print(json.dumps(out), flush=True)


def summarize_sq(args):
    """Per-kernel SQ ratios from one rocprofv3 --pmc run holding SQ_INSTS_MFMA,
    SQ_INSTS_VALU, SQ_INSTS_LDS, SQ_VALU_MFMA_BUSY_CYCLES, SQ_LDS_IDX_ACTIVE,
    SQ_LDS_BANK_CONFLICT, SQ_WAIT_ANY, SQ_ACTIVE_INST_ANY and GRBM_GUI_ACTIVE.
    GRBM_GUI_ACTIVE is counted per XCC (8 of them), so one XCC's active cycles
    are the sum over 8; the MFMA and LDS busy fractions divide by those cycles
    times the SIMD (1024) or CU (256) count, as the MfmaUtil and LdsUtil
    metrics rocprofv3 lists do."""
    rows = _pmc_rows(args.sq)
    per = {}
    for (_, _, name), d in rows.items():
        if "ikbo" not in name:
            continue
        per.setdefault(name.replace("(anonymous namespace)::", "").split("(")[0].replace("void ", ""), []).append(d)
    out = {}
    for name, ds in per.items():
        keys = set().union(*ds)
        m = {k: float(np.mean([d.get(k, 0.0) for d in ds])) for k in keys}
        g = lambda k: m.get(k, float("nan"))  # noqa: E731
        cyc = g("GRBM_GUI_ACTIVE") / 8.0
        mfma = max(g("SQ_INSTS_MFMA"), 1.0)
        out[name] = {"dispatches": len(ds), "mfma_busy": g("SQ_VALU_MFMA_BUSY_CYCLES") / (cyc * 1024),
                     "valu_per_mfma": (g("SQ_INSTS_VALU") - g("SQ_INSTS_MFMA")) / mfma,
                     "lds_per_mfma": g("SQ_INSTS_LDS") / mfma, "lds_busy": g("SQ_LDS_IDX_ACTIVE") / (cyc * 256),
                     "lds_bank_conflicts": g("SQ_LDS_BANK_CONFLICT"),
                     "wait_share": g("SQ_WAIT_ANY") / max(g("SQ_WAIT_ANY") + g("SQ_ACTIVE_INST_ANY"), 1.0)}
    print(json.dumps(out, indent=1), flush=True)


def summarize_trace(args):
    """Per-kernel durations from a rocprofv3 --kernel-trace run of the
    benchmark: over all dispatches, and over the dispatches of timed region 2
    (the ones bench.py's roofline durations come from: each kernel's dispatches
    number warmup + steps .. warmup + 2 * steps - 1, in launch order)."""
    import csv
    import glob
    path = args.trace
    files = [path] if os.path.isfile(path) else sorted(glob.glob(os.path.join(path, "**", "*kernel_trace.csv"),
                                                                 recursive=True))
    if not files:
        raise FileNotFoundError(f"no kernel_trace.csv under {path}")
    per = {}
    for f in files:
        with open(f, newline="") as fh:
            for r in csv.DictReader(fh):
                per.setdefault(r["Kernel_Name"], []).append(
                    (int(r["Start_Timestamp"]), int(r["End_Timestamp"]) - int(r["Start_Timestamp"])))
    out = {}
    for name, v in per.items():
        v.sort()
        d = np.array([x[1] for x in v], dtype=np.float64) / 1e3  # ns -> us
        rec = {"dispatches": int(d.size), "avg_us_all": float(d.mean())}
        lo, hi = args.warmup + args.steps, args.warmup + 2 * args.steps
        if d.size >= hi:
            rec["avg_us_timed_region_2"] = float(d[lo:hi].mean())
        out[name] = rec
    print(json.dumps(out, indent=1), flush=True)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--config", default="c2_typical")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-reps", type=int, default=15)
    ap.add_argument("--report", action="store_true",
                    help="linear compression: also time the materialised-broadcast comparator")
    ap.add_argument("--kernel-only", action="store_true", help="loop only the planned launch (for profiling)")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="run only a plain 1 GiB device-to-device copy (to scale memory counters)")
    ap.add_argument("--materialized-only", action="store_true",
                    help="loop only the materialised-broadcast comparator (for profiling)")
    ap.add_argument("--summarize-pmc", action="store_true",
                    help="CPU only: turn rocprofv3 FETCH_SIZE/WRITE_SIZE runs into the traffic summary JSON")
    ap.add_argument("--fetch", help="--summarize-pmc: output directory of the FETCH_SIZE run")
    ap.add_argument("--write", help="--summarize-pmc: output directory of the WRITE_SIZE run")
    ap.add_argument("--copy-fetch", help="--summarize-pmc: FETCH_SIZE run of --copy-calibration")
    ap.add_argument("--copy-write", help="--summarize-pmc: WRITE_SIZE run of --copy-calibration")
    ap.add_argument("--kernels", default="ikbo_attn_bf16;ikbo_merge_kernel",
                    help="--summarize-pmc: ';'-separated kernel-name substrings, the roofline's kernel first")
    ap.add_argument("--fetch-cmd", default="", help="--summarize-pmc: the profiled command, recorded in the summary")
    ap.add_argument("--out", help="--summarize-pmc: path of the JSON summary")
    ap.add_argument("--summarize-trace", dest="trace",
                    help="CPU only: per-kernel durations from a rocprofv3 --kernel-trace output directory")
    ap.add_argument("--summarize-sq", dest="sq",
                    help="CPU only: per-kernel SQ ratios from a rocprofv3 --pmc output directory")
    args = ap.parse_args()
    if args.sq:
        summarize_sq(args)
        return
    if args.trace:
        summarize_trace(args)
        return
    if args.summarize_pmc:
        summarize_pmc(args)
        return
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: this benchmark has no multi-GPU path (run with --gpus 1)",
              file=sys.stderr)
        sys.exit(2)

    import torch
    import broadcast_free_target_amd as ikbo
    from workloads import make_workload

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    torch.cuda.set_device(0)
    if args.copy_calibration:
        n = 1 << 30
        src = torch.ones(n, dtype=torch.uint8, device="cuda")
        dst = torch.empty(n, dtype=torch.uint8, device="cuda")
        for _ in range(args.steps):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_calibration_bytes_read": n, "copy_calibration_bytes_written": n,
                          "launches": args.steps}), flush=True)
        return
    if args.config.startswith("mx_"):
        main_mx(args)
        return
    if args.config.startswith("lce3_"):
        main_lce3(args)
        return
    if args.config.startswith("lce_"):
        main_lce(args)
        return
    if args.config.startswith("bwd_"):
        main_bwd(args)
        return
    w = make_workload(args.config)
    dev = upload(w)
    dt_code = ikbo.IKBO_DTYPE_BF16 if w.dtype == "bf16" else ikbo.IKBO_DTYPE_F32
    tdt = torch.bfloat16 if w.dtype == "bf16" else torch.float32
    out_c = torch.empty(w.raw("q_cand").shape, dtype=tdt, device="cuda")
    out_u = torch.empty(w.raw("q_user").shape, dtype=tdt, device="cuda") if w.with_self else None
    stream = torch.cuda.current_stream()
    offs_h = np.ascontiguousarray(w.user_offsets, dtype=np.int32)
    c2u_h = np.ascontiguousarray(w.cand_to_user, dtype=np.int32)
    ws = 1 if w.with_self else 0

    def materialized():
        ikbo.ikbo_attn_fwd_materialized(dev["q_cand"], dev["k_user"], dev["v_user"], dev["user_offsets"],
                                        dev["cand_to_user"], w.n_users, w.n_cand, w.H, w.d, w.scale, out_c, stream,
                                        n_q=w.n_q, dtype=dt_code)

    if args.materialized_only:
        for _ in range(args.steps):
            materialized()
        torch.cuda.synchronize()
        print(json.dumps({"materialized_launches": args.steps, "config": args.config}), flush=True)
        return
    plan = ikbo.ikbo_plan_create(offs_h, c2u_h, w.n_users, w.n_cand, w.n_q, w.H, w.d, dt_code, ws, stream)

    def build():
        ikbo.ikbo_plan_build(plan, offs_h, c2u_h, w.n_users, w.n_cand, w.n_q, w.H, w.d, dt_code, ws, stream)

    def launch():
        ikbo.ikbo_attn_fwd_planned(plan, dev["q_cand"], dev.get("q_user"), dev["k_user"], dev["v_user"], w.scale,
                                   out_c, out_u, stream)

    # One step is one ikbo_attn_fwd_hostmap call, made on the C ABI directly as
    # a runtime would; the binding checks the same arguments once, in the first
    # warm-up step.
    ikbo.ikbo_attn_fwd_hostmap(plan, offs_h, c2u_h, w.n_users, w.n_cand, w.n_q, w.H, w.d, dt_code, ws,
                               dev["q_cand"], dev.get("q_user"), dev["k_user"], dev["v_user"], w.scale, out_c,
                               out_u, stream)
    c_hostmap = ikbo.load_library().ikbo_attn_fwd_hostmap
    qu = dev.get("q_user")
    c_args = (plan, offs_h.ctypes.data, c2u_h.ctypes.data, w.n_users, w.n_cand, w.n_q, w.H, w.d, dt_code, ws,
              dev["q_cand"].data_ptr(), qu.data_ptr() if qu is not None else None, dev["k_user"].data_ptr(),
              dev["v_user"].data_ptr(), float(w.scale), out_c.data_ptr(),
              out_u.data_ptr() if out_u is not None else None, stream.cuda_stream)

    def step():  # plan build from the host mapping and launch, in one library call
        rc = c_hostmap(*c_args)
        if rc != 0:
            raise ikbo.IkboError(rc, ikbo.ikbo_last_error())

    info = ikbo.ikbo_plan_info(plan)
    for _ in range(args.warmup - 1):
        step()
    torch.cuda.synchronize()

    K = args.steps
    one = launch if args.kernel_only else step
    # Timed region 1: K whole steps, nothing else on the stream (the value).
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(K):
        one()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    # Timed region 2: the same K steps with the kernels' dispatches stamping HIP
    # events on this stream at their start and end (the roofline's durations).
    ikbo.ikbo_plan_timing(plan, True)
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    for i in range(K):
        one()
    torch.cuda.synchronize()
    wall_timed = time.perf_counter() - t1
    kern_ms, merge_ms = ikbo.ikbo_plan_timing_read(plan, K)
    ikbo.ikbo_plan_timing(plan, False)
    k_avg_ms = float(np.mean(kern_ms))
    merge_avg_ms = float(np.mean(merge_ms))
    path_ms = k_avg_ms + merge_avg_ms  # attention kernel + split-KV merge, per launch

    flops, byts, mat_bytes = algorithmic_counts(w)
    ms_per_step = wall * 1e3 / K
    value = flops / (ms_per_step * 1e-3) / 1e12
    ai = flops / byts
    peak_flops = (PEAK_BF16_TFLOPS if w.dtype == "bf16" else PEAK_F32_TFLOPS) * 1e12
    bound = "hbm" if ai < peak_flops / (PEAK_HBM_GBS * 1e9) else "mfma"
    # The roofline covers the launch's kernels together: the attention kernel
    # and, when key ranges were split, the merge of its partials.
    if bound == "hbm":
        achieved = byts / (path_ms * 1e-3) / 1e9
        roof = {"bound": "hbm", "achieved": achieved, "peak": PEAK_HBM_GBS, "unit": "GB/s",
                "frac": achieved / PEAK_HBM_GBS}
        attn_only = byts / (k_avg_ms * 1e-3) / 1e9 / PEAK_HBM_GBS
    else:
        achieved = flops / (path_ms * 1e-3) / 1e12
        pk = peak_flops / 1e12
        roof = {"bound": "mfma", "achieved": achieved, "peak": pk, "unit": "TFLOP/s", "frac": achieved / pk}
        attn_only = flops / (k_avg_ms * 1e-3) / peak_flops
    attn_name = KERNEL_NAMES[int(info["kernel"])].format(d=w.d)
    roof["traffic"] = traffic_from_profiles(args.config)
    roof["kernel"] = attn_name + (" + " + MERGE_KERNEL.format(d=w.d) if merge_avg_ms > 0 else "")
    roof["kernel_avg_us"] = path_ms * 1e3
    roof["attn_kernel_avg_us"] = k_avg_ms * 1e3
    roof["merge_kernel_avg_us"] = merge_avg_ms * 1e3
    roof["frac_attention_kernel_only"] = attn_only
    roof["algorithmic_bytes_per_launch"] = byts
    roof["algorithmic_flops_per_launch"] = flops

    extra = {
        "ms_per_step_with_kernel_timing": wall_timed * 1e3 / K,
        "attn_plus_merge_us": path_ms * 1e3,
        "kernel_tflops": flops / (path_ms * 1e-3) / 1e12,
        "kernel_frac_mfma_peak": flops / (path_ms * 1e-3) / peak_flops,
        "kernel_hbm_gbs": byts / (path_ms * 1e-3) / 1e9,
        "attn_kernel_us_median": float(np.median(kern_ms)) * 1e3,
        "arith_intensity": ai,
        "applicable_roof_tflops": min(peak_flops, ai * PEAK_HBM_GBS * 1e9) / 1e12,
        "cands_per_s": w.n_cand / (ms_per_step * 1e-3),
        "plan": info,
        "materialized_algorithmic_bytes": mat_bytes,
        "ikbo_vs_materialized_bytes_ratio": mat_bytes / byts,
    }
    mat_measured = materialized_traffic_from_profiles(args.config)
    if mat_measured is not None and roof.get("traffic"):
        # both sides' bytes as rocprofv3 counted them (FETCH_SIZE + WRITE_SIZE)
        extra["materialized_measured_bytes"] = mat_measured
        extra["ikbo_vs_materialized_bytes_ratio_measured"] = mat_measured / roof["traffic"]

    def extras():
        """Cold-cache kernel times, host times of the step's calls, the
        device-mapping entry point end to end and the materialised comparator
        (skipped with --kernel-only, which profiles the timed launches alone)."""
        # Cold cache: 2 GiB overwritten between launches so that neither L2 nor the
        # Infinity Cache holds K/V; the flush stays outside the kernels' events.
        flush = torch.empty(2 << 30, dtype=torch.uint8, device="cuda")
        n_cold = 20
        ikbo.ikbo_plan_timing(plan, True)
        for _ in range(n_cold):
            flush.fill_(1)
            launch()
            torch.cuda.synchronize()
        cold_a, cold_m = ikbo.ikbo_plan_timing_read(plan, n_cold)
        ikbo.ikbo_plan_timing(plan, False)
        del flush
        c_ms = float(np.median(np.asarray(cold_a) + np.asarray(cold_m)))
        extra["cold_attn_plus_merge_us_median"] = c_ms * 1e3
        extra["cold_kernel_tflops"] = flops / (c_ms * 1e-3) / 1e12
        extra["cold_kernel_hbm_gbs"] = byts / (c_ms * 1e-3) / 1e9
        extra["cold_frac_applicable_roof"] = (flops / (c_ms * 1e-3)) / min(peak_flops, ai * PEAK_HBM_GBS * 1e9)
        extra["warm_frac_applicable_roof"] = (flops / (path_ms * 1e-3)) / min(peak_flops, ai * PEAK_HBM_GBS * 1e9)
        # Host time of each call of a step (the GPU idle first, so nothing waits on it).
        torch.cuda.synchronize()
        t1 = time.perf_counter()
        for _ in range(100):
            build()
        extra["host_plan_build_us"] = (time.perf_counter() - t1) / 100 * 1e6
        torch.cuda.synchronize()
        t1 = time.perf_counter()
        for _ in range(20):
            launch()
        extra["host_launch_us"] = (time.perf_counter() - t1) / 20 * 1e6
        torch.cuda.synchronize()
        t1 = time.perf_counter()
        for _ in range(20):
            step()
        extra["host_step_us"] = (time.perf_counter() - t1) / 20 * 1e6  # one ikbo_attn_fwd_hostmap call
        torch.cuda.synchronize()
        if not w.with_self:
            # End to end through the device-mapping entry point: D2H copy of the
            # mapping, synchronisation, host plan and launch.
            def e2e():
                ikbo.ikbo_attn_fwd_mt(dev["q_cand"], dev["k_user"], dev["v_user"], dev["user_offsets"],
                                      dev["cand_to_user"], w.n_users, w.n_cand, w.H, w.d, w.scale, out_c, stream,
                                      n_q=w.n_q, dtype=dt_code)
            for _ in range(5):
                e2e()
            torch.cuda.synchronize()
            t1 = time.perf_counter()
            n_e2e = 50
            for _ in range(n_e2e):
                e2e()
            torch.cuda.synchronize()
            extra["e2e_device_mapping_us"] = (time.perf_counter() - t1) / n_e2e * 1e6
            # The materialised-broadcast comparator: copy kernel + the same attention kernel.
            if mat_bytes < 64e9:
                for _ in range(2):
                    materialized()
                torch.cuda.synchronize()
                t1 = time.perf_counter()
                n_mat = 5
                for _ in range(n_mat):
                    materialized()
                torch.cuda.synchronize()
                extra["materialized_us"] = (time.perf_counter() - t1) / n_mat * 1e6
                extra["materialized_vs_ikbo_step"] = extra["materialized_us"] / (ms_per_step * 1e3)

    if not args.kernel_only:
        extras()

    ikbo.ikbo_plan_destroy(plan)
    result = {
        "metric": METRIC,
        "value": value,
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": args.warmup,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": w.dtype,
        "data": "synthetic (seeded N(0,1) inputs, jagged lengths and mappings drawn per config)",
        "config": {"workload": f"{args.config}: {WORKLOAD_TEXT[args.config]}", "n_cand": w.n_cand,
                   "n_users": w.n_users, "n_q": w.n_q, "H": w.H, "d": w.d, "total_len": w.total_len,
                   "seed": w.seed},
        "roofline": roof,
        "cpu_baseline": None,
        "extra": extra,
    }
    if not args.no_cpu_baseline:
        result["cpu_baseline"] = cpu_baseline(w, args.cpu_reps)
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
