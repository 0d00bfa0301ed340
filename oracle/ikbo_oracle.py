"""fp64 CPU oracle for IKBO target attention -- TEST INFRASTRUCTURE ONLY.

Only the test suite, the package smoke check and the benchmark's CPU-baseline
leg may import or call this module.  The product path never routes through
it: it shares no code with the HIP library, and nothing in the library
imports it.

What it computes, and where the pages say so:

* In-Kernel Broadcast Optimization blog, section 3.1 and Fig. 10: IKBO target
  attention is the same result as SDPA applied after the user's K/V has been
  broadcast (replicated) to every candidate of that user; the kernel only
  avoids materialising the copy.  The oracle therefore *does* materialise it:
  every candidate gets a real fp64 copy of its user's K and V
  (``_broadcast_user_kv``), and then runs plain softmax attention.
* Same blog, section 3 (opening): the model is encoder-driven, so target
  attention is full (non-causal) over the user's sequence.
* Same blog, section 3.3: self-attention over the user's own sequence shares
  the K/V source; only the queries differ.  The fused configuration asks for
  *causal* self-attention; key j is visible to query t iff j <= t.
* Softmax is the two-pass definition: subtract the row maximum, exponentiate,
  normalise.  (The GPU uses the online recurrence of the AI-infra guide,
  section 4.6.1, which equals this in exact arithmetic.)
* CSR grouping of candidates by user is this library's own contract (the pages
  hand the kernel a mapping tensor, section 1.3 and Alg. 1, and pair
  neighbouring candidates of one user): counts, exclusive prefix sum,
  a *stable* sort of candidate indices by user, and row tiles of at most
  ``bm`` rows.
* The split-KV merge is the log-sum-exp combination of the AI-infra guide,
  section 4.6.4 (Flash-Decoding).

Readings where the pages are silent (each also listed in the design notes):
a user with zero keys produces zero output rows; ``scale`` is the fp32 value
that crosses the C ABI, widened to fp64; n_q query tokens of one candidate
attend independently, each over the whole user sequence.

Parity pins: every function here is pinned by tests that do not re-type its
formula (brute-force loops, closed forms, invariances, torch SDPA as an
independent library implementation, and the pages' printed figures for the
measurement model).
"""

from __future__ import annotations

from typing import Iterable, Optional, Sequence

import numpy as np

__all__ = [
    "OracleInputError",
    "validate",
    "group_csr",
    "target_attention",
    "target_attention_rows",
    "target_attention_lse",
    "self_attention_causal",
    "self_attention_rows",
    "chunk_partial",
    "merge_partials",
    "flops_target",
    "bytes_ikbo",
    "ai_standard",
    "ai_ikbo",
    "ai_gemm",
    "machine_balance",
]


class OracleInputError(ValueError):
    """Invalid problem description.  ``code`` names the failed rule."""

    def __init__(self, code: str, msg: str):
        super().__init__(f"{code}: {msg}")
        self.code = code


# --------------------------------------------------------------------------
# validation (the problem statement: two batch sizes, offsets, mapping)
# --------------------------------------------------------------------------

def validate(user_offsets, cand_to_user, n_users: int, H: int, d: int) -> None:
    """Rules on the inputs of one call.

    * ``user_offsets`` has ``n_users + 1`` entries, starts at 0 and never decreases;
    * every ``cand_to_user[c]`` names a user in ``[0, n_users)``;
    * ``H >= 1`` and ``d`` is one of 32, 64, 128.
    """
    offs = np.asarray(user_offsets, dtype=np.int64)
    c2u = np.asarray(cand_to_user, dtype=np.int64)
    if H < 1:
        raise OracleInputError("invalid_arg", "H must be >= 1")
    if d not in (32, 64, 128):
        raise OracleInputError("unsupported", f"head dim {d}")
    if n_users < 0 or offs.shape != (n_users + 1,):
        raise OracleInputError("invalid_arg", "user_offsets must have n_users+1 entries")
    if offs[0] != 0 or np.any(np.diff(offs) < 0):
        raise OracleInputError("bad_offsets", "offsets must start at 0 and be non-decreasing")
    if c2u.size and (n_users == 0 or c2u.min() < 0 or c2u.max() >= n_users):
        raise OracleInputError("bad_mapping", "cand_to_user out of range")


# --------------------------------------------------------------------------
# CSR grouping of candidates by user
# --------------------------------------------------------------------------

def group_csr(cand_to_user, n_users: int, n_q: int, bm: int) -> dict:
    """Group candidates by user.

    Returns int32 arrays
      counts[u]        candidates of user u
      cand_offsets     exclusive prefix sum of counts, n_users + 1 entries
      cand_perm        candidate indices sorted by user, ascending original
                       index within a user (stable)
      tiles [T, 3]     (u, row_start, row_len) for users in ascending order,
                       tiles in ascending order; user u has c_u * n_q rows, row
                       r is (candidate cand_perm[cand_offsets[u] + r // n_q],
                       query r % n_q); every tile but a user's last has bm rows.
    """
    c2u = np.asarray(cand_to_user, dtype=np.int64)
    counts = np.bincount(c2u, minlength=n_users).astype(np.int64)
    cand_offsets = np.zeros(n_users + 1, dtype=np.int64)
    cand_offsets[1:] = np.cumsum(counts)
    cand_perm = np.argsort(c2u, kind="stable")
    tiles = []
    for u in range(n_users):
        rows = int(counts[u]) * n_q
        for t in range(-(-rows // bm)):
            start = t * bm
            tiles.append((u, start, min(bm, rows - start)))
    tiles_arr = np.asarray(tiles, dtype=np.int32).reshape(-1, 3)
    return {
        "counts": counts.astype(np.int32),
        "cand_offsets": cand_offsets.astype(np.int32),
        "cand_perm": cand_perm.astype(np.int32),
        "tiles": tiles_arr,
    }


# --------------------------------------------------------------------------
# attention
# --------------------------------------------------------------------------

def _as_f64(x) -> np.ndarray:
    return np.asarray(x, dtype=np.float64)


def _broadcast_user_kv(k_user, v_user, user_offsets, u: int):
    """Explicit broadcast: a fresh fp64 copy of user u's K and V for one candidate."""
    lo, hi = int(user_offsets[u]), int(user_offsets[u + 1])
    kc = np.array(k_user[lo:hi], dtype=np.float64, copy=True)
    vc = np.array(v_user[lo:hi], dtype=np.float64, copy=True)
    return kc, vc


def _scores(q, kc, scale: float):
    """s[h, i, j] = scale * sum_e q[i, h, e] * kc[j, h, e]; q [n_q, H, d], kc [L, H, d]."""
    return scale * np.matmul(np.transpose(q, (1, 0, 2)), np.transpose(kc, (1, 2, 0)))


def _softmax_rows(s):
    """Two-pass softmax over the last axis (row max subtracted first)."""
    m = np.max(s, axis=-1, keepdims=True)
    w = np.exp(s - m)
    return w / np.sum(w, axis=-1, keepdims=True)


def _attend(q, kc, vc, scale: float):
    """Softmax attention of q [n_q, H, d] over kc, vc [L, H, d] -> [n_q, H, d] (zeros if L = 0)."""
    n_q, H, d = q.shape
    if kc.shape[0] == 0:
        return np.zeros((n_q, H, d), dtype=np.float64)
    p = _softmax_rows(_scores(q, kc, scale))                 # [H, n_q, L]
    o = np.matmul(p, np.transpose(vc, (1, 0, 2)))            # [H, n_q, d]
    return np.transpose(o, (1, 0, 2))


def _fp32_scale(scale) -> float:
    return float(np.float64(np.float32(scale)))


def target_attention(q_cand, k_user, v_user, user_offsets, cand_to_user, scale,
                     cands: Optional[Iterable[int]] = None) -> np.ndarray:
    """IKBO target attention computed the slow way: broadcast, then attend.

    q_cand [C, n_q, H, d]; k_user, v_user [T, H, d]; returns fp64 [C, n_q, H, d]
    (or [len(cands), n_q, H, d] for a subset, in the given order).  Each
    candidate's user K/V is copied for that candidate before use.
    """
    q_cand = np.asarray(q_cand)
    offs = np.asarray(user_offsets, dtype=np.int64)
    c2u = np.asarray(cand_to_user, dtype=np.int64)
    sc = _fp32_scale(scale)
    idx = range(q_cand.shape[0]) if cands is None else list(cands)
    out = np.empty((len(idx),) + q_cand.shape[1:], dtype=np.float64)
    for n, c in enumerate(idx):
        kc, vc = _broadcast_user_kv(k_user, v_user, offs, int(c2u[c]))
        out[n] = _attend(_as_f64(q_cand[c]), kc, vc, sc)
    return out


def target_attention_rows(q_cand, k_user, v_user, user_offsets, cand_to_user, scale,
                          rows: Sequence[tuple]) -> np.ndarray:
    """Selected output rows (c, i, h) -> fp64 [len(rows), d]; for large sampled checks."""
    offs = np.asarray(user_offsets, dtype=np.int64)
    c2u = np.asarray(cand_to_user, dtype=np.int64)
    sc = _fp32_scale(scale)
    d = np.asarray(q_cand).shape[-1]
    out = np.empty((len(rows), d), dtype=np.float64)
    for n, (c, i, h) in enumerate(rows):
        kc, vc = _broadcast_user_kv(k_user, v_user, offs, int(c2u[c]))
        q = _as_f64(q_cand[c, i, h]).reshape(1, 1, d)
        out[n] = _attend(q, kc[:, h:h + 1, :], vc[:, h:h + 1, :], sc)[0, 0]
    return out


def target_attention_lse(q_cand, k_user, user_offsets, cand_to_user, scale,
                         cands: Optional[Iterable[int]] = None) -> np.ndarray:
    """The per-row statistic a training forward keeps for its backward: the
    natural-log log-sum-exp of each row's scaled scores over its user's keys,
    lse = log sum_j exp(s_j) = m + log sum_j exp(s_j - m) with m = max_j s_j
    (AI-infra guide, section 4.6.3).  Computed on each candidate's own copy of
    its user's keys, like ``target_attention``.  fp64 [C, n_q, H] (or the given
    candidates); -inf for users with no keys (the log of an empty sum).
    """
    q_cand = np.asarray(q_cand)
    offs = np.asarray(user_offsets, dtype=np.int64)
    c2u = np.asarray(cand_to_user, dtype=np.int64)
    sc = _fp32_scale(scale)
    idx = range(q_cand.shape[0]) if cands is None else list(cands)
    out = np.empty((len(idx),) + q_cand.shape[1:3], dtype=np.float64)
    for n, c in enumerate(idx):
        u = int(c2u[c])
        lo, hi = int(offs[u]), int(offs[u + 1])
        if hi == lo:
            out[n] = -np.inf
            continue
        kc = np.array(k_user[lo:hi], dtype=np.float64, copy=True)  # this candidate's copy
        s = _scores(_as_f64(q_cand[c]), kc, sc)                   # [H, n_q, L]
        m = np.max(s, axis=-1)
        out[n] = np.transpose(m + np.log(np.sum(np.exp(s - m[..., None]), axis=-1)), (1, 0))
    return out


def _causal_self_user(qu, ku, vu, scale: float):
    """Causal self-attention of one user: query t sees keys 0..t (diagonal included)."""
    L, H, d = qu.shape
    if L == 0:
        return np.zeros((0, H, d), dtype=np.float64)
    s = scale * np.matmul(np.transpose(qu, (1, 0, 2)), np.transpose(ku, (1, 2, 0)))  # [H, L, L]
    t = np.arange(L)[:, None]
    j = np.arange(L)[None, :]
    s = np.where(j <= t, s, -np.inf)
    p = _softmax_rows(s)
    o = np.matmul(p, np.transpose(vu, (1, 0, 2)))
    return np.transpose(o, (1, 0, 2))


def self_attention_causal(q_user, k_user, v_user, user_offsets, scale,
                          users: Optional[Iterable[int]] = None) -> np.ndarray:
    """Per-user causal self-attention over the packed sequence -> fp64 [T, H, d].

    Rows of users not in ``users`` (when given) are left as NaN.
    """
    offs = np.asarray(user_offsets, dtype=np.int64)
    sc = _fp32_scale(scale)
    q_user = np.asarray(q_user)
    out = np.full(q_user.shape, np.nan, dtype=np.float64)
    us = range(len(offs) - 1) if users is None else users
    for u in us:
        lo, hi = int(offs[u]), int(offs[u + 1])
        out[lo:hi] = _causal_self_user(_as_f64(q_user[lo:hi]), _as_f64(k_user[lo:hi]),
                                       _as_f64(v_user[lo:hi]), sc)
    return out


def self_attention_rows(q_user, k_user, v_user, user_offsets, scale, rows: Sequence[tuple]) -> np.ndarray:
    """Selected self-attention rows (u, t, h) -> fp64 [len(rows), d]."""
    offs = np.asarray(user_offsets, dtype=np.int64)
    sc = _fp32_scale(scale)
    d = np.asarray(q_user).shape[-1]
    out = np.empty((len(rows), d), dtype=np.float64)
    for n, (u, t, h) in enumerate(rows):
        lo = int(offs[u])
        q = _as_f64(q_user[lo + t, h]).reshape(1, 1, d)
        kc = _as_f64(k_user[lo:lo + t + 1, h:h + 1])
        vc = _as_f64(v_user[lo:lo + t + 1, h:h + 1])
        out[n] = _attend(q, kc, vc, sc)[0, 0]
    return out


# --------------------------------------------------------------------------
# split-KV partials and their log-sum-exp merge
# --------------------------------------------------------------------------

def chunk_partial(q, kc, vc, scale):
    """Attention of q [n_q, H, d] over one KV chunk: (normalised output, lse [H, n_q])."""
    sc = _fp32_scale(scale)
    s = _scores(_as_f64(q), _as_f64(kc), sc)                 # [H, n_q, Lc]
    m = np.max(s, axis=-1, keepdims=True)
    w = np.exp(s - m)
    lsum = np.sum(w, axis=-1, keepdims=True)
    o = np.matmul(w / lsum, np.transpose(_as_f64(vc), (1, 0, 2)))
    lse = (m + np.log(lsum))[..., 0]
    return np.transpose(o, (1, 0, 2)), lse


def merge_partials(parts):
    """Merge chunk partials: lse = log sum_c exp(lse_c); o = sum_c exp(lse_c - lse) o_c."""
    lses = np.stack([p[1] for p in parts])                   # [C, H, n_q]
    top = np.max(lses, axis=0)
    lse = top + np.log(np.sum(np.exp(lses - top), axis=0))
    o = np.zeros_like(parts[0][0])
    for oc, lc in parts:
        o = o + np.transpose(np.exp(lc - lse), (1, 0))[..., None] * oc
    return o, lse


# --------------------------------------------------------------------------
# measurement model (roofline bookkeeping)
# --------------------------------------------------------------------------

def flops_target(counts, lengths, n_q: int, H: int, d: int) -> float:
    """Algorithmic FLOPs of target attention: 4 * n_q * L_u * d per (candidate, head)."""
    return 4.0 * n_q * d * H * float(np.dot(np.asarray(counts, np.float64), np.asarray(lengths, np.float64)))




def bytes_ikbo(n_cand: int, n_q: int, total_len: int, H: int, d: int, elem: int,
               with_self: bool = False) -> float:
    """Algorithmic HBM bytes: Q read + O write per candidate row, K + V once per user row."""
    b = float(elem) * H * d * (2.0 * n_cand * n_q + 2.0 * total_len)
    if with_self:
        b += 2.0 * elem * H * d * total_len
    return b




def ai_standard(n_q: int, L: int) -> float:
    """Arithmetic intensity of attention with one query block of n rows against L keys
    (16-bit data; FLOPs 4 n L d over bytes 2 d (2n + 2L)): n L / (n + L)."""
    return n_q * L / float(n_q + L)


def ai_ikbo(n_q: int, L: int, ratio: float) -> float:
    """Same, with the user's K/V read once for ``ratio`` candidates: n L / (n + L / ratio)."""
    return n_q * L / float(n_q + L / float(ratio))


def ai_gemm(B: int, M: int, K: int, N: int, elem: int = 2) -> float:
    """Batched GEMM (M,K) @ (B,K,N): 2 B M K N / ((M K + B K N + B M N) * elem)."""
    return 2.0 * B * M * K * N / ((M * K + B * K * N + B * M * N) * float(elem))


def machine_balance(peak_flops: float, bandwidth: float) -> float:
    return peak_flops / bandwidth

