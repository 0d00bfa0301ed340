"""fp64 CPU oracle for IKBO linear compression -- TEST INFRASTRUCTURE ONLY.

Only the test suite, the package smoke check and the benchmark's CPU-baseline
leg may import or call this module; the product path never routes through it
and shares no code with it.

What it computes, and where the pages say so (IKBO blog, section 2.1, Fig. 2;
App. 2): the linear compression is the batched product ``(M, K) @ (B, K, N)``
of one learned matrix W with every candidate's K input embeddings of width N.
A candidate's K embeddings are the concatenation, along K, of its user's K_u
embeddings and its own K_c embeddings.  The oracle builds that concatenation
explicitly for every candidate (a real fp64 copy of the user block: the
broadcast the method avoids) and multiplies by W, so it is the plain
definition, not the decomposed method.

The method's equivalences are pinned by tests, not built in here: the split of
W along K into user and candidate columns (linearity, section 2.1), zero
padding of each decomposed K (section 2.2, Proof 1), brute-force scalar loops
on tiny inputs, and closed forms for an identity projection.

Three levels (user -> vendor -> item, the pages' conclusion): an item's K
embeddings are its user's, its vendor's and its own blocks; the oracle builds
both broadcast copies explicitly (``lce_baseline_nested``).

Readings where the pages are silent: W holds the user columns first (then,
with three levels, the vendor columns); the pages give K = 2044 without its
split, read here as K_u = K_c = 1022.
"""

from __future__ import annotations

import numpy as np

__all__ = ["lce_baseline", "lce_baseline_nested", "lce_flops_baseline", "lce_flops_ikbo", "lce_bytes_baseline"]


def _f64(x) -> np.ndarray:
    return np.asarray(x, dtype=np.float64)


def lce_baseline(w, x_user, x_cand, cand_to_user) -> np.ndarray:
    """out[b] = W @ concat_K(x_user[u(b)], x_cand[b]), fp64.

    w [M, K_u + K_c], x_user [U, K_u, N], x_cand [B, K_c, N] -> [B, M, N].
    """
    w = _f64(w)
    xu = _f64(x_user)
    xc = _f64(x_cand)
    c2u = np.asarray(cand_to_user, dtype=np.int64)
    B = xc.shape[0]
    M = w.shape[0]
    N = xc.shape[2]
    if w.shape[1] != xu.shape[1] + xc.shape[1]:
        raise ValueError("W columns must equal K_u + K_c")
    if np.any(c2u < 0) or np.any(c2u >= xu.shape[0]):
        raise ValueError("cand_to_user entry outside [0, n_users)")
    out = np.empty((B, M, N), dtype=np.float64)
    for b in range(B):
        xb = np.concatenate([xu[c2u[b]].copy(), xc[b]], axis=0)  # the broadcast copy, [K, N]
        out[b] = w @ xb
    return out


def lce_flops_baseline(B: int, M: int, K: int, N: int) -> float:
    """The batched product on every candidate (App. 2: 2 B M K N)."""
    return 2.0 * B * M * K * N


def lce_flops_ikbo(B: int, U: int, M: int, K_u: int, K_c: int, N: int) -> float:
    """User GEMM at the user batch plus candidate GEMM at the candidate batch (section 2.1)."""
    return 2.0 * M * N * (U * K_u + B * K_c)




def lce_bytes_baseline(B: int, M: int, K: int, N: int, elem: int = 2) -> float:
    """App. 2's byte count of the batched product: (M K + B K N + B M N) elements."""
    return float(elem * (M * K + B * K * N + B * M * N))


def lce_baseline_nested(w, x_user, x_vendor, x_cand, vendor_to_user, cand_to_vendor) -> np.ndarray:
    """Three levels, user -> vendor -> item (IKBO blog, conclusion: a user sees
    several vendors and each vendor offers several items, two nested broadcast
    relations).  An item's K embeddings are its user's K_u block, its vendor's
    K_v block and its own K_c block, concatenated along K in that order:

        out[b] = W @ concat_K(x_user[u], x_vendor[v], x_cand[b]),  v = cand_to_vendor[b],
                                                                    u = vendor_to_user[v]

    built explicitly per item (both broadcast copies are real), fp64.
    w [M, K_u + K_v + K_c]; x_user [U, K_u, N]; x_vendor [V, K_v, N]; x_cand [B, K_c, N].
    """
    w = _f64(w)
    xu = _f64(x_user)
    xv = _f64(x_vendor)
    xc = _f64(x_cand)
    v2u = np.asarray(vendor_to_user, dtype=np.int64)
    c2v = np.asarray(cand_to_vendor, dtype=np.int64)
    B, M, N = xc.shape[0], w.shape[0], xc.shape[2]
    if w.shape[1] != xu.shape[1] + xv.shape[1] + xc.shape[1]:
        raise ValueError("W columns must equal K_u + K_v + K_c")
    if np.any(c2v < 0) or np.any(c2v >= xv.shape[0]) or np.any(v2u < 0) or np.any(v2u >= xu.shape[0]):
        raise ValueError("mapping entry out of range")
    out = np.empty((B, M, N), dtype=np.float64)
    for b in range(B):
        v = c2v[b]
        u = v2u[v]
        xb = np.concatenate([xu[u].copy(), xv[v].copy(), xc[b]], axis=0)  # both broadcast copies, [K, N]
        out[b] = w @ xb
    return out

