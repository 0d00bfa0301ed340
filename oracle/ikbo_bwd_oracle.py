"""fp64 CPU oracle for the backward of IKBO target attention -- TEST INFRASTRUCTURE ONLY.

Only the test suite, the package smoke check and the benchmark's CPU-baseline
leg may import or call this module; the product path never routes through it
and shares no code with it.

What it computes, and where the pages say so:

* The forward is the one of ``ikbo_oracle.target_attention``: IKBO target
  attention equals softmax attention applied after each user's K/V has been
  copied to every candidate of that user (IKBO blog, section 3.1, Fig. 10).
  The same blog notes (section 1.2) that the kernels also cut training cost
  when candidates outnumber users.
* The gradient is therefore the gradient of that explicit-copy computation.
  For one candidate c of user u and one head, with scores s = scale * q K^T,
  P = softmax(s), O = P V and the output gradient dO:
      dV_c = P^T dO,   dP = dO V^T,   D = rowsum(dO * O),
      dS = P * (dP - D),   dQ_c = scale * dS K,   dK_c = scale * dS^T q,
  the textbook softmax-attention backward that recomputes P from the scores
  (AI-infra guide, section 4.6.3).  The adjoint of copying the user's K/V to
  every candidate is a sum: dK_u and dV_u are the sums of the candidates'
  dK_c and dV_c.  The oracle builds every candidate's copy explicitly, takes
  each candidate's gradient and adds the copies' gradients into the user's
  rows, so the reduction over candidates is written out, not assumed.
* D uses the fp64 output the oracle recomputes (not a stored bf16 output).

Readings where the pages are silent (also listed in the design notes): a
user with zero keys gives zero query gradients; a user with zero candidates
gives zero key and value gradients; n_q query tokens of one candidate each
attend over the whole user sequence, so their gradients add into the same
user rows.

Parity pins (tests/test_bwd_oracle.py): central finite differences of the
forward oracle, torch autograd in fp64 on the explicit-copy forward, closed
forms (one key; the sum of a user's key gradients is zero; the sum of its
value gradients is the sum of its output gradients), linearity of the
reduction over candidates, and planted mistakes that those pins reject.
"""

from __future__ import annotations

import numpy as np

__all__ = ["target_attention_bwd", "flops_target_bwd"]


def _f64(x) -> np.ndarray:
    return np.asarray(x, dtype=np.float64)


def _fp32_scale(scale) -> float:
    return float(np.float32(scale))


def _candidate_bwd(q, kc, vc, do, scale: float):
    """One candidate, one head.  q, do: [n_q, d]; kc, vc: [L, d] (an explicit
    copy of the user's rows).  Returns dq [n_q, d], dkc [L, d], dvc [L, d]."""
    s = scale * (q @ kc.T)                       # [n_q, L]
    s = s - s.max(axis=1, keepdims=True)
    e = np.exp(s)
    p = e / e.sum(axis=1, keepdims=True)
    o = p @ vc                                    # [n_q, d]
    dvc = p.T @ do
    dp = do @ vc.T
    dd = np.sum(do * o, axis=1, keepdims=True)    # D = rowsum(dO * O)
    ds = p * (dp - dd)
    dq = scale * (ds @ kc)
    dkc = scale * (ds.T @ q)
    return dq, dkc, dvc


def target_attention_bwd(q_cand, k_user, v_user, dout, user_offsets, cand_to_user, scale):
    """Gradients of target attention with respect to its three inputs.

    q_cand, dout [C, n_q, H, d]; k_user, v_user [T, H, d]; user_offsets [U+1];
    cand_to_user [C].  Returns (dq_cand [C, n_q, H, d], dk_user [T, H, d],
    dv_user [T, H, d]), fp64.
    """
    q = _f64(q_cand)
    k = _f64(k_user)
    v = _f64(v_user)
    do = _f64(dout)
    offs = np.asarray(user_offsets, dtype=np.int64)
    c2u = np.asarray(cand_to_user, dtype=np.int64)
    sc = _fp32_scale(scale)
    C, n_q, H, d = q.shape
    dq = np.zeros_like(q)
    dk = np.zeros_like(k)
    dv = np.zeros_like(v)
    for c in range(C):
        u = int(c2u[c])
        a, b = int(offs[u]), int(offs[u + 1])
        if b == a:
            continue  # no keys: the output is the constant 0, its gradient is 0
        kc = k[a:b].copy()  # the broadcast copy this candidate would receive
        vc = v[a:b].copy()
        dkc = np.zeros_like(kc)
        dvc = np.zeros_like(vc)
        for h in range(H):
            g_q, g_k, g_v = _candidate_bwd(q[c, :, h, :], kc[:, h, :], vc[:, h, :], do[c, :, h, :], sc)
            dq[c, :, h, :] = g_q
            dkc[:, h, :] = g_k
            dvc[:, h, :] = g_v
        dk[a:b] += dkc  # adjoint of the copy: gradients of all copies add up
        dv[a:b] += dvc
    return dq, dk, dv


def flops_target_bwd(counts, lengths, n_q: int, H: int, d: int) -> float:
    """Backward FLOPs by the forward's convention (2 per multiply-add, softmax
    not counted): the five products of the recompute-based backward (S, dP,
    dV, dK, dQ), 10 * n_q * L_u * d per candidate and head."""
    c = np.asarray(counts, dtype=np.float64)
    L = np.asarray(lengths, dtype=np.float64)
    return 10.0 * n_q * d * H * float(np.dot(c, L))
