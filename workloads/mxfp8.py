"""Seeded synthetic MXFP8 inputs for IKBO target attention.

The attention structure (user lengths, candidate-to-user mapping, n_q, H) of
a workload is drawn with the recipe and seed of the bf16 configuration of the
same name (``workloads.ikbo``), from its own generator, so the shapes match
the bf16 workloads without drawing their values.  The values are then drawn
directly in the MX format, from a second PCG64 stream (seed + 500), in the
order q, k, v:

* per block of 32 elements an offset u ~ U{-1, 0, 1, 2}: the block's scale
  code is E8M0 123 + u (2^(u - 4)) and its element codes are torch's fp32 ->
  float8_e4m3fn conversion of N(0,1) * 16 * 2^-u draws, so every block has
  its own scale and code magnitudes while the dequantized values stay about
  N(0,1), as for the bf16 workloads (every code finite: the draws stay far
  below 448).

No scale is derived from the values: this module holds no part of the
quantization rule the method applies to P.

Layouts (row-major, uint8):
    q_codes [C, n_q, H, d]   q_scales [C, n_q, H, d/32]
    k_codes [T, H, d]        k_scales [T, H, d/32]
    v_codes [T, H, d]        v_scales [NVB, H, d]   (32-key blocks from each user's first key)
"""

from __future__ import annotations

from dataclasses import dataclass

import numpy as np

MX_NAMES = ("mx_tiny", "mx_c2_typical", "mx_c3_skewed", "mx_c4_large")
_BLOCK = 32
_VALUE_SEED_OFFSET = 500


@dataclass
class MxWorkload:
    name: str
    seed: int
    n_users: int
    n_cand: int
    n_q: int
    H: int
    d: int
    lengths: np.ndarray
    user_offsets: np.ndarray      # int32 [U + 1]
    cand_to_user: np.ndarray      # int32 [C]
    v_block_offsets: np.ndarray   # int32 [U + 1], first V-scale block of each user
    scale: np.float32
    q_codes: np.ndarray
    q_scales: np.ndarray
    k_codes: np.ndarray
    k_scales: np.ndarray
    v_codes: np.ndarray
    v_scales: np.ndarray

    @property
    def total_len(self) -> int:
        return int(self.user_offsets[-1])

    @property
    def counts(self) -> np.ndarray:
        return np.bincount(self.cand_to_user, minlength=self.n_users)

    def arrays(self):
        return (self.q_codes, self.q_scales, self.k_codes, self.k_scales, self.v_codes, self.v_scales)


def _blocked(rng: np.random.Generator, shape, along_last: bool, v_blocks=None):
    """Codes [shape] and scale codes: blocks of 32 along the last axis
    (along_last), or along the token axis with v_blocks = (number of blocks,
    block of each token)."""
    import torch
    x = rng.standard_normal(int(np.prod(shape)), dtype=np.float32).reshape(shape) * np.float32(16.0)
    if along_last:
        u = rng.integers(-1, 2, size=shape[:-1] + (shape[-1] // _BLOCK,), endpoint=True)
        x = x * np.repeat(np.exp2(-u), _BLOCK, axis=-1).astype(np.float32)
    else:
        nvb, blk_of_tok = v_blocks
        u = rng.integers(-1, 2, size=(nvb,) + tuple(shape[1:]), endpoint=True)
        x = x * np.exp2(-u).astype(np.float32)[blk_of_tok]
    codes = torch.from_numpy(np.ascontiguousarray(x)).to(torch.float8_e4m3fn).view(torch.uint8).numpy().copy()
    return codes, (123 + u).astype(np.uint8)


def _structure(name: str):
    """(seed, lengths, cand_to_user, n_q, H) with the bf16 config's recipe."""
    from .ikbo import _multinomial_mapping
    if name == "mx_tiny":
        seed = 1201
        rng = np.random.Generator(np.random.PCG64(seed))
        L = np.array([1, 31, 32, 33, 70, 0, 130, 5], dtype=np.int64)
        c2u = np.array([0, 1, 2, 3, 4, 6, 7, 4, 6, 3, 1, 0, 7, 2, 6, 4], dtype=np.int32)
        return seed, L, rng.permutation(c2u).astype(np.int32), 2, 2
    seed = {"mx_c2_typical": 1002, "mx_c3_skewed": 1003, "mx_c4_large": 1004}[name]
    rng = np.random.Generator(np.random.PCG64(seed))
    if name == "mx_c2_typical":
        L = rng.integers(256, 2048, size=15, endpoint=True)
        return seed, L, _multinomial_mapping(rng, 1024, 15), 1, 4
    if name == "mx_c3_skewed":
        L = rng.integers(1, 4096, size=32, endpoint=True)
        L[rng.choice(32, 2, replace=False)] = 1
        k = rng.zipf(1.2, size=1023)
        perm = rng.permutation(32)
        return seed, L, perm[np.minimum(k, 32) - 1].astype(np.int32), 1, 4
    L = rng.integers(512, 4096, size=150, endpoint=True)
    return seed, L, _multinomial_mapping(rng, 10000, 150), 4, 8


def _fill(name, seed, lengths, cand_to_user, n_q, H, d=128) -> MxWorkload:
    lengths = np.asarray(lengths, dtype=np.int64)
    offs = np.zeros(lengths.size + 1, dtype=np.int64)
    np.cumsum(lengths, out=offs[1:])
    nblk = (lengths + _BLOCK - 1) // _BLOCK
    vbo = np.zeros(lengths.size + 1, dtype=np.int64)
    np.cumsum(nblk, out=vbo[1:])
    C, T, NVB = int(cand_to_user.size), int(offs[-1]), int(vbo[-1])
    rng = np.random.Generator(np.random.PCG64(seed + _VALUE_SEED_OFFSET))
    q_codes, q_scales = _blocked(rng, (C, n_q, H, d), True)
    k_codes, k_scales = _blocked(rng, (T, H, d), True)
    # V blocks: 32 keys of one user, per head and column
    u_of_tok = np.repeat(np.arange(lengths.size), lengths)
    blk_of_tok = vbo[u_of_tok] + (np.arange(T) - offs[u_of_tok]) // _BLOCK
    v_codes, v_scales = _blocked(rng, (T, H, d), False, (NVB, blk_of_tok))
    return MxWorkload(name=name, seed=seed, n_users=int(lengths.size), n_cand=C, n_q=n_q, H=H, d=d,
                      lengths=lengths, user_offsets=offs.astype(np.int32),
                      cand_to_user=np.asarray(cand_to_user, dtype=np.int32), v_block_offsets=vbo.astype(np.int32),
                      scale=np.float32(1.0 / np.sqrt(d)), q_codes=q_codes, q_scales=q_scales, k_codes=k_codes,
                      k_scales=k_scales, v_codes=v_codes, v_scales=v_scales)


def make_mxfp8(name: str) -> MxWorkload:
    """mx_tiny        8 users (L = 1, 31, 32, 33, 70, 0, 130, 5), 16 candidates, n_q=2, H=2, d=128.
    mx_c2_typical  the typical request's structure (15 users, Multinomial(1024), L~U{256..2048}), H=4.
    mx_c3_skewed   the skewed request's structure (32 users, Zipf(1.2) counts, two users of length 1), H=4.
    mx_c4_large    the large request's structure (150 users, 10,000 candidates, n_q=4), H=8."""
    if name not in MX_NAMES:
        raise KeyError(f"unknown MXFP8 workload {name!r}; known: {MX_NAMES}")
    seed, L, c2u, n_q, H = _structure(name)
    return _fill(name, seed, L, c2u, n_q, H)


def make_mxfp8_custom(seed: int, lengths, cand_to_user, n_q: int = 1, H: int = 2, name: str = "mx_custom") -> MxWorkload:
    """Caller-chosen lengths and mapping (edge cases), d = 128."""
    return _fill(name, int(seed), lengths, np.asarray(cand_to_user, dtype=np.int32), n_q, H)
