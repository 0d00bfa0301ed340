"""Seeded synthetic inputs for IKBO linear compression (LCE).

The operation (IKBO blog, section 2 and App. 2): a learned projection W of
shape (M, K) maps each candidate's K input embeddings of width N to M
compressed ones, ``(M, K) @ (B, K, N) -> (B, M, N)``.  The K embeddings of a
candidate are the concatenation, along K, of K_u user embeddings (the same for
every candidate of a user) and K_c candidate embeddings.

Tensors (row-major, contiguous; bf16 held as uint16 bit patterns):
    w        [M, K_u + K_c]   user columns first
    x_user   [U, K_u, N]
    x_cand   [B, K_c, N]
    cand_to_user  int32 [B]

Draw order with ``numpy.random.Generator(PCG64(seed))``: mapping -> w -> x_user
-> x_cand.  Values are fp32 standard-normal draws (w scaled by 1/sqrt(K) so
outputs stay O(1)), rounded to bf16 to nearest-even.
"""

from __future__ import annotations

from dataclasses import dataclass, field

import numpy as np

from .ikbo import bf16_bits_to_f32, f32_to_bf16_bits

LCE_NAMES = ("lce_tiny", "lce_typical", "lce_ratio1000")


@dataclass
class LceWorkload:
    name: str
    seed: int
    n_users: int
    n_cand: int
    M: int
    K_u: int
    K_c: int
    N: int
    cand_to_user: np.ndarray
    tensors: dict = field(default_factory=dict)

    @property
    def K(self) -> int:
        return self.K_u + self.K_c

    def raw(self, name: str) -> np.ndarray:
        return self.tensors[name]

    def values(self, name: str) -> np.ndarray:
        return bf16_bits_to_f32(self.tensors[name])

    @property
    def counts(self) -> np.ndarray:
        return np.bincount(self.cand_to_user.astype(np.int64), minlength=self.n_users)


def make_lce_custom(seed: int, n_users: int, cand_to_user, M: int, K_u: int, K_c: int, N: int,
                    name: str = "lce_custom") -> LceWorkload:
    rng = np.random.Generator(np.random.PCG64(int(seed)))
    c2u = np.asarray(cand_to_user, dtype=np.int32)
    return _fill(name, int(seed), rng, n_users, c2u, M, K_u, K_c, N)


def _fill(name, seed, rng, n_users, c2u, M, K_u, K_c, N) -> LceWorkload:
    K = K_u + K_c
    w = rng.standard_normal(M * K, dtype=np.float32).reshape(M, K) * np.float32(1.0 / np.sqrt(K))
    xu = rng.standard_normal(n_users * K_u * N, dtype=np.float32).reshape(n_users, K_u, N)
    xc = rng.standard_normal(len(c2u) * K_c * N, dtype=np.float32).reshape(len(c2u), K_c, N)
    t = {"w": f32_to_bf16_bits(w).reshape(M, K), "x_user": f32_to_bf16_bits(xu).reshape(n_users, K_u, N),
         "x_cand": f32_to_bf16_bits(xc).reshape(len(c2u), K_c, N)}
    return LceWorkload(name=name, seed=seed, n_users=n_users, n_cand=len(c2u), M=M, K_u=K_u, K_c=K_c, N=N,
                       cand_to_user=c2u, tensors=t)


def make_lce(name: str) -> LceWorkload:
    """lce_tiny       3 users, 11 candidates, M=37, K_u=21, K_c=11, N=128 (ragged M and K; oracle-sized).
    lce_typical    the pages' shape: B=1024 candidates over 15 users (Multinomial, ratio ~70),
                   M=433, K=2044 read as K_u = K_c = 1022, N=256.
    lce_ratio1000  B=2000 candidates over 2 users (ratio 1000), same M, K, N.
    """
    seeds = {"lce_tiny": 2001, "lce_typical": 2002, "lce_ratio1000": 2003}
    if name not in seeds:
        raise KeyError(f"unknown LCE workload {name!r}; known: {LCE_NAMES}")
    seed = seeds[name]
    rng = np.random.Generator(np.random.PCG64(seed))
    if name == "lce_tiny":
        U, B, M, K_u, K_c, N = 3, 11, 37, 21, 11, 128
    elif name == "lce_typical":
        U, B, M, K_u, K_c, N = 15, 1024, 433, 1022, 1022, 256
    else:
        U, B, M, K_u, K_c, N = 2, 2000, 433, 1022, 1022, 256
    counts = rng.multinomial(B, [1.0 / U] * U)
    c2u = rng.permutation(np.repeat(np.arange(U, dtype=np.int32), counts)).astype(np.int32)
    return _fill(name, seed, rng, U, c2u, M, K_u, K_c, N)


LCE_NESTED_NAMES = ("lce3_tiny", "lce3_typical")


@dataclass
class LceNestedWorkload:
    """Three levels, user -> vendor -> item: vendor_to_user [V], cand_to_vendor [B];
    w [M, K_u + K_v + K_c] (user, vendor, item columns), x_user [U, K_u, N],
    x_vendor [V, K_v, N], x_cand [B, K_c, N]."""
    name: str
    seed: int
    n_users: int
    n_vendors: int
    n_cand: int
    M: int
    K_u: int
    K_v: int
    K_c: int
    N: int
    vendor_to_user: np.ndarray
    cand_to_vendor: np.ndarray
    tensors: dict = field(default_factory=dict)

    @property
    def K(self) -> int:
        return self.K_u + self.K_v + self.K_c

    def raw(self, name: str) -> np.ndarray:
        return self.tensors[name]

    def values(self, name: str) -> np.ndarray:
        return bf16_bits_to_f32(self.tensors[name])


def _fill_nested(name, seed, rng, n_users, v2u, c2v, M, K_u, K_v, K_c, N) -> LceNestedWorkload:
    K = K_u + K_v + K_c
    V, B = len(v2u), len(c2v)
    w = rng.standard_normal(M * K, dtype=np.float32).reshape(M, K) * np.float32(1.0 / np.sqrt(K))
    t = {"w": f32_to_bf16_bits(w).reshape(M, K)}
    for key, shape in (("x_user", (n_users, K_u, N)), ("x_vendor", (V, K_v, N)), ("x_cand", (B, K_c, N))):
        x = rng.standard_normal(int(np.prod(shape)), dtype=np.float32).reshape(shape)
        t[key] = f32_to_bf16_bits(x).reshape(shape)
    return LceNestedWorkload(name=name, seed=seed, n_users=n_users, n_vendors=V, n_cand=B, M=M, K_u=K_u, K_v=K_v,
                             K_c=K_c, N=N, vendor_to_user=np.asarray(v2u, np.int32),
                             cand_to_vendor=np.asarray(c2v, np.int32), tensors=t)


def make_lce_nested_custom(seed: int, n_users: int, vendor_to_user, cand_to_vendor, M: int, K_u: int, K_v: int,
                           K_c: int, N: int, name: str = "lce3_custom") -> LceNestedWorkload:
    rng = np.random.Generator(np.random.PCG64(int(seed)))
    return _fill_nested(name, int(seed), rng, n_users, np.asarray(vendor_to_user, np.int32),
                        np.asarray(cand_to_vendor, np.int32), M, K_u, K_v, K_c, N)


def make_lce_nested(name: str) -> LceNestedWorkload:
    """lce3_tiny     2 users, 5 vendors, 13 items, M=37, K_u=11, K_v=9, K_c=7, N=128 (oracle-sized).
    lce3_typical  the two-level request's B, M, N and total K (1024 items, M=433, K=2044, N=256) with a
                  vendor level: 15 users, 120 vendors (Multinomial over users), items Multinomial over
                  vendors (about 8 vendors per user and 8.5 items per vendor, ratio ~68 overall), K read as
                  K_u = 682, K_v = K_c = 681.
    Draw order: vendor_to_user, cand_to_vendor (each counts then a permutation), w, x_user, x_vendor, x_cand.
    """
    seeds = {"lce3_tiny": 2101, "lce3_typical": 2102}
    if name not in seeds:
        raise KeyError(f"unknown nested LCE workload {name!r}; known: {LCE_NESTED_NAMES}")
    seed = seeds[name]
    rng = np.random.Generator(np.random.PCG64(seed))
    if name == "lce3_tiny":
        U, V, B, M, K_u, K_v, K_c, N = 2, 5, 13, 37, 11, 9, 7, 128
    else:
        U, V, B, M, K_u, K_v, K_c, N = 15, 120, 1024, 433, 682, 681, 681, 256
    vc = rng.multinomial(V, [1.0 / U] * U)
    v2u = rng.permutation(np.repeat(np.arange(U, dtype=np.int32), vc)).astype(np.int32)
    cc = rng.multinomial(B, [1.0 / V] * V)
    c2v = rng.permutation(np.repeat(np.arange(V, dtype=np.int32), cc)).astype(np.int32)
    return _fill_nested(name, seed, rng, U, v2u, c2v, M, K_u, K_v, K_c, N)
