"""The seeded generator: determinism, quantisation, and the structure each config promises."""

import numpy as np
import pytest

from workloads import bf16_bits_to_f32, f32_to_bf16_bits, make_workload


def test_bf16_round_to_nearest_even():
    # exactly representable values survive; halfway cases go to the even neighbour
    x = np.array([1.0, -2.5, 1.0 + 2.0 ** -8, 1.0 + 3 * 2.0 ** -8, 1.0 + 2.0 ** -9], dtype=np.float32)
    got = bf16_bits_to_f32(f32_to_bf16_bits(x))
    assert got.tolist() == [1.0, -2.5, 1.0, 1.0 + 4 * 2.0 ** -8, 1.0]
    y = np.random.default_rng(0).standard_normal(10000).astype(np.float32)
    r = bf16_bits_to_f32(f32_to_bf16_bits(y))
    assert np.max(np.abs(r - y) / np.abs(y)) <= 2.0 ** -8  # unit roundoff of an 8-bit significand
    import torch
    t = torch.from_numpy(y).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(t, f32_to_bf16_bits(y))


def test_determinism():
    a = make_workload("c2_typical")
    b = make_workload("c2_typical")
    assert np.array_equal(a.cand_to_user, b.cand_to_user)
    assert np.array_equal(a.raw("k_user"), b.raw("k_user"))
    assert np.array_equal(a.user_offsets, b.user_offsets)


def test_config1_shape():
    w = make_workload("c1_tiny_f32")
    assert w.dtype == "f32" and w.n_users == 4 and w.n_cand == 20 and w.H == 2 and w.d == 32
    assert np.all((w.lengths >= 16) & (w.lengths <= 64))
    assert w.raw("q_cand").dtype == np.float32 and w.raw("q_cand").shape == (20, 1, 2, 32)
    assert w.scale == np.float32(1 / np.sqrt(32))


def test_config2_shape():
    w = make_workload("c2_typical")
    assert w.n_cand == 1024 and w.n_users == 15 and w.n_q == 1 and (w.H, w.d) == (4, 128)
    assert np.all((w.lengths >= 256) & (w.lengths <= 2048))
    c = w.counts
    assert c.sum() == 1024 and np.any(c % 2 == 1)
    assert not np.all(np.diff(w.cand_to_user) >= 0)  # arrives unsorted
    assert w.raw("k_user").dtype == np.uint16


def test_config3_skew_and_odd_tail():
    w = make_workload("c3_skewed")
    c = w.counts
    assert w.n_cand == 1023 and w.n_users == 32
    assert c.max() / 1023 > 0.4
    assert np.sum((c >= 1) & (c <= 3)) >= 5
    assert np.sum(c % 2 == 1) >= 10
    ones = np.where(w.lengths == 1)[0]
    assert len(ones) >= 2 and np.all(c[ones] > 0)  # length-1 users that hold candidates


@pytest.mark.slow
def test_config4_and_5_shapes():
    w = make_workload("c4_large")
    assert (w.n_cand, w.n_users, w.n_q, w.H, w.d) == (10000, 150, 4, 8, 128)
    assert np.all((w.lengths >= 512) & (w.lengths <= 4096))
    w5 = make_workload("c5_fused")
    assert w5.with_self and w5.raw("q_user").shape == w5.raw("k_user").shape
    assert (w5.n_cand, w5.n_users) == (2048, 30)
