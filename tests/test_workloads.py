"""The seeded input generator (CPU only)."""
import numpy as np
import torch

from workloads import (WORKLOADS, HEADLINE, bf16_bits_to_f32, generate, random_case,
                       round_to_bf16, padding_mask_from_lengths)


def test_bf16_rounding_matches_torch():
    rng = np.random.default_rng(0)
    x = np.concatenate([rng.standard_normal(100000).astype(np.float32) * 10.0 ** rng.integers(-30, 30, 100000),
                        np.array([0.0, -0.0, np.inf, -np.inf, 1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8,
                                  3.3895314e38], np.float32)]).astype(np.float32)
    ours = round_to_bf16(x)
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(ours, ref)
    assert np.array_equal(bf16_bits_to_f32(ours), torch.from_numpy(x).to(torch.bfloat16).float().numpy())


def test_generation_is_seeded_and_shaped():
    w = WORKLOADS[0]
    a, b = generate(w), generate(w)
    for n in ("q", "k", "v"):
        assert a[n].dtype == np.uint16 and a[n].shape == (1, 1, 128, 64)
        assert np.array_equal(a[n], b[n])
    assert a["kpm"] is None and a["scale"] == np.float32(0.125)
    assert HEADLINE.s_q == 8192 and HEADLINE.causal and HEADLINE.d == 128


def test_padding_workload_lengths():
    w = WORKLOADS[3]
    g = generate(w)
    L = g["lengths"]
    assert L.shape == (4,) and np.all(L >= 1024) and np.all(L <= 2048)
    assert np.array_equal(g["kpm"], padding_mask_from_lengths(L, 2048))
    assert g["kpm"].dtype == np.uint8 and g["kpm"].shape == (4, 2048)


def test_k_multiplier_applied_before_rounding():
    c1 = random_case(7, 1, 1, 8, 8, 16, k_mult=3.0)
    rng = np.random.Generator(np.random.PCG64(7))
    rng.standard_normal(size=(1, 1, 8, 16), dtype=np.float32)
    k = rng.standard_normal(size=(1, 1, 8, 16), dtype=np.float32) * np.float32(3.0)
    assert np.array_equal(c1["k"], round_to_bf16(k))


def test_flop_formula():
    assert WORKLOADS[2].flops() == 4 * 32 * 8192 * 8192 * 128 / 2
    assert WORKLOADS[3].flops() == 4 * 4 * 16 * 2048 * 2048 * 64
