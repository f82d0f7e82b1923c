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


def test_e4m3_rounding_matches_torch():
    """round_to_e4m3 (input generation) rounds like torch's float8_e4m3fn cast
    (round to nearest even) inside the finite range and saturates outside it."""
    from workloads import round_to_e4m3
    rng = np.random.default_rng(7)
    x = (rng.standard_normal(50000) * np.exp2(rng.uniform(-14, 10, 50000))).astype(np.float32)
    x = np.concatenate([x, np.array([0.0, -0.0, 448.0, 2.0 ** -9, 2.0 ** -10, 3 * 2.0 ** -10,
                                     2.0 ** -11, 464.0, 1e9, -1e9], np.float32)])
    ref = torch.from_numpy(np.clip(x, -448, 448)).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(round_to_e4m3(x), ref)


def test_quantize_heads_uses_full_range_per_head():
    from workloads import quantize_heads_e4m3
    rng = np.random.default_rng(8)
    x = rng.standard_normal((2, 3, 40, 16)).astype(np.float32)
    x[1, 2] *= 0  # an all-zero head keeps descale 1
    bits, ds = quantize_heads_e4m3(x)
    assert bits.dtype == np.uint8 and ds.shape == (2, 3) and ds[1, 2] == 1.0
    mags = bits & 0x7F
    for b in range(2):
        for h in range(3):
            if (b, h) != (1, 2):
                assert mags[b, h].max() == 0x7E  # the head's max maps to 448
    vals = torch.from_numpy(bits.copy()).view(torch.float8_e4m3fn).float().numpy() * ds[:, :, None, None]
    assert np.abs(vals - x).max() <= 2.0 ** -4 * np.abs(x).max() + 1e-7
