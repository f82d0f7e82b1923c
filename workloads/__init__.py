"""Seeded synthetic inputs for the attention forward pass.

This module only draws numbers and rounds them to bfloat16. It holds none of
the attention arithmetic, so both the CPU oracle and the GPU path can be fed
from it without sharing any of the method's code.

The five named workloads follow the shapes the pages use: the onecalc.app
"Attention memory" worked example (one sequence, 32 heads, 4,096 and 8,192
tokens, 16-bit scores), and the news.hamidun.com "Flash attention" glossary
example of 32,000-token training sequences for a 7B model (s = 32768, H = 32,
d = 128 stands in for that layer). Every tensor is drawn from N(0, 1) in
float32 with NumPy's PCG64, then rounded to bfloat16 with round-to-nearest-even,
so the oracle and the kernel see bit-identical values.

For the 8-bit-float forward, the same float32 draws are quantised per
(batch item, head) to OCP E4M3 codes with a float32 descale factor each
(``quantize_heads_e4m3``); the rounding is a number-format conversion, not a
step of the attention method.
"""
from __future__ import annotations

import dataclasses
import math
from typing import Optional

import numpy as np

__all__ = [
    "Workload",
    "WORKLOADS",
    "HEADLINE",
    "SPLIT_WORKLOADS",
    "round_to_bf16",
    "bf16_bits_to_f32",
    "round_to_e4m3",
    "quantize_heads_e4m3",
    "generate",
    "random_case",
    "padding_mask_from_lengths",
    "scale_for",
]


def round_to_bf16(x: np.ndarray) -> np.ndarray:
    """Round float32 values to bfloat16, round-to-nearest-even.

    Returns the 16-bit patterns (uint16). NaN stays a quiet NaN; +-inf stay.
    (u + 0x7FFF + lsb) cannot wrap 32 bits for any non-NaN pattern: the largest,
    -inf = 0xFF800000, gives 0xFF807FFF.
    """
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32)
    t = (u >> np.uint32(16)) & np.uint32(1)
    t += np.uint32(0x7FFF)
    t += u
    t >>= np.uint32(16)
    rounded = t.astype(np.uint16)
    nan = np.isnan(x)
    if nan.any():
        rounded[nan] = ((u[nan] >> np.uint32(16)) | np.uint32(0x40)).astype(np.uint16)
    return rounded


def bf16_bits_to_f32(bits: np.ndarray) -> np.ndarray:
    """Widen bfloat16 bit patterns (uint16) to the exactly equal float32 values."""
    return (np.ascontiguousarray(bits, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def round_to_e4m3(x: np.ndarray) -> np.ndarray:
    """Round float32 values to the OCP 8-bit float E4M3 (1 sign, 4 exponent bits
    with bias 7, 3 mantissa bits, subnormals, no infinities, largest finite
    magnitude 448) with round-to-nearest-even, saturating at +-448.

    Returns uint8 bit patterns; NaN becomes 0x7F. Used only to make FP8 inputs.
    """
    x = np.ascontiguousarray(x, dtype=np.float32)
    a = np.abs(x).astype(np.float64)
    a[np.isnan(a)] = 0.0
    # a = f * 2**E with f in [0.5, 1): the binade exponent is E - 1; below 2**-6
    # every value is on the subnormal grid of step 2**-9
    _, E = np.frexp(a)
    e = np.maximum(E.astype(np.float64) - 1.0, -6.0)
    step = np.exp2(e - 3.0)
    r = np.minimum(np.rint(a / step) * step, 448.0)  # may carry into the next binade
    _, E2 = np.frexp(r)
    e2 = E2.astype(np.float64) - 1.0
    sub = r < 2.0 ** -6
    code_sub = np.rint(r / 2.0 ** -9)
    e2n = np.maximum(e2, -6.0)
    code_n = (e2n + 7.0) * 8.0 + np.rint((r / np.exp2(e2n) - 1.0) * 8.0)
    bits = np.where(sub, code_sub, code_n).astype(np.uint8)
    bits |= (np.signbit(x).astype(np.uint8) << np.uint8(7))
    bits[np.isnan(x)] = np.uint8(0x7F)
    return bits


def quantize_heads_e4m3(x: np.ndarray) -> tuple:
    """Per-(b, h) E4M3 quantisation of a float32 [B, H, s, d] tensor.

    descale[b, h] = max|x[b, h]| / 448 (1 for an all-zero head), and the
    returned bits are round_to_e4m3(x / descale): the decoded values times
    descale approximate x, and each head uses the format's full range.
    Returns (bits uint8 [B, H, s, d], descale float32 [B, H]).
    """
    x = np.ascontiguousarray(x, dtype=np.float32)
    amax = np.abs(x).max(axis=(2, 3)) if x.size else np.zeros(x.shape[:2], np.float32)
    descale = np.where(amax > 0, amax / np.float32(448.0), np.float32(1.0)).astype(np.float32)
    bits = round_to_e4m3(x / descale[:, :, None, None])
    return bits, descale


def scale_for(d: int) -> np.float32:
    """The float32 value of 1/sqrt(d) that is handed to both sides."""
    return np.float32(1.0 / math.sqrt(d))


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    B: int
    H: int
    s_q: int
    s_k: int
    d: int
    causal: bool
    padded: bool        # key padding mask with per-sequence valid length ~ U{s/2..s}
    k_mult: float       # K drawn, multiplied in float32, then rounded once
    seed: int

    @property
    def scale(self) -> np.float32:
        return scale_for(self.d)

    def flops(self) -> float:
        """Metric FLOPs: 4*B*H*s_q*s_k*d, halved when causal."""
        f = 4.0 * self.B * self.H * self.s_q * self.s_k * self.d
        return f / 2.0 if self.causal else f


WORKLOADS = (
    Workload("B=1,H=1,s=128,d=64,dense", 1, 1, 128, 128, 64, False, False, 1.0, 44001),
    Workload("B=1,H=32,s=4096,d=128,causal", 1, 32, 4096, 4096, 128, True, False, 1.0, 44002),
    Workload("B=1,H=32,s=8192,d=128,causal", 1, 32, 8192, 8192, 128, True, False, 1.0, 44003),
    Workload("B=4,H=16,s=2048,d=64,key-padding", 4, 16, 2048, 2048, 64, False, True, 1.0, 44004),
    Workload("B=1,H=32,s=32768,d=128,causal,Kx3", 1, 32, 32768, 32768, 128, True, False, 3.0, 44005),
)

# The configuration the headline throughput is quoted on (s = 8192, d = 128, causal).
HEADLINE = WORKLOADS[2]

# Shapes for the key-split forward: a 1024-query chunk against the glossary
# example's 32,000-token context (32768 keys), the prefill step of an inference
# framework (the glossary's fourth paragraph). A plain launch has only
# ceil(1024 / 256) * 32 = 128 workgroups here, half the device's compute units.
SPLIT_WORKLOADS = (
    Workload("B=1,H=32,s_q=1024,s_k=32768,d=128,prefill-chunk", 1, 32, 1024, 32768, 128, False,
             False, 1.0, 44006),
)


def padding_mask_from_lengths(lengths: np.ndarray, s_k: int) -> np.ndarray:
    """uint8 [B, s_k]; 1 marks a padded key (j >= length of that sequence)."""
    lengths = np.asarray(lengths, dtype=np.int64)
    return (np.arange(s_k)[None, :] >= lengths[:, None]).astype(np.uint8)


def _draw(rng: np.random.Generator, shape, mult: float = 1.0) -> np.ndarray:
    x = rng.standard_normal(size=shape, dtype=np.float32)
    if mult != 1.0:
        x *= np.float32(mult)
    return round_to_bf16(x)


def generate(w: Workload, heads: Optional[slice] = None) -> dict:
    """Draw Q, K, V (in that order), then the valid lengths, for one workload.

    Returned arrays hold bfloat16 bit patterns (uint16, [B,H,s,d], contiguous).
    ``heads`` optionally keeps a slice of the head axis after drawing (the draw
    itself is always the full tensor so the values do not depend on it).
    """
    rng = np.random.Generator(np.random.PCG64(w.seed))
    q = _draw(rng, (w.B, w.H, w.s_q, w.d))
    k = _draw(rng, (w.B, w.H, w.s_k, w.d), w.k_mult)
    v = _draw(rng, (w.B, w.H, w.s_k, w.d))
    kpm = None
    lengths = None
    if w.padded:
        lengths = rng.integers(w.s_k // 2, w.s_k, size=w.B, endpoint=True)
        kpm = padding_mask_from_lengths(lengths, w.s_k)
    if heads is not None:
        q, k, v = (np.ascontiguousarray(t[:, heads]) for t in (q, k, v))
    return dict(q=q, k=k, v=v, kpm=kpm, lengths=lengths, scale=w.scale,
                causal=w.causal)


def random_case(seed: int, B: int, H: int, s_q: int, s_k: int, d: int, *,
                causal: bool = False, mask: str = "none", q_mult: float = 1.0,
                k_mult: float = 1.0, scale: Optional[float] = None) -> dict:
    """A seeded case of any shape, for edge and ragged tests.

    mask: "none"; "lengths" (valid length per sequence ~ U{0..s_k}); "random"
    (each key padded independently with probability 1/2, so the mask is not a
    suffix); "all" (every key padded); "blocks" (interior blocks padded: keys
    512 .. 1535, so 64-key tiles 8 .. 23 hold no visible key, and a ragged
    block from s_k - 700 to s_k - 300, in every sequence; sequence 0 also
    pads its first 200 keys and sequence 1, if any, its last 100); "prefix"
    (the first s_k / 3 keys of every sequence padded, as in left-padded
    batches; sequence 1, if any, also pads its last 50).
    """
    rng = np.random.Generator(np.random.PCG64(seed))
    q = _draw(rng, (B, H, s_q, d), q_mult)
    k = _draw(rng, (B, H, s_k, d), k_mult)
    v = _draw(rng, (B, H, s_k, d))
    kpm = None
    if mask == "lengths":
        lengths = rng.integers(0, s_k, size=B, endpoint=True)
        kpm = padding_mask_from_lengths(lengths, s_k)
    elif mask == "random":
        kpm = (rng.random((B, s_k)) < 0.5).astype(np.uint8)
    elif mask == "all":
        kpm = np.ones((B, s_k), dtype=np.uint8)
    elif mask == "blocks":
        kpm = np.zeros((B, s_k), dtype=np.uint8)
        kpm[:, 512:1536] = 1
        kpm[:, max(0, s_k - 700):max(0, s_k - 300)] = 1
        kpm[0, :200] = 1
        if B > 1:
            kpm[1, max(0, s_k - 100):] = 1
    elif mask == "prefix":
        kpm = np.zeros((B, s_k), dtype=np.uint8)
        kpm[:, :s_k // 3] = 1
        if B > 1:
            kpm[1, max(0, s_k - 50):] = 1
    elif mask != "none":
        raise ValueError(f"unknown mask kind {mask!r}")
    sc = scale_for(d) if scale is None else np.float32(scale)
    return dict(q=q, k=k, v=v, kpm=kpm, scale=sc, causal=causal)
