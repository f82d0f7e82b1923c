"""CPU oracle for attention over 8-bit floating-point inputs, float64.

TEST INFRASTRUCTURE. Only the tests, the smoke check and the benchmark's CPU
baseline leg may import or run this module. The GPU library never calls it and
shares no code with it.

The news.hamidun.com glossary entry "Flash attention" (second paragraph) says
the method's third version added FP8 precision. The pages do not say which
8-bit format, how the inputs are scaled, or what the result means. The
readings taken here:
  * the format is E4M3 of the OCP 8-bit floating point specification: 1 sign
    bit, 4 exponent bits with bias 7, 3 mantissa bits, subnormals when the
    exponent field is 0, no infinities, and NaN only for the two codes with
    every exponent and mantissa bit set (0x7F, 0xFF); the largest finite
    magnitude is 448. It is the E4M3 format the gfx950 matrix cores take;
  * each (batch item, head) slice of q, k and v carries one float32 descale
    factor, so the real value of a code x is descale * decode(x) (no factor
    means 1);
  * the result is the attention definition (oracle.attention.attention_fp64)
    evaluated exactly on those real values. How far a kernel may deviate
    because it rounds the softmax weights to the same 8-bit format is a
    tolerance, derived where the tests use it; it is not part of the
    definition.

Functions:
  e4m3_to_fp64         the value of each E4M3 code, from the format's fields;
  dequantize_heads     codes [B, H, s, d] times per-(b, h) descale factors;
  attention_fp8_fp64   the attention definition on the dequantized inputs.
"""
from __future__ import annotations

from typing import Optional

import numpy as np

from .attention import attention_fp64

__all__ = ["e4m3_to_fp64", "dequantize_heads", "attention_fp8_fp64"]


def e4m3_to_fp64(bits) -> np.ndarray:
    """Value of each OCP E4M3 code (uint8) as float64, NaN for 0x7F and 0xFF.

    Fields: sign s = bit 7, exponent e = bits 6..3, mantissa m = bits 2..0.
    e == 0: (-1)^s * (m / 8) * 2^(1 - 7)       (zero and subnormals)
    e >= 1: (-1)^s * (1 + m / 8) * 2^(e - 7)   (normals)
    """
    b = np.asarray(bits, dtype=np.uint8).astype(np.int64)
    s = np.where((b >> 7) & 1, -1.0, 1.0)
    e = (b >> 3) & 0xF
    m = (b & 0x7).astype(np.float64)
    mag = np.where(e == 0, (m / 8.0) * 2.0 ** (1 - 7), (1.0 + m / 8.0) * np.exp2(e - 7.0))
    val = s * mag
    return np.where((e == 0xF) & (m == 7.0), np.nan, val)


def dequantize_heads(bits, descale: Optional[np.ndarray]) -> np.ndarray:
    """codes [B, H, s, d] -> float64 values, each (b, h) slice times descale[b, h]."""
    x = e4m3_to_fp64(bits)
    if descale is None:
        return x
    ds = np.asarray(descale, dtype=np.float64).reshape(x.shape[0], x.shape[1])
    return x * ds[:, :, None, None]


def attention_fp8_fp64(q8, k8, v8, descale_q=None, descale_k=None, descale_v=None,
                       scale: float = 1.0, causal: bool = False, key_padding_mask=None,
                       row_block: int = 2048):
    """Attention definition on E4M3 inputs with per-(b, h) descale factors.

    Returns (O [B, H, s_q, d] float64, lse [B, H, s_q] float64), exactly the
    plain definition applied to descale * decode(code) for q, k and v.
    """
    q = dequantize_heads(q8, descale_q)
    k = dequantize_heads(k8, descale_k)
    v = dequantize_heads(v8, descale_v)
    return attention_fp64(q, k, v, scale, causal, key_padding_mask, row_block=row_block)
