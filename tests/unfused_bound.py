"""Derived error bound of the unfused (materialising) forward path, and a CPU
emulation of its rounding steps that checks the bound.

The unfused path stores every score scale * q.k of a (batch item, head) in an
s_q x s_k matrix of 16-bit (bfloat16) elements, the element size of the
onecalc.app page "Attention memory" ("Worked example": 16-bit scores), applies
the masks and the softmax to that matrix in place, and multiplies the stored
weights (bfloat16) by V. The pages fix no tolerance for it; the bound below
follows from the arithmetic. For row i of one (b, h), over its visible keys j:

  M_i   = max_j |S_ij|                      (S the exact scaled scores)
  A_i   = max_j |scale| sum_c |q_ic k_jc|   (bounds |S_ij| and the float32
                                             error of the score product)
  Delta = 2^-8 M_i + 2^-16 A_i              each stored score is within Delta
                                            of the exact one (float32 sum of
                                            at most 128 exact products, then
                                            rounding to bfloat16, relative
                                            error at most 2^-8)
  A softmax of scores each moved by at most Delta changes every weight by a
  factor in [exp(-2 Delta), exp(2 Delta)]. The float32 softmax (exp2 of a
  fused multiply-add against the row max, a sum of s_k terms, a reciprocal)
  and the rounding of the weights to bfloat16 add a relative error
  eta = 2^-8 + 2^-20 (1 + M_i) + (s_k / 64 + 16) 2^-24, so every stored weight
  is within rho = (1 + eta) exp(2 Delta) - 1 of the exact weight, relatively.
  The value product sums s_k bfloat16 products in float32 (relative error at
  most s_k 2^-24 of sum_j P_j |v_j|), and the output is rounded to bfloat16:

  |O - O_ref| <= (1 + 2^-8) (rho + (1 + rho) s_k 2^-24) (P|V|) + 2^-8 |O_ref| + 1e-6
  |lse - lse_ref| <= Delta + (s_k / 64 + 16) 2^-24 + 2^-20 (1 + |lse_ref|)

with P|V| = sum_j P_ij |v_j| (the oracle run on |v|).
"""
from __future__ import annotations

import numpy as np

from workloads import bf16_bits_to_f32, round_to_bf16


def _visible(s_q, s_k, causal, kpm_row):
    vis = np.ones((s_q, s_k), dtype=bool)
    if causal:
        vis &= np.arange(s_k)[None, :] <= np.arange(s_q)[:, None]
    if kpm_row is not None:
        vis &= (np.asarray(kpm_row) == 0)[None, :]
    return vis


def score_extents(q, k, scale, causal, kpm, rows=None):
    """(M, A) per row: the largest |S_ij| and |scale| sum_c |q_ic k_jc| over
    the row's visible keys (0 for a row with none). q, k float64 [B,H,s,d];
    rows: optional list of (b, h, row_indices) to evaluate only those."""
    B, H, s_q, _ = q.shape
    s_k = k.shape[2]
    picks = rows if rows is not None else [(b, h, np.arange(s_q)) for b in range(B) for h in range(H)]
    out = []
    for b, h, r in picks:
        r = np.asarray(r, dtype=np.int64)
        S = abs(scale) * np.abs(q[b, h, r] @ k[b, h].T)
        Aa = abs(scale) * (np.abs(q[b, h, r]) @ np.abs(k[b, h]).T)
        vis = _visible(s_q, s_k, causal, None if kpm is None else kpm[b])[r]
        M = np.where(vis, S, 0.0).max(axis=1) if s_k else np.zeros(len(r))
        A = np.where(vis, Aa, 0.0).max(axis=1) if s_k else np.zeros(len(r))
        out.append((M, A))
    return out


def bounds(M, A, s_k, O_ref, PV_abs, lse_ref):
    """Per-element bound on |O - O_ref| ([n, d]) and per-row bound on
    |lse - lse_ref| ([n]) for rows with extents M, A ([n])."""
    delta = 2.0 ** -8 * M + 2.0 ** -16 * A
    eta = 2.0 ** -8 + 2.0 ** -20 * (1.0 + M) + (s_k / 64 + 16) * 2.0 ** -24
    rho = (1.0 + eta) * np.exp(2.0 * delta) - 1.0
    acc = s_k * 2.0 ** -24
    bO = ((1 + 2.0 ** -8) * (rho + (1 + rho) * acc))[:, None] * PV_abs + 2.0 ** -8 * np.abs(O_ref) + 1e-6
    fin = np.isfinite(lse_ref)
    bL = delta + (s_k / 64 + 16) * 2.0 ** -24 + 2.0 ** -20 * (1.0 + np.where(fin, np.abs(lse_ref), 0.0))
    return bO, bL


def _bf16(x):
    return bf16_bits_to_f32(round_to_bf16(np.asarray(x, dtype=np.float32))).astype(np.float64)


def emulate_unfused(q, k, v, scale, causal, kpm):
    """The unfused path's rounding steps on the CPU: float32 scores rounded to
    bfloat16, masks, a float32 softmax (exp2 of x log2 e - M log2 e) whose
    weights are rounded to bfloat16, the value product accumulated in float32
    (here: float64 then rounded once, within the bound's accumulation term)
    and a bfloat16 output. Returns (O, lse, P) as float64."""
    B, H, s_q, d = q.shape
    s_k = k.shape[2]
    O = np.zeros((B, H, s_q, d))
    lse = np.full((B, H, s_q), -np.inf)
    P = np.zeros((B, H, s_q, s_k))
    log2e = np.float32(1.4426950408889634)
    for b in range(B):
        vis = _visible(s_q, s_k, causal, None if kpm is None else kpm[b])
        for h in range(H):
            S32 = (np.float32(scale) * (q[b, h] @ k[b, h].T).astype(np.float32)).astype(np.float32)
            S = _bf16(S32).astype(np.float32)
            S = np.where(vis, S, np.float32(-np.inf))
            M = S.max(axis=1) if s_k else np.full(s_q, -np.inf, np.float32)
            full = np.isfinite(M)
            Ms = np.where(full, M, np.float32(0)).astype(np.float32)
            x = (S * log2e - (Ms * log2e)[:, None]).astype(np.float32)
            e = np.exp2(x).astype(np.float32)
            L = e.sum(axis=1, dtype=np.float32)
            inv = np.where(full, np.float32(1) / np.where(full, L, 1), 0).astype(np.float32)
            Pb = _bf16(e * inv[:, None])
            P[b, h] = Pb
            O[b, h] = _bf16((Pb @ v[b, h]).astype(np.float32))
            lse[b, h] = np.where(full, M.astype(np.float64) + np.log(np.where(full, L, 1).astype(np.float64)),
                                 -np.inf)
    return O, lse, P
