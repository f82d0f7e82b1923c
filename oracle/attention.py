"""CPU oracle for scaled-dot-product attention (forward), float64.

TEST INFRASTRUCTURE. Only the tests, the smoke check and the benchmark's CPU
baseline leg may import or run this module. The GPU library never calls it and
shares no code with it.

What is computed is the plain, materialising definition of attention that the
onecalc.app page "Attention memory" describes (sections "The quadratic term"
and "What this memory is"): every query is compared with every key, giving an
s_q x s_k matrix of pre-softmax scores per (batch item, head); a softmax over
each row turns scores into weights; the output is the weighted sum of the value
rows. The news.hamidun.com glossary entry "Flash attention" (first paragraph)
and the "FlashAttention" section of the onecalc.app page both state that the
tiled method reaches the same output as this definition, so the oracle for the
tiled GPU kernel is the definition itself, evaluated in float64.

Conventions that the pages leave open (each is listed with its reason in the
design notes):
  * tensors are [B, H, s, d] (the layout of torch's scaled_dot_product_attention,
    which the glossary entry names as the place the method lives), d_v = d;
  * scores are scale * q.k; ``scale`` is the exact float32 value the kernel gets;
  * causal masking is top-left aligned: key j is visible to query i iff j <= i;
  * key_padding_mask is uint8 [B, s_k], nonzero = padded key, hidden from every
    query and head of that batch item; causal and padding combine by union;
  * lse_i = M_i + ln(L_i), the natural-log log-sum-exp of the scaled, masked
    scores of row i;
  * a row with every key masked has output 0 and lse = -inf.

Functions:
  attention_fp64            the definition, materialising each score block;
  attention_weights_fp64    the full softmax weight matrix P (tiny inputs);
  attention_online_fp64     the page's block-wise walk over keys and values
                            with running softmax statistics (a second,
                            independent CPU path used to pin the first);
  attention_bruteforce      pure-Python loops with math.exp / math.fsum;
  merge_partials_fp64       combination of results over disjoint key sets
                            into the result over their union (for the key-
                            split forward);
  attention_backward_fp64   gradients of the definition with respect to q, k
                            and v for a given output gradient;
  score_matrix_bytes / score_matrix_gb
                            the closed form of the materialised score memory.
"""
from __future__ import annotations

import math
from typing import Iterable, Optional, Tuple

import numpy as np

__all__ = [
    "score_matrix_bytes",
    "score_matrix_gb",
    "attention_fp64",
    "attention_rows_fp64",
    "attention_weights_fp64",
    "attention_online_fp64",
    "attention_bruteforce",
    "merge_partials_fp64",
    "attention_backward_fp64",
]

NEG_INF = -np.inf


# ----------------------------------------------------------------------------
# Closed form of the score-matrix memory.
# onecalc.app "Attention memory", section "The formula": each head builds its
# own s x s score matrix and each sequence of the batch its own copy, so the
# bytes are batch * heads * s^2 * (bytes per stored score); dividing by 10^9
# gives GB. (The displayed formula itself did not survive text extraction; this
# product is the only reading that reproduces the "Worked example" values.)
# ----------------------------------------------------------------------------
def score_matrix_bytes(B: int, H: int, s: int, e: int) -> int:
    return int(B) * int(H) * int(s) * int(s) * int(e)


def score_matrix_gb(B: int, H: int, s: int, e: int) -> float:
    return score_matrix_bytes(B, H, s, e) / 1e9


# ----------------------------------------------------------------------------
# The steps of the definition, for one (batch item, head) and a block of rows.
# ----------------------------------------------------------------------------
def _scores(q_rows: np.ndarray, k_head: np.ndarray, scale: float) -> np.ndarray:
    """Step 1: S[i, j] = scale * sum_c q[i, c] * k[j, c]  (float64)."""
    return np.float64(scale) * (q_rows @ k_head.T)


def _apply_masks(S: np.ndarray, q_pos: np.ndarray, causal: bool,
                 kpm_row: Optional[np.ndarray]) -> np.ndarray:
    """Step 2: hidden keys get score -inf.

    causal: key j is hidden from query i when j > i (top-left alignment).
    kpm_row: key j is hidden from every query when kpm_row[j] != 0.
    """
    s_k = S.shape[1]
    if causal:
        hidden = np.arange(s_k)[None, :] > q_pos[:, None]
        S[hidden] = NEG_INF
    if kpm_row is not None:
        S[:, np.asarray(kpm_row) != 0] = NEG_INF
    return S


def _softmax_rows(S: np.ndarray) -> Tuple[np.ndarray, np.ndarray, np.ndarray]:
    """Steps 3-5: row max M, E = exp(S - M), row sum L, weights P = E / L.

    Rows whose every score is -inf (nothing visible) get M = -inf, L = 0 and an
    all-zero weight row.
    """
    M = S.max(axis=1) if S.shape[1] else np.full(S.shape[0], NEG_INF)
    empty = np.isneginf(M)
    M_safe = np.where(empty, 0.0, M)
    E = np.exp(S - M_safe[:, None])          # exp(-inf) == 0 for hidden keys
    L = E.sum(axis=1)
    P = np.zeros_like(E)
    full = ~empty
    P[full] = E[full] / L[full, None]
    return P, M, L


def _weighted_values(P: np.ndarray, v_head: np.ndarray) -> np.ndarray:
    """Step 6: O[i, :] = sum_j P[i, j] * v[j, :]."""
    return P @ v_head


def _log_sum_exp(M: np.ndarray, L: np.ndarray) -> np.ndarray:
    """Step 7: lse_i = M_i + ln(L_i); -inf for a row with nothing visible."""
    out = np.full(M.shape, NEG_INF)
    full = ~np.isneginf(M)
    out[full] = M[full] + np.log(L[full])
    return out


def _rows(q_rows, k_head, v_head, scale, q_pos, causal, kpm_row):
    S = _scores(q_rows, k_head, scale)
    S = _apply_masks(S, q_pos, causal, kpm_row)
    P, M, L = _softmax_rows(S)
    return _weighted_values(P, v_head), _log_sum_exp(M, L), P


def _as_f64(x) -> np.ndarray:
    return np.ascontiguousarray(x, dtype=np.float64)


def _check(q, k, v, kpm):
    if q.ndim != 4 or k.ndim != 4 or v.ndim != 4:
        raise ValueError("q, k, v must be [B, H, s, d]")
    B, H, s_q, d = q.shape
    if k.shape[:2] != (B, H) or v.shape != k.shape or k.shape[3] != d:
        raise ValueError(f"shape mismatch q{q.shape} k{k.shape} v{v.shape}")
    if kpm is not None and np.asarray(kpm).shape != (B, k.shape[2]):
        raise ValueError("key_padding_mask must be [B, s_k]")


def attention_fp64(q, k, v, scale: float, causal: bool = False,
                   key_padding_mask=None, row_block: int = 2048):
    """The definition, in float64, for every (b, h).

    The s_q x s_k score block is materialised ``row_block`` query rows at a time
    (every step is row-local, so this changes nothing in the result; it only
    keeps the host footprint bounded at long sequence lengths).
    Returns (O [B,H,s_q,d] float64, lse [B,H,s_q] float64).
    """
    q, k, v = _as_f64(q), _as_f64(k), _as_f64(v)
    _check(q, k, v, key_padding_mask)
    B, H, s_q, d = q.shape
    O = np.zeros((B, H, s_q, d))
    lse = np.full((B, H, s_q), NEG_INF)
    for b in range(B):
        kpm_row = None if key_padding_mask is None else np.asarray(key_padding_mask)[b]
        for h in range(H):
            for r0 in range(0, s_q, row_block):
                r1 = min(s_q, r0 + row_block)
                o, l, _ = _rows(q[b, h, r0:r1], k[b, h], v[b, h], scale,
                                np.arange(r0, r1), causal, kpm_row)
                O[b, h, r0:r1] = o
                lse[b, h, r0:r1] = l
    return O, lse


def attention_rows_fp64(q, k, v, scale: float, causal: bool, key_padding_mask,
                        picks: Iterable[Tuple[int, int, np.ndarray]]):
    """The definition for selected rows only: picks = [(b, h, row_indices), ...].

    Each row is computed exactly as attention_fp64 would (rows are independent),
    so sampled parity at full size needs only these rows' scores.
    Returns a list of (O_rows float64 [n, d], lse_rows float64 [n]).
    """
    out = []
    for b, h, rows in picks:
        rows = np.asarray(rows, dtype=np.int64)
        kpm_row = None if key_padding_mask is None else np.asarray(key_padding_mask)[b]
        o, l, _ = _rows(_as_f64(q[b, h, rows]), _as_f64(k[b, h]), _as_f64(v[b, h]),
                        scale, rows, causal, kpm_row)
        out.append((o, l))
    return out


def attention_weights_fp64(q, k, scale: float, causal: bool = False,
                           key_padding_mask=None) -> np.ndarray:
    """The full softmax weight matrix P [B, H, s_q, s_k] (for tiny inputs)."""
    q, k = _as_f64(q), _as_f64(k)
    B, H, s_q, d = q.shape
    s_k = k.shape[2]
    P = np.zeros((B, H, s_q, s_k))
    for b in range(B):
        kpm_row = None if key_padding_mask is None else np.asarray(key_padding_mask)[b]
        for h in range(H):
            S = _apply_masks(_scores(q[b, h], k[b, h], scale), np.arange(s_q), causal, kpm_row)
            P[b, h] = _softmax_rows(S)[0]
    return P


# ----------------------------------------------------------------------------
# Second CPU path: the block-wise walk.
# onecalc.app "Attention memory", section "FlashAttention": keys and values are
# visited in small blocks while running softmax statistics are kept, so only
# one block is needed at a time. news.hamidun.com "Flash attention", second
# paragraph: blocks that fit on-chip memory, a numerically stable softmax that
# merges partial results step by step, and the full matrix is never stored.
# Per row: running max m, running sum l and an unnormalised output acc; a new
# block with row max mb moves the reference to m' = max(m, mb), rescales the old
# sum and output by exp(m - m'), adds exp(s - m') and its weighted values; the
# output is acc / l at the end.
# ----------------------------------------------------------------------------
def attention_online_fp64(q, k, v, scale: float, causal: bool = False,
                          key_padding_mask=None, block: int = 16):
    q, k, v = _as_f64(q), _as_f64(k), _as_f64(v)
    _check(q, k, v, key_padding_mask)
    if block < 1:
        raise ValueError("block must be >= 1")
    B, H, s_q, d = q.shape
    s_k = k.shape[2]
    O = np.zeros((B, H, s_q, d))
    lse = np.full((B, H, s_q), NEG_INF)
    qpos = np.arange(s_q)
    for b in range(B):
        hidden_key = (np.zeros(s_k, bool) if key_padding_mask is None
                      else np.asarray(key_padding_mask)[b] != 0)
        for h in range(H):
            m = np.full(s_q, NEG_INF)
            l = np.zeros(s_q)
            acc = np.zeros((s_q, d))
            for j0 in range(0, s_k, block):
                j1 = min(s_k, j0 + block)
                s = np.float64(scale) * (q[b, h] @ k[b, h, j0:j1].T)
                jpos = np.arange(j0, j1)
                hide = hidden_key[j0:j1][None, :] | (causal & (jpos[None, :] > qpos[:, None]))
                s = np.where(hide, NEG_INF, s)
                m_new = np.maximum(m, s.max(axis=1))
                ref = np.where(np.isneginf(m_new), 0.0, m_new)
                alpha = np.exp(m - ref)               # exp(-inf) = 0 when m was -inf
                p = np.exp(s - ref[:, None])
                l = alpha * l + p.sum(axis=1)
                acc = alpha[:, None] * acc + p @ v[b, h, j0:j1]
                m = m_new
            seen = l > 0
            O[b, h][seen] = acc[seen] / l[seen, None]
            lse[b, h][seen] = m[seen] + np.log(l[seen])
    return O, lse


# ----------------------------------------------------------------------------
# Brute force: the definition with Python scalars, for s <= ~32.
# ----------------------------------------------------------------------------
def attention_bruteforce(q, k, v, scale: float, causal: bool = False,
                         key_padding_mask=None):
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    B, H, s_q, d = q.shape
    s_k = k.shape[2]
    O = np.zeros((B, H, s_q, d))
    lse = np.full((B, H, s_q), NEG_INF)
    for b in range(B):
        for h in range(H):
            for i in range(s_q):
                vis = []
                for j in range(s_k):
                    if causal and j > i:
                        continue
                    if key_padding_mask is not None and key_padding_mask[b][j] != 0:
                        continue
                    dot = math.fsum(float(q[b, h, i, c]) * float(k[b, h, j, c]) for c in range(d))
                    vis.append((j, float(scale) * dot))
                if not vis:
                    continue
                mx = max(s for _, s in vis)
                w = [(j, math.exp(s - mx)) for j, s in vis]
                tot = math.fsum(e for _, e in w)
                for c in range(d):
                    O[b, h, i, c] = math.fsum(e * float(v[b, h, j, c]) for j, e in w) / tot
                lse[b, h, i] = mx + math.log(tot)
    return O, lse


# ----------------------------------------------------------------------------
# Results over disjoint key sets -> result over their union.
# The news.hamidun.com glossary entry "Flash attention" (fourth paragraph)
# names inference frameworks and Ring Attention, which partitions the method's
# work over keys across devices; the pages give no formula for recombining the
# parts. It follows from the definition above (onecalc.app "Attention memory",
# section "What this memory is"): for key sets K_1..K_Z that partition the
# visible keys of row i, the row's exp-sum over the union is the sum of the
# per-set sums, L = sum_z exp(lse_z) (each lse_z = M_z + ln L_z, against any
# common reference), and the union's weighted value sum is the sum of the
# per-set ones, sum_z L_z O_z. Hence lse = ln sum_z exp(lse_z) and
# O = sum_z exp(lse_z - lse) O_z. A set in which the row sees no key has
# lse_z = -inf and weight 0; a row that sees no key in any set gets O = 0 and
# lse = -inf, as in the definition.
# ----------------------------------------------------------------------------
def merge_partials_fp64(outs, lses) -> Tuple[np.ndarray, np.ndarray]:
    """outs: [Z, ..., d] per-set outputs; lses: [Z, ...] per-set log-sum-exps.

    Returns (O, lse) of the union, float64.
    """
    outs = _as_f64(outs)
    lses = _as_f64(lses)
    if outs.shape[:-1] != lses.shape:
        raise ValueError("outs must be lses.shape + (d,)")
    M = lses.max(axis=0)                     # a common reference per row
    empty = np.isneginf(M)
    M_safe = np.where(empty, 0.0, M)
    w = np.exp(lses - M_safe[None])          # exp(-inf) == 0 for empty sets
    total = w.sum(axis=0)
    lse = np.full(M.shape, NEG_INF)
    lse[~empty] = M[~empty] + np.log(total[~empty])
    frac = np.zeros_like(w)
    frac[:, ~empty] = w[:, ~empty] / total[None, ~empty]
    O = (frac[..., None] * outs).sum(axis=0)
    return O, lse


# ----------------------------------------------------------------------------
# Gradients of the definition (the backward pass).
# The onecalc.app page "Attention memory", section "What this memory is", notes
# that training frameworks keep the materialised score matrix for the backward
# pass unless checkpointing or a fused kernel does without it, and the
# news.hamidun.com glossary entry "Flash attention" (third paragraph) puts the
# method's gains in training. The pages give no formulas for the backward pass;
# these are the derivatives of the definition's steps, chained in reverse:
#   O = P V                 ->  dV = P^T dO,   dP = dO V^T
#   P = softmax_row(S)      ->  dS[i, j] = P[i, j] (dP[i, j] - sum_j' P[i, j'] dP[i, j'])
#   S = scale q k^T + mask  ->  dQ = scale dS K,   dK = scale dS^T Q
# (hidden entries have P = 0, so they carry no gradient; a row with no visible
# key has P = 0 and contributes nothing).
# ----------------------------------------------------------------------------
def _softmax_backward(P: np.ndarray, dP: np.ndarray) -> np.ndarray:
    """dS = P * (dP - rowsum(P * dP))."""
    return P * (dP - (P * dP).sum(axis=1, keepdims=True))


def attention_backward_fp64(q, k, v, dout, scale: float, causal: bool = False,
                            key_padding_mask=None, row_block: int = 2048):
    """Returns (dq, dk, dv), float64, shaped like q, k, v.

    P is rebuilt from the definition for each block of ``row_block`` query
    rows (rows are independent in every step except the sums over rows in dK
    and dV, which accumulate over the blocks).
    """
    q, k, v, dout = _as_f64(q), _as_f64(k), _as_f64(v), _as_f64(dout)
    _check(q, k, v, key_padding_mask)
    if dout.shape != q.shape:
        raise ValueError("dout must have q's shape")
    B, H, s_q, d = q.shape
    dq, dk, dv = np.zeros_like(q), np.zeros_like(k), np.zeros_like(v)
    for b in range(B):
        kpm_row = None if key_padding_mask is None else np.asarray(key_padding_mask)[b]
        for h in range(H):
            for r0 in range(0, s_q, row_block):
                r1 = min(s_q, r0 + row_block)
                _, _, P = _rows(q[b, h, r0:r1], k[b, h], v[b, h], scale,
                                np.arange(r0, r1), causal, kpm_row)
                g = dout[b, h, r0:r1]
                dv[b, h] += P.T @ g
                dP = g @ v[b, h].T
                dS = _softmax_backward(P, dP)
                dq[b, h, r0:r1] = np.float64(scale) * (dS @ k[b, h])
                dk[b, h] += np.float64(scale) * (dS.T @ q[b, h, r0:r1])
    return dq, dk, dv
