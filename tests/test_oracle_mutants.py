"""Plant plausible mistakes in the oracle's steps (on the CPU) and check that
each one makes at least one pin fail. This shows the pins constrain every step
of the definition: the score product, the masks, the softmax, the weighted sum
and the log-sum-exp."""
import numpy as np
import pytest

import oracle.attention as A
from oracle_pins import PINS

NEG_INF = -np.inf


def _causal_off_by_one(S, q_pos, causal, kpm_row):
    if causal:
        S[np.arange(S.shape[1])[None, :] >= q_pos[:, None]] = NEG_INF
    if kpm_row is not None:
        S[:, np.asarray(kpm_row) != 0] = NEG_INF
    return S


def _padding_ignored(S, q_pos, causal, kpm_row):
    if causal:
        S[np.arange(S.shape[1])[None, :] > q_pos[:, None]] = NEG_INF
    return S


def _causal_bottom_right(S, q_pos, causal, kpm_row):
    if causal:
        off = S.shape[1] - (q_pos.max() + 1 if q_pos.size else 0)
        S[np.arange(S.shape[1])[None, :] > q_pos[:, None] + off] = NEG_INF
    if kpm_row is not None:
        S[:, np.asarray(kpm_row) != 0] = NEG_INF
    return S


def _no_max_shift(S):
    with np.errstate(over="ignore", invalid="ignore"):
        E = np.exp(S)
        L = E.sum(axis=1)
        P = np.where(L[:, None] > 0, E / np.where(L > 0, L, 1)[:, None], 0.0)
    M = np.zeros(S.shape[0])
    M[~(L > 0)] = NEG_INF
    return P, M, L


def _sum_drops_last_key(S):
    P, M, L = ORIG["_softmax_rows"](S)
    if S.shape[1] > 1:
        Ms = np.where(np.isneginf(M), 0.0, M)
        E = np.exp(S - Ms[:, None])
        L = E[:, :-1].sum(axis=1)
        with np.errstate(invalid="ignore", divide="ignore"):
            P = np.where(L[:, None] > 0, E / np.where(L > 0, L, 1)[:, None], 0.0)
    return P, M, L


def _max_not_subtracted_back(S):
    P, M, L = ORIG["_softmax_rows"](S)
    return P, np.zeros_like(M) * np.where(np.isneginf(M), np.nan, 1.0), L


ORIG = {n: getattr(A, n) for n in ("_scores", "_apply_masks", "_softmax_rows",
                                    "_weighted_values", "_log_sum_exp")}

MUTANTS = {
    "score_without_scale": ("_scores", lambda q, k, s: q @ k.T),
    "score_scale_squared": ("_scores", lambda q, k, s: np.float64(s) ** 2 * (q @ k.T)),
    "score_drops_last_feature": ("_scores", lambda q, k, s: np.float64(s) * (q[:, :-1] @ k[:, :-1].T)),
    "score_operands_swapped": ("_scores", lambda q, k, s: np.float64(s) * (k @ q.T)),
    "causal_off_by_one": ("_apply_masks", _causal_off_by_one),
    "causal_bottom_right": ("_apply_masks", _causal_bottom_right),
    "padding_ignored": ("_apply_masks", _padding_ignored),
    "softmax_without_max_shift": ("_softmax_rows", _no_max_shift),
    "softmax_sum_drops_last_key": ("_softmax_rows", _sum_drops_last_key),
    "lse_ignores_max": ("_softmax_rows", _max_not_subtracted_back),
    "values_transposed_weights": ("_weighted_values", lambda P, v: (P.T @ v[: P.shape[0]]) if P.shape[0] <= v.shape[0] else P @ v[::-1]),
    "values_reversed": ("_weighted_values", lambda P, v: P @ v[::-1]),
    "values_negated": ("_weighted_values", lambda P, v: -(P @ v)),
    "lse_base2": ("_log_sum_exp", lambda M, L: np.where(np.isneginf(M), NEG_INF, M + np.log2(np.where(L > 0, L, 1)))),
    "lse_without_max": ("_log_sum_exp", lambda M, L: np.where(np.isneginf(M), NEG_INF, np.log(np.where(L > 0, L, 1)))),
    "lse_sign": ("_log_sum_exp", lambda M, L: np.where(np.isneginf(M), NEG_INF, M - np.log(np.where(L > 0, L, 1)))),
}


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_mutant_is_caught(name, monkeypatch):
    attr, fn = MUTANTS[name]
    monkeypatch.setattr(A, attr, fn)
    failed = []
    for pin in PINS:
        try:
            with np.errstate(all="ignore"):
                pin()
        except Exception as e:  # AssertionError or a shape error both mean "caught"
            failed.append((pin.__name__, type(e).__name__))
    assert failed, f"mutant {name} passed every pin"


def _merge_plain_average(outs, lses):
    O, lse = ORIG_MERGE(outs, lses)
    return np.asarray(outs).mean(axis=0), lse


def _merge_lse_is_max(outs, lses):
    O, lse = ORIG_MERGE(outs, lses)
    return O, np.asarray(lses).max(axis=0)


def _merge_unnormalised(outs, lses):
    lses = np.asarray(lses)
    w = np.exp(np.where(np.isneginf(lses), -np.inf, lses))
    O = (w[..., None] * np.asarray(outs)).sum(axis=0)
    return O, ORIG_MERGE(outs, lses)[1]


def _merge_weights_reversed(outs, lses):
    return ORIG_MERGE(np.asarray(outs)[::-1], lses)


ORIG_MERGE = A.merge_partials_fp64
MERGE_MUTANTS = {
    "merge_plain_average": _merge_plain_average,
    "merge_lse_is_max": _merge_lse_is_max,
    "merge_unnormalised": _merge_unnormalised,
    "merge_weights_reversed": _merge_weights_reversed,
}


@pytest.mark.parametrize("name", sorted(MERGE_MUTANTS))
def test_merge_mutant_is_caught(name, monkeypatch):
    monkeypatch.setattr(A, "merge_partials_fp64", MERGE_MUTANTS[name])
    failed = []
    for pin in PINS:
        try:
            with np.errstate(all="ignore"):
                pin()
        except Exception as e:
            failed.append((pin.__name__, type(e).__name__))
    assert failed, f"mutant {name} passed every pin"


ORIG_BWD = A.attention_backward_fp64


def _bwd_variant(dq_f=None, dk_f=None, dv_f=None):
    def f(q, k, v, dout, scale, causal=False, key_padding_mask=None, row_block=2048):
        dq, dk, dv = ORIG_BWD(q, k, v, dout, scale, causal, key_padding_mask, row_block)
        return (dq_f(dq, dk, dv) if dq_f else dq, dk_f(dq, dk, dv) if dk_f else dk,
                dv_f(dq, dk, dv) if dv_f else dv)
    return f


BWD_MUTANTS = {
    "softmax_backward_without_rowsum": ("_softmax_backward", lambda P, dP: P * dP),
    "softmax_backward_sign": ("_softmax_backward", lambda P, dP: P * ((P * dP).sum(axis=1, keepdims=True) - dP)),
    "dq_without_scale": ("attention_backward_fp64",
                         _bwd_variant(dq_f=lambda dq, dk, dv: dq * 1.37)),
    "dk_transposed_role": ("attention_backward_fp64",
                           _bwd_variant(dk_f=lambda dq, dk, dv: dk[:, :, ::-1])),
    "dv_off_by_one_key": ("attention_backward_fp64",
                          _bwd_variant(dv_f=lambda dq, dk, dv: np.roll(dv, 1, axis=2))),
}


@pytest.mark.parametrize("name", sorted(BWD_MUTANTS))
def test_backward_mutant_is_caught(name, monkeypatch):
    attr, fn = BWD_MUTANTS[name]
    monkeypatch.setattr(A, attr, fn)
    failed = []
    for pin in PINS:
        try:
            with np.errstate(all="ignore"):
                pin()
        except Exception as e:
            failed.append((pin.__name__, type(e).__name__))
    assert failed, f"mutant {name} passed every pin"


import oracle.fp8 as F8  # noqa: E402

ORIG_DEC = F8.e4m3_to_fp64
ORIG_DEQ = F8.dequantize_heads


def _dec_fields(bias=7, mant_div=8.0, sub_as_normal=False, signed=True):
    def f(bits):
        b = np.asarray(bits, dtype=np.uint8).astype(np.int64)
        s = np.where((b >> 7) & 1, -1.0, 1.0) if signed else 1.0
        e = (b >> 3) & 0xF
        m = (b & 7).astype(np.float64)
        if sub_as_normal:
            mag = (1.0 + m / mant_div) * np.exp2(np.maximum(e, 1) - float(bias))
        else:
            mag = np.where(e == 0, (m / mant_div) * 2.0 ** (1 - bias),
                           (1.0 + m / mant_div) * np.exp2(e - float(bias)))
        return np.where((e == 15) & (m == 7), np.nan, s * mag)
    return f


FP8_MUTANTS = {
    "e4m3_bias_8": ("e4m3_to_fp64", _dec_fields(bias=8)),
    "e4m3_mantissa_quarters": ("e4m3_to_fp64", _dec_fields(mant_div=4.0)),
    "e4m3_subnormals_as_normals": ("e4m3_to_fp64", _dec_fields(sub_as_normal=True)),
    "e4m3_sign_dropped": ("e4m3_to_fp64", _dec_fields(signed=False)),
    "descale_ignored": ("dequantize_heads", lambda bits, ds: ORIG_DEQ(bits, None)),
    "descale_batch_head_swapped": (
        "dequantize_heads",
        lambda bits, ds: ORIG_DEQ(bits, None if ds is None else
                                  np.asarray(ds).T.reshape(np.asarray(ds).shape))),
    "descale_squared": ("dequantize_heads",
                        lambda bits, ds: ORIG_DEQ(bits, None if ds is None else np.asarray(ds) ** 2)),
}


@pytest.mark.parametrize("name", sorted(FP8_MUTANTS))
def test_fp8_mutant_is_caught(name, monkeypatch):
    attr, fn = FP8_MUTANTS[name]
    monkeypatch.setattr(F8, attr, fn)
    failed = []
    for pin in PINS:
        try:
            with np.errstate(all="ignore"):
                pin()
        except Exception as e:
            failed.append((pin.__name__, type(e).__name__))
    assert failed, f"mutant {name} passed every pin"
