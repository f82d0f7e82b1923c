"""Pins for the CPU oracle: checks against things other than the oracle itself.

Each pin is a plain function that raises AssertionError when the oracle is
wrong. test_oracle_pins.py runs them; test_oracle_mutants.py plants plausible
mistakes in the oracle's steps and shows every mistake trips at least one pin.

What the pins stand on:
  * the numbers the onecalc.app "Attention memory" page prints in its
    "Worked example" (tests/golden/attention_memory_worked_example.json);
  * the mathematics of softmax (rows sum to one, hidden keys weigh exactly
    zero, closed forms for zero keys, one key and two keys, invariances);
  * the block-wise walk with running statistics (the page's "FlashAttention"
    section), implemented separately in the oracle, which must reach the same
    result (the glossary entry "Flash attention" states the results agree);
  * pure-Python brute force and a high-precision Decimal evaluation;
  * torch's CPU scaled_dot_product_attention and logsumexp in float64;
  * for the 8-bit-float inputs: torch's float8_e4m3fn dtype and the field
    layout of the OCP E4M3 format (closed-form code values), plus the scaling
    identities of per-head descale factors.
"""
from __future__ import annotations

import json
import math
import os
from decimal import Decimal, getcontext

import numpy as np
import torch

import oracle.attention as A
import oracle.fp8 as F8
from workloads import WORKLOADS, bf16_bits_to_f32, generate, quantize_heads_e4m3, random_case

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def f64_case(seed, B, H, s_q, s_k, d, **kw):
    c = random_case(seed, B, H, s_q, s_k, d, **kw)
    for n in ("q", "k", "v"):
        c[n] = bf16_bits_to_f32(c[n]).astype(np.float64)
    c["scale"] = float(c["scale"])
    return c


def visible(c):
    """Boolean [B, s_q, s_k]: key j visible to query i in batch item b."""
    B, _, s_q, _ = c["q"].shape
    s_k = c["k"].shape[2]
    vis = np.ones((B, s_q, s_k), bool)
    if c["causal"]:
        vis &= np.tril(np.ones((s_q, s_k), bool))[None]
    if c["kpm"] is not None:
        vis &= (c["kpm"] == 0)[:, None, :]
    return vis


def run(c, fn=None, **kw):
    fn = fn or A.attention_fp64
    return fn(c["q"], c["k"], c["v"], c["scale"], c["causal"], c["kpm"], **kw)


def close(a, b, tol, what):
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    assert a.shape == b.shape, f"{what}: shape {a.shape} != {b.shape}"
    ninf_a, ninf_b = np.isneginf(a), np.isneginf(b)
    assert np.array_equal(ninf_a, ninf_b), f"{what}: -inf pattern differs"
    fa, fb = a[~ninf_a], b[~ninf_b]
    assert np.all(np.isfinite(fa)), f"{what}: non-finite values"
    if fa.size:
        err = np.max(np.abs(fa - fb) / np.maximum(1.0, np.abs(fb)))
        assert err <= tol, f"{what}: max rel err {err:.3e} > {tol:.1e}"


# ---------------------------------------------------------------- the page's numbers
def pin_worked_example():
    """onecalc.app "Attention memory", "Worked example": 1.07 GB and 4.29 GB."""
    with open(os.path.join(GOLDEN, "attention_memory_worked_example.json")) as f:
        g = json.load(f)
    sizes = []
    for case in g["cases"]:
        gb = A.score_matrix_gb(case["B"], case["H"], case["s"], case["e"])
        assert round(gb, 2) == case["gb_printed"], (case, gb)
        sizes.append(A.score_matrix_bytes(case["B"], case["H"], case["s"], case["e"]))
    assert sizes[1] == g["ratio_when_s_doubles"] * sizes[0]


def pin_oracle_materialises_closed_form():
    """The score block the oracle builds per (b, h) is s_q x s_k float64, i.e.
    score_matrix_bytes(1, 1, s, 8) for a square problem (the quantity the tiled
    kernel must never allocate)."""
    c = f64_case(11, 1, 2, 48, 48, 16, causal=True)
    seen = []
    orig = A._scores

    def spy(q_rows, k_head, scale):
        S = orig(q_rows, k_head, scale)
        seen.append(S.nbytes)
        return S

    A._scores = spy
    try:
        run(c, row_block=4096)
    finally:
        A._scores = orig
    assert seen == [A.score_matrix_bytes(1, 1, 48, 8)] * 2, seen


# ---------------------------------------------------------------- softmax structure
def pin_row_sums_and_masked_zero():
    for c in (f64_case(21, 2, 2, 20, 26, 8, causal=True, mask="random"),
              f64_case(22, 2, 1, 17, 17, 8, mask="lengths"),
              f64_case(23, 1, 2, 9, 30, 4, causal=True)):
        P = A.attention_weights_fp64(c["q"], c["k"], c["scale"], c["causal"], c["kpm"])
        vis = visible(c)[:, None, :, :].repeat(P.shape[1], axis=1)
        assert np.all(P[~vis] == 0.0), "a hidden key has nonzero weight"
        assert np.all(P[vis] > 0.0), "a visible key has zero weight"
        rows_any = vis.any(axis=-1)
        sums = P.sum(axis=-1)
        assert np.all(np.abs(sums[rows_any] - 1.0) <= 1e-12), "a row does not sum to 1"
        assert np.all(sums[~rows_any] == 0.0)


def pin_online_equals_definition():
    """The block-wise walk (running max/sum, rescale) equals the definition."""
    cases = [f64_case(31, 2, 2, 23, 23, 8, causal=True, mask="lengths"),
             f64_case(32, 1, 2, 19, 27, 8, mask="random"),
             f64_case(33, 1, 1, 29, 13, 4, causal=True),
             f64_case(34, 2, 1, 7, 40, 16, causal=True, mask="random")]
    for c in cases:
        O, lse = run(c)
        s_k = c["k"].shape[2]
        for blk in (1, 3, 16, s_k, s_k + 5):
            O2, lse2 = run(c, A.attention_online_fp64, block=blk)
            close(O, O2, 1e-12, f"O block={blk}")
            close(lse, lse2, 1e-12, f"lse block={blk}")


def pin_bruteforce():
    for c in (f64_case(41, 1, 2, 7, 9, 5, causal=True, mask="random"),
              f64_case(42, 2, 1, 12, 12, 8, mask="lengths"),
              f64_case(43, 1, 1, 6, 3, 4, causal=True),
              f64_case(44, 1, 1, 3, 11, 6, causal=True, mask="random")):
        O, lse = run(c)
        O2, lse2 = run(c, A.attention_bruteforce)
        close(O, O2, 1e-12, "O vs brute force")
        close(lse, lse2, 1e-12, "lse vs brute force")


def _torch_reference(c):
    q, k, v = (torch.from_numpy(c[n]) for n in ("q", "k", "v"))
    vis = torch.from_numpy(visible(c))[:, None]          # [B,1,s_q,s_k]
    O = torch.nn.functional.scaled_dot_product_attention(q, k, v, attn_mask=vis, scale=c["scale"])
    S = (q @ k.transpose(-1, -2)) * c["scale"]
    S = S.masked_fill(~vis, float("-inf"))
    lse = torch.logsumexp(S, dim=-1)
    return O.numpy(), lse.numpy()


def pin_torch_sdpa():
    w = WORKLOADS[0]
    g = generate(w)
    c0 = dict(q=bf16_bits_to_f32(g["q"]).astype(np.float64),
              k=bf16_bits_to_f32(g["k"]).astype(np.float64),
              v=bf16_bits_to_f32(g["v"]).astype(np.float64),
              scale=float(g["scale"]), causal=g["causal"], kpm=g["kpm"])
    cases = [c0,
             f64_case(51, 2, 3, 33, 33, 16, causal=True),
             f64_case(52, 3, 2, 40, 40, 8, mask="lengths"),
             f64_case(53, 1, 2, 24, 37, 8, causal=True, mask="random")]
    for c in cases:
        O, lse = run(c)
        O2, lse2 = _torch_reference(c)
        close(O, O2, 1e-12, "O vs torch sdpa")
        close(lse, lse2, 1e-12, "lse vs torch logsumexp")
    # torch's own causal flag (top-left for square problems)
    c = f64_case(54, 1, 2, 31, 31, 8, causal=True)
    O = run(c)[0]
    q, k, v = (torch.from_numpy(c[n]) for n in ("q", "k", "v"))
    O2 = torch.nn.functional.scaled_dot_product_attention(q, k, v, is_causal=True, scale=c["scale"])
    close(O, O2.numpy(), 1e-12, "O vs torch is_causal")


# ---------------------------------------------------------------- closed forms
def pin_zero_keys_mean_of_values():
    """K == 0: all scores 0, so O_i is the plain mean of the visible value rows
    and lse_i = ln(number of visible keys)."""
    for c in (f64_case(61, 2, 2, 21, 21, 8, causal=True, mask="lengths"),
              f64_case(62, 1, 1, 15, 22, 4, mask="random"),
              f64_case(63, 1, 2, 18, 18, 8, causal=True)):
        c["k"] = np.zeros_like(c["k"])
        O, lse = run(c)
        vis = visible(c).astype(np.float64)             # [B, s_q, s_k]
        cnt = vis.sum(-1)                               # [B, s_q]
        for b in range(O.shape[0]):
            for h in range(O.shape[1]):
                tot = vis[b] @ c["v"][b, h]             # sums of visible rows
                with np.errstate(invalid="ignore", divide="ignore"):
                    mean = np.where(cnt[b][:, None] > 0, tot / np.maximum(cnt[b][:, None], 1), 0.0)
                    want_lse = np.where(cnt[b] > 0, np.log(np.maximum(cnt[b], 1)), -np.inf)
                close(O[b, h], mean, 1e-12, "zero-key mean")
                close(lse[b, h], want_lse, 1e-12, "zero-key lse")
        if c["causal"] and c["kpm"] is None:
            # prefix mean via cumulative sums
            pref = np.cumsum(c["v"], axis=2) / np.arange(1, c["v"].shape[2] + 1)[None, None, :, None]
            close(O, pref, 1e-12, "causal prefix mean")


def pin_causal_first_row_and_single_key():
    c = f64_case(71, 2, 2, 12, 12, 8, causal=True)
    O, lse = run(c)
    close(O[:, :, 0], c["v"][:, :, 0], 1e-15, "causal row 0 = V_0")
    s00 = c["scale"] * np.einsum("bhd,bhd->bh", c["q"][:, :, 0], c["k"][:, :, 0])
    close(lse[:, :, 0], s00, 1e-12, "causal lse_0 = S_00")
    c = f64_case(72, 2, 2, 9, 1, 8)
    O, lse = run(c)
    close(O, np.repeat(c["v"][:, :, :1], 9, axis=2), 1e-15, "one key: O = V_0")
    s = c["scale"] * np.einsum("bhid,bhd->bhi", c["q"], c["k"][:, :, 0])
    close(lse, s, 1e-12, "one key: lse = S_i0")


def pin_two_keys_logistic():
    """Two keys: weight of key 0 is the logistic function of s_0 - s_1."""
    c = f64_case(81, 1, 3, 10, 2, 8, q_mult=3.0)
    O, lse = run(c)
    s = c["scale"] * np.einsum("bhid,bhjd->bhij", c["q"], c["k"])
    w0 = 1.0 / (1.0 + np.exp(-(s[..., 0] - s[..., 1])))
    want = w0[..., None] * c["v"][:, :, 0][:, :, None] + (1 - w0[..., None]) * c["v"][:, :, 1][:, :, None]
    close(O, want, 1e-12, "two-key logistic")
    close(lse, np.logaddexp(s[..., 0], s[..., 1]), 1e-12, "two-key lse")


# ---------------------------------------------------------------- invariances
def pin_invariances():
    c = f64_case(91, 1, 2, 14, 19, 8)
    O, lse = run(c)
    perm = np.random.default_rng(5).permutation(19)
    cp = dict(c, k=c["k"][:, :, perm], v=c["v"][:, :, perm])
    O2, lse2 = run(cp)
    close(O, O2, 1e-12, "key permutation O")
    close(lse, lse2, 1e-12, "key permutation lse")
    # linear in V
    c2 = f64_case(92, 1, 2, 14, 19, 8, causal=True, mask="random")
    v1, v2 = c2["v"], f64_case(93, 1, 2, 14, 19, 8)["v"]
    Oa = run(dict(c2, v=v1))[0]
    Ob = run(dict(c2, v=v2))[0]
    Oc = run(dict(c2, v=2.0 * v1 - 0.5 * v2))[0]
    close(Oc, 2.0 * Oa - 0.5 * Ob, 1e-12, "linear in V")
    # scaling Q by 2 equals doubling scale
    Oq, lq = run(dict(c2, q=2.0 * c2["q"]))
    Os, ls = run(dict(c2, scale=2.0 * c2["scale"]))
    close(Oq, Os, 1e-12, "Q*2 == scale*2 (O)")
    close(lq, ls, 1e-12, "Q*2 == scale*2 (lse)")


# ---------------------------------------------------------------- range safety
def _decimal_row(q_row, k_head, v_head, scale, vis_row):
    getcontext().prec = 60
    sc = []
    for j in range(k_head.shape[0]):
        if vis_row[j]:
            dot = math.fsum(float(a) * float(b) for a, b in zip(q_row, k_head[j]))
            sc.append((j, Decimal(scale) * Decimal(dot)))
    if not sc:
        return None, -math.inf
    e = [(j, s.exp()) for j, s in sc]
    tot = sum(x for _, x in e)
    out = [float(sum(x * Decimal(float(v_head[j, cc])) for j, x in e) / tot)
           for cc in range(v_head.shape[1])]
    return np.array(out), float(tot.ln())


def pin_large_scores():
    """Scores of order +-1000 (Q x 1000): exp without the max shift would
    overflow; the result must still match a 60-digit Decimal evaluation."""
    c = f64_case(101, 1, 2, 6, 7, 8, q_mult=1000.0, causal=True, mask="random")
    O, lse = run(c)
    vis = visible(c)
    for h in range(2):
        for i in range(6):
            o, l = _decimal_row(c["q"][0, h, i], c["k"][0, h], c["v"][0, h], c["scale"], vis[0, i])
            if o is None:
                assert np.all(O[0, h, i] == 0) and np.isneginf(lse[0, h, i])
            else:
                close(O[0, h, i], o, 1e-12, "large-score O")
                close(lse[0, h, i], l, 1e-12, "large-score lse")
    assert np.nanmax(np.abs(c["scale"] * np.einsum("hid,hjd->hij", c["q"][0], c["k"][0]))) > 710


def pin_fully_masked_rows():
    c = f64_case(111, 2, 2, 5, 6, 4, mask="all")
    O, lse = run(c)
    assert np.all(O == 0.0) and np.all(np.isneginf(lse))
    c = f64_case(112, 1, 1, 4, 4, 4, causal=True)
    c["kpm"] = np.array([[1, 0, 0, 0]], np.uint8)      # row 0 sees only key 0, which is padded
    O, lse = run(c)
    assert np.all(O[0, 0, 0] == 0.0) and np.isneginf(lse[0, 0, 0])
    close(O[0, 0, 1], c["v"][0, 0, 1], 1e-15, "row 1 sees only key 1")
    c = f64_case(113, 1, 2, 3, 0, 4)
    O, lse = run(c)
    assert O.shape == (1, 2, 3, 4) and np.all(O == 0.0) and np.all(np.isneginf(lse))


def chunk_partials(c, bounds):
    """The oracle on each key chunk [lo, hi) alone (keys outside it padded)."""
    B, s_k = c["q"].shape[0], c["k"].shape[2]
    outs, lses = [], []
    for lo, hi in bounds:
        outside = np.ones(s_k, bool)
        outside[lo:hi] = False
        kpm = np.broadcast_to(outside, (B, s_k)).astype(np.uint8)
        if c["kpm"] is not None:
            kpm = kpm | c["kpm"]
        O, lse = A.attention_fp64(c["q"], c["k"], c["v"], c["scale"], c["causal"], kpm)
        outs.append(O)
        lses.append(lse)
    return np.stack(outs), np.stack(lses)


def pin_merge_of_key_chunks():
    """Merging the definition's results over key chunks gives the definition
    over all keys (softmax over a union of disjoint key sets), for chunkings
    with empty chunks, single keys, and chunks some rows see nothing of."""
    for seed, causal, mask in ((121, False, "none"), (122, True, "none"), (123, True, "lengths"),
                               (124, False, "random"), (125, True, "all")):
        c = f64_case(seed, 2, 2, 23, 37, 8, causal=causal, mask=mask)
        O, lse = run(c)
        for bounds in ([(0, 37)], [(0, 10), (10, 37)], [(0, 5), (5, 6), (6, 30), (30, 37)],
                       [(0, 0), (0, 37), (37, 37)]):
            outs, lses = chunk_partials(c, bounds)
            Om, lm = A.merge_partials_fp64(outs, lses)
            close(Om, O, 1e-13, f"merged O seed={seed} chunks={bounds}")
            close(lm, lse, 1e-13, f"merged lse seed={seed} chunks={bounds}")
    # closed forms: two parts with equal lse average, and the lse gains ln 2;
    # a part with lse -inf has no weight
    o1, o2 = np.array([[1.0, -2.0]]), np.array([[3.0, 4.0]])
    Om, lm = A.merge_partials_fp64(np.stack([o1, o2]), np.array([[0.7], [0.7]]))
    close(Om, (o1 + o2) / 2, 1e-15, "equal halves")
    close(lm, np.array([0.7 + np.log(2.0)]), 1e-15, "equal halves lse")
    Om, lm = A.merge_partials_fp64(np.stack([o1, o2]), np.array([[-np.inf], [1.5]]))
    close(Om, o2, 1e-15, "empty part")
    close(lm, np.array([1.5]), 1e-15, "empty part lse")


# ---------------------------------------------------------------- the backward pass


def _grad_case(seed, B, H, s_q, s_k, d, **kw):
    c = f64_case(seed, B, H, s_q, s_k, d, **kw)
    c["dout"] = np.random.default_rng(seed + 1000).standard_normal(c["q"].shape)
    return c


def run_bwd(c, **kw):
    return A.attention_backward_fp64(c["q"], c["k"], c["v"], c["dout"], c["scale"], c["causal"],
                                     c["kpm"], **kw)


def pin_backward_torch_autograd():
    """torch's scaled_dot_product_attention differentiated by autograd in
    float64 on the CPU (rows with a visible key only: torch's softmax over an
    all -inf row is not defined)."""
    torch = __import__("torch")
    F = torch.nn.functional
    for seed, causal, mask in ((131, True, "none"), (132, False, "lengths"), (133, True, "random")):
        c = _grad_case(seed, 2, 3, 13, 17, 16, causal=causal, mask=mask)
        vis = visible(c)
        if mask != "none":  # keep every row non-empty for torch
            vis[:, :, 0] = True
            c["kpm"][:, 0] = 0
        q, k, v = (torch.tensor(c[n], requires_grad=True) for n in ("q", "k", "v"))
        attn_mask = torch.tensor(vis)[:, None]
        o = F.scaled_dot_product_attention(q, k, v, attn_mask=attn_mask, scale=c["scale"])
        o.backward(torch.tensor(c["dout"]))
        dq, dk, dv = run_bwd(c)
        close(dq, q.grad.numpy(), 1e-12, f"dq seed={seed}")
        close(dk, k.grad.numpy(), 1e-12, f"dk seed={seed}")
        close(dv, v.grad.numpy(), 1e-12, f"dv seed={seed}")


def pin_backward_finite_differences():
    """Central differences of L = sum(dout * O) through the forward
    definition, for every input element of a tiny problem."""
    c = _grad_case(134, 1, 1, 4, 5, 3, causal=True, mask="random")
    c["kpm"][0, 0] = 0
    dq, dk, dv = run_bwd(c)
    eps = 1e-6

    def loss():
        O, _ = run(c)
        return float((c["dout"] * O).sum())

    for name, grad in (("q", dq), ("k", dk), ("v", dv)):
        x = c[name]
        num = np.zeros_like(x)
        for idx in np.ndindex(x.shape):
            keep = x[idx]
            x[idx] = keep + eps
            lp = loss()
            x[idx] = keep - eps
            lm = loss()
            x[idx] = keep
            num[idx] = (lp - lm) / (2 * eps)
        close(grad, num, 1e-7, f"d{name} vs finite differences")


def pin_backward_identities():
    """Each softmax row's gradient sums to zero over its keys, so the key
    gradients of a (b, h) sum to zero and the query gradient does not change
    when one vector is added to every key; padded keys get no gradient; with
    one visible key the value gradient is the sum of the output gradients."""
    c = _grad_case(135, 2, 2, 11, 9, 8, causal=True, mask="lengths")
    c["kpm"][:, 0] = 0
    dq, dk, dv = run_bwd(c)
    close(dk.sum(axis=2), np.zeros((2, 2, 8)), 1e-12, "sum_j dk_j")
    pad = c["kpm"] != 0
    for b in range(2):
        assert np.all(dk[b][:, pad[b]] == 0.0) and np.all(dv[b][:, pad[b]] == 0.0)
    shifted = dict(c)
    shifted["k"] = c["k"] + np.random.default_rng(7).standard_normal(8)[None, None, None, :]
    dq2, _, _ = run_bwd(shifted)
    close(dq2, dq, 1e-11, "dq under a common key shift")
    one = _grad_case(136, 1, 2, 6, 1, 4)
    _, _, dv1 = run_bwd(one)
    close(dv1[:, :, 0], one["dout"].sum(axis=2), 1e-14, "one key: dv = sum of dout")


def pin_e4m3_decode_against_torch():
    """Every one of the 256 E4M3 codes decodes to the value torch's float8_e4m3fn
    dtype (the OCP E4M3 format) widens to, sign of zero and NaN codes included."""
    codes = np.arange(256, dtype=np.uint8)
    ref = torch.from_numpy(codes.copy()).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    got = F8.e4m3_to_fp64(codes)
    nan = np.isnan(ref)
    assert nan.sum() == 2 and np.array_equal(np.isnan(got), nan), "NaN codes differ"
    assert np.array_equal(got[~nan], ref[~nan]), "decoded values differ from torch"
    assert np.array_equal(np.signbit(got[~nan]), np.signbit(ref[~nan])), "signs differ"


def pin_e4m3_decode_closed_forms():
    """Code values that follow from the field layout (bias 7, 3 mantissa bits,
    subnormal step 2^-9, largest finite 448), monotonicity and sign symmetry."""
    table = {0x00: 0.0, 0x01: 2.0 ** -9, 0x04: 0.5 * 2.0 ** -6, 0x07: 7 * 2.0 ** -9,
             0x08: 2.0 ** -6, 0x0F: 1.875 * 2.0 ** -6, 0x30: 0.5, 0x38: 1.0, 0x39: 1.125,
             0x3F: 1.875, 0x40: 2.0, 0x55: 1.625 * 2.0 ** 3, 0x77: 1.875 * 2.0 ** 7,
             0x78: 256.0, 0x7E: 448.0, 0x80: -0.0, 0xB8: -1.0, 0xFE: -448.0}
    for c, want in table.items():
        got = float(F8.e4m3_to_fp64(np.array([c], np.uint8))[0])
        assert got == want and math.copysign(1, got) == math.copysign(1, want), (hex(c), got, want)
    assert np.isnan(F8.e4m3_to_fp64(np.array([0x7F, 0xFF], np.uint8))).all()
    pos = F8.e4m3_to_fp64(np.arange(0x7F, dtype=np.uint8))
    assert np.all(np.diff(pos) > 0), "positive codes must increase"
    neg = F8.e4m3_to_fp64(np.arange(0x80, 0xFF, dtype=np.uint8))
    assert np.array_equal(neg, -pos), "negative codes mirror positive ones"


def _fp8_case(seed, B, H, s_q, s_k, d, **kw):
    c = random_case(seed, B, H, s_q, s_k, d, **kw)
    out = dict(causal=c["causal"], kpm=c["kpm"], scale=float(c["scale"]))
    for n in ("q", "k", "v"):
        x = bf16_bits_to_f32(c[n])
        bits, ds = quantize_heads_e4m3(x)
        out[n + "8"], out["d" + n] = bits, ds
    return out


def run_fp8(c, **kw):
    return F8.attention_fp8_fp64(c["q8"], c["k8"], c["v8"], c["dq"], c["dk"], c["dv"],
                                 c["scale"], c["causal"], c["kpm"], **kw)


def pin_fp8_attention_on_library_values():
    """The FP8 oracle is the definition on descale * value: values widened by
    torch's float8_e4m3fn and scaled per (b, h) here give the same result."""
    for seed, causal, mask in ((4501, False, "none"), (4502, True, "lengths"), (4503, False, "random")):
        c = _fp8_case(seed, 2, 3, 37, 53, 16, causal=causal, mask=mask)
        vals = {}
        for n in ("q", "k", "v"):
            t = torch.from_numpy(c[n + "8"].copy()).view(torch.float8_e4m3fn).to(torch.float64).numpy()
            ds = c["d" + n].astype(np.float64)
            vals[n] = t * ds[:, :, None, None]
        assert len(np.unique(c["dq"])) == 6, "per-head descales must differ for this pin"
        O_ref, lse_ref = A.attention_fp64(vals["q"], vals["k"], vals["v"], c["scale"], causal, c["kpm"])
        O, lse = run_fp8(c)
        close(O, O_ref, 1e-13, "fp8 O vs definition on library-decoded values")
        fin = np.isfinite(lse_ref)
        assert np.array_equal(np.isfinite(lse), fin)
        close(lse[fin], lse_ref[fin], 1e-13, "fp8 lse vs definition")


def pin_fp8_descale_identities():
    """Doubling descale_v doubles O and leaves lse; doubling descale_q is the same
    as doubling the scale; changing one head's descale_k changes only that head."""
    c = _fp8_case(4504, 2, 2, 29, 41, 16, causal=True)
    O, lse = run_fp8(c)
    c2 = dict(c, dv=c["dv"] * np.float32(2))
    O2, lse2 = run_fp8(c2)
    close(O2, 2 * O, 1e-13, "descale_v doubled")
    close(lse2, lse, 1e-13, "lse independent of descale_v")
    c3 = dict(c, dq=c["dq"] * np.float32(2))
    O3, lse3 = run_fp8(c3)
    O4, lse4 = run_fp8(dict(c, scale=2 * c["scale"]))
    close(O3, O4, 1e-13, "descale_q doubled vs scale doubled")
    close(lse3, lse4, 1e-13, "lse: descale_q doubled vs scale doubled")
    dk = c["dk"].copy()
    dk[1, 0] *= np.float32(3)
    O5, _ = run_fp8(dict(c, dk=dk))
    changed = np.abs(O5 - O).max(axis=(2, 3)) > 1e-9
    assert changed.tolist() == [[False, False], [True, False]], changed


PINS = [
    pin_worked_example,
    pin_oracle_materialises_closed_form,
    pin_row_sums_and_masked_zero,
    pin_online_equals_definition,
    pin_bruteforce,
    pin_torch_sdpa,
    pin_zero_keys_mean_of_values,
    pin_causal_first_row_and_single_key,
    pin_two_keys_logistic,
    pin_invariances,
    pin_large_scores,
    pin_fully_masked_rows,
    pin_merge_of_key_chunks,
    pin_backward_torch_autograd,
    pin_backward_finite_differences,
    pin_backward_identities,
    pin_e4m3_decode_against_torch,
    pin_e4m3_decode_closed_forms,
    pin_fp8_attention_on_library_values,
    pin_fp8_descale_identities,
]
