"""GPU parity of the 8-bit-float forward (attn_fwd_fp8) against the float64
oracle of attention over E4M3 inputs (oracle.fp8.attention_fp8_fp64).

Tolerance, derived from the kernel's arithmetic.

Scores. The 8-bit matrix instruction does not accumulate its 64 products
exactly in float32: measured on random codes over the whole E4M3 range
(two chained instructions, k = 128), its error stays below 2^-11.1 times the
largest single product |a_k b_k|. With a 2x margin, each score of row i is
off by at most
    Delta_i = (d / 64) 2^-10 |scale dq dk| max_f |q8_if| max_j |k8_jf|.
lse is a smooth maximum of the scores, so |lse - lse_ref| <= Delta_i (+1e-5
for float32 sums), and the exact softmax weights move by a factor of at most
exp(+-2 Delta_i).

Weights. Each weight p_j (taken against a reference max m no larger than the
row's true max M, so the row sum l = sum_j p_j >= 1) is rounded to E4M3
before the value product: |round(p) - p| <= 2^-4 p for p >= 2^-6 and <= 2^-10
below. Hence, for every output element,

    |O - O_ref| <= (2^-4 + 2 Delta_i) (P |V|) + 2^-10 sum_j |v_j| / L + 2^-8 |O_ref|

where P|V| is the exact softmax average of |v| (the oracle on |v| codes), the
sum runs over visible keys, and L = sum_j exp(s_j - M) >= 1 bounds l from
below (l = L exp(M - m)). The last term covers the bf16 rounding of the output
(2^-9) and float32 sums; a 5 % slack on 2^-4 covers second-order terms. The
mean error must also be at most 2^-6 of mean(P|V|): the roundings of
different weights are independent and of zero mean, so their sum falls far
inside the worst case.
"""
import numpy as np
import pytest

from gpu_util import say
from oracle import attention_fp8_fp64, attention_rows_fp64, dequantize_heads
from workloads import HEADLINE, bf16_bits_to_f32, quantize_heads_e4m3, random_case

pytestmark = pytest.mark.gpu

LSE_FLOOR = 1e-5


def score_error_bound(q, k, scale):
    """Delta [B, H, s_q] for dequantized q [B,H,s_q,d], k [B,H,s_k,d] (see the header)."""
    d = q.shape[-1]
    kmax = np.abs(k).max(axis=2, initial=0.0)  # [B, H, d]
    return (d / 64) * 2.0 ** -10 * abs(scale) * (np.abs(q) * kmax[:, :, None, :]).max(axis=-1)


def fp8_case(seed, B, H, s_q, s_k, d, descale_sign=None, **kw):
    c = random_case(seed, B, H, s_q, s_k, d, **kw)
    out = dict(causal=bool(c["causal"]), kpm=c["kpm"], scale=float(c["scale"]))
    for n in ("q", "k", "v"):
        bits, ds = quantize_heads_e4m3(bf16_bits_to_f32(c[n]))
        out[n + "8"], out["d" + n] = bits, ds
    if descale_sign is not None:  # flip the sign of chosen heads' q descale (negates their scores)
        out["dq"] = (out["dq"] * descale_sign).astype(np.float32)
    return out


def run_gpu8(c, with_descale=True):
    import torch

    import exact_attention_44_amd as E
    dev = "cuda:0"
    t = {n: torch.from_numpy(np.ascontiguousarray(c[n + "8"])).to(dev) for n in ("q", "k", "v")}
    ds = {n: (torch.from_numpy(np.ascontiguousarray(c["d" + n])).to(dev) if with_descale else None)
          for n in ("q", "k", "v")}
    kpm = None if c["kpm"] is None else torch.from_numpy(np.ascontiguousarray(c["kpm"])).to(dev)
    out, lse = E.fwd_fp8(t["q"], t["k"], t["v"], descale_q=ds["q"], descale_k=ds["k"],
                         descale_v=ds["v"], causal=c["causal"], key_padding_mask=kpm,
                         scale=c["scale"])
    torch.cuda.synchronize()
    return out.float().cpu().numpy().astype(np.float64), lse.cpu().numpy().astype(np.float64)


def visible(c, B, s_q, s_k):
    vis = np.ones((B, s_q, s_k), bool)
    if c["causal"]:
        vis &= np.tril(np.ones((s_q, s_k), bool))[None]
    if c["kpm"] is not None:
        vis &= (c["kpm"] == 0)[:, None, :]
    return vis


def bound_terms(c):
    """(O_ref, lse_ref, elementwise bound) for a case small enough to hold the scores."""
    O_ref, lse_ref = attention_fp8_fp64(c["q8"], c["k8"], c["v8"], c["dq"], c["dk"], c["dv"],
                                        c["scale"], c["causal"], c["kpm"])
    absv = c["v8"] & np.uint8(0x7F)
    dv_abs = None if c["dv"] is None else np.abs(c["dv"])
    A, _ = attention_fp8_fp64(c["q8"], c["k8"], absv, c["dq"], c["dk"], dv_abs,
                              c["scale"], c["causal"], c["kpm"])
    q = dequantize_heads(c["q8"], c["dq"])
    k = dequantize_heads(c["k8"], c["dk"])
    v = np.abs(dequantize_heads(c["v8"], c["dv"]))
    B, H, s_q, _ = q.shape
    s_k = k.shape[2]
    vis = visible(c, B, s_q, s_k)
    sub = np.zeros_like(O_ref)
    for b in range(B):
        for h in range(H):
            S = c["scale"] * (q[b, h] @ k[b, h].T)
            S[~vis[b]] = -np.inf
            M = S.max(axis=1, initial=-np.inf)
            rows = np.isfinite(M)
            L = np.ones(s_q)
            L[rows] = np.exp(lse_ref[b, h, rows] - M[rows])
            sub[b, h] = (vis[b].astype(np.float64) @ v[b, h]) / L[:, None]
    delta = score_error_bound(q, k, c["scale"])
    bound = (1.05 * 2.0 ** -4 + 2 * delta[..., None]) * A + 2.0 ** -10 * sub \
        + 2.0 ** -8 * np.abs(O_ref)
    return O_ref, lse_ref, bound, A, delta + LSE_FLOOR


def check(O, lse, O_ref, lse_ref, bound, A, lse_bound, what):
    assert O.shape == O_ref.shape and lse.shape == lse_ref.shape
    assert np.all(np.isfinite(O)), f"{what}: non-finite output"
    empty = np.isneginf(lse_ref)
    assert np.array_equal(np.isneginf(lse), empty), f"{what}: -inf lse pattern differs"
    assert np.all(O[empty] == 0.0), f"{what}: rows with no visible key must be zero"
    err = np.abs(O - O_ref)
    ratio = float((err / np.maximum(bound, 1e-30)).max()) if err.size else 0.0
    mean, mean_a = (float(err.mean()), float(A.mean())) if err.size else (0.0, 0.0)
    lerr_all = np.abs(lse[~empty] - lse_ref[~empty])
    lerr = float(lerr_all.max()) if lerr_all.size else 0.0
    lratio = float((lerr_all / lse_bound[~empty]).max()) if lerr_all.size else 0.0
    say(f"  {what}: max|dO|={err.max() if err.size else 0:.3e} max err/bound={ratio:.3f} "
        f"mean|dO|={mean:.3e} (mean P|V| {mean_a:.3e}) max|dlse|={lerr:.3e} "
        f"(max dlse/bound {lratio:.3f})")
    assert ratio <= 1.0, f"{what}: error exceeds the derived bound (ratio {ratio})"
    assert mean <= 2.0 ** -6 * mean_a + 1e-7, f"{what}: mean|dO| {mean} > 2^-6 mean(P|V|)"
    assert lratio <= 1.0, f"{what}: lse error exceeds its bound (ratio {lratio})"


EDGE_CASES = {
    # name: (seed, B, H, s_q, s_k, d, kwargs)
    "single": (101, 1, 1, 1, 1, 64, {}),
    "ragged_causal_sq_lt_sk": (102, 2, 3, 300, 517, 128, dict(causal=True)),
    "ragged_causal_d64": (103, 1, 2, 777, 777, 64, dict(causal=True)),
    "random_mask": (104, 2, 2, 129, 1000, 64, dict(mask="random")),
    "random_mask_causal_d128": (105, 2, 2, 260, 333, 128, dict(mask="random", causal=True)),
    "causal_sq_gt_sk": (106, 3, 1, 200, 70, 128, dict(causal=True)),
    "lengths_incl_zero": (107, 4, 2, 96, 160, 128, dict(mask="lengths")),
    "all_padded": (108, 2, 1, 64, 100, 64, dict(mask="all")),
    "negative_scale": (109, 1, 2, 256, 256, 128, dict(scale=-0.09)),
    "zero_scale_causal": (110, 1, 2, 130, 300, 64, dict(scale=0.0, causal=True)),
    "large_scores_q30": (111, 1, 2, 300, 600, 128, dict(q_mult=30.0, causal=True)),
    "large_scores_padded": (112, 2, 1, 140, 700, 64, dict(q_mult=20.0, mask="random")),
    "causal_padded": (113, 2, 2, 513, 513, 128, dict(causal=True, mask="lengths")),
    "full_tiles": (114, 1, 1, 512, 512, 128, dict(causal=True)),
    "many_heads_tiny": (115, 4, 8, 33, 33, 64, {}),
    "one_key": (116, 1, 2, 70, 1, 128, {}),
    "long_keys_few_queries": (117, 1, 1, 3, 2500, 128, {}),
    "long_rows_d128": (118, 1, 2, 256, 4096, 128, dict(causal=True)),
    # d = 64 runs a persistent grid: more items than CUs, each head with its
    # own descales, a partial last round
    "rounds_causal_d64": (119, 3, 37, 600, 600, 64, dict(causal=True)),
    "rounds_lengths_d64": (120, 6, 16, 700, 650, 64, dict(mask="lengths")),
    # whole 64-key tiles of padding inside the sequence: those tiles are not walked
    "interior_padding_causal_d128": (121, 2, 2, 700, 3000, 128, dict(mask="blocks", causal=True)),
    "interior_padding_rounds_d64": (122, 4, 24, 520, 2100, 64, dict(mask="blocks")),
    # left padding: the visible tiles are one range that starts past key 0
    "prefix_padding_causal_d128": (124, 2, 2, 900, 2000, 128, dict(mask="prefix", causal=True)),
    "prefix_padding_rounds_d64": (125, 4, 24, 520, 1500, 64, dict(mask="prefix")),
    "interior_padding_beyond_list": (123, 1, 1, 20, 4096 * 64 + 900, 64, dict(mask="blocks")),
}


@pytest.mark.parametrize("name", list(EDGE_CASES))
def test_fp8_edge_and_ragged(name):
    seed, B, H, s_q, s_k, d, kw = EDGE_CASES[name]
    say(f"case fp8 {name}: B={B} H={H} s_q={s_q} s_k={s_k} d={d} {kw}")
    c = fp8_case(seed, B, H, s_q, s_k, d, **kw)
    O, lse = run_gpu8(c)
    check(O, lse, *bound_terms(c), name)


def test_fp8_negative_descale_heads():
    say("case fp8 negative descale on some heads")
    sign = np.array([[1.0, -1.0, 1.0], [-1.0, 1.0, -1.0]], np.float32)
    c = fp8_case(121, 2, 3, 200, 300, 128, descale_sign=sign, causal=True)
    O, lse = run_gpu8(c)
    check(O, lse, *bound_terms(c), "negative_descale")


def test_fp8_without_descale_arrays():
    say("case fp8 descale arrays omitted (all factors 1)")
    c = fp8_case(122, 1, 2, 150, 180, 64)
    c = dict(c, scale=c["scale"] * 1e-3)  # raw codes reach 448: keep scores moderate
    O, lse = run_gpu8(c, with_descale=False)
    ones = {n: None for n in ("dq", "dk", "dv")}
    check(O, lse, *bound_terms(dict(c, **ones)), "no_descale")


def test_fp8_no_keys_and_empty():
    import torch

    import exact_attention_44_amd as E
    say("case fp8 no keys / empty batch")
    q = torch.randint(0, 0x70, (2, 2, 100, 128), dtype=torch.uint8, device="cuda:0")
    k = torch.empty(2, 2, 0, 128, dtype=torch.uint8, device="cuda:0")
    out, lse = E.fwd_fp8(q, k, k, causal=True)
    torch.cuda.synchronize()
    assert torch.all(out == 0) and torch.all(torch.isneginf(lse))
    z = torch.empty(0, 2, 5, 64, dtype=torch.float8_e4m3fn, device="cuda:0")
    out, lse = E.fwd_fp8(z, z, z)
    assert out.shape == (0, 2, 5, 64)


def test_fp8_deterministic():
    say("case fp8 determinism")
    c = fp8_case(123, 1, 4, 700, 700, 128, causal=True)
    O1, l1 = run_gpu8(c)
    O2, l2 = run_gpu8(c)
    assert np.array_equal(O1, O2) and np.array_equal(l1, l2)


def test_fp8_headline_workload_sampled_rows():
    """The s=8192 causal workload (all 32 heads, the launch the benchmark times),
    checked on seeded rows of every head against the oracle row by row."""
    from workloads import generate
    w = HEADLINE
    say(f"case fp8 workload {w.name}: all heads, sampled rows")
    g = generate(w)
    c = dict(causal=w.causal, kpm=g["kpm"], scale=float(g["scale"]))
    for n in ("q", "k", "v"):
        bits, ds = quantize_heads_e4m3(bf16_bits_to_f32(g[n]))
        c[n + "8"], c["d" + n] = bits, ds
    O, lse = run_gpu8(c)
    rng = np.random.default_rng(4601)
    rows = np.unique(np.concatenate([[0, 1, 255, 256, w.s_q - 1], rng.integers(0, w.s_q, 14)]))
    picks = [(0, h, rows) for h in range(w.H)]
    q = dequantize_heads(c["q8"], c["dq"])
    k = dequantize_heads(c["k8"], c["dk"])
    v = dequantize_heads(c["v8"], c["dv"])
    res = attention_rows_fp64(q, k, v, c["scale"], w.causal, c["kpm"], picks)
    resA = attention_rows_fp64(q, k, np.abs(v), c["scale"], w.causal, c["kpm"], picks)
    delta = score_error_bound(q[:, :, rows], k, c["scale"])  # [B, H, len(rows)]
    worst = 0.0
    for (b, h, r), (o_ref, l_ref), (a, _) in zip(picks, res, resA):
        err = np.abs(O[b, h, r] - o_ref)
        # rows of this workload have >= 1 visible key and L >= 1; sum_j |v_j| / L is bounded
        # by the row count of visible keys times max|v| over L, computed from the scores
        S = c["scale"] * (q[b, h, r] @ k[b, h].T)
        vis = np.arange(w.s_k)[None, :] <= r[:, None]
        S[~vis] = -np.inf
        M = S.max(axis=1)
        L = np.exp(l_ref - M)
        sub = (vis.astype(np.float64) @ np.abs(v[b, h])) / L[:, None]
        dl = delta[b, h][:, None]
        bound = (1.05 * 2.0 ** -4 + 2 * dl) * a + 2.0 ** -10 * sub + 2.0 ** -8 * np.abs(o_ref)
        worst = max(worst, float((err / bound).max()))
        assert np.all(err <= bound), (h, float((err / bound).max()))
        assert np.all(np.abs(lse[b, h, r] - l_ref) <= delta[b, h] + LSE_FLOOR)
    say(f"  workload rows: max err/bound={worst:.3f}")


def test_fp8_no_device_allocation_and_side_stream():
    """With out and lse given, the FP8 forward allocates nothing and runs on
    whatever stream is current, with the same result as on the default stream."""
    import torch

    import exact_attention_44_amd as E
    say("case fp8 allocation + side stream")
    c = fp8_case(124, 1, 4, 600, 600, 128, causal=True)
    dev = "cuda:0"
    t = {n: torch.from_numpy(np.ascontiguousarray(c[n + "8"])).to(dev) for n in ("q", "k", "v")}
    ds = {n: torch.from_numpy(np.ascontiguousarray(c["d" + n])).to(dev) for n in ("q", "k", "v")}

    def call(**kw):
        return E.fwd_fp8(t["q"], t["k"], t["v"], descale_q=ds["q"], descale_k=ds["k"],
                         descale_v=ds["v"], causal=True, scale=c["scale"], **kw)

    ref_o, ref_l = call()
    torch.cuda.synchronize()
    out, lse = torch.empty_like(ref_o), torch.empty_like(ref_l)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        call(out=out, lse=lse)
    side.synchronize()
    out.zero_()
    torch.cuda.synchronize()
    free0, _ = torch.cuda.mem_get_info()
    torch.cuda.reset_peak_memory_stats()
    a0 = torch.cuda.memory_allocated()
    with torch.cuda.stream(side):
        call(out=out, lse=lse)
    side.synchronize()
    free1, _ = torch.cuda.mem_get_info()
    assert torch.cuda.max_memory_allocated() - a0 == 0
    assert free0 == free1, (free0, free1)
    assert torch.equal(out, ref_o) and torch.equal(lse, ref_l)
