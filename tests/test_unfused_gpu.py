"""GPU parity of the unfused (materialising) forward, attn_fwd_unfused, against
the float64 oracle, to the bound derived from its bf16 score matrix
(tests/unfused_bound.py); on the workloads also to the bf16 bar on the mean
error. The materialised buffer is checked too: it holds the softmax weights,
exactly 0 where a key is hidden, and it is exactly B*H*s_q*s_k*2 bytes."""
import numpy as np
import pytest

from gpu_util import O_MEAN_ABS, f64, say, to_device
from oracle import attention_rows_fp64, attention_weights_fp64, score_matrix_bytes
from unfused_bound import bounds, score_extents
from workloads import WORKLOADS, generate, random_case

pytestmark = pytest.mark.gpu


def run_unfused(case):
    import torch

    import exact_attention_44_amd as E
    q, k, v, kpm = to_device(case)
    out, lse, S = E.fwd_unfused(q, k, v, causal=bool(case["causal"]), key_padding_mask=kpm,
                                scale=float(case["scale"]))
    torch.cuda.synchronize()
    return (out.float().cpu().numpy().astype(np.float64), lse.cpu().numpy().astype(np.float64), S)


def check(case, O, lse, picks, what, mean_bar=False):
    """Compare rows `picks` = [(b, h, rows)] with the oracle to the derived
    bound; returns the largest error / bound ratio."""
    q, k, v = f64(case, "q"), f64(case, "k"), f64(case, "v")
    scale, causal, kpm = float(case["scale"]), bool(case["causal"]), case["kpm"]
    refs = attention_rows_fp64(q, k, v, scale, causal, kpm, picks)
    pvs = attention_rows_fp64(q, k, np.abs(v), scale, causal, kpm, picks)
    ext = score_extents(q, k, scale, causal, kpm, rows=picks)
    worst, errs = 0.0, []
    for (b, h, rows), (Or, Lr), (PV, _), (M, A) in zip(picks, refs, pvs, ext):
        o, l = O[b, h, rows], lse[b, h, rows]
        assert np.all(np.isfinite(o)), what
        empty = np.isneginf(Lr)
        assert np.array_equal(np.isneginf(l), empty), f"{what}: -inf lse pattern differs"
        assert np.all(o[empty] == 0.0), f"{what}: rows with no visible key must be zero"
        bO, bL = bounds(M, A, k.shape[2], Or, PV, Lr)
        e = np.abs(o - Or)
        errs.append(e)
        worst = max(worst, float(np.max(e / bO)) if e.size else 0.0)
        if (~empty).any():
            worst = max(worst, float(np.max(np.abs(l - Lr)[~empty] / bL[~empty])))
    e = np.concatenate([x.ravel() for x in errs])
    say(f"  {what}: max|dO|={e.max():.3e} mean|dO|={e.mean():.3e} worst err/bound={worst:.3f}")
    assert worst <= 1.0, f"{what}: error beyond the derived bound ({worst:.3f} of it)"
    if mean_bar:
        assert e.mean() <= O_MEAN_ABS, f"{what}: mean|dO| {e.mean()} > {O_MEAN_ABS}"
    return worst


def all_rows(case):
    B, H, s_q = case["q"].shape[:3]
    return [(b, h, np.arange(s_q)) for b in range(B) for h in range(H)]


CASES = {
    # name: (seed, B, H, s_q, s_k, d, kwargs); s_k % 8 != 0 takes the 2-byte path
    "square_d128": (81, 1, 2, 256, 256, 128, {}),
    "ragged_odd_keys": (82, 2, 2, 300, 517, 128, {}),
    "causal_more_keys": (83, 1, 3, 200, 700, 64, dict(causal=True)),
    "causal_more_queries": (84, 1, 2, 650, 190, 128, dict(causal=True)),
    "lengths_empty_rows": (85, 3, 2, 130, 1000, 128, dict(mask="lengths")),
    "random_mask_causal_d64": (86, 2, 2, 260, 904, 64, dict(mask="random", causal=True)),
    "all_padded": (87, 2, 1, 64, 296, 64, dict(mask="all")),
    "negative_scale": (88, 1, 2, 128, 640, 128, dict(scale=-0.09)),
    "one_key": (89, 1, 2, 70, 1, 64, {}),
    "one_query_long_keys": (90, 1, 4, 1, 3000, 128, dict(mask="random")),
    "more_than_1024_keys_ragged": (91, 1, 1, 129, 2049, 128, dict(causal=True)),
}


@pytest.mark.parametrize("name", list(CASES))
def test_unfused_parity(name):
    seed, B, H, s_q, s_k, d, kw = CASES[name]
    say(f"case unfused {name}: B={B} H={H} s_q={s_q} s_k={s_k} d={d} {kw}")
    c = random_case(seed, B, H, s_q, s_k, d, **kw)
    O, lse, _ = run_unfused(c)
    check(c, O, lse, all_rows(c), name)


def test_unfused_no_keys():
    import torch

    import exact_attention_44_amd as E
    say("case unfused s_k = 0")
    q = torch.randn(1, 2, 50, 64, device="cuda:0").to(torch.bfloat16)
    k = torch.empty(1, 2, 0, 64, device="cuda:0", dtype=torch.bfloat16)
    out, lse, S = E.fwd_unfused(q, k, k)
    torch.cuda.synchronize()
    assert S.numel() == 0
    assert torch.all(out == 0) and torch.all(torch.isneginf(lse))


def test_unfused_unaligned_mask_pointer():
    """A key-padding mask that is not 8-byte aligned takes the byte-wise path."""
    import torch

    import exact_attention_44_amd as E
    say("case unfused unaligned mask")
    c = random_case(92, 2, 2, 100, 256, 128, mask="random")
    q, k, v, kpm = to_device(c)
    buf = torch.zeros(kpm.numel() + 1, dtype=torch.uint8, device=q.device)
    buf[1:] = kpm.reshape(-1)
    kpm1 = buf[1:].view(kpm.shape)
    assert kpm1.data_ptr() % 8 != 0
    out, lse, _ = E.fwd_unfused(q, k, v, key_padding_mask=kpm1, scale=float(c["scale"]))
    torch.cuda.synchronize()
    check(c, out.float().cpu().numpy().astype(np.float64), lse.cpu().numpy().astype(np.float64),
          all_rows(c), "unaligned mask")


def test_unfused_buffer_holds_the_weights():
    """On return the score buffer holds P = softmax(bf16 scores) in bf16: each
    weight within the derived relative bound of the exact weight, exactly 0
    where the key is hidden, and rows that sum to 1 within bf16 rounding."""
    import torch

    say("case unfused weights buffer")
    c = random_case(93, 2, 2, 96, 200, 64, causal=True, mask="lengths")
    _, _, S = run_unfused(c)
    P = S.float().cpu().numpy().astype(np.float64)
    q, k = f64(c, "q"), f64(c, "k")
    P_ref = attention_weights_fp64(q, k, float(c["scale"]), True, c["kpm"])
    assert np.all(P[P_ref == 0.0] == 0.0)
    for (b, h, rows), (M, A) in zip(all_rows(c), score_extents(q, k, float(c["scale"]), True, c["kpm"])):
        delta = 2.0 ** -8 * M + 2.0 ** -16 * A
        eta = 2.0 ** -8 + 2.0 ** -20 * (1 + M) + (200 / 64 + 16) * 2.0 ** -24
        rho = (1 + eta) * np.exp(2 * delta) - 1
        assert np.all(np.abs(P[b, h] - P_ref[b, h]) <= rho[:, None] * P_ref[b, h] + 1e-30)
    sums = P.sum(axis=-1)
    seen = P_ref.sum(axis=-1) > 0
    assert np.all(np.abs(sums[seen] - 1.0) <= 200 * 2.0 ** -8)
    assert torch.cuda.is_available()


def test_unfused_workload_small_full():
    w = WORKLOADS[0]
    say(f"workload unfused {w.name}")
    c = generate(w)
    O, lse, S = run_unfused(c)
    assert S.numel() * 2 == score_matrix_bytes(w.B, w.H, w.s_q, 2)
    check(c, O, lse, all_rows(c), w.name, mean_bar=True)


@pytest.mark.parametrize("idx", [1, 2])
def test_unfused_workload_causal_sampled(idx):
    """The "Worked example" shapes: the buffer is the page's 1.07 GB / 4.29 GB."""
    w = WORKLOADS[idx]
    say(f"workload unfused {w.name}")
    c = generate(w)
    O, lse, S = run_unfused(c)
    nbytes = S.numel() * S.element_size()
    assert nbytes == score_matrix_bytes(w.B, w.H, w.s_q, 2)
    say(f"  score matrix {nbytes / 1e9:.2f} GB")
    del S
    rng = np.random.default_rng(idx)
    picks = []
    for h in range(w.H):
        rows = np.arange(w.s_q) if h in (0, w.H - 1) else np.sort(rng.choice(w.s_q, 128, replace=False))
        picks.append((0, h, rows))
    check(c, O, lse, picks, w.name, mean_bar=True)
