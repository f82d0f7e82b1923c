"""GPU parity of the backward pass (attn_bwd) against the float64 oracle's
gradients of the definition. The GPU's backward gets the GPU forward's
outputs (bf16 O, float32 lse), as a training step would; the oracle
differentiates the exact definition."""
import numpy as np
import pytest

from gpu_util import f64, say, to_device
from oracle import attention_backward_fp64
from workloads import WORKLOADS, bf16_bits_to_f32, generate, random_case, round_to_bf16

pytestmark = pytest.mark.gpu

# Gradient tolerances, relative to each tensor's scale plus a float32 floor.
# The kernel rounds P and dS to bf16 (relative 2^-9) as MFMA operands, which
# gives errors of a few parts in 1e3 of the summed terms; and it forms
# D_i = dO_i . O_i from the forward's bf16 output, whose rounding (2^-9 of
# |dO_i| |O_i|) enters dS = P (dP - D) unscaled: where a row's softmax is
# nearly one-hot, dP - D cancels and this term sets the error (a case with
# scores 8x the usual size measures mean errors of 0.7 % of mean |ref|). The
# floors cover outputs that are exactly zero in exact arithmetic (one key:
# dq = 0) but come out as float32 rounding on the GPU.
G_MAX_REL, G_MAX_ABS = 2e-2, 1e-4    # max |err| <= rel * max |ref| + abs
G_MEAN_REL, G_MEAN_ABS = 1e-2, 1e-5  # mean |err| <= rel * mean |ref| + abs


def dout_for(case, seed):
    x = np.random.default_rng(seed).standard_normal(case["q"].shape, dtype=np.float32)
    return round_to_bf16(x)


def run_bwd(case, dout_bits, heads=None):
    import torch

    import exact_attention_44_amd as E
    q, k, v, kpm = to_device(case)
    g = torch.from_numpy(dout_bits.view(np.int16)).view(torch.bfloat16).to("cuda:0")
    causal, scale = bool(case["causal"]), float(case["scale"])
    out, lse = E.fwd(q, k, v, causal=causal, key_padding_mask=kpm, scale=scale)
    dq, dk, dv = E.bwd(q, k, v, out, g, lse, causal=causal, key_padding_mask=kpm, scale=scale)
    torch.cuda.synchronize()
    sel = (lambda t: t) if heads is None else (lambda t: t[:, heads])
    return tuple(sel(t).float().cpu().numpy().astype(np.float64) for t in (dq, dk, dv))


def oracle_bwd(case, dout_bits, heads=None):
    sel = (lambda a: a) if heads is None else (lambda a: np.ascontiguousarray(a[:, heads]))
    return attention_backward_fp64(sel(f64(case, "q")), sel(f64(case, "k")), sel(f64(case, "v")),
                                   sel(bf16_bits_to_f32(dout_bits).astype(np.float64)),
                                   float(case["scale"]), bool(case["causal"]), case["kpm"])


def compare_grads(got, ref, what):
    for name, a, r in zip(("dq", "dk", "dv"), got, ref):
        assert np.all(np.isfinite(a)), f"{what} {name}: non-finite"
        err = np.abs(a - r)
        scale_max, scale_mean = float(np.abs(r).max()), float(np.abs(r).mean())
        mx, mean = float(err.max()), float(err.mean())
        say(f"  {what} {name}: max|err|={mx:.3e} (max|ref| {scale_max:.3e}) "
            f"mean|err|={mean:.3e} (mean|ref| {scale_mean:.3e})")
        assert mx <= G_MAX_REL * scale_max + G_MAX_ABS, f"{what} {name}: max err {mx} (max|ref| {scale_max})"
        assert mean <= G_MEAN_REL * scale_mean + G_MEAN_ABS, f"{what} {name}: mean err {mean} (mean|ref| {scale_mean})"


CASES = {
    # name: (seed, B, H, s_q, s_k, d, kwargs)
    "dense_d64_small": (51, 1, 2, 128, 128, 64, {}),
    "causal_ragged_d128": (52, 2, 2, 300, 300, 128, dict(causal=True)),
    "causal_sq_lt_sk": (53, 1, 2, 200, 450, 128, dict(causal=True)),
    "causal_sq_gt_sk": (54, 1, 2, 333, 150, 64, dict(causal=True)),
    "padding_lengths": (55, 2, 2, 257, 400, 128, dict(mask="lengths")),
    "random_mask_causal": (56, 2, 1, 190, 190, 64, dict(mask="random", causal=True)),
    "negative_scale": (57, 1, 2, 160, 200, 128, dict(scale=-0.09)),
    "large_scores_causal": (58, 1, 2, 256, 256, 128, dict(q_mult=8.0, causal=True)),
    "all_padded": (59, 2, 1, 64, 100, 64, dict(mask="all")),
    "one_key": (60, 1, 2, 70, 1, 128, {}),
    "many_key_tiles": (61, 1, 1, 96, 1100, 128, {}),
    # whole tiles and 128-key blocks of padding inside the sequence: the dq
    # kernel does not walk those tiles, the dk/dv kernel skips those blocks
    "interior_padding_causal_d128": (62, 2, 2, 300, 2000, 128, dict(mask="blocks", causal=True)),
    "interior_padding_d64": (63, 2, 2, 260, 1800, 64, dict(mask="blocks")),
    # left padding: the visible tiles are one range that starts past key 0
    "prefix_padding_causal_d128": (65, 2, 2, 300, 1000, 128, dict(mask="prefix", causal=True)),
    "prefix_padding_d64": (66, 2, 2, 260, 900, 64, dict(mask="prefix")),
    # more 32-key tiles than the tile list holds: the dq kernel walks every
    # tile up to the last unpadded key
    "interior_padding_beyond_list_d128": (64, 1, 1, 24, 4096 * 32 + 700, 128, dict(mask="blocks")),
}


@pytest.mark.parametrize("name", list(CASES))
def test_bwd_parity(name):
    seed, B, H, s_q, s_k, d, kw = CASES[name]
    say(f"case bwd {name}: B={B} H={H} s_q={s_q} s_k={s_k} d={d} {kw}")
    c = random_case(seed, B, H, s_q, s_k, d, **kw)
    g = dout_for(c, seed + 7)
    compare_grads(run_bwd(c, g), oracle_bwd(c, g), name)


def test_bwd_bench_workload_two_heads():
    """The s = 8192 causal workload: all 32 heads on the GPU, heads 0 and 31
    compared in full."""
    w = WORKLOADS[2]
    say(f"workload {w.name} backward, heads 0 and {w.H - 1}")
    c = generate(w)
    g = dout_for(c, 4403)
    heads = [0, w.H - 1]
    compare_grads(run_bwd(c, g, heads=heads), oracle_bwd(c, g, heads=heads), w.name)


def test_bwd_deterministic():
    import torch

    import exact_attention_44_amd as E
    say("case bwd determinism")
    c = random_case(62, 1, 2, 300, 300, 128, causal=True, mask="random")
    q, k, v, kpm = to_device(c)
    g = torch.from_numpy(dout_for(c, 5).view(np.int16)).view(torch.bfloat16).to("cuda:0")
    out, lse = E.fwd(q, k, v, causal=True, key_padding_mask=kpm)
    a = E.bwd(q, k, v, out, g, lse, causal=True, key_padding_mask=kpm)
    b = E.bwd(q, k, v, out, g, lse, causal=True, key_padding_mask=kpm)
    torch.cuda.synchronize()
    assert all(torch.equal(x, y) for x, y in zip(a, b))


def test_bwd_no_device_allocation_and_side_stream():
    """With the caller's gradients and workspace given, the backward pass
    allocates nothing (no s x s buffer) and runs on whatever stream is
    current, with the same result as on the default stream."""
    import torch

    import exact_attention_44_amd as E
    say("case bwd allocation + side stream")
    c = random_case(63, 1, 4, 1000, 1000, 128, causal=True)
    q, k, v, _ = to_device(c)
    g = torch.from_numpy(dout_for(c, 6).view(np.int16)).view(torch.bfloat16).to(q.device)
    out, lse = E.fwd(q, k, v, causal=True)
    ref = E.bwd(q, k, v, out, g, lse, causal=True)
    torch.cuda.synchronize()
    dq, dk, dv = (torch.empty_like(t) for t in (q, k, v))
    ws = torch.empty(E.attn_bwd_workspace_bytes(1, 4, 1000), dtype=torch.uint8, device=q.device)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        E.bwd(q, k, v, out, g, lse, causal=True, dq=dq, dk=dk, dv=dv, workspace=ws)
    side.synchronize()
    for t in (dq, dk, dv):
        t.zero_()
    torch.cuda.synchronize()
    free0, _ = torch.cuda.mem_get_info()
    torch.cuda.reset_peak_memory_stats()
    a0 = torch.cuda.memory_allocated()
    with torch.cuda.stream(side):
        E.bwd(q, k, v, out, g, lse, causal=True, dq=dq, dk=dk, dv=dv, workspace=ws)
    side.synchronize()
    free1, _ = torch.cuda.mem_get_info()
    assert torch.cuda.max_memory_allocated() - a0 == 0
    assert free0 == free1, (free0, free1)
    assert all(torch.equal(x, y) for x, y in zip((dq, dk, dv), ref))
