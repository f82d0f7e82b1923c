"""GPU parity: the HIP kernel (through the C ABI) against the float64 oracle.

Small and ragged shapes are compared in full, element by element. The large
workloads (s = 4096 ... 32768) are compared on whole heads where the oracle is
quick and on seeded samples of rows elsewhere; rows are independent, so each
sampled row is checked exactly as in a full comparison.
"""
import numpy as np
import pytest

from gpu_util import compare, f64, run_gpu, say, to_device
from oracle import attention_fp64, attention_rows_fp64
from workloads import WORKLOADS, generate, random_case

pytestmark = pytest.mark.gpu


def oracle_full(case):
    return attention_fp64(f64(case, "q"), f64(case, "k"), f64(case, "v"), float(case["scale"]),
                          bool(case["causal"]), case["kpm"])


EDGE_CASES = {
    # name: (seed, B, H, s_q, s_k, d, kwargs)
    "single": (1, 1, 1, 1, 1, 64, {}),
    "ragged_causal_sq_lt_sk": (2, 2, 3, 300, 517, 128, dict(causal=True)),
    "ragged_causal_d64": (3, 1, 2, 777, 777, 64, dict(causal=True)),
    "random_mask": (4, 2, 2, 129, 1000, 64, dict(mask="random")),
    "random_mask_causal_d128": (5, 2, 2, 260, 333, 128, dict(mask="random", causal=True)),
    "causal_sq_gt_sk": (6, 3, 1, 200, 70, 128, dict(causal=True)),
    "lengths_incl_zero": (7, 4, 2, 96, 160, 128, dict(mask="lengths")),
    "all_padded": (8, 2, 1, 64, 100, 64, dict(mask="all")),
    "negative_scale": (9, 1, 2, 256, 256, 128, dict(scale=-0.09)),
    "zero_scale_causal": (10, 1, 2, 130, 300, 64, dict(scale=0.0, causal=True)),
    "large_scores_q30": (11, 1, 2, 300, 600, 128, dict(q_mult=30.0, causal=True)),
    "large_scores_padded": (12, 2, 1, 140, 700, 64, dict(q_mult=20.0, mask="random")),
    "causal_padded": (13, 2, 2, 513, 513, 128, dict(causal=True, mask="lengths")),
    "full_tiles": (14, 1, 1, 512, 512, 128, dict(causal=True)),
    "many_heads_tiny": (15, 4, 8, 33, 33, 64, {}),
    "one_key": (16, 1, 2, 70, 1, 128, {}),
    "long_keys_few_queries": (17, 1, 1, 3, 2500, 128, dict(causal=False)),
    # d = 64 runs a persistent grid (one workgroup per CU, one item per round):
    # more items than CUs, a partial last round, heads not a multiple of 8
    "rounds_causal_d64": (18, 3, 37, 600, 600, 64, dict(causal=True)),
    "rounds_lengths_d64": (19, 6, 16, 700, 650, 64, dict(mask="lengths")),
    "rounds_dense_d64": (28, 3, 37, 600, 650, 64, {}),
    # whole 64-key tiles of padding inside the sequence (tiles 8 .. 23 and a
    # ragged block near the end): those tiles are not walked
    "interior_padding_causal_d128": (22, 2, 2, 700, 3000, 128, dict(mask="blocks", causal=True)),
    "interior_padding_d64": (23, 3, 3, 300, 2600, 64, dict(mask="blocks")),
    "interior_padding_rounds_d64": (24, 4, 24, 520, 2100, 64, dict(mask="blocks", causal=True)),
    # more key tiles than the tile list holds (4096): the walk covers every
    # tile up to the last unpadded key instead
    # left padding: the visible tiles are one range that starts past key 0
    "prefix_padding_causal_d128": (26, 2, 2, 900, 2000, 128, dict(mask="prefix", causal=True)),
    "prefix_padding_rounds_d64": (27, 4, 24, 520, 1500, 64, dict(mask="prefix")),
    "interior_padding_beyond_list": (25, 2, 1, 40, 4096 * 64 + 900, 64, dict(mask="blocks")),
}


@pytest.mark.parametrize("name", list(EDGE_CASES))
def test_edge_and_ragged(name):
    seed, B, H, s_q, s_k, d, kw = EDGE_CASES[name]
    say(f"case {name}: B={B} H={H} s_q={s_q} s_k={s_k} d={d} {kw}")
    c = random_case(seed, B, H, s_q, s_k, d, **kw)
    O, lse = run_gpu(c)
    O_ref, lse_ref = oracle_full(c)
    compare(O, lse, O_ref, lse_ref, name)


def test_no_keys():
    import torch

    import exact_attention_44_amd as E
    say("case no_keys: s_k = 0")
    q = torch.randn(2, 2, 100, 128, device="cuda:0").to(torch.bfloat16)
    k = torch.empty(2, 2, 0, 128, device="cuda:0", dtype=torch.bfloat16)
    out, lse = E.fwd(q, k, k, causal=True)
    torch.cuda.synchronize()
    assert torch.all(out == 0) and torch.all(torch.isneginf(lse))


def test_empty_batch_writes_nothing():
    import torch

    import exact_attention_44_amd as E
    say("case empty: B = 0 and s_q = 0")
    z = torch.empty(0, 2, 5, 64, device="cuda:0", dtype=torch.bfloat16)
    out, lse = E.fwd(z, z, z)
    assert out.shape == (0, 2, 5, 64) and lse.shape == (0, 2, 5)
    z2 = torch.empty(1, 2, 0, 64, device="cuda:0", dtype=torch.bfloat16)
    k2 = torch.randn(1, 2, 7, 64, device="cuda:0").to(torch.bfloat16)
    out, lse = E.fwd(z2, k2, k2)
    assert out.shape == (1, 2, 0, 64)


def _sampled(case, picks, what):
    O, lse = run_gpu(case)
    refs = attention_rows_fp64(f64(case, "q"), f64(case, "k"), f64(case, "v"), float(case["scale"]),
                               bool(case["causal"]), case["kpm"], picks)
    Os = np.concatenate([O[b, h, rows] for b, h, rows in picks])
    Ls = np.concatenate([lse[b, h, rows] for b, h, rows in picks])
    Or = np.concatenate([r[0] for r in refs])
    Lr = np.concatenate([r[1] for r in refs])
    return compare(Os, Ls, Or, Lr, what)


def _picks(w, full_heads, rows_per_head, seed):
    rng = np.random.default_rng(seed)
    picks = []
    for b in range(w.B):
        for h in range(w.H):
            if (b, h) in full_heads:
                picks.append((b, h, np.arange(w.s_q)))
            else:
                picks.append((b, h, np.sort(rng.choice(w.s_q, rows_per_head, replace=False))))
    return picks


def test_workload_dense_small_full():
    w = WORKLOADS[0]
    say(f"workload {w.name}")
    c = generate(w)
    O, lse = run_gpu(c)
    compare(O, lse, *oracle_full(c), w.name)


def test_workload_key_padding_full():
    w = WORKLOADS[3]
    say(f"workload {w.name}")
    c = generate(w)
    O, lse = run_gpu(c)
    compare(O, lse, *oracle_full(c), w.name)


@pytest.mark.parametrize("idx", [1, 2])
def test_workload_causal_sampled(idx):
    w = WORKLOADS[idx]
    say(f"workload {w.name}")
    c = generate(w)
    picks = _picks(w, {(0, 0), (0, w.H - 1)}, 128, seed=idx)
    _sampled(c, picks, w.name)


def test_workload_long_context_sampled():
    w = WORKLOADS[4]
    say(f"workload {w.name}")
    c = generate(w)
    rng = np.random.default_rng(5)
    picks = []
    for h in range(w.H):
        n = 512 if h in (0, w.H - 1) else 48
        rows = np.sort(rng.choice(w.s_q, n, replace=False))
        if h == 0:
            rows = np.unique(np.concatenate([rows, np.arange(64), np.arange(w.s_q - 64, w.s_q)]))
        picks.append((0, h, rows))
    _sampled(c, picks, w.name)


def test_deterministic():
    import torch

    from gpu_util import to_device
    import exact_attention_44_amd as E
    say("case determinism")
    c = random_case(21, 1, 4, 1000, 1000, 128, causal=True, mask="random")
    q, k, v, kpm = to_device(c)
    o1, l1 = E.fwd(q, k, v, causal=True, key_padding_mask=kpm)
    o2, l2 = E.fwd(q, k, v, causal=True, key_padding_mask=kpm)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(l1, l2)


def test_no_device_allocation_and_side_stream():
    """The call allocates nothing beyond the caller's out/lse (no s x s buffer)
    and runs on whatever stream is current."""
    import torch

    from gpu_util import to_device
    import exact_attention_44_amd as E
    say("case allocation + side stream")
    w = WORKLOADS[1]
    c = generate(w, heads=slice(0, 8))
    q, k, v, _ = to_device(c)
    out = torch.empty_like(q)
    lse = torch.empty(q.shape[:3], dtype=torch.float32, device=q.device)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    # first launch on this stream loads the code object; measure after it
    with torch.cuda.stream(side):
        E.fwd(q, k, v, causal=True, out=out, lse=lse)
    side.synchronize()
    out.zero_()
    torch.cuda.synchronize()
    free0, _ = torch.cuda.mem_get_info()
    torch.cuda.reset_peak_memory_stats()
    a0 = torch.cuda.memory_allocated()
    with torch.cuda.stream(side):
        E.fwd(q, k, v, causal=True, out=out, lse=lse)
    side.synchronize()
    free1, _ = torch.cuda.mem_get_info()
    # nothing allocated by the call: no s x s score buffer (B*H*s^2*2 bytes
    # would be 0.27 GB here), no workspace
    assert torch.cuda.max_memory_allocated() - a0 == 0
    assert free0 == free1, (free0, free1)
    picks = [(0, 3, np.arange(0, w.s_q, 97))]
    ref = attention_rows_fp64(f64(c, "q"), f64(c, "k"), f64(c, "v"), float(c["scale"]), True, None, picks)[0]
    compare(out.float().cpu().numpy()[0, 3, picks[0][2]].astype(np.float64),
            lse.cpu().numpy()[0, 3, picks[0][2]].astype(np.float64), ref[0], ref[1], "side stream")


def test_concurrent_streams():
    """Launches on two streams that may overlap on the device (the d = 64
    persistent grid included: each holds at most one workgroup per CU and
    keeps no state between workgroups) give the same results as alone."""
    import torch

    from gpu_util import to_device
    import exact_attention_44_amd as E
    say("case concurrent streams")
    cases = [random_case(31, 2, 24, 700, 700, 64, causal=True, mask="lengths"),
             random_case(32, 2, 24, 600, 650, 64, mask="random"),
             random_case(33, 1, 16, 520, 520, 128, causal=True)]
    streams = [torch.cuda.Stream() for _ in cases]
    base = torch.cuda.current_stream()
    ins = [to_device(c) for c in cases]
    outs = []
    for st in streams:
        st.wait_stream(base)
    for (q, k, v, kpm), c, st in zip(ins, cases, streams):
        with torch.cuda.stream(st):
            outs.append(E.fwd(q, k, v, causal=bool(c["causal"]), key_padding_mask=kpm,
                              scale=float(c["scale"])))
    torch.cuda.synchronize()
    for (o, l), c, i in zip(outs, cases, range(len(cases))):
        O_ref, lse_ref = oracle_full(c)
        compare(o.float().cpu().numpy().astype(np.float64), l.cpu().numpy().astype(np.float64),
                O_ref, lse_ref, f"stream {i}")


def test_wrappers_refuse_wrong_outputs():
    """Outputs and workspaces given by the caller are checked before any launch."""
    import torch

    import exact_attention_44_amd as E
    c = random_case(20, 1, 2, 100, 100, 64)
    q, k, v, _ = to_device(c)
    dev = q.device
    with pytest.raises(ValueError):
        E.fwd(q, k, v, out=torch.empty(1, 2, 99, 64, dtype=torch.bfloat16, device=dev))
    with pytest.raises(ValueError):
        E.fwd(q, k, v, lse=torch.empty(1, 2, 100, dtype=torch.bfloat16, device=dev))
    with pytest.raises(ValueError):
        E.fwd_split(q, k, v, n_splits=2, workspace=torch.empty(1 << 20, dtype=torch.uint8))
    out, lse = E.fwd(q, k, v)
    with pytest.raises(ValueError):
        E.bwd(q, k, v, out, out, lse, dq=torch.empty(1, 2, 100, 32, dtype=torch.bfloat16, device=dev))
    with pytest.raises(ValueError):
        E.bwd(q, k, v, out, out, lse.cpu())
    torch.cuda.synchronize()
