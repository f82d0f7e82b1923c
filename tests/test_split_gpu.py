"""GPU parity of the key-split forward (attn_fwd_split) against the float64
oracle: the merged result against the definition over all keys, and the
per-chunk partial results the kernel leaves in the workspace against the
definition over each chunk's keys alone."""
import numpy as np
import pytest

from gpu_util import compare, f64, say, to_device
from oracle import attention_fp64, attention_rows_fp64
from workloads import SPLIT_WORKLOADS, generate, random_case

pytestmark = pytest.mark.gpu


def oracle_full(case, kpm=None):
    return attention_fp64(f64(case, "q"), f64(case, "k"), f64(case, "v"), float(case["scale"]),
                          bool(case["causal"]), case["kpm"] if kpm is None else kpm)


def run_split(case, n_splits, workspace=None):
    import torch

    import exact_attention_44_amd as E
    q, k, v, kpm = to_device(case)
    out, lse = E.fwd_split(q, k, v, n_splits=n_splits, causal=bool(case["causal"]),
                           key_padding_mask=kpm, scale=float(case["scale"]), workspace=workspace)
    torch.cuda.synchronize()
    return out.float().cpu().numpy().astype(np.float64), lse.cpu().numpy().astype(np.float64)


CASES = {
    # name: (seed, B, H, s_q, s_k, d, kwargs, n_splits)
    "two_chunks_causal_d128": (31, 1, 2, 300, 517, 128, dict(causal=True), 2),
    "ragged_d64_three": (32, 2, 2, 200, 777, 64, {}, 3),
    "padding_lengths_four": (33, 2, 2, 129, 1000, 128, dict(mask="lengths"), 4),
    "random_mask_causal_seven": (34, 1, 2, 260, 900, 64, dict(mask="random", causal=True), 7),
    "more_splits_than_tiles": (35, 1, 1, 70, 130, 128, {}, 50),
    "causal_chunks_past_diagonal": (36, 1, 3, 100, 1500, 128, dict(causal=True), 8),
    "large_scores_causal": (37, 1, 2, 256, 800, 128, dict(q_mult=30.0, causal=True), 3),
    "all_padded": (38, 2, 1, 64, 300, 64, dict(mask="all"), 3),
    "single_tile_runs_plain": (39, 1, 2, 50, 64, 128, {}, 4),
    "negative_scale": (40, 1, 2, 128, 640, 128, dict(scale=-0.09), 5),
    # d = 64 runs a persistent grid: more (chunk, query tile, head) items than CUs
    "rounds_d64_causal_lengths": (41, 2, 8, 1000, 3000, 64, dict(causal=True, mask="lengths"), 5),
}


@pytest.mark.parametrize("name", list(CASES))
def test_split_parity(name):
    seed, B, H, s_q, s_k, d, kw, n = CASES[name]
    say(f"case split {name}: B={B} H={H} s_q={s_q} s_k={s_k} d={d} {kw} n_splits={n}")
    c = random_case(seed, B, H, s_q, s_k, d, **kw)
    O, lse = run_split(c, n)
    compare(O, lse, *oracle_full(c), name)


@pytest.mark.parametrize("causal", [True, False], ids=["causal", "dense"])
def test_split_partials_are_the_chunks_own_results(causal):
    """The workspace holds, per chunk, attention over that chunk's keys alone
    (every chunk here has rows that see some of its keys and, with padding or
    causal masking, rows that see none)."""
    import torch

    import exact_attention_44_amd as E
    B, H, s_q, s_k, d, n = 2, 2, 700, 700, 128, 3
    say(f"case split partials: B={B} H={H} s_q={s_q} s_k={s_k} d={d} n_splits={n} causal={causal}")
    c = random_case(41, B, H, s_q, s_k, d, causal=causal, mask="lengths")
    c["kpm"][0, :] = 0  # batch item 0 sees all keys, so every chunk has data
    chunks = min(n, (s_k + 63) // 64)
    per = -(-s_k // chunks)
    k_chunk = -(-per // 64) * 64
    need = E.attn_fwd_split_workspace_bytes(B, H, s_q, d, chunks)
    ws = torch.full((need,), 0xFF, dtype=torch.uint8, device="cuda:0")  # NaN-filled on entry
    assert ws.data_ptr() % 256 == 0
    run_split(c, n, workspace=ws)
    rows = B * H * s_q
    o_bytes = -(-(chunks * rows * d * 4) // 256) * 256
    raw = ws.cpu()
    O_parts = raw[: chunks * rows * d * 4].view(torch.float32).numpy().reshape(chunks, B, H, s_q, d)
    L_parts = raw[o_bytes: o_bytes + chunks * rows * 4].view(torch.float32).numpy().reshape(chunks, B, H, s_q)
    for z in range(chunks):
        lo, hi = z * k_chunk, min((z + 1) * k_chunk, s_k)
        outside = np.ones(s_k, bool)
        outside[lo:hi] = False
        kpm = np.broadcast_to(outside, (B, s_k)).astype(np.uint8) | c["kpm"]
        Or, Lr = oracle_full(c, kpm=kpm)
        assert np.isfinite(Lr).any(), "every chunk must carry data"
        compare(O_parts[z].astype(np.float64), L_parts[z].astype(np.float64), Or, Lr,
                f"chunk {z} keys [{lo}, {hi})")


def test_split_prefill_chunk_workload_sampled():
    w = SPLIT_WORKLOADS[0]
    say(f"workload {w.name} n_splits=4")
    c = generate(w)
    rng = np.random.default_rng(7)
    picks = [(0, h, np.arange(w.s_q) if h in (0, w.H - 1) else np.sort(rng.choice(w.s_q, 64, replace=False)))
             for h in range(w.H)]
    O, lse = run_split(c, 4)
    refs = attention_rows_fp64(f64(c, "q"), f64(c, "k"), f64(c, "v"), float(c["scale"]), False, None, picks)
    Os = np.concatenate([O[b, h, r] for b, h, r in picks])
    Ls = np.concatenate([lse[b, h, r] for b, h, r in picks])
    compare(Os, Ls, np.concatenate([r[0] for r in refs]), np.concatenate([r[1] for r in refs]), w.name)


def test_split_deterministic_and_equal_across_calls():
    import torch

    import exact_attention_44_amd as E
    say("case split determinism")
    c = random_case(42, 1, 4, 300, 2000, 128, causal=True, mask="random")
    q, k, v, kpm = to_device(c)
    a = E.fwd_split(q, k, v, n_splits=6, causal=True, key_padding_mask=kpm)
    b = E.fwd_split(q, k, v, n_splits=6, causal=True, key_padding_mask=kpm)
    torch.cuda.synchronize()
    assert torch.equal(a[0], b[0]) and torch.equal(a[1], b[1])


def test_split_no_device_allocation_and_side_stream():
    """With out, lse and the workspace given, the key-split forward allocates
    nothing and runs on whatever stream is current, with the same result as on
    the default stream."""
    import torch

    import exact_attention_44_amd as E
    say("case split allocation + side stream")
    c = random_case(71, 1, 4, 300, 3000, 128, causal=True)
    q, k, v, _ = to_device(c)
    ref_o, ref_l = E.fwd_split(q, k, v, n_splits=5, causal=True)
    torch.cuda.synchronize()
    out, lse = torch.empty_like(ref_o), torch.empty_like(ref_l)
    ws = torch.empty(E.attn_fwd_split_workspace_bytes(1, 4, 300, 128, 5), dtype=torch.uint8,
                     device=q.device)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        E.fwd_split(q, k, v, n_splits=5, causal=True, out=out, lse=lse, workspace=ws)
    side.synchronize()
    out.zero_()
    torch.cuda.synchronize()
    free0, _ = torch.cuda.mem_get_info()
    torch.cuda.reset_peak_memory_stats()
    a0 = torch.cuda.memory_allocated()
    with torch.cuda.stream(side):
        E.fwd_split(q, k, v, n_splits=5, causal=True, out=out, lse=lse, workspace=ws)
    side.synchronize()
    free1, _ = torch.cuda.mem_get_info()
    assert torch.cuda.max_memory_allocated() - a0 == 0
    assert free0 == free1, (free0, free1)
    assert torch.equal(out, ref_o) and torch.equal(lse, ref_l)
