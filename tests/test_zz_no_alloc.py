"""The key-split forward without a workspace (attn_fwd_split_noalloc) against
the key-split forward with one (attn_fwd_split): two calls in a row through
the C ABI, the second on a smaller problem (so the fixed array still holds
the first call's partial results when it starts), each equal to the
workspace entry point's result bit for bit and within the parity bar of the
float64 oracle; neither call allocates device memory."""
import numpy as np
import pytest

from gpu_util import compare, f64, say, to_device
from oracle import attention_fp64
from workloads import random_case

pytestmark = pytest.mark.gpu

# (seed, B, H, s_q, s_k, d, kwargs, n_splits): the first uses more of the
# array than the second
CALLS = [
    (61, 2, 4, 700, 3000, 128, dict(causal=True, mask="lengths"), 5),
    (62, 1, 2, 130, 900, 64, dict(mask="random"), 3),
]


def _with_workspace(case, n):
    import torch

    import exact_attention_44_amd as E
    q, k, v, kpm = to_device(case)
    out, lse = E.fwd_split(q, k, v, n_splits=n, causal=bool(case["causal"]), key_padding_mask=kpm,
                           scale=float(case["scale"]))
    torch.cuda.synchronize()
    return out.cpu(), lse.cpu()


def _noalloc(case, n):
    import torch

    import exact_attention_44_amd as E
    q, k, v, kpm = to_device(case)
    B, H, s_q, d = q.shape
    out = torch.full_like(q, float("nan"))
    lse = torch.full((B, H, s_q), float("nan"), dtype=torch.float32, device=q.device)
    torch.cuda.synchronize()
    alloc0 = torch.cuda.memory_allocated()
    free0 = torch.cuda.mem_get_info()[0]
    st = E.attn_fwd_split_noalloc(q, k, v, out, lse, B, H, s_q, k.shape[2], d,
                                  float(case["scale"]), bool(case["causal"]), kpm, n,
                                  torch.cuda.current_stream().cuda_stream)
    assert st == E.ATTN_OK, E.attn_status_str(st)
    torch.cuda.synchronize()
    assert torch.cuda.memory_allocated() == alloc0
    assert torch.cuda.mem_get_info()[0] >= free0 - (1 << 20)
    return out.cpu(), lse.cpu()


def test_noalloc_matches_the_workspace_entry_point_twice():
    import torch

    import exact_attention_44_amd as E

    for seed, B, H, s_q, s_k, d, kw, n in CALLS:
        say(f"case noalloc: seed={seed} B={B} H={H} s_q={s_q} s_k={s_k} d={d} {kw} n_splits={n}")
        c = random_case(seed, B, H, s_q, s_k, d, **kw)
        chunks = min(n, (s_k + 63) // 64)
        need = E.attn_fwd_split_workspace_bytes(B, H, s_q, d, chunks)
        assert 0 < need <= E.ATTN_SPLIT_SCRATCH_BYTES
        out_ws, lse_ws = _with_workspace(c, n)
        out_na, lse_na = _noalloc(c, n)
        assert torch.equal(out_na.view(torch.int16), out_ws.view(torch.int16))
        assert torch.equal(lse_na.view(torch.int32), lse_ws.view(torch.int32))
        O_ref, lse_ref = attention_fp64(f64(c, "q"), f64(c, "k"), f64(c, "v"), float(c["scale"]),
                                        bool(c["causal"]), c["kpm"])
        compare(out_na.float().numpy().astype(np.float64), lse_na.numpy().astype(np.float64),
                O_ref, lse_ref, f"noalloc seed {seed}")
