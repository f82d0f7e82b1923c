"""The entry points captured into a HIP graph (torch.cuda.CUDAGraph).

The library's calls enqueue kernels only (no memory set, copy, allocation or
synchronisation), so a caller can capture them with caller-owned buffers and
replay them. Each replay below follows eager work on the same buffers (a fill
kernel that overwrites every output) and a device synchronisation, and must
reproduce the eager result bit for bit: the forward, the key-split forward
and the backward pass in one graph; the FP8 forward, the materialising path
and the key-split forward without a workspace in another; each at d = 128
(one workgroup per item) and at d = 64 (the persistent grid, whose
compute-unit count is taken before the capture).
"""
import numpy as np
import pytest

from gpu_util import say, to_device
from workloads import random_case

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("d,causal,mask", [(128, True, "none"), (64, False, "lengths")])
def test_graph_replays_match_eager(d, causal, mask):
    import torch

    import exact_attention_44_amd as E
    say(f"case graph capture d={d} causal={causal} mask={mask}")
    B, H, s = 2, 4, 700
    c = random_case(80 + d, B, H, s, s, d, causal=causal, mask=mask)
    q, k, v, kpm = to_device(c)
    gen = torch.Generator(device="cpu").manual_seed(d)
    g = torch.randn(q.shape, generator=gen).to(torch.bfloat16).to(q.device)
    kw = dict(causal=causal, key_padding_mask=kpm, scale=float(c["scale"]))

    # eager results (these calls also load the code objects)
    o_ref, l_ref = E.fwd(q, k, v, **kw)
    os_ref, ls_ref = E.fwd_split(q, k, v, n_splits=3, **kw)
    b_ref = E.bwd(q, k, v, o_ref, g, l_ref, **kw)
    torch.cuda.synchronize()

    out, lse = torch.empty_like(o_ref), torch.empty_like(l_ref)
    out_s, lse_s = torch.empty_like(o_ref), torch.empty_like(l_ref)
    ws_s = torch.empty(max(E.attn_fwd_split_workspace_bytes(B, H, s, d, 3), 256),
                       dtype=torch.uint8, device=q.device)
    dq, dk, dv = (torch.empty_like(t) for t in (q, k, v))
    ws_b = torch.empty(E.attn_bwd_workspace_bytes(B, H, s), dtype=torch.uint8, device=q.device)

    def step():
        E.fwd(q, k, v, out=out, lse=lse, **kw)
        E.fwd_split(q, k, v, n_splits=3, out=out_s, lse=lse_s, workspace=ws_s, **kw)
        E.bwd(q, k, v, out, g, lse, dq=dq, dk=dk, dv=dv, workspace=ws_b, **kw)

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step()  # warm-up on a side stream, as the capture API asks
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()

    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        step()
    torch.cuda.synchronize()

    outs = (out, lse, out_s, lse_s, dq, dk, dv)
    refs = (o_ref, l_ref, os_ref, ls_ref) + tuple(b_ref)
    names = ("out", "lse", "split out", "split lse", "dq", "dk", "dv")
    for r in range(3):
        for t in outs:
            t.fill_(3.0 + r)  # eager work that overwrites every output
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        for name, a, b in zip(names, outs, refs):
            assert torch.equal(a, b), f"replay {r}: {name} differs from the eager result"
        say(f"  replay {r}: all {len(outs)} outputs equal the eager results")
    # eager calls still work after the capture
    o2, l2 = E.fwd(q, k, v, **kw)
    torch.cuda.synchronize()
    assert torch.equal(o2, o_ref) and torch.equal(l2, l_ref)
    assert np.isfinite(out.float().cpu().numpy()).all()


@pytest.mark.parametrize("d,causal,mask", [(128, True, "none"), (64, False, "lengths")])
def test_graph_replays_match_eager_fp8_unfused_noalloc(d, causal, mask):
    """The FP8 forward, the materialising path and the key-split forward
    without a workspace (its partial results in the library's fixed device
    array, set up by the eager call before the capture) in one graph."""
    import torch

    import exact_attention_44_amd as E
    say(f"case graph capture (fp8, unfused, noalloc) d={d} causal={causal} mask={mask}")
    B, H, s = 2, 3, 600
    c = random_case(90 + d, B, H, s, s, d, causal=causal, mask=mask)
    q, k, v, kpm = to_device(c)
    kw = dict(causal=causal, key_padding_mask=kpm, scale=float(c["scale"]))
    gen = torch.Generator(device="cpu").manual_seed(7 + d)
    q8, k8, v8 = (torch.randn((B, H, s, d), generator=gen).mul(4.0).to(torch.float8_e4m3fn)
                  .view(torch.uint8).to(q.device) for _ in range(3))
    dq8, dk8, dv8 = (torch.rand((B, H), generator=gen).add(0.25).to(q.device) for _ in range(3))
    kw8 = dict(descale_q=dq8, descale_k=dk8, descale_v=dv8, **kw)

    o8_ref, l8_ref = E.fwd_fp8(q8, k8, v8, **kw8)
    ou_ref, lu_ref, p_ref = E.fwd_unfused(q, k, v, **kw)
    on_ref, ln_ref = E.fwd_split_noalloc(q, k, v, n_splits=3, **kw)
    torch.cuda.synchronize()

    o8, l8 = torch.empty_like(o8_ref), torch.empty_like(l8_ref)
    ou, lu, pu = torch.empty_like(ou_ref), torch.empty_like(lu_ref), torch.empty_like(p_ref)
    on, ln = torch.empty_like(on_ref), torch.empty_like(ln_ref)

    def step():
        E.fwd_fp8(q8, k8, v8, out=o8, lse=l8, **kw8)
        E.fwd_unfused(q, k, v, out=ou, lse=lu, scores=pu, **kw)
        E.fwd_split_noalloc(q, k, v, n_splits=3, out=on, lse=ln, **kw)

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()

    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        step()
    torch.cuda.synchronize()

    outs = (o8, l8, ou, lu, pu, on, ln)
    refs = (o8_ref, l8_ref, ou_ref, lu_ref, p_ref, on_ref, ln_ref)
    names = ("fp8 out", "fp8 lse", "unfused out", "unfused lse", "unfused weights",
             "no-workspace split out", "no-workspace split lse")
    for r in range(3):
        for t in outs:
            t.fill_(3.0 + r)  # eager work that overwrites every output
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        for name, a, b in zip(names, outs, refs):
            assert torch.equal(a, b), f"replay {r}: {name} differs from the eager result"
        say(f"  replay {r}: all {len(outs)} outputs equal the eager results")
    assert np.isfinite(o8.float().cpu().numpy()).all()
