"""GPU parity at the longest sequences the entry points accept (2^22 query or
key positions per (b, h), the limit their host checks enforce).

Two shapes, one long side each (and the FP8 forward on the long-key one, with 16 queries):
  long keys     200 queries (48 for the backward) against 2^22 keys, d = 64,
                every key padded with probability 1/2 and the last 4097 keys
                all padded. The two query tiles walk 65536 key tiles (the
                plain and the key-split forward), the padding scan covers
                4 MiB of mask, and the backward's dq kernel walks 65536 key
                tiles.
  long queries  2^22 queries against 77 keys, d = 128, causal: 16384 query
                tiles of one key tile each (the first ones on the causal
                diagonal), and one dk/dv workgroup that walks 65536 query
                tiles.
Forward outputs are compared on sampled rows (rows are independent, so each
sampled row is checked exactly as in a full comparison); the backward's
gradients on their whole short side and on sampled rows of the long side.
"""
import numpy as np
import pytest

from gpu_util import compare, f64, say, to_device
from oracle import attention_backward_fp64, attention_rows_fp64
from test_bwd_gpu import compare_grads, dout_for
from workloads import bf16_bits_to_f32, random_case

pytestmark = pytest.mark.gpu

MAX_SEQ = 1 << 22


def long_keys_case(s_q=200):
    c = random_case(4420, 1, 1, s_q, MAX_SEQ, 64, mask="random")
    c["kpm"][:, -4097:] = 1
    return c


def long_queries_case():
    return random_case(4421, 1, 1, MAX_SEQ, 77, 128, causal=True)


def sample_rows(s, seed, n=256, edge=128):
    rng = np.random.default_rng(seed)
    rows = np.concatenate([np.arange(min(edge, s)), np.arange(max(0, s - edge), s),
                           rng.choice(s, min(n, s), replace=False)])
    return np.unique(rows)


def oracle_rows(c, rows):
    (o, l), = attention_rows_fp64(f64(c, "q"), f64(c, "k"), f64(c, "v"), float(c["scale"]),
                                  bool(c["causal"]), c["kpm"], [(0, 0, rows)])
    return o, l


def test_forward_longest_key_range():
    import torch

    import exact_attention_44_amd as E
    c = long_keys_case()
    say(f"long keys: s_q=200 s_k={MAX_SEQ} d=64, random padding, "
        f"{int((c['kpm'] == 0).sum())} visible keys")
    q, k, v, kpm = to_device(c)
    rows = sample_rows(200, 1, n=40, edge=8)
    rows = np.unique(np.concatenate([rows, [127, 128]]))
    O_ref, lse_ref = oracle_rows(c, rows)
    scale = float(c["scale"])
    idx = torch.from_numpy(rows).to(q.device)
    out, lse = E.fwd(q, k, v, key_padding_mask=kpm, scale=scale)
    torch.cuda.synchronize()
    compare(out[0, 0].index_select(0, idx).float().cpu().numpy().astype(np.float64),
            lse[0, 0].index_select(0, idx).cpu().numpy().astype(np.float64), O_ref, lse_ref,
            "attn_fwd")
    out_s, lse_s = E.fwd_split(q, k, v, n_splits=16, key_padding_mask=kpm, scale=scale)
    torch.cuda.synchronize()
    compare(out_s[0, 0].index_select(0, idx).float().cpu().numpy().astype(np.float64),
            lse_s[0, 0].index_select(0, idx).cpu().numpy().astype(np.float64), O_ref, lse_ref,
            "attn_fwd_split, 16 chunks")


def test_forward_longest_query_range():
    import torch

    import exact_attention_44_amd as E
    c = long_queries_case()
    say(f"long queries: s_q={MAX_SEQ} s_k=77 d=128 causal")
    q, k, v, kpm = to_device(c)
    rows = sample_rows(MAX_SEQ, 2)
    O_ref, lse_ref = oracle_rows(c, rows)
    out, lse = E.fwd(q, k, v, causal=True, scale=float(c["scale"]))
    torch.cuda.synchronize()
    idx = torch.from_numpy(rows).to(q.device)
    compare(out[0, 0].index_select(0, idx).float().cpu().numpy().astype(np.float64),
            lse[0, 0].index_select(0, idx).cpu().numpy().astype(np.float64), O_ref, lse_ref,
            "attn_fwd")


def run_bwd_rows(c, dout_bits, q_rows=None, k_rows=None):
    """GPU forward + backward; returns (dq, dk, dv) as float64, restricted to
    the given rows of the query side and of the key side (None = all)."""
    import torch

    import exact_attention_44_amd as E
    q, k, v, kpm = to_device(c)
    g = torch.from_numpy(dout_bits.view(np.int16)).view(torch.bfloat16).to(q.device)
    causal, scale = bool(c["causal"]), float(c["scale"])
    out, lse = E.fwd(q, k, v, causal=causal, key_padding_mask=kpm, scale=scale)
    dq, dk, dv = E.bwd(q, k, v, out, g, lse, causal=causal, key_padding_mask=kpm, scale=scale)
    torch.cuda.synchronize()

    def pick(t, rows):
        t = t[0, 0]
        if rows is not None:
            t = t.index_select(0, torch.from_numpy(rows).to(t.device))
        return t.float().cpu().numpy().astype(np.float64)[None, None]

    return pick(dq, q_rows), pick(dk, k_rows), pick(dv, k_rows)


def oracle_bwd(c, dout_bits, row_block):
    return attention_backward_fp64(f64(c, "q"), f64(c, "k"), f64(c, "v"),
                                   bf16_bits_to_f32(dout_bits).astype(np.float64),
                                   float(c["scale"]), bool(c["causal"]), c["kpm"],
                                   row_block=row_block)


def test_backward_longest_key_range():
    c = long_keys_case(48)
    say(f"backward, long keys: s_q=48 s_k={MAX_SEQ} d=64, random padding")
    g = dout_for(c, 4422)
    k_rows = sample_rows(MAX_SEQ, 3, n=4096)
    got = run_bwd_rows(c, g, None, k_rows)
    # 16 query rows at a time keep the oracle's 16 x 2^22 score blocks small
    dq, dk, dv = oracle_bwd(c, g, 16)
    compare_grads(got, (dq, dk[:, :, k_rows], dv[:, :, k_rows]), "long keys")


def test_backward_longest_query_range():
    c = long_queries_case()
    say(f"backward, long queries: s_q={MAX_SEQ} s_k=77 d=128 causal")
    g = dout_for(c, 4423)
    q_rows = sample_rows(MAX_SEQ, 4, n=4096)
    got = run_bwd_rows(c, g, q_rows, None)
    dq, dk, dv = oracle_bwd(c, g, 2048)
    compare_grads(got, (dq[:, :, q_rows], dk, dv), "long queries")


def test_fp8_forward_longest_key_range():
    """attn_fwd_fp8 with 16 queries against 2^22 keys (d = 64, random padding,
    the last 4097 keys padded), every row checked against the derived FP8
    bound (the header of tests/test_fp8_gpu.py)."""
    from test_fp8_gpu import bound_terms, check, fp8_case, run_gpu8

    c = fp8_case(4424, 1, 1, 16, MAX_SEQ, 64, mask="random")
    c["kpm"][:, -4097:] = 1
    say(f"fp8, long keys: s_q=16 s_k={MAX_SEQ} d=64, random padding")
    O, lse = run_gpu8(c)
    check(O, lse, *bound_terms(c), "attn_fwd_fp8")
