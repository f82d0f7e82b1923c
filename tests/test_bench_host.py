"""Host-side logic of bench.py (no GPU): the one-GPU guard, the algorithmic
byte counts behind the roofline's traffic figure, the measured-traffic table
and the source hash that keys it."""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402
from workloads import WORKLOADS  # noqa: E402


def _run_bench(args, env_extra=None):
    env = dict(os.environ)
    env.update(env_extra or {})
    return subprocess.run([sys.executable, os.path.join(ROOT, "bench.py")] + args, env=env,
                          capture_output=True, text=True, timeout=120)


def test_more_than_one_gpu_is_refused():
    r = _run_bench(["--gpus", "2"])
    assert r.returncode == 2
    assert "one GPU only" in r.stderr
    assert r.stdout == ""


def test_a_multi_rank_launch_is_refused():
    r = _run_bench([], {"WORLD_SIZE": "2"})
    assert r.returncode == 2
    assert "one GPU only" in r.stderr


def _tensor_bytes(w):
    """Bytes of each tensor of one call, element count times element size."""
    q = w.B * w.H * w.s_q * w.d
    kv = w.B * w.H * w.s_k * w.d
    rows = w.B * w.H * w.s_q
    return {"q": q, "k": kv, "v": kv, "o": q, "lse_rows": rows, "scores": w.B * w.H * w.s_q * w.s_k}


@pytest.mark.parametrize("i", range(len(WORKLOADS)))
def test_forward_bytes_are_inputs_once_and_outputs_once(i):
    w = WORKLOADS[i]
    t = _tensor_bytes(w)
    reads = 2 * (t["q"] + t["k"] + t["v"])           # bf16 Q, K, V
    writes = 2 * t["o"] + 4 * t["lse_rows"]          # bf16 O, float32 lse
    assert bench.algorithmic_bytes_of(w, "forward") == reads + writes
    fp8_reads = t["q"] + t["k"] + t["v"] + 3 * 4 * w.B * w.H   # one byte each, 3 descales per head
    assert bench.algorithmic_bytes_of(w, "fp8") == fp8_reads + writes
    # backward: reads Q, K, V, O, dO (bf16) and lse; writes dQ, dK, dV
    bwd = 2 * (t["q"] + t["k"] + t["v"] + t["o"] + t["o"]) + 4 * t["lse_rows"] \
        + 2 * (t["q"] + t["k"] + t["v"])
    assert bench.algorithmic_bytes_of(w, "backward") == bwd
    # materialising path: the 2-byte score matrix is written, read, rewritten
    # in place and read again, on top of the forward's own traffic
    assert bench.algorithmic_bytes_of(w, "unfused") == reads + writes + 4 * 2 * t["scores"]


def test_forward_bytes_of_the_named_workloads():
    """The decimal byte counts of the five workloads (Q, K, V read once; O and
    lse written once): 66.0 KB, 134.7 MB, 269.5 MB, 67.6 MB, 1.078 GB."""
    got = [bench.algorithmic_bytes_of(w, "forward") for w in WORKLOADS]
    assert got == [66048, 134742016, 269484032, 67633152, 1077936128]


def test_unknown_mode_is_an_error():
    with pytest.raises(ValueError):
        bench.algorithmic_bytes_of(WORKLOADS[0], "sideways")


def test_measured_writes_are_the_outputs():
    """WRITE_SIZE scaled by the copy calibration must come to the bytes the
    kernel stores (bf16 O and float32 lse) within 0.1 %: a check of the
    counter's scale factor against a closed form."""
    by_name = {w.name: w for w in WORKLOADS}
    assert bench.MEASURED_TRAFFIC
    for key, m in bench.MEASURED_TRAFFIC.items():
        w = by_name[key.split(":", 1)[-1]]
        t = _tensor_bytes(w)
        outputs = 2 * t["o"] + 4 * t["lse_rows"]
        assert abs(m["write_bytes"] - outputs) <= 1e-3 * outputs, key
        assert m["fetch_bytes"] > 0
        assert len(m["code_sha256"]) == 64 and int(m["code_sha256"], 16) >= 0


def test_code_hash_ignores_comments_and_blank_lines(tmp_path):
    a = tmp_path / "a.hip"
    b = tmp_path / "b.hip"
    c = tmp_path / "c.hip"
    a.write_text("int f(int x) {\n  return x + 1;\n}\n")
    b.write_text("// a comment\nint f(int x) {  // trailing comment\n\n  return x + 1;   \n}\n")
    c.write_text("int f(int x) {\n  return x + 2;\n}\n")
    assert bench.code_sha256(str(a)) == bench.code_sha256(str(b))
    assert bench.code_sha256(str(a)) != bench.code_sha256(str(c))


def test_peaks():
    # 256 CUs x 4096 dense bf16 FLOP per clock per CU x 2.4 GHz
    assert abs(bench.PEAK_BF16_TFLOPS - 2516.5824) < 1e-6
    assert bench.PEAK_FP8_TFLOPS == 2 * bench.PEAK_BF16_TFLOPS
    assert bench.PEAK_HBM_GBS == 8000.0
