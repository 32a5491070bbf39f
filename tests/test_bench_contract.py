"""bench.py's contract pieces that need no GPU: the one-GPU refusal, the algorithmic work it
divides by (checked against the per-token and per-expert figures worked out from the layer's
shapes), and the staleness rule of the stored HBM counter traffic."""
import json
import os
import subprocess
import sys

import numpy as np
import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402
from synth import get_config  # noqa: E402


def test_more_than_one_gpu_is_refused_with_a_message():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=300, cwd=ROOT)
    assert r.returncode == 2
    assert "one GPU" in r.stderr or "--gpus 1" in r.stderr
    assert r.stdout.strip() == ""


@pytest.mark.parametrize("name,fmt_bytes_per_expert", [
    ("C2", 2 * 2880 * 2880 * 2 + 2 * 2880 * 2 + 2880 * 2880 * 2 + 2880 * 2),          # 49.78 MB bf16
    ("X1", 2 * 2880 * (1440 + 90) + 2 * 2880 * 2 + 2880 * (1440 + 90) + 2880 * 2),    # 13.24 MB MXFP4
])
def test_algorithmic_work_of_the_20b_layer(name, fmt_bytes_per_expert):
    cfg = get_config(name)
    counts = np.full(cfg.E, cfg.T * cfg.k // cfg.E)          # every expert touched
    alg = bench.algorithmic(cfg, counts)
    # flops per token: router 2 D E, and per selected expert mlp1 4 D F plus mlp2 2 D F
    assert alg["flops"] == cfg.T * (2 * 2880 * 32 + 4 * 6 * 2880 * 2880)
    assert round(alg["flops"] / cfg.T / 1e6, 2) == 199.25
    # bytes: touched experts' weights and biases, the router, x in bf16 and out in fp32
    assert alg["bytes"] == (32 * fmt_bytes_per_expert + 32 * 2880 * 2 + 32 * 2
                            + cfg.T * 2880 * 2 + cfg.T * 2880 * 4)
    assert alg["mlp1"]["unit_bytes"] + alg["mlp2"]["unit_bytes"] == fmt_bytes_per_expert
    # an expert no token reaches costs no weight bytes
    counts2 = counts.copy()
    counts2[3] = 0
    assert bench.algorithmic(cfg, counts2)["bytes"] == alg["bytes"] - fmt_bytes_per_expert


@pytest.mark.parametrize("name,h_bytes_per_row", [
    ("C2", 2880 * 2),                  # h in bf16
    ("X1", 2880 * 4),                  # MXFP4 at few rows per expert: h as a bf16 pair
    ("X2", 2880 * 6 * 3 // 8 + 96 * 4),  # scaled engine: three fp6 pieces, a scale dword per 32 (96 per row)
])
def test_per_kernel_bytes_of_the_20b_layer(name, h_bytes_per_row):
    """The bytes each grouped GEMM's roofline divides by: its touched experts' weights and
    biases, what it reads of the activations and what it writes (mlp1: x in bf16 and h; mlp2:
    h and the fp32 slot rows), with h in the representation the kernels use."""
    cfg = get_config(name)
    counts = np.full(cfg.E, cfg.T * cfg.k // cfg.E)
    alg = bench.algorithmic(cfg, counts)
    assert bench.mx_engine(cfg) == (name == "X2")
    rows = cfg.T * 4                   # routed rows, top-4
    w1 = alg["mlp1"]["unit_bytes"]
    w2 = alg["mlp2"]["unit_bytes"]
    assert alg["mlp1"]["bytes"] == 32 * w1 + cfg.T * 2880 * 2 + rows * h_bytes_per_row
    assert alg["mlp2"]["bytes"] == 32 * w2 + rows * h_bytes_per_row + rows * 2880 * 4
    assert alg["mlp1"]["flops"] == 4 * rows * 2880 * 2880
    assert alg["mlp2"]["flops"] == 2 * rows * 2880 * 2880


def test_stored_traffic_goes_stale_when_the_kernel_source_changes(tmp_path, monkeypatch):
    src = tmp_path / "gemm.hip"
    src.write_text("int a; // one comment\n/* block\ncomment */\nint b;\n")
    monkeypatch.setattr(bench, "GEMM_SRC", str(src))
    key = bench.source_key()
    src.write_text("int a;   // another comment\n\nint b;\n")
    assert bench.source_key() == key                         # comments and blank lines do not count
    traffic = tmp_path / "traffic.json"
    traffic.write_text(json.dumps({"C2/mlp1": {"bytes_per_launch": 123, "source_sha": key}}))
    monkeypatch.setattr(bench, "TRAFFIC_FILE", str(traffic))
    assert bench.stored_traffic("C2", "mlp1") == 123
    assert bench.stored_traffic("C2", "mlp2") is None
    src.write_text("int a;\nint c;\n")                       # a code change
    assert bench.stored_traffic("C2", "mlp1") is None
