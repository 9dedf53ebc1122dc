"""Host logic of bench.py (no GPU): the one-GPU refusal, the algorithmic byte
model the roofline divides by, and the committed traffic records."""
import json
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402
import synth  # noqa: E402


def test_more_than_one_gpu_is_refused_before_touching_a_device():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout == ""


@pytest.mark.parametrize("name", ["tiny", "tiny_bf16_2step"])
def test_byte_model_equals_the_bytes_of_the_streamed_weights(name):
    """Every weight the step streams, counted from the arrays the benchmark
    generates: E, W_lm, the fusion and the DiT blocks (the adaLN and time-MLP
    weights feed the precomputed schedule and are not streamed per step)."""
    cfg = synth.CONFIGS["tiny"]
    if name == "tiny_bf16_2step":   # bf16 storage and two jumps: every streamed weight counted twice
        cfg = cfg.with_(dtype="bf16", times=(0.0, 0.5, 1.0))
    w = synth.make_weights(cfg)
    p = bench.alg_bytes(cfg)
    n = cfg.num_steps
    assert p["E"] == n * w["E"].nbytes
    assert p["W_lm"] == n * w["W_lm"].nbytes
    assert p["fusion"] == w["W_f"].nbytes + w["b_f"].nbytes
    block = 0
    for l in range(cfg.L):
        for t in ("W_qkv", "b_qkv", "W_o", "b_o", "W_1", "b_1", "W_2", "b_2"):
            block += w[f"blk{l}.{t}"].nbytes
    assert p["blocks"] == n * block
    assert p["total"] == sum(v for k, v in p.items() if k != "total")


def test_headline_bytes_match_the_planned_step():
    """The Qwen3-8B-shaped step: 622.3 MB each for E and W_lm, 604 MB of DiT
    weights, 83.9 MB of fusion weights, 1,969 MB in all."""
    p = bench.alg_bytes(synth.CONFIGS["qwen3_8b"])
    assert round(p["E"] / 1e6, 1) == 622.3
    assert round(p["W_lm"] / 1e6, 1) == 622.3
    assert round(p["blocks"] / 1e6) == 604
    assert round(p["fusion"] / 1e6, 1) == 83.9
    assert round(p["total"] / 1e6) == 1969
    # the roofline kernels: the embedding reads E and x and writes e and h;
    # the LM head reads W_lm and z and writes the tokens
    cfg = synth.CONFIGS["qwen3_8b"]
    assert bench.kernel_alg_bytes(cfg, "embed_kernel") == 627_453_952
    assert bench.kernel_alg_bytes(cfg, "lmhead_ks_kernel") == 622_395_456


def test_committed_traffic_records_follow_the_kernel_source():
    for kern in ("embed_kernel", "lmhead_ks_kernel"):
        path = os.path.join(ROOT, "profiles", f"{kern}_qwen3_8b_traffic.json")
        rec = json.load(open(path))
        assert rec["alg_bytes_per_launch"] == bench.kernel_alg_bytes(synth.CONFIGS["qwen3_8b"], kern)
        # a record taken on another kernel source is not reported
        if rec["source_hash"] == bench.source_hash(kern):
            assert bench.measured_traffic(kern, "qwen3_8b") == rec["bytes_per_launch"]
            # measured HBM bytes within 2% of the algorithmic bytes: no re-reads
            assert abs(rec["bytes_per_launch"] / rec["alg_bytes_per_launch"] - 1) < 0.02
        else:
            assert bench.measured_traffic(kern, "qwen3_8b") is None
