"""The benchmark's host-side arithmetic (no GPU): algorithmic bytes and FLOPs
of one layer call, the layer-output tolerance statistic, the roofline bound
and the single-GPU contract."""
import os
import subprocess
import sys
from types import SimpleNamespace

import numpy as np
import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402

BEAM = SimpleNamespace(T=4096, H=5120, I=2560, K=8, E=256)


def test_algorithmic_bytes_and_flops_bf16():
    counts = np.zeros(256, np.int64)
    counts[:147] = 1                     # 147 touched experts
    a = bench.algorithmic(BEAM, counts)
    T, H, I = 4096, 5120, 2560
    assert a["touched"] == 147
    # a touched expert streams gate, up and down rows once: 3 * H * I bf16
    assert a["layer_bytes"] == 147 * 3 * H * I * 2 + 256 * H * 4 + 2 * T * H * 2
    assert a["gate_up_bytes"] == 147 * 2 * I * H * 2 + T * H * 2
    assert a["down_bytes"] == 147 * H * I * 2
    # 8 experts per token, three H x I matrices, 2 FLOP per multiply-add
    assert a["expert_flops"] == 8 * T * 2 * 3 * H * I
    assert a["gate_up_flops"] + a["down_flops"] == a["expert_flops"]
    # 78.6 MB per touched expert, 629.1 MFLOP per token
    assert abs(3 * H * I * 2 / 1e6 - 78.64) < 0.01
    assert abs(a["expert_flops"] / T / 1e6 - 629.1) < 0.1


def test_algorithmic_bytes_fp8():
    counts = np.full(256, 16, np.int64)
    a = bench.algorithmic(BEAM, counts, "fp8")
    H, I = 5120, 2560
    # one byte per code plus an fp32 scale per output row of each matrix
    assert a["layer_bytes"] == 256 * (3 * H * I + (2 * I + H) * 4) + 256 * H * 4 + 2 * 4096 * H * 2
    assert a["down_bytes"] == 256 * (H * I + H * 4)


def test_tolerance_statistic_hand_cases():
    r = np.array([[3.0, -4.0], [0.0, 0.0]])      # RMS = sqrt(25 / 4) = 2.5
    assert bench.tolerance_stats(r.copy(), r) == (0.0, 0.0)
    y = r.copy()
    y[0, 0] += 0.3                                # relative to |r| = 3 (above the RMS)
    mx, mn = bench.tolerance_stats(y, r)
    assert mx == pytest.approx(0.1) and mn == pytest.approx(0.3 / 4 / 2.5)
    y = r.copy()
    y[1, 1] = 0.05                                # near zero: the RMS floor applies
    mx, _ = bench.tolerance_stats(y, r)
    assert mx == pytest.approx(0.05 / 2.5)


def test_roofline_bound_switches_at_the_ridge():
    ridge = bench.BF16_PEAK_TFLOPS * 1e12 / (bench.HBM_PEAK_GBS * 1e9)   # ~315 FLOP/B
    assert 310 < ridge < 320
    alg = {"gate_up_bytes": 10**10, "gate_up_flops": int(100 * 10**10)}
    r = bench.kernel_roofline("gate_up", alg, {"gate_up": 2.0}, "mid")
    assert r["bound"] == "hbm" and r["unit"] == "GB/s"
    assert r["achieved"] == pytest.approx(5000.0) and r["frac"] == pytest.approx(0.625)
    assert r["traffic"] is None                     # counters are kept for the prefill batch only
    alg = {"gate_up_bytes": 10**10, "gate_up_flops": int(500 * 10**10)}
    r = bench.kernel_roofline("gate_up", alg, {"gate_up": 5.0}, "skew")
    assert r["bound"] == "mfma" and r["unit"] == "TFLOP/s"
    assert r["achieved"] == pytest.approx(1000.0, rel=1e-3)
    assert r["frac"] == pytest.approx(1000.0 / bench.BF16_PEAK_TFLOPS, rel=1e-3)


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr and r.stdout == ""


def test_parity_and_cpu_baseline_on_the_oracle_itself():
    """The benchmark's parity blocks and its CPU baseline, fed the oracle's
    own bf16-rounded output on the small workload (CPU tensors): no routing
    difference, errors at the bf16 rounding level, timings recorded."""
    import torch
    import oracle
    import synth
    d = synth.make_inputs("tiny", 0)
    w = d["workload"]
    npw = {k: d[k].float().numpy().astype(np.float64) for k in ("x", "w_router", "w_gate_up",
                                                                 "w_down")}
    ref = oracle.layer_forward(npw["x"], npw["w_router"], (npw["w_gate_up"], npw["w_down"]))
    out = torch.from_numpy(ref["out"]).to(torch.bfloat16)
    ids = torch.from_numpy(ref["ids"].astype(np.int32))
    wts = {"w_router": d["w_router"], "w_gate_up": d["w_gate_up"], "w_down": d["w_down"]}
    p = bench.layer_parity(w, d["x"], out, ids, wts)
    assert p["routing_sets_differing"] == 0 and p["output_tokens_compared"] == w.T
    assert p["within_tolerance"] and p["max_rel"] < 1e-2 and p["mean_rel"] < 3e-3
    assert set(p["oracle_seconds"]) == {"route_all_tokens", "expert_mlps_compared_tokens", "cores"}
    p = bench.layer_parity(w, d["x"], out, ids, wts, sample=16, seed=1)
    assert p["output_tokens_compared"] == 16 and p["within_tolerance"]
    c = bench.cpu_baseline(w, d["x"], wts, 256, torch, gpu_out=out, gpu_ids=ids)
    assert c["kind"] == "oracle" and c["unit"] == "tokens/s" and c["value"] > 0
    assert c["parity"]["within_tolerance"] and c["parity"]["routing_sets_differing"] == 0
