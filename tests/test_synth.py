"""The seeded input generators: determinism, distributions, and the skewed
workload's construction."""
import numpy as np
import torch

import synth


def test_mix32_tensor_matches_int():
    xs = [0, 1, 2, 12345, 0xDEADBEEF, 0xFFFFFFFF, 0x80000000]
    t = synth.mix32(torch.tensor(xs, dtype=torch.int64))
    assert t.tolist() == [synth.mix32_int(v) for v in xs]


def test_mix32_is_a_bijection_on_a_window():
    v = synth.mix32(torch.arange(0, 1 << 20, dtype=torch.int64))
    assert torch.unique(v).numel() == 1 << 20
    assert int(v.min()) >= 0 and int(v.max()) <= 0xFFFFFFFF


def test_counter_normal_moments_and_determinism():
    z = synth.counter_normal(synth.stream_key(0, 9), 1 << 20)
    assert abs(float(z.mean())) < 5e-3
    assert abs(float(z.std()) - 1) < 5e-3
    assert float(z.abs().max()) <= 2 * 3 ** 0.5 + 1e-6
    z2 = synth.counter_normal(synth.stream_key(0, 9), 1 << 10, start=1000)
    assert torch.equal(z[1000:2024], z2)


def test_streams_differ():
    a = synth.counter_normal(synth.stream_key(0, 2, 0), 4096)
    b = synth.counter_normal(synth.stream_key(0, 2, 1), 4096)
    c = synth.counter_normal(synth.stream_key(1, 2, 0), 4096)
    assert abs(float(torch.corrcoef(torch.stack([a, b]))[0, 1])) < 0.1
    assert abs(float(torch.corrcoef(torch.stack([a, c]))[0, 1])) < 0.1


def test_tiny_inputs_shapes_and_dtypes():
    d = synth.make_inputs("tiny", 0)
    w = d["workload"]
    assert d["x"].shape == (128, 256) and d["x"].dtype == torch.bfloat16
    assert d["w_router"].shape == (256, 256) and d["w_router"].dtype == torch.float32
    assert d["w_gate_up"].shape == (256, 256, 256) and d["w_gate_up"].dtype == torch.bfloat16
    assert d["w_down"].shape == (256, 256, 128)
    assert abs(float(d["w_router"].std()) - w.router_std) < 1e-3
    assert abs(float(d["w_gate_up"].float().std()) - w.expert_std) < 1e-3
    d2 = synth.make_inputs("tiny", 0)
    assert torch.equal(d["x"], d2["x"]) and torch.equal(d["w_down"], d2["w_down"])


def test_skew_hot_set_and_shift():
    w = synth.workload("skew")
    hot = synth.hot_experts(w)
    assert len(hot) == 16 and len(set(hot)) == 16
    groups = sorted(np.bincount([e // 32 for e in hot], minlength=8).tolist(), reverse=True)
    assert groups[:4] == [6, 5, 5, 0]
    wr = synth.make_router(synth.workload("skew", H=512), 0)
    shift = synth.skew_shift(wr, hot)
    delta = wr.double() @ shift
    target = torch.zeros(256, dtype=torch.float64)
    target[hot] = 2.0
    assert torch.allclose(delta, target, atol=1e-9)
