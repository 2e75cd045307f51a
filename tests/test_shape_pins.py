"""Pins the Beam-shape workload sizes against totals printed on the pages
(tests/golden/beam_shape_pins.json cites each one).  A shared expert, another
intermediate size or a fourth expert matrix would break these sums."""
import json
import os

import synth


def test_beam_shape_totals(golden_dir):
    with open(os.path.join(golden_dir, "beam_shape_pins.json")) as f:
        p = json.load(f)
    w = synth.workload("prefill")
    assert (w.H, w.I, w.E, w.G, w.KG, w.K) == (p["hidden"]["value"], p["intermediate"]["value"],
                                                p["experts"]["value"], p["groups"]["value"],
                                                p["groups"]["kept"], p["groups"]["topk"])
    assert w.E // w.G == p["groups"]["group_size"]
    per_expert = 3 * w.H * w.I                      # gate, up, down; no biases
    assert abs(per_expert / p["params_per_expert"]["value"] - 1) < p["params_per_expert"]["rel_tol"]
    layers = p["moe_layers"]["value"]
    expert_total = layers * w.E * per_expert
    total = p["total_params"]["value"]
    assert abs(expert_total / total - p["expert_share"]["value"]) < p["expert_share"]["abs_tol"]
    replicated = total - expert_total
    assert abs(replicated / p["replicated_params"]["value"] - 1) < p["replicated_params"]["rel_tol"]
    active = replicated + layers * w.K * per_expert   # no shared expert
    assert abs(active / p["active_params"]["value"] - 1) < p["active_params"]["rel_tol"]
    ep = p["ep_weights_per_gpu_bytes"]
    for n in (16, 8):
        per_gpu = (expert_total / n + replicated) * 2
        assert abs(per_gpu / ep[str(n)] - 1) < ep["rel_tol"], n


def test_shared_expert_would_break_the_pins(golden_dir):
    with open(os.path.join(golden_dir, "beam_shape_pins.json")) as f:
        p = json.load(f)
    per_expert = 3 * 5120 * 2560
    layers, total = 49, p["total_params"]["value"]
    # one shared expert per layer (an extra expert-sized MLP) moves the share off 98.4%
    expert_total = layers * 257 * per_expert
    assert abs(expert_total / total - p["expert_share"]["value"]) > p["expert_share"]["abs_tol"]
    # an intermediate size of 2048 misses "about 39M" per expert
    assert abs(3 * 5120 * 2048 / p["params_per_expert"]["value"] - 1) > p["params_per_expert"]["rel_tol"]
