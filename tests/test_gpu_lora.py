"""GPU parity of expert LoRA ("Beam 1.0" miles recipes, section 5.5: rank 16,
alpha 32 on every routed expert) against the oracle, at the tiny workload with
ragged tiles and several ranks, and at Beam shape on sampled experts and
tokens.  The oracle evaluates W a + s B (A a) in fp64 on the same bf16
adapters."""
import numpy as np
import pytest
import torch

import grouped_top_routing_amd as gtr
import oracle
import synth
from parity_util import assert_close, check_routing, say, to_np

pytestmark = pytest.mark.gpu
DEV = torch.device("cuda", 0)


def _dev(a):
    return torch.from_numpy(np.asarray(a).astype(np.int32)).to(DEV)


@pytest.fixture(scope="module")
def tiny():
    say("[lora tiny] generating inputs on", DEV)
    d = synth.make_inputs("tiny", 0, device=DEV)
    d["np"] = {k: to_np(d[k]) for k in ("x", "w_router", "w_gate_up", "w_down")}
    return d


def _adapters(w, rank, seed=0, scale=None):
    ts = synth.make_lora(w, seed, DEV, rank=rank)
    s = oracle.lora_scale(oracle.LORA_ALPHA, rank) if scale is None else scale
    return gtr.LoraWeights(*ts, scale=s), tuple(to_np(t) for t in ts), s


@pytest.mark.parametrize("rank", [16, 32, 64])
def test_expert_ffn_lora(tiny, rank):
    say(f"[lora] expert_ffn tiny rank={rank}")
    npd = tiny["np"]
    lw, lnp, s = _adapters(tiny["workload"], rank)
    rr = oracle.route(npd["x"], npd["w_router"])
    counts, offsets, psrc, pdst = oracle.permute(rr.ids, 256)
    y = gtr.expert_ffn_lora(tiny["x"], _dev(psrc), _dev(offsets), tiny["w_gate_up"],
                            tiny["w_down"], lw)
    ref = oracle.expert_ffn(npd["x"], psrc, offsets, (npd["w_gate_up"], npd["w_down"]),
                            lora=lnp, lora_scale_=s)
    assert_close(to_np(y), ref, "y_perm")
    # the adapter term is really there: the base output is far off
    base = oracle.expert_ffn(npd["x"], psrc, offsets, (npd["w_gate_up"], npd["w_down"]))
    d = np.abs(base - ref).mean() / np.sqrt(np.mean(ref * ref))
    say(f"  adapter share of the output: {d:.3f}")
    assert d > 0.05


@pytest.mark.parametrize("hot_rows,T", [(1, 64), (40, 200), (130, 700), (1000, 2048)])
def test_expert_ffn_lora_ragged_tiles(tiny, hot_rows, T):
    say(f"[lora] ragged hot_rows={hot_rows} T={T}")
    npd = tiny["np"]
    lw, lnp, s = _adapters(tiny["workload"], 16, seed=3)
    rng = np.random.default_rng(hot_rows + 7)
    ids = np.stack([rng.choice(np.arange(1, 256), 8, replace=False) for _ in range(T)])
    ids[:hot_rows, 0] = 0
    x = synth.make_x(synth.workload("tiny", T=T), 5, DEV)
    xn = to_np(x)
    counts, offsets, psrc, pdst = oracle.permute(ids, 256)
    y = gtr.expert_ffn_lora(x, _dev(psrc), _dev(offsets), tiny["w_gate_up"], tiny["w_down"], lw)
    ref = oracle.expert_ffn(xn, psrc, offsets, (npd["w_gate_up"], npd["w_down"]), lora=lnp,
                            lora_scale_=s)
    assert_close(to_np(y), ref, "y_perm")


def test_zero_adapter_is_the_base_path_bitwise(tiny):
    say("[lora] zero B == no adapter, bitwise")
    a_gu, b_gu, a_d, b_d = synth.make_lora(tiny["workload"], 1, DEV)
    lw = gtr.LoraWeights(a_gu, torch.zeros_like(b_gu), a_d, torch.zeros_like(b_d), 2.0)
    ids, wt = gtr.route(tiny["x"], tiny["w_router"])
    c, o, ps, pd = gtr.permute(ids)
    y = gtr.expert_ffn_lora(tiny["x"], ps, o, tiny["w_gate_up"], tiny["w_down"], lw)
    y0 = gtr.expert_ffn(tiny["x"], ps, o, tiny["w_gate_up"], tiny["w_down"])
    assert torch.equal(y, y0)


@pytest.mark.parametrize("T", [128, 1, 300])
def test_layer_lora(tiny, T):
    say(f"[lora] layer T={T}")
    npd = tiny["np"]
    lw, lnp, s = _adapters(tiny["workload"], 16)
    x = tiny["x"] if T == 128 else synth.make_x(synth.workload("tiny", T=T), 17, DEV)
    xn = to_np(x)
    out, ids, w = gtr.layer_forward_lora(x, tiny["w_router"], tiny["w_gate_up"], tiny["w_down"],
                                         lw, return_routing=True)
    ref = oracle.layer_forward(xn, npd["w_router"], (npd["w_gate_up"], npd["w_down"]), lora=lnp,
                               lora_scale_=s)
    check_routing(to_np(ids), to_np(w), ref["route"])
    lora_fn = lambda e: tuple(t[e] for t in lnp)
    experts = lambda e: (npd["w_gate_up"][e], npd["w_down"][e])
    # tokens routed across a tie are re-evaluated on the GPU's set with adapters
    ref_out = np.array(ref["out"], copy=True)
    for t in range(T):
        S = to_np(ids)[t].astype(np.int64)
        if set(S.tolist()) != set(ref["route"].ids[t].tolist()):
            sc = ref["route"].scores[t, S]
            wt = sc / sc.sum()
            ref_out[t] = 2.5 * sum(wt[j] * oracle.ffn_rows_lora(xn[t:t + 1], *experts(e),
                                                                lora_fn(e), s)[0]
                                   for j, e in enumerate(S))
    assert_close(to_np(out), ref_out, "out")
    # the packed base layout gives the same bits
    pgu, pdn = gtr.pack_weights(tiny["w_gate_up"], tiny["w_down"])
    outp = gtr.layer_forward_lora(x, tiny["w_router"], pgu, pdn, lw,
                                  weight_layout=gtr.LAYOUT_PACKED)
    assert torch.equal(out, outp)
