"""GPU parity at the full Beam-1.0 shapes (hidden 5120, intermediate 2560,
256 experts, ~20 GB of bf16 expert weights resident on the device), in the
launch configuration the benchmark times:

* routing for every token against the oracle (sets bit-exact except tokens
  whose oracle margin is below 1e-5, which must be admissible);
* the permutation for every pair, exact;
* the expert GEMMs on every permuted row, and every 192-row tile of the
  busiest expert on its own, against the oracle's fp64 expert MLPs;
* the whole layer output over every token (max |y - r| / max(|r|, RMS) and
  mean |y - r| / RMS);
* the selection-bias switch and routing replay at the 4096-token shape;
* the same with FP8 per-channel weights, quantised on the device, against the
  oracle's own quantisation of the sampled experts (codes and scales bit-exact,
  outputs on the oracle's dequantised weights);
* the same with rank-16 expert LoRA adapters (scale 32 / 16).
"""
import numpy as np
import pytest
import torch

import grouped_top_routing_amd as gtr
import oracle
import synth
from parity_util import (MAX_REL, MEAN_REL, OracleFp8Experts, assert_close, check_routing,
                         err_stats, layer_reference, say, to_np, unpack_fp8_codes)

pytestmark = pytest.mark.gpu
DEV = torch.device("cuda", 0)
CONFIGS = ["decode", "mid", "prefill", "skew"]


@pytest.fixture(scope="module")
def beam():
    w = synth.workload("prefill")
    say("[beam] generating router and 256 experts on the device")
    wr = synth.make_router(w, 0, DEV)
    wgu, wd = synth.make_experts(w, 0, DEV)
    pgu, pd = gtr.pack_weights(wgu, wd)
    torch.cuda.synchronize()
    return {"w_router": wr, "w_gate_up": wgu, "w_down": wd, "wr_np": to_np(wr),
            "p_gate_up": pgu, "p_down": pd}


def _expert_np(beam, e):
    return to_np(beam["w_gate_up"][e]), to_np(beam["w_down"][e])


def _oracle_y_perm(beam, xn, rps, ro, tag):
    """The oracle's expert MLPs over every permuted row, expert by expert
    (fp64; each expert's bf16 weights are copied to the host in turn)."""
    y = np.zeros((len(rps), xn.shape[1]))
    done = 0
    for e in range(256):
        r0, r1 = int(ro[e]), int(ro[e + 1])
        if r1 == r0:
            continue
        gu, dn = _expert_np(beam, e)
        y[r0:r1] = oracle.ffn_rows(xn[rps[r0:r1] // 8], gu, dn)
        done += 1
        if done % 32 == 0:
            say(f"  [{tag}] oracle experts done: {done}")
    return y


@pytest.mark.timeout(900)
@pytest.mark.parametrize("name", CONFIGS)
def test_beam_layer(beam, name):
    """The whole layer output and every expert row at a Beam-shape workload,
    against the oracle evaluated on every token."""
    w = synth.workload(name)
    say(f"[beam:{name}] T={w.T} generating x")
    x = synth.make_x(w, 0, DEV, w_router=beam["w_router"])
    say(f"[beam:{name}] layer_forward (packed weights)")
    out, ids, wts = gtr.layer_forward(x, beam["w_router"], beam["p_gate_up"], beam["p_down"],
                                      weight_layout=gtr.LAYOUT_PACKED, return_routing=True)
    torch.cuda.synchronize()
    assert torch.isfinite(out.float()).all()
    # the row-major weights give the same bits
    outr = gtr.layer_forward(x, beam["w_router"], beam["w_gate_up"], beam["w_down"])
    assert torch.equal(out, outr)
    del outr
    xn = to_np(x)
    say(f"[beam:{name}] oracle routing")
    rr = oracle.route(xn, beam["wr_np"])
    nf, nd = check_routing(to_np(ids), to_np(wts), rr)
    counts = np.bincount(rr.ids.ravel(), minlength=256)
    say(f"  flagged={nf} flagged_differing={nd} touched={int((counts > 0).sum())} "
        f"max={counts.max()} min={counts.min()} lt10={int((counts < 10).sum())} "
        f"empty={int((counts == 0).sum())}")

    # permutation of the oracle's ids, exact
    say(f"[beam:{name}] permute")
    c, o, ps, pd = gtr.permute(torch.from_numpy(rr.ids.astype(np.int32)).to(DEV))
    rc, ro, rps, rpd = oracle.permute(rr.ids, 256)
    assert np.array_equal(to_np(c), rc) and np.array_equal(to_np(o), ro)
    assert np.array_equal(to_np(ps), rps) and np.array_equal(to_np(pd), rpd)

    # expert GEMMs on the oracle's permutation, as the benchmark calls them
    say(f"[beam:{name}] expert gate/up + down")
    h = gtr.expert_gate_up(x, ps, o, beam["p_gate_up"], weight_layout=gtr.LAYOUT_PACKED)
    y = to_np(gtr.expert_down(h, o, beam["p_down"], weight_layout=gtr.LAYOUT_PACKED))
    del h
    say(f"[beam:{name}] oracle expert MLPs over all {len(rps)} rows")
    yr = _oracle_y_perm(beam, xn, rps, ro, name)
    assert_close(y, yr, f"y_perm, all {len(rps)} rows")
    # every 192-row m-tile of the busiest expert on its own
    e = int(np.argmax(rc))
    for r0 in range(int(ro[e]), int(ro[e + 1]), 192):
        r1 = min(r0 + 192, int(ro[e + 1]))
        mx, mn, _ = err_stats(y[r0:r1], yr[r0:r1])
        assert mx <= MAX_REL and mn <= MEAN_REL, f"expert {e} rows {r0}:{r1}: {mx:.3e} {mn:.3e}"
    say(f"  busiest expert {e}: {rc[e]} rows, every 192-row tile within tolerance")
    del y

    # the whole layer output; tokens the GPU routed differently (only inside
    # the selection margin) are evaluated by the oracle on the GPU's set
    ref = {"out": oracle.combine(yr, rpd, rr.weights, 2.5), "route": rr}
    del yr
    want = layer_reference(to_np(ids), ref, xn, lambda e: _expert_np(beam, e))
    mx, mn = assert_close(to_np(out), want, f"[beam:{name}] layer output, all {w.T} tokens")
    say(f"PARITY {name} T={w.T} max_rel={mx:.4e} mean_rel={mn:.4e} flagged={nf} "
        f"flagged_differing={nd}")


def test_beam_route_bias_and_replay(beam):
    # the selection-bias switch and routing replay at the Beam shape
    w = synth.workload("prefill")
    say("[beam:bias+replay] prefill")
    x = synth.make_x(w, 0, DEV)
    xn = to_np(x)
    bias = synth.make_sel_bias(w, 0, device=DEV)
    ids, wt = gtr.route(x, beam["w_router"], sel_bias=bias)
    rr = oracle.route(xn, beam["wr_np"], sel_bias=to_np(bias))
    nf, nd = check_routing(to_np(ids), to_np(wt), rr)
    say(f"  bias: flagged={nf} flagged_differing={nd}")
    ref_ids = rr.ids.astype(np.int32)
    for renorm in (True, False):
        wr = gtr.route_replay(x, beam["w_router"], torch.from_numpy(ref_ids).to(DEV),
                              renormalize=renorm)
        want, _ = oracle.route_replay(xn, beam["wr_np"], ref_ids, renormalize=renorm)
        np.testing.assert_allclose(to_np(wr), want, rtol=1e-5, atol=1e-7)


def test_beam_staged_calls_match_layer(beam):
    # the five-call sequence the benchmark times equals moe_layer_forward, bitwise
    w = synth.workload("prefill")
    say("[beam:staged] prefill")
    x = synth.make_x(w, 0, DEV)
    out = gtr.layer_forward(x, beam["w_router"], beam["w_gate_up"], beam["w_down"])
    ids, wt = gtr.route(x, beam["w_router"])
    c, o, ps, pd = gtr.permute(ids)
    h = gtr.expert_gate_up(x, ps, o, beam["p_gate_up"], weight_layout=gtr.LAYOUT_PACKED)
    y = gtr.expert_down(h, o, beam["p_down"], weight_layout=gtr.LAYOUT_PACKED)
    out2 = gtr.combine(y, pd, wt)
    assert torch.equal(out, out2)
    y2 = gtr.expert_ffn(x, ps, o, beam["w_gate_up"], beam["w_down"])
    assert torch.equal(y, y2)


@pytest.fixture(scope="module")
def beam_fp8(beam):
    say("[beam:fp8] quantising 256 experts on the device")
    f = gtr.quantize_fp8(beam["w_gate_up"], beam["w_down"])
    torch.cuda.synchronize()
    ref = OracleFp8Experts(lambda e: to_np(beam["w_gate_up"][e]),
                           lambda e: to_np(beam["w_down"][e]))
    return f, ref


def _check_fp8_expert(f, ref, e):
    (qg, sg), (qd, sd) = ref.quantized(e)
    assert np.array_equal(to_np(f.s_gate_up[e]).view(np.uint32), sg.view(np.uint32))
    assert np.array_equal(to_np(f.s_down[e]).view(np.uint32), sd.view(np.uint32))
    assert np.array_equal(unpack_fp8_codes(to_np(f.q_gate_up[e:e + 1]))[0], qg)
    assert np.array_equal(unpack_fp8_codes(to_np(f.q_down[e:e + 1]))[0], qd)


@pytest.mark.parametrize("name", ["decode", "prefill"])
def test_beam_layer_fp8(beam, beam_fp8, name):
    f, ref = beam_fp8
    w = synth.workload(name)
    say(f"[beam:fp8:{name}] T={w.T} layer_forward_fp8")
    x = synth.make_x(w, 0, DEV, w_router=beam["w_router"])
    out, ids, wts = gtr.layer_forward_fp8(x, beam["w_router"], f, return_routing=True)
    torch.cuda.synchronize()
    assert torch.isfinite(out.float()).all()
    # routing is the bf16 path's, bit for bit
    out16, ids16, w16 = gtr.layer_forward(x, beam["w_router"], beam["w_gate_up"],
                                          beam["w_down"], return_routing=True)
    assert torch.equal(ids, ids16) and torch.equal(wts, w16)
    xn = to_np(x)
    say(f"[beam:fp8:{name}] oracle routing")
    rr = oracle.route(xn, beam["wr_np"])
    check_routing(to_np(ids), to_np(wts), rr)
    rc, ro, rps, rpd = oracle.permute(rr.ids, 256)
    y = gtr.expert_ffn_fp8(x, torch.from_numpy(rps.astype(np.int32)).to(DEV),
                           torch.from_numpy(ro.astype(np.int32)).to(DEV), f)
    # one sampled unflagged token: its 8 experts' codes and scales, their
    # rows of the expert MLPs, and the layer output
    rng = np.random.default_rng(1)
    cand = np.nonzero(rr.margin >= oracle.MARGIN_TOL)[0]
    t = int(rng.choice(cand))
    outn = to_np(out)
    acc = np.zeros(xn.shape[1])
    for j, e in enumerate(rr.ids[t]):
        e = int(e)
        say(f"[beam:fp8:{name}] token {t} expert {e}")
        _check_fp8_expert(f, ref, e)
        gu, dn = ref(e)
        r0, r1 = int(ro[e]), int(ro[e + 1])
        r1 = min(r1, r0 + 192)
        assert_close(to_np(y[r0:r1]), oracle.ffn_rows(xn[rps[r0:r1] // 8], gu, dn),
                     f"y_perm expert {e} rows {r1 - r0}/{rc[e]}")
        acc += rr.weights[t, j] * oracle.ffn_rows(xn[t:t + 1], gu, dn)[0]
    assert_close(outn[t], 2.5 * acc, f"out token {t}")


@pytest.mark.parametrize("name", ["decode", "prefill"])
def test_beam_layer_lora(beam, name):
    w = synth.workload(name)
    say(f"[beam:lora:{name}] T={w.T} adapters + layer_forward_lora")
    ts = synth.make_lora(synth.workload("prefill"), 0, DEV, rank=oracle.LORA_RANK)
    s = oracle.lora_scale()
    lw = gtr.LoraWeights(*ts, scale=s)
    x = synth.make_x(w, 0, DEV, w_router=beam["w_router"])
    out, ids, wts = gtr.layer_forward_lora(x, beam["w_router"], beam["p_gate_up"],
                                           beam["p_down"], lw, weight_layout=gtr.LAYOUT_PACKED,
                                           return_routing=True)
    torch.cuda.synchronize()
    assert torch.isfinite(out.float()).all()
    xn = to_np(x)
    rr = oracle.route(xn, beam["wr_np"])
    check_routing(to_np(ids), to_np(wts), rr)
    rc, ro, rps, rpd = oracle.permute(rr.ids, 256)
    y = gtr.expert_ffn_lora(x, torch.from_numpy(rps.astype(np.int32)).to(DEV),
                            torch.from_numpy(ro.astype(np.int32)).to(DEV), beam["w_gate_up"],
                            beam["w_down"], lw)
    lora_e = lambda e: tuple(to_np(t[e]) for t in ts)
    rng = np.random.default_rng(2)
    cand = np.nonzero(rr.margin >= oracle.MARGIN_TOL)[0]
    t = int(rng.choice(cand))
    outn = to_np(out)
    acc = np.zeros(xn.shape[1])
    for j, e in enumerate(rr.ids[t]):
        e = int(e)
        gu, dn = _expert_np(beam, e)
        le = lora_e(e)
        r0, r1 = int(ro[e]), int(ro[e + 1])
        r1 = min(r1, r0 + 192)
        if j < 2:  # two experts' rows of the expert MLPs
            assert_close(to_np(y[r0:r1]), oracle.ffn_rows_lora(xn[rps[r0:r1] // 8], gu, dn, le, s),
                         f"y_perm expert {e} rows {r1 - r0}/{rc[e]}")
        acc += rr.weights[t, j] * oracle.ffn_rows_lora(xn[t:t + 1], gu, dn, le, s)[0]
    assert_close(outn[t], 2.5 * acc, f"out token {t}")
