"""GPU parity of the FP8 per-channel expert-weight path (vLLM recipe JSON
"Beam-1.0-501B-A23B", precision variant fp8) against the oracle.

* moe_quantize_fp8 against the oracle's quantiser, bit for bit (codes and
  scales), on the tiny workload's weights and on hand-made rows that hit every
  rounding case: ties, the subnormal range, zero rows, signed zeros, tiny and
  huge row scales.
* The fp8 expert GEMMs and the fp8 layer against the oracle evaluated on the
  weights the oracle dequantises from its own codes (never the library's).
"""
import numpy as np
import pytest
import torch

import grouped_top_routing_amd as gtr
import oracle
import synth
from parity_util import (OracleFp8Experts, assert_close, check_routing, layer_reference, say,
                         to_np, unpack_fp8_codes)

pytestmark = pytest.mark.gpu
DEV = torch.device("cuda", 0)


@pytest.fixture(scope="module")
def tiny():
    say("[fp8 tiny] generating inputs on", DEV)
    d = synth.make_inputs("tiny", 0, device=DEV)
    d["np"] = {k: to_np(d[k]) for k in ("x", "w_router", "w_gate_up", "w_down")}
    say("[fp8 tiny] quantising on the device")
    d["fp8"] = gtr.quantize_fp8(d["w_gate_up"], d["w_down"])
    torch.cuda.synchronize()
    d["ref_experts"] = OracleFp8Experts(d["np"]["w_gate_up"], d["np"]["w_down"])
    return d


def _check_quantized(fq, fs, w_np, what):
    q_ref, s_ref = oracle.quantize_fp8_per_channel(w_np)
    s_gpu = to_np(fs)
    assert np.array_equal(s_gpu.view(np.uint32), s_ref.astype(np.float32).view(np.uint32)), \
        f"{what}: scales differ"
    q_gpu = unpack_fp8_codes(to_np(fq))
    bad = np.argwhere(q_gpu != q_ref)
    assert bad.size == 0, f"{what}: {len(bad)} codes differ, first {bad[:3].tolist()}: " \
                          f"gpu {q_gpu[tuple(bad[0])]:#04x} oracle {q_ref[tuple(bad[0])]:#04x}"


def test_quantize_bits_exact(tiny):
    say("[fp8] quantiser, tiny weights")
    f = tiny["fp8"]
    _check_quantized(f.q_gate_up, f.s_gate_up, tiny["np"]["w_gate_up"], "gate_up")
    _check_quantized(f.q_down, f.s_down, tiny["np"]["w_down"], "down")


def _edge_rows(K, rng):
    """bf16-representable rows that hit the quantiser's corner cases."""
    rows = []
    # amax 448 -> scale exactly 1: midpoints between adjacent codes (ties to
    # even), in the normal and the subnormal range, both signs
    mids = np.array([1.0625, 1.1875, 3.25, 3.75, 17.0, 200.0, 2.0 ** -10, 3 * 2.0 ** -10,
                     5 * 2.0 ** -10, 15 * 2.0 ** -10, 2.0 ** -12, 416.0])
    r = np.zeros(K, np.float32)
    r[0] = 448.0
    r[1:1 + len(mids)] = mids
    r[1 + len(mids):1 + 2 * len(mids)] = -mids
    r[40] = -0.0
    rows.append(r)
    rows.append(np.zeros(K, np.float32))                                   # zero row: s = 1
    rows.append(np.where(np.arange(K) % 2 == 0, -0.0, 0.0).astype(np.float32))
    for scale in (1e-30, 1e-3, 1.0, 7.0, 1e30):                            # tiny .. huge rows
        rows.append((rng.standard_normal(K) * scale).astype(np.float32))
    r = (rng.standard_normal(K) * 0.02).astype(np.float32)                 # one outlier
    r[K // 2] = 3.0
    rows.append(r)
    r = (rng.standard_normal(K)).astype(np.float32)                        # negative amax
    r[3] = -20.0
    rows.append(r)
    return rows


def test_quantize_edge_rows():
    say("[fp8] quantiser, edge rows")
    rng = np.random.default_rng(3)
    E, H, I = 256, 256, 128
    gu = (rng.standard_normal((E, 2 * I, H)) * 0.05).astype(np.float32)
    dn = (rng.standard_normal((E, H, I)) * 0.05).astype(np.float32)
    for j, r in enumerate(_edge_rows(H, rng)):
        gu[j % E, (7 * j) % (2 * I)] = r
    for j, r in enumerate(_edge_rows(I, rng)):
        dn[(5 * j + 1) % E, (3 * j) % H] = r
    gu_bf = torch.from_numpy(gu).to(torch.bfloat16)
    dn_bf = torch.from_numpy(dn).to(torch.bfloat16)
    f = gtr.quantize_fp8(gu_bf.to(DEV), dn_bf.to(DEV))
    _check_quantized(f.q_gate_up, f.s_gate_up, to_np(gu_bf), "gate_up")
    _check_quantized(f.q_down, f.s_down, to_np(dn_bf), "down")


def _dev(a):
    return torch.from_numpy(np.asarray(a).astype(np.int32)).to(DEV)


def test_expert_ffn_fp8(tiny):
    say("[fp8] expert_ffn tiny")
    npd = tiny["np"]
    rr = oracle.route(npd["x"], npd["w_router"])
    counts, offsets, psrc, pdst = oracle.permute(rr.ids, 256)
    y = gtr.expert_ffn_fp8(tiny["x"], _dev(psrc), _dev(offsets), tiny["fp8"])
    ref = oracle.expert_ffn(npd["x"], psrc, offsets, tiny["ref_experts"])
    assert_close(to_np(y), ref, "y_perm")


@pytest.mark.parametrize("hot_rows,T", [(1, 64), (17, 64), (40, 700), (130, 700), (300, 1024),
                                        (1000, 3072), (3000, 16384)])
def test_expert_ffn_fp8_ragged_tiles(tiny, hot_rows, T):
    # one hot expert plus thin ones: ragged m-tiles at every tile height the
    # fp8 path picks (mean rows per expert 2 and 21 -> 32-row tiles, 32 ->
    # 128 rows, 96 and 512 -> 192 rows; at 16384 tokens each workgroup runs
    # several items back to back)
    say(f"[fp8] expert_ffn ragged hot_rows={hot_rows} T={T}")
    rng = np.random.default_rng(hot_rows + 1)
    ids = np.stack([rng.choice(np.arange(1, 256), 8, replace=False) for _ in range(T)])
    ids[:hot_rows, 0] = 0
    x = synth.make_x(synth.workload("tiny", T=T), 9, DEV)
    xn = to_np(x)
    counts, offsets, psrc, pdst = oracle.permute(ids, 256)
    y = gtr.expert_ffn_fp8(x, _dev(psrc), _dev(offsets), tiny["fp8"])
    ref = oracle.expert_ffn(xn, psrc, offsets, tiny["ref_experts"])
    assert_close(to_np(y), ref, "y_perm")


def test_fp8_stages_equal_ffn(tiny):
    say("[fp8] gate_up + down == expert_ffn, bitwise")
    ids, wt = gtr.route(tiny["x"], tiny["w_router"])
    c, o, ps, pd = gtr.permute(ids)
    y = gtr.expert_ffn_fp8(tiny["x"], ps, o, tiny["fp8"])
    h = gtr.expert_gate_up_fp8(tiny["x"], ps, o, tiny["fp8"])
    y2 = gtr.expert_down_fp8(h, o, tiny["fp8"])
    assert torch.equal(y, y2)


@pytest.mark.parametrize("T", [128, 1, 77, 300])
def test_layer_fp8(tiny, T):
    say(f"[fp8] layer T={T}")
    npd = tiny["np"]
    x = tiny["x"] if T == 128 else synth.make_x(synth.workload("tiny", T=T), 13, DEV)
    xn = to_np(x)
    out, ids, w = gtr.layer_forward_fp8(x, tiny["w_router"], tiny["fp8"], return_routing=True)
    ref = oracle.layer_forward(xn, npd["w_router"], tiny["ref_experts"])
    nf, nd = check_routing(to_np(ids), to_np(w), ref["route"])
    say(f"  flagged={nf} differing={nd}")
    assert_close(to_np(out), layer_reference(to_np(ids), ref, xn, tiny["ref_experts"]), "out")
    # routing does not depend on the expert weights' format
    out16, ids16, w16 = gtr.layer_forward(x, tiny["w_router"], tiny["w_gate_up"], tiny["w_down"],
                                          return_routing=True)
    assert torch.equal(ids, ids16) and torch.equal(w, w16)


def test_layer_fp8_identical_experts_closed_form(tiny):
    # every expert the same: the layer is 2.5 * FFN(x) whatever the routing
    say("[fp8] identical experts")
    gu = tiny["w_gate_up"][:1].expand(256, -1, -1).contiguous()
    dn = tiny["w_down"][:1].expand(256, -1, -1).contiguous()
    f = gtr.quantize_fp8(gu, dn)
    out = gtr.layer_forward_fp8(tiny["x"], tiny["w_router"], f)
    g0, d0 = tiny["ref_experts"](0)
    ref = 2.5 * oracle.ffn_rows(tiny["np"]["x"], g0, d0)
    assert_close(to_np(out), ref, "out")
