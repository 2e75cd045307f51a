"""moe_layer_forward_noalloc: the whole block with the library's static
scratch array instead of a caller workspace, for callers that cannot
allocate.  Its outputs must equal moe_layer_forward's (same kernels, same
order) on consecutive calls that share the array, the second smaller than the
first, and a configuration needing more than the array holds is refused on
the host before anything is enqueued."""
import ctypes

import numpy as np
import pytest
import torch

import grouped_top_routing_amd as gtr
from grouped_top_routing_amd import _lib as L
import synth

DEV = torch.device("cuda", 0)


def test_noalloc_refuses_more_than_the_static_array():
    # 4096 tokens at the Beam shape need ~0.8 GB of scratch: refused on the
    # host (fake, aligned, never dereferenced pointers; no device is touched)
    cfg = gtr.make_config(4096, 5120, 2560)
    fake = ctypes.c_void_p(1 << 20)
    st = gtr.lib().moe_layer_forward_noalloc(ctypes.byref(cfg), fake, fake, None, fake, fake,
                                             fake, None, None, None)
    assert st == L.MOE_ERR_TOO_LARGE
    assert gtr.status_string(st).startswith("MOE_ERR_TOO_LARGE")
    # 512 tokens fit
    assert gtr.workspace_bytes(gtr.make_config(512, 5120, 2560), gtr.ENTRY_LAYER) <= 128 << 20


def _inputs(H, I, T, seed):
    w = synth.workload("tiny", T=T, H=H, I=I)
    return synth.make_inputs(w, seed, device=DEV)


@pytest.mark.gpu
@pytest.mark.parametrize("H,I,T1,T2", [(256, 128, 128, 37), (512, 384, 3000, 700)])
def test_noalloc_matches_layer_forward(H, I, T1, T2):
    print(f"[noalloc] H={H} I={I} T={T1} then T={T2}", flush=True)
    d = _inputs(H, I, T1, 0)
    for T in (T1, T2):
        x = d["x"][:T].contiguous()
        want, ids_w, w_w = gtr.layer_forward(x, d["w_router"], d["w_gate_up"], d["w_down"],
                                             return_routing=True)
        ids = torch.full((T, 8), -5, dtype=torch.int32, device=DEV)
        wt = torch.full((T, 8), -5.0, dtype=torch.float32, device=DEV)
        got, _, _ = gtr.layer_forward_noalloc(x, d["w_router"], d["w_gate_up"], d["w_down"],
                                              ids=ids, w=wt)
        torch.cuda.synchronize()
        assert torch.equal(got, want), f"T={T}: output differs from moe_layer_forward"
        assert torch.equal(ids, ids_w) and torch.equal(wt, w_w), f"T={T}: routing differs"
        assert torch.isfinite(got.float()).all()


@pytest.mark.gpu
def test_noalloc_packed_weights_and_bias():
    print("[noalloc] packed weights, selection bias", flush=True)
    d = _inputs(512, 384, 900, 1)
    pgu, pd = gtr.pack_weights(d["w_gate_up"], d["w_down"])
    bias = synth.make_sel_bias(synth.workload("tiny", H=512, I=384), 1, device=DEV)
    for T in (900, 64):
        x = d["x"][:T].contiguous()
        want = gtr.layer_forward(x, d["w_router"], pgu, pd, sel_bias=bias,
                                 weight_layout=gtr.LAYOUT_PACKED)
        got = gtr.layer_forward_noalloc(x, d["w_router"], pgu, pd, sel_bias=bias,
                                        weight_layout=gtr.LAYOUT_PACKED)
        torch.cuda.synchronize()
        assert torch.equal(got, want), f"T={T}: output differs from moe_layer_forward"
