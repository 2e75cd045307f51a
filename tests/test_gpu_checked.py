"""The checked build (libbeam_moe_checked.so, include/beam_moe_debug.h) on
the GPU: on valid inputs of every path (routing, permutation with dropped
ids, the bf16 expert GEMMs at every m-tile height, fp8, LoRA, combine) it
records no check and gives the normal build's results bit for bit; on
inputs that name rows outside their buffers it records the check that
caught them (the kernels clamp such indices, so they stay inside their
buffers; such inputs are given to the checked build only)."""
import numpy as np
import pytest
import torch

import grouped_top_routing_amd as gtr
import oracle
import synth
from parity_util import say, to_np

pytestmark = pytest.mark.gpu
DEV = torch.device("cuda", 0)


@pytest.fixture(scope="module")
def tiny():
    d = synth.make_inputs("tiny", 0, device=DEV)
    return d


def _no_checks(what):
    flags = gtr.check_flags()
    assert not any(flags.values()), f"{what}: checks fired: {[k for k, v in flags.items() if v]}"


@pytest.mark.parametrize("T", [37, 128, 700, 3000, 9000])
def test_checked_build_is_silent_and_bitwise_equal(tiny, T):
    say(f"[checked] layer T={T}")
    x = synth.make_x(synth.workload("tiny", T=T), 3, DEV)
    args = (x, tiny["w_router"], tiny["w_gate_up"], tiny["w_down"])
    want = gtr.layer_forward(*args)
    f8 = gtr.quantize_fp8(tiny["w_gate_up"], tiny["w_down"])
    want8 = gtr.layer_forward_fp8(x, tiny["w_router"], f8)
    lw = gtr.LoraWeights(*synth.make_lora(tiny["workload"], 0, DEV), scale=2.0)
    wantl = gtr.layer_forward_lora(*args, lw)
    torch.cuda.synchronize()
    with gtr.use_library(gtr.LIB_CHECKED_PATH):
        gtr.check_flags()  # clear
        got = gtr.layer_forward(*args)
        got8 = gtr.layer_forward_fp8(x, tiny["w_router"], f8)
        gotl = gtr.layer_forward_lora(*args, lw)
        _no_checks(f"layer T={T}")
    assert torch.equal(got, want) and torch.equal(got8, want8) and torch.equal(gotl, wantl)


def test_checked_build_dropped_ids_are_not_violations(tiny):
    say("[checked] permute + replay with out-of-range ids")
    rr = oracle.route(to_np(tiny["x"]), to_np(tiny["w_router"]))
    ids = rr.ids.astype(np.int32)
    ids[3, 1], ids[9, 0] = -1, 300
    ids_d = torch.from_numpy(ids).to(DEV)
    with gtr.use_library(gtr.LIB_CHECKED_PATH):
        gtr.check_flags()
        w = gtr.route_replay(tiny["x"], tiny["w_router"], ids_d)
        c, o, ps, pd = gtr.permute(ids_d)
        y = gtr.expert_ffn(tiny["x"], ps, o, tiny["w_gate_up"], tiny["w_down"])
        gtr.combine(y, pd, w)
        _no_checks("dropped ids")


def test_checked_build_catches_bad_combine_rows(tiny):
    # perm_dst naming rows past y_perm: caught and clamped
    say("[checked] combine rows out of range")
    T = 64
    y = torch.zeros(T * 8, 256, dtype=torch.bfloat16, device=DEV)
    w = torch.full((T, 8), 0.125, dtype=torch.float32, device=DEV)
    pdst = torch.arange(T * 8, dtype=torch.int32, device=DEV)
    pdst[5] = T * 8 + 1000
    with gtr.use_library(gtr.LIB_CHECKED_PATH):
        gtr.check_flags()
        gtr.combine(y, pdst, w)
        flags = gtr.check_flags()
    assert flags["combine_row"] and sum(flags.values()) == 1, flags


def test_checked_build_catches_bad_gather_rows(tiny):
    # a permutation naming a pair past T*topk (so a token past the
    # activations): caught and clamped, at a 64- and a 192-row tile height
    for T in (128, 3000):
        say(f"[checked] expert gather out of range T={T}")
        x = synth.make_x(synth.workload("tiny", T=T), 5, DEV)
        rng = np.random.default_rng(T)
        ids = np.stack([rng.choice(256, 8, replace=False) for _ in range(T)])
        counts, offsets, psrc, pdst = oracle.permute(ids, 256)
        psrc = psrc.astype(np.int32)
        psrc[7] = T * 8 + 77
        with gtr.use_library(gtr.LIB_CHECKED_PATH):
            gtr.check_flags()
            gtr.expert_ffn(x, torch.from_numpy(psrc).to(DEV),
                           torch.from_numpy(offsets.astype(np.int32)).to(DEV),
                           tiny["w_gate_up"], tiny["w_down"])
            flags = gtr.check_flags()
        assert flags["gather_index"] or flags["token_index"], flags
        assert not flags["weight_offset"] and not flags["plan_rows"], flags
