"""CPU-side checks of the C ABI: the library loads, exports every declared
symbol, and rejects bad arguments before touching the GPU."""
import ctypes
import os
import re

import pytest

import grouped_top_routing_amd as gtr
from grouped_top_routing_amd import _lib as L

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _declared_symbols():
    import glob
    text = "".join(open(h).read() for h in sorted(glob.glob(os.path.join(ROOT, "include", "*.h"))))
    return sorted(set(re.findall(r"^\s*(?:int|const char\*)\s+(moe_\w+)\s*\(", text, re.M)))


def test_library_exports_every_declared_symbol():
    lib = gtr.lib()
    declared = _declared_symbols()
    assert declared == sorted(L.EXPORTS)
    for name in declared:
        assert hasattr(lib, name), name


def test_checked_library_exports_every_declared_symbol():
    # the debug build with the kernels' index checks has the same ABI
    lib = L.load(L.LIB_CHECKED_PATH)
    for name in _declared_symbols():
        assert hasattr(lib, name), name


def test_debug_query_of_the_normal_build():
    # the normal build has no checks: the query says so without a device
    f = ctypes.c_uint32(5)
    assert gtr.lib().moe_debug_check_flags(ctypes.byref(f)) == L.MOE_ERR_UNSUPPORTED
    assert f.value == 0
    assert gtr.lib().moe_debug_check_flags(None) == L.MOE_ERR_INVALID_ARG


def test_status_strings():
    for code in (0, -1, -2, -3, -4, -5):
        assert gtr.status_string(code).startswith("MOE_")
    assert "unknown" in gtr.status_string(7)


def _cfg(**kw):
    base = dict(num_tokens=64, hidden=256, intermediate=128)
    base.update(kw)
    return gtr.make_config(base.pop("num_tokens"), base.pop("hidden"), base.pop("intermediate"),
                           **base)


@pytest.mark.parametrize("kw,code", [
    (dict(num_tokens=-1), L.MOE_ERR_INVALID_ARG),
    (dict(hidden=0), L.MOE_ERR_INVALID_ARG),
    (dict(num_groups=3), L.MOE_ERR_INVALID_ARG),          # 256 % 3 != 0
    (dict(topk_groups=9), L.MOE_ERR_INVALID_ARG),
    (dict(num_groups=8, topk_groups=1, topk=33), L.MOE_ERR_INVALID_ARG),
    (dict(renormalize=True, routed_scaling=float("nan")), L.MOE_ERR_INVALID_ARG),
    (dict(num_experts=128, num_groups=8), L.MOE_ERR_UNSUPPORTED),
    (dict(num_groups=128, topk_groups=4), L.MOE_ERR_UNSUPPORTED),
    (dict(topk=9), L.MOE_ERR_UNSUPPORTED),
    (dict(hidden=320), L.MOE_ERR_UNSUPPORTED),
    (dict(intermediate=96), L.MOE_ERR_UNSUPPORTED),
    (dict(num_tokens=1 << 28), L.MOE_ERR_UNSUPPORTED),
])
def test_config_validation(kw, code):
    cfg = _cfg(**kw)
    n = ctypes.c_size_t(0)
    assert gtr.lib().moe_workspace_bytes(ctypes.byref(cfg), L.ENTRY_LAYER, ctypes.byref(n)) == code


def test_null_config_and_bad_entry():
    n = ctypes.c_size_t(0)
    assert gtr.lib().moe_workspace_bytes(None, 0, ctypes.byref(n)) == L.MOE_ERR_INVALID_ARG
    cfg = _cfg()
    assert gtr.lib().moe_workspace_bytes(ctypes.byref(cfg), 9, ctypes.byref(n)) == L.MOE_ERR_INVALID_ARG
    assert gtr.lib().moe_workspace_bytes(ctypes.byref(cfg), 0, None) == L.MOE_ERR_INVALID_ARG


def test_workspace_sizes_grow_with_tokens():
    small = gtr.workspace_bytes(_cfg(num_tokens=32), L.ENTRY_LAYER)
    big = gtr.workspace_bytes(_cfg(num_tokens=4096), L.ENTRY_LAYER)
    assert 0 < small < big
    for e in (L.ENTRY_ROUTE, L.ENTRY_PERMUTE, L.ENTRY_EXPERT_FFN):
        assert 0 < gtr.workspace_bytes(_cfg(), e) <= gtr.workspace_bytes(_cfg(), L.ENTRY_LAYER)


# Fake, never-dereferenced, 16-byte aligned "device" addresses: every call
# below must fail validation on the host and enqueue nothing.
A = ctypes.c_void_p(0x10000)
MIS = ctypes.c_void_p(0x10004)


def _layer(cfg, x=A, wr=A, wgu=A, wd=A, out=A, ws=A, nb=1 << 40):
    return gtr.lib().moe_layer_forward(ctypes.byref(cfg), x, wr, None, wgu, wd, out, None, None,
                                       ws, nb, None)


def test_layer_rejects_null_and_misaligned_pointers():
    cfg = _cfg()
    assert _layer(cfg, x=None) == L.MOE_ERR_INVALID_ARG
    assert _layer(cfg, wgu=None) == L.MOE_ERR_INVALID_ARG
    assert _layer(cfg, out=None) == L.MOE_ERR_INVALID_ARG
    assert _layer(cfg, x=MIS) == L.MOE_ERR_INVALID_ARG
    assert _layer(cfg, wd=MIS) == L.MOE_ERR_INVALID_ARG


def test_layer_rejects_small_or_missing_workspace():
    cfg = _cfg()
    need = gtr.workspace_bytes(cfg, L.ENTRY_LAYER)
    assert _layer(cfg, nb=need - 1) == L.MOE_ERR_WORKSPACE
    assert _layer(cfg, ws=None, nb=need) == L.MOE_ERR_WORKSPACE
    assert _layer(cfg, ws=MIS, nb=need) == L.MOE_ERR_INVALID_ARG


def test_zero_tokens_is_a_noop():
    cfg = _cfg(num_tokens=0)
    need = gtr.workspace_bytes(cfg, L.ENTRY_LAYER)
    assert _layer(cfg, nb=need) == L.MOE_OK
    lib = gtr.lib()
    assert lib.moe_combine(ctypes.byref(cfg), A, A, A, A, None) == L.MOE_OK


def test_entry_points_reject_nulls():
    cfg = _cfg()
    lib = gtr.lib()
    big = 1 << 40
    assert lib.moe_route(ctypes.byref(cfg), None, A, None, A, A, A, big, None) == L.MOE_ERR_INVALID_ARG
    assert lib.moe_route_replay(ctypes.byref(cfg), A, A, None, A, A, big, None) == L.MOE_ERR_INVALID_ARG
    assert lib.moe_permute(ctypes.byref(cfg), A, A, None, A, A, A, big, None) == L.MOE_ERR_INVALID_ARG
    assert lib.moe_expert_ffn(ctypes.byref(cfg), A, A, A, None, A, A, A, big, None) == L.MOE_ERR_INVALID_ARG
    assert lib.moe_combine(ctypes.byref(cfg), A, None, A, A, None) == L.MOE_ERR_INVALID_ARG
    assert lib.moe_route(ctypes.byref(cfg), A, A, None, A, A, None, big, None) == L.MOE_ERR_WORKSPACE


def test_no_device_reports_hip_error():
    # In a container without a GPU a valid call must return MOE_ERR_HIP (the
    # library never falls back to the CPU).  On a GPU machine this check is moot.
    import torch
    if torch.cuda.is_available():
        pytest.skip("a GPU is present")
    cfg = _cfg()
    need = gtr.workspace_bytes(cfg, L.ENTRY_LAYER)
    assert _layer(cfg, nb=need) == L.MOE_ERR_HIP


def test_python_binding_requires_device_tensors():
    import torch
    x = torch.zeros(4, 256, dtype=torch.bfloat16)
    with pytest.raises((ValueError, TypeError)):
        gtr.route(x, torch.zeros(256, 256))


def test_weight_layout_and_pack_validation():
    cfg = _cfg(weight_layout=3)
    n = ctypes.c_size_t(0)
    lib = gtr.lib()
    assert lib.moe_workspace_bytes(ctypes.byref(cfg), L.ENTRY_LAYER, ctypes.byref(n)) == L.MOE_ERR_INVALID_ARG
    cfg = _cfg()
    B = ctypes.c_void_p(0x100000000)
    # one side of a pair missing
    assert lib.moe_pack_weights(ctypes.byref(cfg), A, None, None, None, None) == L.MOE_ERR_INVALID_ARG
    # misaligned
    assert lib.moe_pack_weights(ctypes.byref(cfg), MIS, None, B, None, None) == L.MOE_ERR_INVALID_ARG
    # output overlapping the input
    assert lib.moe_pack_weights(ctypes.byref(cfg), A, None, ctypes.c_void_p(0x10000 + 4096), None,
                                None) == L.MOE_ERR_INVALID_ARG
    # nothing to do
    assert lib.moe_pack_weights(ctypes.byref(cfg), None, None, None, None, None) == L.MOE_OK


def _fp8_cfg(**kw):
    kw.setdefault("weight_layout", L.LAYOUT_FP8_PACKED)
    return _cfg(**kw)


def test_fp8_entry_points_validate_layout_pointers_and_workspace():
    lib = gtr.lib()
    cfg = _fp8_cfg()
    big = 1 << 40
    ffn = lambda c, **p: lib.moe_expert_ffn_fp8(
        ctypes.byref(c), p.get("x", A), A, A, p.get("qgu", A), p.get("sgu", A), p.get("qd", A),
        p.get("sd", A), A, p.get("ws", A), p.get("nb", big), None)
    # the fp8 calls need the fp8 layout, the bf16 calls refuse it
    assert ffn(_cfg()) == L.MOE_ERR_INVALID_ARG
    assert lib.moe_expert_ffn(ctypes.byref(cfg), A, A, A, A, A, A, A, big, None) == L.MOE_ERR_INVALID_ARG
    assert ffn(cfg, qgu=None) == L.MOE_ERR_INVALID_ARG
    assert ffn(cfg, sd=None) == L.MOE_ERR_INVALID_ARG
    assert ffn(cfg, qd=MIS) == L.MOE_ERR_INVALID_ARG
    assert ffn(cfg, sgu=ctypes.c_void_p(0x10002)) == L.MOE_ERR_INVALID_ARG   # scales need 4 B
    assert ffn(cfg, sgu=MIS) != L.MOE_ERR_INVALID_ARG                         # 4 B is enough
    need = gtr.workspace_bytes(cfg, L.ENTRY_EXPERT_FFN)
    assert ffn(cfg, nb=need - 1) == L.MOE_ERR_WORKSPACE
    assert gtr.workspace_bytes(cfg, L.ENTRY_EXPERT_FFN) == gtr.workspace_bytes(_cfg(), L.ENTRY_EXPERT_FFN)
    assert lib.moe_expert_gate_up_fp8(ctypes.byref(cfg), A, A, A, None, A, A, A, big, None) == L.MOE_ERR_INVALID_ARG
    assert lib.moe_expert_down_fp8(ctypes.byref(cfg), A, A, A, None, A, A, big, None) == L.MOE_ERR_INVALID_ARG
    layer = lambda c, **p: lib.moe_layer_forward_fp8(
        ctypes.byref(c), A, A, None, A, A, p.get("qd", A), A, A, None, None, A,
        p.get("nb", big), None)
    assert layer(cfg, qd=None) == L.MOE_ERR_INVALID_ARG
    assert layer(cfg, nb=gtr.workspace_bytes(cfg, L.ENTRY_LAYER) - 1) == L.MOE_ERR_WORKSPACE
    zero = _fp8_cfg(num_tokens=0)
    assert layer(zero, nb=gtr.workspace_bytes(zero, L.ENTRY_LAYER)) == L.MOE_OK
    # calls that read no expert weights take any layout
    assert lib.moe_combine(ctypes.byref(_fp8_cfg(num_tokens=0)), A, A, A, A, None) == L.MOE_OK


def test_fp8_quantize_validation():
    lib = gtr.lib()
    cfg = _fp8_cfg()
    B, C = ctypes.c_void_p(0x100000000), ctypes.c_void_p(0x200000000)
    q = lambda *p: lib.moe_quantize_fp8(ctypes.byref(cfg), *p, None)
    assert q(None, None, None, None, None, None) == L.MOE_OK           # nothing to do
    assert q(A, None, B, None, None, None) == L.MOE_ERR_INVALID_ARG    # scales missing
    assert q(MIS, None, B, C, None, None) == L.MOE_ERR_INVALID_ARG     # misaligned weights
    assert q(A, None, ctypes.c_void_p(0x10000 + 4096), C, None, None) == L.MOE_ERR_INVALID_ARG
    assert q(A, None, B, ctypes.c_void_p(0x100000000 + 64), None, None) == L.MOE_ERR_INVALID_ARG
    if not __import__("torch").cuda.is_available():
        assert q(A, None, B, C, None, None) == L.MOE_ERR_HIP            # valid, no device


def test_fp8_binding_checks_dtypes():
    import torch
    w = gtr.Fp8Weights(torch.zeros(256, 256, 256, dtype=torch.uint8),
                       torch.zeros(256, 256), torch.zeros(256, 256, 128, dtype=torch.uint8),
                       torch.zeros(256, 256))
    assert w.shape == (256, 256, 128)
    with pytest.raises((ValueError, TypeError)):
        gtr.expert_ffn_fp8(torch.zeros(4, 256, dtype=torch.bfloat16),
                           torch.zeros(32, dtype=torch.int32), torch.zeros(257, dtype=torch.int32), w)


def test_lora_entry_points_validate_adapter():
    lib = gtr.lib()
    cfg = _cfg()
    big = 1 << 40

    def lora(**kw):
        d = dict(a_gate_up=0x10000, b_gate_up=0x20000, a_down=0x30000, b_down=0x40000, rank=16,
                 scale=2.0)
        d.update(kw)
        return L.MoeLora(d["a_gate_up"], d["b_gate_up"], d["a_down"], d["b_down"], d["rank"],
                         d["scale"])

    def ffn(lo, nb=big, c=cfg):
        return lib.moe_expert_ffn_lora(ctypes.byref(c), A, A, A, A, A,
                                       None if lo is None else ctypes.byref(lo), A, A, nb, None)

    assert ffn(None) == L.MOE_ERR_INVALID_ARG
    for bad in (dict(rank=8), dict(rank=24), dict(rank=128), dict(rank=0),
                dict(scale=float("nan")), dict(a_down=0), dict(b_gate_up=0x20008)):
        assert ffn(lora(**bad)) == L.MOE_ERR_INVALID_ARG, bad
    need = gtr.workspace_bytes(cfg, L.ENTRY_EXPERT_FFN_LORA)
    assert need > gtr.workspace_bytes(cfg, L.ENTRY_EXPERT_FFN)
    assert ffn(lora(), nb=need - 1) == L.MOE_ERR_WORKSPACE
    zero = _cfg(num_tokens=0)
    assert ffn(lora(), nb=gtr.workspace_bytes(zero, L.ENTRY_EXPERT_FFN_LORA), c=zero) == L.MOE_OK
    lay = lambda lo, nb: lib.moe_layer_forward_lora(ctypes.byref(cfg), A, A, None, A, A,
                                                    ctypes.byref(lo), A, None, None, A, nb, None)
    assert lay(lora(rank=20), big) == L.MOE_ERR_INVALID_ARG
    assert lay(lora(), gtr.workspace_bytes(cfg, L.ENTRY_LAYER_LORA) - 1) == L.MOE_ERR_WORKSPACE
    if not __import__("torch").cuda.is_available():
        assert ffn(lora(rank=64), nb=need) == L.MOE_ERR_HIP
