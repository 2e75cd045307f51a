"""The C ABI's host-side validation under AddressSanitizer and
UndefinedBehaviorSanitizer: a C program built with both sanitizers drives
every entry point of the sanitized library (libbeam_moe_sanitized.so: host
code instrumented, device code as in the normal build) with valid and
invalid configurations, pointers and workspaces.  No GPU is needed: every
call returns from its host-side checks before any device work, and the
program checks the documented status codes."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
LIBDIR = os.path.join(ROOT, "grouped_top_routing_amd")
CLANG = "/opt/rocm/llvm/bin/clang"

C_SOURCE = r"""
#include <stdint.h>
#include <stdio.h>
#include <string.h>
#include "beam_moe.h"
#include "beam_moe_debug.h"

static int fails = 0;
#define EXPECT(cond) do { if (!(cond)) { printf("FAIL line %d: %s\n", __LINE__, #cond); ++fails; } } while (0)

static moe_config_t beam(int64_t t) {
  moe_config_t c;
  memset(&c, 0, sizeof c);
  c.num_tokens = t; c.hidden = 5120; c.intermediate = 2560; c.num_experts = 256;
  c.num_groups = 8; c.topk_groups = 4; c.topk = 8; c.renormalize = 1;
  c.routed_scaling = 2.5f; c.weight_layout = MOE_LAYOUT_PACKED;
  return c;
}

int main(void) {
  /* fake device pointers: aligned, never dereferenced (every call below
     fails validation or is a no-op) */
  void* p = (void*)(uintptr_t)0x100000;
  void* odd = (void*)(uintptr_t)0x100002;
  size_t n = 0, prev = 0;
  int e;
  moe_config_t c = beam(4096), d;
  moe_lora_t l;
  uint32_t flags = 7;

  /* workspace sizes for every entry and a range of batch sizes, including
     the largest supported one */
  int64_t ts[] = {0, 1, 7, 32, 512, 4096, 16384, 1000000, (((int64_t)1 << 31) - 1) / 8};
  for (unsigned i = 0; i < sizeof ts / sizeof ts[0]; ++i) {
    d = beam(ts[i]);
    for (e = MOE_ENTRY_ROUTE; e <= MOE_ENTRY_LAYER_LORA; ++e)
      EXPECT(moe_workspace_bytes(&d, e, &n) == MOE_OK);
    EXPECT(moe_workspace_bytes(&d, MOE_ENTRY_LAYER, &n) == MOE_OK && n >= prev);
    prev = n;
  }
  d = beam((int64_t)1 << 28);
  EXPECT(moe_workspace_bytes(&d, MOE_ENTRY_LAYER, &n) == MOE_ERR_UNSUPPORTED);
  d = beam(-1);
  EXPECT(moe_workspace_bytes(&d, MOE_ENTRY_LAYER, &n) == MOE_ERR_INVALID_ARG);
  EXPECT(moe_workspace_bytes(NULL, MOE_ENTRY_LAYER, &n) == MOE_ERR_INVALID_ARG);
  EXPECT(moe_workspace_bytes(&c, MOE_ENTRY_LAYER, NULL) == MOE_ERR_INVALID_ARG);
  EXPECT(moe_workspace_bytes(&c, -1, &n) == MOE_ERR_INVALID_ARG);
  EXPECT(moe_workspace_bytes(&c, 7, &n) == MOE_ERR_INVALID_ARG);

  /* configuration checks */
  d = c; d.num_groups = 3;       EXPECT(moe_workspace_bytes(&d, 0, &n) == MOE_ERR_INVALID_ARG);
  d = c; d.topk_groups = 9;      EXPECT(moe_workspace_bytes(&d, 0, &n) == MOE_ERR_INVALID_ARG);
  d = c; d.topk = 0;             EXPECT(moe_workspace_bytes(&d, 0, &n) == MOE_ERR_INVALID_ARG);
  d = c; d.renormalize = 2;      EXPECT(moe_workspace_bytes(&d, 0, &n) == MOE_ERR_INVALID_ARG);
  d = c; d.weight_layout = 3;    EXPECT(moe_workspace_bytes(&d, 0, &n) == MOE_ERR_INVALID_ARG);
  d = c; d.routed_scaling = 1.0f / 0.0f; EXPECT(moe_workspace_bytes(&d, 0, &n) == MOE_ERR_INVALID_ARG);
  d = c; d.num_experts = 128;    EXPECT(moe_workspace_bytes(&d, 0, &n) == MOE_ERR_UNSUPPORTED);
  d = c; d.hidden = 5000;        EXPECT(moe_workspace_bytes(&d, 0, &n) == MOE_ERR_UNSUPPORTED);
  d = c; d.intermediate = 2500;  EXPECT(moe_workspace_bytes(&d, 0, &n) == MOE_ERR_UNSUPPORTED);
  d = c; d.topk = 9; d.topk_groups = 8; EXPECT(moe_workspace_bytes(&d, 0, &n) == MOE_ERR_UNSUPPORTED);

  /* every entry point: null and misaligned pointers, small workspaces */
  EXPECT(moe_route(&c, NULL, p, NULL, p, p, p, 1 << 30, NULL) == MOE_ERR_INVALID_ARG);
  EXPECT(moe_route(&c, odd, p, NULL, p, p, p, 1 << 30, NULL) == MOE_ERR_INVALID_ARG);
  EXPECT(moe_route(&c, p, p, NULL, p, p, p, 4, NULL) == MOE_ERR_WORKSPACE);
  EXPECT(moe_route(&c, p, p, NULL, p, p, NULL, 0, NULL) == MOE_ERR_WORKSPACE);
  EXPECT(moe_route_replay(&c, p, p, NULL, p, p, 1 << 30, NULL) == MOE_ERR_INVALID_ARG);
  EXPECT(moe_permute(&c, p, p, p, p, NULL, p, 1 << 30, NULL) == MOE_ERR_INVALID_ARG);
  EXPECT(moe_permute(&c, p, p, p, p, p, p, 0, NULL) == MOE_ERR_WORKSPACE);
  EXPECT(moe_expert_ffn(&c, p, p, p, odd, p, p, p, 1 << 30, NULL) == MOE_ERR_INVALID_ARG);
  EXPECT(moe_expert_ffn(&c, p, p, p, p, p, p, p, 16, NULL) == MOE_ERR_WORKSPACE);
  EXPECT(moe_expert_gate_up(&c, p, p, p, p, NULL, p, 1 << 30, NULL) == MOE_ERR_INVALID_ARG);
  EXPECT(moe_expert_down(&c, p, p, p, p, p, 0, NULL) == MOE_ERR_WORKSPACE);
  EXPECT(moe_combine(&c, p, p, p, NULL, NULL) == MOE_ERR_INVALID_ARG);
  EXPECT(moe_combine(&c, odd, p, p, p, NULL) == MOE_ERR_INVALID_ARG);
  EXPECT(moe_layer_forward(&c, p, p, NULL, p, p, p, NULL, NULL, p, 64, NULL) == MOE_ERR_WORKSPACE);
  EXPECT(moe_layer_forward(&c, p, p, odd, p, p, p, NULL, NULL, p, 1 << 30, NULL)
         == MOE_ERR_INVALID_ARG);
  EXPECT(moe_layer_forward(NULL, p, p, NULL, p, p, p, NULL, NULL, p, 1 << 30, NULL)
         == MOE_ERR_INVALID_ARG);
  EXPECT(moe_layer_forward_noalloc(&c, p, p, NULL, p, p, p, NULL, NULL, NULL) == MOE_ERR_TOO_LARGE);
  EXPECT(moe_layer_forward_noalloc(&c, p, p, NULL, NULL, p, p, NULL, NULL, NULL)
         == MOE_ERR_INVALID_ARG);
  d = c; d.weight_layout = MOE_LAYOUT_FP8_PACKED;
  EXPECT(moe_layer_forward(&d, p, p, NULL, p, p, p, NULL, NULL, p, 1 << 30, NULL)
         == MOE_ERR_INVALID_ARG);
  EXPECT(moe_layer_forward_fp8(&c, p, p, NULL, p, p, p, p, p, NULL, NULL, p, 1 << 30, NULL)
         == MOE_ERR_INVALID_ARG);
  EXPECT(moe_expert_ffn_fp8(&d, p, p, p, p, NULL, p, p, p, p, 1 << 30, NULL) == MOE_ERR_INVALID_ARG);
  EXPECT(moe_expert_gate_up_fp8(&d, p, p, p, p, p, p, p, 0, NULL) == MOE_ERR_WORKSPACE);
  EXPECT(moe_expert_down_fp8(&d, p, p, p, p, p, p, 0, NULL) == MOE_ERR_WORKSPACE);
  EXPECT(moe_quantize_fp8(&c, p, NULL, p, NULL, NULL, NULL, NULL) == MOE_ERR_INVALID_ARG);
  EXPECT(moe_quantize_fp8(&c, p, NULL, p, (float*)p, NULL, NULL, NULL) == MOE_ERR_INVALID_ARG);
  EXPECT(moe_quantize_fp8(&c, NULL, NULL, NULL, NULL, NULL, NULL, NULL) == MOE_OK);
  EXPECT(moe_pack_weights(&c, p, NULL, NULL, NULL, NULL) == MOE_ERR_INVALID_ARG);
  EXPECT(moe_pack_weights(&c, p, NULL, (uint16_t*)p, NULL, NULL) == MOE_ERR_INVALID_ARG);
  EXPECT(moe_pack_weights(&c, NULL, NULL, NULL, NULL, NULL) == MOE_OK);
  memset(&l, 0, sizeof l);
  l.rank = 16; l.scale = 2.0f;
  EXPECT(moe_expert_ffn_lora(&c, p, p, p, p, p, &l, p, p, 1 << 30, NULL) == MOE_ERR_INVALID_ARG);
  l.a_gate_up = l.b_gate_up = l.a_down = l.b_down = (const uint16_t*)p; l.rank = 12;
  EXPECT(moe_expert_ffn_lora(&c, p, p, p, p, p, &l, p, p, 1 << 30, NULL) == MOE_ERR_INVALID_ARG);
  l.rank = 16; l.scale = 0.0f / 0.0f;
  EXPECT(moe_layer_forward_lora(&c, p, p, NULL, p, p, &l, p, NULL, NULL, p, 1 << 30, NULL)
         == MOE_ERR_INVALID_ARG);
  l.scale = 2.0f;
  EXPECT(moe_layer_forward_lora(&c, p, p, NULL, p, p, &l, p, NULL, NULL, p, 16, NULL)
         == MOE_ERR_WORKSPACE);

  /* an empty batch is a no-op once its arguments are valid */
  d = beam(0);
  EXPECT(moe_workspace_bytes(&d, MOE_ENTRY_LAYER, &n) == MOE_OK);
  EXPECT(moe_layer_forward(&d, p, p, NULL, p, p, p, NULL, NULL, p, n, NULL) == MOE_OK);
  EXPECT(moe_layer_forward(&d, p, p, NULL, p, p, p, NULL, NULL, NULL, 0, NULL)
         == (n ? MOE_ERR_WORKSPACE : MOE_OK));
  EXPECT(moe_combine(&d, p, p, p, p, NULL) == MOE_OK);
  EXPECT(moe_layer_forward_noalloc(&d, p, p, NULL, p, p, p, NULL, NULL, NULL) == MOE_OK);

  /* status strings and the debug query of the normal build */
  for (e = -6; e <= 1; ++e) EXPECT(moe_status_string(e) != NULL && strlen(moe_status_string(e)) > 0);
  EXPECT(moe_debug_check_flags(NULL) == MOE_ERR_INVALID_ARG);
  EXPECT(moe_debug_check_flags(&flags) == MOE_ERR_UNSUPPORTED && flags == 0);

  printf("%s (%d failures)\n", fails ? "sanitized C ABI checks failed" : "sanitized C ABI checks passed",
         fails);
  return fails != 0;
}
"""


def test_c_abi_validation_under_asan_and_ubsan(tmp_path):
    from grouped_top_routing_amd import build as b
    if not os.path.exists(CLANG):
        pytest.skip("ROCm clang not available")
    if not os.path.exists(b.LIB_SANITIZED):
        pytest.fail(f"{b.LIB_SANITIZED} is missing: build it with "
                    "`python -m grouped_top_routing_amd.build`")
    # the library's host code really is instrumented by both sanitizers
    syms = subprocess.run(["nm", "-D", b.LIB_SANITIZED], capture_output=True, text=True).stdout
    assert "__asan_report_load" in syms and "__ubsan_handle_" in syms
    src = tmp_path / "abi_sanitized.c"
    src.write_text(C_SOURCE)
    exe = tmp_path / "abi_sanitized"
    r = subprocess.run([CLANG, "-std=c99", "-g", "-Wall", "-Werror", "-fsanitize=address,undefined",
                        "-fno-omit-frame-pointer", "-shared-libasan", str(src),
                        "-I", os.path.join(ROOT, "include"), "-L", LIBDIR, "-lbeam_moe_sanitized",
                        "-Wl,-rpath," + LIBDIR, "-o", str(exe)], capture_output=True, text=True)
    assert r.returncode == 0, r.stderr
    env = dict(os.environ)
    env["LD_LIBRARY_PATH"] = b.clang_rt_dir() + ":" + env.get("LD_LIBRARY_PATH", "")
    # leak checking stays off: the HIP runtime keeps allocations for the life
    # of the process; every memory error and undefined behaviour aborts
    env["ASAN_OPTIONS"] = "detect_leaks=0:abort_on_error=0:halt_on_error=1"
    env["UBSAN_OPTIONS"] = "halt_on_error=1:print_stacktrace=1"
    r = subprocess.run([str(exe)], capture_output=True, text=True, timeout=300, env=env)
    assert r.returncode == 0, r.stdout + r.stderr
    assert "sanitized C ABI checks passed" in r.stdout
    assert "runtime error" not in r.stderr and "AddressSanitizer" not in r.stderr, r.stderr
