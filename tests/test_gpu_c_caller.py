"""A plain C program drives the block on the GPU through the C ABI alone: no
torch, no Python binding.  It allocates device memory with the HIP runtime,
runs moe_layer_forward and the staged calls (moe_route -> moe_permute ->
moe_expert_ffn -> moe_combine) on the tiny workload's inputs read from files,
checks that both give the same bits, and writes the output and routing back;
the test compares them with the oracle and with the Python binding's output.
"""
import os
import shutil
import subprocess

import numpy as np
import pytest
import torch

import grouped_top_routing_amd as gtr
import oracle
import synth
from parity_util import assert_close, check_routing, layer_reference, say, to_np

pytestmark = pytest.mark.gpu
DEV = torch.device("cuda", 0)
ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
LIBDIR = os.path.join(ROOT, "grouped_top_routing_amd")

C_SOURCE = r"""
#include <stdio.h>
#include <stdlib.h>
#include <string.h>
#include "beam_moe.h"

/* the HIP runtime calls this program makes (libamdhip64) */
typedef int hipError_t;
hipError_t hipMalloc(void** ptr, size_t size);
hipError_t hipFree(void* ptr);
hipError_t hipMemcpy(void* dst, const void* src, size_t size, int kind);
hipError_t hipDeviceSynchronize(void);
enum { kHostToDevice = 1, kDeviceToHost = 2 };

#define CHECK(x) do { int s_ = (x); if (s_ != 0) { \
  printf("FAIL %s -> %d\n", #x, s_); return 1; } } while (0)

static const char* dir;

static void* load(const char* name, size_t n) {
  char path[4096];
  snprintf(path, sizeof path, "%s/%s", dir, name);
  FILE* f = fopen(path, "rb");
  void* p = malloc(n);
  if (!f || !p || fread(p, 1, n, f) != n) { printf("FAIL reading %s\n", path); exit(1); }
  fclose(f);
  return p;
}

static void save(const char* name, const void* p, size_t n) {
  char path[4096];
  snprintf(path, sizeof path, "%s/%s", dir, name);
  FILE* f = fopen(path, "wb");
  if (!f || fwrite(p, 1, n, f) != n) { printf("FAIL writing %s\n", path); exit(1); }
  fclose(f);
}

static void* dev(size_t n) {
  void* p = NULL;
  if (hipMalloc(&p, n ? n : 16) != 0) { printf("FAIL hipMalloc %zu\n", n); exit(1); }
  return p;
}

static void* upload(const char* name, size_t n) {
  void* h = load(name, n);
  void* d = dev(n);
  if (hipMemcpy(d, h, n, kHostToDevice) != 0) { printf("FAIL upload %s\n", name); exit(1); }
  free(h);
  return d;
}

int main(int argc, char** argv) {
  if (argc != 5) return 2;
  dir = argv[1];
  const long T = atol(argv[2]);
  const int H = atoi(argv[3]), I = atoi(argv[4]), E = 256, K = 8;
  moe_config_t c;
  memset(&c, 0, sizeof c);
  c.num_tokens = T; c.hidden = H; c.intermediate = I; c.num_experts = E;
  c.num_groups = 8; c.topk_groups = 4; c.topk = K; c.renormalize = 1;
  c.routed_scaling = 2.5f; c.weight_layout = MOE_LAYOUT_ROW_MAJOR;

  const size_t nx = (size_t)T * H * 2, nk = (size_t)T * K;
  uint16_t* x = upload("x.bin", nx);
  float* wr = upload("w_router.bin", (size_t)E * H * 4);
  uint16_t* wgu = upload("w_gate_up.bin", (size_t)E * 2 * I * H * 2);
  uint16_t* wd = upload("w_down.bin", (size_t)E * H * I * 2);

  size_t ws_bytes = 0;
  const int entries[4] = {MOE_ENTRY_LAYER, MOE_ENTRY_ROUTE, MOE_ENTRY_PERMUTE,
                          MOE_ENTRY_EXPERT_FFN};
  for (int i = 0; i < 4; ++i) {
    size_t b = 0;
    CHECK(moe_workspace_bytes(&c, entries[i], &b));
    if (b > ws_bytes) ws_bytes = b;
  }
  void* ws = dev(ws_bytes);

  uint16_t* out_l = dev(nx);
  int32_t* ids_l = dev(nk * 4);
  float* w_l = dev(nk * 4);
  CHECK(moe_layer_forward(&c, x, wr, NULL, wgu, wd, out_l, ids_l, w_l, ws, ws_bytes, NULL));

  int32_t* ids = dev(nk * 4);
  float* w = dev(nk * 4);
  int32_t* counts = dev((size_t)E * 4);
  int32_t* offsets = dev((size_t)(E + 1) * 4);
  int32_t* psrc = dev(nk * 4);
  int32_t* pdst = dev(nk * 4);
  uint16_t* y = dev(nk * H * 2);
  uint16_t* out_s = dev(nx);
  CHECK(moe_route(&c, x, wr, NULL, ids, w, ws, ws_bytes, NULL));
  CHECK(moe_permute(&c, ids, counts, offsets, psrc, pdst, ws, ws_bytes, NULL));
  CHECK(moe_expert_ffn(&c, x, psrc, offsets, wgu, wd, y, ws, ws_bytes, NULL));
  CHECK(moe_combine(&c, y, pdst, w, out_s, NULL));
  CHECK(hipDeviceSynchronize());

  void* h_out_l = malloc(nx); void* h_out_s = malloc(nx);
  void* h_ids_l = malloc(nk * 4); void* h_ids = malloc(nk * 4);
  void* h_w_l = malloc(nk * 4); void* h_w = malloc(nk * 4);
  CHECK(hipMemcpy(h_out_l, out_l, nx, kDeviceToHost));
  CHECK(hipMemcpy(h_out_s, out_s, nx, kDeviceToHost));
  CHECK(hipMemcpy(h_ids_l, ids_l, nk * 4, kDeviceToHost));
  CHECK(hipMemcpy(h_ids, ids, nk * 4, kDeviceToHost));
  CHECK(hipMemcpy(h_w_l, w_l, nk * 4, kDeviceToHost));
  CHECK(hipMemcpy(h_w, w, nk * 4, kDeviceToHost));
  if (memcmp(h_out_l, h_out_s, nx) || memcmp(h_ids_l, h_ids, nk * 4) ||
      memcmp(h_w_l, h_w, nk * 4)) {
    printf("FAIL staged calls differ from moe_layer_forward\n");
    return 1;
  }
  save("out.bin", h_out_l, nx);
  save("ids.bin", h_ids_l, nk * 4);
  save("w.bin", h_w_l, nk * 4);
  hipFree(x); hipFree(wr); hipFree(wgu); hipFree(wd); hipFree(ws);
  hipFree(out_l); hipFree(ids_l); hipFree(w_l); hipFree(ids); hipFree(w); hipFree(counts);
  hipFree(offsets); hipFree(psrc); hipFree(pdst); hipFree(y); hipFree(out_s);
  printf("C caller: staged calls == moe_layer_forward\n");
  return 0;
}
"""


def _bits(t):
    """Raw bytes of a device tensor (bf16 as its uint16 bit patterns)."""
    t = t.contiguous().cpu()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).numpy().view(np.uint16)
    return t.numpy()


@pytest.mark.parametrize("T", [128, 300])
def test_c_program_runs_the_block(tmp_path, T):
    gcc = shutil.which("gcc")
    if gcc is None:
        pytest.skip("gcc not available")
    say(f"[c caller] tiny shape T={T}")
    w = synth.workload("tiny", T=T)
    d = synth.make_inputs("tiny", 0, device=DEV)
    x = synth.make_x(w, 0, DEV)
    for name, t in (("x", x), ("w_router", d["w_router"]), ("w_gate_up", d["w_gate_up"]),
                    ("w_down", d["w_down"])):
        _bits(t).tofile(tmp_path / f"{name}.bin")
    src = tmp_path / "caller.c"
    src.write_text(C_SOURCE)
    exe = tmp_path / "caller"
    r = subprocess.run([gcc, "-std=c99", "-Wall", "-Werror", str(src), "-I",
                        os.path.join(ROOT, "include"), "-L", LIBDIR, "-lbeam_moe",
                        "-L/opt/rocm/lib", "-lamdhip64", "-Wl,-rpath," + LIBDIR,
                        "-Wl,-rpath,/opt/rocm/lib", "-o", str(exe)],
                       capture_output=True, text=True)
    assert r.returncode == 0, r.stderr
    H, I = w.H, w.I
    r = subprocess.run([str(exe), str(tmp_path), str(T), str(H), str(I)], capture_output=True,
                       text=True, timeout=120)
    say("  " + r.stdout.strip().replace("\n", " | "))
    assert r.returncode == 0, r.stdout + r.stderr
    out = np.fromfile(tmp_path / "out.bin", dtype=np.uint16).reshape(T, H)
    ids = np.fromfile(tmp_path / "ids.bin", dtype=np.int32).reshape(T, 8)
    wts = np.fromfile(tmp_path / "w.bin", dtype=np.float32).reshape(T, 8)
    # the same bits as the Python binding's call on the same inputs
    pout, pids, pw = gtr.layer_forward(x, d["w_router"], d["w_gate_up"], d["w_down"],
                                       return_routing=True)
    torch.cuda.synchronize()
    assert np.array_equal(out, _bits(pout))
    assert np.array_equal(ids, _bits(pids)) and np.array_equal(wts, _bits(pw))
    # and the oracle's block
    xn = to_np(x)
    npw = {k: to_np(d[k]) for k in ("w_router", "w_gate_up", "w_down")}
    ref = oracle.layer_forward(xn, npw["w_router"], (npw["w_gate_up"], npw["w_down"]))
    nf, nd = check_routing(ids, wts, ref["route"])
    outf = (out.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    assert_close(outf, layer_reference(ids, ref, xn, (npw["w_gate_up"], npw["w_down"])),
                 f"C caller output T={T}")
    say(f"  flagged={nf} differing={nd}")
