"""Builds libbeam_moe.so in-tree with hipcc for gfx950.

Usage: python -m grouped_top_routing_amd.build   (or call build()).
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys
import tempfile

PKG = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(PKG, "csrc")
LIB = os.path.join(PKG, "libbeam_moe.so")
SOURCES = ["capi.hip", "route.hip", "permute.hip", "ffn.hip", "ffn_fp8.hip", "lora.hip", "combine.hip"]
ARCH = "gfx950"


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found: the HIP library cannot be built")


def _flags() -> list:
    return [f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC",
            # packed fp32 VALU ops stay off: plain fp32 arithmetic only
            "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
            "-Wno-unused-command-line-argument",
            "-I", os.path.join(os.path.dirname(PKG), "include")]


def _filtered(text: str) -> str:
    return "\n".join(l for l in text.splitlines() if "packed-fp32-ops" not in l)


def build(verbose: bool = False) -> str:
    """Compile every HIP source (one hipcc process per file, in parallel) and
    link them into one shared library; returns its path."""
    cc = hipcc()
    tmpdir = tempfile.mkdtemp(prefix="beam_moe_build_")
    try:
        procs = []
        for s in SOURCES:
            obj = os.path.join(tmpdir, s.replace(".hip", ".o"))
            cmd = [cc, *_flags(), "-c", os.path.join(CSRC, s), "-o", obj]
            if verbose:
                print(" ".join(cmd), flush=True)
            procs.append((s, obj, subprocess.Popen(cmd, stdout=subprocess.PIPE,
                                                   stderr=subprocess.STDOUT, text=True)))
        errors = []
        for s, obj, p in procs:
            out = _filtered(p.communicate()[0])
            if p.returncode != 0:
                errors.append(f"{s}: hipcc failed ({p.returncode}):\n{out}")
            elif verbose and out.strip():
                print(out)
        if errors:
            raise RuntimeError("\n".join(errors))
        tmp = LIB + ".tmp"
        cmd = [cc, f"--offload-arch={ARCH}", "-shared", "-fPIC", *[o for _, o, _ in procs],
               "-o", tmp]
        r = subprocess.run(cmd, capture_output=True, text=True)
        if r.returncode != 0:
            raise RuntimeError(f"link failed ({r.returncode}):\n{_filtered(r.stdout + r.stderr)}")
        os.replace(tmp, LIB)
    finally:
        shutil.rmtree(tmpdir, ignore_errors=True)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
