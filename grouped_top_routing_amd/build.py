"""Builds libbeam_moe.so in-tree with hipcc for gfx950.

Usage: python -m grouped_top_routing_amd.build [--normal | --checked | --sanitized]
(all three libraries by default; or call build() / build_all()).
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
# the debug build: kernels verify their derived indices (include/beam_moe_debug.h)
LIB_CHECKED = os.path.join(PKG, "libbeam_moe_checked.so")
# host code built with AddressSanitizer and UndefinedBehaviorSanitizer (the
# device code is the normal build's), for running the C ABI's host-side
# validation under the sanitizers
LIB_SANITIZED = os.path.join(PKG, "libbeam_moe_sanitized.so")


def clang_rt_dir() -> str:
    """Directory of the clang sanitizer runtimes that LIB_SANITIZED needs."""
    import glob
    hits = sorted(glob.glob("/opt/rocm/lib/llvm/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so"))
    if not hits:
        raise RuntimeError("clang's AddressSanitizer runtime was not found under /opt/rocm")
    return os.path.dirname(hits[-1])
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


def build(verbose: bool = False, checked: bool = False, sanitized: bool = False) -> str:
    """Compile every HIP source (one hipcc process per file, in parallel) and
    link them into one shared library; returns its path.  checked: the debug
    library with the kernels' index checks (BEAM_MOE_CHECKED=1); sanitized:
    host code under AddressSanitizer and UndefinedBehaviorSanitizer."""
    cc = hipcc()
    lib = LIB_CHECKED if checked else LIB_SANITIZED if sanitized else LIB
    extra = ["-DBEAM_MOE_CHECKED=1"] if checked else []
    if sanitized:
        # each sanitizer flag applies to the host compilation only
        extra = ["-g", "-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
                 "-Xarch_host", "-fno-omit-frame-pointer"]
    tmpdir = tempfile.mkdtemp(prefix="beam_moe_build_")
    try:
        procs = []
        for s in SOURCES:
            obj = os.path.join(tmpdir, s.replace(".hip", ".o"))
            cmd = [cc, *_flags(), *extra, "-c", os.path.join(CSRC, s), "-o", obj]
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
        tmp = lib + ".tmp"
        cmd = [cc, f"--offload-arch={ARCH}", "-shared", "-fPIC", *[o for _, o, _ in procs],
               "-o", tmp]
        if sanitized:
            # the host link with the shared sanitizer runtimes
            cmd = [os.path.join(os.path.dirname(cc), "..", "llvm", "bin", "clang++"), "-shared",
                   "-fPIC", "-fsanitize=address,undefined", "-shared-libasan",
                   *[o for _, o, _ in procs], "-L/opt/rocm/lib", "-lamdhip64",
                   "-Wl,-rpath,/opt/rocm/lib", "-o", tmp]
        r = subprocess.run(cmd, capture_output=True, text=True)
        if r.returncode != 0:
            raise RuntimeError(f"link failed ({r.returncode}):\n{_filtered(r.stdout + r.stderr)}")
        os.replace(tmp, lib)
        if not checked and not sanitized:
            _write_build_info()
    finally:
        shutil.rmtree(tmpdir, ignore_errors=True)
    return lib


def build_all(verbose: bool = False) -> list:
    """The three libraries (normal, checked, sanitized), compiled concurrently."""
    from concurrent.futures import ThreadPoolExecutor
    with ThreadPoolExecutor(3) as pool:
        futs = [pool.submit(build, verbose, c, z) for c, z in ((False, False), (True, False),
                                                                 (False, True))]
        return [f.result() for f in futs]


def _write_build_info() -> None:
    """Records, next to the library, the commit it was built from and whether
    the tree had uncommitted changes (a copy of the tree without .git can
    still name its build)."""
    import hashlib
    import json
    root = os.path.dirname(PKG)
    info = {"git": None, "dirty": None,
            "sources_sha256": hashlib.sha256(b"".join(
                open(os.path.join(CSRC, f), "rb").read() for f in sorted(os.listdir(CSRC))
            )).hexdigest()}
    try:
        sha = subprocess.run(["git", "rev-parse", "--short=12", "HEAD"], cwd=root,
                             capture_output=True, text=True, timeout=10)
        if sha.returncode == 0:
            info["git"] = sha.stdout.strip()
            st = subprocess.run(["git", "status", "--porcelain", "--untracked-files=no"],
                                cwd=root, capture_output=True, text=True, timeout=10)
            info["dirty"] = bool(st.stdout.strip())
    except (OSError, subprocess.SubprocessError):
        pass
    with open(os.path.join(PKG, "_build_info.json"), "w") as f:
        json.dump(info, f)


if __name__ == "__main__":
    if "--checked" in sys.argv:
        print(build(verbose="-v" in sys.argv, checked=True))
    elif "--sanitized" in sys.argv:
        print(build(verbose="-v" in sys.argv, sanitized=True))
    elif "--normal" in sys.argv:
        print(build(verbose="-v" in sys.argv))
    else:
        print("\n".join(build_all(verbose="-v" in sys.argv)))
