#!/usr/bin/env python3
"""Benchmark of the Beam-1.0 MoE block on one MI355X.

One step = one pass of the whole block (router GEMM + sigmoid + group-limited
top-8, permutation, gate/up grouped GEMM with fused SwiGLU, down grouped GEMM,
weighted combine x2.5) over one batch of synthetic tokens: one call of the C
ABI's moe_layer_forward.  The same block is also run as its five separate
calls with HIP events between them, for per-stage and per-kernel times.
Inputs and all ~20 GB of expert weights are generated on the device before
timing and stay resident in HBM.

Prints ONE JSON line.  `value` is tokens/s of the prefill chunk (T=4096,
hidden 5120, intermediate 2560, 256 experts); `roofline` describes the
dominant kernel (the gate/up grouped GEMM), timed with HIP events on the
stream it runs on; `decode` reports the weight-streaming T=32 batch in GB/s;
`fp8` times the same layer with FP8 per-channel expert weights (prefill and
decode); `lora` times it with rank-16 expert LoRA adapters; `cpu_baseline` times the CPU oracle on a bounded sample of the same
workload.
"""
from __future__ import annotations

import argparse
import json
import os
import subprocess
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E
BF16_PEAK_TFLOPS = 2516.6      # MI355X dense bf16 MFMA (256 CU x 2.4 GHz x 4096 FLOP/clk)


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=20)
    p.add_argument("--warmup", type=int, default=5)
    p.add_argument("--workload", default="prefill", choices=["decode", "mid", "prefill", "skew"])
    p.add_argument("--seed", type=int, default=0)
    p.add_argument("--no-decode", action="store_true", help="skip the T=32 decode measurement")
    p.add_argument("--no-other-workloads", action="store_true",
                   help="skip the T=512 and skewed T=16384 measurements")
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--no-fp8", action="store_true", help="skip the FP8-weight variant")
    p.add_argument("--no-lora", action="store_true", help="skip the expert-LoRA variant")
    p.add_argument("--no-attainable", action="store_true",
                   help="skip the torch copy / matmul reference points")
    p.add_argument("--cpu-experts", type=int, default=256,
                   help="experts whose rows the CPU oracle processes in its timed sample")
    p.add_argument("--no-row-major-ref", action="store_true",
                   help="skip the reference timing with row-major weights (profiling runs)")
    p.add_argument("--no-parity", action="store_true",
                   help="skip the oracle comparison of the decode, mid and skewed outputs")
    p.add_argument("--decode-seeds", type=int, default=4,
                   help="seeds of the decode batch to time (the touched-expert count varies)")
    p.add_argument("--copy-calibration-gib", type=float, default=0.0,
                   help="run one device-to-device copy of this size first (a known byte "
                        "count for scaling hardware byte counters)")
    return p.parse_args()


def git_sha():
    """The commit the library was built from (recorded by the build next to
    the library; a snapshot without .git has no other source), and whether the
    tree had uncommitted changes then."""
    info = {}
    try:
        with open(os.path.join(ROOT, "grouped_top_routing_amd", "_build_info.json")) as f:
            info = json.load(f)
    except (OSError, ValueError):
        pass
    if not info.get("git"):
        try:
            sha = subprocess.run(["git", "rev-parse", "--short=12", "HEAD"], cwd=ROOT,
                                 capture_output=True, text=True, timeout=10).stdout.strip()
            info = {"git": sha or None, "source": "git at run time"}
        except Exception:
            pass
    return info or None


PROFILE = os.path.join(ROOT, "profiles", "grouped_gemm_prefill_T4096.md")


def kernel_source_sha256():
    """Hash of the grouped GEMM's sources with `//` comments and blank lines
    removed (comment edits do not change what the counters measured)."""
    import hashlib
    import re
    code = []
    for f in ("ffn.hip", "common.h", "half_ring.h", "item_order.h"):
        with open(os.path.join(ROOT, "grouped_top_routing_amd", "csrc", f)) as fh:
            for line in fh:
                line = re.sub(r"//.*", "", line).rstrip()
                if line:
                    code.append(line)
    return hashlib.sha256("\n".join(code).encode()).hexdigest()


def measured_traffic(kernel):
    """HBM bytes per launch of `kernel` ("gate_up" or "down") from the
    committed rocprofv3 counter runs (FETCH_SIZE and WRITE_SIZE, each scaled
    by the same counter's reading for a 1 GiB copy), or None when the kernel
    source changed since they were taken or the summary is missing."""
    try:
        text = open(PROFILE).read()
        blob = json.loads(text.split("```json", 1)[1].split("```", 1)[0])
        if kernel_source_sha256() != blob["kernel_source_sha256"]:
            return None
        return int(blob[kernel]["read_bytes"] + blob[kernel]["write_bytes"])
    except (OSError, IndexError, KeyError, ValueError):
        return None


def algorithmic(w, counts, fmt="bf16"):
    """Algorithmic HBM bytes and MFMA FLOPs of one layer call (and of the
    gate/up kernel alone) from the realised routing histogram.  fp8 weights
    are one byte per element plus an fp32 scale per row."""
    touched = int((counts > 0).sum())
    T, H, I, K = w.T, w.H, w.I, w.K
    if fmt == "fp8":
        b_expert = 3 * H * I + (2 * I + H) * 4    # codes + per-row scales
        b_gu = 2 * I * H + 2 * I * 4
    else:
        b_expert = 3 * H * I * 2                  # gate, up, down rows of one expert, bf16
        b_gu = 2 * I * H * 2
    b_dn = b_expert - b_gu
    layer_bytes = touched * b_expert + w.E * H * 4 + T * H * 2 + T * H * 2
    # per kernel: the weights it streams (+ the x rows the gate/up kernel
    # gathers); the intermediates h and y_perm are implementation traffic
    gu_bytes = touched * b_gu + T * H * 2
    dn_bytes = touched * b_dn
    flops = K * T * 2 * 3 * H * I
    return {"touched": touched, "layer_bytes": layer_bytes, "gate_up_bytes": gu_bytes,
            "down_bytes": dn_bytes, "expert_flops": flops,
            "gate_up_flops": K * T * 2 * 2 * H * I, "down_flops": K * T * 2 * H * I}


def run_workload(name, wts, args, steps, warmup, gtr, synth, torch, fmt="bf16", rowmajor=True,
                 seed=None, layer_ref=True):
    """Times `steps` staged layer passes; returns timing dict and routing.
    fmt "bf16": fragment-packed bf16 expert weights; "fp8": E4M3FN codes
    with per-row scales."""
    dev = wts["dev"]
    w = synth.workload(name)
    x = synth.make_x(w, args.seed if seed is None else seed, dev, w_router=wts["w_router"])
    wr, wgu, wd = wts["w_router"], wts["p_gate_up"], wts["p_down"]
    lay = gtr.LAYOUT_PACKED
    ws = gtr.Workspace()
    f8 = wts.get("fp8")
    if fmt == "fp8":
        gate_up = lambda x, ps, o: gtr.expert_gate_up_fp8(x, ps, o, f8, workspace=ws)
        down = lambda h, o: gtr.expert_down_fp8(h, o, f8, workspace=ws)
    else:
        gate_up = lambda x, ps, o: gtr.expert_gate_up(x, ps, o, wgu, weight_layout=lay,
                                                      workspace=ws)
        down = lambda h, o: gtr.expert_down(h, o, wd, weight_layout=lay, workspace=ws)

    if fmt == "fp8":
        layer = lambda: gtr.layer_forward_fp8(x, wr, f8, workspace=ws, return_routing=True)
    else:
        layer = lambda: gtr.layer_forward(x, wr, wgu, wd, weight_layout=lay, workspace=ws,
                                          return_routing=True)

    # The timed step: the whole block as one call of the product's entry point
    # (moe_layer_forward), `warmup` untimed calls, then `steps` calls bracketed
    # by synchronisations.
    for _ in range(warmup):
        layer()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(steps):
        out, ids, topw = layer()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0

    # The same block as its five calls with HIP events between them (on the
    # stream the library runs on): per-stage and per-kernel times.
    def step(ev=None):
        if ev is not None:
            ev[0].record()
        ids, tw = gtr.route(x, wr, workspace=ws)
        if ev is not None:
            ev[1].record()
        c, o, ps, pd = gtr.permute(ids, workspace=ws)
        if ev is not None:
            ev[2].record()
        h = gate_up(x, ps, o)
        if ev is not None:
            ev[3].record()
        y = down(h, o)
        if ev is not None:
            ev[4].record()
        out = gtr.combine(y, pd, tw)
        if ev is not None:
            ev[5].record()
        return out, ids, c, tw

    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(6)] for _ in range(steps)]
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    for i in range(steps):
        s_out, s_ids, counts, s_topw = step(evs[i])
    torch.cuda.synchronize()
    staged_wall = time.perf_counter() - t1
    # both forms compute the same bits (reported, never assumed)
    same_bits = bool(torch.equal(s_out, out) and torch.equal(s_ids, ids)
                     and torch.equal(s_topw, topw))
    del s_out, s_ids, s_topw
    names = ["route", "permute", "gate_up", "down", "combine"]
    stage = {n: sum(evs[i][j].elapsed_time(evs[i][j + 1]) for i in range(steps)) / steps
             for j, n in enumerate(names)}
    # device time of each step (first to last event of the step)
    per_step = sorted(evs[i][0].elapsed_time(evs[i][5]) for i in range(steps))
    pct = lambda q: per_step[min(len(per_step) - 1, int(q * (len(per_step) - 1) + 0.5))]
    # the single-call entry point with row-major expert weights, for reference
    def time_layer(a, b, layout):
        for _ in range(2):
            gtr.layer_forward(x, wr, a, b, weight_layout=layout, workspace=ws)
        torch.cuda.synchronize()
        t1 = time.perf_counter()
        for _ in range(steps):
            gtr.layer_forward(x, wr, a, b, weight_layout=layout, workspace=ws)
        torch.cuda.synchronize()
        return (time.perf_counter() - t1) * 1e3 / steps
    rowmajor_ms = (None if not layer_ref or fmt == "fp8" or args.no_row_major_ref or not rowmajor
                   else time_layer(wts["w_gate_up"], wts["w_down"], gtr.LAYOUT_ROW_MAJOR))
    layer_ms = wall * 1e3 / steps
    return {"w": w, "x": x, "ms_per_step": layer_ms, "stage_ms": stage,
            "staged_ms_per_step": staged_wall * 1e3 / steps, "staged_equals_layer": same_bits,
            "device_step_ms": {"p10": pct(0.1), "p50": pct(0.5), "p90": pct(0.9)},
            "layer_forward_ms": layer_ms, "row_major_layer_ms": rowmajor_ms,
            "counts": counts.cpu().numpy(), "ids": ids, "out": out, "topw": topw}


def expert_host(wts, e):
    """Expert e's bf16 weights on the host as fp64 (exact), moving 2 bytes per
    element: (gate_up [2I, H], down [H, I])."""
    import numpy as np

    def conv(t):
        import torch
        u = t.contiguous().view(torch.int16).cpu().numpy().view(np.uint16).astype(np.uint32)
        return (u << 16).view(np.float32).astype(np.float64)
    return conv(wts["w_gate_up"][e]), conv(wts["w_down"][e])


def tolerance_stats(y, r):
    """max |y - r| / max(|r|, RMS(r)) and mean |y - r| / RMS(r) (the layer
    output tolerance: 2e-2 and 5e-3)."""
    import numpy as np
    rms = float(np.sqrt(np.mean(r * r)))
    d = np.abs(y - r)
    return float(np.max(d / np.maximum(np.abs(r), rms))), float(np.mean(d) / rms)


def layer_parity(wl, x, out, ids, wts, sample=None, seed=0):
    """The timed GPU layer output against the oracle on the same input:
    routing of every token (expert sets; tokens inside the oracle's 1e-5
    selection margin may differ), then the output over every token, or over
    `sample` tokens drawn with `seed`, evaluated by the oracle expert by
    expert on the GPU's expert sets (identical to the oracle's outside the
    margin) with the oracle's own scores."""
    import numpy as np
    import oracle
    xn = x.float().cpu().numpy()
    wr = wts["w_router"].cpu().numpy()
    t0 = time.perf_counter()
    rr = oracle.route(xn, wr)
    t_route = time.perf_counter() - t0
    gid = ids.cpu().numpy().astype(np.int64)
    same = np.all(np.sort(gid, 1) == np.sort(rr.ids, 1), axis=1)
    flagged = rr.margin < oracle.MARGIN_TOL
    T = xn.shape[0]
    toks = (np.arange(T) if sample is None or sample >= T else
            np.sort(np.random.default_rng(seed).choice(T, sample, replace=False)))
    s = rr.scores[toks][np.arange(len(toks))[:, None], gid[toks]].astype(np.float64)
    wgt = s / s.sum(axis=1, keepdims=True)
    ref = np.zeros((len(toks), xn.shape[1]))
    t_ffn = 0.0  # the oracle's expert MLPs and combine, without the weight copies to the host
    for e in np.unique(gid[toks]):
        rows, slots = np.nonzero(gid[toks] == e)
        gu, dn = expert_host(wts, int(e))
        t0 = time.perf_counter()
        ref[rows] += wgt[rows, slots][:, None] * oracle.ffn_rows(xn[toks[rows]], gu, dn)
        t_ffn += time.perf_counter() - t0
    ref *= 2.5
    mx, mn = tolerance_stats(out.float().cpu().numpy()[toks].astype(np.float64), ref)
    return {"tokens": int(T), "output_tokens_compared": int(len(toks)),
            "routing_sets_differing": int((~same).sum()),
            "differing_outside_margin": int((~same & ~flagged).sum()),
            "margin_flagged": int(flagged.sum()), "max_rel": mx, "mean_rel": mn,
            "within_tolerance": bool(mx <= 2e-2 and mn <= 5e-3 and not (~same & ~flagged).any()),
            # the oracle on the host cores: routing of every token, expert MLPs
            # and combine of the compared tokens
            "oracle_seconds": {"route_all_tokens": round(t_route, 3),
                               "expert_mlps_compared_tokens": round(t_ffn, 3),
                               "cores": os.cpu_count()}}


def cpu_baseline(w, x, wts, n_experts, torch, gpu_out=None, gpu_ids=None):
    """The oracle as it stands, timed on this host's cores: routing and
    permutation of every token, then the SwiGLU MLPs of the first `n_experts`
    experts with all their rows (each expert's weights are copied to the host
    outside the timed region), then the combine; when only some experts are
    run, expert time is scaled by rows to the whole layer."""
    import numpy as np
    import oracle
    blas = None
    try:
        from threadpoolctl import threadpool_info
        libs = [i for i in threadpool_info() if i.get("user_api") == "blas"]
        threads = max([i.get("num_threads", 1) for i in libs] or [1])
        if libs:
            blas = {"library": libs[0].get("internal_api"), "version": libs[0].get("version"),
                    "threads": libs[0].get("num_threads")}
    except Exception:
        threads = os.cpu_count()
    xn = x.float().cpu().numpy()
    wrn = wts["w_router"].cpu().numpy()
    t0 = time.perf_counter()
    rr = oracle.route(xn, wrn)
    counts, offsets, psrc, pdst = oracle.permute(rr.ids, w.E)
    t_route = time.perf_counter() - t0
    rows, t_ffn = 0, 0.0
    y = np.zeros((w.K * w.T, w.H))
    for e in range(min(n_experts, w.E)):
        r0, r1 = int(offsets[e]), int(offsets[e + 1])
        if r1 == r0:
            continue
        gu, dn = expert_host(wts, e)
        t1 = time.perf_counter()
        y[r0:r1] = oracle.ffn_rows(xn[psrc[r0:r1] // w.K], gu, dn)
        t_ffn += time.perf_counter() - t1
        rows += r1 - r0
    t2 = time.perf_counter()
    ref = oracle.combine(y, pdst, rr.weights, 2.5)
    t_comb = time.perf_counter() - t2
    est = t_route + t_ffn * (w.K * w.T) / max(rows, 1) + t_comb
    whole = rows == w.K * w.T
    return {"value": w.T / est, "unit": "tokens/s", "cores": int(threads), "kind": "oracle",
            "sample": (f"the whole {w.T}-token layer" if whole else
                       f"routing of all {w.T} tokens + experts 0-{n_experts - 1} "
                       f"({rows} of {w.K * w.T} rows, scaled by rows)")
                      + f": route+permute {t_route:.2f} s, expert MLPs {t_ffn:.2f} s, combine "
                        f"{t_comb:.2f} s; fp64 NumPy/BLAS; host os.cpu_count()={os.cpu_count()}",
            "sample_seconds": round(t_route + t_ffn + t_comb, 2), "blas": blas,
            "parity": _parity(ref, rr, gpu_out, gpu_ids, rows == w.K * w.T, xn, wts)}


def _parity(ref, rr, gpu_out, gpu_ids, whole, xn, wts):
    """The timed GPU output against this oracle run, for the same input:
    routing sets (tokens within the oracle's selection margin may
    legitimately differ; such a token's reference is the oracle evaluated on
    the GPU's set) and the layer-output statistics max |y - r| / max(|r|, RMS)
    and mean |y - r| / RMS over every token."""
    import numpy as np
    import oracle
    if gpu_out is None or gpu_ids is None or not whole:
        return None
    gid = gpu_ids.cpu().numpy().astype(np.int64)
    same = np.all(np.sort(gid, 1) == np.sort(rr.ids, 1), axis=1)
    flagged = rr.margin < oracle.MARGIN_TOL
    ref = np.array(ref, copy=True)
    for t in np.nonzero(~same)[0]:
        S = gid[t]
        sc = rr.scores[t, S].astype(np.float64)
        acc = np.zeros(ref.shape[1])
        for j, e in enumerate(S):
            gu, dn = expert_host(wts, int(e))
            acc += sc[j] / sc.sum() * oracle.ffn_rows(xn[t:t + 1], gu, dn)[0]
        ref[t] = 2.5 * acc
    mx, mn = tolerance_stats(gpu_out.float().cpu().numpy().astype(np.float64), ref)
    return {"tokens": int(gid.shape[0]), "output_tokens_compared": int(gid.shape[0]),
            "routing_sets_differing": int((~same).sum()),
            "differing_outside_margin": int((~same & ~flagged).sum()),
            "margin_flagged": int(flagged.sum()), "max_rel": mx, "mean_rel": mn,
            "within_tolerance": bool(mx <= 2e-2 and mn <= 5e-3 and not (~same & ~flagged).any())}


def kernel_roofline(kernel, alg, stage_ms, workload):
    """Roofline of one grouped-GEMM launch: algorithmic bytes (the weights of
    the touched experts it streams, plus the gathered x rows for gate/up) over
    its average launch time from HIP events on the stream it runs on.  Bound
    by HBM while the FLOPs per byte stay under the ridge (~315), else by the
    bf16 matrix cores."""
    ms = stage_ms[kernel]
    nbytes, flops = alg[f"{kernel}_bytes"], alg[f"{kernel}_flops"]
    hbm = nbytes / (ms * 1e-3) / 1e9
    tf = flops / (ms * 1e-3) / 1e12
    mfma = flops / nbytes > BF16_PEAK_TFLOPS * 1e12 / (HBM_PEAK_GBS * 1e9)
    inst = "gate/up + SwiGLU" if kernel == "gate_up" else "down"
    return {"kernel": f"beam::stream_gemm_kernel, {inst} instance",
            "bound": "mfma" if mfma else "hbm",
            "achieved": round(tf if mfma else hbm, 1),
            "peak": BF16_PEAK_TFLOPS if mfma else HBM_PEAK_GBS,
            "unit": "TFLOP/s" if mfma else "GB/s",
            "frac": round((tf / BF16_PEAK_TFLOPS) if mfma else (hbm / HBM_PEAK_GBS), 4),
            "traffic": measured_traffic(kernel) if workload == "prefill" else None,
            "bytes_per_launch": nbytes, "flops_per_launch": flops,
            "avg_launch_ms": round(ms, 4), "hbm_gbs": round(hbm, 1), "tflops": round(tf, 1)}


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py: the MoE block runs on exactly one GPU (asked for --gpus {args.gpus}); "
              "it is not sharded across GPUs.", file=sys.stderr)
        sys.exit(2)
    import numpy as np
    import torch

    import grouped_top_routing_amd as gtr
    import synth

    if not torch.cuda.is_available():
        print("bench.py: no HIP device visible", file=sys.stderr)
        sys.exit(3)
    gtr.lib()  # fail loudly if the HIP library is missing
    dev = torch.device("cuda", 0)
    beam = synth.workload("prefill")
    print(f"[bench] generating router + 256 experts ({3 * beam.H * beam.I * 2 * beam.E / 1e9:.1f} GB "
          f"bf16) on {torch.cuda.get_device_name(dev)}", file=sys.stderr, flush=True)
    wts = {"dev": dev, "w_router": synth.make_router(beam, args.seed, dev)}
    wts["w_gate_up"], wts["w_down"] = synth.make_experts(beam, args.seed, dev)
    # the library's fragment-packed weight layout, written once at load time
    wts["p_gate_up"], wts["p_down"] = gtr.pack_weights(wts["w_gate_up"], wts["w_down"])
    torch.cuda.synchronize()

    if args.copy_calibration_gib > 0:
        n = int(args.copy_calibration_gib * (1 << 30))
        src = torch.empty(n, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst
    print(f"[bench] timing {args.workload}: warmup {args.warmup}, steps {args.steps}",
          file=sys.stderr, flush=True)
    r = run_workload(args.workload, wts, args, args.steps, args.warmup, gtr, synth, torch)
    w = r["w"]
    alg = algorithmic(w, r["counts"])
    ms = r["ms_per_step"]
    gu_ms = r["stage_ms"]["gate_up"]
    layer_gbs = alg["layer_bytes"] / (ms * 1e-3) / 1e9
    mfma_frac = alg["expert_flops"] / (ms * 1e-3) / (BF16_PEAK_TFLOPS * 1e12)
    c = r["counts"]
    result = {
        "metric": "Beam MoE layer tokens/s at T=4096; % bf16 MFMA peak; decode HBM GB/s",
        "value": round(w.T / (ms * 1e-3), 1),
        "unit": "tokens/s",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": round(ms, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded counter-based generator; random-init weights)",
        "config": {"workload": f"{w.name}: T={w.T} hidden={w.H} intermediate={w.I} experts={w.E} "
                               f"groups={w.G} kept={w.KG} topk={w.K}",
                   "tokens": w.T, "hidden": w.H, "intermediate": w.I, "experts": w.E,
                   "seed": args.seed},
        "roofline": kernel_roofline("gate_up", alg, r["stage_ms"], w.name),
        "roofline_down": kernel_roofline("down", alg, r["stage_ms"], w.name),
        "layer": {"hbm_gbs": round(layer_gbs, 1), "hbm_frac": round(layer_gbs / HBM_PEAK_GBS, 4),
                  "roofline_frac": round(max(layer_gbs / HBM_PEAK_GBS, mfma_frac), 4),
                  "device_step_ms": {k: round(v, 4) for k, v in r["device_step_ms"].items()},
                  "bf16_mfma_frac": round(mfma_frac, 4), "algorithmic_bytes": alg["layer_bytes"],
                  "expert_flops": alg["expert_flops"], "touched_experts": alg["touched"],
                  "layer_forward_ms": round(r["layer_forward_ms"], 4),
                  "staged_ms_per_step": round(r["staged_ms_per_step"], 4),
                  "staged_equals_layer": r["staged_equals_layer"],
                  "row_major_weights_layer_ms": (None if r["row_major_layer_ms"] is None
                                                 else round(r["row_major_layer_ms"], 4)),
                  "weight_layout": "packed (moe_pack_weights, once at load)",
                  "stage_ms": {k: round(v, 4) for k, v in r["stage_ms"].items()},
                  "histogram": {"max": int(c.max()), "min": int(c.min()),
                                "lt10": int((c < 10).sum()), "empty": int((c == 0).sum())}},
        "git": git_sha(),
    }
    if not args.no_attainable:
        # reference points measured with torch's own kernels (not this library):
        # a device-to-device copy and a large bf16 matmul
        a = torch.empty(1 << 31, dtype=torch.uint8, device=dev)
        b = torch.empty_like(a)
        m = torch.randn(8192, 8192, device=dev).to(torch.bfloat16)
        for _ in range(2):
            b.copy_(a)
            torch.matmul(m, m)
        torch.cuda.synchronize()
        e = [torch.cuda.Event(enable_timing=True) for _ in range(4)]
        e[0].record()
        for _ in range(5):
            b.copy_(a)
        e[1].record()
        for _ in range(5):
            torch.matmul(m, m)
        e[2].record()
        torch.cuda.synchronize()
        copy_ms = e[0].elapsed_time(e[1]) / 5
        mm_ms = e[1].elapsed_time(e[2]) / 5
        result["attainable_reference"] = {
            "torch_copy_gbs_read_plus_write": round(2 * a.numel() / (copy_ms * 1e-3) / 1e9, 1),
            "torch_bf16_matmul_8192_tflops": round(2 * 8192 ** 3 / (mm_ms * 1e-3) / 1e12, 1)}
        del a, b, m
    if not args.no_decode and args.workload != "decode":
        print("[bench] timing decode T=32", file=sys.stderr, flush=True)
        d = run_workload("decode", wts, args, max(args.steps, 10), 3, gtr, synth, torch)
        da = algorithmic(d["w"], d["counts"])
        result["decode"] = {"tokens": d["w"].T, "ms_per_step": round(d["ms_per_step"], 4),
                            "hbm_gbs": round(da["layer_bytes"] / (d["ms_per_step"] * 1e-3) / 1e9, 1),
                            "hbm_frac": round(da["layer_bytes"] / (d["ms_per_step"] * 1e-3) / 1e9
                                              / HBM_PEAK_GBS, 4),
                            "touched_experts": da["touched"],
                            "stage_ms": {k: round(v, 4) for k, v in d["stage_ms"].items()},
                            "roofline_gate_up": kernel_roofline("gate_up", da, d["stage_ms"], "decode")}
        if not args.no_parity:
            print("[bench] decode parity against the oracle", file=sys.stderr, flush=True)
            result["decode"]["parity"] = layer_parity(d["w"], d["x"], d["out"], d["ids"], wts)
        # the touched-expert count (and so the bytes streamed) varies with the
        # draw: the same batch size at other seeds
        per_seed = []
        for sd in range(args.seed + 1, args.seed + args.decode_seeds):
            ds = run_workload("decode", wts, args, max(args.steps, 10), 3, gtr, synth, torch,
                              seed=sd, layer_ref=False)
            dsa = algorithmic(ds["w"], ds["counts"])
            t_s = ds["ms_per_step"] * 1e-3
            per_seed.append({"seed": sd, "touched_experts": dsa["touched"],
                             "ms_per_step": round(ds["ms_per_step"], 4),
                             "tokens_per_s": round(ds["w"].T / t_s, 1),
                             "hbm_frac": round(dsa["layer_bytes"] / t_s / 1e9 / HBM_PEAK_GBS, 4)})
            del ds
        if per_seed:
            result["decode"]["other_seeds"] = per_seed
        del d
    if not args.no_other_workloads:
        # the other shapes of the layer's operating range: a 512-token batch
        # (HBM-bound) and a skewed 16K-token batch (MFMA-bound; inputs shifted
        # so that 16 hot experts gain +2.0 on their router logits)
        result["other_workloads"] = {}
        for name in [n for n in ("mid", "skew") if n != args.workload]:
            print(f"[bench] timing {name}", file=sys.stderr, flush=True)
            o = run_workload(name, wts, args, max(args.steps // 2, 5), 3, gtr, synth, torch,
                             rowmajor=False)
            oa = algorithmic(o["w"], o["counts"])
            t_s = o["ms_per_step"] * 1e-3
            result["other_workloads"][name] = {
                "tokens": o["w"].T, "ms_per_step": round(o["ms_per_step"], 4),
                "tokens_per_s": round(o["w"].T / t_s, 1),
                "hbm_frac": round(oa["layer_bytes"] / t_s / 1e9 / HBM_PEAK_GBS, 4),
                "bf16_mfma_frac": round(oa["expert_flops"] / t_s / 1e12 / BF16_PEAK_TFLOPS, 4),
                "roofline_frac": round(max(oa["layer_bytes"] / (HBM_PEAK_GBS * 1e9),
                                           oa["expert_flops"] / (BF16_PEAK_TFLOPS * 1e12)) / t_s, 4),
                "touched_experts": oa["touched"],
                "max_rows_per_expert": int(o["counts"].max()),
                "histogram": {"max": int(o["counts"].max()), "min": int(o["counts"].min()),
                              "lt10": int((o["counts"] < 10).sum()),
                              "empty": int((o["counts"] == 0).sum())},
                "roofline_gate_up": kernel_roofline("gate_up", oa, o["stage_ms"], name),
                "roofline_down": kernel_roofline("down", oa, o["stage_ms"], name),
                "stage_ms": {k: round(v, 4) for k, v in o["stage_ms"].items()}}
            if not args.no_parity:
                # every token of the 512-token batch; 1024 sampled tokens of the
                # 16K-token one (its routing is still checked for every token)
                print(f"[bench] {name} parity against the oracle", file=sys.stderr, flush=True)
                result["other_workloads"][name]["parity"] = layer_parity(
                    o["w"], o["x"], o["out"], o["ids"], wts,
                    sample=None if o["w"].T <= 4096 else 1024, seed=args.seed)
            del o
    if not args.no_fp8:
        # the FP8 per-channel variant of the same layer (weights quantised once
        # at load time); reported beside the bf16 headline, never in `value`
        print("[bench] quantising experts to fp8 and timing the fp8 variant", file=sys.stderr,
              flush=True)
        wts["fp8"] = gtr.quantize_fp8(wts["w_gate_up"], wts["w_down"])
        torch.cuda.synchronize()
        fp8 = {"weights": "E4M3FN codes + fp32 scale per output row; bf16 activations, "
                          "fp32 accumulation",
               "weight_bytes": wts["fp8"].nbytes()}
        for name in ([args.workload] + ([] if args.no_decode or args.workload == "decode"
                                        else ["decode"])):
            f = run_workload(name, wts, args, args.steps if name == args.workload
                             else max(args.steps, 10), 3, gtr, synth, torch, fmt="fp8")
            fa = algorithmic(f["w"], f["counts"], "fp8")
            fms, fgu = f["ms_per_step"], f["stage_ms"]["gate_up"]
            fp8[name] = {"tokens": f["w"].T, "ms_per_step": round(fms, 4),
                         "tokens_per_s": round(f["w"].T / (fms * 1e-3), 1),
                         "layer_hbm_gbs": round(fa["layer_bytes"] / (fms * 1e-3) / 1e9, 1),
                         "layer_hbm_frac": round(fa["layer_bytes"] / (fms * 1e-3) / 1e9
                                                 / HBM_PEAK_GBS, 4),
                         "gate_up_gbs": round(fa["gate_up_bytes"] / (fgu * 1e-3) / 1e9, 1),
                         "gate_up_frac": round(fa["gate_up_bytes"] / (fgu * 1e-3) / 1e9
                                               / HBM_PEAK_GBS, 4),
                         "layer_forward_ms": round(f["layer_forward_ms"], 4),
                         "stage_ms": {k: round(v, 4) for k, v in f["stage_ms"].items()}}
            del f
        result["fp8"] = fp8
    if not args.no_lora:
        # rank-16 expert LoRA (scale 32 / 16) on the packed bf16 experts
        print("[bench] timing expert LoRA (rank 16)", file=sys.stderr, flush=True)
        ad = synth.make_lora(beam, args.seed, dev, rank=16)
        lw = gtr.LoraWeights(*ad, scale=2.0)
        lo = {"rank": 16, "scale": 2.0, "adapter_bytes": sum(t.numel() * 2 for t in ad)}
        for name in ([args.workload] + ([] if args.no_decode or args.workload == "decode"
                                        else ["decode"])):
            wl = synth.workload(name)
            xl = synth.make_x(wl, args.seed, dev, w_router=wts["w_router"])
            ws = gtr.Workspace()
            call = lambda: gtr.layer_forward_lora(xl, wts["w_router"], wts["p_gate_up"],
                                                  wts["p_down"], lw,
                                                  weight_layout=gtr.LAYOUT_PACKED, workspace=ws)
            base = lambda: gtr.layer_forward(xl, wts["w_router"], wts["p_gate_up"],
                                             wts["p_down"], weight_layout=gtr.LAYOUT_PACKED,
                                             workspace=ws)
            n = args.steps if name == args.workload else max(args.steps, 10)
            res = {}
            for tag, fn in (("lora", call), ("base", base)):
                for _ in range(3):
                    fn()
                torch.cuda.synchronize()
                t1 = time.perf_counter()
                for _ in range(n):
                    fn()
                torch.cuda.synchronize()
                res[tag] = (time.perf_counter() - t1) * 1e3 / n
            lo[name] = {"tokens": wl.T, "layer_forward_ms": round(res["lora"], 4),
                        "tokens_per_s": round(wl.T / (res["lora"] * 1e-3), 1),
                        "overhead_vs_bf16_layer": round(res["lora"] / res["base"] - 1.0, 4)}
        result["lora"] = lo
        del ad, lw
    if not args.no_cpu_baseline:
        print("[bench] CPU oracle baseline", file=sys.stderr, flush=True)
        result["cpu_baseline"] = cpu_baseline(w, r["x"], wts, args.cpu_experts, torch,
                                              gpu_out=r["out"], gpu_ids=r["ids"])
    # the layer-output tolerance statistics of every workload in one place
    par = {}
    if result.get("decode", {}).get("parity"):
        par["decode"] = result["decode"]["parity"]
    for name, o in result.get("other_workloads", {}).items():
        if o.get("parity"):
            par[name] = o["parity"]
    if result.get("cpu_baseline", {}).get("parity"):
        par[w.name] = result["cpu_baseline"]["parity"]
    if par:
        result["parity"] = par
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
