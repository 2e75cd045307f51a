"""Helpers shared by the GPU parity tests (test infrastructure only)."""
from __future__ import annotations

import sys

import numpy as np
import torch

import oracle

#: Layer-output tolerance: max |y - r| / max(|r|, RMS(r)) and mean |y - r| / RMS(r).
MAX_REL = 2e-2
MEAN_REL = 5e-3


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def err_stats(y, r):
    y = np.asarray(y, dtype=np.float64)
    r = np.asarray(r, dtype=np.float64)
    rms = float(np.sqrt(np.mean(r * r))) if r.size else 0.0
    if r.size == 0 or rms == 0.0:
        return 0.0, 0.0, rms
    d = np.abs(y - r)
    return float(np.max(d / np.maximum(np.abs(r), rms))), float(np.mean(d) / rms), rms


def assert_close(y, r, what, max_rel=MAX_REL, mean_rel=MEAN_REL):
    mx, mn, rms = err_stats(y, r)
    say(f"  {what}: max_rel={mx:.3e} mean_rel={mn:.3e} rms={rms:.3e}")
    assert mx <= max_rel, f"{what}: max relative error {mx:.3e} > {max_rel}"
    assert mn <= mean_rel, f"{what}: mean abs error {mn:.3e} > {mean_rel} * RMS"
    return mx, mn


def to_np(t):
    if t.dtype == torch.bfloat16:
        t = t.float()
    return t.detach().cpu().numpy()


def check_routing(ids_gpu, w_gpu, rr, *, n_groups=8, topk_groups=4, topk=8, w_rtol=1e-5):
    """Routing parity: chosen-expert sets bit-exact for tokens whose oracle
    margin is at least MARGIN_TOL; flagged tokens must be admissible.  Sets are
    compared (the order inside a set follows values that may sit closer than
    fp32 rounding); weights are compared expert by expert.  Returns
    (n_flagged, n_flagged_differing)."""
    ids_gpu = np.asarray(ids_gpu).astype(np.int64)
    w_gpu = np.asarray(w_gpu, dtype=np.float64)
    flagged = rr.margin < oracle.MARGIN_TOL
    ok = ~flagged
    og, oo = np.argsort(ids_gpu, axis=1), np.argsort(rr.ids, axis=1)
    ids_gpu = np.take_along_axis(ids_gpu, og, 1)
    w_gpu = np.take_along_axis(w_gpu, og, 1)
    ids_ref = np.take_along_axis(rr.ids, oo, 1)
    w_ref = np.take_along_axis(rr.weights, oo, 1)
    same = np.all(ids_gpu == ids_ref, axis=1)
    bad = np.nonzero(ok & ~same)[0]
    assert bad.size == 0, f"{bad.size} unflagged tokens differ, first {bad[:5]}: " \
                          f"gpu {ids_gpu[bad[0]]} oracle {ids_ref[bad[0]]} margin {rr.margin[bad[0]]}"
    for t in np.nonzero(flagged & ~same)[0]:
        assert oracle.selection_admissible(rr.sel[t], rr.group_scores[t], ids_gpu[t],
                                           n_groups=n_groups, topk_groups=topk_groups,
                                           topk=topk), f"token {t}: inadmissible {ids_gpu[t]}"
    m = ok | same
    np.testing.assert_allclose(w_gpu[m], w_ref[m], rtol=w_rtol, atol=1e-7)
    return int(flagged.sum()), int((flagged & ~same).sum())


def layer_reference(ids_gpu, ref, x, experts, *, renormalize=True, scale=2.5):
    """The oracle's layer output, except that tokens whose GPU expert set
    differs from the oracle's (only allowed at a selection tie, see
    check_routing) are evaluated by the oracle on the GPU's set, with weights
    from the oracle's own scores."""
    out = np.array(ref["out"], copy=True)
    ids_gpu = np.asarray(ids_gpu).astype(np.int64)
    rr = ref["route"]
    get = experts if callable(experts) else (lambda e: (experts[0][e], experts[1][e]))
    for t in range(ids_gpu.shape[0]):
        S = ids_gpu[t]
        if set(S.tolist()) == set(rr.ids[t].tolist()):
            continue
        s = rr.scores[t, S].astype(np.float64)
        wt = s / s.sum() if renormalize else s
        acc = np.zeros(out.shape[1])
        for j, e in enumerate(S):
            acc += wt[j] * oracle.ffn_rows(np.asarray(x)[t:t + 1], *get(int(e)))[0]
        out[t] = scale * acc
    return out


def unpack_fp8_codes(q):
    """Row-major [E, N, K] codes from the library's fp8 fragment layout
    ([N/16][K/64][2][64 lanes][8 bytes] per expert; entry (b, s, h, l) with
    l = r + 16g holds row 16b + r at k = 64s + 32h + 8g + j, j = 0..7)."""
    q = np.asarray(q, dtype=np.uint8)
    E, N, K = q.shape
    p = q.reshape(E, N // 16, K // 64, 2, 4, 16, 8)        # e, b, s, h, g, r, j
    return p.transpose(0, 1, 5, 2, 3, 4, 6).reshape(E, N, K)  # e, b, r, s, h, g, j


class OracleFp8Experts:
    """Expert weights as the oracle quantises them (from the bf16 weights),
    dequantised to fp64: a callable e -> (gate_up, down), cached per expert."""

    def __init__(self, w_gate_up, w_down):
        self._gu, self._dn = w_gate_up, w_down
        self._cache = {}

    def quantized(self, e):
        """((codes, scales) of gate_up, (codes, scales) of down) of expert e."""
        e = int(e)
        if e not in self._cache:
            gu = np.asarray(self._gu[e] if not callable(self._gu) else self._gu(e), np.float32)
            dn = np.asarray(self._dn[e] if not callable(self._dn) else self._dn(e), np.float32)
            self._cache[e] = (oracle.quantize_fp8_per_channel(gu),
                              oracle.quantize_fp8_per_channel(dn), {})
        return self._cache[e][:2]

    def __call__(self, e):
        (qg, sg), (qd, sd) = self.quantized(e)
        deq = self._cache[int(e)][2]
        if not deq:
            deq["w"] = (oracle.dequantize_fp8(qg, sg), oracle.dequantize_fp8(qd, sd))
        return deq["w"]
