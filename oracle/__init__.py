"""CPU oracle for the Beam-1.0 MoE block -- TEST INFRASTRUCTURE ONLY.

Plain, slow, obviously-correct NumPy implementation of what the layer computes,
used to check the HIP library.  Only the test-suite, the smoke entry point and
the benchmark's CPU-baseline leg may import it; the product path never does and
shares no code with it.

Sources (page titles and sections):

* "Welcome Beam: a 501B open model you can own, customize, and scale",
  section "Mixture of Experts": 256 SwiGLU experts of intermediate size 2,560;
  sigmoid scores over all 256 experts; 8 groups of 32; keep the 4 groups with
  the largest sum of their two best scores; top 8 experts inside them; no shared
  expert; each token's output is the sum of its chosen experts' outputs, each
  weighted by its score divided by the sum of the chosen scores, times 2.5.
  Same page, section "Residual Stream": the router and the SwiGLU product are
  computed in FP32.
* "Beam 1.0" (miles launch recipes), section 1 "Model Introduction": grouped
  top-8 sigmoid routing, no shared expert; router weights kept in FP32.
* vLLM recipe "Beam-1.0-501B-A23B", bf16 variant: native BF16 checkpoint with
  FP32 router weights and expert biases.

Precision: the router GEMM accumulates in fp64 and rounds once to fp32 (the
pages fix the router in FP32); sigmoid is evaluated in fp64 and rounded to fp32;
selection compares those fp32 values; the expert MLPs and the combine run in
fp64 with no intermediate rounding.

Readings taken where the pages are silent (each is mirrored by the HIP path and
listed in the design notes): groups are contiguous blocks of E/G experts; ties
break towards the lower group / expert index; a duplicated maximum counts twice
in a group's top-two sum; the fused gate/up weight is [E, 2I, H] with the gate
rows first and SiLU applied to the gate; the down weight is [E, H, I]; weights
are normalised over the k chosen unbiased scores before the 2.5 scale
(``renormalize`` switch); an optional per-expert selection bias is added to the
scores for choosing only (off by default).

Parity pins: every function here is checked in tests/test_oracle_*.py against
brute-force enumeration, textbook reductions, closed forms and invariants.
"""
from __future__ import annotations

from dataclasses import dataclass
from itertools import combinations

import numpy as np

__all__ = [
    "RouteResult", "route", "route_replay", "select", "router_logits", "sigmoid_f32",
    "permute", "expert_ffn", "ffn_rows", "combine", "layer_forward",
    "selection_admissible", "MARGIN_TOL", "E4M3_MAX", "e4m3_encode", "e4m3_decode",
    "quantize_fp8_per_channel", "dequantize_fp8", "LORA_RANK", "LORA_ALPHA", "lora_scale",
    "ffn_rows_lora",
]

#: Selection margin under which GPU and oracle may legitimately disagree.
MARGIN_TOL = 1e-5


@dataclass
class RouteResult:
    ids: np.ndarray          # [T, k] int64, ordered by (selection value desc, index asc)
    weights: np.ndarray      # [T, k] fp64 combine weights (before the routed scale)
    scores: np.ndarray       # [T, E] fp32 sigmoid scores
    sel: np.ndarray          # [T, E] fp32 selection values (scores + optional bias)
    group_scores: np.ndarray # [T, G] fp32 sum of each group's top-two selection values
    group_keep: np.ndarray   # [T, G] bool, the kept groups
    margin: np.ndarray       # [T] fp64 smallest gap at either selection cut
    logits: np.ndarray       # [T, E] fp32


def _f32(a):
    return np.asarray(a, dtype=np.float32)


def router_logits(x, w_router):
    """logits[t, e] = sum_h x[t, h] * W_r[e, h], accumulated in fp64, rounded once to fp32."""
    x64 = np.asarray(x, dtype=np.float64)
    w64 = np.asarray(w_router, dtype=np.float64)
    return (x64 @ w64.T).astype(np.float32)


def sigmoid_f32(logits):
    """s = 1 / (1 + exp(-logit)) evaluated in fp64, rounded once to fp32."""
    l64 = np.asarray(logits, dtype=np.float64)
    with np.errstate(over="ignore"):
        return (1.0 / (1.0 + np.exp(-l64))).astype(np.float32)


def select(sel, n_groups, topk_groups, topk):
    """Group-limited top-k on fp32 selection values ``sel`` [T, E].

    Returns (ids [T, k], group_scores [T, G] fp32, kept-group mask [T, G],
    margin [T])."""
    sel = _f32(sel)
    T, E = sel.shape
    gsize = E // n_groups
    grouped = sel.reshape(T, n_groups, gsize)
    # top two of each group (a duplicated maximum counts twice), summed in fp32
    top2 = -np.sort(-grouped, axis=2)[:, :, :2]
    gs = (top2[:, :, 0] + top2[:, :, 1]).astype(np.float32)
    # groups ranked by (score desc, index asc); keep the first topk_groups
    g_order = np.argsort(-gs, axis=1, kind="stable")
    keep = np.zeros((T, n_groups), dtype=bool)
    np.put_along_axis(keep, g_order[:, :topk_groups], True, axis=1)
    # experts outside kept groups can never be chosen
    eligible = np.repeat(keep, gsize, axis=1)
    cand = np.where(eligible, sel.astype(np.float64), -np.inf)
    e_order = np.argsort(-cand, axis=1, kind="stable")
    ids = e_order[:, :topk].astype(np.int64)
    # selection margin at both cuts (fp64 differences of fp32 values)
    gs_sorted = np.take_along_axis(gs.astype(np.float64), g_order, axis=1)
    if topk_groups < n_groups:
        g_margin = gs_sorted[:, topk_groups - 1] - gs_sorted[:, topk_groups]
    else:
        g_margin = np.full(T, np.inf)
    c_sorted = np.take_along_axis(cand, e_order, axis=1)
    if topk < topk_groups * gsize:
        e_margin = c_sorted[:, topk - 1] - c_sorted[:, topk]
    else:
        e_margin = np.full(T, np.inf)
    return ids, gs, keep, np.minimum(g_margin, e_margin)


def _weights(scores, ids, renormalize):
    r = np.take_along_axis(scores.astype(np.float64), ids, axis=1)
    if renormalize:
        r = r / r.sum(axis=1, keepdims=True)
    return r


def route(x, w_router, *, n_groups=8, topk_groups=4, topk=8, renormalize=True, sel_bias=None):
    """Router GEMM, sigmoid scoring, group-limited top-k and combine weights."""
    logits = router_logits(x, w_router)
    scores = sigmoid_f32(logits)
    sel = scores if sel_bias is None else (scores + _f32(sel_bias)[None, :]).astype(np.float32)
    ids, gs, keep, margin = select(sel, n_groups, topk_groups, topk)
    weights = _weights(scores, ids, renormalize)
    return RouteResult(ids, weights, scores, sel, gs, keep, margin, logits)


def route_replay(x, w_router, ids, *, renormalize=True):
    """Routing replay: caller-supplied expert ids; only the router GEMM, the
    sigmoid and the combine weights are recomputed.  An id outside [0, E)
    names no expert and is dropped (the reading matches ``permute``): its
    weight is 0 and it is left out of the normalising sum; a token with no
    valid id gets weights 0."""
    logits = router_logits(x, w_router)
    scores = sigmoid_f32(logits)
    ids = np.asarray(ids, dtype=np.int64)
    E = scores.shape[1]
    valid = (ids >= 0) & (ids < E)
    r = np.where(valid, np.take_along_axis(scores.astype(np.float64), np.clip(ids, 0, E - 1),
                                           axis=1), 0.0)
    if renormalize:
        tot = r.sum(axis=1, keepdims=True)
        r = np.divide(r, tot, out=np.zeros_like(r), where=tot > 0)
    return r, scores


def permute(ids, n_experts):
    """Per-expert histogram, exclusive offsets and the expert-major permutation.

    Row r of the permuted order holds flat slot perm_src[r] = t*k + j; rows are
    ordered by expert, then by token (slot index) ascending.  perm_dst is the
    inverse: perm_dst[t*k + j] = r.  A slot whose id lies outside
    [0, n_experts) names no expert: it is not counted, has no row
    (perm_dst = -1), and perm_src holds only the offsets[-1] valid rows.
    """
    flat = np.asarray(ids, dtype=np.int64).reshape(-1)
    valid = (flat >= 0) & (flat < n_experts)
    counts = np.bincount(flat[valid], minlength=n_experts).astype(np.int64)
    offsets = np.concatenate([[0], np.cumsum(counts)]).astype(np.int64)
    slots = np.nonzero(valid)[0]
    perm_src = slots[np.argsort(flat[slots], kind="stable")].astype(np.int64)
    perm_dst = np.full(flat.size, -1, dtype=np.int64)
    perm_dst[perm_src] = np.arange(perm_src.size)
    return counts, offsets, perm_src, perm_dst


def ffn_rows(x_rows, w_gate_up, w_down):
    """One expert's SwiGLU MLP on a block of rows, fp64 throughout:
    g = X Wg^T, u = X Wu^T, h = SiLU(g) * u, y = h Wd^T."""
    X = np.asarray(x_rows, dtype=np.float64)
    gu = np.asarray(w_gate_up, dtype=np.float64)
    inter = gu.shape[0] // 2
    g = X @ gu[:inter].T
    u = X @ gu[inter:].T
    with np.errstate(over="ignore"):
        h = g / (1.0 + np.exp(-g)) * u
    return h @ np.asarray(w_down, dtype=np.float64).T


# ---------------------------------------------------------------------------
# Expert LoRA ("Beam 1.0" miles recipes, section 5.5 "LoRA": an adapter on
# each routed expert with rank 16, alpha 32, dropout 0, the router frozen;
# the Axolotl Beam guide: LoRA on the fused expert weights).  Each adapted
# weight W [out, in] gains W x + (alpha / rank) * B (A x) with A [rank, in]
# and B [out, rank]; the fused gate/up weight carries one adapter
# (A [rank, H], B [2I, rank]) and the down weight another (A [rank, I],
# B [H, rank]).
# ---------------------------------------------------------------------------
LORA_RANK = 16
LORA_ALPHA = 32


def lora_scale(alpha=LORA_ALPHA, rank=LORA_RANK):
    """The adapter's output multiplier alpha / rank (2.0 for Beam's recipe)."""
    return float(alpha) / float(rank)


def ffn_rows_lora(x_rows, w_gate_up, w_down, lora, scale):
    """ffn_rows with one LoRA adapter on each expert weight, fp64 throughout:
    [g | u] = X Wgu^T + s (X Agu^T) Bgu^T, h = SiLU(g) * u,
    y = h Wd^T + s (h Ad^T) Bd^T.  ``lora`` = (a_gate_up, b_gate_up, a_down,
    b_down) of this expert."""
    X = np.asarray(x_rows, dtype=np.float64)
    a_gu, b_gu, a_d, b_d = (np.asarray(t, dtype=np.float64) for t in lora)
    gu = np.asarray(w_gate_up, dtype=np.float64)
    inter = gu.shape[0] // 2
    z = X @ gu.T + scale * ((X @ a_gu.T) @ b_gu.T)
    g, u = z[:, :inter], z[:, inter:]
    with np.errstate(over="ignore"):
        h = g / (1.0 + np.exp(-g)) * u
    return h @ np.asarray(w_down, dtype=np.float64).T + scale * ((h @ a_d.T) @ b_d.T)


def expert_ffn(x, perm_src, offsets, experts, topk=8, lora=None, lora_scale_=None):
    """All experts over the permuted rows.  ``experts`` is either a pair of
    arrays ([E, 2I, H], [E, H, I]) or a callable ``e -> (gate_up, down)``;
    ``lora`` (optional) is a 4-tuple of arrays ([E, r, H], [E, 2I, r],
    [E, r, I], [E, H, r]) or a callable ``e -> 4-tuple``, applied with the
    multiplier ``lora_scale_`` (default alpha / rank of Beam's recipe).
    Returns y_perm, fp64 [T*k, H], row r belonging to slot perm_src[r]."""
    x = np.asarray(x)
    get = experts if callable(experts) else (lambda e: (experts[0][e], experts[1][e]))
    if lora is not None and not callable(lora):
        arrs = lora
        lora = lambda e: tuple(t[e] for t in arrs)
    s = lora_scale() if lora_scale_ is None else lora_scale_
    y = np.zeros((len(perm_src), x.shape[1]), dtype=np.float64)
    for e in range(len(offsets) - 1):
        r0, r1 = int(offsets[e]), int(offsets[e + 1])
        if r1 == r0:
            continue  # an expert that receives no token does no work
        tokens = np.asarray(perm_src[r0:r1]) // topk
        gu, dn = get(e)
        if lora is None:
            y[r0:r1] = ffn_rows(x[tokens], gu, dn)
        else:
            y[r0:r1] = ffn_rows_lora(x[tokens], gu, dn, lora(e), s)
    return y


def combine(y_perm, perm_dst, weights, scale=2.5):
    """out[t] = scale * sum_j w[t, j] * y_perm[perm_dst[t*k + j]], in fp64;
    slots without a row (perm_dst < 0) contribute nothing."""
    T, k = weights.shape
    dst = np.asarray(perm_dst).reshape(T, k)
    y = np.asarray(y_perm, dtype=np.float64)
    rows = np.zeros((T, k, y.shape[1]))
    has = dst >= 0
    rows[has] = y[dst[has]]
    return scale * np.einsum("tj,tjh->th", np.asarray(weights, dtype=np.float64), rows)


def layer_forward(x, w_router, experts, *, n_groups=8, topk_groups=4, topk=8,
                  renormalize=True, scale=2.5, sel_bias=None, ids=None, lora=None,
                  lora_scale_=None):
    """The whole block: route, permute, expert MLPs, weighted combine.
    With ``ids`` given, routing is replayed instead of selected; ``lora`` adds
    the expert adapters (see expert_ffn)."""
    E = np.asarray(w_router).shape[0]
    if ids is None:
        rr = route(x, w_router, n_groups=n_groups, topk_groups=topk_groups, topk=topk,
                   renormalize=renormalize, sel_bias=sel_bias)
        ids, weights = rr.ids, rr.weights
    else:
        rr = None
        weights, _ = route_replay(x, w_router, ids, renormalize=renormalize)
    counts, offsets, perm_src, perm_dst = permute(ids, E)
    y = expert_ffn(x, perm_src, offsets, experts, topk=ids.shape[1], lora=lora,
                   lora_scale_=lora_scale_)
    out = combine(y, perm_dst, weights, scale)
    return {"route": rr, "ids": ids, "weights": weights, "counts": counts, "offsets": offsets,
            "perm_src": perm_src, "perm_dst": perm_dst, "y_perm": y, "out": out}


def selection_admissible(sel_row, gs_row, chosen, *, n_groups=8, topk_groups=4, topk=8,
                         tol=MARGIN_TOL):
    """Is ``chosen`` (k expert ids) the group-limited top-k of some perturbation
    of this token's fp32 selection values by at most ``tol``?

    A kept-group set A is admissible if every group in A scores at least the
    best group outside A minus ``tol``; the chosen set is admissible within A if
    it lies inside A's experts and its weakest member scores at least the best
    unchosen expert of A minus ``tol``.
    """
    sel_row = np.asarray(sel_row, dtype=np.float64)
    gs_row = np.asarray(gs_row, dtype=np.float64)
    chosen = [int(e) for e in chosen]
    E = sel_row.size
    gsize = E // n_groups
    if len(set(chosen)) != topk or len(chosen) != topk:
        return False
    need = {e // gsize for e in chosen}
    for A in combinations(range(n_groups), topk_groups):
        if not need <= set(A):
            continue
        outside = [g for g in range(n_groups) if g not in A]
        if outside and min(gs_row[list(A)]) < max(gs_row[outside]) - tol:
            continue
        pool = [e for g in A for e in range(g * gsize, (g + 1) * gsize)]
        rest = [e for e in pool if e not in set(chosen)]
        if rest and min(sel_row[chosen]) < max(sel_row[rest]) - tol:
            continue
        return True
    return False


# ---------------------------------------------------------------------------
# FP8 per-channel expert weights ("Beam-1.0-501B-A23B" vLLM recipe, FP8
# variant: FP8 per-channel weights, with the router left unquantized).
#
# Reading of "per-channel" (the recipe does not spell it out): one fp32 scale
# per output row of each expert matrix, s = max|row| / 448 (448 is the largest
# finite E4M3FN value), q = E4M3FN(w / s) by round-to-nearest-even, the
# quotient clamped to +-448 first (fp32 rounding of s can push the row maximum
# a hair past 448); a row of zeros gets s = 1.  The GEMM uses s * q.
# ---------------------------------------------------------------------------
E4M3_MAX = 448.0


def _e4m3_table():
    """fp64 value of every E4M3FN bit pattern (OCP FP8: bias 7, 3 mantissa
    bits, S.1111.111 is NaN, no infinities), from the format definition."""
    vals = np.empty(256)
    for b in range(256):
        sgn = -1.0 if b & 0x80 else 1.0
        e, m = (b >> 3) & 0xF, b & 0x7
        if e == 0xF and m == 0x7:
            vals[b] = np.nan
        elif e == 0:
            vals[b] = sgn * m * 2.0 ** -9
        else:
            vals[b] = sgn * (1 + m / 8.0) * 2.0 ** (e - 7)
    return vals


_E4M3 = _e4m3_table()


def e4m3_decode(q):
    """fp64 values of E4M3FN codes (uint8 array)."""
    return _E4M3[np.asarray(q, dtype=np.uint8)]


def e4m3_encode(x):
    """Round fp32 values (|x| <= 448) to the nearest E4M3FN code, ties to the
    code with an even mantissa (round-to-nearest-even), by search over the
    finite codes of the same sign."""
    x = np.asarray(x, dtype=np.float32).astype(np.float64)
    if np.any(np.abs(x) > E4M3_MAX) or np.any(~np.isfinite(x)):
        raise ValueError("e4m3_encode: value outside the finite E4M3FN range")
    pos = np.array([b for b in range(0x7F)])          # 0x00 .. 0x7E: +0 .. +448
    pv = _E4M3[pos]
    a = np.abs(x).ravel()
    idx = np.searchsorted(pv, a)                      # pv[idx-1] < a <= pv[idx]
    idx = np.clip(idx, 1, len(pv) - 1)
    lo, hi = pv[idx - 1], pv[idx]
    pick_hi = (a - lo > hi - a) | ((a - lo == hi - a) & ((pos[idx] & 1) == 0))
    code = np.where(a <= lo, pos[idx - 1], np.where(pick_hi, pos[idx], pos[idx - 1]))
    code = np.where(a == 0, 0, code)
    sign = (x.ravel() < 0) | ((x.ravel() == 0) & np.signbit(x.ravel()))
    return (code | (sign.astype(np.int64) << 7)).astype(np.uint8).reshape(x.shape)


def quantize_fp8_per_channel(w):
    """(codes uint8 [..., N, K], scales fp32 [..., N]) of a row-major weight
    [..., N, K]: s = fp32(max|row| / 448), q = E4M3FN(clamp(fp32(w / s), +-448))."""
    w32 = np.asarray(w, dtype=np.float32)
    amax = np.max(np.abs(w32), axis=-1)
    s = np.where(amax > 0, (amax / np.float32(E4M3_MAX)).astype(np.float32), np.float32(1.0))
    s = s.astype(np.float32)
    ratio = (w32 / s[..., None]).astype(np.float32)
    ratio = np.clip(ratio, np.float32(-E4M3_MAX), np.float32(E4M3_MAX))
    return e4m3_encode(ratio), s


def dequantize_fp8(q, s):
    """fp64 weights s * decode(q)."""
    return e4m3_decode(q) * np.asarray(s, dtype=np.float64)[..., None]
