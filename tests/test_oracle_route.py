"""Pins for the oracle's router and group-limited selection.

The rule being pinned ("Welcome Beam: a 501B open model you can own, customize,
and scale", section Mixture of Experts): sigmoid scores for all experts, 8
contiguous groups of 32, keep the 4 groups with the largest top-two sum, then
the top 8 experts inside the kept groups.  Each test checks the oracle against
something other than itself: hand-worked cases, exhaustive enumeration, a
textbook reduction to plain top-k, or an invariant of the rule.
"""
import json
import os
from itertools import combinations

import numpy as np
import pytest

import oracle


def _scores_from_case(case, E=256):
    s = np.full(E, case["base"], dtype=np.float32)
    for k, v in case["set"].items():
        s[int(k)] = v
    return s


def _load_cases(golden_dir):
    with open(os.path.join(golden_dir, "routing_hand_cases.json")) as f:
        return json.load(f)["cases"]


def test_hand_cases_select(golden_dir):
    for case in _load_cases(golden_dir):
        s = _scores_from_case(case)[None, :]
        ids, gs, keep, margin = oracle.select(s, 8, 4, 8)
        assert list(ids[0]) == case["ids"], case["name"]
        assert list(np.nonzero(keep[0])[0]) == case["kept_groups"], case["name"]
        assert (margin[0] == 0) == case["margin_zero"], case["name"]


def test_hand_cases_through_router(golden_dir):
    # x = [1.0] and W_r[e, 0] = logit(score_e): the router reproduces the scores
    # (up to fp32 rounding, which preserves order and ties).
    for case in _load_cases(golden_dir):
        s = _scores_from_case(case).astype(np.float64)
        w = np.log(s / (1 - s)).astype(np.float32)[:, None]
        rr = oracle.route(np.ones((1, 1), np.float32), w)
        assert list(rr.ids[0]) == case["ids"], case["name"]
        if "weights" in case:
            np.testing.assert_allclose(rr.weights[0], case["weights"], rtol=1e-6)
        if "weights_unnormalised" in case:
            raw = oracle.route(np.ones((1, 1), np.float32), w, renormalize=False)
            np.testing.assert_allclose(raw.weights[0], case["weights_unnormalised"], rtol=1e-6)


def test_normalised_weights_by_hand(golden_dir):
    # unequal chosen scores: the normalised weights are each score over the sum
    # of the eight chosen scores (hand-worked in the fixture), which neither a
    # softmax over the chosen scores nor a division by the sum of all 256
    # scores reproduces
    case = {c["name"]: c for c in _load_cases(golden_dir)}["unequal_scores_normalised"]
    s = _scores_from_case(case)
    ids = np.array([case["ids"]], dtype=np.int64)
    w = oracle._weights(s[None, :], ids, True)
    np.testing.assert_allclose(w[0], case["weights"], rtol=1e-6)
    np.testing.assert_allclose(oracle._weights(s[None, :], ids, False)[0],
                               case["weights_unnormalised"], rtol=1e-6)
    soft = np.exp(np.float64(case["weights_unnormalised"]))
    assert not np.allclose(case["weights"], soft / soft.sum(), rtol=1e-3)
    assert not np.allclose(case["weights"], s[case["ids"]] / s.sum(dtype=np.float64), rtol=1e-3)


def test_normalised_and_raw_weights_relation():
    # with normalisation on, the weights are the raw (normalisation off)
    # weights divided by their per-token sum; the raw weights are the chosen
    # experts' own sigmoid scores, so their ratios are the score ratios
    rng = np.random.default_rng(31)
    x = rng.standard_normal((64, 96)).astype(np.float32)
    w = (0.3 * rng.standard_normal((256, 96))).astype(np.float32)
    on = oracle.route(x, w, renormalize=True)
    off = oracle.route(x, w, renormalize=False)
    assert np.array_equal(on.ids, off.ids)
    raw = off.weights
    assert np.ptp(raw, axis=1).min() > 1e-4          # the chosen scores are unequal
    np.testing.assert_allclose(on.weights, raw / raw.sum(axis=1, keepdims=True), rtol=1e-12)
    np.testing.assert_allclose(on.weights[:, 0] / on.weights[:, 1], raw[:, 0] / raw[:, 1],
                               rtol=1e-12)


def _brute_force(sel_row, G, KG, K):
    """Exhaustive search: the group subset maximising the sum of top-two sums
    (each a maximum over distinct pairs), then the expert subset of the kept
    groups maximising the sum of scores."""
    E = sel_row.size
    gsize = E // G
    s = sel_row.astype(np.float64)
    pair_best = []
    for g in range(G):
        m = s[g * gsize:(g + 1) * gsize]
        pair_best.append(max(m[i] + m[j] for i, j in combinations(range(gsize), 2)))
    best_groups = max(combinations(range(G), KG), key=lambda A: sum(pair_best[g] for g in A))
    pool = [e for g in best_groups for e in range(g * gsize, (g + 1) * gsize)]
    best = max(combinations(pool, K), key=lambda S: sum(s[e] for e in S))
    return set(best_groups), set(best)


@pytest.mark.parametrize("seed", range(4))
def test_bruteforce_small_shape(seed):
    # (E, G, kG, k) = (16, 4, 2, 4): all 6 group pairs x all 70 expert subsets
    rng = np.random.default_rng(seed)
    T, E, H = 64, 16, 24
    x = rng.standard_normal((T, H)).astype(np.float32)
    w = (0.3 * rng.standard_normal((E, H))).astype(np.float32)
    rr = oracle.route(x, w, n_groups=4, topk_groups=2, topk=4)
    for t in range(T):
        groups, chosen = _brute_force(rr.sel[t], 4, 2, 4)
        assert set(rr.ids[t]) == chosen
        assert set(np.nonzero(rr.group_keep[t])[0]) == groups


def test_full_shape_group_enumeration():
    # Beam shape: enumerate all C(8,4) = 70 kept-group sets; experts by rank predicate
    rng = np.random.default_rng(7)
    T, E = 200, 256
    sel = (1 / (1 + np.exp(-1.4 * rng.standard_normal((T, E))))).astype(np.float32)
    ids, gs, keep, margin = oracle.select(sel, 8, 4, 8)
    s = sel.astype(np.float64)
    for t in range(T):
        pair = [np.max(s[t, 32 * g:32 * g + 32][:, None] + s[t, 32 * g:32 * g + 32][None, :]
                       - 1e9 * np.eye(32)) for g in range(8)]
        A = max(combinations(range(8), 4), key=lambda A: sum(pair[g] for g in A))
        assert set(np.nonzero(keep[t])[0]) == set(A)
        elig = np.zeros(E, bool)
        for g in A:
            elig[32 * g:32 * g + 32] = True
        # e is chosen iff eligible and fewer than 8 eligible experts rank before it
        chosen = set()
        for e in np.nonzero(elig)[0]:
            before = np.sum(elig & ((s[t] > s[t, e]) | ((s[t] == s[t, e]) & (np.arange(E) < e))))
            if before < 8:
                chosen.add(int(e))
        assert set(ids[t]) == chosen
        assert len(set(ids[t])) == 8


def test_textbook_single_group_is_plain_topk():
    # G = 1 (or kG = G): the rule reduces to the top-k of sigmoid(logits), i.e.
    # the top-k of the logits themselves (sigmoid is increasing)
    rng = np.random.default_rng(3)
    x = rng.standard_normal((50, 40)).astype(np.float32)
    w = (0.1 * rng.standard_normal((32, 40))).astype(np.float32)
    logits = x.astype(np.float64) @ w.astype(np.float64).T
    ref = np.argsort(-logits, axis=1)[:, :6]
    for G, KG in [(1, 1), (4, 4), (8, 8)]:
        rr = oracle.route(x, w, n_groups=G, topk_groups=KG, topk=6)
        assert np.array_equal(rr.ids, ref), (G, KG)
        assert np.all(np.isinf(rr.margin) | (rr.margin > 0))


def test_textbook_k1_is_argmax():
    rng = np.random.default_rng(4)
    x = rng.standard_normal((50, 40)).astype(np.float32)
    w = (0.1 * rng.standard_normal((16, 40))).astype(np.float32)
    rr = oracle.route(x, w, n_groups=4, topk_groups=4, topk=1)
    assert np.array_equal(rr.ids[:, 0], np.argmax(x @ w.T, axis=1))
    np.testing.assert_array_equal(rr.weights, 1.0)


def test_router_uses_weight_rows():
    # a one-hot token picks column h of W_r: logits[e] = W_r[e, h] exactly
    rng = np.random.default_rng(5)
    E, H = 256, 256   # square on purpose: a transposed product would not fail on shape
    w = rng.standard_normal((E, H)).astype(np.float32)
    x = np.zeros((3, H), np.float32)
    x[0, 0] = 1
    x[1, 17] = 1
    x[2, 255] = 1
    rr = oracle.route(x, w)
    np.testing.assert_array_equal(rr.logits[0], w[:, 0])
    np.testing.assert_array_equal(rr.logits[1], w[:, 17])
    np.testing.assert_array_equal(rr.logits[2], w[:, 255])


def test_sigmoid_values():
    # closed form points of the logistic function, each exactly representable
    lg = np.array([[0.0, np.log(3.0), -np.log(3.0), 80.0, -200.0]])
    s = oracle.sigmoid_f32(lg)
    np.testing.assert_array_equal(s[0, :3], np.float32([0.5, 0.75, 0.25]))
    assert s[0, 3] == np.float32(1.0) and s[0, 4] == 0.0


def test_invariants_beam_shape():
    rng = np.random.default_rng(11)
    T = 300
    x = rng.standard_normal((T, 512)).astype(np.float32)
    w = (0.02 * rng.standard_normal((256, 512))).astype(np.float32)
    rr = oracle.route(x, w)
    for t in range(T):
        ids = rr.ids[t]
        assert len(set(ids)) == 8
        groups = set(ids // 32)
        kept = set(np.nonzero(rr.group_keep[t])[0])
        assert len(kept) == 4 and groups <= kept
        # ordered by score desc
        assert np.all(np.diff(rr.sel[t, ids].astype(np.float64)) <= 0)
    np.testing.assert_allclose(rr.weights.sum(axis=1), 1.0, atol=1e-12)
    assert np.all(rr.weights > 0)


def test_group_score_is_top_two_sum():
    rng = np.random.default_rng(2)
    sel = rng.random((20, 256)).astype(np.float32)
    _, gs, _, _ = oracle.select(sel, 8, 4, 8)
    for t in range(20):
        for g in range(8):
            v = sorted(sel[t, 32 * g:32 * g + 32].tolist(), reverse=True)
            assert gs[t, g] == np.float32(np.float32(v[0]) + np.float32(v[1]))


def test_renormalize_switch_and_bias():
    rng = np.random.default_rng(9)
    x = rng.standard_normal((40, 64)).astype(np.float32)
    w = (0.2 * rng.standard_normal((256, 64))).astype(np.float32)
    rr = oracle.route(x, w, renormalize=False)
    np.testing.assert_array_equal(rr.weights, np.take_along_axis(rr.scores, rr.ids, 1).astype(np.float64))
    # a large bias on one expert forces its selection; its weight uses the unbiased score
    bias = np.zeros(256, np.float32)
    bias[200] = 5.0
    rb = oracle.route(x, w, sel_bias=bias, renormalize=False)
    assert np.all(rb.ids[:, 0] == 200)
    np.testing.assert_array_equal(rb.weights[:, 0], rb.scores[:, 200].astype(np.float64))


def test_token_permutation_equivariance():
    rng = np.random.default_rng(12)
    x = rng.standard_normal((64, 128)).astype(np.float32)
    w = (0.05 * rng.standard_normal((256, 128))).astype(np.float32)
    P = rng.permutation(64)
    a = oracle.route(x, w)
    b = oracle.route(x[P], w)
    assert np.array_equal(a.ids[P], b.ids)
    assert np.array_equal(a.weights[P], b.weights)


def test_hidden_permutation_invariance():
    # permuting hidden dims of x and W together leaves the routing unchanged
    rng = np.random.default_rng(13)
    x = rng.standard_normal((32, 96)).astype(np.float32)
    w = (0.05 * rng.standard_normal((256, 96))).astype(np.float32)
    Q = rng.permutation(96)
    a = oracle.route(x, w)
    b = oracle.route(x[:, Q], w[:, Q])
    assert np.array_equal(a.ids, b.ids)


def test_margin_flags_ties():
    sel = np.full((1, 256), 0.1, np.float32)
    sel[0, :16] = 0.5   # sixteen tied experts in group 0; groups 1..7 tie at 0.2
    ids, gs, keep, margin = oracle.select(sel, 8, 4, 8)
    assert list(ids[0]) == list(range(8)) and margin[0] == 0


def test_selection_admissible():
    rng = np.random.default_rng(21)
    sel = (1 / (1 + np.exp(-1.4 * rng.standard_normal((50, 256))))).astype(np.float32)
    ids, gs, keep, margin = oracle.select(sel, 8, 4, 8)
    for t in range(50):
        assert oracle.selection_admissible(sel[t], gs[t], ids[t])
        # swapping the 8th expert for the best unchosen eligible one is admissible
        # only when the expert cut is within the tolerance
        elig = np.repeat(keep[t], 32)
        cand = np.where(elig, sel[t], -np.inf)
        order = np.argsort(-cand.astype(np.float64), kind="stable")
        alt = list(order[:7]) + [order[8]]
        gap = float(cand[order[7]]) - float(cand[order[8]])
        assert oracle.selection_admissible(sel[t], gs[t], alt) == (gap <= oracle.MARGIN_TOL)
    # duplicated ids are never admissible
    assert not oracle.selection_admissible(sel[0], gs[0], [ids[0][0]] * 8)
