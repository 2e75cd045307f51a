"""Pins for the oracle's permutation, expert SwiGLU MLPs and weighted combine.

What is pinned ("Welcome Beam: a 501B open model you can own, customize, and
scale", section Mixture of Experts): each expert is a SwiGLU MLP; outputs of
the 8 chosen experts are summed with weights equal to each score over the sum
of the chosen scores, and the sum is multiplied by 2.5; there is no shared
expert.  Checks use a library SwiGLU (torch, fp64, CPU),
closed forms with identical or proportional experts, and invariants.
"""
import numpy as np
import pytest
import torch

import oracle


def _rand_layer(rng, T=48, H=64, I=32, E=256, wstd=0.1):
    x = rng.standard_normal((T, H)).astype(np.float32)
    wr = (0.1 * rng.standard_normal((E, H))).astype(np.float32)
    gu = (wstd * rng.standard_normal((E, 2 * I, H))).astype(np.float32)
    dn = (wstd * rng.standard_normal((E, H, I))).astype(np.float32)
    return x, wr, gu, dn


def test_ffn_rows_matches_library_swiglu():
    rng = np.random.default_rng(0)
    H, I = 40, 24
    x = rng.standard_normal((7, H))
    gu = rng.standard_normal((2 * I, H))
    dn = rng.standard_normal((H, I))
    X = torch.from_numpy(x)
    gate = torch.nn.functional.linear(X, torch.from_numpy(gu[:I]))
    up = torch.nn.functional.linear(X, torch.from_numpy(gu[I:]))
    ref = torch.nn.functional.linear(torch.nn.functional.silu(gate) * up, torch.from_numpy(dn))
    np.testing.assert_allclose(oracle.ffn_rows(x, gu, dn), ref.numpy(), rtol=1e-12, atol=1e-12)


def test_silu_is_on_the_gate_half():
    # gate rows zero -> SiLU(0) = 0 -> output zero whatever the up rows hold
    rng = np.random.default_rng(1)
    H, I = 16, 8
    gu = rng.standard_normal((2 * I, H))
    gu[:I] = 0
    y = oracle.ffn_rows(rng.standard_normal((3, H)), gu, rng.standard_normal((H, I)))
    assert np.all(y == 0)
    # up rows zero -> output zero as well; gate alone contributes nothing
    gu = rng.standard_normal((2 * I, H))
    gu[I:] = 0
    y = oracle.ffn_rows(rng.standard_normal((3, H)), gu, rng.standard_normal((H, I)))
    assert np.all(y == 0)


def test_permute_invariants():
    rng = np.random.default_rng(2)
    T, E, k = 333, 256, 8
    ids = np.stack([rng.choice(E, k, replace=False) for _ in range(T)])
    counts, offsets, src, dst = oracle.permute(ids, E)
    assert counts.sum() == T * k and offsets[0] == 0 and offsets[-1] == T * k
    assert np.all(np.diff(offsets) == counts)
    assert sorted(src.tolist()) == list(range(T * k))
    assert np.array_equal(dst[src], np.arange(T * k))
    flat = ids.reshape(-1)
    for e in range(E):
        rows = src[offsets[e]:offsets[e + 1]]
        assert np.all(flat[rows] == e)
        assert np.all(np.diff(rows // k) > 0)  # stable: tokens ascending
    # histogram against a plain loop
    ref = np.zeros(E, np.int64)
    for v in flat:
        ref[v] += 1
    assert np.array_equal(ref, counts)


def test_identical_experts_closed_form():
    # all experts equal: out = 2.5 * FFN_0(x) with normalized weights,
    # out = 2.5 * (sum of the 8 chosen scores) * FFN_0(x) without
    rng = np.random.default_rng(3)
    x, wr, gu, dn = _rand_layer(rng)
    gu[:] = gu[0]
    dn[:] = dn[0]
    f0 = oracle.ffn_rows(x, gu[0], dn[0])
    res = oracle.layer_forward(x, wr, (gu, dn))
    np.testing.assert_allclose(res["out"], 2.5 * f0, rtol=1e-12, atol=1e-12)
    res = oracle.layer_forward(x, wr, (gu, dn), renormalize=False)
    ssum = np.take_along_axis(res["route"].scores.astype(np.float64), res["ids"], 1).sum(1)
    np.testing.assert_allclose(res["out"], 2.5 * ssum[:, None] * f0, rtol=1e-12, atol=1e-12)


def test_proportional_experts_closed_form():
    # W_d,e = c_e * W_d,0 -> FFN_e = c_e * FFN_0, so out = 2.5 * sum_j w_j c_{e_j} * FFN_0.
    # Pins the pairing of each weight with its own expert's rows.
    rng = np.random.default_rng(4)
    x, wr, gu, dn = _rand_layer(rng)
    gu[:] = gu[0]
    c = np.arange(1, 257, dtype=np.float64) / 256.0
    dn = (c[:, None, None] * dn[0][None].astype(np.float64))
    f0 = oracle.ffn_rows(x, gu[0], dn[0] / c[0])
    res = oracle.layer_forward(x, wr, (gu, dn))
    coef = 2.5 * (res["weights"] * c[res["ids"]]).sum(1)
    np.testing.assert_allclose(res["out"], coef[:, None] * f0, rtol=1e-10, atol=1e-12)


def test_single_expert_per_token():
    # k = 1 with normalized weights: out = 2.5 * FFN_{argmax}(x)
    rng = np.random.default_rng(5)
    x, wr, gu, dn = _rand_layer(rng, E=16)
    res = oracle.layer_forward(x, wr, (gu, dn), n_groups=4, topk_groups=4, topk=1)
    am = np.argmax(x.astype(np.float64) @ wr.astype(np.float64).T, axis=1)
    for t in range(x.shape[0]):
        np.testing.assert_allclose(res["out"][t], 2.5 * oracle.ffn_rows(x[t:t + 1], gu[am[t]], dn[am[t]])[0],
                                   rtol=1e-12, atol=1e-12)


def test_no_shared_expert():
    # if every chosen expert's down projection is zero, the block outputs exactly zero:
    # nothing else is added
    rng = np.random.default_rng(6)
    x, wr, gu, dn = _rand_layer(rng)
    dn[:] = 0
    res = oracle.layer_forward(x, wr, (gu, dn))
    assert np.all(res["out"] == 0)


def test_layer_token_permutation_equivariance():
    rng = np.random.default_rng(7)
    x, wr, gu, dn = _rand_layer(rng)
    P = rng.permutation(x.shape[0])
    a = oracle.layer_forward(x, wr, (gu, dn))["out"]
    b = oracle.layer_forward(x[P], wr, (gu, dn))["out"]
    np.testing.assert_allclose(a[P], b, rtol=1e-12, atol=1e-14)


def test_lazy_expert_callable_matches_arrays():
    rng = np.random.default_rng(8)
    x, wr, gu, dn = _rand_layer(rng)
    a = oracle.layer_forward(x, wr, (gu, dn))["out"]
    b = oracle.layer_forward(x, wr, lambda e: (gu[e], dn[e]))["out"]
    assert np.array_equal(a, b)


def test_empty_batch():
    rng = np.random.default_rng(9)
    x, wr, gu, dn = _rand_layer(rng, T=0)
    res = oracle.layer_forward(x, wr, (gu, dn))
    assert res["out"].shape == (0, x.shape[1])
    assert res["counts"].sum() == 0 and len(res["offsets"]) == 257


def test_route_replay_matches_route():
    rng = np.random.default_rng(10)
    x, wr, gu, dn = _rand_layer(rng)
    a = oracle.layer_forward(x, wr, (gu, dn))
    b = oracle.layer_forward(x, wr, (gu, dn), ids=a["ids"])
    assert np.array_equal(a["out"], b["out"])


@pytest.mark.parametrize("renorm", [True, False])
def test_combine_weighted_sum_by_hand(renorm):
    # two tokens, k = 2, explicit rows: out = 2.5 * (w0 * row_a + w1 * row_b)
    y = np.arange(4 * 3, dtype=np.float64).reshape(4, 3)
    perm_dst = np.array([2, 0, 3, 1])
    w = np.array([[0.25, 0.75], [0.5, 0.5]])
    out = oracle.combine(y, perm_dst, w, 2.5)
    np.testing.assert_allclose(out[0], 2.5 * (0.25 * y[2] + 0.75 * y[0]))
    np.testing.assert_allclose(out[1], 2.5 * (0.5 * y[3] + 0.5 * y[1]))


def _bad_ids(rng, T, E=256):
    ids = np.stack([rng.choice(E, 8, replace=False) for _ in range(T)]).astype(np.int64)
    ids[1, 3] = -1            # one dropped slot
    ids[4, 0] = E             # one past the last expert
    ids[6, :] = -7            # a token with no valid id
    ids[9, 7] = 1 << 30
    return ids


def test_permute_drops_invalid_ids_by_loop():
    # brute force: for every expert in turn, the slots naming it in increasing
    # order; slots naming no expert get no row
    rng = np.random.default_rng(41)
    ids = _bad_ids(rng, 40)
    counts, offsets, perm_src, perm_dst = oracle.permute(ids, 256)
    flat = ids.reshape(-1)
    want = [s for e in range(256) for s in range(flat.size) if flat[s] == e]
    assert list(perm_src) == want
    assert counts.sum() == len(want) == offsets[-1] == 8 * 40 - 11
    for s in range(flat.size):
        if 0 <= flat[s] < 256:
            assert perm_src[perm_dst[s]] == s
        else:
            assert perm_dst[s] == -1


def test_replay_drops_invalid_ids():
    # a dropped slot has weight 0, and the other slots' weights are those of a
    # replay of the valid ids alone (normalised over them)
    rng = np.random.default_rng(42)
    x, wr, gu, dn = _rand_layer(rng, T=12)
    ids = _bad_ids(rng, 12)
    for renorm in (True, False):
        w, s = oracle.route_replay(x, wr, ids, renormalize=renorm)
        for t in range(12):
            ok = (ids[t] >= 0) & (ids[t] < 256)
            assert np.all(w[t, ~ok] == 0)
            if ok.any():
                wv, _ = oracle.route_replay(x[t:t + 1], wr, ids[t:t + 1, ok], renormalize=renorm)
                np.testing.assert_allclose(w[t, ok], wv[0], rtol=1e-14)
                r = s[t, ids[t, ok]].astype(np.float64)
                np.testing.assert_allclose(w[t, ok], r / r.sum() if renorm else r, rtol=1e-14)


def test_layer_with_dropped_ids_by_hand():
    # the replayed layer with dropped slots: each token's output is 2.5 times
    # the weighted sum over its valid slots only, worked token by token
    rng = np.random.default_rng(43)
    x, wr, gu, dn = _rand_layer(rng, T=12)
    ids = _bad_ids(rng, 12)
    res = oracle.layer_forward(x, wr, (gu, dn), ids=ids)
    s = oracle.sigmoid_f32(oracle.router_logits(x, wr)).astype(np.float64)
    for t in range(12):
        ok = [j for j in range(8) if 0 <= ids[t, j] < 256]
        want = np.zeros(x.shape[1])
        tot = sum(s[t, ids[t, j]] for j in ok)
        for j in ok:
            e = ids[t, j]
            want += s[t, e] / tot * oracle.ffn_rows(x[t:t + 1], gu[e], dn[e])[0]
        np.testing.assert_allclose(res["out"][t], 2.5 * want, rtol=1e-10, atol=1e-12)
    assert np.all(res["out"][6] == 0)
