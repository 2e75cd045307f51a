"""Pins of the oracle's expert LoRA ("Beam 1.0" miles recipes, section 5.5
"LoRA": rank 16, alpha 32, an adapter on every routed expert, router frozen)."""
import json
import os

import numpy as np
import torch

import oracle

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "lora_recipe.json")


def _rand(rng, *shape, std=0.1):
    return rng.standard_normal(shape) * std


def test_recipe_constants_and_scale():
    g = json.load(open(GOLDEN))
    assert (oracle.LORA_RANK, oracle.LORA_ALPHA) == (g["lora_rank"], g["lora_alpha"])
    assert oracle.lora_scale() == 2.0                      # alpha / rank
    assert oracle.lora_scale(16, 16) == 1.0


def test_zero_b_is_the_base_mlp():
    rng = np.random.default_rng(0)
    H, I, r = 64, 32, 16
    X = _rand(rng, 5, H, std=1.0)
    gu, dn = _rand(rng, 2 * I, H), _rand(rng, H, I)
    lora = (_rand(rng, r, H), np.zeros((2 * I, r)), _rand(rng, r, I), np.zeros((H, r)))
    assert np.array_equal(oracle.ffn_rows_lora(X, gu, dn, lora, 2.0), oracle.ffn_rows(X, gu, dn))


def test_equals_the_merged_weights():
    # W x + s B (A x) == (W + s B A) x: the adapter acts before the SiLU on the
    # gate/up output and before the down output, with A on the input side
    rng = np.random.default_rng(1)
    H, I, r, s = 48, 24, 16, 2.0
    X = _rand(rng, 7, H, std=1.0)
    gu, dn = _rand(rng, 2 * I, H), _rand(rng, H, I)
    a_gu, b_gu, a_d, b_d = _rand(rng, r, H), _rand(rng, 2 * I, r), _rand(rng, r, I), _rand(rng, H, r)
    got = oracle.ffn_rows_lora(X, gu, dn, (a_gu, b_gu, a_d, b_d), s)
    merged = oracle.ffn_rows(X, gu + s * b_gu @ a_gu, dn + s * b_d @ a_d)
    np.testing.assert_allclose(got, merged, rtol=1e-10, atol=1e-12)
    # and against a library SwiGLU on the merged weights
    Xt = torch.tensor(X)
    z = Xt @ torch.tensor(gu + s * b_gu @ a_gu).T
    h = torch.nn.functional.silu(z[:, :I]) * z[:, I:]
    ref = (h @ torch.tensor(dn + s * b_d @ a_d).T).numpy()
    np.testing.assert_allclose(got, ref, rtol=1e-10, atol=1e-12)


def test_rank_one_hand_case():
    # zero base weights; A_gu picks x_j, B_gu writes 0.5 into gate row o and 2
    # into up row o; A_d picks h_o, B_d writes the vector d:
    #   g_o = 2 * 0.5 * x_j, u_o = 2 * 2 * x_j, h_o = SiLU(g_o) u_o, y = 2 h_o d
    H, I, r, j, o = 8, 4, 16, 3, 1
    x = np.zeros((1, H)); x[0, j] = 1.5
    a_gu = np.zeros((r, H)); a_gu[0, j] = 1.0
    b_gu = np.zeros((2 * I, r)); b_gu[o, 0] = 0.5; b_gu[I + o, 0] = 2.0
    a_d = np.zeros((r, I)); a_d[5, o] = 1.0
    d = np.arange(1, H + 1, dtype=np.float64)
    b_d = np.zeros((H, r)); b_d[:, 5] = d
    y = oracle.ffn_rows_lora(x, np.zeros((2 * I, H)), np.zeros((H, I)), (a_gu, b_gu, a_d, b_d), 2.0)
    g, u = 1.5, 6.0
    h = g / (1 + np.exp(-g)) * u
    np.testing.assert_allclose(y[0], 2.0 * h * d, rtol=1e-14)


def test_adapter_goes_to_its_own_expert():
    # identical base experts; only expert 5 has a nonzero adapter: rows routed
    # to expert 5 change, every other row equals the base output exactly
    rng = np.random.default_rng(2)
    E, H, I, r, T = 8, 32, 16, 16, 12
    x = _rand(rng, T, H, std=1.0)
    gu0, dn0 = _rand(rng, 2 * I, H), _rand(rng, H, I)
    gu = np.repeat(gu0[None], E, 0); dn = np.repeat(dn0[None], E, 0)
    lora = [np.zeros((E, r, H)), np.zeros((E, 2 * I, r)), np.zeros((E, r, I)), np.zeros((E, H, r))]
    lora[0][5], lora[1][5] = _rand(rng, r, H), _rand(rng, 2 * I, r)
    lora[2][5], lora[3][5] = _rand(rng, r, I), _rand(rng, H, r)
    ids = np.stack([rng.choice(E, 2, replace=False) for _ in range(T)])
    counts, offsets, psrc, pdst = oracle.permute(ids, E)
    base = oracle.expert_ffn(x, psrc, offsets, (gu, dn), topk=2)
    got = oracle.expert_ffn(x, psrc, offsets, (gu, dn), topk=2, lora=tuple(lora))
    r5 = slice(int(offsets[5]), int(offsets[6]))
    other = np.ones(len(psrc), bool); other[r5] = False
    assert np.array_equal(got[other], base[other])
    assert counts[5] > 0 and np.all(np.abs(got[r5] - base[r5]).max(axis=1) > 0)
