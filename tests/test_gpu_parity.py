"""GPU parity of every entry point against the CPU oracle at oracle-sized
shapes (the tiny workload: T=128, hidden 256, intermediate 128, 256 experts in
8 groups of 32), plus ragged sizes, edge cases and determinism."""
import numpy as np
import pytest
import torch

import grouped_top_routing_amd as gtr
import oracle
import synth
from parity_util import assert_close, check_routing, layer_reference, say, to_np

pytestmark = pytest.mark.gpu
DEV = torch.device("cuda", 0)


@pytest.fixture(scope="module")
def tiny():
    say("[tiny] generating inputs on", DEV)
    d = synth.make_inputs("tiny", 0, device=DEV)
    d["np"] = {k: to_np(d[k]) for k in ("x", "w_router", "w_gate_up", "w_down")}
    return d


def _rand_ids(T, k=8, E=256, seed=0, hot=None):
    rng = np.random.default_rng(seed)
    if hot is not None:
        return np.tile(np.asarray(hot, np.int32), (T, 1))
    return np.stack([rng.choice(E, k, replace=False) for _ in range(T)]).astype(np.int32)


# --------------------------------------------------------------------- route
@pytest.mark.parametrize("G,KG,K,renorm,bias", [
    (8, 4, 8, True, False),     # Beam's rule
    (8, 4, 8, False, False),    # raw scores as weights
    (8, 4, 8, True, True),      # selection bias on
    (1, 1, 8, True, False),     # plain top-k
    (4, 2, 6, True, False),
    (64, 8, 8, True, False),    # groups of 4 experts
    (16, 3, 5, False, False),
    (8, 8, 1, True, False),     # argmax
])
def test_route(tiny, G, KG, K, renorm, bias):
    say(f"[route] tiny G={G} kG={KG} k={K} renorm={renorm} bias={bias}")
    sb = synth.make_sel_bias(tiny["workload"], 0, device=DEV) if bias else None
    ids, w = gtr.route(tiny["x"], tiny["w_router"], sel_bias=sb, num_groups=G, topk_groups=KG,
                       topk=K, renormalize=renorm)
    torch.cuda.synchronize()
    rr = oracle.route(tiny["np"]["x"], tiny["np"]["w_router"], n_groups=G, topk_groups=KG,
                      topk=K, renormalize=renorm, sel_bias=None if sb is None else to_np(sb))
    nf, nd = check_routing(to_np(ids), to_np(w), rr, n_groups=G, topk_groups=KG, topk=K)
    say(f"  flagged={nf} differing={nd}")
    # ids come out in (value desc, index asc) order
    sel = rr.sel
    g = np.take_along_axis(sel, to_np(ids).astype(np.int64), 1).astype(np.float64)
    assert np.all(np.diff(g, axis=1) <= 1e-6)


@pytest.mark.parametrize("shift", [-2.0, -0.5])
def test_route_negative_biased_scores(tiny, shift):
    """A selection bias that makes the biased scores negative (all of them at
    -2, about half at -0.5): the kept groups' top-two sums and the expert
    ranking must treat negative values as values (only ineligible experts are
    minus infinity); combine weights still come from the unbiased scores."""
    say(f"[route] negative biased scores, shift {shift}")
    sb = synth.make_sel_bias(tiny["workload"], 1, device=DEV) + shift
    ids, w = gtr.route(tiny["x"], tiny["w_router"], sel_bias=sb)
    torch.cuda.synchronize()
    rr = oracle.route(tiny["np"]["x"], tiny["np"]["w_router"], sel_bias=to_np(sb))
    assert (rr.sel < 0).mean() > (0.99 if shift < -1 else 0.2)
    nf, nd = check_routing(to_np(ids), to_np(w), rr)
    say(f"  flagged={nf} differing={nd}")


def test_route_replay(tiny):
    say("[route_replay] tiny")
    rr = oracle.route(tiny["np"]["x"], tiny["np"]["w_router"])
    ids = torch.from_numpy(rr.ids.astype(np.int32)).to(DEV)
    for renorm in (True, False):
        w = gtr.route_replay(tiny["x"], tiny["w_router"], ids, renormalize=renorm)
        ref, _ = oracle.route_replay(tiny["np"]["x"], tiny["np"]["w_router"], rr.ids,
                                     renormalize=renorm)
        np.testing.assert_allclose(to_np(w), ref, rtol=1e-5, atol=1e-7)


@pytest.mark.parametrize("T", [1, 3, 63, 65, 127])
def test_route_ragged(tiny, T):
    say(f"[route] tiny T={T}")
    x = tiny["x"][:T].contiguous()
    ids, w = gtr.route(x, tiny["w_router"])
    rr = oracle.route(tiny["np"]["x"][:T], tiny["np"]["w_router"])
    check_routing(to_np(ids), to_np(w), rr)


def test_route_200_tokens():
    # more tokens than one logits tile column, ragged against 64
    say("[route] T=200 hidden 512")
    w = synth.workload("tiny", T=200, H=512)
    x = synth.make_x(w, 3, DEV)
    wr = synth.make_router(w, 3, DEV)
    ids, wt = gtr.route(x, wr)
    check_routing(to_np(ids), to_np(wt), oracle.route(to_np(x), to_np(wr)))


# ------------------------------------------------------------------- permute
# T <= 512 (at most 4096 pairs) runs the one-workgroup kernel, larger batches
# the chunked kernels; 512 and 513 straddle the boundary
@pytest.mark.parametrize("T,hot", [(1, None), (3, None), (32, None), (128, None), (512, None),
                                   (513, None), (4097, None), (500, list(range(40, 48))),
                                   (2000, list(range(100, 108)))])
def test_permute_exact(T, hot):
    say(f"[permute] T={T} hot={hot is not None}")
    ids = _rand_ids(T, seed=T, hot=hot)
    c, o, ps, pd = gtr.permute(torch.from_numpy(ids).to(DEV))
    rc, ro, rps, rpd = oracle.permute(ids, 256)
    assert np.array_equal(to_np(c), rc)
    assert np.array_equal(to_np(o), ro)
    assert np.array_equal(to_np(ps), rps)
    assert np.array_equal(to_np(pd), rpd)


@pytest.mark.parametrize("T", [1, 64, 700])
def test_layer_all_ties_zero_input(tiny, T):
    """x = 0: every logit is 0 and every score exactly 0.5, so all groups and
    all experts tie; the lower index wins each tie, giving experts 0..7 (all
    in group 0) with weights 0.5 / 4 = 0.125, and the output is exactly 0.
    Both sides reach these values exactly, so they are compared exactly."""
    say(f"[layer] all-zero input T={T}")
    x = torch.zeros(T, 256, dtype=torch.bfloat16, device=DEV)
    out, ids, w = gtr.layer_forward(x, tiny["w_router"], tiny["w_gate_up"], tiny["w_down"],
                                    return_routing=True)
    torch.cuda.synchronize()
    want = np.tile(np.arange(8, dtype=np.int32), (T, 1))
    assert np.array_equal(to_np(ids), want)
    assert np.array_equal(to_np(w), np.full((T, 8), 0.125, np.float32))
    assert not to_np(out).any()
    rr = oracle.route(to_np(x), tiny["np"]["w_router"])
    assert np.array_equal(rr.ids, want) and np.all(rr.margin == 0.0)


def test_layer_saturated_scores(tiny):
    """x scaled by 64: logits up to ~90, about 50 experts per token score
    exactly 1.0 in fp32, and many groups tie at 2.0; every token sits at a
    selection tie (margin 0), so the GPU's set must be admissible and the
    output is compared with the oracle evaluated on that set."""
    say("[layer] saturated sigmoid scores")
    x = (tiny["x"].float() * 64).to(torch.bfloat16)
    out, ids, w = gtr.layer_forward(x, tiny["w_router"], tiny["w_gate_up"], tiny["w_down"],
                                    return_routing=True)
    torch.cuda.synchronize()
    npd = tiny["np"]
    xn = to_np(x)
    ref = oracle.layer_forward(xn, npd["w_router"], (npd["w_gate_up"], npd["w_down"]))
    assert (ref["route"].scores == 1.0).sum(axis=1).mean() > 8
    nf, nd = check_routing(to_np(ids), to_np(w), ref["route"])
    say(f"  flagged={nf} differing={nd}")
    assert_close(to_np(out), layer_reference(to_np(ids), ref, xn,
                                             (npd["w_gate_up"], npd["w_down"])), "out")


@pytest.mark.parametrize("T", [300, 2000])
def test_permute_drops_out_of_range_ids(T):
    say(f"[permute] out-of-range ids T={T}")
    ids = _rand_ids(T, seed=5)
    ids[3, 2] = -1
    ids[77, 0] = 256
    ids[T - 1, 7] = 1 << 30
    c, o, ps, pd = gtr.permute(torch.from_numpy(ids).to(DEV))
    rc, ro, rorder, rdst = oracle.permute(ids, 256)
    n = int(ro[-1])
    assert n == T * 8 - 3
    assert np.array_equal(to_np(c), rc) and np.array_equal(to_np(o), ro)
    assert np.array_equal(to_np(ps)[:n], rorder)
    assert np.array_equal(to_np(pd), rdst)


def _with_bad_ids(ids):
    ids = ids.copy()
    ids[1, 3] = -1
    ids[4, 0] = 256
    ids[6, :] = -7          # a token with no valid id
    ids[9, 7] = 1 << 30
    return ids


def test_route_replay_drops_out_of_range_ids(tiny):
    # ids outside [0, E) get weight 0 and leave the normalising sum, as the
    # permutation drops them
    say("[route_replay] out-of-range ids")
    rr = oracle.route(tiny["np"]["x"], tiny["np"]["w_router"])
    bad = _with_bad_ids(rr.ids.astype(np.int32))
    ids = torch.from_numpy(bad).to(DEV)
    for renorm in (True, False):
        w = gtr.route_replay(tiny["x"], tiny["w_router"], ids, renormalize=renorm)
        ref, _ = oracle.route_replay(tiny["np"]["x"], tiny["np"]["w_router"], bad,
                                     renormalize=renorm)
        got = to_np(w)
        assert np.all(got[(bad < 0) | (bad >= 256)] == 0) and np.all(got[6] == 0)
        np.testing.assert_allclose(got, ref, rtol=1e-5, atol=1e-7)


def test_replayed_layer_with_dropped_ids(tiny):
    # the staged block on replayed ids with dropped slots against the oracle's
    # layer on the same ids
    say("[layer] replayed ids with out-of-range entries")
    npd = tiny["np"]
    rr = oracle.route(npd["x"], npd["w_router"])
    bad = _with_bad_ids(rr.ids.astype(np.int32))
    ids = torch.from_numpy(bad).to(DEV)
    w = gtr.route_replay(tiny["x"], tiny["w_router"], ids)
    c, o, ps, pd = gtr.permute(ids)
    y = gtr.expert_ffn(tiny["x"], ps, o, tiny["w_gate_up"], tiny["w_down"])
    out = gtr.combine(y, pd, w)
    torch.cuda.synchronize()
    ref = oracle.layer_forward(npd["x"], npd["w_router"], (npd["w_gate_up"], npd["w_down"]),
                               ids=bad)
    assert np.all(to_np(out)[6] == 0)
    assert_close(to_np(out), ref["out"], "out with dropped slots")


# ----------------------------------------------------------------------- ffn
def test_expert_ffn(tiny):
    say("[expert_ffn] tiny")
    npd = tiny["np"]
    rr = oracle.route(npd["x"], npd["w_router"])
    counts, offsets, psrc, pdst = oracle.permute(rr.ids, 256)
    y = gtr.expert_ffn(tiny["x"], torch.from_numpy(psrc.astype(np.int32)).to(DEV),
                       torch.from_numpy(offsets.astype(np.int32)).to(DEV),
                       tiny["w_gate_up"], tiny["w_down"])
    ref = oracle.expert_ffn(npd["x"], psrc, offsets, (npd["w_gate_up"], npd["w_down"]))
    assert_close(to_np(y), ref, "y_perm")


@pytest.mark.parametrize("hot_rows,T", [(1, 64), (17, 64), (40, 200), (130, 700), (300, 1024),
                                        (1000, 2048), (700, 3072), (2500, 4096),
                                        (3000, 16384)])
def test_expert_ffn_ragged_tiles(tiny, hot_rows, T):
    # one expert gets `hot_rows` rows, the rest spread thinly: m-tiles with
    # ragged tails, experts with a single row, and every m-tile height the
    # library picks from the mean rows per expert (up to 1024 tokens -> 64-row
    # tiles, 2048 -> 128, 3072 and 4096 -> 192, above 5120 -> 256; at 16384
    # tokens there are more m-tiles than workgroups, so each workgroup runs
    # several items back to back and starts each next item's weight stream
    # early)
    say(f"[expert_ffn] ragged hot_rows={hot_rows} T={T}")
    npd = tiny["np"]
    rng = np.random.default_rng(hot_rows)
    ids = np.stack([rng.choice(np.arange(1, 256), 8, replace=False) for _ in range(T)])
    ids[:hot_rows, 0] = 0
    x = synth.make_x(synth.workload("tiny", T=T), 7, DEV)
    xn = to_np(x)
    counts, offsets, psrc, pdst = oracle.permute(ids, 256)
    y = gtr.expert_ffn(x, torch.from_numpy(psrc.astype(np.int32)).to(DEV),
                       torch.from_numpy(offsets.astype(np.int32)).to(DEV),
                       tiny["w_gate_up"], tiny["w_down"])
    ref = oracle.expert_ffn(xn, psrc, offsets, (npd["w_gate_up"], npd["w_down"]))
    assert_close(to_np(y), ref, "y_perm")


# ------------------------------------------------------------------- combine
def test_combine(tiny):
    say("[combine] tiny")
    npd = tiny["np"]
    rr = oracle.route(npd["x"], npd["w_router"])
    counts, offsets, psrc, pdst = oracle.permute(rr.ids, 256)
    y = oracle.expert_ffn(npd["x"], psrc, offsets, (npd["w_gate_up"], npd["w_down"]))
    y_bf = torch.from_numpy(y.astype(np.float32)).to(torch.bfloat16)
    w32 = rr.weights.astype(np.float32)
    out = gtr.combine(y_bf.to(DEV), torch.from_numpy(pdst.astype(np.int32)).to(DEV),
                      torch.from_numpy(w32).to(DEV), routed_scaling=2.5)
    ref = oracle.combine(to_np(y_bf), pdst, w32.astype(np.float64), 2.5)
    # only the final bf16 rounding separates the two
    assert_close(to_np(out), ref, "combine", max_rel=8e-3, mean_rel=2e-3)


# --------------------------------------------------------------------- layer
@pytest.mark.parametrize("renorm,bias", [(True, False), (False, False), (True, True)])
def test_layer(tiny, renorm, bias):
    say(f"[layer] tiny renorm={renorm} bias={bias}")
    npd = tiny["np"]
    sb = synth.make_sel_bias(tiny["workload"], 0, device=DEV) if bias else None
    out, ids, w = gtr.layer_forward(tiny["x"], tiny["w_router"], tiny["w_gate_up"],
                                    tiny["w_down"], sel_bias=sb, renormalize=renorm,
                                    return_routing=True)
    ref = oracle.layer_forward(npd["x"], npd["w_router"], (npd["w_gate_up"], npd["w_down"]),
                               renormalize=renorm, sel_bias=None if sb is None else to_np(sb))
    nf, nd = check_routing(to_np(ids), to_np(w), ref["route"])
    say(f"  flagged={nf} differing={nd}")
    assert_close(to_np(out), layer_reference(to_np(ids), ref, npd["x"],
                                             (npd["w_gate_up"], npd["w_down"]),
                                             renormalize=renorm), "out")


@pytest.mark.parametrize("T", [1, 5, 127, 129, 300])
def test_layer_ragged_tokens(tiny, T):
    say(f"[layer] tiny-shape T={T}")
    npd = tiny["np"]
    # seed 11 puts token 66 one ulp from a selection tie (margin 6e-8): the
    # GPU may pick the other side; that token is then checked on the GPU's set
    x = synth.make_x(synth.workload("tiny", T=T), 11, DEV)
    out, ids, w = gtr.layer_forward(x, tiny["w_router"], tiny["w_gate_up"], tiny["w_down"],
                                    return_routing=True)
    xn = to_np(x)
    ref = oracle.layer_forward(xn, npd["w_router"], (npd["w_gate_up"], npd["w_down"]))
    nf, nd = check_routing(to_np(ids), to_np(w), ref["route"])
    say(f"  flagged={nf} differing={nd}")
    assert_close(to_np(out), layer_reference(to_np(ids), ref, xn,
                                             (npd["w_gate_up"], npd["w_down"])), "out")


def test_layer_identical_experts_closed_form(tiny):
    # every expert equal -> out = 2.5 * FFN_0(x) whatever the routing
    say("[layer] identical experts")
    wgu = tiny["w_gate_up"][:1].expand_as(tiny["w_gate_up"]).contiguous()
    wd = tiny["w_down"][:1].expand_as(tiny["w_down"]).contiguous()
    out = gtr.layer_forward(tiny["x"], tiny["w_router"], wgu, wd)
    f0 = oracle.ffn_rows(tiny["np"]["x"], tiny["np"]["w_gate_up"][0], tiny["np"]["w_down"][0])
    assert_close(to_np(out), 2.5 * f0, "out")


def test_layer_deterministic_and_equivariant(tiny):
    say("[layer] determinism / token permutation")
    a = gtr.layer_forward(tiny["x"], tiny["w_router"], tiny["w_gate_up"], tiny["w_down"])
    b = gtr.layer_forward(tiny["x"], tiny["w_router"], tiny["w_gate_up"], tiny["w_down"])
    assert torch.equal(a, b)
    P = torch.from_numpy(np.random.default_rng(1).permutation(128)).to(DEV)
    c = gtr.layer_forward(tiny["x"][P].contiguous(), tiny["w_router"], tiny["w_gate_up"],
                          tiny["w_down"])
    assert torch.equal(a[P], c)


def test_layer_on_side_stream(tiny):
    say("[layer] non-default stream")
    ref = gtr.layer_forward(tiny["x"], tiny["w_router"], tiny["w_gate_up"], tiny["w_down"])
    s = torch.cuda.Stream(DEV)
    s.wait_stream(torch.cuda.current_stream(DEV))
    with torch.cuda.stream(s):
        out = gtr.layer_forward(tiny["x"], tiny["w_router"], tiny["w_gate_up"], tiny["w_down"],
                                workspace=gtr.Workspace())
    torch.cuda.current_stream(DEV).wait_stream(s)
    torch.cuda.synchronize()
    assert torch.equal(out, ref)


def test_default_workspaces_on_two_streams(tiny):
    # calls without a workspace on two streams at once: each stream gets its
    # own default workspace, so the concurrent layers do not share scratch
    say("[layer] two streams, default workspaces")
    x1 = synth.make_x(synth.workload("tiny", T=700), 21, DEV)
    x2 = synth.make_x(synth.workload("tiny", T=300), 22, DEV)
    args = (tiny["w_router"], tiny["w_gate_up"], tiny["w_down"])
    r1, r2 = gtr.layer_forward(x1, *args), gtr.layer_forward(x2, *args)
    torch.cuda.synchronize()
    s1, s2 = torch.cuda.Stream(DEV), torch.cuda.Stream(DEV)
    for _ in range(3):
        s1.wait_stream(torch.cuda.current_stream(DEV))
        s2.wait_stream(torch.cuda.current_stream(DEV))
        with torch.cuda.stream(s1):
            o1 = gtr.layer_forward(x1, *args)
        with torch.cuda.stream(s2):
            o2 = gtr.layer_forward(x2, *args)
        torch.cuda.current_stream(DEV).wait_stream(s1)
        torch.cuda.current_stream(DEV).wait_stream(s2)
        torch.cuda.synchronize()
        assert torch.equal(o1, r1) and torch.equal(o2, r2)


# ------------------------------------------------------------ packed layout
def test_pack_weights_is_the_documented_permutation(tiny):
    say("[pack] tiny weights")
    pgu, pd = gtr.pack_weights(tiny["w_gate_up"], tiny["w_down"])
    for W, P in ((tiny["w_gate_up"], pgu), (tiny["w_down"], pd)):
        E, N, K = W.shape
        w = W.view(torch.int16).cpu().numpy()
        p = P.view(torch.int16).cpu().numpy().reshape(E, N // 16, K // 32, 64, 8)
        lane = np.arange(64)
        for e in (0, 17, 255):
            for b in (0, N // 16 - 1):
                for s in (0, K // 32 - 1):
                    rows = 16 * b + lane % 16
                    cols = 32 * s + 8 * (lane // 16)
                    ref = np.stack([w[e, rows, cols + j] for j in range(8)], axis=1)
                    assert np.array_equal(p[e, b, s], ref)
        # a permutation: same multiset of values
        assert np.array_equal(np.sort(w.ravel()), np.sort(P.view(torch.int16).cpu().numpy().ravel()))


@pytest.mark.parametrize("T", [64, 128, 700, 2048, 16384])
def test_packed_layout_matches_row_major_bitwise(tiny, T):
    # same operands, same k order: the packed path must reproduce the row-major
    # path bit for bit at every m-tile height
    say(f"[pack] layer T={T}")
    pgu, pd = gtr.pack_weights(tiny["w_gate_up"], tiny["w_down"])
    x = synth.make_x(synth.workload("tiny", T=T), 5, DEV)
    a = gtr.layer_forward(x, tiny["w_router"], tiny["w_gate_up"], tiny["w_down"])
    b = gtr.layer_forward(x, tiny["w_router"], pgu, pd, weight_layout=gtr.LAYOUT_PACKED)
    assert torch.equal(a, b)


# --------------------------------------------------------------- hip graphs
@pytest.mark.parametrize("variant", ["bf16", "fp8", "lora"])
def test_layer_replays_from_a_captured_graph(tiny, variant):
    # every launch of a layer call goes on the caller's stream with no host
    # synchronisation or allocation inside the library, so the call can be
    # captured into a HIP graph once and replayed on new inputs
    say(f"[graph] {variant}")
    ws = gtr.Workspace()
    wr, wgu, wd = tiny["w_router"], tiny["w_gate_up"], tiny["w_down"]
    f8 = gtr.quantize_fp8(wgu, wd) if variant == "fp8" else None
    lw = (gtr.LoraWeights(*synth.make_lora(tiny["workload"], 0, DEV), scale=2.0)
          if variant == "lora" else None)

    def call(x):
        if variant == "fp8":
            return gtr.layer_forward_fp8(x, wr, f8, workspace=ws)
        if variant == "lora":
            return gtr.layer_forward_lora(x, wr, wgu, wd, lw, workspace=ws)
        return gtr.layer_forward(x, wr, wgu, wd, workspace=ws)

    static_x = tiny["x"].clone()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        call(static_x)  # warm-up: workspace sized, launch shapes cached
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        static_out = call(static_x)
    for rep in range(3):
        x = synth.make_x(synth.workload("tiny"), 100 + rep, DEV)
        static_x.copy_(x)
        graph.replay()
        torch.cuda.synchronize()
        got = static_out.clone()
        want = call(x)          # eager work between the replays
        torch.cuda.synchronize()
        assert torch.equal(got, want), f"replay {rep} differs from the eager call"


# -------------------------------------------------------- grid independence
@pytest.mark.parametrize("variant,T", [("bf16", 128), ("bf16", 2048), ("bf16", 4096),
                                       ("bf16", 8192), ("fp8", 64), ("fp8", 2048),
                                       ("fp8", 4096), ("lora", 4096), ("lora", 8192)])
def test_layer_independent_of_grid_size(tiny, variant, T, monkeypatch):
    # each work item is computed whole by one workgroup, so capping the
    # persistent GEMM grid must not change a bit; with 8 workgroups every
    # workgroup runs a long chain of items (each starting the next one's
    # weight stream early) at every m-tile height (T 64..128 -> 32/64 rows,
    # 2048 -> 128, 4096 -> 192, 8192 -> 256 for bf16 and LoRA)
    say(f"[grid] {variant} T={T}")
    wr, wgu, wd = tiny["w_router"], tiny["w_gate_up"], tiny["w_down"]
    f8 = gtr.quantize_fp8(wgu, wd) if variant == "fp8" else None
    lw = (gtr.LoraWeights(*synth.make_lora(tiny["workload"], 0, DEV), scale=2.0)
          if variant == "lora" else None)
    x = synth.make_x(synth.workload("tiny", T=T), 11, DEV)

    def call():
        if variant == "fp8":
            return gtr.layer_forward_fp8(x, wr, f8)
        if variant == "lora":
            return gtr.layer_forward_lora(x, wr, wgu, wd, lw)
        return gtr.layer_forward(x, wr, wgu, wd)

    ref = call()
    for cap in ("8", "24", "200"):
        monkeypatch.setenv("BEAM_MOE_MAX_GRID", cap)
        out = call()
        torch.cuda.synchronize()
        assert torch.equal(out, ref), f"grid cap {cap} changes the result"
    monkeypatch.delenv("BEAM_MOE_MAX_GRID")


# ------------------------------------------------- seeded random batch shapes
@pytest.mark.parametrize("seed", range(6))
def test_expert_ffn_random_batches(tiny, seed):
    # random batch sizes and routing skews (one to three hot experts, the rest
    # uniform) for the bf16 and fp8 expert paths against the oracle; the
    # sizes land on every m-tile height and on item counts below, near and
    # above one item per workgroup
    rng = np.random.default_rng(1000 + seed)
    T = int(rng.choice([1, 7, 100, 333, 1024, 2600, 5000, 9000]))
    p = np.ones(256)
    p[rng.choice(256, int(rng.integers(1, 4)), replace=False)] = rng.uniform(20, 200)
    p /= p.sum()
    ids = np.stack([rng.choice(256, 8, replace=False, p=p) for _ in range(T)])
    say(f"[random] seed={seed} T={T}")
    npd = tiny["np"]
    x = synth.make_x(synth.workload("tiny", T=T), 40 + seed, DEV)
    xn = to_np(x)
    counts, offsets, psrc, pdst = oracle.permute(ids, 256)
    ps = torch.from_numpy(psrc.astype(np.int32)).to(DEV)
    of = torch.from_numpy(offsets.astype(np.int32)).to(DEV)
    y = gtr.expert_ffn(x, ps, of, tiny["w_gate_up"], tiny["w_down"])
    ref = oracle.expert_ffn(xn, psrc, offsets, (npd["w_gate_up"], npd["w_down"]))
    assert_close(to_np(y), ref, "y_perm")
    # the fp8 path on the same batch agrees with its bf16 result to fp8 accuracy
    f8 = gtr.quantize_fp8(tiny["w_gate_up"], tiny["w_down"])
    y8 = gtr.expert_ffn_fp8(x, ps, of, f8)
    rel = (y8.float() - y.float()).norm() / y.float().norm()
    assert float(rel) < 0.1, f"fp8 vs bf16 relative error {float(rel):.3f}"


# ---------------------------------------------------- other supported shapes
@pytest.mark.parametrize("H,I", [(512, 384), (768, 640)])
@pytest.mark.parametrize("T", [96, 2048, 4096, 8192])
def test_expert_paths_other_shapes(H, I, T):
    # hidden and intermediate sizes other than the tiny and Beam ones (I not a
    # multiple of 256: odd 64-k stage counts, 3 or 5 n-tiles per m-tile) at
    # every m-tile height, for the bf16 (row-major and packed), fp8 and LoRA
    # expert paths against the oracle
    say(f"[shapes] H={H} I={I} T={T}")
    w = synth.workload("tiny", T=T, H=H, I=I)
    wgu, wd = synth.make_experts(w, 3, DEV)
    x = synth.make_x(w, 4, DEV)
    rng = np.random.default_rng(T + H)
    ids = np.stack([rng.choice(256, 8, replace=False) for _ in range(T)])
    counts, offsets, psrc, pdst = oracle.permute(ids, 256)
    ps = torch.from_numpy(psrc.astype(np.int32)).to(DEV)
    of = torch.from_numpy(offsets.astype(np.int32)).to(DEV)
    xn, gn, dn = to_np(x), to_np(wgu), to_np(wd)
    ref = oracle.expert_ffn(xn, psrc, offsets, (gn, dn))
    y = gtr.expert_ffn(x, ps, of, wgu, wd)
    assert_close(to_np(y), ref, "y_perm")
    pgu, pdn = gtr.pack_weights(wgu, wd)
    assert torch.equal(gtr.expert_ffn(x, ps, of, pgu, pdn, weight_layout=gtr.LAYOUT_PACKED), y)
    f8 = gtr.quantize_fp8(wgu, wd)
    y8 = gtr.expert_ffn_fp8(x, ps, of, f8)
    rel = (y8.float() - y.float()).norm() / y.float().norm()
    assert float(rel) < 0.1, f"fp8 vs bf16 relative error {float(rel):.3f}"
    ts = synth.make_lora(w, 5, DEV)
    s = oracle.lora_scale(oracle.LORA_ALPHA, oracle.LORA_RANK)
    yl = gtr.expert_ffn_lora(x, ps, of, wgu, wd, gtr.LoraWeights(*ts, scale=s))
    refl = oracle.expert_ffn(xn, psrc, offsets, (gn, dn), lora=tuple(to_np(t) for t in ts),
                             lora_scale_=s)
    assert_close(to_np(yl), refl, "y_perm lora")
