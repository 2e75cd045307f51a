"""The largest batch the tests run: 2^20 tokens at the small layer shape
(hidden 256, intermediate 128, 256 experts), i.e. 8,388,608 (token, slot)
pairs, 8,192 permutation chunks, a 4.3 GB y_perm and 2 GB of h (byte offsets
past 2^32).  Global invariants are checked on the device for every pair;
the routing and the output of sampled tokens (each token's result depends
only on its own row) against the oracle."""
import numpy as np
import pytest
import torch

import grouped_top_routing_amd as gtr
import oracle
import synth
from parity_util import assert_close, check_routing, layer_reference, say, to_np

pytestmark = pytest.mark.gpu
DEV = torch.device("cuda", 0)


@pytest.mark.timeout(600)
def test_million_token_batch():
    T = 1 << 20
    w = synth.workload("tiny", T=T)
    d = synth.make_inputs("tiny", 0, device=DEV)
    x = synth.make_x(w, 3, DEV)
    say(f"[large] T={T}: layer_forward")
    ws = gtr.Workspace()
    out, ids, wts = gtr.layer_forward(x, d["w_router"], d["w_gate_up"], d["w_down"],
                                      return_routing=True, workspace=ws)
    torch.cuda.synchronize()
    assert torch.isfinite(out.float()).all()

    # every pair: a stable permutation of the pairs by expert
    say("[large] permutation invariants on the device")
    c, o, ps, pd = gtr.permute(ids, workspace=ws)
    n = 8 * T
    assert int(c.sum()) == n and int(o[-1]) == n and int(o[0]) == 0
    assert bool((o[1:] - o[:-1] == c).all())
    assert torch.equal(torch.sort(ps.long()).values, torch.arange(n, device=DEV))
    assert torch.equal(pd.long()[ps.long()], torch.arange(n, device=DEV))
    # rows of one expert hold its pairs in token order
    e_of_row = ids.reshape(-1).long()[ps.long()]
    assert bool((e_of_row[1:] >= e_of_row[:-1]).all())
    same = e_of_row[1:] == e_of_row[:-1]
    assert bool((ps[1:][same] > ps[:-1][same]).all())
    # 8 distinct experts per token
    srt = torch.sort(ids.long(), dim=1).values
    assert bool((srt[:, 1:] != srt[:, :-1]).all())
    del c, o, ps, pd, e_of_row, same, srt

    # sampled tokens, the last one included, against the oracle
    rng = np.random.default_rng(7)
    sample = np.unique(np.concatenate([rng.choice(T, 500, replace=False), [0, T - 1]]))
    st = torch.from_numpy(sample).to(DEV)
    xs = to_np(x[st])
    npw = {k: to_np(d[k]) for k in ("w_router", "w_gate_up", "w_down")}
    say(f"[large] oracle on {len(sample)} sampled tokens")
    ref = oracle.layer_forward(xs, npw["w_router"], (npw["w_gate_up"], npw["w_down"]))
    ids_s, w_s = to_np(ids[st]), to_np(wts[st])
    nf, nd = check_routing(ids_s, w_s, ref["route"])
    mx, mn = assert_close(to_np(out[st]),
                          layer_reference(ids_s, ref, xs, (npw["w_gate_up"], npw["w_down"])),
                          f"layer output, {len(sample)} sampled tokens of {T}")
    say(f"  flagged={nf} differing={nd} max_rel={mx:.3e} mean_rel={mn:.3e}")
