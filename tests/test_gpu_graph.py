"""GPU: a whole multi-layer step (verify of every layer, then the multi-layer
commit) captured as one HIP graph and replayed; every replay must give the same
bits as the same step run eagerly, with eager work and synchronisations between
the replays."""
import pytest

from speculative_tree_verification_amd import workloads as W
from tests.gpu_util import say

pytestmark = pytest.mark.gpu


def test_captured_step_replays_match_eager():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from speculative_tree_verification_amd import binding as bnd
    L = 4
    inps = [W.make_custom(600 + l, batch=2, n_nodes=15, n_heads=8, head_dim=64, d_state=128,
                          n_groups=1, dtype=W.BF16) for l in range(L)]
    for inp in inps[1:]:
        for k in ("parent", "accepted", "accepted_len"):
            inp[k] = inps[0][k].copy()
    eager = [bnd.to_device(i) for i in inps]
    graphd = [{k: v.clone() for k, v in d.items()} for d in eager]

    def prepare(ds, stream):
        vc = []
        for d in ds:
            d["y"] = torch.full_like(d["x"], float("nan"))
            vc.append(bnd.PreparedVerify(d["x"], d["dt"], d["A"], d["B"], d["C"], d["D"], d["h0"],
                                         d["parent"], d["y"], stream=stream))
        cc = bnd.PreparedCommitLayers([(d["x"], d["dt"], d["A"], d["B"], d["h0"]) for d in ds],
                                      ds[0]["parent"], ds[0]["accepted"], ds[0]["accepted_len"],
                                      stream=stream)
        return vc, cc

    ev, ec = prepare(eager, None)
    cap = torch.cuda.Stream()
    gv, gc = prepare(graphd, cap)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=cap):
        for f in gv:
            f()
        gc()
    torch.cuda.synchronize()
    for rep in range(3):
        say(f"[graph] replay {rep}")
        for f in ev:
            f()
        ec()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for l in range(L):
            assert torch.equal(eager[l]["y"].view(torch.int16), graphd[l]["y"].view(torch.int16)), (rep, l)
            assert torch.equal(eager[l]["h0"].view(torch.int32), graphd[l]["h0"].view(torch.int32)), (rep, l)
