"""GPU: tree_ssd_commit_layers_static, the multi-layer commit that allocates
nothing (its layer table is staged into the library's fixed device array),
through the C ABI.

Two calls in a row, the second with fewer layers, a smaller batch and a
smaller tree, each checked bit for bit against tree_ssd_commit_layers on the
same operands (the same commit kernel runs in both, so the states and status
words must agree exactly). The first call takes two staging launches (more
than 64 layers); the second has an item with an invalid tree, which must keep
its state untouched. The static call must leave torch's allocator untouched.
"""
import pytest

from speculative_tree_verification_amd import workloads as W
from tests.gpu_util import say

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def bnd():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from speculative_tree_verification_amd import binding
    return binding


def _inputs(bnd, seed, n_layers, batch, T, H, dtype):
    inps = [W.make_custom(seed + l, batch=batch, n_nodes=T, n_heads=H, head_dim=64, d_state=128,
                          n_groups=1, dtype=dtype, max_path_len=min(T, 6)) for l in range(n_layers)]
    for inp in inps[1:]:  # one tree and one accepted path for every layer, as in a model step
        for k in ("parent", "accepted", "accepted_len"):
            inp[k] = inps[0][k].copy()
    return [bnd.to_device(i) for i in inps]


def _compare(bnd, devs, label, stream=None):
    import torch
    d0 = devs[0]
    B = d0["x"].shape[0]
    ref_h = [d["h0"].clone() for d in devs]
    got_h = [d["h0"].clone() for d in devs]
    ref_st = torch.full((B,), -7, dtype=torch.int32, device="cuda")
    got_st = torch.full((B,), -7, dtype=torch.int32, device="cuda")
    torch.cuda.synchronize()
    say(f"[commit_layers_static] {label}: {len(devs)} layers, B={B}, T={d0['parent'].shape[1]}")
    bnd.commit_layers([(d["x"], d["dt"], d["A"], d["B"], h) for d, h in zip(devs, ref_h)],
                      d0["parent"], d0["accepted"], d0["accepted_len"], tree_status=ref_st)
    torch.cuda.synchronize()
    before = torch.cuda.memory_stats().get("allocation.all.allocated", 0)
    layers = [(d["x"], d["dt"], d["A"], d["B"], h) for d, h in zip(devs, got_h)]
    if stream is None:
        bnd.commit_layers_static(layers, d0["parent"], d0["accepted"], d0["accepted_len"], tree_status=got_st)
    else:
        stream.wait_stream(torch.cuda.current_stream())
        bnd.commit_layers_static(layers, d0["parent"], d0["accepted"], d0["accepted_len"], tree_status=got_st,
                                 stream=stream)
        stream.synchronize()
    torch.cuda.synchronize()
    after = torch.cuda.memory_stats().get("allocation.all.allocated", 0)
    assert after == before, "the static commit allocated through torch"
    for l in range(len(devs)):
        assert torch.equal(got_h[l].view(torch.int32), ref_h[l].view(torch.int32)), (label, l)
    assert torch.equal(got_st, ref_st), label
    return got_h, got_st


def test_two_calls_in_a_row_match_commit_layers(bnd):
    import torch
    # 70 layers: two staging launches (64 + 6 table entries)
    big = _inputs(bnd, 900, 70, batch=3, T=31, H=4, dtype=W.BF16)
    _compare(bnd, big, "call 1")
    # smaller: fewer layers, items and nodes; item 1's tree is invalid (a parent
    # listed after its child), so its state must stay as it was
    small = _inputs(bnd, 1900, 3, batch=2, T=15, H=4, dtype=W.BF16)
    small[0]["parent"][1, 3] = 9
    h, st = _compare(bnd, small, "call 2")
    assert st.cpu().tolist()[0] == 0 and st.cpu().tolist()[1] != 0
    for l, d in enumerate(small):
        assert torch.equal(h[l][1].view(torch.int32), d["h0"][1].view(torch.int32)), l
        assert not torch.equal(h[l][0].view(torch.int32), d["h0"][0].view(torch.int32)), l


def test_fp32_on_a_side_stream(bnd):
    import torch
    devs = _inputs(bnd, 2900, 5, batch=2, T=9, H=2, dtype=W.F32)
    s = torch.cuda.Stream()
    _compare(bnd, devs, "fp32, side stream", stream=s)
