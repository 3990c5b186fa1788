"""GPU parity of the unrolled and snapshot forms against the fp64 oracle.

Unrolled: the plan (leaves and their root paths) is bit-exact against
oracle/unroll.py; after the gather and the plain sequence scan, every
position of every sequence must carry the oracle's output for the node there,
and each sequence's final state the oracle's state after its leaf's root path.
Snapshot: every node's output, every node's stored state, and the commit
(a copy of the last accepted node's state) against the oracle.
"""
import numpy as np
import pytest

from oracle import unroll as U
from speculative_tree_verification_amd import workloads as W
from tests.gpu_util import COMMIT_TOL, TOL, gpu_h_slices, gpu_y_slices, say, slice_err

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def bnd():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from speculative_tree_verification_amd import binding
    return binding


def _i32(torch, a):
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.int32)).cuda()


PLAN_CASES = [("binary", 7), ("recursive", 31), ("level", 255), ("geometric", 63), ("chain", 40),
              ("star", 100), ("recursive", 700)]


@pytest.mark.parametrize("tree,T", PLAN_CASES)
def test_unroll_plan_bit_exact(bnd, tree, T):
    import torch
    inp = W.make_custom(5100 + T, batch=4, n_nodes=T, n_heads=1, head_dim=4, d_state=4, n_groups=1,
                        dtype=W.F32, tree=tree, max_depth=9)
    par = inp["parent"]
    Lcap, S = bnd.unroll_capacity(par)
    say(f"[unroll_plan] {tree} T={T} Lcap={Lcap} S={S}")
    nodes, lens, nl, st = bnd.unroll_plan(_i32(torch, par), Lcap, S)
    rn, rl, rnl, rst = U.unroll_plan(par, Lcap, S)
    torch.cuda.synchronize()
    assert np.array_equal(st.cpu().numpy(), rst) and not rst.any()
    assert np.array_equal(nl.cpu().numpy(), rnl)
    assert np.array_equal(lens.cpu().numpy(), rl)
    assert np.array_equal(nodes.cpu().numpy(), rn)


def test_unroll_plan_invalid_and_over_capacity(bnd):
    import torch
    par = np.array([[-1, 0, 0, 0, 1], [-1, 0, 1, 2, 3], [0, 0, 0, 0, 0], [-1, 2, 0, 1, 1],
                    [-1, 0, 0, 1, 1]], np.int32)
    nodes, lens, nl, st = bnd.unroll_plan(_i32(torch, par), 3, 4)
    rn, rl, rnl, rst = U.unroll_plan(par, 3, 4)
    torch.cuda.synchronize()
    assert st.cpu().tolist() == rst.tolist() == [0, 8, 1, 2, 0]
    assert np.array_equal(nl.cpu().numpy(), rnl)
    assert np.array_equal(lens.cpu().numpy(), rl)
    assert np.array_equal(nodes.cpu().numpy(), rn)


def _unrolled_check(bnd, oracle_mod, inp, dtype, label):
    import torch
    dev = bnd.to_device(inp)
    B, T, H, P, N, G = W.shape_of(inp)
    Lcap, S = bnd.unroll_capacity(inp["parent"])
    say(f"[unrolled] {label} B={B} T={T} H={H} Lcap={Lcap} S={S}")
    nodes, lens, nl, st = bnd.unroll_plan(dev["parent"], Lcap, S)
    u = bnd.unroll_gather(dev["x"], dev["dt"], dev["B"], dev["C"], dev["h0"], nodes, lens)
    ns = B * Lcap
    y_u = bnd.seq_scan(u["x_u"], u["dt_u"], dev["A"], u["B_u"], u["C_u"], dev["D"], u["h0_u"],
                       lens.reshape(ns))
    torch.cuda.synchronize()
    nodes, lens, nl = nodes.cpu().numpy(), lens.cpu().numpy(), nl.cpu().numpy()
    yref, _ = oracle_mod.verify_full(inp, dtype)                     # [B, T, H, P]
    yu = y_u.float().cpu().double().numpy().reshape(B, Lcap, S, H, P)
    hu = u["h0_u"].cpu().double().numpy().reshape(B, Lcap, H, P, N)
    got, want, hgot, hwant = [], [], [], []
    for b in range(B):
        for l in range(nl[b]):
            path = nodes[b, l, :lens[b, l]]
            for h in range(H):
                got.append(yu[b, l, :len(path), h])
                want.append(yref[b, path, h])
            # final state of the sequence: the oracle's commit along the leaf's path
            d = dict(inp)
            acc = np.full((B, S), -1, np.int32)
            alen = np.zeros(B, np.int32)
            acc[b, :len(path)] = path
            alen[b] = len(path)
            d["accepted"], d["accepted_len"] = acc, alen
            href, _ = oracle_mod.commit(d, dtype, [(b, h) for h in range(H)])
            hgot.append(hu[b, l])
            hwant.append(href)
    err = max(slice_err(g[None], w[None]) for g, w in zip(got, want))
    herr = slice_err(np.concatenate(hgot), np.concatenate(hwant))
    say(f"    unrolled y err {err:.3e}, final-state err {herr:.3e}")
    assert err <= TOL[dtype], (label, err)
    assert herr <= COMMIT_TOL, (label, herr)


@pytest.mark.parametrize("cid", [0, 1, 2, 3])
def test_unrolled_scan_parity(bnd, oracle_mod, cid):
    cfg = W.CONFIGS[cid]
    inp = W.make_inputs(cid, 0)
    if cid in (2, 3):  # a few items keep the per-sequence oracle calls short
        inp = {k: (v[:3] if k not in ("A", "D") else v) for k, v in inp.items()}
    _unrolled_check(bnd, oracle_mod, inp, cfg.dtype, cfg.name)


@pytest.mark.parametrize("T,P,N,G,dtype", [(9, 16, 8, 1, W.F32), (40, 64, 128, 2, W.BF16),
                                           (25, 24, 40, 1, W.BF16), (120, 64, 64, 1, W.F32)])
def test_unrolled_scan_shapes(bnd, oracle_mod, T, P, N, G, dtype):
    inp = W.make_custom(5200 + T, batch=2, n_nodes=T, n_heads=2 * G, head_dim=P, d_state=N, n_groups=G,
                        dtype=dtype, max_depth=20)
    _unrolled_check(bnd, oracle_mod, inp, dtype, f"T={T} P={P} N={N}")


def _snapshot_check(bnd, oracle_mod, inp, dtype, label, sel=None):
    import torch
    dev = bnd.to_device(inp)
    B, T, H, P, N, G = W.shape_of(inp)
    st = torch.full((B,), -7, dtype=torch.int32, device="cuda")
    say(f"[snapshot] {label} B={B} T={T} H={H}")
    y, states = bnd.snapshot_verify(dev["x"], dev["dt"], dev["A"], dev["B"], dev["C"], dev["D"], dev["h0"],
                                    dev["parent"], tree_status=st)
    h = dev["h0"].clone()
    st2 = torch.full((B,), -7, dtype=torch.int32, device="cuda")
    bnd.snapshot_commit(states, h, dev["parent"], dev["accepted"], dev["accepted_len"], tree_status=st2)
    torch.cuda.synchronize()
    assert st.cpu().tolist() == [0] * B and st2.cpu().tolist() == [0] * B
    sel = oracle_mod.all_pairs(inp) if sel is None else sel
    yref, _ = oracle_mod.verify(inp, dtype, sel)
    err = slice_err(gpu_y_slices(y, sel), yref)
    href, _ = oracle_mod.commit(inp, dtype, sel)
    herr = slice_err(gpu_h_slices(h, sel), href)
    few = sel[:4]
    sref = U.node_states(oracle_mod, inp, dtype, few)
    serr = max(slice_err(states[b, hh].cpu().double().numpy()[None], sref[k][None])
               for k, (b, hh) in enumerate(few))
    say(f"    y err {err:.3e}, commit err {herr:.3e}, node-state err {serr:.3e}")
    assert err <= TOL[dtype], (label, err)
    assert herr <= COMMIT_TOL, (label, herr)
    assert serr <= COMMIT_TOL, (label, serr)


@pytest.mark.parametrize("cid", [0, 1, 2, 3])
def test_snapshot_parity(bnd, oracle_mod, cid):
    cfg = W.CONFIGS[cid]
    inp = W.make_inputs(cid, 0)
    sel = None
    if cid in (2, 3):
        rng = np.random.default_rng(52 + cid)
        B, T, H, P = inp["x"].shape
        sel = sorted({(int(rng.integers(0, B)), int(rng.integers(0, H))) for _ in range(12)})
    _snapshot_check(bnd, oracle_mod, inp, cfg.dtype, cfg.name, sel=sel)


@pytest.mark.parametrize("T,P,N,tree,dtype", [(33, 16, 24, "chain", W.F32), (64, 64, 128, "star", W.BF16),
                                              (255, 64, 128, "level", W.BF16), (5, 8, 256, "binary", W.F32)])
def test_snapshot_shapes(bnd, oracle_mod, T, P, N, tree, dtype):
    inp = W.make_custom(5300 + T, batch=2, n_nodes=T, n_heads=2, head_dim=P, d_state=N, n_groups=1,
                        dtype=dtype, tree=tree, max_depth=10, max_path_len=min(T, 12))
    _snapshot_check(bnd, oracle_mod, inp, dtype, f"{tree} T={T} P={P} N={N}")


def test_snapshot_invalid_items_untouched(bnd):
    import torch
    inp = W.make_custom(5400, batch=4, n_nodes=20, n_heads=2, head_dim=16, d_state=16, n_groups=1,
                        dtype=W.F32, max_path_len=5)
    inp["parent"][1, 0] = 2
    inp["parent"][2, 9] = 12
    inp["accepted"][3, 0] = 4  # a path that does not start at the root
    dev = bnd.to_device(inp)
    y = torch.full_like(dev["x"], 77.0)
    states = torch.full((4, 2, 20, 16, 16), 55.0, device="cuda")
    st = torch.full((4,), -1, dtype=torch.int32, device="cuda")
    bnd.snapshot_verify(dev["x"], dev["dt"], dev["A"], dev["B"], dev["C"], dev["D"], dev["h0"], dev["parent"],
                        y=y, states=states, tree_status=st)
    h = dev["h0"].clone()
    st2 = torch.full((4,), -1, dtype=torch.int32, device="cuda")
    bnd.snapshot_commit(states, h, dev["parent"], dev["accepted"], dev["accepted_len"], tree_status=st2)
    torch.cuda.synchronize()
    assert st.cpu().tolist() == [0, 1, 2, 0] and st2.cpu().tolist() == [0, 1, 2, 4]
    for b in (1, 2):
        assert (y[b] == 77.0).all() and (states[b] == 55.0).all()
    for b in (1, 2, 3):
        assert torch.equal(h[b], dev["h0"][b])
