"""GPU parity of the gated-delta-rule tree kernels (tree_gdn_verify /
tree_gdn_commit) against the fp64 oracle (oracle/gdn.py, the unrolled
recurrence), normwise per (item, head) at the fp32 bar 1e-4; status bits
bit-exact; invalid items untouched."""
import numpy as np
import pytest

from oracle import gdn as O
from speculative_tree_verification_amd import workloads as W
from tests.gpu_util import say

pytestmark = pytest.mark.gpu
TOL = 1e-4


@pytest.fixture(scope="module")
def bnd():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from speculative_tree_verification_amd import binding
    return binding


def f64(d):
    return {k: (v.astype(np.float64) if v.dtype == np.float32 else v) for k, v in d.items()}


def run(bnd, d):
    import torch
    dev = {k: torch.from_numpy(v).cuda() for k, v in d.items()}
    st = torch.full((d["k"].shape[0],), -7, dtype=torch.int32, device="cuda")
    o, e = bnd.gdn_verify(dev["q"], dev["k"], dev["v"], dev["g"], dev["beta"], dev["S0"], dev["parent"],
                          tree_status=st)
    S = dev["S0"].clone()
    st2 = torch.full_like(st, -7)
    bnd.gdn_commit(dev["k"], dev["g"], e, S, dev["parent"], dev["accepted"], dev["accepted_len"],
                   tree_status=st2)
    torch.cuda.synchronize()
    return o.cpu().double().numpy(), e.cpu().double().numpy(), S.cpu().double().numpy(), \
        st.cpu().numpy(), st2.cpu().numpy()


@pytest.mark.parametrize("B,T,H,dk,dv,tree", [
    (2, 1, 2, 16, 16, "recursive"), (3, 7, 2, 8, 6, "recursive"), (4, 15, 4, 128, 128, "recursive"),
    (2, 31, 3, 64, 128, "recursive"), (2, 64, 2, 128, 64, "chain"), (2, 64, 2, 32, 32, "star"),
    (2, 63, 2, 48, 40, "geometric"), (1, 40, 1, 100, 70, "recursive"),
    (2, 64, 2, 128, 128, "recursive")])
def test_gdn_matches_oracle(bnd, B, T, H, dk, dv, tree):
    d = W.make_gdn(B * 1000 + T + dk, batch=B, n_nodes=T, n_heads=H, dk=dk, dv=dv, tree=tree,
                   max_depth=8 if tree != "chain" else T, max_path_len=min(T, 9))
    say(f"[gdn] B={B} T={T} H={H} dk={dk} dv={dv} {tree}")
    o, e, S, st, st2 = run(bnd, d)
    x = f64(d)
    ref, rst = O.verify_unrolled(x["q"], x["k"], x["v"], x["g"], x["beta"], x["S0"], x["parent"])
    _, eref = O.verify_wy(x["q"], x["k"], x["v"], x["g"], x["beta"], x["S0"], x["parent"])
    Sref, cst = O.commit_unrolled(x["k"], x["v"], x["g"], x["beta"], x["S0"], x["parent"],
                                  x["accepted"], x["accepted_len"])
    assert st.tolist() == rst.tolist() == [0] * B and st2.tolist() == cst.tolist()
    err_o = max(np.max(np.abs(o[b, :, h] - ref[b, :, h])) / np.max(np.abs(ref[b, :, h]))
                for b in range(B) for h in range(H))
    err_e = max(np.max(np.abs(e[b, :, h] - eref[b, :, h])) / np.max(np.abs(eref[b, :, h]))
                for b in range(B) for h in range(H))
    err_S = max(np.max(np.abs(S[b, h] - Sref[b, h])) / np.max(np.abs(Sref[b, h]))
                for b in range(B) for h in range(H))
    say(f"    o err {err_o:.2e}  e err {err_e:.2e}  S' err {err_S:.2e}")
    assert err_o <= TOL and err_e <= TOL and err_S <= TOL, (err_o, err_e, err_S)


def test_gdn_invalid_items_untouched(bnd):
    import torch
    d = W.make_gdn(77, batch=4, n_nodes=20, n_heads=2, dk=32, dv=32, max_path_len=5)
    d["parent"][1, 0] = 4
    d["parent"][2, 11] = 13
    d["accepted"][3, 0] = 2
    d["accepted_len"][3] = max(int(d["accepted_len"][3]), 1)
    dev = {k: torch.from_numpy(v).cuda() for k, v in d.items()}
    o = torch.full_like(dev["v"], 5.0)
    st = torch.zeros(4, dtype=torch.int32, device="cuda")
    _, e = bnd.gdn_verify(dev["q"], dev["k"], dev["v"], dev["g"], dev["beta"], dev["S0"],
                          dev["parent"], o=o, tree_status=st)
    S = dev["S0"].clone()
    st2 = torch.zeros_like(st)
    bnd.gdn_commit(dev["k"], dev["g"], e, S, dev["parent"], dev["accepted"], dev["accepted_len"],
                   tree_status=st2)
    torch.cuda.synchronize()
    assert st.cpu().tolist() == [0, 1, 2, 0] and st2.cpu().tolist() == [0, 1, 2, 4]
    for b in (1, 2):
        assert (o[b] == 5.0).all()
    for b in (1, 2, 3):
        assert torch.equal(S[b], dev["S0"][b])


def test_gdn_pseudo_values_optional_and_streams(bnd):
    """o is bitwise the same when e is not requested (NULL through the C ABI)
    and when verify and commit run on another stream."""
    import ctypes
    import torch
    d = W.make_gdn(5, batch=3, n_nodes=40, n_heads=2, dk=64, dv=96, max_path_len=6)
    dev = {k: torch.from_numpy(v).cuda() for k, v in d.items()}
    args = [dev[x] for x in ("q", "k", "v", "g", "beta", "S0", "parent")]
    o1, e1 = bnd.gdn_verify(*args)
    S1 = dev["S0"].clone()
    bnd.gdn_commit(dev["k"], dev["g"], e1, S1, dev["parent"], dev["accepted"], dev["accepted_len"])
    torch.cuda.synchronize()
    o2 = torch.full_like(o1, 7.0)
    shape = bnd._gdn_shape(dev["k"], dev["v"])
    say("[gdn] verify without pseudo-values")
    rc = bnd.lib.tree_gdn_verify(ctypes.byref(shape), *[bnd._ptr(t) for t in args], bnd._ptr(o2), None,
                                 None, bnd._stream(None))
    torch.cuda.synchronize()
    assert rc == 0 and torch.equal(o1, o2)
    side = torch.cuda.Stream()
    with torch.cuda.stream(side):
        say("[gdn] verify and commit on another stream")
        o3, e3 = bnd.gdn_verify(*args, stream=side)
        S3 = dev["S0"].clone()
        bnd.gdn_commit(dev["k"], dev["g"], e3, S3, dev["parent"], dev["accepted"], dev["accepted_len"],
                       stream=side)
    side.synchronize()
    assert torch.equal(o1, o3) and torch.equal(e1, e3) and torch.equal(S1, S3)


def _dev_io(d):
    """Upload: bf16 bit patterns (uint16) become torch.bfloat16 tensors."""
    import torch
    out = {}
    for k, v in d.items():
        t = torch.from_numpy(np.ascontiguousarray(v))
        if v.dtype == np.uint16:
            t = t.view(torch.int16).view(torch.bfloat16)
        out[k] = t.cuda()
    return out


@pytest.mark.parametrize("B,T,H,dk,dv,tree", [
    (2, 1, 2, 16, 16, "recursive"), (3, 15, 4, 128, 128, "recursive"), (2, 31, 3, 64, 128, "recursive"),
    (2, 64, 2, 128, 64, "chain"), (2, 63, 2, 48, 40, "geometric"), (1, 40, 1, 100, 70, "recursive"),
    (2, 17, 2, 6, 10, "star")])
def test_gdn_bf16_inputs(bnd, B, T, H, dk, dv, tree):
    """q, k, v (and o) in bf16: o within the bf16 bar of the oracle run on the
    same (bf16-exact) values, e and S' within the fp32 bar; and the bf16 call
    equals the fp32 call on those values converted to fp32 (e and S' bit for
    bit, o as its bf16 rounding)."""
    import torch
    d = W.make_gdn(B * 2000 + T + dk, batch=B, n_nodes=T, n_heads=H, dk=dk, dv=dv, tree=tree,
                   max_depth=8 if tree != "chain" else T, max_path_len=min(T, 9), dtype=W.BF16)
    say(f"[gdn bf16] B={B} T={T} H={H} dk={dk} dv={dv} {tree}")
    dev = _dev_io(d)
    st = torch.full((B,), -7, dtype=torch.int32, device="cuda")
    o, e = bnd.gdn_verify(dev["q"], dev["k"], dev["v"], dev["g"], dev["beta"], dev["S0"], dev["parent"],
                          tree_status=st)
    S = dev["S0"].clone()
    bnd.gdn_commit(dev["k"], dev["g"], e, S, dev["parent"], dev["accepted"], dev["accepted_len"])
    # the same values as fp32
    f32 = {k: (dev[k].float() if k in ("q", "k", "v") else dev[k]) for k in dev}
    o32, e32 = bnd.gdn_verify(f32["q"], f32["k"], f32["v"], f32["g"], f32["beta"], f32["S0"], f32["parent"])
    S32 = dev["S0"].clone()
    bnd.gdn_commit(f32["k"], f32["g"], e32, S32, f32["parent"], f32["accepted"], f32["accepted_len"])
    torch.cuda.synchronize()
    assert st.cpu().tolist() == [0] * B
    assert o.dtype == torch.bfloat16 and e.dtype == torch.float32
    assert torch.equal(e, e32) and torch.equal(S, S32)
    assert torch.equal(o, o32.to(torch.bfloat16))
    x = {k: (W.to_f64(v, W.BF16) if v.dtype == np.uint16 else
             (v.astype(np.float64) if v.dtype == np.float32 else v)) for k, v in d.items()}
    ref, _ = O.verify_unrolled(x["q"], x["k"], x["v"], x["g"], x["beta"], x["S0"], x["parent"])
    _, eref = O.verify_wy(x["q"], x["k"], x["v"], x["g"], x["beta"], x["S0"], x["parent"])
    Sref, _ = O.commit_unrolled(x["k"], x["v"], x["g"], x["beta"], x["S0"], x["parent"],
                                x["accepted"], x["accepted_len"])
    on, en, Sn = (t.float().cpu().double().numpy() for t in (o, e, S))
    err = lambda a, r, sl: np.max(np.abs(a[sl] - r[sl])) / np.max(np.abs(r[sl]))
    err_o = max(err(on, ref, (b, slice(None), h)) for b in range(B) for h in range(H))
    err_e = max(err(en, eref, (b, slice(None), h)) for b in range(B) for h in range(H))
    err_S = max(err(Sn, Sref, (b, h)) for b in range(B) for h in range(H))
    say(f"    o err {err_o:.2e}  e err {err_e:.2e}  S' err {err_S:.2e}")
    assert err_o <= 2.0 ** -8 + TOL and err_e <= TOL and err_S <= TOL, (err_o, err_e, err_S)


@pytest.mark.parametrize("B,T,H,dk,dv,tree,dtype", [
    (2, 65, 2, 64, 64, "recursive", W.F32), (2, 100, 2, 128, 128, "recursive", W.F32),
    (2, 255, 2, 128, 128, "level", W.F32), (1, 256, 2, 100, 70, "recursive", W.F32),
    (2, 200, 1, 6, 10, "star", W.F32), (2, 120, 2, 32, 48, "geometric", W.F32),
    (2, 90, 1, 16, 16, "chain", W.F32),
    (2, 255, 2, 128, 128, "level", W.BF16), (2, 90, 3, 64, 128, "recursive", W.BF16)])
def test_gdn_large_trees(bnd, B, T, H, dk, dv, tree, dtype):
    """Trees of 65 to 256 nodes (the plain kernel): o within the bar of its
    dtype, e and the committed state within the fp32 bar, against the
    unrolled recurrence."""
    import torch
    d = W.make_gdn(B * 3000 + T + dk, batch=B, n_nodes=T, n_heads=H, dk=dk, dv=dv, tree=tree,
                   max_depth=8 if tree != "chain" else T, max_path_len=min(T, 9), dtype=dtype)
    say(f"[gdn large] B={B} T={T} H={H} dk={dk} dv={dv} {tree} {dtype}")
    dev = _dev_io(d)
    st = torch.full((B,), -7, dtype=torch.int32, device="cuda")
    o, e = bnd.gdn_verify(dev["q"], dev["k"], dev["v"], dev["g"], dev["beta"], dev["S0"], dev["parent"],
                          tree_status=st)
    S = dev["S0"].clone()
    st2 = torch.full_like(st, -7)
    bnd.gdn_commit(dev["k"], dev["g"], e, S, dev["parent"], dev["accepted"], dev["accepted_len"],
                   tree_status=st2)
    torch.cuda.synchronize()
    x = {k: (W.to_f64(v, W.BF16) if v.dtype == np.uint16 else
             (v.astype(np.float64) if v.dtype == np.float32 else v)) for k, v in d.items()}
    ref, rst = O.verify_unrolled(x["q"], x["k"], x["v"], x["g"], x["beta"], x["S0"], x["parent"])
    _, eref = O.verify_wy(x["q"], x["k"], x["v"], x["g"], x["beta"], x["S0"], x["parent"])
    Sref, cst = O.commit_unrolled(x["k"], x["v"], x["g"], x["beta"], x["S0"], x["parent"],
                                  x["accepted"], x["accepted_len"])
    assert st.cpu().tolist() == rst.tolist() == [0] * B and st2.cpu().tolist() == cst.tolist()
    on, en, Sn = (t.float().cpu().double().numpy() for t in (o, e, S))
    err = lambda a, r, sl: np.max(np.abs(a[sl] - r[sl])) / np.max(np.abs(r[sl]))
    err_o = max(err(on, ref, (b, slice(None), h)) for b in range(B) for h in range(H))
    err_e = max(err(en, eref, (b, slice(None), h)) for b in range(B) for h in range(H))
    err_S = max(err(Sn, Sref, (b, h)) for b in range(B) for h in range(H))
    say(f"    o err {err_o:.2e}  e err {err_e:.2e}  S' err {err_S:.2e}")
    # bf16 o: the fp32 bar plus rounding to bf16 (half an ulp, 2^-9 of the
    # element, at most 2^-8 of the row's largest magnitude)
    assert err_o <= (2.0 ** -8 + TOL if dtype == W.BF16 else TOL) and err_e <= TOL and err_S <= TOL, \
        (err_o, err_e, err_S)


def _random_case(seed):
    """A seeded shape across both kernels: T in 1..256, dk and dv in 1..128
    (sizes that are not multiples of 4 included), fp32 or bf16 rows, random
    recursive, geometric, star or chain trees."""
    rng = np.random.default_rng([4242, seed])
    T = int(rng.choice([int(rng.integers(1, 65)), int(rng.integers(65, 257))]))
    tree = str(rng.choice(["recursive", "geometric", "star"] + (["chain"] if T <= 90 else [])))
    dk, dv = (int(rng.choice([int(rng.integers(1, 129)), 128, 64])) for _ in range(2))
    dtype = W.BF16 if rng.random() < 0.4 else W.F32
    return dict(B=int(rng.integers(1, 3)), T=T, H=int(rng.integers(1, 4)), dk=dk, dv=dv, tree=tree,
                dtype=dtype)


@pytest.mark.parametrize("seed", range(12))
def test_gdn_random_shapes(bnd, seed):
    """Seeded random shapes through both kernels: o, e and the committed state
    against the unrolled recurrence (o of bf16 rows at the fp32 bar plus one
    bf16 rounding), status bits against the oracle's."""
    import torch
    c = _random_case(seed)
    B, T, H, dk, dv, tree, dtype = (c[k] for k in ("B", "T", "H", "dk", "dv", "tree", "dtype"))
    d = W.make_gdn(5000 + seed, batch=B, n_nodes=T, n_heads=H, dk=dk, dv=dv, tree=tree,
                   max_depth=T if tree == "chain" else 8, max_path_len=min(T, 9), dtype=dtype)
    say(f"[gdn random {seed}] B={B} T={T} H={H} dk={dk} dv={dv} {tree} {dtype}")
    dev = _dev_io(d)
    st = torch.full((B,), -7, dtype=torch.int32, device="cuda")
    o, e = bnd.gdn_verify(dev["q"], dev["k"], dev["v"], dev["g"], dev["beta"], dev["S0"], dev["parent"],
                          tree_status=st)
    S = dev["S0"].clone()
    st2 = torch.full_like(st, -7)
    bnd.gdn_commit(dev["k"], dev["g"], e, S, dev["parent"], dev["accepted"], dev["accepted_len"],
                   tree_status=st2)
    torch.cuda.synchronize()
    x = {k: (W.to_f64(v, W.BF16) if v.dtype == np.uint16 else
             (v.astype(np.float64) if v.dtype == np.float32 else v)) for k, v in d.items()}
    ref, rst = O.verify_unrolled(x["q"], x["k"], x["v"], x["g"], x["beta"], x["S0"], x["parent"])
    _, eref = O.verify_wy(x["q"], x["k"], x["v"], x["g"], x["beta"], x["S0"], x["parent"])
    Sref, cst = O.commit_unrolled(x["k"], x["v"], x["g"], x["beta"], x["S0"], x["parent"],
                                  x["accepted"], x["accepted_len"])
    assert st.cpu().tolist() == rst.tolist() == [0] * B and st2.cpu().tolist() == cst.tolist()
    on, en, Sn = (t.float().cpu().double().numpy() for t in (o, e, S))
    err = lambda a, r, sl: np.max(np.abs(a[sl] - r[sl])) / max(np.max(np.abs(r[sl])), 1e-30)
    err_o = max(err(on, ref, (b, slice(None), h)) for b in range(B) for h in range(H))
    err_e = max(err(en, eref, (b, slice(None), h)) for b in range(B) for h in range(H))
    err_S = max(err(Sn, Sref, (b, h)) for b in range(B) for h in range(H))
    say(f"    o err {err_o:.2e}  e err {err_e:.2e}  S' err {err_S:.2e}")
    assert err_o <= (2.0 ** -8 + TOL if dtype == W.BF16 else TOL) and err_e <= TOL and err_S <= TOL, \
        (c, err_o, err_e, err_S)


def test_gdn_large_capacity_invalid_and_optional_e(bnd):
    """A tree with more ancestor pairs than the kernel holds (a 200-node
    chain) gets status 8 and untouched outputs; invalid trees 1/2; e is
    optional (NULL gives the same o); a path row longer than 64 is
    TSV_E_UNSUPPORTED for trees past 64 nodes."""
    import ctypes
    import torch
    T = 200
    d = W.make_gdn(91, batch=4, n_nodes=T, n_heads=2, dk=16, dv=16, max_path_len=5)
    d["parent"][0] = np.array([-1] + list(range(T - 1)), np.int32)  # chain: 20100 pairs
    d["parent"][1, 0] = 3
    d["parent"][2, 150] = 170
    dev = _dev_io(d)
    o = torch.full_like(dev["v"], 5.0)
    st = torch.full((4,), -7, dtype=torch.int32, device="cuda")
    bnd.gdn_verify(dev["q"], dev["k"], dev["v"], dev["g"], dev["beta"], dev["S0"], dev["parent"], o=o,
                   tree_status=st)
    torch.cuda.synchronize()
    assert st.cpu().tolist() == [8, 1, 2, 0]
    for b in (0, 1, 2):
        assert (o[b] == 5.0).all()
    assert not (o[3] == 5.0).any()
    shape = bnd._gdn_shape(dev["k"], dev["v"])
    args = [dev[x] for x in ("q", "k", "v", "g", "beta", "S0", "parent")]
    o2 = torch.full_like(dev["v"], 5.0)
    rc = bnd.lib.tree_gdn_verify(ctypes.byref(shape), *[bnd._ptr(t) for t in args], bnd._ptr(o2), None,
                                 None, bnd._stream(None))
    torch.cuda.synchronize()
    assert rc == 0 and torch.equal(o2, o)
    acc = torch.full((4, 129), -1, dtype=torch.int32, device="cuda")
    rc = bnd.lib.tree_gdn_commit(ctypes.byref(shape), bnd._ptr(dev["k"]), bnd._ptr(dev["g"]),
                                 bnd._ptr(o), bnd._ptr(dev["S0"]), bnd._ptr(dev["parent"]), bnd._ptr(acc),
                                 bnd._ptr(dev["accepted_len"]), 129, None, bnd._stream(None))
    assert rc == 4


@pytest.mark.parametrize("L,dtype", [(65, W.F32), (80, W.BF16), (90, W.F32)])
def test_gdn_commit_long_paths(bnd, L, dtype):
    """Accepted paths past 64 nodes (90-node chains, the paths 0 .. L-1): the
    committed state against the unrolled recurrence."""
    import torch
    T = 90
    d = W.make_gdn(7000 + L, batch=2, n_nodes=T, n_heads=2, dk=64, dv=96, tree="chain", max_depth=T,
                   max_path_len=L, dtype=dtype)
    d["accepted"] = np.tile(np.arange(L, dtype=np.int32), (2, 1))
    d["accepted_len"] = np.array([L, L - 7], np.int32)
    say(f"[gdn long path] T={T} L={L} {dtype}")
    dev = _dev_io(d)
    _, e = bnd.gdn_verify(dev["q"], dev["k"], dev["v"], dev["g"], dev["beta"], dev["S0"], dev["parent"])
    S = dev["S0"].clone()
    st = torch.full((2,), -7, dtype=torch.int32, device="cuda")
    bnd.gdn_commit(dev["k"], dev["g"], e, S, dev["parent"], dev["accepted"], dev["accepted_len"], tree_status=st)
    torch.cuda.synchronize()
    x = {k: (W.to_f64(v, W.BF16) if v.dtype == np.uint16 else
             (v.astype(np.float64) if v.dtype == np.float32 else v)) for k, v in d.items()}
    Sref, cst = O.commit_unrolled(x["k"], x["v"], x["g"], x["beta"], x["S0"], x["parent"],
                                  x["accepted"], x["accepted_len"])
    assert st.cpu().tolist() == cst.tolist() == [0, 0]
    Sn = S.cpu().double().numpy()
    err = max(np.max(np.abs(Sn[b, h] - Sref[b, h])) / np.max(np.abs(Sref[b, h])) for b in range(2) for h in range(2))
    say(f"    S' err {err:.2e}")
    assert err <= TOL, err
