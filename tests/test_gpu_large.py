"""GPU parity for trees of 257 to 1024 nodes (the kernels of large.hip: the
MFMA verify for bf16 head_dim 64 / d_state 64 or 128, including trees deep
enough for many 32-step passes, and the plain kernels for other shapes;
tree_info with more than four ancestor words; acceptance with 1024 threads)
against the fp64 oracle; integer outputs bit for bit."""
import numpy as np
import pytest

from speculative_tree_verification_amd import workloads as W
from tests.gpu_util import (COMMIT_TOL, TOL, gpu_h_slices, gpu_y_slices, run_commit, run_verify,
                            say, slice_err)

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def bnd():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from speculative_tree_verification_amd import binding
    return binding


def test_tree_info_large_bit_exact(bnd, oracle_mod):
    import torch
    rng = np.random.default_rng(55)
    cases = [np.arange(-1, 1023, dtype=np.int32)[None],                    # chain of 1024
             np.array([[-1] + [0] * 999], np.int32),                         # star of 1000
             W.make_custom(1, 1, 1023, 1, 1, 1, 1, W.F32, tree="binary")["parent"],
             np.stack([W.random_recursive_tree(rng, 257, 40) for _ in range(3)]),
             np.stack([W.random_recursive_tree(rng, 700, 700) for _ in range(2)]),
             np.stack([W.random_recursive_tree(rng, 1024, 12) for _ in range(2)])]
    for par in cases:
        say(f"[tree_info] batch={par.shape[0]} T={par.shape[1]}")
        d, a, s = bnd.tree_info(torch.from_numpy(par).cuda())
        rd, ra, rs = oracle_mod.tree_info(par)
        assert a.shape[2] == bnd.anc_words(par.shape[1]) == ra.shape[2]
        assert np.array_equal(s.cpu().numpy(), rs)
        assert np.array_equal(d.cpu().numpy(), rd)
        assert np.array_equal(a.cpu().numpy().view(np.uint64), ra)


def check(bnd, oracle_mod, inp, dtype, label):
    import torch
    dev = bnd.to_device(inp)
    B, T, H, P, N, G = W.shape_of(inp)
    say(f"[large] {label} B={B} T={T} H={H} P={P} N={N} G={G} {dtype}")
    st = torch.full((B,), -7, dtype=torch.int32, device="cuda")
    y = run_verify(bnd, dev, tree_status=st)
    torch.cuda.synchronize()
    assert st.cpu().tolist() == [0] * B
    sel = oracle_mod.all_pairs(inp)
    ref, rst = oracle_mod.verify(inp, dtype, sel)
    assert not rst.any()
    err = slice_err(gpu_y_slices(y, sel), ref)
    st2 = torch.full((B,), -7, dtype=torch.int32, device="cuda")
    h = run_commit(bnd, dev, tree_status=st2)
    torch.cuda.synchronize()
    assert st2.cpu().tolist() == [0] * B
    href, hst = oracle_mod.commit(inp, dtype, sel)
    herr = slice_err(gpu_h_slices(h, sel), href)
    say(f"    verify err {err:.3e}  commit err {herr:.3e}")
    assert err <= TOL[dtype] and herr <= COMMIT_TOL, (label, err, herr)


@pytest.mark.parametrize("T,H,P,N,G,dtype,tree,depth,lmax", [
    (300, 2, 16, 8, 1, W.F32, "recursive", 12, 9),
    (257, 4, 64, 128, 2, W.BF16, "recursive", 8, 9),
    (1023, 2, 64, 128, 1, W.BF16, "binary", 9, 10),
    (1000, 3, 70, 20, 1, W.F32, "star", 1, 2),
    (1024, 1, 8, 8, 1, W.F32, "chain", 1024, 700),
    (260, 1, 256, 128, 1, W.BF16, "recursive", 8, 9),
    (600, 2, 100, 36, 2, W.BF16, "geometric", 12, 13),
    (1024, 1, 64, 64, 1, W.BF16, "chain", 1024, 600),
    (700, 2, 64, 128, 1, W.BF16, "recursive", 100, 60),
    (1000, 2, 64, 128, 2, W.BF16, "star", 1, 2)])
def test_large_tree_parity(bnd, oracle_mod, T, H, P, N, G, dtype, tree, depth, lmax):
    inp = W.make_custom(T + P, batch=2, n_nodes=T, n_heads=H, head_dim=P, d_state=N, n_groups=G,
                        dtype=dtype, tree=tree, max_depth=depth, max_path_len=lmax)
    check(bnd, oracle_mod, inp, dtype, tree)


def test_large_workload_full_size_sampled(bnd, oracle_mod):
    """The 1023-node workload the benchmark times (batch 4, 80 heads, complete
    binary trees, each (item, head) split over two work-groups), on sampled
    (item, head) slices the oracle computes one by one."""
    import torch
    inp = W.make_custom(23, batch=4, n_nodes=1023, n_heads=80, head_dim=64, d_state=128, n_groups=1,
                        dtype=W.BF16, tree="binary", max_path_len=10)
    rng = np.random.default_rng(45)
    sel = sorted({(int(rng.integers(0, 4)), int(rng.integers(0, 80))) for _ in range(10)} | {(0, 0), (3, 79)})
    dev = bnd.to_device(inp)
    say("[large] full-size workload B=4 T=1023 H=80")
    st = torch.full((4,), -7, dtype=torch.int32, device="cuda")
    y = torch.full_like(dev["x"], float("nan"))
    run_verify(bnd, dev, y=y, tree_status=st)
    h = run_commit(bnd, dev, tree_status=st)
    torch.cuda.synchronize()
    assert st.cpu().tolist() == [0] * 4
    assert torch.isfinite(y.float()).all()
    ref, _ = oracle_mod.verify(inp, W.BF16, sel)
    href, _ = oracle_mod.commit(inp, W.BF16, sel)
    err, herr = slice_err(gpu_y_slices(y, sel), ref), slice_err(gpu_h_slices(h, sel), href)
    say(f"    verify err {err:.3e}  commit err {herr:.3e}")
    assert err <= TOL[W.BF16] and herr <= COMMIT_TOL, (err, herr)


def test_large_mfma_units_across_items(bnd, oracle_mod):
    """The MFMA kernel over more (item, head) units than compute units: 4 items
    x 95 heads of 300-node trees, items 1 and 2 with invalid trees, whose
    outputs stay untouched while every head of items 0 and 3 is computed."""
    import torch
    inp = W.make_custom(77, batch=4, n_nodes=300, n_heads=95, head_dim=64, d_state=64, n_groups=1,
                        dtype=W.BF16, tree="recursive", max_depth=12, max_path_len=9)
    inp["parent"][1, 200] = 250  # parent after child
    inp["parent"][2, 0] = 5      # bad root
    dev = bnd.to_device(inp)
    say("[large] persistent units B=4 T=300 H=95, items 1 and 2 invalid")
    y = torch.full_like(dev["x"], 1232.0)
    st = torch.full((4,), -1, dtype=torch.int32, device="cuda")
    run_verify(bnd, dev, y=y, tree_status=st)
    torch.cuda.synchronize()
    assert st.cpu().tolist() == [0, 2, 1, 0]
    assert (y[1].float() == 1232.0).all() and (y[2].float() == 1232.0).all()
    good = [(b, h) for b in (0, 3) for h in range(95)]
    ref, _ = oracle_mod.verify(inp, W.BF16, good)
    err = slice_err(gpu_y_slices(y, good), ref)
    say(f"    verify err {err:.3e}")
    assert err <= TOL[W.BF16], err


def test_large_invalid_items_untouched(bnd, oracle_mod):
    import torch
    inp = W.make_custom(91, batch=5, n_nodes=400, n_heads=2, head_dim=32, d_state=16, n_groups=1,
                        dtype=W.BF16, max_depth=10, max_path_len=8)
    inp["parent"][1, 0] = 3        # bad root
    inp["parent"][2, 350] = 360    # parent after child
    inp["accepted"][3, 0] = 1      # path not from the root
    inp["accepted_len"][3] = max(int(inp["accepted_len"][3]), 1)
    inp["accepted_len"][4] = 9     # longer than max_path_len
    dev = bnd.to_device(inp)
    sentinel = torch.full_like(dev["x"], 1232.0)
    st = torch.full((5,), -1, dtype=torch.int32, device="cuda")
    y = run_verify(bnd, dev, y=sentinel, tree_status=st)
    assert st.cpu().tolist() == [0, 1, 2, 0, 0]
    yc = y.float().cpu()
    assert (yc[1] == 1232.0).all() and (yc[2] == 1232.0).all()
    good = [(b, h) for b in (0, 3, 4) for h in range(2)]
    ref, _ = oracle_mod.verify(inp, W.BF16, good)
    assert slice_err(gpu_y_slices(y, good), ref) <= TOL[W.BF16]
    st = torch.full((5,), -1, dtype=torch.int32, device="cuda")
    h = run_commit(bnd, dev, tree_status=st)
    _, rst = oracle_mod.commit(inp, W.BF16, [(b, 0) for b in range(5)])
    assert st.cpu().tolist() == rst.tolist() == [0, 1, 2, 4, 4]
    for b in (1, 2, 3, 4):
        assert torch.equal(h[b], dev["h0"][b])


def test_large_commit_layers_match_single(bnd):
    import torch
    layers_in = [W.make_custom(300 + l, batch=2, n_nodes=500, n_heads=3, head_dim=64, d_state=128,
                               n_groups=1, dtype=W.BF16, max_depth=9, max_path_len=10)
                 for l in range(3)]
    par, acc, alen = (layers_in[0][k] for k in ("parent", "accepted", "accepted_len"))
    devs = []
    for inp in layers_in:
        inp["parent"], inp["accepted"], inp["accepted_len"] = par, acc, alen
        devs.append(bnd.to_device(inp))
    singles = [run_commit(bnd, d) for d in devs]
    hs = [d["h0"].clone() for d in devs]
    say("[large] commit_layers T=500 x3")
    bnd.commit_layers([(d["x"], d["dt"], d["A"], d["B"], hh) for d, hh in zip(devs, hs)],
                      devs[0]["parent"], devs[0]["accepted"], devs[0]["accepted_len"])
    torch.cuda.synchronize()
    for a, b in zip(singles, hs):
        assert torch.equal(a, b)


def test_large_accept_greedy(bnd):
    import torch
    from oracle import accept as OA
    rng = np.random.default_rng(66)
    par = np.stack([W.random_recursive_tree(rng, 1000, 40) for _ in range(3)]
                   + [np.arange(-1, 999, dtype=np.int32)])
    for repeats in (False, True):
        draft, target = W.make_tokens(81 + repeats, par, p_hit=0.8, repeats=repeats)
        for lmax in (1, 16, 1000):
            say(f"[large] accept T=1000 repeats={repeats} max_path_len={lmax}")
            acc, alen, nxt, st = bnd.accept_greedy(
                torch.from_numpy(par).cuda(), torch.from_numpy(draft).cuda(),
                torch.from_numpy(target).cuda(), lmax)
            racc, ralen, rnxt, rst = OA.accept_greedy(par, draft, target, lmax)
            assert np.array_equal(st.cpu().numpy(), rst)
            assert np.array_equal(alen.cpu().numpy(), ralen)
            assert np.array_equal(acc.cpu().numpy(), racc)
            assert np.array_equal(nxt.cpu().numpy(), rnxt)
