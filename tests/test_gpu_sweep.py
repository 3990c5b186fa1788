"""GPU parity sweep: seeded random shapes, trees and dtypes across every
kernel family (small-tree and wide-tree MFMA, plain, large trees), each
checked through the C ABI against the fp64 oracle: verify and commit at the
usual bars, tree_info and greedy acceptance bit for bit."""
import numpy as np
import pytest

from speculative_tree_verification_amd import workloads as W
from tests.gpu_util import (COMMIT_TOL, TOL, gpu_h_slices, gpu_y_slices, run_commit, run_verify,
                            say, slice_err)

pytestmark = pytest.mark.gpu

N_CASES = 40
TREES = ["recursive", "chain", "star", "geometric", "binary"]


@pytest.fixture(scope="module")
def bnd():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from speculative_tree_verification_amd import binding
    return binding


def draw_case(i):
    """Shape of sweep case i: tree sizes from 1 to 300 nodes (every kernel
    family), head_dim / d_state MFMA-eligible or odd, groups dividing heads."""
    rng = np.random.default_rng([5150, i])
    T = int(rng.choice([int(rng.integers(1, 65)), int(rng.integers(65, 257)), int(rng.integers(257, 301))],
                       p=[0.45, 0.35, 0.2]))
    G = int(rng.choice([1, 1, 2]))
    H = G * int(rng.integers(1, 4))
    mfma = rng.random() < 0.6
    P = 64 if mfma else int(rng.integers(4, 97))
    N = int(rng.choice([64, 128])) if mfma else int(rng.integers(4, 81))
    dtype = W.BF16 if (mfma or rng.random() < 0.5) else W.F32
    tree = TREES[int(rng.integers(0, len(TREES)))]
    if tree == "geometric" and not 8 <= T <= 63:
        tree = "recursive"   # the generator's geometric trees reach exactly depth 6
    if tree == "chain":
        T = min(T, 96)       # keeps the oracle's unrolled paths short
    depth = 6 if tree == "geometric" else int(rng.integers(1, 14)) if tree == "recursive" else T
    B = int(rng.integers(1, 4))
    return dict(seed=6000 + i, batch=B, n_nodes=T, n_heads=H, head_dim=P, d_state=N, n_groups=G,
                dtype=dtype, tree=tree, max_depth=depth, max_path_len=int(rng.integers(1, 12)))


@pytest.mark.parametrize("i", range(N_CASES))
def test_sweep_case(bnd, oracle_mod, i):
    import torch
    from oracle import accept as OA
    kw = draw_case(i)
    inp = W.make_custom(**kw)
    B, T, H, P, N, G = W.shape_of(inp)
    say(f"[sweep {i}] B={B} T={T} H={H} P={P} N={N} G={G} {kw['dtype']} {kw['tree']} depth<={kw['max_depth']}")
    dev = bnd.to_device(inp)
    st = torch.full((B,), -7, dtype=torch.int32, device="cuda")
    y = run_verify(bnd, dev, tree_status=st)
    h = run_commit(bnd, dev)
    d, a, s = bnd.tree_info(dev["parent"])
    draft, target = W.make_tokens(kw["seed"], inp["parent"], p_hit=0.8)
    acc, alen, nxt, ast = bnd.accept_greedy(dev["parent"], torch.from_numpy(draft).cuda(),
                                            torch.from_numpy(target).cuda(), kw["max_path_len"])
    torch.cuda.synchronize()
    assert st.cpu().tolist() == [0] * B
    sel = oracle_mod.all_pairs(inp)
    ref, _ = oracle_mod.verify(inp, kw["dtype"], sel)
    href, _ = oracle_mod.commit(inp, kw["dtype"], sel)
    err = slice_err(gpu_y_slices(y, sel), ref)
    herr = slice_err(gpu_h_slices(h, sel), href)
    say(f"    verify err {err:.2e}  commit err {herr:.2e}")
    assert err <= TOL[kw["dtype"]] and herr <= COMMIT_TOL, (err, herr)
    rd, ra, rs = oracle_mod.tree_info(inp["parent"])
    assert np.array_equal(d.cpu().numpy(), rd) and np.array_equal(a.cpu().numpy().view(np.uint64), ra)
    racc, ralen, rnxt, rst = OA.accept_greedy(inp["parent"], draft, target, kw["max_path_len"])
    assert np.array_equal(acc.cpu().numpy(), racc) and np.array_equal(alen.cpu().numpy(), ralen)
    assert np.array_equal(nxt.cpu().numpy(), rnxt)
