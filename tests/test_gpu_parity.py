"""GPU parity: the HIP path through the C ABI against the fp64 oracle.

Floating-point outputs are compared with the normwise per-(item, head) error
max|gpu - ref| / max|ref| (bar: 1e-4 for fp32 inputs, 2e-2 for bf16 inputs);
integer outputs (depth, ancestor bits, status bits) must match bit for bit.
"""
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


def check_full(bnd, oracle_mod, inp, dtype, label, sel=None, **kw):
    """Verify + commit of one input dict; compares the selected (b, h) slices."""
    import torch
    dev = bnd.to_device(inp)
    B, T, H, P, N, G = W.shape_of(inp)
    st = torch.full((B,), -7, dtype=torch.int32, device="cuda")
    say(f"[verify] {label} B={B} T={T} H={H} P={P} N={N} G={G} {dtype} {kw}")
    y = run_verify(bnd, dev, tree_status=st, **kw)
    torch.cuda.synchronize()
    assert st.cpu().tolist() == [0] * B
    sel = oracle_mod.all_pairs(inp) if sel is None else sel
    ref, rst = oracle_mod.verify(inp, dtype, sel)
    assert not rst.any()
    err = slice_err(gpu_y_slices(y, sel), ref)
    say(f"    verify err {err:.3e}")
    assert err <= TOL[dtype], (label, err)
    st2 = torch.full((B,), -7, dtype=torch.int32, device="cuda")
    say(f"[commit] {label}")
    h = run_commit(bnd, dev, tree_status=st2)
    torch.cuda.synchronize()
    assert st2.cpu().tolist() == [0] * B
    href, hst = oracle_mod.commit(inp, dtype, sel)
    assert not hst.any()
    herr = slice_err(gpu_h_slices(h, sel), href)
    say(f"    commit err {herr:.3e}")
    assert herr <= COMMIT_TOL, (label, herr)
    return y, h, dev


@pytest.mark.parametrize("cid", [0, 1, 2, 3])
def test_config_parity(bnd, oracle_mod, cid):
    cfg = W.CONFIGS[cid]
    layers = [0, cfg.layers - 1] if cfg.layers > 1 else [0]
    for layer in layers:
        inp = W.make_inputs(cid, layer)
        check_full(bnd, oracle_mod, inp, cfg.dtype, f"config {cid} layer {layer}")


def test_config4_full_size_sampled(bnd, oracle_mod):
    """Wide-tree stress at full size (64 x 80 heads, T = 255) with the launch the
    benchmark times; outputs checked on sampled (item, head) slices."""
    import torch
    inp = W.make_inputs(4)
    rng = np.random.default_rng(44)
    sel = sorted({(int(rng.integers(0, 64)), int(rng.integers(0, 80))) for _ in range(24)})
    sel += [(0, 0), (63, 79)]
    y, h, dev = check_full(bnd, oracle_mod, inp, W.BF16, "config 4", sel=sel)
    assert torch.isfinite(y.float()).all()
    assert torch.isfinite(h).all()


def test_tree_info_bit_exact(bnd, oracle_mod):
    import torch
    rng = np.random.default_rng(5)
    cases = [W.make_inputs(c)["parent"] for c in range(4)]
    cases.append(W.make_tree_and_path(4)[0])
    cases.append(np.arange(-1, 255, dtype=np.int32)[None])          # chain of 256
    cases.append(np.array([[-1] + [0] * 255], np.int32))             # star of 256
    cases.append(np.stack([W.random_recursive_tree(rng, 200, 199) for _ in range(5)]))
    cases.append(np.array([[-1]], np.int32))
    for par in cases:
        say(f"[tree_info] batch={par.shape[0]} T={par.shape[1]}")
        d, a, s = bnd.tree_info(torch.from_numpy(par).cuda())
        rd, ra, rs = oracle_mod.tree_info(par)
        assert np.array_equal(s.cpu().numpy(), rs)
        assert np.array_equal(d.cpu().numpy(), rd)
        assert np.array_equal(a.cpu().numpy().view(np.uint64), ra)


def test_tree_info_invalid_items(bnd, oracle_mod):
    import torch
    par = np.tile(np.array([-1, 0, 0, 1, 1, 2, 2], np.int32), (4, 1))
    par[1, 0] = 0
    par[2, 4] = 6
    par[3, 3] = -2
    d = torch.full((4, 7), -5, dtype=torch.int32, device="cuda")
    a = torch.full((4, 7, 4), -5, dtype=torch.int64, device="cuda")
    d, a, s = bnd.tree_info(torch.from_numpy(par).cuda(), depth=d, anc=a)
    rd, ra, rs = oracle_mod.tree_info(par)
    assert s.cpu().tolist() == rs.tolist() == [0, 1, 2, 2]
    assert np.array_equal(d.cpu().numpy()[0], rd[0])
    assert (d.cpu().numpy()[1:] == -5).all() and (a.cpu().numpy()[1:] == -5).all()


TINY = [(1, 128, 1, "chain"), (2, 64, 1, "chain"), (7, 128, 2, "binary"), (11, 64, 1, "recursive"),
        (15, 128, 1, "recursive"), (15, 128, 2, "binary"), (16, 64, 2, "chain"), (16, 128, 1, "star")]


@pytest.mark.parametrize("T,N,G,tree", TINY)
def test_tiny_tree_kernel(bnd, oracle_mod, T, N, G, tree):
    """Trees of at most 16 nodes take the one-wave kernel by default (outputs
    written into NaN-filled buffers); the 64-node small-tree kernel, forced,
    meets the same bar on the same inputs."""
    import torch
    inp = W.make_custom(900 + 17 * T + N + G, batch=3, n_nodes=T, n_heads=6, head_dim=64, d_state=N,
                        n_groups=G, dtype=W.BF16, tree=tree, max_depth=min(T, 5), max_path_len=T)
    dev = bnd.to_device(inp)
    y_nan = torch.full_like(dev["x"], float("nan"))
    check_full(bnd, oracle_mod, inp, W.BF16, f"tiny T={T} {tree}", y=y_nan)
    assert torch.isfinite(y_nan.float()).all()
    check_full(bnd, oracle_mod, inp, W.BF16, f"tiny T={T} {tree} small kernel", force_small=True)


def test_tiny_tree_invalid_items_untouched(bnd, oracle_mod):
    import torch
    inp = W.make_custom(77, batch=4, n_nodes=12, n_heads=4, head_dim=64, d_state=128, n_groups=2,
                        dtype=W.BF16, max_depth=4)
    inp["parent"][1, 0] = 2        # bad root
    inp["parent"][2, 9] = 9        # own parent
    inp["parent"][3, 4] = -3       # negative parent
    dev = bnd.to_device(inp)
    sentinel = torch.full_like(dev["x"], 1232.0)
    st = torch.full((4,), -1, dtype=torch.int32, device="cuda")
    say("[verify] tiny-tree invalid items")
    y = run_verify(bnd, dev, y=sentinel, tree_status=st)
    torch.cuda.synchronize()
    assert st.cpu().tolist() == [0, 1, 2, 2]
    yc = y.float().cpu()
    assert (yc[1:] == 1232.0).all()
    good = [(0, h) for h in range(4)]
    ref, _ = oracle_mod.verify(inp, W.BF16, good)
    assert slice_err(gpu_y_slices(y, good), ref) <= TOL[W.BF16]


RAGGED = [(1, 128, 1), (5, 64, 1), (16, 128, 2), (17, 128, 1), (31, 64, 2), (33, 128, 1),
          (64, 64, 1), (65, 128, 2), (100, 64, 1), (129, 128, 1), (200, 64, 2), (256, 128, 1)]


@pytest.mark.parametrize("T,N,G", RAGGED)
def test_ragged_bf16(bnd, oracle_mod, T, N, G):
    inp = W.make_custom(T * 7 + N + G, batch=3, n_nodes=T, n_heads=4, head_dim=64, d_state=N,
                        n_groups=G, dtype=W.BF16, tree="recursive", max_depth=10)
    check_full(bnd, oracle_mod, inp, W.BF16, f"ragged T={T}")
    check_full(bnd, oracle_mod, inp, W.BF16, f"ragged T={T} generic", force_generic=True)
    if T <= 64:  # the wide-tree kernel also takes small trees when asked
        check_full(bnd, oracle_mod, inp, W.BF16, f"ragged T={T} wide", force_wide=True)


@pytest.mark.parametrize("T,P,N,G,H", [(7, 16, 8, 1, 1), (45, 24, 12, 1, 3), (70, 64, 128, 2, 4),
                                       (1, 8, 4, 1, 2), (130, 32, 16, 3, 6), (5, 256, 256, 1, 1)])
def test_fp32_generic(bnd, oracle_mod, T, P, N, G, H):
    inp = W.make_custom(T + P, batch=2, n_nodes=T, n_heads=H, head_dim=P, d_state=N, n_groups=G,
                        dtype=W.F32, tree="recursive", max_depth=12)
    check_full(bnd, oracle_mod, inp, W.F32, f"fp32 T={T} P={P} N={N}")


@pytest.mark.parametrize("T,tree", [(256, "chain"), (100, "chain"), (256, "star"),
                                    (255, "level"), (63, "geometric"), (64, "chain"),
                                    (64, "star"), (17, "chain"), (1, "chain")])
def test_tree_shapes_bf16(bnd, oracle_mod, T, tree):
    """Deep chains exceed the cached ancestor-pair budget and take the on-the-fly
    score path; stars and level trees are the wide extremes."""
    inp = W.make_custom(T, batch=2, n_nodes=T, n_heads=2, head_dim=64, d_state=128, n_groups=1,
                        dtype=W.BF16, tree=tree, max_depth=6, max_path_len=T)
    check_full(bnd, oracle_mod, inp, W.BF16, f"{tree} T={T}")


@pytest.mark.parametrize("T,N", [(15, 128), (40, 128), (200, 128), (31, 64)])
def test_heads_per_block_bitwise_invariant(bnd, T, N):
    """Every heads-per-block choice gives the same bits, call after call, into
    NaN-filled outputs (a missed write or a race shows up as a difference).
    One-head work-groups of the small-tree kernel stage h0 and y through LDS,
    wider ones do not, so this also pins those two forms to each other."""
    import torch
    inp = W.make_custom(3 + T, batch=2, n_nodes=T, n_heads=20, head_dim=64, d_state=N,
                        n_groups=1, dtype=W.BF16)
    dev = bnd.to_device(inp)
    ref = None
    for rep in range(3):
        for hb in (1, 2, 4, 5, 10, 20):
            say(f"[verify] T={T} heads_per_block={hb} rep {rep}")
            y = torch.full_like(dev["x"], float("nan"))
            run_verify(bnd, dev, heads_per_block=hb, y=y, force_small=T <= 16)
            y = y.view(torch.int16).cpu()
            ref = y if ref is None else ref
            assert torch.equal(y, ref), (T, hb, rep)


def test_invalid_trees_leave_outputs_untouched(bnd, oracle_mod):
    import torch
    inp = W.make_custom(11, batch=5, n_nodes=20, n_heads=4, head_dim=64, d_state=64, n_groups=2,
                        dtype=W.BF16)
    inp["parent"][1, 0] = 3        # bad root
    inp["parent"][2, 7] = 9        # parent after child
    inp["parent"][3, 5] = -1       # second root
    inp["accepted_len"][4] = 0     # empty path: commit is a no-op
    dev = bnd.to_device(inp)
    for generic in (False, True):
        sentinel = torch.full_like(dev["x"], 1232.0)  # exactly representable in bf16
        st = torch.full((5,), -1, dtype=torch.int32, device="cuda")
        say(f"[verify] invalid trees generic={generic}")
        y = run_verify(bnd, dev, y=sentinel, tree_status=st, force_generic=generic)
        assert st.cpu().tolist() == [0, 1, 2, 2, 0]
        yc = y.float().cpu()
        for b in (1, 2, 3):
            assert (yc[b] == 1232.0).all()
        good = [(b, h) for b in (0, 4) for h in range(4)]
        ref, _ = oracle_mod.verify(inp, W.BF16, good)
        assert slice_err(gpu_y_slices(y, good), ref) <= TOL[W.BF16]
    st = torch.full((5,), -1, dtype=torch.int32, device="cuda")
    h = run_commit(bnd, dev, tree_status=st)
    assert st.cpu().tolist() == [0, 1, 2, 2, 0]
    for b in (1, 2, 3, 4):
        assert torch.equal(h[b], dev["h0"][b])


def test_invalid_paths_leave_state_untouched(bnd, oracle_mod):
    import torch
    inp = W.make_custom(12, batch=6, n_nodes=30, n_heads=2, head_dim=64, d_state=128, n_groups=1,
                        dtype=W.BF16, max_path_len=6)
    par = inp["parent"]
    acc, alen = inp["accepted"], inp["accepted_len"]
    for b in range(6):
        p = W.root_path(par[b], 29)[:6]
        acc[b] = -1
        acc[b, :len(p)] = p
        alen[b] = len(p)
    acc[1, 0] = 2                      # does not start at the root
    if alen[2] >= 2:
        acc[2, 1] = 0                  # broken chain
    else:
        alen[2] = 2
        acc[2, 1] = 0
    alen[3] = 7                        # longer than max_path_len
    alen[4] = -1
    acc[5, alen[5] - 1] = 31 if alen[5] > 1 else acc[5, 0]   # index out of range
    if alen[5] == 1:
        acc[5, 0] = 3
    dev = bnd.to_device(inp)
    st = torch.full((6,), -1, dtype=torch.int32, device="cuda")
    h = run_commit(bnd, dev, tree_status=st)
    _, rst = oracle_mod.commit(inp, W.BF16, [(b, 0) for b in range(6)])
    assert st.cpu().tolist() == rst.tolist() == [0, 4, 4, 4, 4, 4]
    for b in range(1, 6):
        assert torch.equal(h[b], dev["h0"][b])
    ref, _ = oracle_mod.commit(inp, W.BF16, [(0, 0), (0, 1)])
    assert slice_err(gpu_h_slices(h, [(0, 0), (0, 1)]), ref) <= COMMIT_TOL


def test_non_descendants_bitwise_unchanged(bnd):
    """Changing node k's inputs leaves every non-descendant's y bitwise equal."""
    import torch
    inp = W.make_custom(13, batch=1, n_nodes=60, n_heads=3, head_dim=64, d_state=128, n_groups=1,
                        dtype=W.BF16)
    par = inp["parent"][0]
    dev = bnd.to_device(inp)
    y1 = run_verify(bnd, dev).view(torch.int16).cpu()
    for k in (0, 5, 33, 59):
        dev2 = {kk: v.clone() for kk, v in dev.items()}
        dev2["x"][0, k] += 1.0
        dev2["dt"][0, k] *= 1.5
        dev2["B"][0, k] -= 0.5
        dev2["C"][0, k] += 0.25
        y2 = run_verify(bnd, dev2).view(torch.int16).cpu()
        desc = {i for i in range(60) if k in W.root_path(par, i)}
        for i in range(60):
            same = torch.equal(y1[0, i], y2[0, i])
            assert same == (i not in desc), (k, i)


def test_verify_commit_consistency(bnd):
    """y at the last accepted node equals the committed state read out there."""
    import torch
    inp = W.make_custom(14, batch=4, n_nodes=50, n_heads=4, head_dim=64, d_state=128, n_groups=2,
                        dtype=W.BF16)
    dev = bnd.to_device(inp)
    y = run_verify(bnd, dev).float().cpu().double().numpy()
    h = run_commit(bnd, dev).cpu().double().numpy()
    C = W.to_f64(inp["C"], W.BF16)
    x = W.to_f64(inp["x"], W.BF16)
    for b in range(4):
        l = inp["accepted"][b, inp["accepted_len"][b] - 1]
        for hh in range(4):
            rhs = h[b, hh] @ C[b, l, hh // 2] + inp["D"][hh] * x[b, l, hh]
            err = np.max(np.abs(y[b, l, hh] - rhs)) / np.max(np.abs(rhs))
            assert err <= TOL[W.BF16], (b, hh, err)


def test_commit_twice_advances_again(bnd, oracle_mod):
    """Commit is not idempotent: a second call replays the path from the new state."""
    import torch
    inp = W.make_custom(15, batch=2, n_nodes=20, n_heads=2, head_dim=64, d_state=64, n_groups=1,
                        dtype=W.BF16)
    dev = bnd.to_device(inp)
    h = run_commit(bnd, dev)
    h = run_commit(bnd, dev, h=h)
    inp2 = dict(inp)
    h1, _ = oracle_mod.commit(inp, W.BF16)
    inp2["h0"] = h1.reshape(inp["h0"].shape).astype(np.float64)
    h2, _ = oracle_mod.commit(inp2, W.BF16)
    assert slice_err(gpu_h_slices(h, oracle_mod.all_pairs(inp)), h2) <= COMMIT_TOL


def test_empty_and_degenerate(bnd):
    import torch
    inp = W.make_custom(16, batch=2, n_nodes=9, n_heads=2, head_dim=64, d_state=64, n_groups=1,
                        dtype=W.BF16)
    dev = bnd.to_device(inp)
    empty = {k: v[:0] for k, v in dev.items() if k not in ("A", "D")}
    empty.update(A=dev["A"], D=dev["D"])
    y = run_verify(bnd, empty)
    assert y.shape[0] == 0
    run_commit(bnd, empty)
    dev["accepted_len"].zero_()
    h = run_commit(bnd, dev)
    assert torch.equal(h, dev["h0"])


def test_nondefault_stream(bnd, oracle_mod):
    import torch
    inp = W.make_inputs(2)
    dev = bnd.to_device(inp)
    s = torch.cuda.Stream()
    torch.cuda.synchronize()
    with torch.cuda.stream(s):
        y = run_verify(bnd, dev, stream=s)
    s.synchronize()
    sel = [(0, 0), (15, 79)]
    ref, _ = oracle_mod.verify(inp, W.BF16, sel)
    assert slice_err(gpu_y_slices(y, sel), ref) <= TOL[W.BF16]


@pytest.mark.parametrize("T,P,N,G,H", [(37, 32, 16, 1, 2), (9, 128, 64, 2, 2), (6, 256, 256, 1, 2)])
def test_bf16_generic_shapes(bnd, oracle_mod, T, P, N, G, H):
    """bf16 inputs whose head_dim / d_state have no MFMA kernel use the VALU kernel."""
    inp = W.make_custom(T * 3 + P, batch=2, n_nodes=T, n_heads=H, head_dim=P, d_state=N,
                        n_groups=G, dtype=W.BF16)
    check_full(bnd, oracle_mod, inp, W.BF16, f"bf16 generic T={T} P={P} N={N}")


@pytest.mark.parametrize("T,dtype", [(31, W.BF16), (200, W.BF16), (40, W.F32)])
def test_linear_attention_special_case(bnd, oracle_mod, T, dtype):
    """Tree linear attention (no decay, no skip): y_i = h0 q_i + sum over the root
    path of (q_i . k_j) v_j is the verify call with A = 0, dt = 1, D = 0 and
    (x, B, C) = (v, k, q). Commit then gives h0 + sum of v_j k_j^T on the path."""
    inp = W.make_custom(800 + T, batch=3, n_nodes=T, n_heads=4, head_dim=64, d_state=128,
                        n_groups=1, dtype=dtype)
    inp["A"] = np.zeros_like(inp["A"])
    inp["D"] = np.zeros_like(inp["D"])
    one = np.ones(inp["dt"].shape, np.float32)
    inp["dt"] = W.f32_to_bf16_bits(one) if dtype == W.BF16 else one
    check_full(bnd, oracle_mod, inp, dtype, f"linear attention T={T}")
