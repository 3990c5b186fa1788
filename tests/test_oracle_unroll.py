"""Pins of the unrolled-form and snapshot references (oracle/unroll.py), no GPU.

The unroll plan is checked on worked examples (the 7-node binary tree and the
15-node tree of the 64-layer workload, whose leaves follow from the listed
parents), by a recursive enumeration of maximal root paths that shares no
code with it, and on invariants over every topologically labelled tree of up
to 6 nodes. The per-node states are checked against the recurrence's own
consequences: a node's output from its state equals the oracle's verify, and
the state of a child follows from its parent's by one step of the recurrence
written out here on the exact inputs."""
import itertools

import numpy as np
import pytest

from oracle import unroll as U
from speculative_tree_verification_amd import workloads as W


def test_worked_examples():
    nodes, lens, nl, st = U.unroll_plan(np.array([[-1, 0, 0, 1, 1, 2, 2]]), 4, 3)
    assert st.tolist() == [0] and nl.tolist() == [4]
    assert nodes[0].tolist() == [[0, 1, 3], [0, 1, 4], [0, 2, 5], [0, 2, 6]]
    assert lens[0].tolist() == [3, 3, 3, 3]
    # the 64-layer workload's tree: leaves 8, 9, 11, 12, 13, 14 (the root's
    # three children 1..3 have children 4..9; 4..7 have 10..13; 10 has 14)
    par = W.make_inputs(1)["parent"]
    nodes, lens, nl, st = U.unroll_plan(par, 6, 5)
    assert nl.tolist() == [6]
    assert [row[:n].tolist() for row, n in zip(nodes[0], lens[0])] == [
        [0, 3, 8], [0, 3, 9], [0, 1, 5, 11], [0, 2, 6, 12], [0, 2, 7, 13], [0, 1, 4, 10, 14]]


def _maximal_paths(par):
    """Root-to-leaf paths by recursive descent from the root (children lists)."""
    T = len(par)
    kids = {i: [c for c in range(1, T) if par[c] == i] for i in range(T)}

    def go(i, path):
        if not kids[i]:
            return [path + [i]]
        out = []
        for c in kids[i]:
            out += go(c, path + [i])
        return out
    return sorted(go(0, []), key=lambda p: p[-1])


def _all_trees(T):
    for choice in itertools.product(*[range(i) for i in range(1, T)]):
        yield [-1] + list(choice)


@pytest.mark.parametrize("T", [1, 2, 3, 4, 5, 6])
def test_every_small_tree(T):
    for par in _all_trees(T):
        nodes, lens, nl, st = U.unroll_plan(np.array([par]), T, T)
        assert st[0] == 0
        got = [nodes[0, l, :lens[0, l]].tolist() for l in range(nl[0])]
        assert got == _maximal_paths(par)
        # leaves = nodes that are no node's parent; their count
        assert nl[0] == T - len(set(par[1:]))
        # every node lies on some sequence, and slots past the leaves are empty
        assert set(itertools.chain(*got)) == set(range(T))
        assert (lens[0, nl[0]:] == 0).all() and (nodes[0, nl[0]:] == -1).all()
        assert (nodes[0][np.arange(T)[None, :] >= lens[0][:, None]] == -1).all()


def test_capacity_and_invalid_trees():
    par = np.array([[-1, 0, 0, 0], [-1, 0, 1, 2], [0, 0, 0, 0], [-1, 2, 0, 1]])
    nodes, lens, nl, st = U.unroll_plan(par, 2, 3)
    # star: 3 leaves > 2 slots; chain: path of 4 > 3; bad root; parent after child
    assert st.tolist() == [8, 8, 1, 2]
    assert nl.tolist() == [0, 0, 0, 0] and (lens == 0).all() and (nodes == -1).all()


def test_node_states_follow_the_recurrence(oracle_mod):
    """H_child = exp(dt_c A) H_parent + dt_c x_c (outer) B_c on the exact
    inputs, H_root the same from h0, and y_i = H_i C_i + D x_i is the oracle's
    verify output."""
    inp = W.make_custom(81, batch=2, n_nodes=12, n_heads=2, head_dim=5, d_state=3, n_groups=1,
                        dtype=W.BF16, max_depth=4)
    sel = [(0, 0), (1, 1)]
    Hs = U.node_states(oracle_mod, inp, W.BF16, sel)
    x, dt = W.to_f64(inp["x"], W.BF16), W.to_f64(inp["dt"], W.BF16)
    Bm, C = W.to_f64(inp["B"], W.BF16), W.to_f64(inp["C"], W.BF16)
    y, _ = oracle_mod.verify(inp, W.BF16, sel)
    for k, (b, h) in enumerate(sel):
        for i in range(12):
            p = inp["parent"][b, i]
            prev = inp["h0"][b, h].astype(np.float64) if p < 0 else Hs[k, p]
            step = np.exp(dt[b, i, h] * inp["A"][h]) * prev + dt[b, i, h] * np.outer(x[b, i, h], Bm[b, i, 0])
            assert np.allclose(Hs[k, i], step, rtol=1e-12, atol=1e-14)
            yi = Hs[k, i] @ C[b, i, 0] + inp["D"][h] * x[b, i, h]
            assert np.allclose(y[k, i], yi, rtol=1e-10, atol=1e-12)
