"""The two forms a packed tree replaces, as plain references. TEST
INFRASTRUCTURE ONLY: imported by tests/ and the benchmark's CPU-baseline leg
alone, never by the product path.

"STree: Speculative Tree Decoding for Hybrid State Space Models"
(atlas.scime.ai summary): without a packed-tree scan an SSM must unroll the
draft tree into repeated sequences, with extra states and memory (section
"Problem"), and the paper's baselines run such unrolled trees through a fused
selective scan (section "Experimental setup"; "Key results" compares the two
forward times). The Bole and TreeWY abstracts (mlsanity and fugumt pages)
name the other form: a full recurrent state materialised for every draft node.

Unrolled form, as read here: every leaf (a node that is nobody's parent)
defines one sequence, its root path from node 0 to the leaf; the sequences of
an item are listed by increasing leaf index; each runs the ordinary recurrence
from h0, so position s of a sequence gives the output of the node found there.

Snapshot form: the state H_i after every node's root path, i.e. what the
recurrence holds after node i, for all nodes.

Pure Python loops over trees; the floating-point references call the pinned
oracle (oracle.py), so nothing here repeats its arithmetic.
"""
from __future__ import annotations

from typing import Dict, Tuple

import numpy as np

BAD_ROOT, BAD_PARENT, BAD_PATH, OVER_CAPACITY = 1, 2, 4, 8


def _tree_status(par) -> int:
    st = 0
    if len(par) and par[0] != -1:
        st |= BAD_ROOT
    for i in range(1, len(par)):
        if not (0 <= par[i] < i):
            st |= BAD_PARENT
    return st


def leaves(par) -> list:
    """Nodes that are no node's parent, in increasing order."""
    has_child = [False] * len(par)
    for i in range(1, len(par)):
        has_child[par[i]] = True
    return [i for i in range(len(par)) if not has_child[i]]


def root_path(par, i) -> list:
    path = []
    while i >= 0:
        path.append(int(i))
        i = par[i]
    return path[::-1]


def unroll_plan(parent, max_leaves: int, max_len: int) -> Tuple[np.ndarray, np.ndarray,
                                                               np.ndarray, np.ndarray]:
    """(seq_nodes [B][max_leaves][max_len] with -1 padding, seq_len
    [B][max_leaves] (0 past the item's leaves), n_leaves [B], status [B]).

    Sequence l of item b is the root path of its l-th leaf. An invalid tree
    sets status bits 1 | 2; more leaves than max_leaves, or a root path longer
    than max_len, sets bit 8. Rows of such items are left -1 / 0 and n_leaves
    is 0."""
    parent = np.asarray(parent)
    B, T = parent.shape
    nodes = np.full((B, max_leaves, max_len), -1, np.int64)
    lens = np.zeros((B, max_leaves), np.int64)
    nl = np.zeros(B, np.int64)
    st = np.zeros(B, np.int64)
    for b in range(B):
        par = [int(p) for p in parent[b]]
        s = _tree_status(par)
        if not s:
            lv = leaves(par)
            paths = [root_path(par, l) for l in lv]
            if len(lv) > max_leaves or max(len(p) for p in paths) > max_len:
                s |= OVER_CAPACITY
            else:
                nl[b] = len(lv)
                for l, p in enumerate(paths):
                    nodes[b, l, :len(p)] = p
                    lens[b, l] = len(p)
        st[b] = s
    return nodes, lens, nl, st


def node_states(oracle_mod, inp: Dict[str, np.ndarray], dtype: str, sel) -> np.ndarray:
    """H_i [n][T][P][N] (float64) for the selected (b, h) pairs: the state the
    recurrence holds after node i's root path, computed by the oracle's commit
    along that path."""
    B, T, H, P = inp["x"].shape
    N = inp["B"].shape[-1]
    out = np.zeros((len(sel), T, P, N))
    for i in range(T):
        paths = [root_path([int(p) for p in inp["parent"][b]], i) for b in range(B)]
        Lmax = max(len(p) for p in paths)
        acc = np.full((B, Lmax), -1, np.int32)
        alen = np.zeros(B, np.int32)
        for b, p in enumerate(paths):
            acc[b, :len(p)] = p
            alen[b] = len(p)
        d = dict(inp)
        d["accepted"], d["accepted_len"] = acc, alen
        h, _ = oracle_mod.commit(d, dtype, sel)
        out[:, i] = h
    return out
