"""Acceptance of a verified draft tree: greedy (temperature 0) and stochastic
(multi-step speculative sampling, below). TEST
INFRASTRUCTURE ONLY: imported by tests/ alone, never by the product path.

At temperature 0 the target model's choice after node i is its argmax token
target[i], and a child c of an accepted node i is kept when draft[c] equals
that choice ("TreeSpark: Adaptive Draft Trees Accelerate Speculative Decoding
by 8-14%", section on the lossless guarantee: the target model keeps or rejects
draft tokens, and a draft tree offers several candidate paths checked in one
pass). The root is the token the tree grows from and is always kept.

Written as a descent from the root: every kept node hands on to its kept
children; the path ends at the deepest kept node (smallest index among equally
deep ones, which only repeated sibling tokens can produce) and is cut after
max_path_len entries. Pure Python loops; trees of at most 256 nodes.
"""
from __future__ import annotations

from typing import Tuple

import numpy as np

BAD_ROOT, BAD_PARENT = 1, 2


def _tree_status(par) -> int:
    st = 0
    if len(par) and par[0] != -1:
        st |= BAD_ROOT
    for i in range(1, len(par)):
        if not (0 <= par[i] < i):
            st |= BAD_PARENT
    return st


def accept_greedy(parent, draft, target, max_path_len: int) -> Tuple[np.ndarray, np.ndarray,
                                                                    np.ndarray, np.ndarray]:
    """(accepted [B][max_path_len] with -1 padding, accepted_len [B],
    next_token [B], status [B]); rows of invalid items stay -1 / 0."""
    parent, draft, target = (np.asarray(a) for a in (parent, draft, target))
    B, T = parent.shape
    acc = np.full((B, max_path_len), -1, np.int64)
    alen = np.zeros(B, np.int64)
    nxt = np.full(B, -1, np.int64)
    status = np.zeros(B, np.int64)
    for b in range(B):
        par = [int(v) for v in parent[b]]
        status[b] = _tree_status(par)
        if status[b]:
            continue
        children = [[] for _ in range(T)]
        for c in range(1, T):
            children[par[c]].append(c)
        # descent: (depth, node) of every kept node
        kept = [(0, 0)]
        stack = [(0, 0)]
        while stack:
            d, i = stack.pop()
            for c in children[i]:
                if int(draft[b, c]) == int(target[b, i]):
                    kept.append((d + 1, c))
                    stack.append((d + 1, c))
        depth = max(d for d, _ in kept)
        last = min(i for d, i in kept if d == depth)
        path = []
        j = last
        while j >= 0:
            path.append(j)
            j = par[j]
        path.reverse()
        n = min(len(path), max_path_len)
        acc[b, :n] = path[:n]
        alen[b] = n
        nxt[b] = int(target[b, path[n - 1]])
    return acc, alen, nxt, status


# ---------------------------------------------------------------------------
# stochastic acceptance: multi-step speculative sampling over the tree
# ---------------------------------------------------------------------------
BAD_TOKEN = 16


def _first_crossing(r: np.ndarray, u: float) -> int:
    """Inverse-CDF draw from the unnormalised weights r with the uniform u:
    the first index whose running sum exceeds u times the total (the running
    sum taken left to right); -1 when the total is 0."""
    cs = np.cumsum(r)
    if not len(cs) or cs[-1] <= 0.0:
        return -1
    return int(np.argmax(cs > u * cs[-1]))


def accept_stochastic(parent, draft, p_target, q_draft, u_node, u_final, max_path_len: int,
                      with_margins: bool = False):
    """Stochastic acceptance of a verified draft tree at temperature > 0.

    Follows "STree: Speculative Tree Decoding for Hybrid State-Space Models"
    (atlas.scime.ai summary, measured-effects table: multi-step speculative
    sampling as the acceptance rule) with siblings drawn without replacement
    ("TreeSpark: Adaptive Draft Trees Accelerate Speculative Decoding by
    8-14%", section on the lossless guarantee: siblings sampled without
    replacement, rejected tokens resampled from the residual of target and
    draft, recursively). Inputs of item b:

      parent [T], draft [T]   tree and each node's draft token (root's unused)
      p_target [T][V]         target distribution of the token after node u
      q_draft [T][V]          draft distribution the children of u were drawn
                              from, one after another without replacement, in
                              increasing node index
      u_node [T]              uniform of each non-root node's test
      u_final                 uniform of the final draw

    Starting at the root with residual r = p_target[u], the children of the
    current node u are tested in index order. The k-th child's token t was
    drawn from d = q_draft[u] with the tokens of the earlier children removed
    and renormalised (d = q / (1 - removed mass)); it is accepted when
    u_node * d[t] < r[t] (probability min(1, r[t] / d[t])). An accepted child
    becomes the current node. A rejection replaces r by max(r - d, 0)
    renormalised (r is kept when that has no mass) and removes t from d. When
    no child is accepted the next token is drawn from r with u_final (first
    index whose running sum exceeds u_final times the total). The path is cut
    after max_path_len nodes; a child accepted below the cut gives the next
    token instead (its token is a draw from the cut node's target).

    Returns (accepted [B][L] with -1 padding, accepted_len [B], next_token
    [B], status [B]); with ``with_margins`` also the smallest relative
    distance of any decision from its threshold per item (tests use it to show
    that rounding order cannot flip a decision). Status 1/2 as for the tree
    check, 16 when a non-root draft token is outside [0, V). Everything in
    fp64; pure Python loops over the nodes, numpy over the vocabulary.
    """
    parent, draft = np.asarray(parent), np.asarray(draft)
    p_target, q_draft = np.asarray(p_target), np.asarray(q_draft)
    u_node, u_final = np.asarray(u_node, np.float64), np.asarray(u_final, np.float64)
    B, T = parent.shape
    V = p_target.shape[-1]
    L = max_path_len
    acc = np.full((B, L), -1, np.int64)
    alen = np.zeros(B, np.int64)
    nxt = np.full(B, -1, np.int64)
    status = np.zeros(B, np.int64)
    margin = np.full(B, np.inf)
    for b in range(B):
        par = [int(v) for v in parent[b]]
        st = _tree_status(par)
        if any(not (0 <= int(draft[b, c]) < V) for c in range(1, T)):
            st |= BAD_TOKEN
        status[b] = st
        if st:
            continue
        children = [[] for _ in range(T)]
        for c in range(1, T):
            children[par[c]].append(c)
        path, u, token = [0], 0, -1
        while True:
            r = p_target[b, u].astype(np.float64)
            q = q_draft[b, u].astype(np.float64)
            kept = np.ones(V, bool)      # tokens not yet drawn at this node
            removed = 0.0                # draft mass of the drawn tokens
            child = -1
            for c in children[u]:
                t = int(draft[b, c])
                mass = 1.0 - removed
                d = np.where(kept, q / mass, 0.0) if mass > 0.0 else np.zeros(V)
                lhs, rhs = u_node[b, c] * d[t], r[t]
                margin[b] = min(margin[b], abs(lhs - rhs) / max(abs(lhs), abs(rhs)) if lhs != rhs else 0.0)
                if lhs < rhs:
                    child = c
                    break
                res = np.maximum(r - d, 0.0)
                z = res.sum()
                if z > 0.0:
                    r = res / z
                if kept[t]:
                    kept[t] = False
                    removed += q[t]
            if child >= 0:
                if len(path) == L:
                    token = int(draft[b, child])
                    break
                path.append(child)
                u = child
                continue
            token = _first_crossing(r, float(u_final[b]))
            if token >= 0:
                cs = np.cumsum(r)
                thr = u_final[b] * cs[-1]
                lo = cs[token - 1] if token > 0 else 0.0
                gap = min(cs[token] - thr, thr - lo) / cs[-1]
                margin[b] = min(margin[b], gap) if gap > 0 else 0.0
            break
        n = len(path)
        acc[b, :n] = path
        alen[b] = n
        nxt[b] = token
    if with_margins:
        return acc, alen, nxt, status, margin
    return acc, alen, nxt, status
