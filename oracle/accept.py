"""Greedy (temperature 0) acceptance of a verified draft tree. TEST
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
