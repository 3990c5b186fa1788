"""Tree verification and commit for the gated delta rule, in fp64. TEST
INFRASTRUCTURE ONLY: imported by tests/ alone, never by the product path.

"TreeWY: Speculative Verification for Gated DeltaNet Hybrids" (fugumt page,
abstract): with a tree-structured WY transform of the gated delta rule every
draft node's output comes from one triangular solve, and commit rebuilds only
the accepted state from a small pseudo-value matrix. The pages name the
recurrence but do not write it out; the plain reading (the gated delta rule of
Gated DeltaNet) is, per head, with state S (dv x dk), token inputs q, k (dk),
v (dv), log gate g <= 0 (alpha = exp(g)) and step beta in [0, 1]:

    S <- exp(g) S (I - beta k k^T) + beta v k^T,      o = S q

run from S0 (the state before the root) along each node's root path.

``verify_unrolled`` / ``commit_unrolled`` are the definition: every root path
unrolled and the recurrence run token by token. ``verify_wy`` is the second
formulation (used only to check the first): with G_i the sum of g over the
root path of i, pseudo-values e solve the unit lower-triangular system

    e_i + beta_i sum_{j strict ancestor of i} exp(G_i - G_j) (k_i . k_j) e_j
        = beta_i (v_i - exp(G_i) S0 k_i)

and o_i = exp(G_i) S0 q_i + sum_{j on path(i)} exp(G_i - G_j) (q_i . k_j) e_j;
commit is S' = exp(G_l) S0 + sum_{j on path(l)} exp(G_l - G_j) e_j k_j^T.
"""
from __future__ import annotations

import numpy as np

BAD_ROOT, BAD_PARENT, BAD_PATH = 1, 2, 4


def tree_status(par) -> int:
    st = 0
    if len(par) and par[0] != -1:
        st |= BAD_ROOT
    for i in range(1, len(par)):
        if not (0 <= par[i] < i):
            st |= BAD_PARENT
    return st


def root_path(par, i):
    path = []
    while i >= 0:
        path.append(int(i))
        i = par[i]
    return path[::-1]


def _step(S, q, k, v, g, beta):
    S = np.exp(g) * (S - beta * np.outer(S @ k, k)) + beta * np.outer(v, k)
    return S


def verify_unrolled(q, k, v, g, beta, S0, parent):
    """o [B][T][H][dv] and status [B]; q, k [B][T][H][dk], v [B][T][H][dv],
    g, beta [B][T][H], S0 [B][H][dv][dk], parent [B][T] (all float64 / int)."""
    B, T, H, dk = k.shape
    dv = v.shape[-1]
    o = np.zeros((B, T, H, dv))
    status = np.zeros(B, np.int64)
    for b in range(B):
        par = [int(p) for p in parent[b]]
        status[b] = tree_status(par)
        if status[b]:
            continue
        for h in range(H):
            for i in range(T):
                S = S0[b, h].copy()
                for j in root_path(par, i):
                    S = _step(S, q[b, j, h], k[b, j, h], v[b, j, h], g[b, j, h], beta[b, j, h])
                o[b, i, h] = S @ q[b, i, h]
    return o, status


def commit_unrolled(k, v, g, beta, S0, parent, accepted, accepted_len):
    """S' [B][H][dv][dk] after each item's accepted path (S0 where invalid or
    the path is empty) and status [B] (bits 1 | 2 | 4)."""
    B, T, H, dk = k.shape
    Lmax = accepted.shape[1]
    out = S0.copy()
    status = np.zeros(B, np.int64)
    for b in range(B):
        par = [int(p) for p in parent[b]]
        st = tree_status(par)
        n = int(accepted_len[b])
        if not st:
            if not 0 <= n <= Lmax:
                st |= BAD_PATH
            else:
                path = [int(a) for a in accepted[b, :n]]
                for t, node in enumerate(path):
                    if (t == 0 and node != 0) or not 0 <= node < T or (t > 0 and par[node] != path[t - 1]):
                        st |= BAD_PATH
        status[b] = st
        if st or n == 0:
            continue
        for h in range(H):
            S = S0[b, h].copy()
            for j in accepted[b, :n]:
                S = _step(S, None, k[b, j, h], v[b, j, h], g[b, j, h], beta[b, j, h])
            out[b, h] = S
    return out, status


def verify_wy(q, k, v, g, beta, S0, parent):
    """(o, e): the closed form through the pseudo-values e [B][T][H][dv]."""
    B, T, H, dk = k.shape
    dv = v.shape[-1]
    o = np.zeros((B, T, H, dv))
    e = np.zeros((B, T, H, dv))
    for b in range(B):
        par = [int(p) for p in parent[b]]
        paths = [root_path(par, i) for i in range(T)]
        for h in range(H):
            Gc = np.array([sum(g[b, j, h] for j in paths[i]) for i in range(T)])
            for i in range(T):          # topological order: ancestors solved first
                rhs = beta[b, i, h] * (v[b, i, h] - np.exp(Gc[i]) * (S0[b, h] @ k[b, i, h]))
                for j in paths[i][:-1]:
                    rhs = rhs - beta[b, i, h] * np.exp(Gc[i] - Gc[j]) * (k[b, i, h] @ k[b, j, h]) * e[b, j, h]
                e[b, i, h] = rhs
            for i in range(T):
                oi = np.exp(Gc[i]) * (S0[b, h] @ q[b, i, h])
                for j in paths[i]:
                    oi = oi + np.exp(Gc[i] - Gc[j]) * (q[b, i, h] @ k[b, j, h]) * e[b, j, h]
                o[b, i, h] = oi
    return o, e


def commit_wy(k, e, g, S0, parent, accepted, accepted_len):
    """S' from the pseudo-values along each item's accepted path (no checks)."""
    B, T, H, dk = k.shape
    out = S0.copy()
    for b in range(B):
        n = int(accepted_len[b])
        if n == 0:
            continue
        path = [int(a) for a in accepted[b, :n]]
        for h in range(H):
            Gc = np.cumsum([g[b, j, h] for j in path])
            S = np.exp(Gc[-1]) * S0[b, h]
            for t, j in enumerate(path):
                S = S + np.exp(Gc[-1] - Gc[t]) * np.outer(e[b, j, h], k[b, j, h])
            out[b, h] = S
    return out
