"""Seeded synthetic workloads for packed-tree SSD verification.

This module is data only: tree shapes, accepted paths and random tensors with
the distributions of the five workload configurations, plus bf16 encoding.
It holds none of the method's arithmetic (no decay, no recurrence, no
contraction), so both the HIP path and the CPU oracle can consume what it
produces without sharing computation.

Method context: "STree: Speculative Tree Decoding for Hybrid State Space
Models" (atlas.scime.ai summary, section "Approach"): a draft token tree is
packed into one sequence (nodes in topological order, root first) and verified
in one pass of a Mamba2/SSD layer. The pages print no workload recipe; the
shapes and distributions below are the five named configurations.

Layouts (all C-contiguous, row-major):
    x      [B, T, H, P]   bf16 bits (uint16) or float32
    dt     [B, T, H]      bf16 bits or float32 (already positive: softplus)
    A, D   [H]            float32
    Bm, Cm [B, T, G, N]   bf16 bits or float32
    h0     [B, H, P, N]   float32 (state stored P x N, n fastest)
    parent [B, T]         int32, parent[b, 0] == -1, 0 <= parent[b, i] < i
    accepted     [B, Lmax] int32 (root-path node list, -1 padded)
    accepted_len [B]       int32
"""
from __future__ import annotations

import dataclasses
from typing import Dict, List, Optional

import numpy as np

F32 = "f32"
BF16 = "bf16"


@dataclasses.dataclass(frozen=True)
class WorkloadConfig:
    cid: int
    name: str
    batch: int
    n_heads: int
    head_dim: int
    d_state: int
    n_groups: int
    n_nodes: int
    dtype: str
    layers: int
    max_path_len: int
    description: str


CONFIGS: Dict[int, WorkloadConfig] = {
    0: WorkloadConfig(0, "toy-binary-7", 1, 1, 16, 8, 1, 7, F32, 1, 3,
                      "toy fp32 tree scan, complete binary tree of 7 nodes"),
    1: WorkloadConfig(1, "mamba2-2.7b-tree15-x64layers", 1, 80, 64, 128, 1, 15, BF16, 64, 5,
                      "Mamba2-2.7B-shaped layer, 15-node static tree, 64 layer calls"),
    2: WorkloadConfig(2, "mamba2-2.7b-b16-tree31", 16, 80, 64, 128, 1, 31, BF16, 1, 5,
                      "batched Mamba2-2.7B-shaped layer, 31-node random recursive trees"),
    3: WorkloadConfig(3, "hybrid-8b-b32-tree63-g8", 32, 64, 64, 64, 8, 63, BF16, 1, 7,
                      "8B-hybrid-scale layer, 63-node geometric-branching trees, 8 groups"),
    4: WorkloadConfig(4, "mamba2-2.7b-b64-tree255-wide", 64, 80, 64, 128, 1, 255, BF16, 1, 9,
                      "wide-tree stress, 255-node level-structured trees"),
}

# Static 15-node tree of the Mamba2-2.7B workload: root; 3 children; 6
# grandchildren (2 per child); the first 4 grandchildren in breadth-first
# order get one child each; node 10 gets the single depth-4 leaf.
TREE15 = np.array([-1, 0, 0, 0, 1, 1, 2, 2, 3, 3, 4, 5, 6, 7, 10], dtype=np.int32)
TREE7 = np.array([-1, 0, 0, 1, 1, 2, 2], dtype=np.int32)
LEVELS255 = (1, 8, 32, 64, 64, 48, 24, 10, 4)


# --------------------------------------------------------------------------
# bf16 encoding (round to nearest, ties to even) -- data encoding only
# --------------------------------------------------------------------------
def f32_to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """Round float32 values to bf16 (RNE) and return the 16-bit patterns."""
    a = np.ascontiguousarray(a, dtype=np.float32)
    u = a.view(np.uint32).astype(np.uint64)
    rounded = (u + 0x7FFF + ((u >> 16) & 1)) >> 16
    out = rounded.astype(np.uint16)
    nan = np.isnan(a)
    if nan.any():
        out[nan] = 0x7FC0
    return out


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    """Widen bf16 bit patterns to float32 exactly."""
    b = np.ascontiguousarray(b, dtype=np.uint16)
    return (b.astype(np.uint32) << 16).view(np.float32)


def to_f64(arr: np.ndarray, dtype: str) -> np.ndarray:
    """Exact widening of a stored tensor (bf16 bits or float32) to float64."""
    if dtype == BF16:
        return bf16_bits_to_f32(arr).astype(np.float64)
    return np.asarray(arr, dtype=np.float32).astype(np.float64)


# --------------------------------------------------------------------------
# tree shapes (parent pointers in topological order, root = node 0)
# --------------------------------------------------------------------------
def depths_of(parent: np.ndarray) -> np.ndarray:
    """Depth (edges to the root) of each node; parent[i] < i is assumed."""
    d = np.zeros(len(parent), dtype=np.int64)
    for i in range(1, len(parent)):
        d[i] = d[parent[i]] + 1
    return d


def root_path(parent: np.ndarray, node: int) -> List[int]:
    """Node list from the root down to ``node``."""
    path = []
    j = int(node)
    while j >= 0:
        path.append(j)
        j = int(parent[j])
    return path[::-1]


def random_recursive_tree(rng: np.random.Generator, T: int, max_depth: int) -> np.ndarray:
    """parent[i] ~ U{0..i-1}, redrawn until the node's depth is <= max_depth."""
    parent = np.full(T, -1, dtype=np.int32)
    depth = np.zeros(T, dtype=np.int64)
    for i in range(1, T):
        while True:
            p = int(rng.integers(0, i))
            if depth[p] + 1 <= max_depth:
                break
        parent[i] = p
        depth[i] = depth[p] + 1
    return parent


def geometric_tree(rng: np.random.Generator, T: int, depth_cap: int, p_stop: float = 1.0 / 3.0) -> np.ndarray:
    """Random frontier expansion with Geometric(p) children on {0,1,...}.

    Mean branching (1-p)/p = 2 at p = 1/3. A uniformly chosen unexpanded node is
    expanded next; nodes at ``depth_cap`` get no children; growth stops at T
    nodes. Trees that do not reach exactly T nodes and depth ``depth_cap`` are
    redrawn.
    """
    while True:
        parent = [-1]
        depth = [0]
        frontier = [0]
        while frontier and len(parent) < T:
            u = frontier.pop(int(rng.integers(0, len(frontier))))
            if depth[u] >= depth_cap:
                continue
            k = int(rng.geometric(p_stop)) - 1  # numpy's geometric is on {1,2,...}
            k = min(k, T - len(parent))
            for _ in range(k):
                parent.append(u)
                depth.append(depth[u] + 1)
                frontier.append(len(parent) - 1)
        if len(parent) == T and max(depth) == depth_cap:
            return np.array(parent, dtype=np.int32)


def level_tree(rng: np.random.Generator, levels=LEVELS255) -> np.ndarray:
    """Nodes numbered level by level; each picks a parent uniformly in the level above."""
    parent = [-1]
    prev = [0]
    for size in levels[1:]:
        cur = []
        for _ in range(size):
            parent.append(int(prev[int(rng.integers(0, len(prev)))]))
            cur.append(len(parent) - 1)
        prev = cur
    return np.array(parent, dtype=np.int32)


def path_of_length(rng: np.random.Generator, parent: np.ndarray, max_len: int) -> List[int]:
    """L ~ U{1..min(max_len, maxdepth+1)}, then a uniform node at depth L-1 -> its root path."""
    d = depths_of(parent)
    top = min(max_len, int(d.max()) + 1)
    L = int(rng.integers(1, top + 1))
    cands = np.nonzero(d == L - 1)[0]
    node = int(cands[int(rng.integers(0, len(cands)))])
    return root_path(parent, node)


def _draw_tree_and_path(cfg: WorkloadConfig, rng: np.random.Generator):
    B, T = cfg.batch, cfg.n_nodes
    parents = np.zeros((B, T), dtype=np.int32)
    paths: List[List[int]] = []
    for b in range(B):
        if cfg.cid == 0:
            par = TREE7.copy()
            path = [0, 1, 4]
        elif cfg.cid == 1:
            par = TREE15.copy()
            leaves = [i for i in range(T) if not np.any(par == i)]
            leaf = leaves[int(rng.integers(0, len(leaves)))]
            path = root_path(par, leaf)
        elif cfg.cid == 2:
            par = random_recursive_tree(rng, T, max_depth=8)
            path = path_of_length(rng, par, cfg.max_path_len)
        elif cfg.cid == 3:
            par = geometric_tree(rng, T, depth_cap=6)
            node = int(rng.integers(0, T))
            path = root_path(par, node)
        elif cfg.cid == 4:
            par = level_tree(rng)
            path = path_of_length(rng, par, cfg.max_path_len)
        else:
            raise ValueError(cfg.cid)
        parents[b] = par
        paths.append(path)
    acc = np.full((B, cfg.max_path_len), -1, dtype=np.int32)
    acc_len = np.zeros(B, dtype=np.int32)
    for b, path in enumerate(paths):
        acc[b, :len(path)] = path
        acc_len[b] = len(path)
    return parents, acc, acc_len


def softplus(z: np.ndarray) -> np.ndarray:
    """log(1 + e^z), the dt distribution's transform (input generation only)."""
    z = np.asarray(z, dtype=np.float64)
    return np.where(z > 20.0, z, np.log1p(np.exp(np.minimum(z, 20.0))))


def make_inputs(cid: int, layer: int = 0) -> Dict[str, np.ndarray]:
    """Seeded inputs of configuration ``cid`` (one layer instance).

    Draw order: tree -> path -> A -> D -> dt bias -> dt -> x -> B -> C -> h0,
    from ``numpy.random.default_rng([1000 + cid, layer])``. Layers of the same
    configuration share the layer-0 tree and accepted path.
    """
    cfg = CONFIGS[cid]
    rng = np.random.default_rng([1000 + cid, layer])
    parents, acc, acc_len = _draw_tree_and_path(cfg, rng)
    if layer != 0:
        parents, acc, acc_len = make_tree_and_path(cid)
    B, T, H, P, N, G = cfg.batch, cfg.n_nodes, cfg.n_heads, cfg.head_dim, cfg.d_state, cfg.n_groups
    A = (-np.exp(rng.uniform(0.0, np.log(16.0), size=H))).astype(np.float32)
    D = rng.standard_normal(H).astype(np.float32)
    if cfg.cid == 3:
        bias = rng.uniform(-6.0, -2.0, size=H)
        z = rng.standard_normal((B, T, H)) + bias[None, None, :]
    else:
        z = rng.standard_normal((B, T, H)) - 4.0
    dt = softplus(z).astype(np.float32)
    x = rng.standard_normal((B, T, H, P), dtype=np.float32)
    Bm = rng.standard_normal((B, T, G, N), dtype=np.float32)
    Cm = rng.standard_normal((B, T, G, N), dtype=np.float32)
    h0 = (0.1 * rng.standard_normal((B, H, P, N), dtype=np.float32)).astype(np.float32)
    out = dict(parent=parents, accepted=acc, accepted_len=acc_len, A=A, D=D, h0=h0)
    if cfg.dtype == BF16:
        out.update(x=f32_to_bf16_bits(x), dt=f32_to_bf16_bits(dt),
                   B=f32_to_bf16_bits(Bm), C=f32_to_bf16_bits(Cm))
    else:
        out.update(x=x, dt=dt, B=Bm, C=Cm)
    return out


def make_tree_and_path(cid: int):
    """The layer-0 tree and accepted path of configuration ``cid``."""
    cfg = CONFIGS[cid]
    rng = np.random.default_rng([1000 + cid, 0])
    return _draw_tree_and_path(cfg, rng)


def make_custom(seed: int, batch: int, n_nodes: int, n_heads: int, head_dim: int, d_state: int,
                n_groups: int, dtype: str, parents: Optional[np.ndarray] = None,
                tree: str = "recursive", max_depth: int = 8, max_path_len: int = 9,
                dt_shift: float = -4.0) -> Dict[str, np.ndarray]:
    """Inputs of an arbitrary shape with the configurations' distributions.

    ``tree`` selects the shape when ``parents`` is not given: "recursive"
    (uniform earlier parent, depth <= max_depth), "chain", "star", "binary"
    (complete binary tree in breadth-first order), "level" (the 255-node level
    layout) or "geometric".
    """
    rng = np.random.default_rng([7000, seed])
    B, T, H, P, N, G = batch, n_nodes, n_heads, head_dim, d_state, n_groups
    if parents is None:
        parents = np.zeros((B, T), dtype=np.int32)
        for b in range(B):
            if T == 0:
                continue
            if tree == "recursive":
                parents[b] = random_recursive_tree(rng, T, max_depth)
            elif tree == "chain":
                parents[b] = np.arange(-1, T - 1, dtype=np.int32)
            elif tree == "star":
                parents[b] = np.array([-1] + [0] * (T - 1), dtype=np.int32)
            elif tree == "binary":
                parents[b] = (np.arange(T, dtype=np.int32) - 1) // 2
                parents[b, 0] = -1
            elif tree == "level":
                parents[b] = level_tree(rng)
            elif tree == "geometric":
                parents[b] = geometric_tree(rng, T, depth_cap=max_depth)
            else:
                raise ValueError(tree)
    parents = np.ascontiguousarray(parents, dtype=np.int32).reshape(B, T)
    acc = np.full((B, max_path_len), -1, dtype=np.int32)
    acc_len = np.zeros(B, dtype=np.int32)
    for b in range(B):
        if T == 0:
            continue
        path = path_of_length(rng, parents[b], max_path_len)
        acc[b, :len(path)] = path
        acc_len[b] = len(path)
    A = (-np.exp(rng.uniform(0.0, np.log(16.0), size=H))).astype(np.float32)
    D = rng.standard_normal(H).astype(np.float32)
    dt = softplus(rng.standard_normal((B, T, H)) + dt_shift).astype(np.float32)
    x = rng.standard_normal((B, T, H, P), dtype=np.float32)
    Bm = rng.standard_normal((B, T, G, N), dtype=np.float32)
    Cm = rng.standard_normal((B, T, G, N), dtype=np.float32)
    h0 = (0.1 * rng.standard_normal((B, H, P, N), dtype=np.float32)).astype(np.float32)
    out = dict(parent=parents, accepted=acc, accepted_len=acc_len, A=A, D=D, h0=h0)
    if dtype == BF16:
        out.update(x=f32_to_bf16_bits(x), dt=f32_to_bf16_bits(dt),
                   B=f32_to_bf16_bits(Bm), C=f32_to_bf16_bits(Cm))
    else:
        out.update(x=x, dt=dt, B=Bm, C=Cm)
    return out


def shape_of(inp: Dict[str, np.ndarray]):
    """(B, T, H, P, N, G) of an input dict."""
    B, T, H, P = inp["x"].shape
    G, N = inp["B"].shape[2], inp["B"].shape[3]
    return B, T, H, P, N, G


def make_tokens(seed: int, parent: np.ndarray, vocab: int = 32000, p_hit: float = 0.7,
                repeats: bool = False):
    """Seeded draft and target tokens for trees ``parent`` [B][T] (int32 each).

    Siblings get distinct draft tokens (a draft tree proposes different tokens
    at one position) unless ``repeats``, in which case they are drawn from a
    vocabulary of 3 with replacement. Each node's target token is, with
    probability ``p_hit``, the draft token of one of its children (uniform),
    otherwise a uniform token.
    """
    rng = np.random.default_rng([8100, seed])
    parent = np.asarray(parent)
    B, T = parent.shape
    draft = np.zeros((B, T), np.int32)
    target = np.zeros((B, T), np.int32)
    for b in range(B):
        kids = [[] for _ in range(T)]
        for c in range(1, T):
            kids[parent[b, c]].append(c)
        draft[b, 0] = rng.integers(0, vocab)
        for i in range(T):
            if not kids[i]:
                continue
            if repeats:
                draft[b, kids[i]] = rng.integers(0, 3, size=len(kids[i]))
            else:
                draft[b, kids[i]] = rng.choice(vocab, size=len(kids[i]), replace=False)
        for i in range(T):
            if kids[i] and rng.random() < p_hit:
                target[b, i] = draft[b, kids[i][rng.integers(0, len(kids[i]))]]
            else:
                target[b, i] = rng.integers(0, 3 if repeats else vocab)
    return draft, target


# Vocabulary sizes of the model families the configurations are shaped on
# (GPT-NeoX tokenizer of Mamba2-2.7B, Llama-3 tokenizer of the 8B hybrid).
VOCAB = {0: 64, 1: 50280, 2: 50280, 3: 128256, 4: 50280}


def make_sampling(seed: int, parent: np.ndarray, vocab: int, temperature: float = 1.0,
                  draft_noise: float = 2.0, logit_scale: float = 2.0) -> Dict[str, np.ndarray]:
    """Seeded inputs of stochastic tree acceptance for trees ``parent`` [B][T].

    Synthetic logits per node: the target's are logit_scale times standard
    Gumbel noise (a peaked, heavy-tailed distribution over the vocabulary),
    the drafter's the same plus draft_noise times standard normal noise (a
    drafter that roughly tracks the target; with the defaults the 15-node
    tree accepts about 2.4 nodes per step at temperature 1, the range of
    acceptance lengths the STree pages report). Both are turned into fp32
    distributions by a softmax at ``temperature``. The children of each node
    draw their tokens from the node's draft distribution one after another
    without replacement, in increasing node index (Gumbel top-k on the log
    probabilities). Uniforms are fp32 in [0, 1).

    Returns parent, draft [B][T] int32, p_target and q_draft [B][T][V] fp32,
    u_node [B][T] fp32 and u_final [B] fp32.
    """
    rng = np.random.default_rng([8200, seed])
    parent = np.asarray(parent, np.int32)
    B, T = parent.shape
    V = int(vocab)
    zt = logit_scale * rng.gumbel(size=(B, T, V))
    zd = zt + draft_noise * rng.standard_normal((B, T, V))

    def softmax(z):
        z = z / temperature
        z = z - z.max(axis=-1, keepdims=True)
        e = np.exp(z)
        return (e / e.sum(axis=-1, keepdims=True)).astype(np.float32)

    p = softmax(zt)
    del zt
    q = softmax(zd)
    del zd
    draft = np.zeros((B, T), np.int32)
    for b in range(B):
        kids = [[] for _ in range(T)]
        for c in range(1, T):
            kids[parent[b, c]].append(c)
        draft[b, 0] = rng.integers(0, V)
        for u in range(T):
            if not kids[u]:
                continue
            with np.errstate(divide="ignore"):
                keys = np.log(q[b, u].astype(np.float64)) + rng.gumbel(size=V)
            order = np.argsort(-keys, kind="stable")[:len(kids[u])]
            draft[b, kids[u]] = order
    return {"parent": parent, "draft": draft, "p_target": p, "q_draft": q,
            "u_node": rng.random((B, T), dtype=np.float32),
            "u_final": rng.random(B, dtype=np.float32)}


def make_sampling_device(seed: int, parent: np.ndarray, vocab: int, device, temperature: float = 1.0,
                         draft_noise: float = 2.0, logit_scale: float = 2.0) -> Dict[str, object]:
    """make_sampling's recipe drawn with torch on ``device`` (for vocabulary
    rows too large to build on the host): the same distributions, not the
    same numbers. Returns torch tensors under make_sampling's keys."""
    import torch
    parent = np.asarray(parent, np.int32)
    B, T = parent.shape
    V = int(vocab)
    g = torch.Generator(device=device)
    g.manual_seed(8300 + seed)

    def gumbel(shape):
        u = torch.rand(shape, generator=g, device=device, dtype=torch.float32).clamp_(1e-30, 1.0)
        return -torch.log(-torch.log(u).clamp_(max=-1e-30))

    zt = logit_scale * gumbel((B, T, V))
    zd = zt + draft_noise * torch.randn((B, T, V), generator=g, device=device)
    p = torch.softmax(zt / temperature, dim=-1)
    del zt
    q = torch.softmax(zd / temperature, dim=-1)
    del zd
    rank = np.zeros((B, T), np.int64)
    kmax = 1
    for b in range(B):
        seen = np.zeros(T, np.int64)
        for c in range(1, T):
            rank[b, c] = seen[parent[b, c]]
            seen[parent[b, c]] += 1
        kmax = max(kmax, int(seen.max()))
    keys = torch.log(q) + gumbel((B, T, V))
    top = torch.topk(keys, kmax, dim=-1).indices          # draw order, best first
    del keys
    par_t = torch.from_numpy(np.maximum(parent, 0).astype(np.int64)).to(device)
    rank_t = torch.from_numpy(rank).to(device)
    bidx = torch.arange(B, device=device)[:, None].expand(B, T)
    draft = top[bidx, par_t, rank_t].to(torch.int32)
    draft[:, 0] = torch.randint(0, V, (B,), generator=g, device=device, dtype=torch.int32)
    return {"parent": torch.from_numpy(parent).to(device), "draft": draft.contiguous(),
            "p_target": p.contiguous(), "q_draft": q.contiguous(),
            "u_node": torch.rand((B, T), generator=g, device=device),
            "u_final": torch.rand((B,), generator=g, device=device)}


def make_gdn(seed: int, batch: int, n_nodes: int, n_heads: int, dk: int, dv: int,
             tree: str = "recursive", max_depth: int = 8, max_path_len: int = 9,
             parents: Optional[np.ndarray] = None, dtype: str = F32) -> Dict[str, np.ndarray]:
    """Seeded inputs of a gated-delta-rule layer over packed trees:
    q, k [B][T][H][dk] (k scaled to unit length, q by 1/sqrt(dk)), v [B][T][H][dv]
    ~ N(0, 1), log gate g = log U(0.9, 1), step beta = sigmoid(N(0, 1)), state
    S0 [B][H][dv][dk] ~ 0.1 N(0, 1); trees and accepted paths as make_custom.
    With dtype BF16, q, k and v are rounded to bf16 and returned as bit
    patterns (uint16); g, beta and S0 stay fp32."""
    rng = np.random.default_rng([9100, seed])
    B, T, H = batch, n_nodes, n_heads
    if parents is None:
        base = make_custom(seed, batch=B, n_nodes=T, n_heads=1, head_dim=4, d_state=4, n_groups=1,
                           dtype=F32, tree=tree, max_depth=max_depth, max_path_len=max_path_len)
        parents, acc, acc_len = base["parent"], base["accepted"], base["accepted_len"]
    else:
        parents = np.asarray(parents, np.int32)
        acc = np.full((B, max_path_len), -1, np.int32)
        acc_len = np.zeros(B, np.int32)
    k = rng.standard_normal((B, T, H, dk))
    k /= np.linalg.norm(k, axis=-1, keepdims=True)
    q = rng.standard_normal((B, T, H, dk)) / np.sqrt(dk)
    v = rng.standard_normal((B, T, H, dv))
    g = np.log(rng.uniform(0.9, 1.0, size=(B, T, H)))
    beta = 1.0 / (1.0 + np.exp(-rng.standard_normal((B, T, H))))
    S0 = 0.1 * rng.standard_normal((B, H, dv, dk))
    f = lambda a: np.ascontiguousarray(a, dtype=np.float32)
    io = (lambda a: f32_to_bf16_bits(f(a))) if dtype == BF16 else f
    return dict(q=io(q), k=io(k), v=io(v), g=f(g), beta=f(beta), S0=f(S0), parent=parents,
                accepted=acc, accepted_len=acc_len)
