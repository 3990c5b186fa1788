"""Python binding of libtree_ssd.so (argument marshalling only).

Every step of the computation runs in the HIP library; this module checks
tensor placement / dtype / shape, fills the ``tsv_shape`` struct and passes raw
device pointers and torch's current HIP stream through ctypes. PyTorch is used
for device memory and streams only. There is no fallback: if the library is
missing, importing this module raises.

Entry points mirror include/tree_ssd.h: ``verify``, ``commit``,
``commit_layers``, ``accept_greedy``, ``tree_info``, and for the gated delta
rule ``gdn_verify`` and ``gdn_commit``.
"""
from __future__ import annotations

import contextlib
import ctypes
import os
from typing import Dict, Optional

import numpy as np
import torch

PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(PKG, "libtree_ssd.so")

TSV_F32 = 0
TSV_BF16 = 1
TSV_FLAG_FORCE_GENERIC = 1
TSV_FLAG_FORCE_WIDE = 2
TSV_FLAG_FORCE_SMALL = 4
ST_BAD_ROOT, ST_BAD_PARENT, ST_BAD_PATH = 1, 2, 4
STATUS_NAMES = {0: "TSV_OK", 1: "TSV_E_NULL", 2: "TSV_E_SHAPE", 3: "TSV_E_DTYPE",
                4: "TSV_E_UNSUPPORTED", 5: "TSV_E_LAUNCH"}
EXPORTS = ("tree_ssd_verify", "tree_ssd_commit", "tree_ssd_commit_layers", "tree_ssd_accept_greedy",
           "tree_ssd_tree_info", "tree_ssd_status_string", "tree_ssd_abi_version", "tree_gdn_verify",
           "tree_gdn_commit", "tree_ssd_unroll_plan", "tree_ssd_unroll_gather", "tree_ssd_seq_scan",
           "tree_ssd_snapshot_verify", "tree_ssd_snapshot_commit", "tree_ssd_accept_stochastic",
           "tree_ssd_commit_layers_static")
STATIC_MAX_LAYERS = 1024  # TSV_STATIC_MAX_LAYERS
ST_OVER_CAPACITY = 8
ST_BAD_TOKEN = 16


class Shape(ctypes.Structure):
    _fields_ = [("batch", ctypes.c_int32), ("n_nodes", ctypes.c_int32),
                ("n_heads", ctypes.c_int32), ("head_dim", ctypes.c_int32),
                ("d_state", ctypes.c_int32), ("n_groups", ctypes.c_int32),
                ("in_dtype", ctypes.c_int32), ("flags", ctypes.c_int32),
                ("heads_per_block", ctypes.c_int32)]


class CommitLayer(ctypes.Structure):
    """tsv_commit_layer: one layer's device pointers for tree_ssd_commit_layers."""
    _fields_ = [("x", ctypes.c_void_p), ("dt", ctypes.c_void_p), ("A", ctypes.c_void_p),
                ("B", ctypes.c_void_p), ("h0_inout", ctypes.c_void_p)]


class TreeSSDError(RuntimeError):
    def __init__(self, code: int, where: str):
        self.code = code
        super().__init__(f"{where}: {STATUS_NAMES.get(code, code)} ({status_string(code)})")


_VP = ctypes.c_void_p


def _load():
    if not os.path.exists(LIB_PATH):
        raise ImportError(
            f"{LIB_PATH} is missing: build it with `python -m speculative_tree_verification_amd.build`"
            " (there is no CPU fallback)")
    L = ctypes.CDLL(LIB_PATH)
    L.tree_ssd_verify.argtypes = [ctypes.POINTER(Shape)] + [_VP] * 11
    L.tree_ssd_verify.restype = ctypes.c_int
    L.tree_ssd_commit.argtypes = [ctypes.POINTER(Shape)] + [_VP] * 8 + [ctypes.c_int32, _VP, _VP]
    L.tree_ssd_commit.restype = ctypes.c_int
    L.tree_ssd_commit_layers.argtypes = [ctypes.POINTER(Shape), ctypes.c_int32] + [_VP] * 4 + \
        [ctypes.c_int32, _VP, _VP]
    L.tree_ssd_commit_layers.restype = ctypes.c_int
    L.tree_ssd_commit_layers_static.argtypes = [ctypes.POINTER(Shape), ctypes.c_int32] + [_VP] * 4 + \
        [ctypes.c_int32, _VP, _VP]
    L.tree_ssd_commit_layers_static.restype = ctypes.c_int
    L.tree_ssd_accept_greedy.argtypes = [ctypes.c_int32, ctypes.c_int32] + [_VP] * 3 + \
        [ctypes.c_int32] + [_VP] * 5
    L.tree_ssd_accept_greedy.restype = ctypes.c_int
    L.tree_ssd_accept_stochastic.argtypes = [ctypes.c_int32] * 3 + [_VP] * 6 + [ctypes.c_int32] + [_VP] * 5
    L.tree_ssd_accept_stochastic.restype = ctypes.c_int
    L.tree_gdn_verify.argtypes = [ctypes.POINTER(Shape)] + [_VP] * 11
    L.tree_gdn_verify.restype = ctypes.c_int
    L.tree_gdn_commit.argtypes = [ctypes.POINTER(Shape)] + [_VP] * 7 + [ctypes.c_int32, _VP, _VP]
    L.tree_gdn_commit.restype = ctypes.c_int
    L.tree_ssd_tree_info.argtypes = [ctypes.c_int32, ctypes.c_int32] + [_VP] * 5
    L.tree_ssd_tree_info.restype = ctypes.c_int
    L.tree_ssd_status_string.argtypes = [ctypes.c_int32]
    L.tree_ssd_status_string.restype = ctypes.c_char_p
    L.tree_ssd_abi_version.argtypes = []
    L.tree_ssd_abi_version.restype = ctypes.c_int32
    L.tree_ssd_unroll_plan.argtypes = [ctypes.c_int32, ctypes.c_int32, _VP, ctypes.c_int32, ctypes.c_int32] + \
        [_VP] * 5
    L.tree_ssd_unroll_plan.restype = ctypes.c_int
    L.tree_ssd_unroll_gather.argtypes = [ctypes.POINTER(Shape), ctypes.c_int32, ctypes.c_int32] + [_VP] * 13
    L.tree_ssd_unroll_gather.restype = ctypes.c_int
    L.tree_ssd_seq_scan.argtypes = [ctypes.POINTER(Shape)] + [_VP] * 10
    L.tree_ssd_seq_scan.restype = ctypes.c_int
    L.tree_ssd_snapshot_verify.argtypes = [ctypes.POINTER(Shape)] + [_VP] * 12
    L.tree_ssd_snapshot_verify.restype = ctypes.c_int
    L.tree_ssd_snapshot_commit.argtypes = [ctypes.POINTER(Shape)] + [_VP] * 5 + [ctypes.c_int32, _VP, _VP]
    L.tree_ssd_snapshot_commit.restype = ctypes.c_int
    return L


lib = _load()


def status_string(code: int) -> str:
    return lib.tree_ssd_status_string(int(code)).decode()


def abi_version() -> int:
    return int(lib.tree_ssd_abi_version())


def _ptr(t: Optional[torch.Tensor]):
    if t is None:
        return None
    return ctypes.c_void_p(t.data_ptr()) if t.numel() > 0 else None


def _stream(stream) -> ctypes.c_void_p:
    if stream is None:
        stream = torch.cuda.current_stream()
    if isinstance(stream, torch.cuda.Stream):
        return ctypes.c_void_p(stream.cuda_stream)
    return ctypes.c_void_p(int(stream))


def _on_stream(stream):
    """Context under which the binding allocates and fills default outputs and
    temporary tables: the stream the kernel is launched on, so that the fill is
    ordered before the kernel and a freed temporary is reused only by later
    work on that stream (torch's caching allocator ties a block to the stream
    it was allocated on)."""
    if stream is None:
        return contextlib.nullcontext()
    if isinstance(stream, torch.cuda.Stream):
        return torch.cuda.stream(stream)
    return torch.cuda.stream(torch.cuda.ExternalStream(int(stream)))


def _dtype_code(t: torch.Tensor) -> int:
    if t.dtype == torch.float32:
        return TSV_F32
    if t.dtype == torch.bfloat16:
        return TSV_BF16
    raise TypeError(f"unsupported input dtype {t.dtype} (float32 or bfloat16)")


def _check(t: torch.Tensor, name: str, shape, dtype, device):
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name}: shape {tuple(t.shape)} != {tuple(shape)}")
    if t.dtype != dtype:
        raise TypeError(f"{name}: dtype {t.dtype} != {dtype}")
    if t.device != device:
        raise ValueError(f"{name}: device {t.device} != {device}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def make_shape(x: torch.Tensor, Bm: torch.Tensor, flags: int = 0, heads_per_block: int = 0) -> Shape:
    Bt, T, H, P = x.shape
    G, N = Bm.shape[2], Bm.shape[3]
    return Shape(Bt, T, H, P, N, G, _dtype_code(x), flags, heads_per_block)


def _flags(force_generic: bool, force_wide: bool, force_small: bool = False, extra: int = 0) -> int:
    return ((TSV_FLAG_FORCE_GENERIC if force_generic else 0) | (TSV_FLAG_FORCE_WIDE if force_wide else 0)
            | (TSV_FLAG_FORCE_SMALL if force_small else 0) | int(extra))


def verify(x, dt, A, B, C, D, h0, parent, y=None, tree_status=None, stream=None,
           force_generic: bool = False, heads_per_block: int = 0, check: bool = True,
           force_wide: bool = False, force_small: bool = False, flags: int = 0):
    """y [Bt,T,H,P] of one SSD layer over packed trees (tree_ssd_verify).
    ``flags`` adds further TSV_FLAG_* kernel choices (testing aids)."""
    Bt, T, H, P = x.shape
    G, N = B.shape[2], B.shape[3]
    dev, io = x.device, x.dtype
    if check:
        _check(dt, "dt", (Bt, T, H), io, dev)
        _check(B, "B", (Bt, T, G, N), io, dev)
        _check(C, "C", (Bt, T, G, N), io, dev)
        _check(A, "A", (H,), torch.float32, dev)
        _check(D, "D", (H,), torch.float32, dev)
        _check(h0, "h0", (Bt, H, P, N), torch.float32, dev)
        _check(parent, "parent", (Bt, T), torch.int32, dev)
        _check(x, "x", (Bt, T, H, P), io, dev)
    if y is None:
        with _on_stream(stream):
            y = torch.empty_like(x)
    elif check:
        _check(y, "y", (Bt, T, H, P), io, dev)
    if tree_status is not None and check:
        _check(tree_status, "tree_status", (Bt,), torch.int32, dev)
    shape = make_shape(x, B, _flags(force_generic, force_wide, force_small, flags), heads_per_block)
    rc = lib.tree_ssd_verify(ctypes.byref(shape), _ptr(x), _ptr(dt), _ptr(A), _ptr(B), _ptr(C),
                             _ptr(D), _ptr(h0), _ptr(parent), _ptr(y), _ptr(tree_status),
                             _stream(stream))
    if rc != 0:
        raise TreeSSDError(rc, "tree_ssd_verify")
    return y


def commit(x, dt, A, B, h0, parent, accepted, accepted_len, tree_status=None, stream=None,
           check: bool = True):
    """Overwrite h0 [Bt,H,P,N] with the state after each item's accepted path."""
    Bt, T, H, P = x.shape
    G, N = B.shape[2], B.shape[3]
    dev, io = x.device, x.dtype
    Lmax = accepted.shape[1] if accepted.dim() == 2 else 0
    if check:
        _check(dt, "dt", (Bt, T, H), io, dev)
        _check(B, "B", (Bt, T, G, N), io, dev)
        _check(A, "A", (H,), torch.float32, dev)
        _check(h0, "h0", (Bt, H, P, N), torch.float32, dev)
        _check(parent, "parent", (Bt, T), torch.int32, dev)
        _check(accepted, "accepted", (Bt, Lmax), torch.int32, dev)
        _check(accepted_len, "accepted_len", (Bt,), torch.int32, dev)
        if tree_status is not None:
            _check(tree_status, "tree_status", (Bt,), torch.int32, dev)
    shape = make_shape(x, B)
    rc = lib.tree_ssd_commit(ctypes.byref(shape), _ptr(x), _ptr(dt), _ptr(A), _ptr(B), _ptr(h0),
                             _ptr(parent), _ptr(accepted), _ptr(accepted_len), int(Lmax),
                             _ptr(tree_status), _stream(stream))
    if rc != 0:
        raise TreeSSDError(rc, "tree_ssd_commit")
    return h0


def layer_table(layers, device) -> torch.Tensor:
    """Device array of tsv_commit_layer for ``layers``, a sequence of
    (x, dt, A, B, h0) tensor tuples (the caller keeps the tensors alive)."""
    n = len(layers)
    table = (CommitLayer * max(n, 1))()
    for i, (x, dt, A, B, h0) in enumerate(layers):
        table[i] = CommitLayer(x.data_ptr(), dt.data_ptr(), A.data_ptr(), B.data_ptr(), h0.data_ptr())
    raw = np.frombuffer(bytes(table), dtype=np.uint8)[: n * ctypes.sizeof(CommitLayer)].copy()
    return torch.from_numpy(raw).to(device)


def _check_commit_layer(x, dt, A, B, h0, x0, B0, i):
    Bt, T, H, P = x0.shape
    G, N = B0.shape[2], B0.shape[3]
    io, dev = x0.dtype, x0.device
    for t, name, shp, dty in ((x, "x", (Bt, T, H, P), io), (dt, "dt", (Bt, T, H), io),
                              (B, "B", (Bt, T, G, N), io), (A, "A", (H,), torch.float32),
                              (h0, "h0", (Bt, H, P, N), torch.float32)):
        _check(t, f"layers[{i}].{name}", shp, dty, dev)


def commit_layers(layers, parent, accepted, accepted_len, tree_status=None, stream=None,
                  table: Optional[torch.Tensor] = None):
    """tree_ssd_commit for every (x, dt, A, B, h0) of ``layers`` in one launch;
    all layers share the tree and the accepted path. ``table`` may be a table
    already built by ``layer_table`` for these layers."""
    n = len(layers)
    if n == 0:
        return
    x0, _, _, B0, _ = layers[0]
    Bt, T = parent.shape
    dev = x0.device
    Lmax = accepted.shape[1] if accepted.dim() == 2 else 0
    for i, (x, dt, A, B, h0) in enumerate(layers):
        _check_commit_layer(x, dt, A, B, h0, x0, B0, i)
    _check(parent, "parent", (x0.shape[0], x0.shape[1]), torch.int32, dev)
    _check(accepted, "accepted", (Bt, Lmax), torch.int32, dev)
    _check(accepted_len, "accepted_len", (Bt,), torch.int32, dev)
    if tree_status is not None:
        _check(tree_status, "tree_status", (Bt,), torch.int32, dev)
    with _on_stream(stream):
        if table is None:
            table = layer_table(layers, dev)
        shape = make_shape(x0, B0)
        rc = lib.tree_ssd_commit_layers(ctypes.byref(shape), int(n), _ptr(table), _ptr(parent),
                                        _ptr(accepted), _ptr(accepted_len), int(Lmax),
                                        _ptr(tree_status), _stream(stream))
    if rc != 0:
        raise TreeSSDError(rc, "tree_ssd_commit_layers")


def commit_layers_static(layers, parent, accepted, accepted_len, tree_status=None, stream=None):
    """commit_layers without any device allocation: the layer table goes to
    tree_ssd_commit_layers_static as a host array, which the library stages
    into its own fixed device array (at most STATIC_MAX_LAYERS layers; calls
    that overlap on one GPU race). Results are bitwise those of commit_layers."""
    n = len(layers)
    if n == 0:
        return
    x0, _, _, B0, _ = layers[0]
    Bt, T = parent.shape
    dev = x0.device
    Lmax = accepted.shape[1] if accepted.dim() == 2 else 0
    for i, (x, dt, A, B, h0) in enumerate(layers):
        _check_commit_layer(x, dt, A, B, h0, x0, B0, i)
    _check(parent, "parent", (x0.shape[0], x0.shape[1]), torch.int32, dev)
    _check(accepted, "accepted", (Bt, Lmax), torch.int32, dev)
    _check(accepted_len, "accepted_len", (Bt,), torch.int32, dev)
    if tree_status is not None:
        _check(tree_status, "tree_status", (Bt,), torch.int32, dev)
    table = (CommitLayer * n)()
    for i, (x, dt, A, B, h0) in enumerate(layers):
        table[i] = CommitLayer(x.data_ptr(), dt.data_ptr(), A.data_ptr(), B.data_ptr(), h0.data_ptr())
    shape = make_shape(x0, B0)
    with torch.cuda.device(dev):
        rc = lib.tree_ssd_commit_layers_static(ctypes.byref(shape), int(n), ctypes.cast(table, _VP),
                                               _ptr(parent), _ptr(accepted), _ptr(accepted_len), int(Lmax),
                                               _ptr(tree_status), _stream(stream))
    if rc != 0:
        raise TreeSSDError(rc, "tree_ssd_commit_layers_static")


def accept_greedy(parent, draft_tokens, target_tokens, max_path_len: int, accepted=None,
                  accepted_len=None, next_token=None, tree_status=None, stream=None):
    """Greedy (temperature 0) acceptance of each item's verified tree:
    (accepted [Bt, max_path_len] int32, accepted_len [Bt], next_token [Bt],
    tree_status [Bt]). Outputs of invalid items are left as passed in."""
    Bt, T = parent.shape
    dev = parent.device
    _check(parent, "parent", (Bt, T), torch.int32, dev)
    _check(draft_tokens, "draft_tokens", (Bt, T), torch.int32, dev)
    _check(target_tokens, "target_tokens", (Bt, T), torch.int32, dev)
    with _on_stream(stream):
        if accepted is None:
            accepted = torch.full((Bt, max_path_len), -1, dtype=torch.int32, device=dev)
        if accepted_len is None:
            accepted_len = torch.zeros((Bt,), dtype=torch.int32, device=dev)
        if next_token is None:
            next_token = torch.full((Bt,), -1, dtype=torch.int32, device=dev)
        if tree_status is None:
            tree_status = torch.zeros((Bt,), dtype=torch.int32, device=dev)
    _check(accepted, "accepted", (Bt, max_path_len), torch.int32, dev)
    _check(accepted_len, "accepted_len", (Bt,), torch.int32, dev)
    _check(next_token, "next_token", (Bt,), torch.int32, dev)
    _check(tree_status, "tree_status", (Bt,), torch.int32, dev)
    rc = lib.tree_ssd_accept_greedy(int(Bt), int(T), _ptr(parent), _ptr(draft_tokens),
                                    _ptr(target_tokens), int(max_path_len), _ptr(accepted),
                                    _ptr(accepted_len), _ptr(next_token), _ptr(tree_status),
                                    _stream(stream))
    if rc != 0:
        raise TreeSSDError(rc, "tree_ssd_accept_greedy")
    return accepted, accepted_len, next_token, tree_status


def _sampling_args(parent, draft_tokens, p_target, q_draft, u_node, u_final):
    Bt, T = parent.shape
    V = p_target.shape[-1]
    dev = parent.device
    _check(parent, "parent", (Bt, T), torch.int32, dev)
    _check(draft_tokens, "draft_tokens", (Bt, T), torch.int32, dev)
    _check(p_target, "p_target", (Bt, T, V), torch.float32, dev)
    _check(q_draft, "q_draft", (Bt, T, V), torch.float32, dev)
    _check(u_node, "u_node", (Bt, T), torch.float32, dev)
    _check(u_final, "u_final", (Bt,), torch.float32, dev)
    return Bt, T, V, dev


def _accept_outputs(Bt, max_path_len, dev, stream):
    with _on_stream(stream):
        return (torch.full((Bt, max_path_len), -1, dtype=torch.int32, device=dev),
                torch.zeros((Bt,), dtype=torch.int32, device=dev),
                torch.full((Bt,), -1, dtype=torch.int32, device=dev),
                torch.zeros((Bt,), dtype=torch.int32, device=dev))


def accept_stochastic(parent, draft_tokens, p_target, q_draft, u_node, u_final, max_path_len: int,
                      accepted=None, accepted_len=None, next_token=None, tree_status=None, stream=None):
    """Stochastic acceptance (multi-step speculative sampling, siblings drawn
    without replacement) of each item's verified tree: (accepted [Bt,
    max_path_len] int32, accepted_len [Bt], next_token [Bt], tree_status
    [Bt]). Outputs of invalid items are left as passed in."""
    Bt, T, V, dev = _sampling_args(parent, draft_tokens, p_target, q_draft, u_node, u_final)
    outs = _accept_outputs(Bt, max_path_len, dev, stream)
    accepted = outs[0] if accepted is None else accepted
    accepted_len = outs[1] if accepted_len is None else accepted_len
    next_token = outs[2] if next_token is None else next_token
    tree_status = outs[3] if tree_status is None else tree_status
    _check(accepted, "accepted", (Bt, max_path_len), torch.int32, dev)
    _check(accepted_len, "accepted_len", (Bt,), torch.int32, dev)
    _check(next_token, "next_token", (Bt,), torch.int32, dev)
    _check(tree_status, "tree_status", (Bt,), torch.int32, dev)
    rc = lib.tree_ssd_accept_stochastic(int(Bt), int(T), int(V), _ptr(parent), _ptr(draft_tokens),
                                        _ptr(p_target), _ptr(q_draft), _ptr(u_node), _ptr(u_final),
                                        int(max_path_len), _ptr(accepted), _ptr(accepted_len),
                                        _ptr(next_token), _ptr(tree_status), _stream(stream))
    if rc != 0:
        raise TreeSSDError(rc, "tree_ssd_accept_stochastic")
    return accepted, accepted_len, next_token, tree_status


def _gdn_shape(k, v) -> Shape:
    Bt, T, H, dk = k.shape
    return Shape(Bt, T, H, v.shape[-1], dk, 1, _dtype_code(k), 0, 0)


def gdn_verify(q, k, v, g, beta, S0, parent, o=None, e=None, tree_status=None, stream=None):
    """(o, e) of one gated-delta-rule layer over packed trees (tree_gdn_verify).
    q, k, v (and o) float32 or bfloat16; g, beta, S0 and e float32."""
    Bt, T, H, dk = k.shape
    dv = v.shape[-1]
    dev, io = k.device, k.dtype
    f32 = torch.float32
    for t, name, shp, dt in ((q, "q", (Bt, T, H, dk), io), (k, "k", (Bt, T, H, dk), io),
                             (v, "v", (Bt, T, H, dv), io), (g, "g", (Bt, T, H), f32),
                             (beta, "beta", (Bt, T, H), f32), (S0, "S0", (Bt, H, dv, dk), f32)):
        _check(t, name, shp, dt, dev)
    _check(parent, "parent", (Bt, T), torch.int32, dev)
    with _on_stream(stream):
        o = torch.empty_like(v) if o is None else o
        e = torch.empty(v.shape, dtype=f32, device=dev) if e is None else e
    _check(o, "o", (Bt, T, H, dv), io, dev)
    _check(e, "e", (Bt, T, H, dv), f32, dev)
    shape = _gdn_shape(k, v)
    rc = lib.tree_gdn_verify(ctypes.byref(shape), _ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta),
                             _ptr(S0), _ptr(parent), _ptr(o), _ptr(e), _ptr(tree_status),
                             _stream(stream))
    if rc != 0:
        raise TreeSSDError(rc, "tree_gdn_verify")
    return o, e


def gdn_commit(k, g, e, S0, parent, accepted, accepted_len, tree_status=None, stream=None):
    """Overwrite S0 [Bt,H,dv,dk] with the state after each item's accepted path."""
    Bt, T, H, dk = k.shape
    dv = e.shape[-1]
    dev = k.device
    Lmax = accepted.shape[1] if accepted.dim() == 2 else 0
    f32 = torch.float32
    for t, name, shp, dt in ((k, "k", (Bt, T, H, dk), k.dtype), (g, "g", (Bt, T, H), f32),
                             (e, "e", (Bt, T, H, dv), f32), (S0, "S0", (Bt, H, dv, dk), f32)):
        _check(t, name, shp, dt, dev)
    _check(parent, "parent", (Bt, T), torch.int32, dev)
    _check(accepted, "accepted", (Bt, Lmax), torch.int32, dev)
    _check(accepted_len, "accepted_len", (Bt,), torch.int32, dev)
    shape = _gdn_shape(k, e)
    rc = lib.tree_gdn_commit(ctypes.byref(shape), _ptr(k), _ptr(g), _ptr(e), _ptr(S0), _ptr(parent),
                             _ptr(accepted), _ptr(accepted_len), int(Lmax), _ptr(tree_status),
                             _stream(stream))
    if rc != 0:
        raise TreeSSDError(rc, "tree_gdn_commit")
    return S0


def anc_words(T: int) -> int:
    """64-bit words of one node's ancestor set: 4 up to 256 nodes, then one per 64."""
    return max(4, -(-T // 64))


def tree_info(parent: torch.Tensor, depth=None, anc=None, tree_status=None, stream=None):
    """(depth [Bt,T] int32, anc [Bt,T,W] int64 bit patterns with W = anc_words(T),
    status [Bt] int32)."""
    Bt, T = parent.shape
    dev = parent.device
    with _on_stream(stream):
        if depth is None:
            depth = torch.zeros((Bt, T), dtype=torch.int32, device=dev)
        if anc is None:
            anc = torch.zeros((Bt, T, anc_words(T)), dtype=torch.int64, device=dev)
        if tree_status is None:
            tree_status = torch.zeros((Bt,), dtype=torch.int32, device=dev)
    rc = lib.tree_ssd_tree_info(int(Bt), int(T), _ptr(parent), _ptr(depth), _ptr(anc),
                                _ptr(tree_status), _stream(stream))
    if rc != 0:
        raise TreeSSDError(rc, "tree_ssd_tree_info")
    return depth, anc, tree_status


# ---------------------------------------------------------------------------
# host <-> device marshalling of the seeded workloads
# ---------------------------------------------------------------------------
def to_device(inp: Dict[str, np.ndarray], device="cuda") -> Dict[str, torch.Tensor]:
    """Upload a workload dict: bf16 bit patterns become torch.bfloat16 tensors."""
    out = {}
    for k, v in inp.items():
        if v.dtype == np.uint16:
            t = torch.from_numpy(np.ascontiguousarray(v).view(np.int16)).view(torch.bfloat16)
        else:
            t = torch.from_numpy(np.ascontiguousarray(v))
        out[k] = t.to(device)
    return out


def to_numpy_f64(t: torch.Tensor) -> np.ndarray:
    """Exact float64 copy of a device tensor (bf16 widened exactly)."""
    return t.detach().to("cpu", torch.float32).double().numpy()


# ---------------------------------------------------------------------------
# prepared calls: arguments checked and marshalled once, launched many times
# ---------------------------------------------------------------------------
class PreparedVerify:
    """tree_ssd_verify with fixed buffers; calling it enqueues one launch."""

    def __init__(self, x, dt, A, B, C, D, h0, parent, y, tree_status=None, stream=None,
                 force_generic: bool = False, heads_per_block: int = 0, force_wide: bool = False,
                 force_small: bool = False, flags: int = 0):
        Bt, T, H, P = x.shape
        G, N = B.shape[2], B.shape[3]
        io, dev = x.dtype, x.device
        for t, name, shp, dty in ((dt, "dt", (Bt, T, H), io), (B, "B", (Bt, T, G, N), io),
                                  (C, "C", (Bt, T, G, N), io), (A, "A", (H,), torch.float32),
                                  (D, "D", (H,), torch.float32),
                                  (h0, "h0", (Bt, H, P, N), torch.float32),
                                  (parent, "parent", (Bt, T), torch.int32),
                                  (y, "y", (Bt, T, H, P), io)):
            _check(t, name, shp, dty, dev)
        self.shape = make_shape(x, B, _flags(force_generic, force_wide, force_small, flags), heads_per_block)
        self._keep = (x, dt, A, B, C, D, h0, parent, y, tree_status)
        self.args = (ctypes.byref(self.shape), _ptr(x), _ptr(dt), _ptr(A), _ptr(B), _ptr(C),
                     _ptr(D), _ptr(h0), _ptr(parent), _ptr(y), _ptr(tree_status),
                     _stream(stream))

    def __call__(self):
        rc = lib.tree_ssd_verify(*self.args)
        if rc != 0:
            raise TreeSSDError(rc, "tree_ssd_verify")


class PreparedCommit:
    """tree_ssd_commit with fixed buffers; calling it enqueues one launch."""

    def __init__(self, x, dt, A, B, h0, parent, accepted, accepted_len, tree_status=None,
                 stream=None):
        Bt, T, H, P = x.shape
        G, N = B.shape[2], B.shape[3]
        io, dev = x.dtype, x.device
        Lmax = accepted.shape[1]
        for t, name, shp, dty in ((dt, "dt", (Bt, T, H), io), (B, "B", (Bt, T, G, N), io),
                                  (A, "A", (H,), torch.float32),
                                  (h0, "h0", (Bt, H, P, N), torch.float32),
                                  (parent, "parent", (Bt, T), torch.int32),
                                  (accepted, "accepted", (Bt, Lmax), torch.int32),
                                  (accepted_len, "accepted_len", (Bt,), torch.int32)):
            _check(t, name, shp, dty, dev)
        self.shape = make_shape(x, B)
        self._keep = (x, dt, A, B, h0, parent, accepted, accepted_len, tree_status)
        self.args = (ctypes.byref(self.shape), _ptr(x), _ptr(dt), _ptr(A), _ptr(B), _ptr(h0),
                     _ptr(parent), _ptr(accepted), _ptr(accepted_len), int(Lmax),
                     _ptr(tree_status), _stream(stream))

    def __call__(self):
        rc = lib.tree_ssd_commit(*self.args)
        if rc != 0:
            raise TreeSSDError(rc, "tree_ssd_commit")


class PreparedCommitLayers:
    """tree_ssd_commit_layers with fixed buffers and a resident layer table;
    calling it enqueues one launch that commits every layer."""

    def __init__(self, layers, parent, accepted, accepted_len, tree_status=None, stream=None):
        n = len(layers)
        if n == 0:
            raise ValueError("PreparedCommitLayers needs at least one layer")
        x0, _, _, B0, _ = layers[0]
        Bt = x0.shape[0]
        dev = x0.device
        Lmax = accepted.shape[1]
        for i, (x, dt, A, B, h0) in enumerate(layers):
            _check_commit_layer(x, dt, A, B, h0, x0, B0, i)
        _check(parent, "parent", (Bt, x0.shape[1]), torch.int32, dev)
        _check(accepted, "accepted", (Bt, Lmax), torch.int32, dev)
        _check(accepted_len, "accepted_len", (Bt,), torch.int32, dev)
        with _on_stream(stream):
            self.table = layer_table(layers, dev)
        self.shape = make_shape(x0, B0)
        self._keep = (list(layers), parent, accepted, accepted_len, tree_status)
        self.args = (ctypes.byref(self.shape), int(n), _ptr(self.table), _ptr(parent),
                     _ptr(accepted), _ptr(accepted_len), int(Lmax), _ptr(tree_status),
                     _stream(stream))

    def __call__(self):
        rc = lib.tree_ssd_commit_layers(*self.args)
        if rc != 0:
            raise TreeSSDError(rc, "tree_ssd_commit_layers")


class PreparedAccept:
    """tree_ssd_accept_greedy with fixed buffers; calling it enqueues one launch."""

    def __init__(self, parent, draft_tokens, target_tokens, max_path_len: int, stream=None):
        Bt, T = parent.shape
        dev = parent.device
        for t, name in ((parent, "parent"), (draft_tokens, "draft_tokens"),
                        (target_tokens, "target_tokens")):
            _check(t, name, (Bt, T), torch.int32, dev)
        with _on_stream(stream):
            self.accepted = torch.full((Bt, max_path_len), -1, dtype=torch.int32, device=dev)
            self.accepted_len = torch.zeros((Bt,), dtype=torch.int32, device=dev)
            self.next_token = torch.full((Bt,), -1, dtype=torch.int32, device=dev)
            self.tree_status = torch.zeros((Bt,), dtype=torch.int32, device=dev)
        self._keep = (parent, draft_tokens, target_tokens)
        self.args = (int(Bt), int(T), _ptr(parent), _ptr(draft_tokens), _ptr(target_tokens),
                     int(max_path_len), _ptr(self.accepted), _ptr(self.accepted_len),
                     _ptr(self.next_token), _ptr(self.tree_status), _stream(stream))

    def __call__(self):
        rc = lib.tree_ssd_accept_greedy(*self.args)
        if rc != 0:
            raise TreeSSDError(rc, "tree_ssd_accept_greedy")


class PreparedAcceptStochastic:
    """tree_ssd_accept_stochastic with fixed buffers; calling it enqueues one launch."""

    def __init__(self, parent, draft_tokens, p_target, q_draft, u_node, u_final, max_path_len: int,
                 stream=None):
        Bt, T, V, dev = _sampling_args(parent, draft_tokens, p_target, q_draft, u_node, u_final)
        self.accepted, self.accepted_len, self.next_token, self.tree_status = \
            _accept_outputs(Bt, max_path_len, dev, stream)
        self._keep = (parent, draft_tokens, p_target, q_draft, u_node, u_final)
        self.args = (int(Bt), int(T), int(V), _ptr(parent), _ptr(draft_tokens), _ptr(p_target),
                     _ptr(q_draft), _ptr(u_node), _ptr(u_final), int(max_path_len), _ptr(self.accepted),
                     _ptr(self.accepted_len), _ptr(self.next_token), _ptr(self.tree_status),
                     _stream(stream))

    def __call__(self):
        rc = lib.tree_ssd_accept_stochastic(*self.args)
        if rc != 0:
            raise TreeSSDError(rc, "tree_ssd_accept_stochastic")


# ---------------------------------------------------------------------------
# the forms a packed tree replaces: unrolled sequences and per-node snapshots
# ---------------------------------------------------------------------------
def unroll_capacity(parent) -> tuple:
    """(max_leaves, max_len) that hold the unrolled form of every item of a
    host copy of ``parent`` [Bt, T]: the most leaves of any item and the
    longest root path. Buffer sizing only."""
    par = np.asarray(parent)
    Bt, T = par.shape
    most, longest = 1, 1
    for row in par:
        has_child = np.zeros(T, bool)
        has_child[row[1:][row[1:] >= 0]] = True
        depth = np.zeros(T, np.int64)
        for i in range(1, T):
            depth[i] = depth[row[i]] + 1 if 0 <= row[i] < i else 0
        most = max(most, int((~has_child).sum()))
        longest = max(longest, int(depth.max()) + 1)
    return most, longest


def unroll_plan(parent, max_leaves: int, max_len: int, stream=None):
    """(seq_nodes [Bt, max_leaves, max_len], seq_len [Bt, max_leaves],
    n_leaves [Bt], tree_status [Bt]) of tree_ssd_unroll_plan."""
    Bt, T = parent.shape
    dev = parent.device
    _check(parent, "parent", (Bt, T), torch.int32, dev)
    with _on_stream(stream):
        nodes = torch.empty((Bt, max_leaves, max_len), dtype=torch.int32, device=dev)
        lens = torch.empty((Bt, max_leaves), dtype=torch.int32, device=dev)
        nl = torch.empty((Bt,), dtype=torch.int32, device=dev)
        st = torch.empty((Bt,), dtype=torch.int32, device=dev)
    rc = lib.tree_ssd_unroll_plan(int(Bt), int(T), _ptr(parent), int(max_leaves), int(max_len), _ptr(nodes),
                                  _ptr(lens), _ptr(nl), _ptr(st), _stream(stream))
    if rc != 0:
        raise TreeSSDError(rc, "tree_ssd_unroll_plan")
    return nodes, lens, nl, st


def unroll_gather(x, dt, B, C, h0, seq_nodes, seq_len, out: Optional[Dict[str, torch.Tensor]] = None,
                  stream=None) -> Dict[str, torch.Tensor]:
    """The unrolled sequences of tree_ssd_unroll_gather: x_u [Bt*Lcap, S, H, P],
    dt_u [Bt*Lcap, S, H], B_u / C_u [Bt*Lcap, S, G, N], h0_u [Bt*Lcap, H, P, N]."""
    Bt, T, H, P = x.shape
    G, N = B.shape[2], B.shape[3]
    Lcap, S = seq_nodes.shape[1], seq_nodes.shape[2]
    dev, io = x.device, x.dtype
    for t, name, shp, dty in ((dt, "dt", (Bt, T, H), io), (B, "B", (Bt, T, G, N), io),
                              (C, "C", (Bt, T, G, N), io), (h0, "h0", (Bt, H, P, N), torch.float32),
                              (seq_nodes, "seq_nodes", (Bt, Lcap, S), torch.int32),
                              (seq_len, "seq_len", (Bt, Lcap), torch.int32), (x, "x", (Bt, T, H, P), io)):
        _check(t, name, shp, dty, dev)
    ns = Bt * Lcap
    shapes = {"x_u": ((ns, S, H, P), io), "dt_u": ((ns, S, H), io), "B_u": ((ns, S, G, N), io),
              "C_u": ((ns, S, G, N), io), "h0_u": ((ns, H, P, N), torch.float32)}
    if out is None:
        with _on_stream(stream):
            out = {k: torch.zeros(shp, dtype=dty, device=dev) for k, (shp, dty) in shapes.items()}
    for k, (shp, dty) in shapes.items():
        _check(out[k], k, shp, dty, dev)
    shape = make_shape(x, B)
    rc = lib.tree_ssd_unroll_gather(ctypes.byref(shape), int(Lcap), int(S), _ptr(x), _ptr(dt), _ptr(B), _ptr(C),
                                    _ptr(h0), _ptr(seq_nodes), _ptr(seq_len), _ptr(out["x_u"]),
                                    _ptr(out["dt_u"]), _ptr(out["B_u"]), _ptr(out["C_u"]), _ptr(out["h0_u"]),
                                    _stream(stream))
    if rc != 0:
        raise TreeSSDError(rc, "tree_ssd_unroll_gather")
    return out


def seq_scan(x_u, dt_u, A, B_u, C_u, D, h_u, seq_len, y_u=None, stream=None):
    """Plain Mamba2 scan over sequences (tree_ssd_seq_scan): returns y_u; the
    final state of each sequence overwrites h_u."""
    ns, S, H, P = x_u.shape
    G, N = B_u.shape[2], B_u.shape[3]
    dev, io = x_u.device, x_u.dtype
    for t, name, shp, dty in ((dt_u, "dt_u", (ns, S, H), io), (B_u, "B_u", (ns, S, G, N), io),
                              (C_u, "C_u", (ns, S, G, N), io), (A, "A", (H,), torch.float32),
                              (D, "D", (H,), torch.float32), (h_u, "h_u", (ns, H, P, N), torch.float32),
                              (seq_len, "seq_len", (ns,), torch.int32)):
        _check(t, name, shp, dty, dev)
    if y_u is None:
        with _on_stream(stream):
            y_u = torch.zeros_like(x_u)
    _check(y_u, "y_u", (ns, S, H, P), io, dev)
    shape = Shape(ns, S, H, P, N, G, _dtype_code(x_u), 0, 0)
    rc = lib.tree_ssd_seq_scan(ctypes.byref(shape), _ptr(x_u), _ptr(dt_u), _ptr(A), _ptr(B_u), _ptr(C_u),
                               _ptr(D), _ptr(h_u), _ptr(seq_len), _ptr(y_u), _stream(stream))
    if rc != 0:
        raise TreeSSDError(rc, "tree_ssd_seq_scan")
    return y_u


def snapshot_verify(x, dt, A, B, C, D, h0, parent, y=None, states=None, tree_status=None, stream=None):
    """(y, states [Bt, H, T, P, N]) of tree_ssd_snapshot_verify."""
    Bt, T, H, P = x.shape
    G, N = B.shape[2], B.shape[3]
    dev, io = x.device, x.dtype
    for t, name, shp, dty in ((dt, "dt", (Bt, T, H), io), (B, "B", (Bt, T, G, N), io),
                              (C, "C", (Bt, T, G, N), io), (A, "A", (H,), torch.float32),
                              (D, "D", (H,), torch.float32), (h0, "h0", (Bt, H, P, N), torch.float32),
                              (parent, "parent", (Bt, T), torch.int32), (x, "x", (Bt, T, H, P), io)):
        _check(t, name, shp, dty, dev)
    with _on_stream(stream):
        if y is None:
            y = torch.empty_like(x)
        if states is None:
            states = torch.empty((Bt, H, T, P, N), dtype=torch.float32, device=dev)
    _check(y, "y", (Bt, T, H, P), io, dev)
    _check(states, "states", (Bt, H, T, P, N), torch.float32, dev)
    shape = make_shape(x, B)
    rc = lib.tree_ssd_snapshot_verify(ctypes.byref(shape), _ptr(x), _ptr(dt), _ptr(A), _ptr(B), _ptr(C),
                                      _ptr(D), _ptr(h0), _ptr(parent), _ptr(y), _ptr(states),
                                      _ptr(tree_status), _stream(stream))
    if rc != 0:
        raise TreeSSDError(rc, "tree_ssd_snapshot_verify")
    return y, states


def snapshot_commit(states, h0, parent, accepted, accepted_len, tree_status=None, stream=None):
    """Copy each item's last accepted node's stored state into h0 (tree_ssd_snapshot_commit)."""
    Bt, H, T, P, N = states.shape
    dev = states.device
    Lmax = accepted.shape[1] if accepted.dim() == 2 else 0
    _check(states, "states", (Bt, H, T, P, N), torch.float32, dev)
    _check(h0, "h0", (Bt, H, P, N), torch.float32, dev)
    _check(parent, "parent", (Bt, T), torch.int32, dev)
    _check(accepted, "accepted", (Bt, Lmax), torch.int32, dev)
    _check(accepted_len, "accepted_len", (Bt,), torch.int32, dev)
    shape = Shape(Bt, T, H, P, N, 1, TSV_F32, 0, 0)
    rc = lib.tree_ssd_snapshot_commit(ctypes.byref(shape), _ptr(states), _ptr(h0), _ptr(parent), _ptr(accepted),
                                      _ptr(accepted_len), int(Lmax), _ptr(tree_status), _stream(stream))
    if rc != 0:
        raise TreeSSDError(rc, "tree_ssd_snapshot_commit")
    return h0


class PreparedUnrolled:
    """The unrolled form of one verify call with fixed buffers: calling it
    enqueues tree_ssd_unroll_plan, tree_ssd_unroll_gather and
    tree_ssd_seq_scan (outputs y_u per sequence position; h0_u ends holding
    each sequence's final state). ``max_leaves`` / ``max_len`` size the
    sequence buffers (unroll_capacity gives exact ones)."""

    def __init__(self, x, dt, A, B, C, D, h0, parent, max_leaves: int, max_len: int, stream=None):
        Bt, T, H, P = x.shape
        G, N = B.shape[2], B.shape[3]
        dev, io = x.device, x.dtype
        for t, name, shp, dty in ((dt, "dt", (Bt, T, H), io), (B, "B", (Bt, T, G, N), io),
                                  (C, "C", (Bt, T, G, N), io), (A, "A", (H,), torch.float32),
                                  (D, "D", (H,), torch.float32), (h0, "h0", (Bt, H, P, N), torch.float32),
                                  (parent, "parent", (Bt, T), torch.int32)):
            _check(t, name, shp, dty, dev)
        Lc, S = int(max_leaves), int(max_len)
        ns = Bt * Lc
        with _on_stream(stream):
            self.seq_nodes = torch.empty((Bt, Lc, S), dtype=torch.int32, device=dev)
            self.seq_len = torch.empty((Bt, Lc), dtype=torch.int32, device=dev)
            self.n_leaves = torch.empty((Bt,), dtype=torch.int32, device=dev)
            self.tree_status = torch.empty((Bt,), dtype=torch.int32, device=dev)
            self.x_u = torch.zeros((ns, S, H, P), dtype=io, device=dev)
            self.dt_u = torch.zeros((ns, S, H), dtype=io, device=dev)
            self.B_u = torch.zeros((ns, S, G, N), dtype=io, device=dev)
            self.C_u = torch.zeros((ns, S, G, N), dtype=io, device=dev)
            self.h0_u = torch.zeros((ns, H, P, N), dtype=torch.float32, device=dev)
            self.y_u = torch.zeros((ns, S, H, P), dtype=io, device=dev)
        self.shape = make_shape(x, B)
        self.seq_shape = Shape(ns, S, H, P, N, G, _dtype_code(x), 0, 0)
        self._keep = (x, dt, A, B, C, D, h0, parent)
        st = _stream(stream)
        self.plan_args = (int(Bt), int(T), _ptr(parent), Lc, S, _ptr(self.seq_nodes), _ptr(self.seq_len),
                          _ptr(self.n_leaves), _ptr(self.tree_status), st)
        self.gather_args = (ctypes.byref(self.shape), Lc, S, _ptr(x), _ptr(dt), _ptr(B), _ptr(C), _ptr(h0),
                            _ptr(self.seq_nodes), _ptr(self.seq_len), _ptr(self.x_u), _ptr(self.dt_u),
                            _ptr(self.B_u), _ptr(self.C_u), _ptr(self.h0_u), st)
        self.scan_args = (ctypes.byref(self.seq_shape), _ptr(self.x_u), _ptr(self.dt_u), _ptr(A), _ptr(self.B_u),
                          _ptr(self.C_u), _ptr(D), _ptr(self.h0_u), _ptr(self.seq_len), _ptr(self.y_u), st)

    def materialised_bytes(self) -> int:
        """Bytes of the unrolled copies this form writes (inputs, states, outputs)."""
        return sum(t.numel() * t.element_size() for t in (self.x_u, self.dt_u, self.B_u, self.C_u,
                                                          self.h0_u, self.y_u))

    def __call__(self):
        for fn, args, name in ((lib.tree_ssd_unroll_plan, self.plan_args, "tree_ssd_unroll_plan"),
                               (lib.tree_ssd_unroll_gather, self.gather_args, "tree_ssd_unroll_gather"),
                               (lib.tree_ssd_seq_scan, self.scan_args, "tree_ssd_seq_scan")):
            rc = fn(*args)
            if rc != 0:
                raise TreeSSDError(rc, name)


class PreparedSnapshot:
    """The snapshot form with fixed buffers: ``verify()`` enqueues
    tree_ssd_snapshot_verify (every node's state into ``states``),
    ``commit(h)`` tree_ssd_snapshot_commit into h."""

    def __init__(self, x, dt, A, B, C, D, h0, parent, accepted, accepted_len, stream=None):
        Bt, T, H, P = x.shape
        G, N = B.shape[2], B.shape[3]
        dev, io = x.device, x.dtype
        for t, name, shp, dty in ((dt, "dt", (Bt, T, H), io), (B, "B", (Bt, T, G, N), io),
                                  (C, "C", (Bt, T, G, N), io), (A, "A", (H,), torch.float32),
                                  (D, "D", (H,), torch.float32), (h0, "h0", (Bt, H, P, N), torch.float32),
                                  (parent, "parent", (Bt, T), torch.int32)):
            _check(t, name, shp, dty, dev)
        Lmax = accepted.shape[1]
        _check(accepted, "accepted", (Bt, Lmax), torch.int32, dev)
        _check(accepted_len, "accepted_len", (Bt,), torch.int32, dev)
        with _on_stream(stream):
            self.y = torch.empty_like(x)
            self.states = torch.empty((Bt, H, T, P, N), dtype=torch.float32, device=dev)
        self.shape = make_shape(x, B)
        self.cshape = Shape(Bt, T, H, P, N, 1, TSV_F32, 0, 0)
        self._keep = (x, dt, A, B, C, D, h0, parent, accepted, accepted_len)
        self.st = _stream(stream)
        self.verify_args = (ctypes.byref(self.shape), _ptr(x), _ptr(dt), _ptr(A), _ptr(B), _ptr(C), _ptr(D),
                            _ptr(h0), _ptr(parent), _ptr(self.y), _ptr(self.states), None, self.st)
        self.commit_tail = (_ptr(parent), _ptr(accepted), _ptr(accepted_len), int(Lmax), None, self.st)

    def materialised_bytes(self) -> int:
        return self.states.numel() * 4

    def verify(self):
        rc = lib.tree_ssd_snapshot_verify(*self.verify_args)
        if rc != 0:
            raise TreeSSDError(rc, "tree_ssd_snapshot_verify")

    def commit(self, h):
        rc = lib.tree_ssd_snapshot_commit(ctypes.byref(self.cshape), _ptr(self.states), _ptr(h), *self.commit_tail)
        if rc != 0:
            raise TreeSSDError(rc, "tree_ssd_snapshot_commit")
