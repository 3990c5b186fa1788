"""ctypes front end of the fp64 C oracle (oracle.c). TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and the benchmark's CPU-baseline
leg import this module; the product path never does. It shares no code with
the HIP library: it gathers per-(batch item, head) slices from the seeded input
dict (plain indexing and exact bf16 -> float64 widening) and hands them to the
C routines, which follow "STree: Speculative Tree Decoding for Hybrid State
Space Models" (atlas.scime.ai summary, section "Approach").
"""
from __future__ import annotations

import ctypes
import os
from typing import Dict, Optional, Sequence, Tuple

import numpy as np

from speculative_tree_verification_amd.workloads import BF16, F32, to_f64

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "liboracle.so")

_lib = None

_dp = ctypes.POINTER(ctypes.c_double)
_ip = ctypes.POINTER(ctypes.c_int32)
_up = ctypes.POINTER(ctypes.c_uint64)


def lib():
    """Load (building first if needed) the oracle shared library."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH) or os.path.getmtime(LIB_PATH) < os.path.getmtime(
                os.path.join(HERE, "oracle.c")):
            from oracle.build import build
            build()
        L = ctypes.CDLL(LIB_PATH)
        L.oracle_tree_check.argtypes = [ctypes.c_int, _ip]
        L.oracle_tree_check.restype = ctypes.c_int
        L.oracle_tree_info.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_int, _ip, _ip, _up, _ip]
        L.oracle_tree_info.restype = None
        vargs = [ctypes.c_int] * 4 + [_dp] * 7 + [_ip, _dp, _ip]
        L.oracle_verify.argtypes = vargs
        L.oracle_verify.restype = None
        L.oracle_packed_verify.argtypes = vargs
        L.oracle_packed_verify.restype = None
        L.oracle_commit.argtypes = [ctypes.c_int] * 4 + [_dp] * 5 + [_ip, _ip, _ip, ctypes.c_int, _dp, _ip]
        L.oracle_commit.restype = None
        L.oracle_num_threads.argtypes = []
        L.oracle_num_threads.restype = ctypes.c_int
        L.oracle_set_num_threads.argtypes = [ctypes.c_int]
        L.oracle_set_num_threads.restype = None
        _lib = L
    return _lib


def _d(a: np.ndarray):
    return a.ctypes.data_as(_dp)


def _i(a: np.ndarray):
    return a.ctypes.data_as(_ip)


def num_threads() -> int:
    return lib().oracle_num_threads()


def set_num_threads(t: int) -> None:
    lib().oracle_set_num_threads(int(t))


# ---------------------------------------------------------------------------
# slice-level API: every slice is one (item, head) problem with its own tree
# ---------------------------------------------------------------------------
def verify_slices(x, dt, A, Bm, Cm, D, h0, parent, packed: bool = False):
    """y [n, T, P] from slice arrays x [n,T,P], dt [n,T], A [n], B/C [n,T,N],
    D [n], h0 [n,P,N], parent [n,T]. Returns (y, status)."""
    x = np.ascontiguousarray(x, np.float64)
    n, T, P = x.shape
    N = Bm.shape[-1]
    arrs = [np.ascontiguousarray(a, np.float64) for a in (dt, A, Bm, Cm, D, h0)]
    parent = np.ascontiguousarray(parent, np.int32).reshape(n, T)
    y = np.zeros((n, T, P), np.float64)
    st = np.zeros(n, np.int32)
    fn = lib().oracle_packed_verify if packed else lib().oracle_verify
    fn(n, T, P, N, _d(x), *[_d(a) for a in arrs], _i(parent), _d(y), _i(st))
    return y, st


def commit_slices(x, dt, A, Bm, h0, parent, accepted, accepted_len, Lmax: Optional[int] = None):
    """Final state [n, P, N] after the accepted path of every slice. Returns (h, status)."""
    x = np.ascontiguousarray(x, np.float64)
    n, T, P = x.shape
    N = Bm.shape[-1]
    dt, A, Bm, h0 = [np.ascontiguousarray(a, np.float64) for a in (dt, A, Bm, h0)]
    parent = np.ascontiguousarray(parent, np.int32).reshape(n, T)
    accepted = np.ascontiguousarray(accepted, np.int32)
    if Lmax is None:
        Lmax = accepted.shape[-1]
    accepted = accepted.reshape(n, Lmax)
    accepted_len = np.ascontiguousarray(accepted_len, np.int32).reshape(n)
    h = np.array(h0, copy=True)
    st = np.zeros(n, np.int32)
    lib().oracle_commit(n, T, P, N, _d(x), _d(dt), _d(A), _d(Bm), _d(h0), _i(parent),
                        _i(accepted), _i(accepted_len), int(Lmax), _d(h), _i(st))
    return h, st


def anc_words(T: int) -> int:
    """64-bit words per node of an ancestor bit set: 4 up to 256 nodes, then
    one word per 64 nodes."""
    return max(4, -(-T // 64))


def tree_info(parent: np.ndarray):
    """(depth [n,T], anc [n,T,W] uint64 with W = anc_words(T), status [n]) for
    parent [n, T]."""
    parent = np.ascontiguousarray(parent, np.int32)
    n, T = parent.shape
    W = anc_words(T)
    depth = np.zeros((n, T), np.int32)
    anc = np.zeros((n, T, W), np.uint64)
    st = np.zeros(n, np.int32)
    lib().oracle_tree_info(n, T, W, _i(parent), _i(depth), anc.ctypes.data_as(_up), _i(st))
    return depth, anc, st


def tree_check(parent_row: np.ndarray) -> int:
    p = np.ascontiguousarray(parent_row, np.int32)
    return int(lib().oracle_tree_check(len(p), _i(p)))


# ---------------------------------------------------------------------------
# input-dict API (layouts of the seeded workloads)
# ---------------------------------------------------------------------------
def gather_slices(inp: Dict[str, np.ndarray], dtype: str, sel: Sequence[Tuple[int, int]]):
    """Slice arrays (float64) for the (b, h) pairs in ``sel``. Pure indexing."""
    B, T, H, P = inp["x"].shape
    G = inp["B"].shape[2]
    hpg = H // G
    bs = np.array([s[0] for s in sel], dtype=np.int64)
    hs = np.array([s[1] for s in sel], dtype=np.int64)
    gs = hs // hpg
    x = to_f64(inp["x"][bs, :, hs, :], dtype) if len(sel) else np.zeros((0, T, P))
    dt = to_f64(inp["dt"][bs, :, hs], dtype) if len(sel) else np.zeros((0, T))
    Bm = to_f64(inp["B"][bs, :, gs, :], dtype)
    Cm = to_f64(inp["C"][bs, :, gs, :], dtype)
    A = inp["A"].astype(np.float64)[hs]
    D = inp["D"].astype(np.float64)[hs]
    h0 = inp["h0"].astype(np.float64)[bs, hs]
    parent = inp["parent"][bs]
    return dict(x=x, dt=dt, A=A, B=Bm, C=Cm, D=D, h0=h0, parent=parent,
                accepted=inp["accepted"][bs], accepted_len=inp["accepted_len"][bs])


def all_pairs(inp) -> list:
    B, T, H, P = inp["x"].shape
    return [(b, h) for b in range(B) for h in range(H)]


def verify(inp: Dict[str, np.ndarray], dtype: str, sel=None, packed: bool = False):
    """Oracle y for the selected (b, h) pairs (all if None): ([n, T, P], status[n])."""
    sel = all_pairs(inp) if sel is None else list(sel)
    s = gather_slices(inp, dtype, sel)
    return verify_slices(s["x"], s["dt"], s["A"], s["B"], s["C"], s["D"], s["h0"], s["parent"],
                         packed=packed)


def verify_full(inp: Dict[str, np.ndarray], dtype: str):
    """Oracle y in the [B, T, H, P] layout (float64) and per-item status [B]."""
    B, T, H, P = inp["x"].shape
    y, st = verify(inp, dtype)
    return y.reshape(B, H, T, P).transpose(0, 2, 1, 3).copy(), st.reshape(B, H)[:, 0].copy()


def commit(inp: Dict[str, np.ndarray], dtype: str, sel=None):
    """Oracle committed state for the selected (b, h) pairs: ([n, P, N], status[n])."""
    sel = all_pairs(inp) if sel is None else list(sel)
    s = gather_slices(inp, dtype, sel)
    return commit_slices(s["x"], s["dt"], s["A"], s["B"], s["h0"], s["parent"], s["accepted"],
                         s["accepted_len"], Lmax=inp["accepted"].shape[-1])


def commit_full(inp: Dict[str, np.ndarray], dtype: str):
    """Oracle committed state [B, H, P, N] (float64) and per-item status [B]."""
    B, T, H, P = inp["x"].shape
    N = inp["B"].shape[-1]
    h, st = commit(inp, dtype)
    return h.reshape(B, H, P, N), st.reshape(B, H)[:, 0].copy()
