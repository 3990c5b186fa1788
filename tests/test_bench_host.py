"""Host-side bookkeeping of bench.py (no GPU): algorithmic byte and flop
counts against closed forms, the gpus>1 refusal and the source digest."""
import os
import subprocess
import sys

import numpy as np

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402


def test_ancestor_pairs_closed_forms():
    T = 9
    chain = np.array([[-1] + list(range(T - 1))])
    star = np.array([[-1] + [0] * (T - 1)])
    binary = np.array([[-1, 0, 0, 1, 1, 2, 2]])
    assert bench.ancestor_pairs(chain) == [T * (T + 1) // 2]
    assert bench.ancestor_pairs(star) == [1 + 2 * (T - 1)]
    assert bench.ancestor_pairs(binary) == [1 + 2 * 2 + 4 * 3]
    assert bench.ancestor_pairs(np.concatenate([chain, star])) == [45, 17]


def test_verify_flops_and_bytes():
    # one item, one head, one group: read-out 2 T N P, pair scores 2 N pairs, pair sums 2 P pairs
    assert bench.verify_flops(1, 7, 1, 16, 8, 1, [17]) == 2 * 7 * 8 * 16 + 2 * 8 * 17 + 2 * 16 * 17
    # heads share the pair scores of their group
    assert bench.verify_flops(2, 3, 4, 2, 5, 2, [6, 6]) == 2 * 2 * 4 * 3 * 5 * 2 + 2 * 5 * 2 * 12 + 2 * 2 * 4 * 12
    # bytes: h0 once (4 P N per item and head), x, y, dt, B, C, A, D, parent
    B, T, H, P, N, G, io = 2, 5, 3, 4, 6, 1, 2
    want = 4 * B * H * P * N + io * (2 * B * T * H * P + B * T * H + 2 * B * T * G * N) + 8 * H + 4 * B * T
    assert bench.verify_bytes(B, T, H, P, N, G, io) == want


def test_multi_gpu_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2 and "one GPU" in r.stderr


def test_source_digest_ignores_comments(tmp_path, monkeypatch):
    assert bench._code_only("int a; // note\n/* block\n */ int b;") == "int a; int b;"
    assert len(bench.source_sha("verify")) == 16 and len(bench.source_sha("commit")) == 16
