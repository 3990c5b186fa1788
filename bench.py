#!/usr/bin/env python3
"""Throughput of packed-tree SSD verification + commit on one MI355X.

A step is one pass of the whole hot path over one batch of synthetic input:
tree_ssd_verify for every layer of the workload (one launch per layer: in a
model each layer's input comes from the layer before), then the commit of
every layer (the accepted path is part of the input). The layers' commits are
independent once the path is known, so a multi-layer workload commits all of
them in one tree_ssd_commit_layers launch; a one-layer workload calls
tree_ssd_commit. Inputs are resident in
HBM before the timed region; several copies of the input set rotate so the
256 MB Infinity Cache cannot serve them.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload N]

Prints one JSON line (metric, value in tree nodes/s, roofline of the dominant
kernel from HIP events, CPU-oracle baseline). Diagnostics go to stderr.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "tree-verify nodes/sec (batch×nodes×heads×layers) at 1 GPU; % peak HBM GB/s"
PEAK_HBM_GBS = 8000.0
PEAK_BF16_TFLOPS = 2500.0  # dense bf16 MFMA (no sparsity)
ROTATE_BYTES = 1100 << 20  # rotating input sets: more than 1 GB, far past the 256 MB Infinity Cache


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def parse():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", type=int, default=1,
                    help="workload configuration id (0-4); default 1, the 64-layer Mamba2-2.7B step")
    ap.add_argument("--secondary", default="2,3,4",
                    help="comma list of further workloads measured in the same run ('' for none)")
    ap.add_argument("--secondary-steps", type=int, default=50)
    ap.add_argument("--reps", type=int, default=50,
                    help="timed regions per kernel (median and minimum are taken over them)")
    ap.add_argument("--rotate-mib", type=int, default=ROTATE_BYTES >> 20,
                    help="total size of the rotating input sets (MiB)")
    ap.add_argument("--no-oracle", action="store_true", help="skip the CPU-oracle baseline")
    ap.add_argument("--no-gdn", action="store_true", help="skip the gated-delta-rule tree kernels")
    ap.add_argument("--no-large", action="store_true", help="skip the 1023-node tree measurement")
    ap.add_argument("--baselines", default="1,2,3,4",
                    help="workloads on which the unrolled and snapshot forms are timed beside the packed "
                         "form ('' for none)")
    ap.add_argument("--oracle-seconds", type=float, default=12.0,
                    help="target CPU time of the oracle sample")
    ap.add_argument("--heads-per-block", type=int, default=0)
    ap.add_argument("--copy-calibration", action="store_true",
                    help="only run a plain device copy and a sum of known size (HBM counter calibration)")
    return ap.parse_args()


# ---------------------------------------------------------------------------
# algorithmic bytes per launch (what the method must move; no per-node state)
# ---------------------------------------------------------------------------
def step_hbm(v, c, ms_per_step):
    """The whole layer's algorithmic HBM rate: the bytes of every verify and
    commit launch of one step over the step time (verify and commit run back
    to back, launch gaps included)."""
    nbytes = v["algorithmic_bytes"] * v["launches_per_step"] + c["algorithmic_bytes"] * c["launches_per_step"]
    gbs = nbytes / (ms_per_step * 1e-3) / 1e9
    return {"algorithmic_bytes": nbytes, "achieved": round(gbs, 1), "unit": "GB/s",
            "frac": round(gbs / PEAK_HBM_GBS, 4), "timing": "step time: every verify and commit launch back to back"}


def verify_bytes(B, T, H, P, N, G, io):
    return (io * (2 * B * T * H * P + B * T * H + 2 * B * T * G * N) + 4 * B * H * P * N
            + 8 * H + 4 * B * T)


def commit_bytes(B, T, H, P, N, G, io, path_lens, Lmax):
    L = int(sum(path_lens))
    return (8 * B * H * P * N + L * io * (H * P + H + G * N) + 4 * B * T + 4 * B * Lmax + 4 * B
            + 4 * H)


def ancestor_pairs(parent):
    """Sum over nodes of (depth + 1) for each row of parent [B][T]: the
    (node, ancestor-or-self) pairs of each item's tree."""
    import numpy as np
    parent = np.asarray(parent)
    out = []
    for row in parent:
        depth = np.zeros(len(row), dtype=np.int64)
        for i in range(1, len(row)):
            depth[i] = depth[row[i]] + 1
        out.append(int(depth.sum() + len(row)))
    return out


def verify_flops(B, T, H, P, N, G, pairs):
    """Algorithmic flops of one verify launch: the dense read-out C h0^T
    (2 T N P per item and head), the pair scores C_i . B_j on ancestor pairs
    only (2 N per pair, per item and group) and the weighted sum over x rows on
    ancestor pairs only (2 P per pair, per item and head)."""
    npairs = sum(pairs)
    return 2 * B * H * T * N * P + 2 * N * G * npairs + 2 * P * H * npairs


def mfma_report(flops, us, nbytes):
    """A verify launch's algorithmic flops over its average duration, against
    the dense bf16 MFMA peak."""
    tf = flops / (us * 1e-6) / 1e12
    return {"bound": "mfma", "achieved": round(tf, 2), "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
            "frac": round(tf / PEAK_BF16_TFLOPS, 5), "algorithmic_flops": int(flops),
            "intensity_flop_per_byte": round(flops / nbytes, 2)}


KERNEL_SOURCES = {
    "verify": ("api.hip", "launch.hpp", "common.hpp", "verify_common.hpp", "verify_tiny.hip",
               "verify_mfma.hip", "verify_wide.hip", "verify_generic.hip"),
    "commit": ("api.hip", "launch.hpp", "common.hpp", "commit.hip"),
}


def _code_only(text):
    """Source text without comments and with whitespace collapsed."""
    import re
    text = re.sub(r"/\*.*?\*/", " ", text, flags=re.S)
    text = re.sub(r"//[^\n]*", " ", text)
    return " ".join(text.split())


def source_sha(kernel):
    """Digest of the code (comments aside) of the sources a kernel is built
    from: its HBM counters are void once any of that code changes."""
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "speculative_tree_verification_amd", "csrc")
    for n in KERNEL_SOURCES[kernel]:
        with open(os.path.join(csrc, n)) as f:
            h.update(n.encode() + b"\0" + _code_only(f.read()).encode())
    return h.hexdigest()[:16]


def traffic_record(kernel, workload, sha):
    """HBM bytes per launch from the committed rocprofv3 counter runs (the fenced
    JSON block of profiles/hbm_traffic.md), if taken on the current sources."""
    path = os.path.join(ROOT, "profiles", "hbm_traffic.md")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        text = f.read()
    a = text.find("```json")
    if a < 0:
        return None
    b = text.find("```", a + 7)
    try:
        recs = json.loads(text[a + 7:b])
    except ValueError:
        return None
    for r in recs.get("records", []):
        if r.get("kernel") == kernel and r.get("workload") == workload and r.get("source_sha") == sha:
            return r
    return None


# ---------------------------------------------------------------------------
class Workload:
    """All layers of one configuration, resident on the GPU, in S rotating sets."""

    def __init__(self, cid, torch, bnd, W, heads_per_block=0, keep_host=False):
        self.cid = cid
        self.cfg = cfg = W.CONFIGS[cid]
        self.io = 2 if cfg.dtype == W.BF16 else 4
        t0 = time.time()
        self.host = []
        layers = []
        for l in range(cfg.layers):
            inp = W.make_inputs(cid, l)
            if keep_host:
                self.host.append(inp)
            layers.append(bnd.to_device(inp))
        log(f"[bench] workload {cid} ({cfg.name}): generated {cfg.layers} layer(s) in {time.time() - t0:.1f}s")
        B, T, H, P = layers[0]["x"].shape
        G, N = layers[0]["B"].shape[2], layers[0]["B"].shape[3]
        self.dims = (B, T, H, P, N, G)
        self.path_lens = [int(v) for v in layers[0]["accepted_len"].cpu().tolist()]
        self.pairs = ancestor_pairs(layers[0]["parent"].cpu().numpy())
        self.Lmax = layers[0]["accepted"].shape[1]
        set_bytes = sum(t.numel() * t.element_size() for d in layers for t in d.values())
        set_bytes += sum(d["x"].numel() * d["x"].element_size() for d in layers)  # y
        self.n_sets = max(2, -(-ROTATE_BYTES // set_bytes))
        self.sets = [layers]
        for s in range(1, self.n_sets):
            self.sets.append([{k: v.clone() for k, v in d.items()} for d in layers])
        self.verify_calls, self.commit_calls = [], []
        for layers_s in self.sets:
            vc = []
            for d in layers_s:
                y = torch.empty_like(d["x"])
                d["y"] = y
                vc.append(bnd.PreparedVerify(d["x"], d["dt"], d["A"], d["B"], d["C"], d["D"],
                                             d["h0"], d["parent"], y,
                                             heads_per_block=heads_per_block))
            d0 = layers_s[0]
            if len(layers_s) > 1:
                # one tree and one accepted path for every layer of the step
                cc = [bnd.PreparedCommitLayers(
                    [(d["x"], d["dt"], d["A"], d["B"], d["h0"]) for d in layers_s],
                    d0["parent"], d0["accepted"], d0["accepted_len"])]
            else:
                cc = [bnd.PreparedCommit(d0["x"], d0["dt"], d0["A"], d0["B"], d0["h0"], d0["parent"],
                                         d0["accepted"], d0["accepted_len"])]
            self.verify_calls.append(vc)
            self.commit_calls.append(cc)
        torch.cuda.synchronize()
        log(f"[bench] {self.n_sets} rotating sets of {set_bytes / 2**20:.1f} MiB")

    @property
    def nodes_per_step(self):
        B, T, H, P, N, G = self.dims
        return B * T * H * self.cfg.layers

    def step(self, s):
        """Enqueue one step on input set s: verify for every layer, then commit
        for every layer."""
        for f in self.verify_calls[s]:
            f()
        for f in self.commit_calls[s]:
            f()

    def algorithmic_bytes(self):
        """Per launch: one layer's verify; the commit launch covers every layer."""
        B, T, H, P, N, G = self.dims
        return (verify_bytes(B, T, H, P, N, G, self.io),
                self.cfg.layers * commit_bytes(B, T, H, P, N, G, self.io, self.path_lens, self.Lmax))

    @property
    def commit_api(self):
        return "tree_ssd_commit_layers" if self.cfg.layers > 1 else "tree_ssd_commit"


def sleep_cycles_for(torch, ms):
    """Cycles of torch.cuda._sleep that keep the GPU busy for about ms."""
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    torch.cuda._sleep(1_000_000)
    e1.record()
    torch.cuda.synchronize()
    per = max(e0.elapsed_time(e1), 1e-3) / 1_000_000
    return int(ms / per)


WARM_MS = 30.0  # GPU time of the untimed burst ahead of each timed region


def timed_region(torch, fn, rounds):
    """Average ms per call over `rounds` back-to-back calls fn(0), fn(1), ...,
    timed with one HIP event pair. An untimed burst of the same calls, about
    WARM_MS of GPU time, goes first: under it the GPU settles into the clock
    and power state it keeps under this load (a GPU left idle, or spinning in
    a sleep kernel, starts the region in a transient that runs several percent
    slower for the first few milliseconds), and the host enqueues the timed
    calls while the burst still runs, so the region measures GPU execution.
    Where one call takes the host about as long to enqueue as the GPU to run,
    a sleep kernel of the region's enqueue time goes between the two."""
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for i in range(3):
        fn(i)
    e1.record()
    torch.cuda.synchronize()
    per_call = max(e0.elapsed_time(e1) / 3, 1e-3)
    nwarm = max(3, int(WARM_MS / per_call) + 1)
    t0 = time.perf_counter()
    for i in range(nwarm):
        fn(i)
    host_ms = (time.perf_counter() - t0) * 1e3 / nwarm
    if host_ms > 0.8 * per_call:
        # the host enqueues a call about as slowly as the GPU runs it: a short
        # sleep kernel, sized to the enqueue time of the region, lets it get
        # ahead (the GPU idles only that long)
        torch.cuda._sleep(sleep_cycles_for(torch, 1.3 * host_ms * rounds + 0.5))
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    start.record()
    for i in range(rounds):
        fn(i)
    end.record()
    torch.cuda.synchronize()
    return start.elapsed_time(end) / rounds


def timed_stats(torch, fn, reps, rounds):
    """Per-call duration statistics over `reps` timed regions of `rounds`
    back-to-back calls each (one HIP event pair per region, the regions back to
    back after one untimed burst as in timed_region). Returns mean, median and
    minimum of the per-region averages, in ms per call."""
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for i in range(3):
        fn(i)
    e1.record()
    torch.cuda.synchronize()
    per_call = max(e0.elapsed_time(e1) / 3, 1e-3)
    nwarm = max(3, int(WARM_MS / per_call) + 1)
    t0 = time.perf_counter()
    for i in range(nwarm):
        fn(i)
    host_ms = (time.perf_counter() - t0) * 1e3 / nwarm
    if host_ms > 0.8 * per_call:
        torch.cuda._sleep(sleep_cycles_for(torch, 1.3 * host_ms * rounds * reps + 0.5))
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(reps + 1)]
    k = 0
    ev[0].record()
    for r in range(reps):
        for _ in range(rounds):
            fn(k)
            k += 1
        ev[r + 1].record()
    torch.cuda.synchronize()
    per = sorted(ev[r].elapsed_time(ev[r + 1]) / rounds for r in range(reps))
    mean = ev[0].elapsed_time(ev[reps]) / (rounds * reps)
    return {"mean": mean, "median": per[len(per) // 2], "min": per[0], "reps": reps,
            "calls_per_rep": rounds}


def graph_step_timing(torch, bnd, wl, steps):
    """The same step captured once per rotating input set as a HIP graph (the
    launches re-pointed at a side stream for the capture), replayed `steps`
    times between two events. Reported beside the stream-launch figure."""
    cap = torch.cuda.Stream()
    graphs, keep = [], []
    for layers_s in wl.sets:
        with torch.cuda.stream(cap):
            vc = [bnd.PreparedVerify(d["x"], d["dt"], d["A"], d["B"], d["C"], d["D"], d["h0"],
                                     d["parent"], d["y"], stream=cap) for d in layers_s]
            d0 = layers_s[0]
            if len(layers_s) > 1:
                cc = bnd.PreparedCommitLayers([(d["x"], d["dt"], d["A"], d["B"], d["h0"]) for d in layers_s],
                                              d0["parent"], d0["accepted"], d0["accepted_len"], stream=cap)
            else:
                cc = bnd.PreparedCommit(d0["x"], d0["dt"], d0["A"], d0["B"], d0["h0"], d0["parent"],
                                        d0["accepted"], d0["accepted_len"], stream=cap)
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=cap):
            for f in vc:
                f()
            cc()
        graphs.append(g)
        keep.append((vc, cc))
    torch.cuda.synchronize()
    ms = timed_region(torch, lambda i: graphs[i % len(graphs)].replay(), steps)
    del graphs, keep
    return ms


def time_steps(torch, wl, steps, warmup, reps=50):
    """Warm up, then time exactly `steps` steps with HIP events (see
    timed_region: an untimed burst of the same steps runs first, so the region
    measures back-to-back launches in the GPU's steady state under this load,
    with the host enqueueing ahead).

    The average launch duration of each kernel comes from two further timed
    regions of the same kind: the step's verify launches alone, then its commit
    launches alone, `steps` rounds each over the rotating input sets, one event
    pair around each region (events between single launches would add their
    own overhead to every launch)."""
    host_t = []
    for i in range(warmup):
        t0 = time.perf_counter()
        wl.step(i % wl.n_sets)
        host_t.append(time.perf_counter() - t0)
        torch.cuda.synchronize()
    host_per_step = min(host_t) if host_t else 5e-3

    def region(fn, rounds):
        # barrier (one rank) + synchronize on both sides of the timed region
        return timed_region(torch, lambda i: fn(i % wl.n_sets), rounds) * rounds

    ms = region(wl.step, steps)
    nv, nc = len(wl.verify_calls[0]), len(wl.commit_calls[0])

    def run_all(calls):
        for f in calls:
            f()

    # per-launch statistics: `reps` regions, each of `rounds` steps' launches of
    # one kernel (about a millisecond of GPU time or more per region)
    step_stats = timed_stats(torch, lambda i: wl.step(i % wl.n_sets), reps, 1)
    rounds = max(1, min(steps, 20))
    vs = timed_stats(torch, lambda i: run_all(wl.verify_calls[i % wl.n_sets]), reps, rounds)
    cs = timed_stats(torch, lambda i: run_all(wl.commit_calls[i % wl.n_sets]), reps, rounds)
    scale = lambda st, n: {k: (v * 1e3 / n if k in ("mean", "median", "min") else v) for k, v in st.items()}
    vs, cs = scale(vs, nv), scale(cs, nc)
    return dict(ms_per_step=ms / steps, verify_us=vs["median"], commit_us=cs["median"],
                verify_stats=vs, commit_stats=cs, step_stats=step_stats,
                host_ms=1e3 * host_per_step, verify_launches=nv, commit_launches=nc)


GDN_SHAPE = dict(batch=16, n_nodes=31, n_heads=16, dk=128, dv=128)


def gdn_cpu_baseline(base, seconds):
    """The fp64 gated-delta-rule oracle (numpy) on a bounded sample of the same
    inputs: whole items (all heads), verify + commit as the unrolled
    recurrence, one item per worker thread (one BLAS thread each) on the
    host's OpenMP thread count, cycled until about `seconds` of wall time."""
    import concurrent.futures
    import numpy as np
    from threadpoolctl import threadpool_limits
    from oracle import gdn as OG
    from oracle import oracle as O
    B, T, H, _ = base["k"].shape
    f = lambda a: a.astype(np.float64) if a.dtype == np.float32 else a
    items = [{k: f(v[b:b + 1]) for k, v in base.items()} for b in range(B)]
    nthr = max(1, O.num_threads())

    def one(sl):
        OG.verify_unrolled(sl["q"], sl["k"], sl["v"], sl["g"], sl["beta"], sl["S0"], sl["parent"])
        OG.commit_unrolled(sl["k"], sl["v"], sl["g"], sl["beta"], sl["S0"], sl["parent"],
                           sl["accepted"], sl["accepted_len"])
        return T * H

    done, parts = 0, 0
    t0 = time.perf_counter()
    with threadpool_limits(1), concurrent.futures.ThreadPoolExecutor(nthr) as ex:
        while time.perf_counter() - t0 < seconds:
            batch = [items[(parts + i) % B] for i in range(nthr)]
            done += sum(ex.map(one, batch))
            parts += nthr
    used = time.perf_counter() - t0
    return {"value": round(done / used, 1), "unit": "nodes/s", "cores": nthr, "kind": "oracle",
            "sample": f"{parts} items cycled over the workload's {B}, all {H} heads each: verify + commit "
                      f"(the unrolled recurrence) in fp64 numpy, {nthr} worker threads (Python loops "
                      f"share one interpreter lock), {used:.1f} s", "seconds": round(used, 2), **host_cpus()}


def large_cpu_baseline(base, seconds):
    """The fp64 C oracle on a bounded sample of the large-tree inputs: items,
    all heads each, verify + commit, cycled until about `seconds`."""
    from oracle import oracle as O
    B, T, H, _ = base["x"].shape
    done, used, parts = 0, 0.0, 0
    while used < seconds:
        b = parts % B
        s = O.gather_slices(base, "bf16", [(b, h) for h in range(H)])
        t0 = time.perf_counter()
        O.verify_slices(s["x"], s["dt"], s["A"], s["B"], s["C"], s["D"], s["h0"], s["parent"])
        O.commit_slices(s["x"], s["dt"], s["A"], s["B"], s["h0"], s["parent"], s["accepted"],
                        s["accepted_len"], Lmax=base["accepted"].shape[-1])
        used += time.perf_counter() - t0
        done += T * H
        parts += 1
    return {"value": round(done / used, 1), "unit": "nodes/s", "cores": O.num_threads(), "kind": "oracle",
            "sample": f"{parts} items cycled over the workload's {B}, all {H} heads each: verify + commit "
                      f"in fp64, {used:.1f} s of oracle time", "seconds": round(used, 2), **host_cpus()}


def gdn_timing(torch, bnd, W, rounds, oracle_seconds=0.0, dtype="f32", shape=None, tree="recursive"):
    """Gated-delta-rule tree verify and commit on a batch-16 layer (16 heads,
    dk = dv = 128; q, k, v and o fp32 or bf16) over 31-node random trees, or
    the shape and trees given, rotating input sets; average durations of
    back-to-back launches of each kernel alone."""
    import numpy as np
    sh = shape or GDN_SHAPE
    base = W.make_gdn(31, **sh, max_path_len=5, dtype=dtype, tree=tree)
    B, T, H, dk, dv = sh["batch"], sh["n_nodes"], sh["n_heads"], sh["dk"], sh["dv"]
    io = 2 if dtype == W.BF16 else 4
    one = sum(a.nbytes for a in base.values()) + base["v"].nbytes + 4 * base["v"].size
    nsets = max(2, -(-ROTATE_BYTES // one))

    def up(v):
        t = torch.from_numpy(np.ascontiguousarray(v))
        return (t.view(torch.int16).view(torch.bfloat16) if v.dtype == np.uint16 else t).cuda()
    sets = []
    for i in range(nsets):
        d = {k: up(v) for k, v in base.items()}
        d["o"] = torch.empty_like(d["v"])
        d["e"] = torch.empty(d["v"].shape, dtype=torch.float32, device=d["v"].device)
        sets.append(d)

    def ver(d):
        bnd.gdn_verify(d["q"], d["k"], d["v"], d["g"], d["beta"], d["S0"], d["parent"], o=d["o"], e=d["e"])

    def com(d):
        bnd.gdn_commit(d["k"], d["g"], d["e"], d["S0"], d["parent"], d["accepted"], d["accepted_len"])

    out = {"workload": f"gdn-b{B}-tree{T}{'-' + tree if tree != 'recursive' else ''}-h{H}-dk{dk}-dv{dv}",
           "dtype": dtype}
    L = int(base["accepted_len"].sum())
    # verify: q, k, v read and o written in the input type; e written, g,
    # beta, S0 and the parents read in fp32 / int32. commit: S0 read and
    # written, the path's k rows (input type), e rows and g.
    nbytes = {"verify": B * T * H * (io * (2 * dk + 2 * dv) + 4 * dv + 8) + 4 * B * H * dv * dk + 4 * B * T,
              "commit": 8 * B * H * dv * dk + L * H * (io * dk + 4 * dv + 4) + 4 * B * (T + 6)}
    for name, fn in (("verify", ver), ("commit", com)):
        for d in sets:
            fn(d)
        us = timed_region(torch, lambda r: fn(sets[r % nsets]), rounds) * 1e3
        gbs = nbytes[name] / (us * 1e-6) / 1e9
        out[name] = {"avg_us": round(us, 3), "algorithmic_bytes": nbytes[name], "achieved": round(gbs, 1),
                     "unit": "GB/s", "frac": round(gbs / PEAK_HBM_GBS, 4)}
    out["nodes_per_s"] = round(B * T * H / ((out["verify"]["avg_us"] + out["commit"]["avg_us"]) * 1e-6), 1)
    if oracle_seconds > 0:
        out["cpu_baseline"] = gdn_cpu_baseline(base, oracle_seconds)
    return out


LARGE_SHAPE = dict(batch=4, n_nodes=1023, n_heads=80, head_dim=64, d_state=128, n_groups=1)


def large_timing(torch, bnd, W, rounds, oracle_seconds=0.0):
    """Packed trees past 256 nodes: complete binary trees of 1023 nodes (depth
    9) at batch 4 with the Mamba2-2.7B head shape, bf16, paths of 1-10 nodes;
    average durations of back-to-back verify and commit launches over rotating
    input sets."""
    sh = LARGE_SHAPE
    base = W.make_custom(23, **sh, dtype=W.BF16, tree="binary", max_path_len=10)
    B, T, H, P, N, G = W.shape_of(base)
    one = sum(a.nbytes for a in base.values()) + base["x"].nbytes
    nsets = max(2, -(-ROTATE_BYTES // one))
    d0 = bnd.to_device(base)
    sets = [d0 if i == 0 else {k: v.clone() for k, v in d0.items()} for i in range(nsets)]
    for d in sets:
        d["y"] = torch.empty_like(d["x"])
    pv = [bnd.PreparedVerify(d["x"], d["dt"], d["A"], d["B"], d["C"], d["D"], d["h0"], d["parent"], d["y"])
          for d in sets]
    pc = [bnd.PreparedCommit(d["x"], d["dt"], d["A"], d["B"], d["h0"], d["parent"], d["accepted"],
                             d["accepted_len"]) for d in sets]
    out = {"workload": f"mamba2-2.7b-b{B}-tree{T}-binary", "dtype": "bf16"}
    nbytes = {"verify": verify_bytes(B, T, H, P, N, G, 2),
              "commit": commit_bytes(B, T, H, P, N, G, 2, [int(v) for v in base["accepted_len"]],
                                     base["accepted"].shape[1])}
    for name, fns in (("verify", pv), ("commit", pc)):
        for f in fns:
            f()
        us = timed_region(torch, lambda r: fns[r % nsets](), rounds) * 1e3
        gbs = nbytes[name] / (us * 1e-6) / 1e9
        out[name] = {"avg_us": round(us, 3), "algorithmic_bytes": nbytes[name], "achieved": round(gbs, 1),
                     "unit": "GB/s", "frac": round(gbs / PEAK_HBM_GBS, 4)}
    out["verify"]["mfma"] = mfma_report(verify_flops(B, T, H, P, N, G, ancestor_pairs(base["parent"])),
                                        out["verify"]["avg_us"], nbytes["verify"])
    out["nodes_per_s"] = round(B * T * H / ((out["verify"]["avg_us"] + out["commit"]["avg_us"]) * 1e-6), 1)
    del sets, pv, pc
    torch.cuda.empty_cache()
    if oracle_seconds > 0:
        out["cpu_baseline"] = large_cpu_baseline(base, oracle_seconds)
    return out


def accept_timing(torch, bnd, W, wl, rounds):
    """Greedy acceptance on the workload's trees with seeded draft and target
    tokens: average duration of back-to-back launches (one per step, outside
    the step: the step's accepted paths come from the workload)."""
    import numpy as np
    par = wl.sets[0][0]["parent"]
    B, T = par.shape
    draft, target = W.make_tokens(17, par.cpu().numpy(), p_hit=0.7)
    dev = lambda a: torch.from_numpy(np.ascontiguousarray(a, dtype=np.int32)).to(par.device)
    pa = bnd.PreparedAccept(par, dev(draft), dev(target), min(T, 16))
    for _ in range(3):
        pa()
    torch.cuda.synchronize()
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda._sleep(sleep_cycles_for(torch, 2.0))
    start.record()
    for _ in range(rounds):
        pa()
    end.record()
    torch.cuda.synchronize()
    us = start.elapsed_time(end) * 1e3 / rounds
    nbytes = 4 * (3 * B * T + B * min(T, 16) + 3 * B)
    mean_len = float(pa.accepted_len.float().mean().item())
    return {"kernel": "accept_greedy", "avg_us": round(us, 3), "algorithmic_bytes": nbytes,
            "achieved_GBps": round(nbytes / (us * 1e-6) / 1e9, 2), "mean_accepted_len": round(mean_len, 3),
            "timing": "HIP events around back-to-back launches of this kernel alone",
            "bound": "latency (a few KB per launch)"}


def accept_stochastic_timing(torch, bnd, W, wl, reps):
    """Stochastic acceptance (multi-step speculative sampling) on the
    workload's trees with synthetic target and draft distributions over the
    model family's vocabulary, drawn on the GPU. Median and minimum over
    timed regions of back-to-back launches. Algorithmic bytes: the p and q
    rows of every visited node read once, plus the small per-node inputs;
    the kernel re-reads a row once per rejected child (from L2)."""
    import numpy as np
    par = wl.sets[0][0]["parent"].cpu().numpy()
    B, T = par.shape
    V = W.VOCAB[wl.cfg.cid]
    d = W.make_sampling_device(31, par, V, "cuda")
    L = wl.cfg.max_path_len
    pa = bnd.PreparedAcceptStochastic(d["parent"], d["draft"], d["p_target"], d["q_draft"], d["u_node"],
                                      d["u_final"], L)
    for _ in range(3):
        pa()
    torch.cuda.synchronize()
    st = _adaptive_stats(torch, lambda i: pa(), reps)
    lens = pa.accepted_len.cpu().numpy().astype(np.int64)
    nbytes = int(lens.sum()) * 8 * V + 4 * (5 * B * T + B * L + 4 * B)
    us = st["median"]
    del d, pa
    torch.cuda.empty_cache()
    return {"kernel": "accept_stochastic", "vocab": V, "avg_us": round(us, 3), "stats_us": st,
            "algorithmic_bytes": nbytes, "achieved_GBps": round(nbytes / (us * 1e-6) / 1e9, 2),
            "mean_accepted_len": round(float(lens.mean()), 3),
            "timing": "HIP events around back-to-back launches of this kernel alone",
            "bound": "latency: one work-group per item walks the tree; a rejection is one pass over "
                     "the node's p and q rows"}


def _adaptive_stats(torch, fn, reps, min_region_ms=2.0):
    """timed_stats with enough calls per region for about min_region_ms of GPU time."""
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    fn(0)
    e1.record()
    torch.cuda.synchronize()
    rounds = max(1, int(min_region_ms / max(e0.elapsed_time(e1), 1e-3)))
    st = timed_stats(torch, fn, reps, rounds)
    return {k: (round(v * 1e3, 3) if k in ("mean", "median", "min") else v) for k, v in st.items()}


def baseline_forms(torch, bnd, W, cid, reps=20):
    """The packed path against the two forms it replaces, on layer 0 of the
    workload (one input set, the same for all three): the tree unrolled into
    per-leaf sequences (plan, gather of the sequences with one h0 copy each,
    plain sequence scan) and per-node state snapshots (every node's state
    written to HBM; commit copies the accepted node's state). Durations are
    per call (us); transient bytes are what each form writes beyond the packed
    inputs and outputs."""
    inp = W.make_inputs(cid, 0)
    d = bnd.to_device(inp)
    B, T, H, P, N, G = W.shape_of(inp)
    cfg = W.CONFIGS[cid]
    out = {"workload": cfg.name, "layer_calls_per_step": cfg.layers}
    y = torch.empty_like(d["x"])
    pv = bnd.PreparedVerify(d["x"], d["dt"], d["A"], d["B"], d["C"], d["D"], d["h0"], d["parent"], y)
    h = d["h0"].clone()
    pc = bnd.PreparedCommit(d["x"], d["dt"], d["A"], d["B"], h, d["parent"], d["accepted"], d["accepted_len"])
    h_rst = lambda: h.copy_(d["h0"])
    packed_v = _adaptive_stats(torch, lambda i: pv(), reps)
    packed_c = _adaptive_stats(torch, lambda i: pc(), reps)
    h_rst()
    out["packed"] = {"verify_us": packed_v["median"], "commit_us": packed_c["median"], "transient_bytes": 0,
                     "verify_stats_us": packed_v}
    Lcap, S = bnd.unroll_capacity(inp["parent"])
    pu = bnd.PreparedUnrolled(d["x"], d["dt"], d["A"], d["B"], d["C"], d["D"], d["h0"], d["parent"], Lcap, S)
    unrolled_v = _adaptive_stats(torch, lambda i: pu(), reps)
    nl = pu.n_leaves.cpu()
    out["unrolled"] = {"verify_us": unrolled_v["median"], "transient_bytes": pu.materialised_bytes(),
                       "sequences": int(nl.sum()), "sequence_slots": B * Lcap, "positions_per_sequence": S,
                       "verify_stats_us": unrolled_v,
                       "what": "tree_ssd_unroll_plan + tree_ssd_unroll_gather (per-leaf copies of x, dt, B, "
                               "C and of h0) + tree_ssd_seq_scan; commit would replay as in the packed form"}
    del pu
    torch.cuda.empty_cache()
    ps = bnd.PreparedSnapshot(d["x"], d["dt"], d["A"], d["B"], d["C"], d["D"], d["h0"], d["parent"],
                              d["accepted"], d["accepted_len"])
    snap_v = _adaptive_stats(torch, lambda i: ps.verify(), reps)
    hs = d["h0"].clone()
    snap_c = _adaptive_stats(torch, lambda i: ps.commit(hs), reps)
    out["snapshot"] = {"verify_us": snap_v["median"], "commit_us": snap_c["median"],
                       "transient_bytes": ps.materialised_bytes(), "verify_stats_us": snap_v,
                       "what": "tree_ssd_snapshot_verify (every node's state written to HBM) + "
                               "tree_ssd_snapshot_commit (copy of the accepted node's state)"}
    del ps
    torch.cuda.empty_cache()
    pk = out["packed"]["verify_us"]
    out["unrolled_over_packed_verify"] = round(out["unrolled"]["verify_us"] / pk, 2)
    out["snapshot_over_packed_verify"] = round(out["snapshot"]["verify_us"] / pk, 2)
    out["timing"] = "HIP events, median over timed regions of back-to-back calls on one input set"
    return out


def kernel_report(name, us, nbytes, workload, sha, launches, stats=None):
    """Roofline record of one kernel: algorithmic bytes over the median launch
    duration (`us`), with the mean and minimum beside it when `stats` is given."""
    gbs = nbytes / (us * 1e-6) / 1e9
    rec = traffic_record(name, workload, sha)
    traffic = None
    if rec is not None:
        traffic = int(rec["fetch_bytes_per_launch"] + rec["write_bytes_per_launch"])
    out = {"bound": "hbm", "achieved": round(gbs, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
           "frac": round(gbs / PEAK_HBM_GBS, 4), "traffic": traffic,
           "kernel": name, "avg_us": round(us, 3), "algorithmic_bytes": int(nbytes),
           "launches_per_step": launches,
           "timing": "HIP events around back-to-back launches of this kernel alone"}
    if stats is not None:
        out["avg_us_is"] = "median over timed regions"
        out["stats_us"] = {k: (round(v, 3) if isinstance(v, float) else v) for k, v in stats.items()}
    return out


def host_cpus():
    """The host's CPU counts beside the OpenMP threads the oracle used (the
    box's OMP_NUM_THREADS, if set, bounds the latter)."""
    try:
        aff = len(os.sched_getaffinity(0))
    except (AttributeError, OSError):
        aff = None
    return {"host_cpus": os.cpu_count(), "affinity_cpus": aff,
            "omp_num_threads_env": os.environ.get("OMP_NUM_THREADS")}


def cpu_baseline(wl, seconds):
    """The fp64 oracle timed on a bounded sample of the same workload on the host:
    (layer, item) units, all heads each, verify + commit, cycled until about
    `seconds` of oracle time have been spent."""
    from oracle import oracle as O
    B, T, H, P, N, G = wl.dims
    units = [(l, b) for l in range(wl.cfg.layers) for b in range(B)]
    done_nodes, used, parts = 0, 0.0, 0
    while used < seconds:
        l, b = units[parts % len(units)]
        inp = wl.host[l]
        s = O.gather_slices(inp, wl.cfg.dtype, [(b, h) for h in range(H)])
        t0 = time.perf_counter()
        O.verify_slices(s["x"], s["dt"], s["A"], s["B"], s["C"], s["D"], s["h0"], s["parent"])
        O.commit_slices(s["x"], s["dt"], s["A"], s["B"], s["h0"], s["parent"], s["accepted"],
                        s["accepted_len"], Lmax=inp["accepted"].shape[-1])
        used += time.perf_counter() - t0
        done_nodes += T * H
        parts += 1
    what = (f"{parts} (layer, item) units cycled over the workload's {len(units)}, all {H} heads "
            f"each: verify + commit in fp64, {used:.1f} s of oracle time")
    return {"value": round(done_nodes / used, 1), "unit": "nodes/s", "cores": O.num_threads(),
            "kind": "oracle", "sample": what, "seconds": round(used, 2), **host_cpus()}


def run_workload(torch, bnd, W, cid, steps, warmup, hpb, keep_host, reps=50):
    wl = Workload(cid, torch, bnd, W, heads_per_block=hpb, keep_host=keep_host)
    t = time_steps(torch, wl, steps, warmup, reps)
    vb, cb = wl.algorithmic_bytes()
    name = wl.cfg.name
    v = kernel_report("verify", t["verify_us"], vb, name, source_sha("verify"), t["verify_launches"],
                      t["verify_stats"])
    B, T, H, P, N, G = wl.dims
    v["mfma"] = mfma_report(verify_flops(B, T, H, P, N, G, wl.pairs), t["verify_us"], vb)
    c = kernel_report("commit", t["commit_us"], cb, name, source_sha("commit"), t["commit_launches"],
                      t["commit_stats"])
    t["accept"] = accept_timing(torch, bnd, W, wl, steps)
    t["accept_stochastic"] = accept_stochastic_timing(torch, bnd, W, wl, reps)
    nodes_s = wl.nodes_per_step / (t["ms_per_step"] * 1e-3)
    sh = step_hbm(v, c, t["ms_per_step"])
    log(f"[bench] workload {cid}: {t['ms_per_step']:.4f} ms/step, {nodes_s:.4g} nodes/s; "
        f"verify {t['verify_us']:.2f} us ({v['achieved']:.0f} GB/s), "
        f"commit {t['commit_us']:.2f} us ({c['achieved']:.0f} GB/s); whole step {sh['achieved']:.0f} GB/s "
        f"({sh['frac']:.1%}); host {t['host_ms']:.3f} ms/step")
    return wl, t, v, c, nodes_s


def copy_calibration(torch):
    n = 256 << 20
    a = torch.empty(n // 4, dtype=torch.float32, device="cuda").normal_()
    b = torch.empty_like(a)
    for _ in range(5):
        b.copy_(a)
    # a read-only kernel of the same size as a second reference for FETCH_SIZE
    # (a reduction: it reads every byte once and writes a few bytes)
    s = torch.zeros((), dtype=torch.float32, device="cuda")
    for _ in range(5):
        s += a.sum()
    torch.cuda.synchronize()
    print(json.dumps({"copy_bytes_each_way": n, "launches": 5, "sum_bytes_read": n, "sum_launches": 5}))


def main():
    global ROTATE_BYTES
    args = parse()
    ROTATE_BYTES = args.rotate_mib << 20
    if args.gpus != 1:
        print(f"bench.py measures one GPU only (asked for --gpus {args.gpus}); the path has no "
              "multi-GPU mode: heads or items would be sharded with no exchange inside it.",
              file=sys.stderr)
        sys.exit(2)
    import torch
    from speculative_tree_verification_amd import binding as bnd
    from speculative_tree_verification_amd import workloads as W
    assert torch.cuda.is_available(), "bench.py needs a GPU"
    torch.cuda.set_device(0)
    if args.copy_calibration:
        copy_calibration(torch)
        return

    wl, t, v, c, nodes_s = run_workload(torch, bnd, W, args.workload, args.steps, args.warmup,
                                        args.heads_per_block, keep_host=not args.no_oracle,
                                        reps=args.reps)
    B, T, H, P, N, G = wl.dims
    layers = wl.cfg.layers
    # the kernel that takes most of the step's time
    dominant = v if v["avg_us"] * v["launches_per_step"] >= c["avg_us"] * c["launches_per_step"] else c
    roofline = {k: dominant[k] for k in ("bound", "achieved", "peak", "unit", "frac", "traffic")}
    roofline["kernel"] = dominant["kernel"]
    out = {
        "metric": METRIC,
        "value": round(nodes_s, 1),
        "unit": "nodes/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(t["ms_per_step"], 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": wl.cfg.dtype,
        "data": "synthetic (seeded generator; shapes and distributions of the named workload)",
        "config": {"workload": wl.cfg.name, "batch": B, "nodes": T, "heads": H, "head_dim": P,
                   "d_state": N, "groups": G, "layers": layers,
                   "step": (f"{layers} x tree_ssd_verify + 1 x {wl.commit_api}"
                            + (f" ({layers} layers)" if layers > 1 else "")),
                   "rotating_sets": wl.n_sets},
        "roofline": roofline,
        "step_hbm": step_hbm(v, c, t["ms_per_step"]),
        "step_stats_ms": {k: (round(vv, 5) if isinstance(vv, float) else vv)
                          for k, vv in t["step_stats"].items()},
        "kernels": {"verify": v, "commit": c},
        "accept": t["accept"],
        "accept_stochastic": t["accept_stochastic"],
    }
    if layers > 1:
        gms = graph_step_timing(torch, bnd, wl, args.steps)
        out["graph"] = {"ms_per_step": round(gms, 5), "nodes_per_s": round(wl.nodes_per_step / (gms * 1e-3), 1),
                        "timing": "one HIP graph per input set holding the whole step, replayed back to back"}
        log(f"[bench] same step as a captured HIP graph: {gms:.4f} ms/step")
    secondary = []
    for sid in [int(s) for s in args.secondary.split(",") if s.strip()]:
        if sid == args.workload:
            continue
        wl2, t2, v2, c2, ns2 = run_workload(torch, bnd, W, sid, args.secondary_steps, 3,
                                            0, keep_host=False, reps=args.reps)
        secondary.append({"workload": wl2.cfg.name, "nodes_per_s": round(ns2, 1),
                          "ms_per_step": round(t2["ms_per_step"], 5),
                          "step_hbm": step_hbm(v2, c2, t2["ms_per_step"]),
                          "verify": v2, "commit": c2, "accept": t2["accept"],
                          "accept_stochastic": t2["accept_stochastic"]})
        del wl2
        torch.cuda.empty_cache()
    if secondary:
        out["secondary"] = secondary
    bl = [int(c) for c in args.baselines.split(",") if c.strip()]
    if bl:
        out["baselines"] = []
        for cid in bl:
            r = baseline_forms(torch, bnd, W, cid)
            log(f"[bench] forms on {r['workload']}: packed {r['packed']['verify_us']:.1f} us, unrolled "
                f"{r['unrolled']['verify_us']:.1f} us ({r['unrolled']['transient_bytes'] / 2**20:.0f} MiB), "
                f"snapshot {r['snapshot']['verify_us']:.1f} us ({r['snapshot']['transient_bytes'] / 2**20:.0f} MiB)")
            out["baselines"].append(r)
            torch.cuda.empty_cache()
    if not args.no_gdn:
        out["gdn"] = gdn_timing(torch, bnd, W, args.secondary_steps, 0.0 if args.no_oracle else 3.0)
        out["gdn_bf16"] = gdn_timing(torch, bnd, W, args.secondary_steps, 0.0, dtype=W.BF16)
        out["gdn_large"] = gdn_timing(torch, bnd, W, args.secondary_steps, 0.0,
                                      shape=dict(GDN_SHAPE, n_nodes=255), tree="level")
        out["gdn_large_bf16"] = gdn_timing(torch, bnd, W, args.secondary_steps, 0.0, dtype=W.BF16,
                                           shape=dict(GDN_SHAPE, n_nodes=255), tree="level")
        for key in ("gdn", "gdn_bf16", "gdn_large", "gdn_large_bf16"):
            r = out[key]
            log(f"[bench] gated delta rule {r['workload']} {r['dtype']}: verify {r['verify']['avg_us']:.2f} us "
                f"({r['verify']['frac']:.1%}), commit {r['commit']['avg_us']:.2f} us ({r['commit']['frac']:.1%})")
    if not args.no_large:
        out["large"] = large_timing(torch, bnd, W, args.secondary_steps, 0.0 if args.no_oracle else 4.0)
        log(f"[bench] large trees {out['large']['workload']}: verify {out['large']['verify']['avg_us']:.2f} us "
            f"({out['large']['verify']['frac']:.1%}), commit {out['large']['commit']['avg_us']:.2f} us "
            f"({out['large']['commit']['frac']:.1%})")
    if not args.no_oracle:
        log("[bench] timing the CPU oracle on a sample of the workload")
        out["cpu_baseline"] = cpu_baseline(wl, args.oracle_seconds)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
