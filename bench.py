"""Benchmark: decode GEMV throughput on one MI355X.

Default workload: the Qwen3-4B-shaped dense stack in affine4 gs32 (36 layers,
hidden 2560, intermediate 9728, q 4096 x 2560, k/v 1024 x 2560, o 2560 x 4096)
plus a 151936 x 2560 Q8_0 lm_head and its argmax, at M = 1 (one decode token),
on seeded synthetic weights. One step = one token through the whole stack:
per layer the row-concatenated q|k|v GEMV, o, row-concatenated gate|up, down
(the order a decoder layer consumes them in), then lm_head and argmax. The
step is captured once as a HIP graph and replayed.

Also measured (extra fields of the same JSON line): the same stack as a
speculative-verify pass at M = 2, 4, 8, 16 and 48 (t(M)/t(1)), per-kernel
durations from HIP events, the single Q8_0 GEMV, the 0.6B-shaped Q4_0 stack
and the Q4_0 MoE layer, a read-only streaming ceiling at the sizes of the
step's matrices, and the CPU oracle (median of 3 after a warm-up) on a bounded
sample of every configuration on the host cores, which also checks the GPU's
outputs of that sample against the oracle at run time.

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu-baseline]
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time
from concurrent.futures import ThreadPoolExecutor

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, published
GROUP_NAMES = ("qkv", "o", "gate_up", "down")

# HBM bytes per launch of the M = 1 GEMV kernels, from two counter passes
# (FETCH_SIZE, then WRITE_SIZE, rocprofv3 --pmc over `bench.py --kernels-only`),
# scaled by what the same counters read for a plain 256 MiB copy (FETCH x 2.0,
# WRITE x 1.0). They hold only for the kernel sources and build flags they were
# taken with: a changed file (sha256 prefix below, paths under the package)
# reports traffic as unknown.
MEASURED_TRAFFIC = {
    "sources": {"csrc/kq_gemv.hip": "aa4a3ae7e7ae15b4", "csrc/kq_dev.h": "46ae285997c1b786",
                "build.py": "f8d9dfd3b4ceed6e"},
    "bytes": {"qkv": 9962552, "o": 6682647, "gate_up": 31326986, "down": 15815734, "lm_head": 414309826},
}


MFMA_PEAK_F16_TFLOPS = 2500.0   # MI355X dense fp16 matrix-core peak, published

# MFMA busy (SQ_VALU_MFMA_BUSY_CYCLES / (GRBM_GUI_ACTIVE * SIMDs), percent) per
# launch group of the verify pass, from a counter run over `bench.py
# --kernels-only M`; valid only for the kernel sources it was taken with.
MEASURED_MFMA = {"sources": {"csrc/kq_mfma.hip": "73969f11f64ff80a", "csrc/kq_dev.h": "46ae285997c1b786", "build.py": "f8d9dfd3b4ceed6e"},
                 "verify_m8": {"qkv": 2.76, "o": 1.83, "gate_up": 6.66, "down": 3.77, "lm_head": 7.76}}


def measured_mfma(run, group):
    pkg = os.path.join(ROOT, "block_quantized_gemv_kq_amd")
    if not MEASURED_MFMA["sources"]:
        return None
    for name, want in MEASURED_MFMA["sources"].items():
        with open(os.path.join(pkg, name), "rb") as f:
            if hashlib.sha256(f.read()).hexdigest()[:16] != want:
                return None
    return MEASURED_MFMA.get(run, {}).get(group)


def measured_traffic(group):
    pkg = os.path.join(ROOT, "block_quantized_gemv_kq_amd")
    for name, want in MEASURED_TRAFFIC["sources"].items():
        with open(os.path.join(pkg, name), "rb") as f:
            if hashlib.sha256(f.read()).hexdigest()[:16] != want:
                return None
    return MEASURED_TRAFFIC["bytes"].get(group)


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


class DeviceStack:
    """Packed weights of the stack resident in HBM, activations and outputs."""

    def __init__(self, torch, kq, S, stack, M, act_workload_id=None, layers=None):
        self.torch, self.kq = torch, kq
        self.stack = stack
        self.M = M
        self.layers = stack.layers if layers is None else layers
        dev = torch.device("cuda")
        self.groups = []          # per layer: list of (fmt, W_dev, x_dev, y_dev, N, K, name)
        self.weight_bytes = 0
        self.alg_bytes = 0
        wid = stack.workload_id if act_workload_id is None else act_workload_id

        def build_group(layer, gi, group):
            mats = [stack.per_layer[i] for i in group]
            K = mats[0].k
            fmt = mats[0].fmt
            N = sum(m.n for m in mats)
            packed = np.empty((N, kq.kq_packed_bytes(fmt, 1, K)), np.uint8)
            r0 = 0
            for i, m in zip(group, mats):
                W = S.weights(stack.weight_seed(layer, i), m.n, m.k)
                kq.kq_pack(fmt, W, out=packed[r0:r0 + m.n])
                r0 += m.n
            x = S.activations((wid, layer, mats[0].input_slot), K, M)
            digest = hashlib.sha256(packed).digest() + hashlib.sha256(x).digest()
            return layer, gi, fmt, packed, x, N, K, digest

        jobs = [(l, gi, g) for l in range(self.layers) for gi, g in enumerate(stack.launch_groups)]
        per_layer = [[None] * len(stack.launch_groups) for _ in range(self.layers)]
        digests = {}
        with ThreadPoolExecutor(4) as ex:
            for layer, gi, fmt, packed, x, N, K, digest in ex.map(lambda j: build_group(*j), jobs):
                digests[(layer, gi)] = digest
                Wd = torch.from_numpy(packed).to(dev)
                xd = torch.from_numpy(x).to(dev)
                yd = torch.empty((M, N), dtype=torch.float32, device=dev)
                per_layer[layer][gi] = (fmt, Wd, xd, yd, N, K, GROUP_NAMES[gi])
                self.weight_bytes += packed.nbytes
                self.alg_bytes += packed.nbytes + x.nbytes + M * N * 4
        self.groups = per_layer
        h = stack.head
        self.head = None
        if h is not None:
            W = S.weights(stack.weight_seed(stack.layers, 0), h.n, h.k)
            packed = kq.kq_pack(h.fmt, W)
            del W
            x = S.activations((wid, stack.layers, 0), h.k, M)
            Wd = torch.from_numpy(packed).to(dev)
            yd = torch.empty((M, h.n), dtype=torch.float32, device=dev)
            wsb = max(kq.kq_argmax_workspace_bytes(h.n, M), kq.kq_gemv_argmax_workspace_bytes(h.fmt, h.n, h.k, M))
            ws = torch.empty(wsb, dtype=torch.uint8, device=dev)
            am = torch.empty(M, dtype=torch.int32, device=dev)
            self.head = (h.fmt, Wd, torch.from_numpy(x).to(dev), yd, h.n, h.k, ws, wsb, am)
            self.weight_bytes += packed.nbytes
            self.alg_bytes += packed.nbytes + x.nbytes + M * h.n * 4 + M * h.n * 4 + M * 4
            digests[(self.layers, 0)] = hashlib.sha256(packed).digest() + hashlib.sha256(x).digest()
        # SHA-256 over every launch's packed weights and activations, in step order
        self.input_sha256 = hashlib.sha256(b"".join(digests[k] for k in sorted(digests))).hexdigest()
        self._split_workspace()

    def _split_workspace(self):
        """One workspace for the launch groups that kq_gemv_ws splits along K
        (their launches run one after another on one stream, so they share it)."""
        self.split_bytes = {gi: self.kq.kq_gemv_workspace_bytes(fmt, N, K, self.M)
                            for gi, (fmt, _, _, _, N, K, _) in enumerate(self.groups[0])} if self.groups else {}
        need = max(self.split_bytes.values(), default=0)
        self.split_ws = self.torch.empty(need, dtype=self.torch.uint8, device="cuda") if need else None

    def with_columns(self, S, M, act_workload_id):
        """A view with the same resident weights and M fresh activation columns."""
        torch = self.torch
        v = object.__new__(DeviceStack)
        v.torch, v.kq, v.stack, v.M, v.layers = torch, self.kq, self.stack, M, self.layers
        v.weight_bytes, v.alg_bytes = self.weight_bytes, 0
        v.groups = []
        for layer, row in enumerate(self.groups):
            new_row = []
            for gi, (fmt, Wd, _, _, N, K, name) in enumerate(row):
                slot = self.stack.per_layer[self.stack.launch_groups[gi][0]].input_slot
                x = S.activations((act_workload_id, layer, slot), K, M)
                xd = torch.from_numpy(x).to("cuda")
                yd = torch.empty((M, N), dtype=torch.float32, device="cuda")
                new_row.append((fmt, Wd, xd, yd, N, K, name))
                v.alg_bytes += Wd.numel() + x.nbytes + M * N * 4
            v.groups.append(new_row)
        v.head = None
        if self.head is not None:
            fmt, Wd, _, _, N, K, _, _, _ = self.head
            x = S.activations((act_workload_id, self.stack.layers, 0), K, M)
            yd = torch.empty((M, N), dtype=torch.float32, device="cuda")
            wsb = max(self.kq.kq_argmax_workspace_bytes(N, M), self.kq.kq_gemv_argmax_workspace_bytes(fmt, N, K, M))
            ws = torch.empty(wsb, dtype=torch.uint8, device="cuda")
            am = torch.empty(M, dtype=torch.int32, device="cuda")
            v.head = (fmt, Wd, torch.from_numpy(x).to("cuda"), yd, N, K, ws, wsb, am)
            v.alg_bytes += Wd.numel() + x.nbytes + 2 * M * N * 4 + M * 4
        v._split_workspace()
        return v

    invariant = False   # kq_gemv_invariant (per-column bits of one-column calls) instead of kq_gemv

    def _gemv(self):
        return self.kq.kq_gemv_invariant if self.invariant else self.kq.kq_gemv

    def launch_group(self, layer, gi):
        fmt, Wd, xd, yd, N, K, _ = self.groups[layer][gi]
        if not self.invariant and self.split_bytes.get(gi):
            self.kq.kq_gemv_ws(fmt, Wd, xd, yd, N, K, self.M, self.split_ws, self.split_bytes[gi])
        else:
            self._gemv()(fmt, Wd, xd, yd, N, K, self.M)

    def launch_head(self):
        fmt, Wd, xd, yd, N, K, ws, wsb, am = self.head
        if self.invariant:
            self.kq.kq_gemv_invariant(fmt, Wd, xd, yd, N, K, self.M)
            self.kq.kq_argmax(yd, N, self.M, am, ws, wsb)
        else:
            self.kq.kq_gemv_argmax(fmt, Wd, xd, yd, N, K, self.M, am, ws, wsb)

    def step(self):
        """One token as separate launches: 4 GEMVs per layer, lm_head, argmax."""
        for layer in range(self.layers):
            for gi in range(len(self.groups[layer])):
                self.launch_group(layer, gi)
        if self.head is not None:
            self.launch_head()

    def make_plan(self):
        """The whole token as one persistent-kernel plan (kq_stack_plan), in
        decode order: every stage reads its activations from the previous
        stage's fp16 output (the first K values of it: q of q|k|v feeds o,
        gate of gate|up feeds down, the last down feeds the next layer and
        finally the lm_head), so each stage waits for the one before it, as in
        a real decode step. The workload has no norm, attention or SwiGLU
        between the GEMVs, so the chained values are not the workload's
        activations and grow past fp16 range after about ten layers; the
        timing does not depend on them. M = 1."""
        torch, kq = self.torch, self.kq
        stages = []
        prev16 = None
        for row in self.groups:
            for fmt, Wd, xd, yd, N, K, _ in row:
                y16 = torch.empty(N, dtype=torch.float16, device="cuda")
                x = xd if prev16 is None else prev16[:K]
                stages.append(dict(fmt=fmt, W=Wd, x=x, y=yd, N=N, K=K, y16=y16))
                prev16 = y16
        if self.head is not None:
            fmt, Wd, xd, yd, N, K, *_ = self.head
            stages.append(dict(fmt=fmt, W=Wd, x=prev16[:K], y=yd, N=N, K=K))
        nb = kq.kq_stack_plan_bytes(stages)
        self.plan = torch.zeros(nb, dtype=torch.uint8, device="cuda")
        self.info = kq.kq_stack_plan(stages, self.plan, nb)
        self.stack_stages = stages
        self.n_stages = len(stages)

    def step_stacked(self):
        """One token in decode order: every GEMV of every layer and the lm_head
        in one persistent launch, then the argmax."""
        self.kq.kq_stack_run(self.plan, self.info)
        if self.head is not None:
            _, _, _, yd, N, _, ws, wsb, am = self.head
            self.kq.kq_argmax(yd, N, self.M, am, ws, wsb)


def capture(torch, fn):
    """Capture fn's launches (on torch's capture stream) as one graph."""
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        fn()                                   # warm (first-launch setup outside capture)
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        fn()
    torch.cuda.synchronize()
    return g


def time_graph(torch, g, reps, warmup):
    """Per-replay times (ms) from events around each replay, plus the total
    wall time of the `reps` timed replays bracketed by synchronisations."""
    for _ in range(warmup):
        g.replay()
    torch.cuda.synchronize()
    evs = [torch.cuda.Event(enable_timing=True) for _ in range(reps + 1)]
    t0 = time.perf_counter()
    evs[0].record()
    for i in range(reps):
        g.replay()
        evs[i + 1].record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    per = np.array([evs[i].elapsed_time(evs[i + 1]) for i in range(reps)])
    total_ms = evs[0].elapsed_time(evs[reps])
    return per, total_ms, wall


def _graph_us(torch, fns, reps):
    """Average duration (us) of one launch: the launches `fns` captured as one
    graph, the replay bracketed by HIP events on the capture stream, median
    over `reps` replays, divided by the number of launches. Back-to-back
    launches of one kernel in a graph: this is the kernel's duration plus the
    dispatch gap between dependent kernels."""
    g = capture(torch, lambda: [f() for f in fns])
    per, _, _ = time_graph(torch, g, reps, 2)
    del g
    return float(np.median(per)) * 1000.0 / len(fns)


def kernel_table(torch, ds, reps=10):
    """Per launch group: bytes per launch (packed weights + x + y) and the
    average duration of one launch (_graph_us over that group's launches of
    all layers; the lm_head and argmax 8 times each)."""
    out = {}
    for gi, name in enumerate(GROUP_NAMES):
        fns = [lambda l=l, gi=gi: ds.launch_group(l, gi) for l in range(ds.layers)]
        us = _graph_us(torch, fns, reps)
        fmt, Wd, xd, yd, N, K, _ = ds.groups[0][gi]
        nbytes = Wd.numel() + xd.numel() * 2 + yd.numel() * 4
        out[name] = {"N": N, "K": K, "fmt": fmt, "M": ds.M, "launches_per_step": ds.layers,
                     "us_per_launch": us, "bytes_per_launch": int(nbytes),
                     "gbps": nbytes / (us * 1e-6) / 1e9}
        if not ds.invariant and ds.split_bytes.get(gi):
            out[name]["entry"] = "kq_gemv_ws"
            out[name]["k_splits"] = ds.split_bytes[gi] // (4 * ds.M * N)
    if ds.head is not None:
        fmt, Wd, xd, yd, N, K, ws, wsb, am = ds.head
        head = lambda: ds.kq.kq_gemv(fmt, Wd, xd, yd, N, K, ds.M)
        us = _graph_us(torch, [head] * 8, reps)
        nbytes = Wd.numel() + xd.numel() * 2 + yd.numel() * 4
        out["lm_head"] = {"N": N, "K": K, "fmt": fmt, "M": ds.M, "launches_per_step": 1,
                          "us_per_launch": us, "bytes_per_launch": int(nbytes),
                          "gbps": nbytes / (us * 1e-6) / 1e9}
        fused = lambda: ds.kq.kq_gemv_argmax(fmt, Wd, xd, yd, N, K, ds.M, am, ws, wsb)
        us_f = _graph_us(torch, [fused] * 8, reps)
        out["lm_head_argmax"] = {"entry": "kq_gemv_argmax", "us_per_call": us_f,
                                 "kernels_per_call": 2 if ds.M == 1 else 3}
        am_fn = lambda: ds.kq.kq_argmax(yd, N, ds.M, am, ws, wsb)
        us = _graph_us(torch, [am_fn] * 8, reps)
        out["argmax"] = {"N": N, "kernels_per_call": 2, "us_per_call": us,
                         "bytes_per_call": int(yd.numel() * 4)}
    return out


def shortlist_head(torch, ds, steps, warmup):
    """The lm_head's argmax through kq_shortlist_argmax (M = 1): the bound copy
    packed on the host from the head's Q8_0 bytes, the call timed alone (a
    graph of 8 calls, as the kernel table) and as the step's last call in
    place of kq_gemv_argmax (the layer launches unchanged, the step captured
    and replayed like the headline's), the rows it scored exactly, and whether
    its index is kq_gemv_argmax's. Bytes read per call: the bound copy, the
    kept rows' Q8_0 bytes, x three times, u written and read."""
    kq = ds.kq
    fmt, Wd, xd, yd, N, K, ws, wsb, am = ds.head
    packed = Wd.cpu().numpy()
    t0 = time.perf_counter()
    copy = kq.kq_shortlist_pack(packed, N, K)
    pack_s = time.perf_counter() - t0
    del packed
    Cd = torch.from_numpy(copy).to("cuda")
    swsb = kq.kq_shortlist_workspace_bytes(N, K)
    sws = torch.empty(swsb, dtype=torch.uint8, device="cuda")
    out = torch.empty(1, dtype=torch.int32, device="cuda")
    kept = torch.empty(1, dtype=torch.int32, device="cuda")
    call = lambda: kq.kq_shortlist_argmax(Wd, Cd, xd, N, K, sws, swsb, out, kept)
    us = _graph_us(torch, [call] * 8, 10)
    call()
    ds.launch_head()
    torch.cuda.synchronize()
    idx, ref, nkept = int(out.cpu()[0]), int(am.cpu()[0]), int(kept.cpu()[0])

    def step():
        for layer in range(ds.layers):
            for gi in range(len(ds.groups[layer])):
                ds.launch_group(layer, gi)
        call()
    g = capture(torch, step)
    per, total, _ = time_graph(torch, g, steps, warmup)
    del g
    ms = total / steps
    nbytes = copy.nbytes + nkept * (K // 32) * 34 + 3 * 2 * K + 2 * 4 * N
    del Cd, sws
    return {"entry": "kq_shortlist_argmax", "us_per_call": us, "kernels_per_call": 4,
            "rows": N, "rows_scored_exactly": nkept, "pct_rows_scored_exactly": 100.0 * nkept / N,
            "bound_copy_bytes": int(copy.nbytes), "bytes_read_per_call": int(nbytes),
            "gbps_of_bytes_read": nbytes / (us * 1e-6) / 1e9,
            "index": idx, "index_equals_kq_gemv_argmax": idx == ref, "host_pack_s": pack_s,
            "step_ms_with_shortlist": ms, "tokens_per_s_with_shortlist": 1000.0 / ms,
            "step_us_p10_p50_p90": [float(np.percentile(per, q)) * 1000 for q in (10, 50, 90)]}


def bench_shortlist_head(torch, kq, S, copies=3, reps=10):
    """The 4B-shaped Q8_0 head alone (151936 x 2560, M = 1): kq_shortlist_argmax
    against kq_gemv_argmax, each as a graph of 9 calls rotating over `copies`
    copies of the weights (and of the bound copy), so every call reads from
    HBM; per call: median over `reps` replays / 9. Also the rows kept for the
    bench's seeded column and the index of both calls."""
    h = S.QWEN3_4B_AFFINE4.head
    W = S.weights(S.QWEN3_4B_AFFINE4.weight_seed(S.QWEN3_4B_AFFINE4.layers, 0), h.n, h.k)
    packed = kq.kq_pack(h.fmt, W)
    del W
    copy = kq.kq_shortlist_pack(packed, h.n, h.k)
    N, K = h.n, h.k
    Ws = [torch.from_numpy(packed).cuda() for _ in range(copies)]
    Cs = [torch.from_numpy(copy).cuda() for _ in range(copies)]
    x = torch.from_numpy(S.activations((S.QWEN3_4B_AFFINE4.workload_id, S.QWEN3_4B_AFFINE4.layers, 0), K, 1)).cuda()
    swsb = kq.kq_shortlist_workspace_bytes(N, K)
    sws = torch.empty(swsb, dtype=torch.uint8, device="cuda")
    awsb = kq.kq_gemv_argmax_workspace_bytes(h.fmt, N, K, 1)
    aws = torch.empty(awsb, dtype=torch.uint8, device="cuda")
    y = torch.empty((1, N), dtype=torch.float32, device="cuda")
    out = torch.zeros(2, dtype=torch.int32, device="cuda")
    kept = torch.zeros(1, dtype=torch.int32, device="cuda")
    sl = [lambda i=i: kq.kq_shortlist_argmax(Ws[i % copies], Cs[i % copies], x, N, K, sws, swsb, out[0:1], kept)
          for i in range(9)]
    ga = [lambda i=i: kq.kq_gemv_argmax(h.fmt, Ws[i % copies], x, y, N, K, 1, out[1:2], aws, awsb)
          for i in range(9)]
    us_sl = _graph_us(torch, sl, reps)
    us_ga = _graph_us(torch, ga, reps)
    o = out.cpu().numpy()
    return {"rows": N, "K": K, "us_per_call_shortlist": us_sl, "us_per_call_gemv_argmax": us_ga,
            "rows_scored_exactly": int(kept.cpu()[0]), "index_shortlist": int(o[0]), "index_gemv_argmax": int(o[1]),
            "bound_copy_bytes": int(copy.nbytes), "copies": copies}


def _graph_time_us(torch, fns, reps, per):
    """Median over `reps` replays of a graph of `fns`, divided by `per`."""
    g = capture(torch, lambda: [f() for f in fns])
    t, _, _ = time_graph(torch, g, reps, 2)
    del g
    return float(np.median(t)) * 1000.0 / per, [float(np.percentile(t, q)) * 1000.0 / per for q in (10, 50, 90)]


def bench_single_q8_0(torch, kq, S, gpu_out=None):
    """Config 1: one Q8_0 1024x1024 GEMV, M=1 (seeded weights and x). Cold:
    rotating through copies totalling >= 1 GB (four times the 256 MB
    last-level cache); warm: one copy, back to back. Each launch in a graph:
    the time includes the dispatch gap between dependent kernels."""
    c = S.SINGLE_Q8_0
    W = S.weights(c.weight_seed, c.n, c.k)
    packed = torch.from_numpy(kq.kq_pack(c.fmt, W)).to("cuda")
    x = torch.from_numpy(S.activation_column(c.act_seed, c.k)[None, :]).to("cuda")
    y = torch.empty((1, c.n), dtype=torch.float32, device="cuda")
    alg = packed.numel() + x.numel() * 2 + y.numel() * 4
    copies = (1 << 30) // packed.numel() + 1
    Ws = packed.reshape(-1).repeat(copies).view(copies, -1)
    cold, cold_p = _graph_time_us(torch, [lambda i=i: kq.kq_gemv(c.fmt, Ws[i], x, y, c.n, c.k, 1)
                                          for i in range(copies)], 7, copies)
    warm, warm_p = _graph_time_us(torch, [lambda: kq.kq_gemv(c.fmt, packed, x, y, c.n, c.k, 1)] * 200, 7, 200)
    if gpu_out is not None:
        gpu_out["single_y"] = _host(y)
    del Ws
    return {"shape": f"q8_0 {c.n}x{c.k}, M=1", "alg_bytes": int(alg), "cold_copies": int(copies),
            "us_per_call_cold": cold, "gbps_cold": alg / (cold * 1e-6) / 1e9, "us_p10_p50_p90_cold": cold_p,
            "us_per_call_warm": warm, "gbps_warm": alg / (warm * 1e-6) / 1e9}


def bench_small_stack(torch, kq, S, steps):
    """Config 2: the 0.6B-shaped Q4_0 stack (28 layers, q|k|v, o, gate|up,
    down per layer), M=1, in decode order. Its 248 MB fit the 256 MB
    last-level cache, so the cold figure rotates through 4 copies of the
    packed weights (the same bytes at four addresses); warm replays one."""
    st = S.QWEN3_0_6B_Q4_0
    ds = DeviceStack(torch, kq, S, st, 1)
    copies = 4
    banks = [[[Wd.clone() for (_, Wd, *_r) in row] for row in ds.groups] for _ in range(copies - 1)]

    def step_copy(cpy):
        for layer, row in enumerate(ds.groups):
            for gi, (fmt, Wd, xd, yd, N, K, _) in enumerate(row):
                W = Wd if cpy == 0 else banks[cpy - 1][layer][gi]
                kq.kq_gemv(fmt, W, xd, yd, N, K, 1)
    cold, cold_p = _graph_time_us(torch, [lambda c=c: step_copy(c) for c in range(copies)], steps, copies)
    warm, warm_p = _graph_time_us(torch, [lambda: step_copy(0)], steps, 1)
    out = {"workload": f"{st.name}, M=1, one decode token ({st.layers} layers x 4 launches)",
           "alg_bytes_per_step": int(ds.alg_bytes), "weight_bytes": int(ds.weight_bytes),
           "us_per_step_cold": cold, "us_p10_p50_p90_cold": cold_p,
           "gbps_cold": ds.alg_bytes / (cold * 1e-6) / 1e9, "tokens_per_s_cold": 1e6 / cold,
           "us_per_step_warm": warm, "gbps_warm": ds.alg_bytes / (warm * 1e-6) / 1e9,
           "tokens_per_s_warm": 1e6 / warm}
    del banks, ds
    torch.cuda.empty_cache()
    return out


VERIFY_INVARIANT_M = (4, 8, 16, 48)   # verify widths also timed through kq_gemv_invariant


def bench_verify_all(torch, kq, S, ds, t1_ms, steps):
    """Config 4: the verify pass at every M on the resident 4B-shaped
    weights: time per pass, t(M)/t(1), M / t as the upper bound on accepted
    tokens per second."""
    out = {}
    for M in S.VERIFY_M:
        dv = ds.with_columns(S, M, S.VERIFY_WORKLOAD_ID)
        g = capture(torch, dv.step)
        per, total, _ = time_graph(torch, g, steps, 3)
        ms = float(np.median(per))
        out[str(M)] = {"ms_per_pass": ms, "ms_p10_p90": [float(np.percentile(per, 10)), float(np.percentile(per, 90))],
                       "alg_bytes": int(dv.alg_bytes), "gbps": dv.alg_bytes / (ms * 1e-3) / 1e9,
                       "t_ratio_vs_m1": ms / t1_ms, "tokens_per_s_upper_bound": M / (ms * 1e-3),
                       "k_split_groups": {GROUP_NAMES[gi]: b // (4 * M * dv.groups[0][gi][4])
                                          for gi, b in dv.split_bytes.items() if b}}
        log(f"verify M={M}: {ms * 1000:.1f} us per pass, t(M)/t(1) = {ms / t1_ms:.2f}")
        if M in VERIFY_INVARIANT_M:
            dv.invariant = True
            g2 = capture(torch, dv.step)
            per2, _, _ = time_graph(torch, g2, steps, 3)
            ms2 = float(np.median(per2))
            out[str(M)]["invariant"] = {"entry": "kq_gemv_invariant", "ms_per_pass": ms2,
                                        "gbps": dv.alg_bytes / (ms2 * 1e-3) / 1e9, "t_ratio_vs_m1": ms2 / t1_ms,
                                        "ratio_vs_kq_gemv": ms2 / ms,
                                        "tokens_per_s_upper_bound": M / (ms2 * 1e-3)}
            log(f"verify M={M} batch-invariant: {ms2 * 1000:.1f} us per pass, t(M)/t(1) = {ms2 / t1_ms:.2f}")
            del g2
        del g, dv
        torch.cuda.empty_cache()
    # decode (one column) through the batch-invariant entry point: the bits a
    # verify pass through it reproduces
    dv = ds.with_columns(S, 1, S.VERIFY_WORKLOAD_ID)
    dv.invariant = True
    g = capture(torch, dv.step)
    per, _, _ = time_graph(torch, g, steps, 3)
    ms = float(np.median(per))
    out["1_invariant"] = {"entry": "kq_gemv_invariant", "M": 1, "ms_per_pass": ms, "t_ratio_vs_m1": ms / t1_ms,
                          "gbps": dv.alg_bytes / (ms * 1e-3) / 1e9, "tokens_per_s": 1 / (ms * 1e-3)}
    log(f"decode M=1 batch-invariant: {ms * 1000:.1f} us per token, {ms / t1_ms:.2f} x kq_gemv")
    del g, dv
    torch.cuda.empty_cache()
    return out


def bench_moe(torch, kq, S, steps):
    """Config 5: the Q4_0 MoE layer (128 experts, hidden 2048, FFN 768,
    top-8) through kq_moe_ffn at M in {1, 4, 16} tokens, with the workload's
    route tables. One expert's packed gate/up/down (seeded) is replicated to
    all 128 experts (time does not depend on values) and the whole set to 3
    copies (1 GB) that the timed calls rotate through. Algorithmic bytes:
    the unique routed experts' weights, plus activations, h and outputs."""
    L = S.MOE_Q4_0
    E = L.n_experts
    mats = []
    for which, (n, k) in enumerate(((L.inter, L.hidden), (L.inter, L.hidden), (L.hidden, L.inter))):
        W = S.weights(L.weight_seed(0, which), n, k)
        mats.append(torch.from_numpy(kq.kq_pack(L.fmt, W)).to("cuda"))
    per_expert = sum(m.numel() for m in mats)
    copies = 3
    banks = [[m.reshape(-1).repeat(E) for m in mats] for _ in range(copies)]
    out = {}
    for M in S.MOE_M:
        ids, rw = S.route_table(L.workload_id, M, E, L.top_k)
        U = len(np.unique(ids))
        x = torch.from_numpy(S.activations(L.act_seed_prefix(), L.hidden, M)).to("cuda")
        idd = torch.from_numpy(ids).to("cuda")
        rwd = torch.from_numpy(rw).to("cuda")
        y = torch.empty((M, L.hidden), dtype=torch.float32, device="cuda")
        h = torch.empty((M, L.top_k, L.inter), dtype=torch.float16, device="cuda")
        wsb = kq.kq_moe_ffn_workspace_bytes(L.hidden, L.inter, M, L.top_k)
        ws = torch.empty(wsb, dtype=torch.uint8, device="cuda")
        fns = [lambda c=c: kq.kq_moe_ffn(L.fmt, banks[c][0], banks[c][1], banks[c][2], x, idd, rwd, y, h,
                                         L.hidden, L.inter, M, L.top_k, E, ws, wsb) for c in range(copies)]
        us, p = _graph_time_us(torch, fns * 4, steps, 4 * copies)
        alg = U * per_expert + x.numel() * 2 + 2 * h.numel() * 2 + y.numel() * 4
        out[str(M)] = {"unique_experts": int(U), "alg_bytes": int(alg), "us_per_layer": us, "us_p10_p50_p90": p,
                       "gbps": alg / (us * 1e-6) / 1e9, "tokens_per_s_per_layer": M / (us * 1e-6)}
        log(f"moe M={M}: {U} experts, {us:.1f} us per layer, {alg / (us * 1e-6) / 1e9:.0f} GB/s")
    del banks
    torch.cuda.empty_cache()
    return out


def bench_moe_eager(torch, kq, S):
    """The Q4_0 MoE layer at each token count, eager (for counter runs): one
    seeded expert replicated to all 128, each call twice."""
    L = S.MOE_Q4_0
    E = L.n_experts
    mats = []
    for which, (n, k) in enumerate(((L.inter, L.hidden), (L.inter, L.hidden), (L.hidden, L.inter))):
        W = S.weights(L.weight_seed(0, which), n, k)
        mats.append(torch.from_numpy(kq.kq_pack(L.fmt, W)).to("cuda").reshape(-1).repeat(E))
    for M in S.MOE_M:
        ids, rw = S.route_table(L.workload_id, M, E, L.top_k)
        x = torch.from_numpy(S.activations(L.act_seed_prefix(), L.hidden, M)).to("cuda")
        idd, rwd = torch.from_numpy(ids).to("cuda"), torch.from_numpy(rw).to("cuda")
        y = torch.empty((M, L.hidden), dtype=torch.float32, device="cuda")
        h = torch.empty((M, L.top_k, L.inter), dtype=torch.float16, device="cuda")
        wsb = kq.kq_moe_ffn_workspace_bytes(L.hidden, L.inter, M, L.top_k)
        ws = torch.empty(wsb, dtype=torch.uint8, device="cuda")
        torch.cuda.synchronize()
        for _ in range(2):
            kq.kq_moe_ffn(L.fmt, mats[0], mats[1], mats[2], x, idd, rwd, y, h, L.hidden, L.inter, M, L.top_k, E,
                          ws, wsb)
        torch.cuda.synchronize()
    del mats


def bench_formats(torch, kq, S, reps=7):
    """One matrix shape (the 4B stack's gate|up, 19456 x 2560, seeded weights)
    in every block format at M = 1 and M = 8: cold per-launch time (rotating
    through copies totalling >= 1 GB, graph-replayed) and GB/s of its packed
    weights + x + y. Q5_0 / Q5_1 run on the VALU kernels only (8 columns per
    weight pass), the others on the matrix cores from 4 columns."""
    N, K = 19456, 2560
    W = S.weights((6, 0, 0, 0), N, K)
    out = {}
    for fmt in ("q8_0", "q4_0", "affine4", "q5_0", "q5_1"):
        packed = torch.from_numpy(kq.kq_pack(fmt, W)).to("cuda").reshape(-1)
        copies = max(2, (1 << 30) // packed.numel() + 1)
        bank = packed.repeat(copies).view(copies, -1)
        row = {"weight_bytes": int(packed.numel())}
        for M in (1, 8):
            x = torch.from_numpy(S.activations((6, 1), K, M)).to("cuda")
            y = torch.empty((M, N), dtype=torch.float32, device="cuda")
            us, _ = _graph_time_us(torch, [lambda c=c: kq.kq_gemv(fmt, bank[c], x, y, N, K, M)
                                           for c in range(copies)], reps, copies)
            alg = packed.numel() + 2 * M * K + 4 * M * N
            row[f"M{M}"] = {"us_per_launch": us, "gbps": alg / (us * 1e-6) / 1e9}
        out[fmt] = row
        log(f"format {fmt}: M=1 {row['M1']['us_per_launch']:.2f} us ({row['M1']['gbps']:.0f} GB/s), "
            f"M=8 {row['M8']['us_per_launch']:.2f} us")
        del bank, packed
        torch.cuda.empty_cache()
    return {"shape": f"{N}x{K} (gate|up), cold", "formats": out}


def _probe_lib():
    import ctypes
    L = ctypes.CDLL(os.path.join(ROOT, "block_quantized_gemv_kq_amd", "libkq_probe.so"))
    L.kq_probe_stream_read.restype = ctypes.c_int
    L.kq_probe_stream_read.argtypes = [ctypes.c_void_p, ctypes.c_int64, ctypes.c_void_p, ctypes.c_int,
                                       ctypes.c_void_p]
    return L


# bytes per launch of the step's matrices (packed weights) and a large read
# packed bytes of the step's matrices: affine4 rows of K/32 blocks of 20 bytes,
# the Q8_0 output layer 34 bytes per block
CEILING_SIZES = {"o": 2560 * 128 * 20, "qkv": 6144 * 80 * 20, "down": 2560 * 304 * 20, "gate_up": 19456 * 80 * 20,
                 "lm_head": 151936 * 80 * 34, "1GiB": 1 << 30}


def stream_ceiling(torch, reps=7):
    """A measured read-only ceiling: a plain streaming kernel (libkq_probe.so:
    each workgroup reads one contiguous chunk, every lane issuing all its
    16-byte buffer loads before using any, XOR-folded, one word per workgroup
    written) reading buffers of the sizes of the step's matrices, cold (each
    launch reads other bytes of a 1 GiB buffer, four times the last-level
    cache), launched back to back in a graph like the GEMVs; the best of 1, 2,
    4, 8 and 16 loads per lane. Also the plain-read step: the same reads in the
    order and number of the M = 1 step's launches."""
    L = _probe_lib()
    buf = torch.empty(1 << 30, dtype=torch.uint8, device="cuda")
    buf.fill_(7)
    sink = torch.empty(1 << 20, dtype=torch.int32, device="cuda")
    base = buf.data_ptr()
    out = {}
    for name, nbytes in CEILING_SIZES.items():
        span = (nbytes + 4095) // 4096 * 4096
        copies = max(1, (1 << 30) // span)
        best = None
        for per in (1, 2, 4, 8, 16):
            def launches(per=per):
                s_ = torch.cuda.current_stream().cuda_stream
                for c in range(copies):
                    st = L.kq_probe_stream_read(base + c * span, nbytes, sink.data_ptr(), per, s_)
                    if st < 0:
                        raise RuntimeError(f"kq_probe_stream_read failed ({st})")
            us, _ = _graph_time_us(torch, [launches], reps, copies)
            if best is None or us < best[0]:
                best = (us, per)
        out[name] = {"bytes": nbytes, "us_per_launch": best[0], "gbps": nbytes / (best[0] * 1e-6) / 1e9,
                     "loads_per_lane": best[1], "workgroups": -(-nbytes // (4096 * best[1])),
                     "cold_copies": copies}
    step_us = 36 * sum(out[k]["us_per_launch"] for k in ("qkv", "o", "gate_up", "down")) + out["lm_head"]["us_per_launch"]
    del buf, sink
    torch.cuda.empty_cache()
    return {"kernel": "read-only streaming (libkq_probe.so), one launch per buffer, cold, graph-timed",
            "sizes": out, "plain_read_step_us": step_us,
            "plain_read_step_gbps": (36 * sum(CEILING_SIZES[k] for k in ("qkv", "o", "gate_up", "down"))
                                     + CEILING_SIZES["lm_head"]) / (step_us * 1e-6) / 1e9}


def _median_timed(fn, reps=3):
    """One warm-up, then the median of `reps` timed runs; returns (median s,
    all times, the last result)."""
    fn()
    ts, out = [], None
    for _ in range(reps):
        t0 = time.perf_counter()
        out = fn()
        ts.append(time.perf_counter() - t0)
    return float(np.median(ts)), ts, out


def _blas_threads():
    try:
        from threadpoolctl import threadpool_info
        return max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:
        return int(os.environ.get("OMP_NUM_THREADS", os.cpu_count() or 1))


def _parity(y_gpu, y_ref, abs_dot):
    """Max error ratio, whether every output is within the bar, and for
    vocabulary-sized outputs the argmax of both sides and the oracle's top-2
    gap per column."""
    from oracle import ref as R
    y_gpu = np.asarray(y_gpu, np.float64).reshape(y_ref.shape)
    return {"max_err_ratio": R.error_ratio(y_gpu, y_ref, abs_dot),
            "within_tolerance": bool(np.all(R.within_tolerance(y_gpu, y_ref, abs_dot)))}


def _argmax_parity(y_gpu, y_ref, am_gpu):
    from oracle import ref as R
    y_gpu = np.asarray(y_gpu, np.float64).reshape(y_ref.shape)
    ref = np.atleast_1d(R.argmax_lowest(y_ref))
    gap = np.atleast_1d(R.top2_gap(y_ref))
    err = np.max(np.abs(y_gpu - y_ref), axis=-1).reshape(-1)
    return {"argmax_gpu": [int(v) for v in np.atleast_1d(am_gpu)], "argmax_ref": [int(v) for v in ref],
            "argmax_equal": bool(np.array_equal(np.atleast_1d(am_gpu), ref)),
            "top2_gap_min": float(gap.min()), "max_abs_err": float(err.max()),
            "pinned": bool(np.all(gap > 4 * err))}


def cpu_baseline(S, stack, kq, gpu_out, budget_layers=2):
    """The oracle as it stands (decode packed bytes, dequantize, fp64 dot) on
    the host cores: for the headline workload, `budget_layers` layers and the
    lm_head with its argmax at M = 1, each timed as the median of 3 runs after
    one warm-up, extrapolated to one token; unit GB/s of packed weights. The
    same oracle results check the GPU's outputs of that sample (gpu_out:
    the M = 1 step's y of those layers' launches and of the lm_head, and the
    argmax) at run time."""
    from oracle import formats as F
    from oracle import ref as R
    units = []
    for layer in range(budget_layers):
        for gi, group in enumerate(stack.launch_groups):
            mats = [stack.per_layer[i] for i in group]
            K, fmt = mats[0].k, mats[0].fmt
            N = sum(m.n for m in mats)
            packed = np.concatenate([kq.kq_pack(fmt, S.weights(stack.weight_seed(layer, i), m.n, m.k))
                                     for i, m in zip(group, mats)])
            x = S.activations((stack.workload_id, layer, mats[0].input_slot), K, 1)
            units.append((layer, gi, fmt, packed, x, N, K))
    h = stack.head
    W = S.weights(stack.weight_seed(stack.layers, 0), h.n, h.k)
    head_packed = kq.kq_pack(h.fmt, W)
    del W
    head_x = S.activations((stack.workload_id, stack.layers, 0), h.k, 1)
    t_layers, ts_l, res = _median_timed(
        lambda: [R.gemv(f, F.decode(f, p, n, k), x) for (_, _, f, p, x, n, k) in units])
    t_head, ts_h, (yh, ah) = _median_timed(
        lambda: R.gemv(h.fmt, F.decode(h.fmt, head_packed, h.n, h.k), head_x))
    R.argmax_lowest(yh[0])
    t_token = t_layers / budget_layers * stack.layers + t_head
    layer_bytes = sum(u[3].nbytes for u in units) / budget_layers
    total_bytes = layer_bytes * stack.layers + head_packed.nbytes
    parity = None
    if gpu_out is not None:
        ratios, ok = [], True
        for (layer, gi, *_), (yr, ad) in zip(units, res):
            p = _parity(gpu_out["layers"][(layer, gi)], yr, ad)
            ratios.append(p["max_err_ratio"])
            ok = ok and p["within_tolerance"]
        ph = _parity(gpu_out["head_y"], yh, ah)
        parity = {"sample": f"{len(units)} launches of layers 0..{budget_layers - 1} and the lm_head, M=1",
                  "max_err_ratio": max(ratios + [ph["max_err_ratio"]]),
                  "within_tolerance": bool(ok and ph["within_tolerance"]),
                  "lm_head": _argmax_parity(gpu_out["head_y"], yh, gpu_out["head_argmax"])}
    return {"value": total_bytes / t_token / 1e9, "unit": "GB/s", "cores": int(_blas_threads()),
            "kind": "oracle",
            "sample": f"{budget_layers} of {stack.layers} layers (as the step's launch groups) + lm_head + "
                      f"argmax at M=1, median of 3 after a warm-up ({t_layers + t_head:.1f} s per sample), "
                      f"extrapolated to one token",
            "s_per_token": t_token, "tokens_per_s": 1.0 / t_token,
            "runs_s": {"layers": ts_l, "lm_head": ts_h},
            "host_cpu_count": os.cpu_count(), "parity": parity}


def oracle_other_configs(S, kq, gpu_out):
    """The oracle on a bounded sample of every other configuration, median of
    3 after a warm-up, with the GPU's outputs checked where the run kept
    them: the single Q8_0 GEMV (whole), the 0.6B stack (2 of 28 layers,
    extrapolated), the verify pass at M = 8 (its lm_head, whose argmax per
    column is compared), and the MoE layer at M = 1 and 4 (whole layer)."""
    from oracle import formats as F
    from oracle import ref as R
    out = {}
    c = S.SINGLE_Q8_0
    packed = kq.kq_pack(c.fmt, S.weights(c.weight_seed, c.n, c.k))
    x = S.activation_column(c.act_seed, c.k)[None, :]
    t, _, (yr, ad) = _median_timed(lambda: R.gemv(c.fmt, F.decode(c.fmt, packed, c.n, c.k), x))
    out["single_q8_0"] = {"s_per_call": t, "gbps": packed.nbytes / t / 1e9}
    if gpu_out and "single_y" in gpu_out:
        out["single_q8_0"]["parity"] = _parity(gpu_out["single_y"], yr, ad)
    st = S.QWEN3_0_6B_Q4_0
    units = []
    for layer in range(2):
        for m_i, m in enumerate(st.per_layer):
            units.append((m.fmt, kq.kq_pack(m.fmt, S.weights(st.weight_seed(layer, m_i), m.n, m.k)),
                          S.activations(st.act_seed_prefix(layer, m.input_slot), m.k, 1), m.n, m.k))
    t, _, _ = _median_timed(lambda: [R.gemv(f, F.decode(f, p, n, k), x) for (f, p, x, n, k) in units])
    tok = t / 2 * st.layers
    out["qwen3_0.6b_q4_0_stack"] = {"s_per_token": tok, "tokens_per_s": 1 / tok,
                                    "gbps": sum(u[1].nbytes for u in units) / 2 * st.layers / tok / 1e9,
                                    "sample": "2 of 28 layers, extrapolated"}
    if gpu_out and "verify8_head_y" in gpu_out:
        h = S.QWEN3_4B_AFFINE4.head
        hp = kq.kq_pack(h.fmt, S.weights(S.QWEN3_4B_AFFINE4.weight_seed(S.QWEN3_4B_AFFINE4.layers, 0), h.n, h.k))
        xv = S.activations((S.VERIFY_WORKLOAD_ID, S.QWEN3_4B_AFFINE4.layers, 0), h.k, 8)
        t, _, (yr, ad) = _median_timed(lambda: R.gemv(h.fmt, F.decode(h.fmt, hp, h.n, h.k), xv))
        out["verify_m8_lm_head"] = {"s_per_pass_head_only": t, "gbps": hp.nbytes / t / 1e9,
                                    "parity": {**_parity(gpu_out["verify8_head_y"], yr, ad),
                                               **_argmax_parity(gpu_out["verify8_head_y"], yr,
                                                                gpu_out["verify8_head_argmax"])}}
        del hp
    L = S.MOE_Q4_0
    for M in (1, 4):
        ids, rw = S.route_table(L.workload_id, M, L.n_experts, L.top_k)
        used = sorted(set(ids.reshape(-1).tolist()))
        packs = {}
        for e in used:
            packs[e] = [kq.kq_pack(L.fmt, S.weights(L.weight_seed(e, w), n, k))
                        for w, (n, k) in enumerate(((L.inter, L.hidden), (L.inter, L.hidden), (L.hidden, L.inter)))]
        x = S.activations(L.act_seed_prefix(), L.hidden, M)

        def run():
            fl = [[None] * L.n_experts for _ in range(3)]
            for e in used:
                for w, (n, k) in enumerate(((L.inter, L.hidden), (L.inter, L.hidden), (L.hidden, L.inter))):
                    fl[w][e] = F.decode(L.fmt, packs[e][w], n, k)
            return R.moe_ffn(L.fmt, fl[0], fl[1], fl[2], x, ids, rw)
        t, _, _ = _median_timed(run)
        out[f"moe_q4_0_m{M}"] = {"s_per_layer": t, "unique_experts": len(used),
                                 "gbps": len(used) * 2654208 / t / 1e9}
    return out


def env_info(torch):
    """GPU, ROCm, torch and numpy versions, and the clocks rocm-smi reports."""
    import subprocess
    props = torch.cuda.get_device_properties(0)
    info = {"gpu": f"{torch.cuda.get_device_name(0)} ({getattr(props, 'gcnArchName', '?')}, "
                   f"{props.multi_processor_count} CUs)",
            "torch": torch.__version__, "numpy": np.__version__}
    try:
        with open("/opt/rocm/.info/version") as f:
            info["rocm"] = f.read().strip()
    except OSError:
        info["rocm"] = None
    try:
        p = subprocess.run(["rocm-smi", "--showclocks"], capture_output=True, text=True, timeout=20)
        info["clocks"] = [ln.split(":", 1)[1].strip() for ln in p.stdout.splitlines()
                          if "clock level" in ln][:4]
    except Exception:
        info["clocks"] = None
    return info


def _copy_calibration(torch):
    """A plain copy of known size (256 MiB read, 256 MiB written), three times,
    to scale the traffic counters against."""
    n = 256 << 20
    a = torch.empty(n // 4, dtype=torch.float32, device="cuda").fill_(1.0)
    b = torch.empty_like(a)
    for _ in range(3):
        b.copy_(a)
    torch.cuda.synchronize()
    return n


def _host(t):
    return t.detach().cpu().numpy()


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-verify", action="store_true", help="skip the verify measurements (M > 1)")
    ap.add_argument("--no-configs", action="store_true",
                    help="skip the other configurations (single Q8_0 GEMV, 0.6B stack, MoE layer)")
    ap.add_argument("--verify-only", type=int, default=0, metavar="M",
                    help="short run for kernel traces: only the M-column verify pass, graph-replayed")
    ap.add_argument("--kernels-only", type=int, nargs="?", const=1, default=0, metavar="M",
                    help="short run for counter collection: eager launches of 4 layers and the lm_head at M "
                         "columns (default 1), then a copy of known size")
    ap.add_argument("--shortlist-only", action="store_true",
                    help="only the Q8_0 head's argmax: kq_shortlist_argmax against kq_gemv_argmax")
    ap.add_argument("--moe-only", action="store_true",
                    help="short run: only the Q4_0 MoE layer at each token count")
    ap.add_argument("--eager", action="store_true",
                    help="with --moe-only: eager launches (for counter collection) instead of graphs")
    args = ap.parse_args()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(json.dumps({"error": "this build runs on one GPU only: the decode GEMV is measured on "
                          "one MI355X; see the sharding notes in DESIGN.md", "n_gpus": args.gpus}))
        sys.exit(2)

    import torch
    import block_quantized_gemv_kq_amd as kq
    from synth import inputs as S
    assert torch.cuda.is_available(), "bench.py needs a GPU"
    kq.lib()
    stack = S.QWEN3_4B_AFFINE4

    if args.shortlist_only:
        print(json.dumps({"shortlist_only": bench_shortlist_head(torch, kq, S, reps=max(5, args.steps))}))
        return
    if args.moe_only:
        if args.eager:
            bench_moe_eager(torch, kq, S)
            n = _copy_calibration(torch)
            print(json.dumps({"moe_only_eager": list(S.MOE_M), "copy_bytes_each_way": n}))
            return
        moe = bench_moe(torch, kq, S, args.steps)
        print(json.dumps({"moe_only": {m: round(v["us_per_layer"], 3) for m, v in moe.items()}}))
        return

    if args.kernels_only:
        # eager launches only (no graphs), for counter collection: each group
        # of the first 4 layers and the lm_head (with its argmax) twice at M
        # columns, then a plain copy of known size to calibrate the counters
        ds = DeviceStack(torch, kq, S, stack, 1, layers=4)
        if args.kernels_only > 1:
            ds = ds.with_columns(S, args.kernels_only, S.VERIFY_WORKLOAD_ID)
        torch.cuda.synchronize()
        for layer in range(4):
            for gi in range(len(GROUP_NAMES)):
                ds.launch_group(layer, gi)
        for _ in range(2):
            ds.launch_head()
        torch.cuda.synchronize()
        n = _copy_calibration(torch)
        print(json.dumps({"kernels_only_M": args.kernels_only, "copy_bytes_each_way": n}))
        return

    t0 = time.perf_counter()
    log("packing and uploading the 4B-shaped stack (M=1) ...")
    ds = DeviceStack(torch, kq, S, stack, 1)
    log(f"  {ds.weight_bytes / 1e9:.3f} GB of packed weights resident in {time.perf_counter() - t0:.1f} s")

    if args.verify_only:
        # the M-column verify pass alone (same resident weights, seeded
        # columns), replayed as a graph: the kernels of one verify width
        dv = ds.with_columns(S, args.verify_only, S.VERIFY_WORKLOAD_ID)
        g = capture(torch, dv.step)
        per, total, _ = time_graph(torch, g, args.steps, args.warmup)
        print(json.dumps({"verify_only": args.verify_only, "ms_per_pass": float(np.median(per)),
                          "steps": args.steps}))
        return

    # path A: every GEMV its own kernel, the step replayed as a graph
    g = capture(torch, ds.step)
    per_l, total_l, _ = time_graph(torch, g, args.steps, args.warmup)
    ms_launches = total_l / args.steps
    log(f"M=1 step as {ds.layers * 4 + 3} launches: {ms_launches * 1000:.1f} us")
    del g
    # the GPU's outputs of the last replay that the oracle checks at the end
    gpu_out = {"layers": {(l, gi): _host(ds.groups[l][gi][3]) for l in range(2) for gi in range(4)},
               "head_y": _host(ds.head[3]), "head_argmax": _host(ds.head[8])}
    # path B: the whole token in one persistent launch in decode order (+ argmax), as a graph
    ds.make_plan()
    g = capture(torch, ds.step_stacked)
    per_s, total_s, _ = time_graph(torch, g, args.steps, args.warmup)
    err = kq.kq_stack_status(ds.plan, ds.info)
    if err:
        raise SystemExit(f"persistent stack reported a wait timeout (error word {err})")
    ms_stacked = total_s / args.steps
    log(f"M=1 step, one persistent launch in decode order + argmax: {ms_stacked * 1000:.1f} us")
    del g
    # the headline is the faster of the two (both run the same work)
    if ms_launches <= ms_stacked:
        ms_per_step, per = ms_launches, per_l
        path = (f"{ds.layers * 4} kq_gemv launches + kq_gemv_argmax (the lm_head kernel leaves per-workgroup "
                "argmax partials, one reduction kernel), captured once as a HIP graph and replayed")
        other = {"path": "kq_stack_run (persistent, decode order) + argmax", "ms_per_step": ms_stacked}
    else:
        ms_per_step, per = ms_stacked, per_s
        path = (f"kq_stack_run: {ds.n_stages} GEMV stages (every layer, then the lm_head) in one "
                "persistent launch, each stage reading the previous stage's fp16 output, then "
                "kq_argmax; captured once as a HIP graph and replayed")
        other = {"path": "per-launch graph", "ms_per_step": ms_launches}
    other["gbps"] = ds.alg_bytes / (other["ms_per_step"] * 1e-3) / 1e9
    gbps = ds.alg_bytes / (ms_per_step * 1e-3) / 1e9
    log(f"headline: {ms_per_step * 1000:.1f} us, {gbps:.0f} GB/s, {1000 / ms_per_step:.0f} tok/s")

    ktab = kernel_table(torch, ds)
    # dominant kernel: the launch group with the largest time per step
    dom = max((k for k in ktab if "gbps" in ktab[k]),
              key=lambda k: ktab[k]["us_per_launch"] * ktab[k]["launches_per_step"])
    d = ktab[dom]
    roofline = {"bound": "hbm", "achieved": d["gbps"], "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": d["gbps"] / HBM_PEAK_GBS, "traffic": measured_traffic(dom),
                "kernel": f"kq_gemv {dom} ({d['fmt']}, {d['N']}x{d['K']}, M=1)",
                "us_per_launch": d["us_per_launch"], "bytes_per_launch": d["bytes_per_launch"],
                "traffic_unit": "HBM bytes per launch (FETCH_SIZE + WRITE_SIZE, copy-calibrated)"}

    shortlist = shortlist_head(torch, ds, args.steps, args.warmup)
    log(f"lm_head argmax through Shortlist: {shortlist['us_per_call']:.1f} us per call "
        f"({shortlist['pct_rows_scored_exactly']:.2f} % of rows scored exactly), step "
        f"{shortlist['step_ms_with_shortlist'] * 1000:.1f} us")
    if not shortlist["index_equals_kq_gemv_argmax"]:
        raise SystemExit("Shortlist argmax differs from kq_gemv_argmax")
    torch.cuda.empty_cache()

    verify = None
    if not args.no_verify:
        dv = ds.with_columns(S, 8, S.VERIFY_WORKLOAD_ID)
        gv = capture(torch, dv.step)
        perv, total_v, _ = time_graph(torch, gv, max(5, args.steps // 2), 3)
        ms_v = total_v / max(5, args.steps // 2)
        gpu_out["verify8_head_y"] = _host(dv.head[3])
        gpu_out["verify8_head_argmax"] = _host(dv.head[8])
        vk = kernel_table(torch, dv, reps=5)
        vdom = max((k for k in vk if "gbps" in vk[k]),
                   key=lambda k: vk[k]["us_per_launch"] * vk[k]["launches_per_step"])
        vd = vk[vdom]
        tflops = 2.0 * 8 * vd["N"] * vd["K"] / (vd["us_per_launch"] * 1e-6) / 1e12
        verify = {"M": 8, "ms_per_pass": ms_v, "gbps": dv.alg_bytes / (ms_v * 1e-3) / 1e9,
                  "t_ratio_vs_m1": ms_v / ms_per_step,
                  "tokens_per_s_upper_bound": 8 / (ms_v * 1e-3),
                  "roofline": {"bound": "hbm", "achieved": vd["gbps"], "peak": HBM_PEAK_GBS, "unit": "GB/s",
                               "frac": vd["gbps"] / HBM_PEAK_GBS,
                               "kernel": f"kq_gemv {vdom} ({vd['fmt']}, {vd['N']}x{vd['K']}, M=8)",
                               "us_per_launch": vd["us_per_launch"],
                               "mfma_useful_tflops": tflops, "mfma_peak_tflops_f16": MFMA_PEAK_F16_TFLOPS,
                               "mfma_util_alg": tflops / MFMA_PEAK_F16_TFLOPS,
                               "mfma_busy_counter": measured_mfma("verify_m8", vdom)},
                  "kernels": vk}
        log(f"M=8 pass: {ms_v * 1000:.1f} us, t(8)/t(1) = {ms_v / ms_per_step:.2f}")
        del gv, dv
        torch.cuda.empty_cache()

    configs = None
    if not args.no_verify:
        verify_all = bench_verify_all(torch, kq, S, ds, float(np.median(per)), max(5, args.steps // 2))
    else:
        verify_all = None
    alg_bytes_step = ds.alg_bytes
    input_sha = ds.input_sha256
    if not args.no_configs:
        del ds
        torch.cuda.empty_cache()
        configs = {"single_q8_0": bench_single_q8_0(torch, kq, S, gpu_out)}
        log(f"single q8_0: {configs['single_q8_0']['us_per_call_cold']:.2f} us cold")
        configs["qwen3_0.6b_q4_0_stack"] = bench_small_stack(torch, kq, S, args.steps)
        log(f"0.6B stack: {configs['qwen3_0.6b_q4_0_stack']['us_per_step_cold']:.1f} us cold")
        configs["moe_q4_0"] = bench_moe(torch, kq, S, max(5, args.steps // 2))
        configs["formats"] = bench_formats(torch, kq, S)
        configs["stream_ceiling"] = stream_ceiling(torch)
        sc = configs["stream_ceiling"]
        log(f"read-only ceiling: {sc['sizes']['1GiB']['gbps']:.0f} GB/s at 1 GiB, plain-read step "
            f"{sc['plain_read_step_us']:.1f} us")
        for name, row in ktab.items():
            if name in sc["sizes"] and "gbps" in row:
                row["pct_of_read_ceiling"] = 100.0 * row["gbps"] / sc["sizes"][name]["gbps"]

    cpu = None
    oracle_configs = None
    if not args.no_cpu_baseline:
        log("timing the CPU oracle on 2 layers + lm_head (median of 3) and checking the GPU's outputs ...")
        cpu = cpu_baseline(S, stack, kq, gpu_out)
        log(f"  oracle {cpu['s_per_token']:.2f} s per token; parity {cpu['parity']}")
        if not args.no_configs:
            oracle_configs = oracle_other_configs(S, kq, gpu_out)

    out = {
        "metric": "achieved HBM GB/s (% of peak) + equiv. decode tokens/s, M=1 and M=8 verify",
        "value": gbps,
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "affine4/q8_0 weights, f16 activations, f32 accumulate",
        "data": "synthetic (seeded N(0,0.02) weights, N(0,1) fp16 activations)",
        "config": {"workload": "qwen3_4b_shaped_affine4_stack+q8_0_lm_head, M=1, one decode token",
                   "layers": stack.layers, "hidden": 2560, "intermediate": 9728, "vocab": 151936,
                   "global_batch": 1, "seq_len": 1, "parallelism": "none (1 GPU)"},
        "pct_of_peak": 100.0 * gbps / HBM_PEAK_GBS,
        "tokens_per_s": 1000.0 / ms_per_step,
        "step_us_p10_p50_p90": [float(np.percentile(per, q)) * 1000 for q in (10, 50, 90)],
        "path": path,
        "other_path": other,
        "alg_bytes_per_step": alg_bytes_step,
        "roofline": roofline,
        "kernels": ktab,
        "lm_head_shortlist": shortlist,
        "verify_m8": verify,
        "verify_all": verify_all,
        "other_configs": configs,
        "cpu_baseline": cpu,
        "oracle_other_configs": oracle_configs,
        "env": {**env_info(torch), "input_sha256": input_sha},
    }
    if configs is not None:
        out["pct_of_read_ceiling_step"] = 100.0 * configs["stream_ceiling"]["plain_read_step_us"] / (ms_per_step * 1000)
    print(json.dumps(out))


if __name__ == "__main__":
    main()
