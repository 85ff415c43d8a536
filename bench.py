#!/usr/bin/env python3
"""Benchmark of gated GQA decode (and prefill) on one MI355X.

A step is one gated_attn_decode call -- stage 1 and stage 2 with the fused
gate, the whole decode path -- over the B=64, L=4096 paged workload (512 MiB of
K/V), inputs resident in HBM.  ``value`` is K/V bytes per second over the timed
steps.  Decode measurements rotate over copies of their inputs (two for this
workload) so that no call can read K/V the previous one left in the 256 MB
Infinity Cache.  The same JSON line also carries:
  * roofline   -- the stage-1 kernel's achieved HBM rate: K launches of that
                  kernel alone, chained in one HIP graph (its node copied from
                  graphs captured from the workload's calls) with an event
                  recorded before and after each, on the stream it runs on; ``traffic`` from the committed rocprofv3
                  counter summary when it was taken on the current kernel
                  source, else null;
  * launches_per_call -- kernel nodes of a HIP graph captured from one call;
  * cold       -- median of single calls, each after a 1 GiB cache flush;
  * b1_l512, b4_ragged -- the latency pair (B=1 L=512; B=4 L=512/495/478/461)
                  in µs/call from replays of a 4-call HIP graph, B=1 also
                  cold; launch_floor -- two dependent tiny kernels the same way;
  * prefill    -- B=2, S=2048 causal gated prefill µs/call and MFMA rate;
  * cpu_baseline -- the fp64 CPU oracle on the same B=64 workload.

    python bench.py [--steps K] [--warmup W] [--gpus 1]
"""
from __future__ import annotations

import argparse
import ctypes
import hashlib
import json
import os
import statistics
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "gated decode attention µs/call + KV HBM GB/s (% of peak), B1/L512 and B64/L4096"
HBM_PEAK_GBS = 8000.0          # MI355X HBM3E
BF16_MFMA_PEAK_TFLOPS = 2500.0  # MI355X dense bf16 matrix peak
COUNTERS = os.path.join(ROOT, "profiles", "decode_stage1_b64_l4096_counters.json")
KERNEL_SOURCES = ["gated_gqa_decode_amd/csrc/decode.hip", "gated_gqa_decode_amd/csrc/ga_device.h",
                  "gated_gqa_decode_amd/csrc/ga_internal.h", "gated_gqa_decode_amd/csrc/capi.cpp"]


PREFILL_COUNTERS = os.path.join(ROOT, "profiles", "prefill_b2_s2048_causal_counters.json")
FP8_COUNTERS = os.path.join(ROOT, "profiles", "decode_stage1_fp8_b64_l4096_counters.json")


def kernel_source_hash(sources=None) -> str:
    h = hashlib.sha256()
    for rel in (KERNEL_SOURCES if sources is None else sources):
        with open(os.path.join(ROOT, rel), "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def fp8_stage1_traffic():
    """HBM bytes per launch of the e4m3 stage-1 kernel (FETCH_SIZE + WRITE_SIZE,
    calibrated) from its committed rocprofv3 counter summary, or None when that
    was taken on other kernel sources."""
    if not os.path.exists(FP8_COUNTERS):
        return None
    with open(FP8_COUNTERS) as f:
        c = json.load(f)
    if c.get("kernel_sources_sha256") != kernel_source_hash():
        return None
    return {"source": os.path.relpath(FP8_COUNTERS, ROOT),
            "hbm_bytes_per_launch": c["hbm_bytes_per_launch"],
            "algorithmic_bytes_per_launch": c["algorithmic_bytes_per_launch"],
            "traffic_over_algorithmic": c["traffic_over_algorithmic"]}


def prefill_counters():
    """MFMA figures of the prefill kernel from its committed rocprofv3 counter
    passes, or None when those were taken on other kernel sources."""
    if not os.path.exists(PREFILL_COUNTERS):
        return None
    with open(PREFILL_COUNTERS) as f:
        c = json.load(f)
    if c.get("kernel_sources_sha256") != kernel_source_hash(c.get("kernel_sources", [])):
        return None
    return {"source": os.path.relpath(PREFILL_COUNTERS, ROOT),
            "mfma_busy_frac": c["mfma_busy_frac_of_counter_run"],
            "issued_over_algorithmic": c["issued_over_algorithmic"],
            "mfma_instructions": c["mfma_instructions"],
            "lds_bank_conflict_frac": c["lds_bank_conflict_frac_of_active"]}


def parse_args():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--settle-s", type=float, default=0.3,
                    help="untimed decode calls for this many seconds before the warm-up "
                         "steps, so the GPU clock has left its idle state")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-extras", action="store_true",
                    help="only the timed decode steps (cold, B1, prefill, CPU legs skipped)")
    ap.add_argument("--prefill-only", action="store_true",
                    help="time only the B=2, S=2048 causal prefill (for profiling)")
    ap.add_argument("--only", choices=["decode_fp8kv", "decode_hq32", "decode_b224",
                                       "decode_fp8kv_page1", "b1_l512", "qk_norm_rope_t4096"],
                    default=None,
                    help="time only this variant (for profiling its kernels): a decode variant at "
                         "B=64, L=4096, the B=224 serving shape, the B=1 L=512 graph replays, or "
                         "the dense T=4096 QK-norm + RoPE step")
    ap.add_argument("--calibration-copy", action="store_true",
                    help="also run one plain 1 GiB device copy (counter calibration)")
    ap.add_argument("--json-out", default=None)
    return ap.parse_args()


class Hip:
    """The few HIP runtime calls the timing needs (events and graphs), from the
    runtime torch loaded."""

    def __init__(self):
        import torch  # noqa: F401  (loads the runtime this binds to)

        vp, P = ctypes.c_void_p, ctypes.POINTER
        self.lib = L = ctypes.CDLL("libamdhip64.so.7")
        L.hipEventCreateWithFlags.argtypes = [P(vp), ctypes.c_uint]
        L.hipEventRecord.argtypes = [vp, vp]
        L.hipEventElapsedTime.argtypes = [P(ctypes.c_float), vp, vp]
        L.hipEventDestroy.argtypes = [vp]
        L.hipStreamBeginCapture.argtypes = [vp, ctypes.c_int]
        L.hipStreamEndCapture.argtypes = [vp, P(vp)]
        L.hipGraphGetNodes.argtypes = [vp, P(vp), P(ctypes.c_size_t)]
        L.hipGraphNodeGetType.argtypes = [vp, P(ctypes.c_int)]
        L.hipGraphNodeGetDependencies.argtypes = [vp, P(vp), P(ctypes.c_size_t)]
        L.hipGraphDestroyNode.argtypes = [vp]
        L.hipGraphInstantiate.argtypes = [P(vp), vp, P(vp), ctypes.c_char_p, ctypes.c_size_t]
        L.hipGraphLaunch.argtypes = [vp, vp]
        L.hipGraphExecDestroy.argtypes = [vp]
        L.hipGraphDestroy.argtypes = [vp]

    def _ok(self, err, what):
        if err != 0:
            raise RuntimeError(f"{what} failed (hipError_t {err})")

    # Timing-only events: no system-scope fence (cache write-back and
    # invalidation) when they are recorded, so the interval between two of
    # them holds the kernel, not a flush after it (the stream is synchronised
    # before the intervals are read).
    EVENT_DISABLE_SYSTEM_FENCE = 0x20000000

    def events(self, n):
        out = []
        for _ in range(n):
            e = ctypes.c_void_p()
            self._ok(self.lib.hipEventCreateWithFlags(ctypes.byref(e), self.EVENT_DISABLE_SYSTEM_FENCE),
                     "hipEventCreateWithFlags")
            out.append(e.value)
        return out

    def record(self, ev, stream):
        self._ok(self.lib.hipEventRecord(ctypes.c_void_p(ev), stream), "hipEventRecord")

    def elapsed_ms(self, a, b) -> float:
        ms = ctypes.c_float()
        self._ok(self.lib.hipEventElapsedTime(ctypes.byref(ms), ctypes.c_void_p(a), ctypes.c_void_p(b)),
                 "hipEventElapsedTime")
        return float(ms.value)

    def destroy(self, evs):
        for e in evs:
            self.lib.hipEventDestroy(ctypes.c_void_p(e))

    # ---- graphs ------------------------------------------------------------
    KERNEL_NODE = 0   # hipGraphNodeTypeKernel
    CAPTURE_RELAXED = 2

    def capture(self, fn, stream) -> int:
        """The hipGraph_t of everything fn() enqueues on `stream` (a torch side
        stream's handle)."""
        self._ok(self.lib.hipStreamBeginCapture(stream, self.CAPTURE_RELAXED), "hipStreamBeginCapture")
        try:
            fn()
        finally:
            g = ctypes.c_void_p()
            self._ok(self.lib.hipStreamEndCapture(stream, ctypes.byref(g)), "hipStreamEndCapture")
        return g.value

    def nodes(self, graph):
        n = ctypes.c_size_t(0)
        self._ok(self.lib.hipGraphGetNodes(ctypes.c_void_p(graph), None, ctypes.byref(n)), "hipGraphGetNodes")
        arr = (ctypes.c_void_p * max(n.value, 1))()
        self._ok(self.lib.hipGraphGetNodes(ctypes.c_void_p(graph), arr, ctypes.byref(n)), "hipGraphGetNodes")
        out = []
        for i in range(n.value):
            t = ctypes.c_int()
            self._ok(self.lib.hipGraphNodeGetType(ctypes.c_void_p(arr[i]), ctypes.byref(t)),
                     "hipGraphNodeGetType")
            d = ctypes.c_size_t(0)
            self._ok(self.lib.hipGraphNodeGetDependencies(ctypes.c_void_p(arr[i]), None, ctypes.byref(d)),
                     "hipGraphNodeGetDependencies")
            out.append((arr[i], t.value, d.value))
        return out

    def instantiate(self, graph) -> int:
        e = ctypes.c_void_p()
        self._ok(self.lib.hipGraphInstantiate(ctypes.byref(e), ctypes.c_void_p(graph), None, None, 0),
                 "hipGraphInstantiate")
        return e.value

    def launch(self, exec_, stream):
        self._ok(self.lib.hipGraphLaunch(ctypes.c_void_p(exec_), stream), "hipGraphLaunch")


def call_graph_census(hip, fn, dev) -> dict:
    """Kernel and non-kernel nodes of one captured call: the measured number of
    launches a call makes (the gate must add none)."""
    import torch

    side = torch.cuda.Stream(device=dev)
    torch.cuda.synchronize()
    keep = fn.stream
    fn.stream = ctypes.c_void_p(side.cuda_stream)
    try:
        g = hip.capture(fn, fn.stream)
    finally:
        fn.stream = keep
    try:
        nodes = hip.nodes(g)
    finally:
        hip.lib.hipGraphDestroy(ctypes.c_void_p(g))
    kernels = sum(1 for _, t, _ in nodes if t == Hip.KERNEL_NODE)
    return {"kernels": kernels, "other_nodes": len(nodes) - kernels,
            "method": "nodes of a HIP graph captured from one call"}


class Dim3(ctypes.Structure):
    _fields_ = [("x", ctypes.c_uint), ("y", ctypes.c_uint), ("z", ctypes.c_uint)]


class KernelNodeParams(ctypes.Structure):
    """hipKernelNodeParams."""
    _fields_ = [("blockDim", Dim3), ("extra", ctypes.c_void_p), ("func", ctypes.c_void_p),
                ("gridDim", Dim3), ("kernelParams", ctypes.c_void_p),
                ("sharedMemBytes", ctypes.c_uint)]


class Stage1Graphs:
    """Stage 1 of a decode call on its own, timed by the GPU.  Each input set's
    call is captured into a HIP graph and its stage-1 kernel node (the root;
    stage 2 depends on it) is read back.  time(n) builds one graph that chains
    n copies of those kernel nodes, input sets in turn, with an event-record
    node before and after each, and launches it once on a stream: each pair
    of events brackets one stage-1 kernel on the stream it runs on, with no
    host work and no hook in the library between them."""

    def __init__(self, hip, calls, dev):
        import torch

        L = hip.lib
        vp, P = ctypes.c_void_p, ctypes.POINTER
        L.hipGraphKernelNodeGetParams.argtypes = [vp, P(KernelNodeParams)]
        L.hipGraphCreate.argtypes = [P(vp), ctypes.c_uint]
        L.hipGraphAddKernelNode.argtypes = [P(vp), vp, P(vp), ctypes.c_size_t,
                                            P(KernelNodeParams)]
        L.hipGraphAddEventRecordNode.argtypes = [P(vp), vp, P(vp), ctypes.c_size_t, vp]
        self.hip = hip
        self.side = torch.cuda.Stream(device=dev)
        self.stream = ctypes.c_void_p(self.side.cuda_stream)
        self.graphs, self.params = [], []
        torch.cuda.synchronize()
        for call in calls:
            keep = call.stream
            call.stream = self.stream
            try:
                g = hip.capture(call, self.stream)
            finally:
                call.stream = keep
            self.graphs.append(g)  # kept alive: the node parameters point into it
            nodes = hip.nodes(g)
            roots = [n for n, t, d in nodes if t == Hip.KERNEL_NODE and d == 0]
            if len(roots) != 1 or len(nodes) != 2:
                raise RuntimeError(f"unexpected decode graph: {nodes}")
            prm = KernelNodeParams()
            hip._ok(L.hipGraphKernelNodeGetParams(ctypes.c_void_p(roots[0]), ctypes.byref(prm)),
                    "hipGraphKernelNodeGetParams")
            self.params.append(prm)

    def time(self, n: int, warm: int = 3) -> list:
        """Per-launch ms of n stage-1 kernels, input sets in turn, after
        `warm` untimed ones, all in one graph launch."""
        import torch

        hip, L = self.hip, self.hip.lib
        starts, stops = hip.events(n), hip.events(n)
        g = ctypes.c_void_p()
        hip._ok(L.hipGraphCreate(ctypes.byref(g), 0), "hipGraphCreate")
        prev = None

        def add(kind, arg):
            nonlocal prev
            node = ctypes.c_void_p()
            deps = (ctypes.c_void_p * 1)(prev) if prev is not None else None
            nd = 1 if prev is not None else 0
            if kind == "kernel":
                hip._ok(L.hipGraphAddKernelNode(ctypes.byref(node), g, deps, nd, ctypes.byref(arg)),
                        "hipGraphAddKernelNode")
            else:
                hip._ok(L.hipGraphAddEventRecordNode(ctypes.byref(node), g, deps, nd,
                                                     ctypes.c_void_p(arg)),
                        "hipGraphAddEventRecordNode")
            prev = node.value
        k = 0
        for _ in range(warm):
            add("kernel", self.params[k % len(self.params)])
            k += 1
        for i in range(n):
            add("event", starts[i])
            add("kernel", self.params[k % len(self.params)])
            k += 1
            add("event", stops[i])
        ex = hip.instantiate(g.value)
        hip.launch(ex, self.stream)
        self.side.synchronize()
        torch.cuda.synchronize()
        ms = [hip.elapsed_ms(a, b) for a, b in zip(starts, stops)]
        hip.destroy(starts + stops)
        L.hipGraphExecDestroy(ctypes.c_void_p(ex))
        L.hipGraphDestroy(g)
        return ms

    def close(self):
        for g in self.graphs:
            self.hip.lib.hipGraphDestroy(ctypes.c_void_p(g))


def to_dev(a, dev):
    import numpy as np
    import torch

    t = torch.from_numpy(np.ascontiguousarray(a))
    if a.dtype == np.uint16:
        t = t.view(torch.int16).view(torch.bfloat16)
    return t.to(dev)


class DecodeCall:
    """Pre-marshalled arguments of one gated_attn_decode call (raw C entry)."""

    def __init__(self, ga, case, dev, sinks=None, window=0, lse=False):
        import torch

        self.ga = ga
        self.t = [to_dev(x, dev) for x in (case.q, case.gate, case.k_pool, case.v_pool,
                                          case.block_table, case.seq_lens)]
        self.dims = ga.decode_dims(**case.dims)
        self.plan = ga.decode_plan(self.dims)
        self.ws = torch.empty(max(self.plan.workspace_bytes, 16), dtype=torch.uint8, device=dev)
        self.out = torch.empty_like(self.t[0])
        self.scale = ctypes.c_float(case.scale)
        self.stream = ctypes.c_void_p(torch.cuda.current_stream(dev).cuda_stream)
        self.args = [ctypes.c_void_p(x.data_ptr()) for x in self.t]
        self.outp = ctypes.c_void_p(self.out.data_ptr())
        self.wsp = ctypes.c_void_p(self.ws.data_ptr())
        self.wsb = ctypes.c_size_t(self.ws.numel())
        self.dref = ctypes.byref(self.dims)
        self.fn = ga.lib.gated_attn_decode
        self.extra = ()
        if sinks is not None or window or lse:
            # attention-spec options through gated_attn_decode_ex
            B, Hq = case.q.shape[:2]
            self.sinks = None if sinks is None else torch.tensor(sinks, dtype=torch.float32,
                                                                 device=dev)
            self.lse = torch.empty((B, Hq), dtype=torch.float32, device=dev) if lse else None
            self.opts = ga.AttnOptions(
                sinks=None if self.sinks is None else self.sinks.data_ptr(),
                lse=None if self.lse is None else self.lse.data_ptr(), window=int(window))
            self.fn = ga.lib.gated_attn_decode_ex
            self.extra = (ctypes.byref(self.opts),)

        self.descales = ()
        if getattr(case, "fp8", False):
            # e4m3 pools through gated_attn_decode_fp8kv (options pointer last, may be NULL)
            self.fn = ga.lib.gated_attn_decode_fp8kv
            self.descales = (ctypes.c_float(case.k_descale), ctypes.c_float(case.v_descale))
            if not self.extra:
                self.extra = (None,)

    def __call__(self):
        st = self.fn(*self.args, self.scale, *self.descales, self.outp, self.stream, self.dref,
                     self.wsp, self.wsb, *self.extra)
        if st != 0:
            self.ga.check(st, "gated_attn_decode")


class PrefillCall:
    """Pre-marshalled arguments of one gated_attn_prefill call (raw C entry)."""

    def __init__(self, ga, p, dev, causal=True):
        import torch

        self.ga = ga
        self.t = [to_dev(x, dev) for x in (p.q, p.gate, p.k, p.v)]
        self.out = torch.empty_like(self.t[0])
        B, S, Hq, D = p.q.shape
        self.dims = ga.PrefillDims(B, S, Hq, p.k.shape[2], D)
        self.args = [ctypes.c_void_p(x.data_ptr()) for x in self.t] + [
            ctypes.c_float(p.scale), ctypes.c_int(int(causal)), ctypes.c_void_p(self.out.data_ptr())]
        self.stream = ctypes.c_void_p(torch.cuda.current_stream(dev).cuda_stream)

    def __call__(self):
        st = self.ga.lib.gated_attn_prefill(*self.args, self.stream, ctypes.byref(self.dims))
        if st != 0:
            self.ga.check(st, "gated_attn_prefill")


def time_prefill(ga, p, dev, n_calls: int, settle_s: float = 0.0) -> dict:
    """Causal gated prefill on case p: n_calls back-to-back calls of the C
    entry point with pre-marshalled arguments (no Python work between calls),
    after settle_s seconds of untimed calls."""
    import torch

    call = PrefillCall(ga, p, dev)
    t0 = time.perf_counter()
    while time.perf_counter() - t0 < settle_s:  # clock settling, untimed
        for _ in range(10):
            call()
        torch.cuda.synchronize()
    for _ in range(3):
        call()
    torch.cuda.synchronize()
    a = torch.cuda.Event(enable_timing=True)
    b = torch.cuda.Event(enable_timing=True)
    a.record()
    for _ in range(n_calls):
        call()
    b.record()
    torch.cuda.synchronize()
    pms = a.elapsed_time(b) / n_calls
    B, S, Hq, D = p.q.shape
    Hkv = p.k.shape[2]
    flops = 4.0 * D * Hq * B * S * (S + 1) / 2
    tflops = flops / (pms * 1e-3) / 1e12
    return {"workload": f"gated causal prefill B={B} S={S} H_q={Hq} H_kv={Hkv} D={D}",
            "us_per_call": round(pms * 1e3, 3),
            "calls": n_calls,
            "algorithmic_flop": flops,
            "tflops": round(tflops, 2),
            "mfma_bf16_frac": round(tflops / BF16_MFMA_PEAK_TFLOPS, 4),
            "counters": prefill_counters() if (B, S, Hq, Hkv, D) == (2, 2048, 16, 2, 256) else None,
            "note": "P is split into two bf16 terms, so the kernel issues 1.5x "
                    "the algorithmic MFMA work"}


def _capture_torch_graph(fn, dev):
    """A torch CUDAGraph of fn(stream): fn enqueues on the stream handle given."""
    import torch

    s = torch.cuda.Stream(device=dev)
    s.wait_stream(torch.cuda.current_stream())
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        fn(ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
    torch.cuda.synchronize()
    return g


def _replay_samples(g, calls_per_graph: int, replays: int = 50, samples: int = 7) -> list:
    import torch

    for _ in range(10):
        g.replay()
    torch.cuda.synchronize()
    out = []
    for _ in range(samples):
        a = torch.cuda.Event(enable_timing=True)
        b = torch.cuda.Event(enable_timing=True)
        a.record()
        for _ in range(replays):
            g.replay()
        b.record()
        torch.cuda.synchronize()
        out.append(a.elapsed_time(b) * 1e3 / (replays * calls_per_graph))
    return out


def graph_latency(ga, case, dev) -> dict:
    """us/call of a latency-bound decode: a HIP graph of 4 calls, 50 replays
    per sample, median of 7 samples (the FreeToken PR's kernel-window method)."""
    sc = DecodeCall(ga, case, dev)
    sc()

    def four(stream):
        sc.stream = stream
        for _ in range(4):
            sc()
    g = _capture_torch_graph(four, dev)
    samples = _replay_samples(g, 4)
    us = statistics.median(samples)
    lens = ",".join(str(int(x)) for x in case.seq_lens)
    return {"workload": f"gated GQA decode B={case.q.shape[0]} L={lens}, paged",
            "us_per_call": round(us, 3),
            "kv_gbs": round(case.kv_bytes() / (us * 1e-6) / 1e9, 2),
            "method": "HIP graph of 4 calls, 50 replays per sample, median of 7",
            "samples_us": [round(x, 3) for x in samples]}


def cold_latency(ga, case, dev, blocks: int = 7, per_block: int = 31) -> dict:
    """us of one call right after a 1 GiB write (every cache level holds other
    lines): a graph of one call replayed between two events, the flush
    enqueued before the first event (outside the timed span); 7 blocks of 31
    samples, median."""
    import torch

    sc = DecodeCall(ga, case, dev)
    sc()

    def one(stream):
        sc.stream = stream
        sc()
    g = _capture_torch_graph(one, dev)
    flush = torch.empty(1 << 30, dtype=torch.uint8, device=dev)
    block_medians, allv = [], []
    for _ in range(blocks):
        xs = []
        for _ in range(per_block):
            flush.fill_(1)
            a = torch.cuda.Event(enable_timing=True)
            b = torch.cuda.Event(enable_timing=True)
            a.record()
            g.replay()
            b.record()
            torch.cuda.synchronize()
            xs.append(a.elapsed_time(b) * 1e3)
        block_medians.append(statistics.median(xs))
        allv += xs
    del flush, g
    return {"us_per_call": round(statistics.median(allv), 3),
            "block_medians_us": [round(x, 3) for x in block_medians],
            "method": "1 GiB write before each single-call graph replay, outside the timed span; "
                      f"{blocks} blocks x {per_block} samples, median"}


def launch_floor(dev) -> dict:
    """The replay floor of two dependent launches: a graph of 4 pairs of
    one-element torch kernels, timed like graph_latency.  A decode call is two
    launches, so this is the least a call can cost in a graph."""
    import torch

    x = torch.zeros(1, dtype=torch.float32, device=dev)

    def pairs(stream):
        for _ in range(4):
            x.add_(1.0)
            x.mul_(0.5)
    g = _capture_torch_graph(pairs, dev)
    samples = _replay_samples(g, 4)
    return {"us_per_pair": round(statistics.median(samples), 3),
            "method": "HIP graph of 4 pairs of dependent one-element kernels, 50 replays per "
                      "sample, median of 7",
            "samples_us": [round(v, 3) for v in samples]}


# The MI355X's 256 MB Infinity Cache (MALL) sits between L2 and HBM.  Back-to-
# back calls on one set of inputs could read part of a call's K/V from what the
# previous call left there, which would overstate HBM bandwidth.  Every decode
# measurement therefore rotates over copies of its inputs (all resident in
# HBM) whose visible K/V add up to at least 768 MiB per rotation, so no call
# finds its rows in the cache.
MALL_DEFEAT_BYTES = 768 << 20


def rotation_sets(visible_bytes: int) -> int:
    return max(2, min(8, -(-MALL_DEFEAT_BYTES // max(int(visible_bytes), 1))))


class Rotation:
    """Calls of one decode configuration over n resident input copies, in turn."""

    def __init__(self, make, n: int):
        self.calls = [make() for _ in range(n)]
        self.i = 0

    def __call__(self):
        self.calls[self.i]()
        self.i = (self.i + 1) % len(self.calls)

    @property
    def plan(self):
        return self.calls[0].plan


def time_decode(ga, case, dev, n_calls: int, settle_s: float = 0.1, **opts) -> dict:
    """Back-to-back decode calls on case: us/call and K/V bytes per second
    (the bytes of the visible keys: a window reads only those)."""
    import numpy as np
    import torch

    import numpy as np

    lens_v = np.clip(case.seq_lens.astype(np.int64), 0, None)
    if opts.get("window"):
        lens_v = np.minimum(lens_v, int(opts["window"]))
    visible = int(lens_v.sum()) * case.k_pool.shape[2] * case.k_pool.shape[3] * case.k_pool.dtype.itemsize * 2
    n_sets = rotation_sets(visible)
    call = Rotation(lambda: DecodeCall(ga, case, dev, **opts), n_sets)
    t0 = time.perf_counter()
    while time.perf_counter() - t0 < settle_s:  # clock settling, untimed
        for _ in range(20):
            call()
        torch.cuda.synchronize()
    for _ in range(10):
        call()
    torch.cuda.synchronize()
    a = torch.cuda.Event(enable_timing=True)
    b = torch.cuda.Event(enable_timing=True)
    a.record()
    for _ in range(n_calls):
        call()
    b.record()
    torch.cuda.synchronize()
    ms = a.elapsed_time(b) / n_calls
    B, Hq, D = case.q.shape
    Hkv = case.k_pool.shape[2]
    lens = np.clip(case.seq_lens.astype(np.int64), 0, None)
    if opts.get("window"):
        lens = np.minimum(lens, int(opts["window"]))
    kv = int(lens.sum()) * Hkv * D * case.k_pool.dtype.itemsize * 2
    gbs = kv / (ms * 1e-3) / 1e9
    desc = ", ".join(f"{k}={'yes' if k == 'sinks' else v}" for k, v in opts.items() if v is not None)
    return {"workload": f"gated GQA decode B={B} L={int(case.seq_lens.max())} H_q={Hq} "
                        f"H_kv={Hkv} D={D}, paged" + (f", {desc}" if desc else ""),
            "us_per_call": round(ms * 1e3, 3), "calls": n_calls,
            "kv_gbs": round(gbs, 2), "hbm_frac": round(gbs / HBM_PEAK_GBS, 4),
            "tokens_per_split": call.plan.tokens_per_split, "num_splits": call.plan.num_splits,
            "input_sets": n_sets}


def stream_read_ceiling(ga, dev, n_calls: int = 20) -> dict:
    """GB/s of a plain read of 1 GiB with the decode's non-temporal 16-byte
    loads (gated_attn_stream_read; two buffers used in turn, so neither is
    served from the Infinity Cache): the streaming-read rate of the device."""
    import torch

    bufs = [torch.ones(1 << 28, dtype=torch.float32, device=dev) for _ in range(2)]
    sink = torch.zeros(1, dtype=torch.int32, device=dev)
    stream = ctypes.c_void_p(torch.cuda.current_stream(dev).cuda_stream)
    args = [(ctypes.c_void_p(x.data_ptr()), ctypes.c_size_t(1 << 30),
             ctypes.c_void_p(sink.data_ptr()), stream) for x in bufs]
    for i in range(6):
        ga.check(ga.lib.gated_attn_stream_read(*args[i % 2]), "gated_attn_stream_read")
    torch.cuda.synchronize()
    a = torch.cuda.Event(enable_timing=True)
    b = torch.cuda.Event(enable_timing=True)
    a.record()
    for i in range(n_calls):
        ga.lib.gated_attn_stream_read(*args[i % 2])
    b.record()
    torch.cuda.synchronize()
    us = a.elapsed_time(b) * 1e3 / n_calls
    return {"method": "gated_attn_stream_read over 1 GiB, two buffers in turn",
            "us_per_call": round(us, 3), "gbs": round((1 << 30) / (us * 1e-6) / 1e9, 2),
            "hbm_frac": round((1 << 30) / (us * 1e-6) / 1e9 / HBM_PEAK_GBS, 4)}


def only_case(workloads, name: str):
    """Decode variants timed on their own with --only: the B=64, L=4096
    variants that run the MFMA stage 1, and the B=224 serving shape."""
    if name == "decode_hq32":  # GQA group 16
        return workloads.make_decode("decode_b64_l4096_hq32", [4096] * 64, seed=2,
                                     num_q_heads=32, num_kv_heads=2, poison=False,
                                     max_pages_per_seq=256)
    if name == "decode_fp8kv":  # e4m3 K / V pools, same shape as the headline
        return workloads.make_decode("decode_b64_l4096_fp8", [4096] * 64, seed=2, poison=False,
                                     max_pages_per_seq=256, kv_dtype="fp8")
    if name == "decode_b224":  # the serving shape: B=224, L ~ U{4094..6142}
        return workloads.workload(3, poison=False)
    if name == "decode_fp8kv_page1":  # e4m3 pools at page size 1 (token slots, shuffled)
        c = workloads.make_decode("decode_b64_l4096_fp8_page1", [4096] * 64, seed=2, poison=False,
                                  max_pages_per_seq=256, kv_dtype="fp8")
        k1, v1, _, _, table = workloads.csr_layout(c, seed=2, poison=False)
        return workloads.DecodeCase(c.name, c.q, c.gate, k1, v1, table, c.seq_lens, c.scale,
                                    c.k_descale, c.v_descale)
    raise ValueError(name)


def time_decode_csr(ga, workloads, case, dev, n_calls: int) -> dict:
    """The headline workload's tokens at page size 1 (one pool row per token,
    shuffled), addressed by CSR row pointers: back-to-back calls."""
    import numpy as np
    import torch

    k1, v1, indptr, idx, _ = workloads.csr_layout(case, seed=2, poison=False)
    cap = case.block_table.shape[1] * case.k_pool.shape[1]
    dims = ga.decode_dims(case.q.shape[0], case.q.shape[1], k1.shape[2], case.q.shape[2], 1, cap,
                          k1.shape[0])
    n_sets = rotation_sets(case.kv_bytes())
    keep, arg_sets = [], []
    for _ in range(n_sets):  # resident copies used in turn (see MALL_DEFEAT_BYTES)
        t = [to_dev(x, dev) for x in (case.q, case.gate, k1, v1, indptr, idx)]
        ws = torch.empty(max(ga.decode_plan(dims).workspace_bytes, 16), dtype=torch.uint8,
                         device=dev)
        out = torch.empty_like(t[0])
        keep.append((t, ws, out))
        arg_sets.append([ctypes.c_void_p(x.data_ptr()) for x in t] + [
            ctypes.c_int64(idx.size), ctypes.c_float(case.scale), ctypes.c_void_p(out.data_ptr()),
            ctypes.c_void_p(torch.cuda.current_stream(dev).cuda_stream), ctypes.byref(dims),
            ctypes.c_void_p(ws.data_ptr()), ctypes.c_size_t(ws.numel()), None])
    fn = ga.lib.gated_attn_decode_csr
    for i in range(30):
        ga.check(fn(*arg_sets[i % n_sets]), "gated_attn_decode_csr")
    torch.cuda.synchronize()
    a = torch.cuda.Event(enable_timing=True)
    b = torch.cuda.Event(enable_timing=True)
    a.record()
    for i in range(n_calls):
        fn(*arg_sets[i % n_sets])
    b.record()
    torch.cuda.synchronize()
    us = a.elapsed_time(b) * 1e3 / n_calls
    gbs = case.kv_bytes() / (us * 1e-6) / 1e9
    return {"workload": "gated GQA decode B=64 L=4096 H_q=16 H_kv=2 D=256, page size 1, "
                        "CSR indexing, shuffled token slots",
            "us_per_call": round(us, 3), "kv_gbs": round(gbs, 2),
            "hbm_frac": round(gbs / HBM_PEAK_GBS, 4), "input_sets": n_sets}


def time_qk_norm_rope(ga, workloads, dev, T: int, slots: bool, n_calls: int = 200) -> dict:
    """QK-RMSNorm + RoPE (+ K/V slot write) over T tokens, H_q=16, H_kv=2,
    rope_dim 64: us/call and bytes moved per second."""
    import numpy as np
    import torch

    r = workloads.make_rope(f"rope_t{T}", T, seed=5, rope_dim=64)
    moved = 2 * T * (16 + 2 + 2) * 256 * 2 + T * 64 * 2 * 2  # rows in + out, tables in
    n_sets = rotation_sets(moved)
    fn = ga.lib.gated_attn_qk_norm_rope
    keep, arg_sets = [], []
    for _ in range(n_sets):  # resident copies used in turn (see MALL_DEFEAT_BYTES)
        t = {n: to_dev(getattr(r, n), dev) for n in ("q", "k", "v", "w_q", "w_k", "cos", "sin")}
        kw = {}
        if slots:
            P = (T + 15) // 16
            kw = dict(slot_mapping=torch.arange(T, dtype=torch.int64, device=dev),
                      k_pool=torch.zeros((P, 16, 2, 256), dtype=torch.bfloat16, device=dev),
                      v_pool=torch.zeros((P, 16, 2, 256), dtype=torch.bfloat16, device=dev))
        q_out = torch.empty_like(t["q"])
        if slots:
            k_out, v_out = kw["k_pool"], kw["v_pool"]
        else:
            k_out, v_out = torch.empty_like(t["k"]), torch.empty_like(t["v"])
        # pre-marshalled raw C call, so the timing is the GPU's and not the wrapper's
        dims = ga.QkNormRopeDims(T, 16, 2, 256, 64, 16, 0, k_out.shape[0] if slots else 0)
        keep.append((t, kw, q_out, k_out, v_out, dims))
        arg_sets.append(
            [ctypes.c_void_p(x.data_ptr()) for x in (t["q"], t["k"], t["v"], t["w_q"], t["w_k"])]
            + [ctypes.c_float(r.eps)]
            + [ctypes.c_void_p(x.data_ptr()) for x in (t["cos"], t["sin"])]
            + [ctypes.c_void_p(kw["slot_mapping"].data_ptr()) if slots else None]
            + [ctypes.c_void_p(x.data_ptr()) for x in (q_out, k_out, v_out)]
            + [ctypes.c_void_p(torch.cuda.current_stream(dev).cuda_stream), ctypes.byref(dims)])
    turn = [0]

    def call():
        st = fn(*arg_sets[turn[0]])
        turn[0] = (turn[0] + 1) % n_sets
        if st != 0:
            ga.check(st, "gated_attn_qk_norm_rope")
    for _ in range(20):
        call()
    torch.cuda.synchronize()
    a = torch.cuda.Event(enable_timing=True)
    b = torch.cuda.Event(enable_timing=True)
    a.record()
    for _ in range(n_calls):
        call()
    b.record()
    torch.cuda.synchronize()
    us = a.elapsed_time(b) * 1e3 / n_calls
    return {"workload": f"QK-RMSNorm + RoPE (rope_dim 64) + K/V {'slot writes' if slots else 'dense'}, "
                        f"T={T}, H_q=16 H_kv=2 D=256",
            "us_per_call": round(us, 3), "gbs": round(moved / (us * 1e-6) / 1e9, 2),
            "input_sets": n_sets}


def calibration_copy(dev) -> None:
    """One plain device copy of 1 GiB (reads 1 GiB, writes 1 GiB): the known
    size that scales the FETCH_SIZE / WRITE_SIZE counter readings."""
    import torch

    src = torch.empty(1 << 30, dtype=torch.uint8, device=dev).fill_(1)
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    dst.copy_(src)
    torch.cuda.synchronize()
    del src, dst


def main() -> int:
    args = parse_args()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(f"bench.py measures one GPU only (asked for --gpus {args.gpus}, WORLD_SIZE {world}): "
              "the library has no multi-GPU path; decode shards by sequence or kv head with no "
              "exchange, so the per-GPU rate is the number to read.", file=sys.stderr)
        return 2

    import numpy as np
    import torch

    import gated_gqa_decode_amd as ga
    import workloads

    dev = torch.device("cuda:0")
    hip = Hip()
    K, W = args.steps, args.warmup

    if args.prefill_only:
        print(json.dumps({"prefill": time_prefill(ga, workloads.workload(4), dev, K,
                                                  settle_s=args.settle_s)}), flush=True)
        return 0
    if args.calibration_copy:
        calibration_copy(dev)
    if args.only == "b1_l512":
        print(json.dumps({args.only: graph_latency(ga, workloads.workload(0, poison=False), dev)}),
              flush=True)
        return 0
    if args.only == "qk_norm_rope_t4096":
        print(json.dumps({args.only: time_qk_norm_rope(ga, workloads, dev, 4096, False, K)}),
              flush=True)
        return 0
    if args.only:
        extra = only_case(workloads, args.only)
        print(json.dumps({args.only: time_decode(ga, extra, dev, K, settle_s=args.settle_s)}),
              flush=True)
        return 0

    # ---------------- headline: B=64, L=4096 paged decode --------------------
    t_gen = time.time()
    case = workloads.workload(2, poison=False)
    gen_s = time.time() - t_gen
    kv_bytes = case.kv_bytes()
    n_sets = rotation_sets(kv_bytes)
    call = Rotation(lambda: DecodeCall(ga, case, dev), n_sets)
    torch.cuda.synchronize()

    # Clock settling: the first few milliseconds of work after idle run at a
    # lower clock (20 warm-up calls left the next 200 at 100.6 us/call vs a
    # steady 90.3), so untimed calls run for settle_s seconds first.
    settle_calls = 0
    t_settle = time.perf_counter()
    while time.perf_counter() - t_settle < args.settle_s:
        for _ in range(50):
            call()
        torch.cuda.synchronize()
        settle_calls += 50
    settle_s = time.perf_counter() - t_settle

    for _ in range(W):
        call()
    torch.cuda.synchronize()

    # Timed steps: back-to-back calls, nothing else on the stream.
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    e0.record()
    for _ in range(K):
        call()
    e1.record()
    torch.cuda.synchronize()
    total_ms = e0.elapsed_time(e1)

    # Stage-1 duration: K launches of the stage-1 kernel alone, chained in one
    # graph with an event recorded before and after each (Stage1Graphs).
    s1 = Stage1Graphs(hip, call.calls, dev)
    kernel_ms = s1.time(K)
    s1.close()
    census = call_graph_census(hip, call.calls[0], dev)
    pcall = PrefillCall(ga, workloads.workload(4), dev)
    census_prefill = call_graph_census(hip, pcall, dev)
    del pcall

    ms_per_step = total_ms / K
    value = kv_bytes / (ms_per_step * 1e-3) / 1e9
    k_mean = statistics.fmean(kernel_ms)
    achieved = kv_bytes / (k_mean * 1e-3) / 1e9
    traffic = None
    counters = None
    if os.path.exists(COUNTERS):
        with open(COUNTERS) as f:
            counters = json.load(f)
        if counters.get("kernel_sources_sha256") == kernel_source_hash():
            traffic = counters.get("hbm_bytes_per_launch")

    result = {
        "metric": METRIC,
        "value": round(value, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": W,
        "ms_per_step": round(ms_per_step, 6),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "accumulate_dtype": "fp32",
        "data": "synthetic",
        "config": {
            "workload": "gated GQA decode B=64 L=4096, paged bf16 KV (16-token pages, shuffled), "
                        "H_q=16 H_kv=2 D=256",
            "batch": 64, "kv_len": 4096, "num_q_heads": 16, "num_kv_heads": 2, "head_dim": 256,
            "page_size": 16, "tokens_per_split": call.plan.tokens_per_split,
            "num_splits": call.plan.num_splits, "input_sets": n_sets,
        },
        "us_per_call": round(ms_per_step * 1e3, 3),
        "kv_bytes_per_call": kv_bytes,
        "hbm_frac": round(value / HBM_PEAK_GBS, 4),
        "launches_per_call": census["kernels"],
        "launch_census": {"decode": census, "prefill": census_prefill},
        "roofline": {
            "kernel": "decode_stage1_kernel",
            "bound": "hbm",
            "achieved": round(achieved, 2),
            "peak": HBM_PEAK_GBS,
            "unit": "GB/s",
            "frac": round(achieved / HBM_PEAK_GBS, 4),
            "traffic": traffic,
            "algorithmic_bytes_per_launch": kv_bytes,
            "avg_launch_us": round(k_mean * 1e3, 3),
            "launches_timed": K,
        },
    }

    if not args.no_extras:
        # ---- cold: each call after a 1 GiB flush (outside the timed span) ----
        flush = torch.empty(1 << 30, dtype=torch.uint8, device=dev)
        cold = []
        for _ in range(31):
            flush.fill_(0)
            a = torch.cuda.Event(enable_timing=True)
            b = torch.cuda.Event(enable_timing=True)
            a.record()
            call()
            b.record()
            torch.cuda.synchronize()
            cold.append(a.elapsed_time(b))
        del flush
        cold_ms = statistics.median(cold)
        result["cold"] = {"us_per_call": round(cold_ms * 1e3, 3),
                          "gbs": round(kv_bytes / (cold_ms * 1e-3) / 1e9, 2),
                          "hbm_frac": round(kv_bytes / (cold_ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
                          "samples": 31, "flush_bytes": 1 << 30}

        # ---- latency pair: B=1 L=512 and B=4 ragged, graph replays -----------
        small = workloads.workload(0, poison=False)
        result["b1_l512"] = graph_latency(ga, small, dev)
        result["b1_l512"]["cold"] = cold_latency(ga, small, dev)
        result["b4_ragged"] = graph_latency(ga, workloads.workload(1, poison=False), dev)
        result["launch_floor"] = launch_floor(dev)

        result["prefill"] = time_prefill(ga, workloads.workload(4), dev, 50, settle_s=0.3)

        # ---- the h_q = 32, h_kv = 2 geometry (GQA group 16) -----------------
        # the serving shape: B=224, L ~ U{4094..6142}, 11 padded slots (HBM-bound)
        c224 = only_case(workloads, "decode_b224")
        result["decode_b224"] = time_decode(ga, c224, dev, 50)
        del c224
        # a plain device-wide read of 1 GiB (a reduction, two buffers in turn):
        # the streaming-read rate the decode's KV GB/s can be set beside
        result["stream_read_ceiling"] = stream_read_ceiling(ga, dev)
        c32 = only_case(workloads, "decode_hq32")
        result["decode_hq32"] = time_decode(ga, c32, dev, 100)
        # attention-spec options on the headline workload
        result["decode_sinks_lse"] = time_decode(ga, case, dev, 100, sinks=[0.5] * 16, lse=True)
        result["decode_window1024"] = time_decode(ga, case, dev, 100, window=1024, lse=True)
        # sequences far shorter than the capacity the call was planned for
        short = workloads.make_decode("decode_b64_l1024_cap32768", [1024] * 64, seed=2,
                                      poison=False, max_pages_per_seq=2048, extra_pages=0)
        result["decode_l1024_cap32768"] = time_decode(ga, short, dev, 100)
        del short
        result["qk_norm_rope_decode_t64"] = time_qk_norm_rope(ga, workloads, dev, 64, True)
        result["qk_norm_rope_prefill_t4096"] = time_qk_norm_rope(ga, workloads, dev, 4096, False)
        # page size 1 with CSR indexing (the FreeToken PR's serving layout)
        result["decode_csr"] = time_decode_csr(ga, workloads, case, dev, 200)
        # FP8 (e4m3) K / V pools, same shape as the headline
        c8 = only_case(workloads, "decode_fp8kv")
        result["decode_fp8kv"] = time_decode(ga, c8, dev, 200)
        result["decode_fp8kv"]["stage1_traffic"] = fp8_stage1_traffic()
        del c8
        del c32
        p32 = workloads.make_prefill("prefill_b2_s2048_hq32", 2, 2048, seed=4, causal=True,
                                     num_q_heads=32, num_kv_heads=2)
        result["prefill_hq32"] = time_prefill(ga, p32, dev, 25, settle_s=0.3)
        del p32

    if not args.no_cpu_baseline and not args.no_extras:
        import oracle

        # The oracle as it stands, on the same B=64 workload, repeated until
        # about 12 thread-seconds of CPU work have been done, on every core of
        # the affinity mask within the process's CPU share.
        threads = oracle.default_threads()
        reps, busy = 0, 0.0
        t = time.time()
        while reps == 0 or busy * threads < 12.0:
            oracle.decode(case.q, case.gate, case.k_pool, case.v_pool, case.block_table,
                          case.seq_lens, case.scale, nthreads=threads)
            reps += 1
            busy = time.time() - t
        result["cpu_baseline"] = {
            "value": round(reps * kv_bytes / busy / 1e9, 4), "unit": "GB/s",
            "cores": threads, "kind": "oracle",
            "sample": f"the whole B=64 L=4096 workload, {reps} call(s) "
                      f"({busy:.2f} s wall, fp64, {threads} threads)",
            "seconds_per_call": round(busy / reps, 3),
            "affinity_cores": oracle.affinity_cores(),
            "cpu_share": oracle.cpu_share(),
            "cpu_model": oracle.cpu_model()}

        # and one thread on each latency workload (B=1 L=512, B=4 ragged)
        def one_thread_ms(c) -> float:
            n, t0 = 0, time.time()
            while n == 0 or time.time() - t0 < 0.5:
                oracle.decode(c.q, c.gate, c.k_pool, c.v_pool, c.block_table, c.seq_lens,
                              c.scale, nthreads=1)
                n += 1
            return round((time.time() - t0) / n * 1e3, 3)
        result["cpu_baseline"]["b1_l512_one_thread_ms"] = one_thread_ms(workloads.workload(0, poison=False))
        result["cpu_baseline"]["b4_ragged_one_thread_ms"] = one_thread_ms(workloads.workload(1, poison=False))
    result["settle"] = {"seconds": round(settle_s, 3), "calls": settle_calls}
    result["input_generation_s"] = round(gen_s, 2)
    line = json.dumps(result)
    print(line, flush=True)
    if args.json_out:
        with open(args.json_out, "w") as f:
            f.write(line + "\n")
    return 0


if __name__ == "__main__":
    sys.exit(main())
