"""Decode-attention benchmark on one MI355X.

One step = one complete decode call (split kernel + combine kernel) over one
batch of the headline workload, the largest configuration that fits one GPU:
long-context paged f16 decode, 4 sequences of 131072 tokens, 64 query / 8 kv
heads, head_dim 128, block size 64, block table a random permutation of a
shared pool, f16 K/V ~ N(0,1), f32 Q, scale 1/sqrt(128), causal (2.15 GB of KV
per call).  Inputs are seeded and synthetic and are resident in HBM before
timing starts; caches smaller than 1 GB are rotated over enough copies that
consecutive steps cannot hit the 256 MB Infinity Cache.

Prints one JSON line.  `value` is KV-read GB/s: algorithmic K+V bytes of the
visible (token, kv_head) rows, each read once per (sequence, kv head), divided
by the wall time per step over the K timed steps.  `roofline` prices the
dominant (split) kernel against MI355X HBM peak with its event-timed duration;
`cpu_baseline` times the fp64 oracle on this host's cores over the same
workload.  `workloads` holds one line per configuration (tiny, paged f16,
tiered int8 at windows 0 and 4096, block-sparse; with --all also the other
caches): step time as median and p10/p90 over >= 50 timed calls, the split
kernel's rate and roofline fraction, the whole output compared with the oracle
element by element, and the oracle's own time on this host.
"""
from __future__ import annotations

import argparse
import ctypes
import dataclasses
import glob
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

import numpy as np  # noqa: E402

HBM_PEAK_GBS = 8000.0
MALL_BYTES = 1.0e9     # rotate cache copies until each step touches new memory
KERNEL_SOURCES = [os.path.join(ROOT, "int8_quantized_kv_amd", "csrc", f) for f in ("decode_kernels.h", "dattn.hip")]
TRAFFIC_GLOB = os.path.join(ROOT, "profiles", "traffic_*.txt")
SAMPLES = 50           # timed calls (batches of back-to-back calls) for the step-time distribution
SAMPLE_US = 500.0      # target GPU time of one sample's batch
# the configurations, as (label, workload index, window)
CONFIGS = [("tiny", 1, 0), ("paged_f16", 2, 0), ("tiered_int8_w0", 3, 0), ("tiered_int8_w4096", 3, 4096),
           ("long_paged_f16", 4, 0), ("block_sparse", 5, 0)]
HEADLINE = 4
# the oracle on one thread, on a bounded sample of sequences (all heads of each)
ONE_THREAD_SEQS = {1: 1, 2: 4, 5: 8}


def log(msg):
    print(msg, file=sys.stderr, flush=True)


# --------------------------------------------------------------- bytes

def visible_range(case, b):
    p = case.params
    L = int(case.seq_lens[b])
    qn = max(1, p.get("query_len", 1))
    q = int(case.q_pos[b]) if case.q_pos is not None else L - qn
    hi = min(q + qn - 1, L - 1) if p["causal"] else L - 1
    W = p["sliding_window"]
    lo = q - W + 1 if (W > 0 and q >= W) else 0
    if case.kind == "ring":
        lo = max(lo, L - case.hot_window)
    return lo, hi, q


def kv_bytes(case, seqs=None) -> int:
    """Algorithmic KV bytes of one decode call: K + V (+ int8 scales) of each visible
    (token, kv head) row once per (sequence, kv head) -- with several queries per
    sequence, a row visible to any of them; for the block-sparse cache a row counts
    once for the union of the blocks its GQA group selects.  `seqs` restricts the
    count to some sequences."""
    p = case.params
    B, H, Hkv, D = p["num_seqs"], p["num_heads"], p["num_kv_heads"], p["head_dim"]
    G = H // Hkv
    total = 0
    for b in (range(B) if seqs is None else seqs):
        lo, hi, q = visible_range(case, b)
        if hi < lo:
            continue
        if case.kind == "paged":
            esz = case.k_cache.dtype.itemsize
            total += (hi - lo + 1) * Hkv * 2 * D * esz
        elif case.kind in ("tiered_f16", "ring"):
            total += (hi - lo + 1) * Hkv * 2 * D * 2
        elif case.kind == "tiered":
            c = int(case.cold_lens[b])
            ncold = max(0, min(hi, c - 1) - lo + 1)
            nhot = (hi - lo + 1) - ncold
            total += ncold * Hkv * 2 * (D + 2) + nhot * Hkv * 2 * D * 2
        else:
            SB = case.sparse_block
            rows = sorted({(q + i) // SB for i in range(max(1, p.get("query_len", 1))) if q + i >= 0})
            for g in range(Hkv):
                union = set()
                for j in range(G):
                    lay = (g * G + j) % case.num_layouts
                    for r in rows:
                        s, e = case.row_ptr[lay, r], case.row_ptr[lay, r + 1]
                        union |= {int(c) for c in case.col_idx[lay, s:e] if 0 <= c <= r}
                for blk in union:
                    t0, t1 = max(lo, blk * SB), min(hi, blk * SB + SB - 1)
                    if t1 >= t0:
                        total += (t1 - t0 + 1) * 2 * D * 2
    return total


# ------------------------------------------------------------ device side

class Runner:
    """Device copies of a case (caches rotated over `copies` replicas) and
    prebuilt ctypes argument lists for split-only, combine-only and full calls."""

    def __init__(self, case, copies):
        import torch
        import int8_quantized_kv_amd as dk
        self.dk = dk
        self.case = case
        dev = "cuda:0"

        def T(a):
            a = np.ascontiguousarray(a)
            if a.dtype == np.uint32:
                a = a.view(np.int32)
            return torch.from_numpy(a).to(dev)

        c = case
        p = c.params
        self.q = T(c.q)
        self.seq_lens = T(c.seq_lens)
        self.q_pos = T(c.q_pos) if c.q_pos is not None else None
        B, H, D = c.q.shape[0], c.q.shape[-2], c.q.shape[-1]
        qn = max(1, p.get("query_len", 1))
        self.out = torch.empty(c.q.shape, dtype=torch.float32, device=dev)
        self.lse = torch.empty(c.q.shape[:-1], dtype=torch.float32, device=dev)
        max_len = int(c.seq_lens.max())
        if c.kind in ("tiered", "tiered_f16"):
            NB, bs = c.k_cold.shape[0], c.k_cold.shape[1]
            mb = c.cold_block_table.shape[1]
            kind = dk.KIND_TIERED_INT8 if c.kind == "tiered" else dk.KIND_TIERED_F16
        elif c.kind == "ring":
            NB, bs, mb, kind = 1, 1, 1, dk.KIND_RING_F16
        else:
            NB, bs = c.k_cache.shape[0], c.k_cache.shape[1]
            mb = c.block_table.shape[1]
            kind = dk.KIND_PAGED if c.kind == "paged" else dk.KIND_BLOCK_SPARSE

        def params(phases):
            return dk.DattnParams(B, H, p["num_kv_heads"], D, p["scale"], p["causal"], p["sliding_window"],
                                  p["softcap"], bs, mb, NB, max_len, 0, phases, dk.F32, qn)

        self.p_all, self.p_split, self.p_comb = params(0), params(dk.PHASE_SPLIT), params(dk.PHASE_COMBINE)
        ws = dk.dattn_workspace_size(self.p_all, kind, c.sparse_block)
        self.ws = torch.empty((ws,), dtype=torch.uint8, device=dev)
        self.stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
        L = dk.lib()
        P = lambda t: ctypes.c_void_p(t.data_ptr()) if t is not None else None  # noqa: E731
        self.calls = []
        if c.kind == "paged" or c.kind == "sparse":
            k0, v0, tbl = T(c.k_cache), T(c.v_cache), T(c.block_table)
            ks = [k0] + [k0.clone() for _ in range(copies - 1)]
            vs = [v0] + [v0.clone() for _ in range(copies - 1)]
            self.keep = (ks, vs, tbl)
            if c.kind == "paged":
                dt = dk.F16 if c.k_cache.dtype == np.float16 else dk.F32
                for k, v in zip(ks, vs):
                    rest = (P(self.q), P(k), P(v), dt, P(tbl), P(self.seq_lens), P(self.q_pos), P(self.out),
                            P(self.lse), P(self.ws), self.ws.numel(), self.stream)
                    self.calls.append(rest)
                self.fn = L.dattn_decode_paged
            else:
                rp, ci = T(c.row_ptr), T(c.col_idx)
                self.keep = self.keep + (rp, ci)
                for k, v in zip(ks, vs):
                    rest = (P(self.q), P(k), P(v), P(tbl), P(self.seq_lens), P(self.q_pos), c.sparse_block,
                            c.num_layouts, P(rp), c.row_ptr.shape[1], P(ci), c.col_idx.shape[1], P(self.out),
                            P(self.lse), P(self.ws), self.ws.numel(), self.stream)
                    self.calls.append(rest)
                self.fn = L.dattn_decode_block_sparse
        elif c.kind == "ring":
            kr0, vr0 = T(c.k_hot), T(c.v_hot)
            reps = [(kr0, vr0)] + [(kr0.clone(), vr0.clone()) for _ in range(copies - 1)]
            self.keep = reps
            for (kr, vr) in reps:
                self.calls.append((P(self.q), P(kr), P(vr), P(self.seq_lens), P(self.q_pos), P(self.out),
                                   P(self.lse), P(self.ws), self.ws.numel(), self.stream))
            self.fn = L.dattn_decode_ring_f16
        elif c.kind == "tiered_f16":
            kh, vh, kc0, vc0 = T(c.k_hot), T(c.v_hot), T(c.k_cold), T(c.v_cold)
            tbl, cl = T(c.cold_block_table), T(c.cold_lens)
            reps = [(kh, vh, kc0, vc0)] + [tuple(x.clone() for x in (kh, vh, kc0, vc0)) for _ in range(copies - 1)]
            self.keep = (reps, tbl, cl)
            for (a, b_, kc, vc) in reps:
                rest = (P(self.q), P(a), P(b_), c.hot_window, P(kc), P(vc), P(tbl), P(self.seq_lens), P(cl),
                        P(self.q_pos), P(self.out), P(self.lse), P(self.ws), self.ws.numel(), self.stream)
                self.calls.append(rest)
            self.fn = L.dattn_decode_tiered_f16
        else:
            kh, vh, kc0, vc0 = T(c.k_hot), T(c.v_hot), T(c.k_cold), T(c.v_cold)
            ks0, vs0, tbl, cl = T(c.k_scale), T(c.v_scale), T(c.cold_block_table), T(c.cold_lens)
            reps = [(kh, vh, kc0, vc0, ks0, vs0)] + [tuple(x.clone() for x in (kh, vh, kc0, vc0, ks0, vs0))
                                                     for _ in range(copies - 1)]
            self.keep = (reps, tbl, cl)
            for (a, b_, kc, vc, ksc, vsc) in reps:
                rest = (P(self.q), P(a), P(b_), c.hot_window, P(kc), P(vc), P(ksc), P(vsc), P(tbl),
                        P(self.seq_lens), P(cl), P(self.q_pos), P(self.out), P(self.lse), P(self.ws),
                        self.ws.numel(), self.stream)
                self.calls.append(rest)
            self.fn = L.dattn_decode_tiered_int8
        self.copies = copies

    def call(self, i, which):
        p = {"all": self.p_all, "split": self.p_split, "combine": self.p_comb}[which]
        rc = self.fn(ctypes.byref(p), *self.calls[i % self.copies])
        if rc != 0:
            raise RuntimeError(f"decode call failed: {rc} {self.dk.dattn_last_error()}")

    def result(self):
        import torch
        torch.cuda.synchronize()
        return self.out.cpu().numpy(), self.lse.cpu().numpy()


def cache_bytes(case):
    if case.kind == "tiered":
        arrs = (case.k_hot, case.v_hot, case.k_cold, case.v_cold, case.k_scale, case.v_scale)
    elif case.kind == "tiered_f16":
        arrs = (case.k_hot, case.v_hot, case.k_cold, case.v_cold)
    elif case.kind == "ring":
        arrs = (case.k_hot, case.v_hot)
    else:
        arrs = (case.k_cache, case.v_cache)
    return sum(a.nbytes for a in arrs)


def sample_times(r, est_us, n=SAMPLES):
    """Step-time distribution: n samples, each a batch of back-to-back full calls
    between two HIP events on the launch stream (consecutive samples share an
    event), sized to about SAMPLE_US of GPU time so that the event's own cost is
    spread over the batch.  Returns per-call microseconds (median, p10, p90)."""
    import torch
    per = max(1, min(64, int(math.ceil(SAMPLE_US / max(est_us, 1.0)))))
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(n + 1)]
    i = 0
    ev[0].record()
    for s in range(n):
        for _ in range(per):
            r.call(i, "all")
            i += 1
        ev[s + 1].record()
    torch.cuda.synchronize()
    us = np.array([ev[s].elapsed_time(ev[s + 1]) * 1e3 / per for s in range(n)])
    return dict(samples=n, calls_per_sample=per, timed_calls=n * per, median_us=round(float(np.median(us)), 3),
                p10_us=round(float(np.percentile(us, 10)), 3), p90_us=round(float(np.percentile(us, 90)), 3))


WARM_MS = 30.0   # the device's clock needs about this much busy time to settle


def preheat(r, ms):
    """About `ms` of the library's streaming-read kernel over the runner's first
    cache tensor (the bytes the calls read, uploaded just before): the device's
    clock settles during it, after the idle spell of the upload."""
    import torch
    import int8_quantized_kv_amd as dk
    def tensors(x):
        if isinstance(x, (list, tuple)):
            for y in x:
                yield from tensors(y)
        elif isinstance(x, torch.Tensor):
            yield x
    src = max(tensors(r.keep), key=lambda t: t.numel() * t.element_size())
    sink = torch.zeros(1, dtype=torch.int32, device="cuda:0")
    t0 = time.perf_counter()
    while (time.perf_counter() - t0) * 1e3 < ms:
        for _ in range(4):
            dk.dattn_stream_read(src, sink)
        torch.cuda.synchronize()


def measure(case, steps, warmup, copies=None, warm_ms=0.0, preheat_ms=0.0):
    """Time `steps` full calls (wall clock, inputs resident), then event-timed
    split-only and combine-only calls on the same stream right after them, then
    the step-time distribution over >= SAMPLES timed calls, then graph replay.
    The `warmup` untimed calls come first; with warm_ms > 0 more untimed calls
    follow them until about warm_ms of wall time has passed.  preheat_ms > 0:
    that much of the streaming-read kernel over the uploaded cache runs before
    the warm-up calls."""
    import torch
    if copies is None:
        copies = max(1, int(math.ceil(MALL_BYTES / max(cache_bytes(case), 1))))
    r = Runner(case, copies)
    if preheat_ms > 0:
        preheat(r, preheat_ms)
    for i in range(warmup):
        r.call(i, "all")
    torch.cuda.synchronize()
    tw, i = time.perf_counter(), warmup
    while (time.perf_counter() - tw) * 1e3 < warm_ms:
        for _ in range(10):
            r.call(i, "all")
            i += 1
        torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(steps):
        r.call(i, "all")
    torch.cuda.synchronize()
    wall = (time.perf_counter() - t0) / steps
    # Per-kernel durations, right after the timed steps: back-to-back launches of
    # one phase between two events recorded on the launch stream (events around
    # a single launch would add the dispatch overhead of that launch to every
    # sample).
    nk = max(steps, SAMPLES)
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(3)]
    ev[0].record()
    for i in range(nk):
        r.call(i, "split")
    ev[1].record()
    for i in range(nk):
        r.call(i, "combine")
    ev[2].record()
    torch.cuda.synchronize()
    split_ms = ev[0].elapsed_time(ev[1]) / nk
    comb_ms = ev[1].elapsed_time(ev[2]) / nk
    dist = sample_times(r, wall * 1e6)
    # the timed region's result (the last full call wrote out / lse; split- and
    # combine-only calls of identical parameters leave the same values)
    out, lse = r.result()
    graph_ms = graph_call_ms(r)
    return dict(wall_s=wall, split_ms=split_ms, combine_ms=comb_ms, copies=copies, graph_ms=graph_ms, dist=dist,
                kernel_launches=nk, out=out, lse=lse)


def measure_append(B=16, Hkv=8, D=128, hot_window=512, bs=16, calls=200, warmup=20):
    """The tiered write path in its steady state: every sequence's ring is full, so
    each call quantises one token per (sequence, kv head) into the cold tier and
    writes the new token to the ring.  Times `calls` back-to-back calls between two
    HIP events on the current stream."""
    import torch
    import int8_quantized_kv_amd as dk
    g = torch.Generator(device="cpu").manual_seed(9)
    dev = "cuda:0"
    total = calls + warmup
    max_blocks = total // bs + 2
    nb = B * max_blocks
    k_hot = torch.randn(B, hot_window, Hkv, D, generator=g).half().to(dev)
    v_hot = torch.randn(B, hot_window, Hkv, D, generator=g).half().to(dev)
    k_new = torch.randn(total, B, Hkv, D, generator=g).half().to(dev)
    v_new = torch.randn(total, B, Hkv, D, generator=g).half().to(dev)
    k_cold = torch.zeros(nb, bs, Hkv, D // 4, dtype=torch.int32, device=dev)
    v_cold = torch.zeros_like(k_cold)
    k_sc = torch.zeros(nb, bs, Hkv, dtype=torch.float16, device=dev)
    v_sc = torch.zeros_like(k_sc)
    table = torch.randperm(nb, generator=g).to(torch.int32).reshape(B, max_blocks).to(dev)
    seq = torch.full((B,), hot_window, dtype=torch.int32, device=dev)
    cold = torch.zeros(B, dtype=torch.int32, device=dev)
    args = (k_hot, v_hot, k_cold, v_cold, k_sc, v_sc, table, seq, cold)
    for i in range(warmup):
        dk.dattn_append_tiered_int8(k_new[i], v_new[i], *args)
    # One call is a few microseconds of GPU work but more of host enqueue, so the
    # GPU is first given a backlog of copies; the calls then queue up behind it and
    # run back to back, and the events bracket GPU time only.
    src = torch.empty(256 << 20, dtype=torch.uint8, device=dev)
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    for i in range(warmup, total):
        dk.dattn_append_tiered_int8(k_new[i], v_new[i], *args)
    torch.cuda.synchronize()
    host_us = (time.perf_counter() - t0) * 1e6 / calls
    seq.fill_(hot_window); cold.zero_()
    for i in range(warmup):
        dk.dattn_append_tiered_int8(k_new[i], v_new[i], *args)
    for _ in range(max(4, int(host_us * calls / 40))):   # each 256 MiB copy is ~80 us
        dst.copy_(src)
    e0.record()
    for i in range(warmup, total):
        dk.dattn_append_tiered_int8(k_new[i], v_new[i], *args)
    e1.record()
    torch.cuda.synchronize()
    assert int(cold[0]) == total and int(seq[0]) == hot_window + total
    us = e0.elapsed_time(e1) * 1e3 / calls
    # per (sequence, kv head): new K, V read; evicted K, V read; codes + scales written; ring written
    nbytes = B * Hkv * (2 * D * 2 + 2 * D * 2 + 2 * (D + 2) + 2 * D * 2)
    return dict(workload=f"append_evict_tiered_int8_B{B}_Hkv{Hkv}_D{D}_hw{hot_window}", us_per_call=round(us, 3),
                host_us_per_call=round(host_us, 3), bytes_per_call=nbytes, gbs=round(nbytes / us / 1e3, 2))


def kernel_source_sha():
    """sha256 over the kernel source and the host planner (worker counts and
    splits change the bytes a launch moves), concatenated in that order."""
    import hashlib
    h = hashlib.sha256()
    for path in KERNEL_SOURCES:
        h.update(open(path, "rb").read())
    return h.hexdigest()


def measured_traffic(workload):
    """HBM bytes per launch of the workload's split kernel from its committed
    counter summary (FETCH_SIZE + WRITE_SIZE, scaled by a copy kernel of known
    size), or None when there is none or it was taken on another kernel source."""
    sha = kernel_source_sha()
    for path in sorted(glob.glob(TRAFFIC_GLOB)):
        try:
            t = json.load(open(path))
        except (OSError, ValueError):
            continue
        if t.get("workload") == workload and t.get("kernel_source_sha256") == sha:
            return t.get("hbm_bytes_per_launch")
    return None


def copy_calibration(mib):
    """A plain streaming kernel of known traffic for scaling the FETCH_SIZE and
    WRITE_SIZE counters: torch.neg over `mib` MiB of float32 reads and writes
    exactly mib MiB each (5 launches)."""
    import torch
    src = torch.ones((mib << 20) // 4, dtype=torch.float32, device="cuda:0")
    dst = torch.empty_like(src)
    for _ in range(5):
        torch.neg(src, out=dst)
    torch.cuda.synchronize()
    log(f"copy calibration: 5 x torch.neg over {mib} MiB float32")


def graph_call_ms(r, reps=20):
    """Full calls (split + combine), one per cache copy, captured into a HIP graph and
    replayed `reps` times back to back: a call's GPU time without host-side enqueue
    cost.  Runs last: afterwards the runner's calls name the capture stream."""
    import torch
    n = min(r.copies, 64)   # the tiny workload has thousands of copies; 64 calls per graph suffice
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        r.stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
        r.calls = [c[:-1] + (r.stream,) for c in r.calls]
        for i in range(n):
            r.call(i, "all")
    g.replay()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(reps):
        g.replay()
    e1.record()
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / (reps * n)


def read_reference(nbytes=300 << 20, copies=4, reps=20):
    """Read GB/s of the library's plain streaming-read kernel (128-bit nontemporal
    loads) over buffers rotated past the Infinity Cache: the measured read ceiling
    for launches that read `nbytes` each (a launch's fixed cost weighs more on
    smaller launches)."""
    import torch
    import int8_quantized_kv_amd as dk
    srcs = [torch.ones(nbytes // 4, dtype=torch.float32, device="cuda:0") for _ in range(copies)]
    sink = torch.zeros(1, dtype=torch.int32, device="cuda:0")
    for x in srcs:
        dk.dattn_stream_read(x, sink)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for i in range(reps):
        dk.dattn_stream_read(srcs[i % copies], sink)
    e1.record()
    torch.cuda.synchronize()
    return round(nbytes * reps / (e0.elapsed_time(e1) / 1e3) / 1e9, 1)


def cpu_model():
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def copy_reference(nbytes=300 << 20, copies=4, reps=20):
    """Read + write GB/s of torch.neg over float32 buffers rotated past the Infinity
    Cache: what a plain streaming elementwise kernel reaches on this GPU."""
    import torch
    srcs = [torch.ones(nbytes // 4, dtype=torch.float32, device="cuda:0") for _ in range(copies)]
    dsts = [torch.empty_like(x) for x in srcs]
    for a, b in zip(srcs, dsts):
        torch.neg(a, out=b)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for i in range(reps):
        torch.neg(srcs[i % copies], out=dsts[i % copies])
    e1.record()
    torch.cuda.synchronize()
    return round(2 * nbytes * reps / (e0.elapsed_time(e1) / 1e3) / 1e9, 1)


def with_window(case, window):
    """The same cache and queries with another sliding window (the tiered
    configuration runs at two windows over identical data)."""
    p = dict(case.params, sliding_window=int(window))
    name = case.name.replace("_W0_", f"_W{window}_") if "_W0_" in case.name else f"{case.name}_W{window}"
    return dataclasses.replace(case, params=p, name=name)


def seq_pairs(case, seqs):
    """Flat (sequence, query, head) row indices of every row of the given sequences."""
    p = case.params
    rows = max(1, p.get("query_len", 1)) * p["num_heads"]
    return np.concatenate([np.arange(b * rows, (b + 1) * rows) for b in seqs]).astype(np.int32)


def oracle_leg(case, min_seconds=0.0, nthreads=0, seqs=None):
    """The fp64 oracle (as it stands) over all rows of the given sequences (all of
    them by default), repeated until at least min_seconds have passed (once at
    least).  Returns (out, lse) of the first run and the timing in the GPU line's
    units: algorithmic KV GB/s of those sequences and sequences (query tokens) per
    second."""
    import oracle
    pairs = None if seqs is None else seq_pairs(case, seqs)
    nseq = case.params["num_seqs"] if seqs is None else len(seqs)
    reps, t0, res = 0, time.perf_counter(), None
    while True:
        r = oracle.run(case, pairs=pairs, nthreads=nthreads)
        res = res or r
        reps += 1
        el = time.perf_counter() - t0
        if el >= min_seconds:
            break
    kvb = kv_bytes(case, seqs)
    threads = nthreads if nthreads > 0 else int(oracle.max_threads())
    what = "whole workload" if seqs is None else f"all rows of {nseq} of {case.params['num_seqs']} sequences"
    qn = max(1, case.params.get("query_len", 1))
    timing = dict(value=round(kvb * reps / el / 1e9, 4), unit="GB/s", cores=threads, kind="oracle",
                  queries_per_s=round(nseq * qn * reps / el, 2), seconds_per_run=round(el / reps, 4),
                  sample=f"{what} ({case.name}), {reps} run(s) in {el:.1f} s, fp64, "
                         f"OpenMP over (sequence, head) rows on {threads} thread(s)")
    return res, timing


def parity(out, lse, ref_o, ref_l):
    """Every output element and every lse against the oracle, at the tolerance the
    tests use: max abs error <= 1e-3 and <= 1e-3 of max |reference| (normwise),
    lse within 1e-3; rows with no visible key must be exactly (0, -inf)."""
    out = np.asarray(out, np.float64).reshape(ref_o.shape)
    lse = np.asarray(lse, np.float64).reshape(ref_l.shape)
    empty = ~np.isfinite(ref_l)
    ok = bool(np.all(lse[empty] == -np.inf) and np.all(out[empty] == 0.0))
    full = ~empty
    err = float(np.max(np.abs(out[full] - ref_o[full]))) if full.any() else 0.0
    ref = float(np.max(np.abs(ref_o[full]))) if full.any() else 1.0
    lerr = float(np.max(np.abs(lse[full] - ref_l[full]))) if full.any() else 0.0
    ok = ok and bool(np.all(np.isfinite(out[full]))) and err <= 1e-3 and err <= 1e-3 * ref and lerr <= 1e-3
    return dict(rows=int(ref_l.size), max_abs_err=err, normwise_rel_err=err / max(ref, 1e-30), lse_err=lerr, ok=ok)


def line_for(case, steps, warmup, label=None, oracle_seconds=0.0, one_thread_seqs=None, check=True, warm_ms=0.0,
             preheat_ms=0.0):
    """One configuration: timing, split-kernel roofline, whole-output parity and
    the oracle's own time on this host (check=False: timing only)."""
    kvb = kv_bytes(case)
    m = measure(case, steps, warmup, warm_ms=warm_ms, preheat_ms=preheat_ms)
    nq = case.params["num_seqs"] * max(1, case.params.get("query_len", 1))   # query tokens per call
    split_gbs = kvb / (m["split_ms"] / 1e3) / 1e9
    res = dict(config=label, workload=case.name, kv_bytes=kvb, ms_per_call=round(m["wall_s"] * 1e3, 5),
               kv_gbs=round(kvb / m["wall_s"] / 1e9, 2), pct_peak=round(100 * kvb / m["wall_s"] / 1e9 / HBM_PEAK_GBS, 2),
               queries_per_s=round(nq / m["wall_s"], 1), step_us=m["dist"],
               step_median_gbs=round(kvb / (m["dist"]["median_us"] / 1e6) / 1e9, 2),
               split_ms=round(m["split_ms"], 5), combine_ms=round(m["combine_ms"], 5),
               split_gbs=round(split_gbs, 2), split_roofline_frac=round(split_gbs / HBM_PEAK_GBS, 4),
               split_traffic=measured_traffic(case.name), kernel_launches=m["kernel_launches"],
               graph_ms_per_call=round(m["graph_ms"], 5), cache_copies=m["copies"])
    if not check:
        return res, m
    (ro, rl), timing = oracle_leg(case, oracle_seconds)
    res["parity"] = parity(m["out"], m["lse"], ro, rl)
    res["oracle"] = timing
    if one_thread_seqs:
        _, t1 = oracle_leg(case, 0.0, nthreads=1, seqs=list(range(one_thread_seqs)))
        res["oracle_1thread"] = t1
    return res, m


def workload(idx, window=0):
    """Workloads 1-5 of the input generators, 6: the tiered workload's shape
    with an f16 cold tier, 7: a sliding-window ring f16 cache, 8 and 9: four
    and sixteen queries per sequence over a paged f16 cache of workload 2's
    shape, 10: four queries per sequence over the block-sparse workload, 11: four
    over the tiered int8 workload."""
    import synth
    if idx == 6:
        return synth.tiered_f16_workload(window)
    if idx == 7:
        return synth.ring_workload()
    if idx == 8:
        return synth.multi_query_workload(4)
    if idx == 9:
        return synth.multi_query_workload(16)
    if idx == 10:
        return synth.sparse_multi_query_workload(4)
    if idx == 11:
        return synth.tiered_multi_query_workload(4)
    return synth.workload(idx, window=window)


def config_case(idx, window, cache):
    """The configuration's case; the tiered data is generated once for both windows."""
    if idx == 3:
        if "tiered" not in cache:
            cache["tiered"] = workload(3)
        return with_window(cache["tiered"], window)
    return workload(idx, window=window)


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=200,
                    help="untimed calls first (about 64 ms of the headline workload; after 10 the clock is still "
                         "ramping and the timed steps run 2-3%% slower)")
    ap.add_argument("--all", action="store_true", help="also measure the other caches' workloads (6-10)")
    ap.add_argument("--only", action="store_true",
                    help="measure the headline workload alone (no other lines, write path or CPU baseline)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--workload", type=int, default=HEADLINE,
                    help="headline workload index (default 4, the long-context paged f16 configuration; 1 tiny, "
                         "2 paged f16, 3 tiered int8, 5 block-sparse, 6 the tiered workload with an f16 cold tier, "
                         "7 a sliding-window ring f16 cache, 8 four queries per sequence, 9 sixteen, 10 four over "
                         "the block-sparse cache, 11 four over the tiered int8 cache)")
    ap.add_argument("--window", type=int, default=0, help="sliding window of the headline workload")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="MIB",
                    help="first run 5 device copies of MIB MiB (for scaling memory counters)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only (asked for --gpus {args.gpus}); the decode path here is the "
              f"single-GPU share. Run with --gpus 1.", file=sys.stderr)
        sys.exit(2)

    import torch
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    import int8_quantized_kv_amd as dk
    dk.lib()
    if args.copy_calibration:
        copy_calibration(args.copy_calibration)

    cache = {}
    log("generating headline workload ...")
    case = config_case(args.workload, args.window, cache)
    log(f"workload {case.name}: KV bytes {kv_bytes(case)}")
    base_s = 0.0 if (args.no_cpu_baseline or args.only) else 10.0
    # The headline's `warmup` calls follow about WARM_MS of the streaming-read kernel over the cache
    # just uploaded: the upload leaves the device idle, and a few warm-up calls alone time the timed
    # steps on a clock that is still ramping (2-4% slower).
    head, m = line_for(case, args.steps, args.warmup, label="headline", oracle_seconds=base_s,
                       one_thread_seqs=ONE_THREAD_SEQS.get(args.workload), check=not args.only, preheat_ms=WARM_MS)
    log(json.dumps(head))
    kvb = head["kv_bytes"]
    achieved = kvb / (m["split_ms"] / 1e3) / 1e9
    B, H, D = case.q.shape[0], case.q.shape[-2], case.q.shape[-1]
    G = H // case.params["num_kv_heads"]
    kind = {"paged": "paged f16" if case.k_cache is not None and case.k_cache.dtype == np.float16 else "paged f32",
            "tiered": "tiered int8 + f16 ring", "tiered_f16": "tiered f16 + f16 ring", "ring": "window ring f16",
            "sparse": "block-sparse f16"}[case.kind]
    lens = case.seq_lens
    out = {
        "metric": "KV-read HBM GB/s (% of peak) and decode queries/sec, 1 MI355X",
        "value": head["kv_gbs"],
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": head["ms_per_call"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f16",
        "data": "synthetic (seeded numpy N(0,1) Q/K/V, permuted block pool)",
        "config": {"workload": case.name, "global_batch": int(B), "num_heads": int(H),
                   "num_kv_heads": int(case.params["num_kv_heads"]), "head_dim": int(D),
                   "block_size": int(case.params["block_size"]), "sliding_window": int(case.params["sliding_window"]),
                   "seq_len_range": [int(lens.min()), int(lens.max())],
                   "total_tokens": int(lens.sum()), "parallelism": "single GPU"},
        "pct_of_hbm_peak": head["pct_peak"],
        "queries_per_s": head["queries_per_s"],
        "step_us": head["step_us"],
        "kernels": {"split_ms": head["split_ms"], "combine_ms": head["combine_ms"],
                    "graph_ms_per_call": head["graph_ms_per_call"], "launches_timed": head["kernel_launches"]},
        "roofline": {"bound": "hbm", "achieved": round(achieved, 2), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": head["split_traffic"],
                     "kernel": f"split kernel <D={D}, G={G}, {kind}>",
                     "bytes_per_launch": kvb},
    }
    if "parity" in head:
        out["parity"] = head["parity"]
    if not args.only:
        out["copy_reference_gbs"] = copy_reference()
        # the streaming ceiling at the headline's bytes per launch (at least 300 MB), and at 300 MB
        nb = max(kvb, 300 << 20) // 16 * 16
        ceiling = read_reference(nbytes=nb, copies=max(2, int(math.ceil(MALL_BYTES / nb))))
        out["roofline"]["measured_read_ceiling_gbs"] = ceiling
        out["roofline"]["frac_of_measured_ceiling"] = round(achieved / ceiling, 4)
        out["roofline"]["measured_read_ceiling_300mb_gbs"] = read_reference()
        log("timing the tiered write path ...")
        out["write_path"] = measure_append()
        if not args.no_cpu_baseline:
            out["cpu_baseline"] = head["oracle"]
            out["cpu_baseline"]["cpu_model"] = cpu_model()
        lines = []
        todo = [(label, idx, w) for label, idx, w in CONFIGS if (idx, w) != (args.workload, args.window)]
        if args.all:
            todo += [("tiered_f16_w0", 6, 0), ("tiered_f16_w4096", 6, 4096), ("ring_f16", 7, 0),
                     ("multi_query_4", 8, 0), ("multi_query_16", 9, 0), ("block_sparse_multi_query_4", 10, 0),
                     ("tiered_int8_multi_query_4", 11, 0)]
        for label, idx, w in todo:
            log(f"generating workload {idx} window {w} ...")
            c = config_case(idx, w, cache)
            # a small configuration's warm-up calls alone do not settle the clock
            res, _ = line_for(c, args.steps, args.warmup, label=label, one_thread_seqs=ONE_THREAD_SEQS.get(idx),
                              warm_ms=WARM_MS)
            # the plain streaming read at this line's KV bytes per launch: what a launch of that size reaches
            nbl = max(res["kv_bytes"], 1 << 20) // 16 * 16
            res["read_ceiling_gbs"] = read_reference(nbytes=nbl, copies=max(2, int(math.ceil(MALL_BYTES / nbl))),
                                                     reps=min(2000, max(20, int(math.ceil(0.005 * 7e12 / nbl)))))
            res["split_frac_of_read_ceiling"] = round(res["split_gbs"] / res["read_ceiling_gbs"], 4)
            log(json.dumps(res))
            lines.append(res)
            del c
        out["workloads"] = lines
        out["parity_all_ok"] = bool(head["parity"]["ok"] and all(x["parity"]["ok"] for x in lines))
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
