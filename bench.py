"""Decode-attention benchmark on one MI355X.

One step = one complete decode call (split kernel + combine kernel) over one
batch of the paged-f16 workload: 32 sequences, 32 query / 8 kv heads,
head_dim 128, block size 16, per-sequence context uniform in [512, 4096],
block table a random permutation of a shared pool, f16 K/V ~ N(0,1), f32 Q,
scale 1/sqrt(128), causal.  Inputs are seeded and synthetic and are resident
in HBM before timing starts; the caches are rotated over enough copies (>= 1
GB) that consecutive steps cannot hit the 256 MB Infinity Cache.

Prints one JSON line.  `value` is KV-read GB/s: algorithmic K+V bytes of the
visible (token, kv_head) rows, each read once per (sequence, kv head), divided
by the wall time per step.  `roofline` prices the dominant (split) kernel
against MI355X HBM peak with its event-timed duration; `cpu_baseline` times the
fp64 oracle on this host's cores over the same workload.  With --all the other
workloads (tiny, tiered int8 W=0/4096, long-context, block-sparse) are
measured the same way and reported under "workloads".
"""
from __future__ import annotations

import argparse
import ctypes
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
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic_balanced_paged_f16_B32_H32x8_D128.txt")


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


def kv_bytes(case) -> int:
    """Algorithmic KV bytes of one decode call: K + V (+ int8 scales) of each visible
    (token, kv head) row once per (sequence, kv head) -- with several queries per
    sequence, a row visible to any of them; for the block-sparse cache a row counts
    once for the union of the blocks its GQA group selects."""
    p = case.params
    B, H, Hkv, D = p["num_seqs"], p["num_heads"], p["num_kv_heads"], p["head_dim"]
    G = H // Hkv
    total = 0
    for b in range(B):
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


def measure(case, steps, warmup, copies=None):
    """Time `steps` full calls (wall clock, inputs resident) and, separately, event-timed
    split-only and combine-only calls on the same stream."""
    import torch
    if copies is None:
        copies = max(1, int(math.ceil(MALL_BYTES / max(cache_bytes(case), 1))))
    r = Runner(case, copies)
    for i in range(warmup):
        r.call(i, "all")
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(steps):
        r.call(i, "all")
    torch.cuda.synchronize()
    wall = (time.perf_counter() - t0) / steps
    # Per-kernel durations: `steps` back-to-back launches of one phase between two
    # events recorded on the launch stream (events around a single launch would add
    # the dispatch overhead of that launch to every sample).
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(4)]
    ev[0].record()
    for i in range(steps):
        r.call(i, "split")
    ev[1].record()
    for i in range(steps):
        r.call(i, "combine")
    ev[2].record()
    torch.cuda.synchronize()
    split_ms = ev[0].elapsed_time(ev[1]) / steps
    comb_ms = ev[1].elapsed_time(ev[2]) / steps
    graph_ms = graph_call_ms(r)
    return r, dict(wall_s=wall, split_ms=split_ms, combine_ms=comb_ms, copies=copies, graph_ms=graph_ms)


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


def measured_traffic(workload=None):
    """HBM bytes per launch of the split kernel from the committed counter summary
    (FETCH_SIZE + WRITE_SIZE, scaled by a copy kernel of known size), or None when
    the summary is missing or was taken on a different kernel source."""
    try:
        t = json.load(open(TRAFFIC_FILE))
    except (OSError, ValueError):
        return None
    if t.get("kernel_source_sha256") != kernel_source_sha() or (workload and t.get("workload") != workload):
        return None
    return t.get("hbm_bytes_per_launch")


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
    loads) over buffers rotated past the Infinity Cache: the measured read ceiling."""
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


def cpu_baseline(case, kvb, min_seconds=10.0):
    """The fp64 oracle (as it stands) over the whole workload, repeated until at least
    min_seconds have passed; returns KV GB/s in the same unit as the GPU line."""
    import oracle
    reps, t0 = 0, time.perf_counter()
    while True:
        oracle.run(case)
        reps += 1
        el = time.perf_counter() - t0
        if el >= min_seconds:
            break
    return dict(value=round(kvb * reps / el / 1e9, 4), unit="GB/s", cores=int(oracle.max_threads()), kind="oracle",
                cpu_model=cpu_model(),
                sample=f"whole workload ({case.name}), {reps} run(s) in {el:.1f} s, fp64, OpenMP over (seq, head)",
                seconds_per_call=round(el / reps, 4))


def line_for(case, steps, warmup, check=True):
    import synth  # noqa: F401
    kvb = kv_bytes(case)
    r, m = measure(case, steps, warmup)
    B = case.params["num_seqs"] * max(1, case.params.get("query_len", 1))   # query tokens per call
    res = dict(workload=case.name, kv_bytes=kvb, ms_per_call=round(m["wall_s"] * 1e3, 5),
               kv_gbs=round(kvb / m["wall_s"] / 1e9, 2), pct_peak=round(100 * kvb / m["wall_s"] / 1e9 / HBM_PEAK_GBS, 2),
               queries_per_s=round(B / m["wall_s"], 1), split_ms=round(m["split_ms"], 5),
               combine_ms=round(m["combine_ms"], 5), split_gbs=round(kvb / (m["split_ms"] / 1e3) / 1e9, 2),
               graph_ms_per_call=round(m["graph_ms"], 5),
               cache_copies=m["copies"])
    if check:
        # sampled parity of the timed launch configuration against the oracle
        import oracle
        out, lse = r.result()
        p = case.params
        rng = np.random.default_rng(0)
        nb = p["num_seqs"] * max(1, p.get("query_len", 1)) * p["num_heads"]
        pairs = np.unique(np.concatenate([[0, nb - 1], rng.integers(0, nb, 14)])).astype(np.int32)
        ro, rl = oracle.run(case, pairs=pairs)
        go = out.reshape(nb, -1)[pairs]
        gl = lse.reshape(nb)[pairs]
        err = float(np.max(np.abs(go - ro)))
        res["sample_max_abs_err"] = err
        res["sample_rel_err"] = err / float(np.max(np.abs(ro)))
        res["sample_lse_err"] = float(np.max(np.abs(gl - rl)))
    return res, m


def workload(idx, window=0):
    """Workloads 1-5 of the input generators, 6: the tiered workload's shape
    with an f16 cold tier, 7: a sliding-window ring f16 cache, 8 and 9: four
    and sixteen queries per sequence over a paged f16 cache of workload 2's
    shape, 10: four queries per sequence over the block-sparse workload."""
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
    return synth.workload(idx, window=window)


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--all", action="store_true", help="also measure the other workloads")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--workload", type=int, default=2,
                    help="headline workload index (default 2; 6 = the tiered workload with an f16 cold tier, "
                         "7 = a sliding-window ring f16 cache, 8 = four queries per sequence, 9 = sixteen, "
                         "10 = four over the block-sparse cache)")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="MIB",
                    help="first run 5 device copies of MIB MiB (for scaling memory counters)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only (asked for --gpus {args.gpus}); the decode path here is the "
              f"single-GPU share. Run with --gpus 1.", file=sys.stderr)
        sys.exit(2)

    import torch
    import synth
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    import int8_quantized_kv_amd as dk
    dk.lib()
    if args.copy_calibration:
        copy_calibration(args.copy_calibration)

    log("generating headline workload ...")
    case = workload(args.workload)
    log(f"workload {case.name}: KV bytes {kv_bytes(case)}")
    head, m = line_for(case, args.steps, args.warmup)
    log(json.dumps(head))
    kvb = head["kv_bytes"]
    split_s = m["split_ms"] / 1e3
    achieved = kvb / split_s / 1e9
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
        "data": "synthetic (seeded numpy N(0,1) Q/K/V, uniform lengths, permuted block pool)",
        "config": {"workload": case.name, "global_batch": int(B), "num_heads": int(H),
                   "num_kv_heads": int(case.params["num_kv_heads"]), "head_dim": int(D),
                   "block_size": int(case.params["block_size"]),
                   "seq_len_range": [int(lens.min()), int(lens.max())],
                   "total_tokens": int(lens.sum()), "parallelism": "single GPU"},
        "pct_of_hbm_peak": head["pct_peak"],
        "queries_per_s": head["queries_per_s"],
        "kernels": {"split_ms": head["split_ms"], "combine_ms": head["combine_ms"],
                    "graph_ms_per_call": head["graph_ms_per_call"]},
        "roofline": {"bound": "hbm", "achieved": round(achieved, 2), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": measured_traffic(case.name),
                     "kernel": f"split kernel <D={D}, G={G}, {kind}>",
                     "bytes_per_launch": kvb},
        "parity_sample": {k: head[k] for k in ("sample_max_abs_err", "sample_rel_err", "sample_lse_err")},
        "copy_reference_gbs": copy_reference(),
    }
    ceiling = read_reference()
    out["roofline"]["measured_read_ceiling_gbs"] = ceiling
    out["roofline"]["frac_of_measured_ceiling"] = round(achieved / ceiling, 4)
    log("timing the tiered write path ...")
    out["write_path"] = measure_append()
    if not args.no_cpu_baseline:
        log("timing the oracle on the host ...")
        out["cpu_baseline"] = cpu_baseline(case, kvb)
    if args.all:
        extra = []
        for idx, kw in ((1, {}), (3, dict(window=0)), (3, dict(window=4096)), (4, {}), (5, {}),
                        (6, dict(window=0)), (6, dict(window=4096)), (7, {}), (8, {}), (9, {}), (10, {})):
            log(f"generating workload {idx} {kw} ...")
            c = workload(idx, **kw)
            res, _ = line_for(c, max(20, args.steps // 4), max(5, args.warmup // 4))
            log(json.dumps(res))
            extra.append(res)
            del c
        out["workloads"] = extra
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
