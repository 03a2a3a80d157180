"""Helpers shared by the GPU tests: move a synthetic case to the device, call the
library through its binding, and compare against the oracle."""
from __future__ import annotations

import sys

import numpy as np

TOL = 1e-3          # max abs error, and max abs error / max |reference|
LSE_TOL = 1e-3


def log(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def dev(a, device="cuda:0"):
    import torch
    if a is None:
        return None
    a = np.ascontiguousarray(a)
    if a.dtype == np.uint32:
        a = a.view(np.int32)
    if a.dtype == np.uint16:
        a = a.view(np.float16)
    return torch.from_numpy(a).to(device)


class DeviceCase:
    """Device copies of a synthetic case's arrays."""

    def __init__(self, case, device="cuda:0"):
        self.case = case
        c = case
        self.q = dev(c.q, device)
        self.seq_lens = dev(c.seq_lens, device)
        self.q_pos = dev(c.q_pos, device)
        if c.kind in ("paged", "sparse"):
            self.k_cache = dev(c.k_cache, device)
            self.v_cache = dev(c.v_cache, device)
            self.block_table = dev(c.block_table, device)
        if c.kind in ("tiered", "tiered_f16"):
            self.k_hot = dev(c.k_hot, device)
            self.v_hot = dev(c.v_hot, device)
            self.k_cold = dev(c.k_cold, device)
            self.v_cold = dev(c.v_cold, device)
            self.cold_block_table = dev(c.cold_block_table, device)
            self.cold_lens = dev(c.cold_lens, device)
        if c.kind == "ring":
            self.k_ring = dev(c.k_hot, device)
            self.v_ring = dev(c.v_hot, device)
        if c.kind == "tiered":
            self.k_scale = dev(c.k_scale, device)
            self.v_scale = dev(c.v_scale, device)
        if c.kind == "sparse":
            self.row_ptr = dev(c.row_ptr, device)
            self.col_idx = dev(c.col_idx, device)

    def kwargs(self, split_tokens=0):
        p = self.case.params
        return dict(q_pos=self.q_pos, scale=p["scale"], causal=bool(p["causal"]), sliding_window=p["sliding_window"],
                    softcap=p["softcap"], max_seq_len=int(self.case.seq_lens.max()) if len(self.case.seq_lens) else 0,
                    split_tokens=split_tokens)

    def run(self, split_tokens=0, **over):
        import int8_quantized_kv_amd as dk
        kw = self.kwargs(split_tokens)
        kw.update(over)
        c = self.case
        if c.kind == "paged":
            return dk.dattn_decode_paged(self.q, self.k_cache, self.v_cache, self.block_table, self.seq_lens, **kw)
        if c.kind == "tiered":
            return dk.dattn_decode_tiered_int8(self.q, self.k_hot, self.v_hot, self.k_cold, self.v_cold,
                                               self.k_scale, self.v_scale, self.cold_block_table, self.seq_lens,
                                               self.cold_lens, **kw)
        if c.kind == "ring":
            kw.pop("sliding_window")
            return dk.dattn_decode_ring_f16(self.q, self.k_ring, self.v_ring, self.seq_lens, **kw)
        if c.kind == "tiered_f16":
            return dk.dattn_decode_tiered_f16(self.q, self.k_hot, self.v_hot, self.k_cold, self.v_cold,
                                              self.cold_block_table, self.seq_lens, self.cold_lens, **kw)
        return dk.dattn_decode_block_sparse(self.q, self.k_cache, self.v_cache, self.block_table, self.seq_lens,
                                            c.sparse_block, self.row_ptr, self.col_idx, **kw)

    def run_np(self, split_tokens=0, **over):
        import torch
        out, lse = self.run(split_tokens, **over)
        torch.cuda.synchronize()
        return (None if out is None else out.cpu().numpy()), (None if lse is None else lse.cpu().numpy())


def oracle_run(case, pairs=None):
    import oracle
    out, lse = oracle.run(case, pairs=pairs)
    if pairs is None:
        p = case.params
        lead = (p["num_seqs"],) if p.get("query_len", 1) <= 1 else (p["num_seqs"], p["query_len"])
        out = out.reshape(*lead, p["num_heads"], p["head_dim"])
        lse = lse.reshape(*lead, p["num_heads"])
    return out, lse


def compare(out_g, lse_g, out_r, lse_r, tol=TOL, what=""):
    """Parity: empty heads exactly (0, -inf); elsewhere max abs error <= tol and
    max abs error / max |reference| <= tol; lse within LSE_TOL."""
    out_g = np.asarray(out_g, np.float64)
    lse_g = np.asarray(lse_g, np.float64)
    empty = ~np.isfinite(lse_r)
    assert np.all(lse_g[empty] == -np.inf), f"{what}: expected -inf lse on empty heads"
    assert np.all(out_g[empty] == 0.0), f"{what}: expected zero output on empty heads"
    full = ~empty
    if not full.any():
        return dict(abs=0.0, rel=0.0, lse=0.0)
    assert np.all(np.isfinite(out_g[full])), f"{what}: non-finite output"
    err = float(np.max(np.abs(out_g[full] - out_r[full])))
    ref = float(np.max(np.abs(out_r[full])))
    lerr = float(np.max(np.abs(lse_g[full] - lse_r[full])))
    elem = float(np.max(np.abs(out_g[full] - out_r[full]) / (np.abs(out_r[full]) + 1e-3)))
    stats = dict(abs=err, rel=err / max(ref, 1e-30), lse=lerr, elem=elem)
    log(f"  parity {what}: max_abs={err:.3e} normwise_rel={stats['rel']:.3e} lse={lerr:.3e} elem_rel={elem:.3e}")
    assert err <= tol, f"{what}: max abs error {err}"
    assert err <= tol * ref, f"{what}: normwise relative error {err / ref}"
    assert lerr <= LSE_TOL, f"{what}: lse error {lerr}"
    return stats
