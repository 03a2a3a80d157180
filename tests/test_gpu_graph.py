"""The library's calls can be captured into a HIP graph (torch.cuda.graph) once
warmed up: no allocation, synchronisation or memset happens inside a call.  A
captured decode step (tiered write path, then the tiered decode, then a paged
decode) is replayed several times with eager work in between -- new inputs
written in place, lengths advancing -- and every replay must equal, bit for
bit, the same calls made eagerly on the same state."""
import numpy as np
import pytest

import synth
from gpu_util import log

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import int8_quantized_kv_amd as dk
    dk.lib()
    yield


def _dev(a):
    import torch
    a = np.ascontiguousarray(a)
    if a.dtype == np.uint32:
        a = a.view(np.int32)
    return torch.from_numpy(a).cuda()


class Step:
    """Device state of one decode step: a tiered cache with its write path and a paged cache."""

    def __init__(self):
        import torch
        import int8_quantized_kv_amd as dk
        self.dk = dk
        rng = np.random.default_rng(601)
        B, Hkv, D, hw, bs = 4, 8, 128, 128, 16
        lens, cold = [300, 517, 64, 1000], [200, 517 - 128, 0, 1000 - 128]
        max_blocks = (max(cold) + 64) // bs + 2      # room for the cold tier to grow during the test
        nb = B * max_blocks
        table = np.arange(nb, dtype=np.int32).reshape(B, max_blocks)   # every entry names a pool block
        self.t = {
            "q": _dev(rng.standard_normal((B, 32, D)).astype(np.float32)),
            "k_hot": _dev(rng.standard_normal((B, hw, Hkv, D)).astype(np.float16)),
            "v_hot": _dev(rng.standard_normal((B, hw, Hkv, D)).astype(np.float16)),
            "k_cold": _dev(rng.integers(0, 2 ** 32, size=(nb, bs, Hkv, D // 4), dtype=np.uint64).astype(np.uint32)),
            "v_cold": _dev(rng.integers(0, 2 ** 32, size=(nb, bs, Hkv, D // 4), dtype=np.uint64).astype(np.uint32)),
            "k_scale": _dev(rng.uniform(1e-3, 2e-2, size=(nb, bs, Hkv)).astype(np.float16)),
            "v_scale": _dev(rng.uniform(1e-3, 2e-2, size=(nb, bs, Hkv)).astype(np.float16)),
            "cold_block_table": _dev(table),
            "seq_lens": _dev(np.array(lens, np.int32)),
            "cold_lens": _dev(np.array(cold, np.int32)),
        }
        p = synth.paged_case(602, 4, 32, 8, 128, 16, lens=[700, 90, 1500, 3], query_len=2)
        self.p = {k: _dev(getattr(p, k)) for k in ("q", "k_cache", "v_cache", "block_table", "seq_lens")}
        # sixteen queries per sequence: row-block waves sharing tiles through LDS, and the
        # one-wave-per-row combine (8 x 16 x 32 rows, eight workers per sequence)
        w = synth.paged_case(603, 8, 32, 8, 128, 16, lens=[900, 40, 1300, 17, 600, 2000, 256, 5], query_len=16)
        self.w = {k: _dev(getattr(w, k)) for k in ("q", "k_cache", "v_cache", "block_table", "seq_lens")}
        self.out_w = torch.empty((8, 16, 32, 128), dtype=torch.float32, device="cuda")
        self.lse_w = torch.empty((8, 16, 32), dtype=torch.float32, device="cuda")
        self.ws3 = torch.empty((128 << 20,), dtype=torch.uint8, device="cuda")
        self.k_new = torch.zeros((B, Hkv, D), dtype=torch.float16, device="cuda")
        self.v_new = torch.zeros_like(self.k_new)
        self.out_t = torch.empty((B, 32, D), dtype=torch.float32, device="cuda")
        self.lse_t = torch.empty((B, 32), dtype=torch.float32, device="cuda")
        self.out_p = torch.empty((4, 2, 32, 128), dtype=torch.float16, device="cuda")
        self.lse_p = torch.empty((4, 2, 32), dtype=torch.float32, device="cuda")
        self.ws = torch.empty((64 << 20,), dtype=torch.uint8, device="cuda")
        self.ws2 = torch.empty((64 << 20,), dtype=torch.uint8, device="cuda")

    def run(self):
        dk, t, p = self.dk, self.t, self.p
        dk.dattn_append_tiered_int8(self.k_new, self.v_new, t["k_hot"], t["v_hot"], t["k_cold"], t["v_cold"],
                                    t["k_scale"], t["v_scale"], t["cold_block_table"], t["seq_lens"], t["cold_lens"])
        dk.dattn_decode_tiered_int8(t["q"], t["k_hot"], t["v_hot"], t["k_cold"], t["v_cold"], t["k_scale"],
                                    t["v_scale"], t["cold_block_table"], t["seq_lens"], t["cold_lens"], softcap=30.0,
                                    max_seq_len=2048, out=self.out_t, lse=self.lse_t, workspace=self.ws)
        dk.dattn_decode_paged(p["q"], p["k_cache"], p["v_cache"], p["block_table"], p["seq_lens"], max_seq_len=1500,
                              out=self.out_p, lse=self.lse_p, out_dtype=self.out_p.dtype, workspace=self.ws2)
        w = self.w
        dk.dattn_decode_paged(w["q"], w["k_cache"], w["v_cache"], w["block_table"], w["seq_lens"], max_seq_len=2000,
                              out=self.out_w, lse=self.lse_w, workspace=self.ws3)

    def snapshot(self):
        import torch
        torch.cuda.synchronize()
        keys = ("k_hot", "v_hot", "k_cold", "v_cold", "k_scale", "v_scale", "seq_lens", "cold_lens")
        return [self.t[k].clone() for k in keys] + [x.clone() for x in (self.out_t, self.lse_t, self.out_p,
                                                                         self.lse_p, self.out_w, self.lse_w)]

    def load(self, snap):
        keys = ("k_hot", "v_hot", "k_cold", "v_cold", "k_scale", "v_scale", "seq_lens", "cold_lens")
        for k, x in zip(keys, snap):
            self.t[k].copy_(x)


def test_decode_step_graph_replays_equal_eager_calls():
    import torch
    st = Step()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):          # warm-up on a side stream (device queries, occupancy cache)
        st.run()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    before_capture = st.snapshot()
    with torch.cuda.graph(g):
        st.run()
    # capture does not execute: the state is unchanged
    after = st.snapshot()
    for a, b in zip(before_capture[:8], after[:8]):
        assert torch.equal(a, b)
    rng = np.random.default_rng(3)
    for rep in range(4):
        # eager work between replays: new tokens and queries written in place
        st.k_new.copy_(torch.from_numpy(rng.standard_normal((4, 8, 128)).astype(np.float16)))
        st.v_new.copy_(torch.from_numpy(rng.standard_normal((4, 8, 128)).astype(np.float16)))
        st.t["q"].mul_(-1.0)
        st.p["q"].add_(0.25)
        st.w["q"].mul_(0.75)
        start = st.snapshot()
        g.replay()
        got = st.snapshot()
        st.load(start)
        st.run()                            # the same calls, eagerly, from the same state
        want = st.snapshot()
        for i, (a, b) in enumerate(zip(got, want)):
            assert torch.equal(a, b), f"replay {rep}, tensor {i}"
        log(f"replay {rep}: equal to eager; tiered lengths {got[6].tolist()}")
        st.load(got)
    assert int(st.t["seq_lens"][0]) == 300 + 1 + 4   # the warm-up call and one per replay
