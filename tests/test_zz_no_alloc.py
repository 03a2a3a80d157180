"""The no-allocation entry point dattn_decode_tiered_int8_static, called
through the C ABI: the same decode as dattn_decode_tiered_int8, with the
split partials in the library's static device scratch instead of a
caller-provided workspace.  Two calls in a row, the second on a smaller input,
each compared with the workspace entry point on the same inputs (bit for bit:
the same kernels and schedule run), and with the fp64 oracle."""
import ctypes

import numpy as np
import pytest

import synth
from gpu_util import DeviceCase, compare, log, oracle_run

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import int8_quantized_kv_amd as dk
    dk.lib()
    yield


def _static_call(dc, out, lse):
    """dattn_decode_tiered_int8_static through ctypes: inputs and outputs are the
    caller's; nothing else is passed."""
    import torch
    import int8_quantized_kv_amd as dk
    L = dk.lib()
    f = L.dattn_decode_tiered_int8_static
    P, i32 = ctypes.c_void_p, ctypes.c_int32
    f.argtypes = [ctypes.POINTER(dk.DattnParams), P, P, P, i32, P, P, P, P, P, P, P, P, P, P, P]
    f.restype = ctypes.c_int
    c = dc.case
    p = c.params
    B, H, D = c.q.shape[0], c.q.shape[-2], c.q.shape[-1]
    NB, bs = c.k_cold.shape[0], c.k_cold.shape[1]
    prm = dk.DattnParams(B, H, p["num_kv_heads"], D, p["scale"], p["causal"], p["sliding_window"], p["softcap"], bs,
                         c.cold_block_table.shape[1], NB, int(c.seq_lens.max()), 0, 0, dk.F32, 1, dk.F32)
    ptr = lambda t: None if t is None else P(t.data_ptr())  # noqa: E731
    rc = f(ctypes.byref(prm), ptr(dc.q), ptr(dc.k_hot), ptr(dc.v_hot), c.hot_window, ptr(dc.k_cold), ptr(dc.v_cold),
           ptr(dc.k_scale), ptr(dc.v_scale), ptr(dc.cold_block_table), ptr(dc.seq_lens), ptr(dc.cold_lens),
           ptr(dc.q_pos), ptr(out), ptr(lse), P(torch.cuda.current_stream().cuda_stream))
    assert rc == 0, dk.dattn_last_error()


def test_static_scratch_matches_the_workspace_entry_point():
    import torch
    cases = [synth.tiered_case(140, 4, 32, 8, 128, 16, [3000, 2900, 1777, 640], [2600, 2400, 1500, 200], 512,
                               softcap=50.0, window=0),
             synth.tiered_case(141, 2, 32, 8, 128, 16, [700, 333], [450, 300], 256, softcap=30.0, window=300)]
    for i, c in enumerate(cases):
        log(f"static scratch call {i}: {c.name} B={c.q.shape[0]}")
        dc = DeviceCase(c)
        out = torch.full(c.q.shape, float("nan"), dtype=torch.float32, device="cuda:0")
        lse = torch.full(c.q.shape[:-1], float("nan"), dtype=torch.float32, device="cuda:0")
        _static_call(dc, out, lse)
        torch.cuda.synchronize()
        og, lg = out.cpu().numpy(), lse.cpu().numpy()
        ow, lw = dc.run_np()
        assert np.array_equal(og.view(np.uint32), ow.view(np.uint32)), f"call {i}: out differs from the workspace call"
        assert np.array_equal(lg.view(np.uint32), lw.view(np.uint32)), f"call {i}: lse differs from the workspace call"
        ro, rl = oracle_run(c)
        compare(og, lg, ro, rl, what=f"static scratch call {i}")


def test_static_scratch_binding_matches_the_workspace_call():
    """The Python binding of the same entry point (argument marshalling only)."""
    import torch
    import int8_quantized_kv_amd as dk
    c = synth.tiered_case(142, 3, 16, 4, 128, 16, [1200, 64, 900], [1000, 0, 700], 256, softcap=0.0, window=0)
    dc = DeviceCase(c)
    kw = dc.kwargs()
    og, lg = dk.dattn_decode_tiered_int8_static(dc.q, dc.k_hot, dc.v_hot, dc.k_cold, dc.v_cold, dc.k_scale,
                                                dc.v_scale, dc.cold_block_table, dc.seq_lens, dc.cold_lens, **kw)
    ow, lw = dc.run_np()
    torch.cuda.synchronize()
    assert np.array_equal(og.cpu().numpy().view(np.uint32), ow.view(np.uint32))
    assert np.array_equal(lg.cpu().numpy().view(np.uint32), lw.view(np.uint32))


def test_static_scratch_refuses_calls_beyond_its_size():
    """A call whose partials would not fit the static scratch is refused on the
    host before anything is enqueued."""
    import int8_quantized_kv_amd as dk
    L = dk.lib()
    f = L.dattn_decode_tiered_int8_static
    f.restype = ctypes.c_int
    # 4096 sequences of up to 2^20 tokens: far more partials than 32 MiB holds
    p = dk.DattnParams(4096, 32, 8, 128, 0.0, 1, 0, 0.0, 16, 65536, 1 << 20, 1 << 20, 0, 0, dk.F32, 1, dk.F32)
    fake = ctypes.c_void_p(0x1000)   # never dereferenced: the call fails its size check first
    rc = f(ctypes.byref(p), fake, fake, fake, ctypes.c_int32(512), fake, fake, fake, fake, fake, fake, fake, None, fake,
           None, None)
    assert rc == dk.ERR_UNSUPPORTED and "static scratch" in dk.dattn_last_error()
