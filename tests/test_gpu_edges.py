"""GPU parity at the edges of the plans: batches larger than the balanced
schedule takes (static splits), the largest GQA group and head counts, one
kv head, head_dim 64 on every cache, sequences of one key, and more tiered
sequences than the balanced kernel keeps in LDS -- checked against the oracle
on sampled (sequence, head) pairs, or on every row where that is cheap."""
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


def _sampled(case, what, n=40):
    log(f"edge {what}")
    og, lg = DeviceCase(case).run_np()
    p = case.params
    nbh = p["num_seqs"] * max(1, p.get("query_len", 1)) * p["num_heads"]
    rng = np.random.default_rng(nbh)
    pairs = np.unique(np.concatenate([[0, nbh - 1], rng.integers(0, nbh, n)])).astype(np.int32)
    ro, rl = oracle_run(case, pairs=pairs)
    compare(og.reshape(nbh, -1)[pairs], lg.reshape(nbh)[pairs], ro, rl, what=what)


@pytest.mark.parametrize("B", [4096, 5000])
def test_many_short_sequences(B):
    # 4096 sequences still fit the balanced schedule's sequence limit; 5000 go to static splits
    rng = np.random.default_rng(B)
    lens = rng.integers(1, 65, size=B)
    c = synth.paged_case(700 + B % 7, B, 32, 8, 128, 16, lens=lens, kv_dtype=synth.F16)
    _sampled(c, f"paged f16 B{B} L 1-64")


def test_combine_many_rows_with_one_long_sequence():
    # 300 sequences share the workers, so the combine takes half a wave per
    # row; the one long sequence's rows have far more partials than 32 lanes
    # fold in one round
    rng = np.random.default_rng(714)
    lens = rng.integers(1, 65, size=300)
    lens[137] = 40000
    c = synth.paged_case(714, 300, 32, 8, 128, 16, lens=lens, kv_dtype=synth.F16, softcap=30.0)
    log("edge combine rows, one long sequence")
    og, lg = DeviceCase(c).run_np()
    H = 32
    pairs = np.unique(np.concatenate([137 * H + np.arange(0, H, 3), [0, 136 * H + 5, 138 * H + 7, 299 * H + 31],
                                      rng.integers(0, 300 * H, 20)])).astype(np.int32)
    ro, rl = oracle_run(c, pairs=pairs)
    compare(og.reshape(300 * H, -1)[pairs], lg.reshape(300 * H)[pairs], ro, rl, what="combine rows, long row")


@pytest.mark.parametrize("D,B", [(128, 32), (64, 40)])
def test_combine_wave_with_one_long_sequence(D, B):
    # fewer than 2048 rows whose sequences meet few workers each: the combine
    # takes one wave per row; the one long sequence's rows have far more
    # partials than a wave folds in one round (D = 64: four lane groups)
    rng = np.random.default_rng(715 + D)
    lens = rng.integers(1, 65, size=B)
    lens[B // 3] = 60000
    c = synth.paged_case(715 + D, B, 32, 8, D, 16, lens=lens, kv_dtype=synth.F16, softcap=30.0)
    log(f"edge combine wave, one long sequence, D={D} B={B}")
    og, lg = DeviceCase(c).run_np()
    ro, rl = oracle_run(c)
    compare(og, lg, ro, rl, what=f"combine wave, long row, D={D}")


def _combine_path_case(path):
    """A call whose combine takes the named kernel: one wave per row (few
    partials per row), half a wave per row (16384 rows of sixteen queries, about
    two workers per sequence, D = 64), one workgroup per row (two long
    sequences), the row-group kernel of static splits (2304 rows, at most 8
    splits each), or one workgroup per row of static splits (few rows)."""
    rng = np.random.default_rng(716)
    if path == "half":
        return synth.paged_case(720, 32, 32, 8, 64, 16, lens=rng.integers(16, 301, size=32), kv_dtype=synth.F16,
                                query_len=16), 0
    if path == "wave":
        return synth.paged_case(716, 32, 32, 8, 128, 16, lens=rng.integers(1, 600, size=32), kv_dtype=synth.F16), 0
    if path == "workgroup":
        return synth.paged_case(717, 2, 32, 8, 128, 16, lens=[20000, 13001], kv_dtype=synth.F16), 0
    if path == "rows":
        return synth.paged_case(718, 72, 32, 8, 128, 16, lens=rng.integers(0, 513, size=72), kv_dtype=synth.F16), 64
    return synth.paged_case(719, 3, 32, 8, 64, 16, lens=[700, 1, 333], kv_dtype=synth.F16), 64


@pytest.mark.parametrize("path", ["wave", "half", "workgroup", "rows", "static"])
def test_combine_outputs_off_vector_alignment(path):
    """The combine kernels store four output elements at once only where the
    output starts on an 8-byte (f16) or 16-byte (f32) boundary: an output one
    element past it must hold the same bits as an aligned one, and the f16
    output the f32 result rounded to f16.  Without an output (lse only) the
    lse is the same."""
    import torch
    c, split_tokens = _combine_path_case(path)
    dc = DeviceCase(c)
    log(f"edge combine {path}: outputs one element off alignment, and lse only")
    o32, l32 = dc.run(split_tokens)
    o16, _ = dc.run(split_tokens, out_dtype=torch.float16)
    o_none, l_only = dc.run(split_tokens, want_out=False)
    assert o_none is None
    shifted = {}
    for dt in (torch.float32, torch.float16):
        buf = torch.full((o32.numel() + 1,), float("nan"), dtype=dt, device=o32.device)
        view = buf[1:].view(o32.shape)
        assert view.data_ptr() % 8 != 0
        o, _ = dc.run(split_tokens, out=view, out_dtype=dt)
        shifted[dt] = o
    torch.cuda.synchronize()
    assert torch.equal(shifted[torch.float32], o32)
    assert torch.equal(shifted[torch.float16], o16)
    assert torch.equal(o16, o32.to(torch.float16))
    assert torch.equal(l_only, l32)
    ro, rl = oracle_run(c)
    compare(o32.cpu().numpy(), l32.cpu().numpy(), ro, rl, what=f"combine {path}")


@pytest.mark.parametrize("longest,split_tokens", [(1024, 64), (1100, 64), (1100, 128)])
def test_combine_rows_static_splits(longest, split_tokens):
    # 72 x 32 rows: with at most 16 splits per row the static path's combine takes
    # eight rows per workgroup (1100 keys in splits of 64 make 18 and take the other)
    rng = np.random.default_rng(715)
    lens = rng.integers(0, 1025, size=72)
    lens[5] = longest
    c = synth.paged_case(715, 72, 32, 8, 128, 16, lens=lens, kv_dtype=synth.F16)
    _sampled(c, f"static splits of {split_tokens}, longest {longest}", n=60)


def test_largest_group_and_many_heads():
    c = synth.paged_case(711, 3, 128, 16, 128, 16, lens=[2000, 1, 777], kv_dtype=synth.F16, softcap=30.0)
    _sampled(c, "H128 / Hkv16 (G8)")


def test_one_kv_head_mha_and_gqa():
    c = synth.paged_case(712, 2, 8, 1, 128, 64, lens=[3000, 100], kv_dtype=synth.F16, window=1000)
    _sampled(c, "Hkv1 G8 bs64 window 1000")
    c = synth.paged_case(713, 2, 16, 16, 64, 16, lens=[900, 33], kv_dtype=synth.F16)
    _sampled(c, "MHA G1 D64")


@pytest.mark.parametrize("kind", ["tiered", "tiered_f16", "ring", "sparse"])
def test_head_dim_64(kind):
    if kind == "tiered":
        c = synth.tiered_case(714, 2, 32, 8, 64, 16, [900, 300], [700, 250], 256, softcap=50.0)
    elif kind == "tiered_f16":
        c = synth.tiered_f16_case(715, 2, 32, 8, 64, 16, [900, 300], [700, 250], 256)
    elif kind == "ring":
        c = synth.ring_case(716, 2, 32, 8, 64, 128, [900, 50])
    else:
        c = synth.sparse_case(717, 2, 32, 8, 64, 64, 64, 4, [2048, 700])
    _sampled(c, f"{kind} D64")


@pytest.mark.parametrize("window", [0, 200])
def test_tiered_int8_beyond_the_per_sequence_stash(window):
    # more sequences than the balanced kernel keeps in LDS (256), so each
    # worker reads a sequence's range and cold length from memory when it
    # starts it; lengths up to 700 with a 128-token ring make most sweeps cross
    # from the int8 tier into the ring (the transition units of the schedule)
    rng = np.random.default_rng(730 + window)
    B = 300
    lens = rng.integers(1, 701, size=B)
    cold = np.maximum(0, lens - rng.integers(0, 129, size=B))
    c = synth.tiered_case(730 + window, B, 32, 8, 128, 16, lens, cold, 128, softcap=30.0, window=window)
    log(f"edge tiered int8 B{B} beyond the stash, window {window}")
    og, lg = DeviceCase(c).run_np()
    ro, rl = oracle_run(c)
    compare(og, lg, ro, rl, what=f"tiered int8 B{B} window {window}, every row")


def test_single_key_sequences_everywhere():
    B = 300
    c = synth.tiered_case(718, B, 32, 8, 128, 16, [1] * B, [i % 2 for i in range(B)], 16)
    _sampled(c, "tiered, one key per sequence (hot or cold)")


@pytest.mark.parametrize("nbytes,pos", [(1 << 20, 12345), ((64 << 20) + 48, (16 << 20) + 3)])
def test_stream_read_touches_every_word(nbytes, pos):
    """The measured read ceiling must read the whole buffer: one marked word among
    zeros reaches the sink."""
    import torch
    import int8_quantized_kv_amd as dk
    buf = torch.zeros(nbytes // 4, dtype=torch.int32, device="cuda")
    buf[pos] = np.int32(np.uint32(0x9E3779B9).view(np.int32))
    sink = torch.zeros(1, dtype=torch.int32, device="cuda")
    dk.dattn_stream_read(buf, sink)
    torch.cuda.synchronize()
    assert np.uint32(sink.cpu().numpy()[0]) == 0x9E3779B9


@pytest.mark.parametrize("qmul", [40.0, 1e-4])
@pytest.mark.parametrize("kind", ["paged", "tiered", "multi_query"])
def test_score_dynamic_range(kind, qmul):
    """Scores of hundreds (the running max moves by far more than its lazy slack, so
    the accumulator is rescaled many times) or nearly flat (weights all ~1)."""
    if kind == "paged":
        c = synth.paged_case(720, 3, 32, 8, 128, 16, lens=[3000, 100, 1000], kv_dtype=synth.F16)
    elif kind == "tiered":
        c = synth.tiered_case(721, 2, 32, 8, 128, 16, [2000, 700], [1800, 600], 256)
    else:
        c = synth.paged_case(722, 2, 32, 8, 128, 16, lens=[2000, 300], kv_dtype=synth.F16, query_len=4)
    # sort keys so that later tiles hold ever larger scores for the first head: increasing max
    c.q = (c.q * np.float32(qmul)).astype(np.float32)
    _sampled(c, f"{kind} q x {qmul}")


def test_extreme_int8_scales():
    """Zero, subnormal and large f16 scales.  Key scales stay below 0.05 so the
    scores keep the O(1) magnitude the absolute tolerance is stated for; value
    scales go up to 60000, so outputs reach ~1e6 and are held to the normwise
    criterion (max |g - r| <= 1e-3 max |r|) alone, as f32 cannot hold 1e-3
    absolute at that size."""
    import torch
    c = synth.tiered_case(723, 2, 32, 8, 128, 16, [900, 400], [800, 300], 128)
    rng = np.random.default_rng(5)
    for sc, choices in ((c.k_scale, [0.0, 1e-4, 6e-5, 3e-3, 0.05]), (c.v_scale, [0.0, 1e-4, 6e-5, 3e-3, 60000.0])):
        pick = rng.random(sc.shape) < 0.3
        sc[pick] = rng.choice(np.array(choices, np.float16), size=int(pick.sum()))
    log("edge int8 scales 0 .. 60000")
    og, lg = DeviceCase(c).run_np()
    ro, rl = oracle_run(c)
    assert np.all(np.isfinite(og)) and np.all(np.isfinite(lg))
    err = np.max(np.abs(og - ro))
    log(f"  max abs {err:.3e}, max |ref| {np.max(np.abs(ro)):.3e}, lse {np.max(np.abs(lg - rl)):.3e}")
    assert err <= 1e-3 * np.max(np.abs(ro))
    assert np.max(np.abs(lg - rl)) <= 1e-3


def test_workspace_reused_across_calls_of_other_shapes():
    # One workspace, first filled with 0xFF bytes, serves calls on other caches and
    # shapes in turn (balanced schedule and static splits).  Each result must equal,
    # bit for bit, the same call with a fresh workspace of its own: no call may read
    # from the workspace anything that it did not write itself.
    import torch
    cases = [
        synth.paged_case(102, 4, 32, 8, 128, 16, len_range=(512, 1200), kv_dtype=synth.F16),
        synth.tiered_case(103, 2, 32, 8, 128, 16, [700, 613], [450, 420], 256, softcap=50.0),
        synth.sparse_case(105, 2, 32, 8, 128, 64, 64, 4, [2048, 1999]),
        synth.ring_case(401, 3, 32, 8, 128, 256, [1000, 100, 257], softcap=30.0),
        synth.paged_case(106, 3, 32, 8, 128, 16, len_range=(100, 900), kv_dtype=synth.F16, query_len=4),
        synth.paged_case(107, 5, 16, 2, 64, 16, len_range=(1, 300), kv_dtype=synth.F16),
        synth.paged_case(102, 4, 32, 8, 128, 16, len_range=(512, 1200), kv_dtype=synth.F16),
    ]
    ws = torch.full((64 << 20,), 255, dtype=torch.uint8, device="cuda:0")
    for i, c in enumerate(cases):
        dc = DeviceCase(c)
        for st in (0, 256):
            log(f"workspace reuse: call {i} ({c.kind}, B={c.params['num_seqs']}) split_tokens={st}")
            o0, l0 = dc.run_np(st)
            o1, l1 = dc.run_np(st, workspace=ws)
            assert np.array_equal(o0, o1) and np.array_equal(l0, l1), (i, c.kind, st)


def test_call_is_ordered_on_the_callers_stream():
    # On a side stream: q zeroed, a backlog of copies, q restored, then the call.  The
    # call sees the restored q only if it runs on that stream, after the restore;
    # launched on any other stream it would run during the backlog and read zeros.
    import torch
    c = synth.paged_case(108, 4, 32, 8, 128, 16, len_range=(300, 2000), kv_dtype=synth.F16)
    dc = DeviceCase(c)
    want_o, want_l = dc.run_np()
    side = torch.cuda.Stream()
    src = torch.empty(128 << 20, dtype=torch.uint8, device="cuda:0")
    dst = torch.empty_like(src)
    keep = dc.q.clone()
    torch.cuda.synchronize()
    with torch.cuda.stream(side):
        dc.q.zero_()
        for _ in range(16):
            dst.copy_(src)
        dc.q.copy_(keep)
        out, lse = dc.run()
    side.synchronize()
    log("side-stream call done")
    assert np.array_equal(out.cpu().numpy(), want_o) and np.array_equal(lse.cpu().numpy(), want_l)
