"""GPU parity of the tiered f16 cache (paged f16 cold tier + f16 hot ring)
against the fp64 oracle, and of the output modes every decode entry point has:
f16 output (the f32 result rounded to nearest even) and lse only."""
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
    dk.lib()   # fail loudly if the library is missing
    yield


def _check(case, split_tokens=0, what=""):
    log(f"case {case.kind} {what} split_tokens={split_tokens}")
    og, lg = DeviceCase(case).run_np(split_tokens)
    orf, lrf = oracle_run(case)
    return compare(og, lg, orf, lrf, what=what)


@pytest.mark.parametrize("window", [0, 300])
def test_tiered_f16_like_the_tiered_workload_small(window):
    c = synth.tiered_f16_case(301, 2, 32, 8, 128, 16, [700, 613], [450, 420], 256, softcap=50.0, window=window)
    _check(c, what=f"tiered f16 B2 L700 W{window} cap50 ring-wrap")


def _rand_case(seed):
    rng = np.random.default_rng(70_000 + seed)
    D = int(rng.choice([64, 128]))
    G = int(rng.choice([1, 2, 4, 8]))
    Hkv = int(rng.choice([1, 2, 3, 4, 8]))
    B = int(rng.integers(1, 4))
    lens = rng.integers(0, 700, size=B)
    if rng.random() < 0.3:
        lens[0] = int(rng.choice([0, 1, 15, 16, 17]))
    qp = None
    if rng.random() < 0.4:
        qp = np.array([int(rng.integers(0, max(1, L))) for L in lens], np.int32)
    bs = int(rng.choice([1, 5, 16, 32]))
    hw = int(rng.choice([1, 16, 50, 128]))
    cold = np.array([max(0, int(L) - int(rng.integers(0, hw + 1))) for L in lens])
    return synth.tiered_f16_case(seed, B, Hkv * G, Hkv, D, bs, lens, cold, hw, q_pos=qp,
                                 causal=int(rng.random() < 0.8), window=int(rng.choice([0, 0, 1, 17, 200])),
                                 softcap=float(rng.choice([0.0, 0.0, 5.0, 50.0])),
                                 scale=float(rng.choice([0.0, np.float32(rng.uniform(0.03, 0.3))])))


@pytest.mark.parametrize("seed", range(24))
def test_tiered_f16_random_sweep(seed):
    case = _rand_case(seed)
    st = int(np.random.default_rng(seed).choice([0, 0, 16, 48, 256]))
    p = case.params
    _check(case, split_tokens=st,
           what=f"seed{seed} B{p['num_seqs']} H{p['num_heads']}/{p['num_kv_heads']} D{p['head_dim']} "
                f"bs{p['block_size']} hw{case.hot_window} W{p['sliding_window']} cap{p['softcap']}")


def test_tiered_f16_split_count_independence():
    c = synth.tiered_f16_case(302, 2, 16, 4, 128, 16, [1500, 999], [1200, 900], 320, softcap=30.0)
    orf, lrf = oracle_run(c)
    dc = DeviceCase(c)
    for st in (0, 16, 64, 256, 2048):
        og, lg = dc.run_np(st)
        compare(og, lg, orf, lrf, what=f"tiered f16 split_tokens={st}")


def test_tiered_f16_nonlive_rows_hold_nan():
    """Cold pool rows and ring slots that hold no live token are NaN / Inf: tiles
    that straddle the hot/cold boundary or a sequence end read whole rows and must
    mask them (p = 0, V zeroed)."""
    c = synth.tiered_f16_case(303, 3, 32, 8, 128, 16, [700, 613, 77], [451, 420, 0], 256, softcap=50.0)
    bs = c.params["block_size"]
    live_cold = np.zeros(c.k_cold.shape[:2], bool)
    live_hot = np.zeros(c.k_hot.shape[:2], bool)
    for b in range(3):
        t = np.arange(int(c.cold_lens[b]))
        live_cold[c.cold_block_table[b, t // bs], t % bs] = True
        t = np.arange(int(c.cold_lens[b]), int(c.seq_lens[b]))
        live_hot[b, t % c.hot_window] = True
    for a, live in ((c.k_cold, live_cold), (c.v_cold, live_cold), (c.k_hot, live_hot), (c.v_hot, live_hot)):
        a[~live] = np.nan
        a[~live, ..., ::3] = np.inf
    _check(c, what="tiered f16 with NaN/Inf in non-live rows")


def test_tiered_f16_boundary_anywhere_matches_oracle():
    # the same logical rows with the hot/cold boundary at several places (the oracle's
    # result is the same bit for bit; the GPU result must stay within tolerance of it)
    ref = None
    for cold in ([700, 613], [444, 357], [449, 360], [460, 613], [700, 400]):
        hw = 256
        cold = [max(c, L - hw) for c, L in zip(cold, [700, 613])]
        c = synth.tiered_f16_case(304, 2, 32, 8, 128, 16, [700, 613], cold, hw, softcap=20.0)
        orf, lrf = oracle_run(c)
        if ref is None:
            ref = (orf, lrf)
        assert np.array_equal(orf, ref[0]) and np.array_equal(lrf, ref[1])
        og, lg = DeviceCase(c).run_np()
        compare(og, lg, orf, lrf, what=f"tiered f16 cold={cold}")


# ------------------------------------------------------------ output modes

def _mode_cases():
    return [
        synth.paged_case(311, 3, 32, 8, 128, 16, lens=[900, 0, 333], kv_dtype=synth.F16),
        synth.paged_case(312, 2, 8, 4, 64, 5, lens=[300, 47], kv_dtype=synth.F32, softcap=10.0),
        synth.tiered_case(313, 2, 32, 8, 128, 16, [700, 613], [450, 420], 256, softcap=50.0),
        synth.tiered_f16_case(314, 2, 16, 8, 64, 16, [500, 16], [300, 0], 208),
        synth.sparse_case(315, 2, 32, 8, 128, 64, 64, 4, [2048, 999]),
    ]


def _f16_half_ulp(x):
    """Half the spacing of f16 values at |x| (2^-25 below the normal range)."""
    a = np.abs(np.asarray(x, np.float64))
    e = np.floor(np.log2(np.maximum(a, 2.0 ** -14)))
    return np.ldexp(1.0, (e - 11).astype(int))


@pytest.mark.parametrize("idx", range(5))
@pytest.mark.parametrize("split_tokens", [0, 64])
def test_f16_output_is_the_rounded_f32_output(idx, split_tokens):
    import torch
    case = _mode_cases()[idx]
    dc = DeviceCase(case)
    o32, l32 = dc.run(split_tokens)
    o16, l16 = dc.run(split_tokens, out_dtype=torch.float16)
    torch.cuda.synchronize()
    assert o16.dtype == torch.float16
    # same partials, same merge: the f16 store is the f32 result rounded to nearest even
    assert torch.equal(o16, o32.to(torch.float16)), f"case {idx}"
    assert torch.equal(l16, l32)
    # against the oracle: |f16(g) - r| <= |f16(g) - g| + |g - r| <= half an f16 ulp + TOL
    orf, lrf = oracle_run(case)
    g = o16.cpu().numpy().astype(np.float64)
    lse = l16.cpu().numpy()
    full = np.isfinite(lrf)
    assert np.all(g[~full] == 0.0) and np.all(lse[~full] == -np.inf)
    err = np.abs(g[full] - orf[full])
    bound = 1e-3 + _f16_half_ulp(np.maximum(np.abs(orf[full]), np.abs(g[full])))
    log(f"  f16 output case {idx}: max err {err.max():.3e}, max err / bound {(err / bound).max():.3f}")
    assert np.all(err <= bound)


@pytest.mark.parametrize("idx", range(5))
def test_lse_only(idx):
    import torch
    case = _mode_cases()[idx]
    dc = DeviceCase(case)
    o32, l32 = dc.run()
    o, lse = dc.run(want_out=False)
    torch.cuda.synchronize()
    assert o is None
    assert torch.equal(lse, l32), f"case {idx}"
    _, lrf = oracle_run(case)
    full = np.isfinite(lrf)
    lg = lse.cpu().numpy()
    assert np.all(lg[~full] == -np.inf)
    assert np.max(np.abs(lg[full] - lrf[full])) <= 1e-3


def _f16_q_cases():
    return _mode_cases() + [
        synth.paged_case(316, 2, 32, 8, 128, 16, lens=[700, 90], query_len=4),
        synth.ring_case(317, 2, 32, 8, 128, 256, [600, 100], softcap=20.0),
    ]


@pytest.mark.parametrize("idx", range(7))
def test_f16_q_input_equals_its_f32_copy(idx):
    """q stored as f16 is converted to f32 exactly, so the result must equal, bit for
    bit, the call on the f32 copy of the same values (and match the oracle on them)."""
    import torch
    case = _f16_q_cases()[idx]
    dc = DeviceCase(case)
    q16 = dc.q.half()
    dc.q = q16.float()
    o32, l32 = dc.run()
    dc.q = q16
    o16, l16 = dc.run(out_dtype=torch.float16)
    torch.cuda.synchronize()
    assert torch.equal(o16, o32.to(torch.float16)) and torch.equal(l16, l32), f"case {idx}"
    case.q = q16.float().cpu().numpy()
    orf, lrf = oracle_run(case)
    compare(o32.cpu().numpy(), l32.cpu().numpy(), orf, lrf, what=f"f16 q case {idx}")
