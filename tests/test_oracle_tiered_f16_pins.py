"""Pins of the oracle's tiered f16 cache (paged f16 cold tier + f16 hot ring)
against a dense numpy/scipy brute force and against exact invariants: since
both tiers store the same f16 values, where the hot/cold boundary lies, how
large the ring is and whether the rows sit in a paged f16 cache instead must
not change a single bit of the result."""
import numpy as np
import pytest

import oracle
import synth
from bruteforce import attend, logical_rows

TOL = 1e-12


def _close(a, b, tol=TOL):
    a, b = np.asarray(a), np.asarray(b)
    fa, fb = np.isfinite(a), np.isfinite(b)
    assert np.array_equal(fa, fb)
    assert np.array_equal(a[~fa], b[~fb])
    if fa.any():
        err = np.max(np.abs(a[fa] - b[fb]))
        assert err <= tol * max(1.0, np.max(np.abs(b[fb]))), err


def _run(case):
    out, lse = oracle.run(case)
    p = case.params
    return out.reshape(p["num_seqs"], p["num_heads"], p["head_dim"]), lse.reshape(p["num_seqs"], p["num_heads"])


@pytest.mark.parametrize("seed", range(60))
def test_tiered_f16_matches_bruteforce(seed):
    rng = np.random.default_rng(6000 + seed)
    Hkv = int(rng.choice([1, 2, 4]))
    G = int(rng.choice([1, 2, 4]))
    D = int(rng.choice([8, 16, 64]))
    B = int(rng.integers(1, 4))
    bs = int(rng.choice([1, 3, 16]))
    hot_window = int(rng.choice([1, 7, 32, 64]))
    lens = rng.integers(0, 300, size=B)
    cold = np.array([max(0, L - int(rng.integers(0, hot_window + 1))) for L in lens])
    q_pos = None
    if rng.random() < 0.5:
        q_pos = np.array([int(rng.integers(0, max(1, L))) for L in lens], np.int32)
    case = synth.tiered_f16_case(seed, B, Hkv * G, Hkv, D, bs, lens, cold, hot_window,
                                 permute=bool(rng.integers(0, 2)), q_pos=q_pos, causal=int(rng.integers(0, 2)),
                                 window=int(rng.choice([0, 0, 1, 5, 64])),
                                 softcap=float(rng.choice([0.0, 0.0, 0.5, 5.0, 50.0])),
                                 scale=float(rng.choice([0.0, np.float32(rng.uniform(0.05, 0.5))])))
    out, lse = _run(case)
    ref_out, ref_lse = attend(case)
    _close(out, ref_out)
    _close(lse, ref_lse)


def _case(cold, hot_window, lens=(70, 45), seed=41):
    return synth.tiered_f16_case(seed, 2, 8, 2, 16, 4, list(lens), list(cold), hot_window, softcap=9.0, window=50)


def test_hot_cold_boundary_does_not_matter():
    ref_out, ref_lse = _run(_case([70, 45], 64))
    for cold in ([20, 0], [64, 10], [10, 40], [69, 44], [6, 0]):
        out, lse = _run(_case(cold, 64))
        assert np.array_equal(out, ref_out) and np.array_equal(lse, ref_lse), cold


def test_ring_size_does_not_matter():
    ref_out, ref_lse = _run(_case([20, 30], 64))
    for W in (50, 51, 97):                      # cold_len mod W != 0: the ring wraps
        out, lse = _run(_case([20, 30], W))
        assert np.array_equal(out, ref_out) and np.array_equal(lse, ref_lse), W


def test_equals_paged_f16_over_the_same_rows():
    tc = _case([33, 12], 64)
    out_t, lse_t = _run(tc)
    B, Hkv, D = 2, 2, 16
    lens = tc.seq_lens
    rows_k, rows_v = zip(*(logical_rows(tc, b) for b in range(B)))
    total = int(lens.sum())
    kc = np.concatenate(rows_k).astype(np.float16).reshape(total, 1, Hkv, D)
    vc = np.concatenate(rows_v).astype(np.float16).reshape(total, 1, Hkv, D)
    table = np.zeros((B, int(lens.max())), np.int32)
    table[0, :lens[0]] = np.arange(lens[0])
    table[1, :lens[1]] = lens[0] + np.arange(lens[1])
    pc = synth.Case("paged", dict(tc.params, block_size=1, max_blocks_per_seq=int(lens.max()), num_blocks=total),
                    tc.q, lens, None, k_cache=kc, v_cache=vc, block_table=table)
    out_p, lse_p = _run(pc)
    assert np.array_equal(out_t, out_p) and np.array_equal(lse_t, lse_p)


def test_unused_rows_are_never_read():
    """Rows of the pool and ring slots that hold no live token are overwritten with NaN;
    a result that reads any of them would turn NaN."""
    tc = _case([33, 12], 40)
    ref_out, ref_lse = _run(tc)
    live_cold = np.zeros(tc.k_cold.shape[:2], bool)
    for b in range(2):
        t = np.arange(int(tc.cold_lens[b]))
        live_cold[tc.cold_block_table[b, t // 4], t % 4] = True
    live_hot = np.zeros(tc.k_hot.shape[:2], bool)
    for b in range(2):
        t = np.arange(int(tc.cold_lens[b]), int(tc.seq_lens[b]))
        live_hot[b, t % tc.hot_window] = True
    for a, live in ((tc.k_cold, live_cold), (tc.v_cold, live_cold), (tc.k_hot, live_hot), (tc.v_hot, live_hot)):
        a[~live] = np.nan
    out, lse = _run(tc)
    assert np.array_equal(out, ref_out) and np.array_equal(lse, ref_lse)


def test_rejects_broken_lengths():
    tc = _case([33, 12], 40)
    tc.cold_lens = np.array([33, 0], np.int32)      # 45 hot tokens in a ring of 40
    with pytest.raises(oracle.OracleError):
        _run(tc)
