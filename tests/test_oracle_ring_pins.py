"""Pins of the oracle's sliding-window ring cache (token t at slot t mod W,
the last W tokens resident) against the dense brute force and against the
paged f16 oracle path over the whole token history: with the query at the
last token, a window of W keys is exactly what the ring holds, so the two
must agree bit for bit."""
import numpy as np
import pytest

import oracle
import synth
from bruteforce import attend

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


@pytest.mark.parametrize("seed", range(50))
def test_ring_matches_bruteforce(seed):
    rng = np.random.default_rng(8000 + seed)
    Hkv = int(rng.choice([1, 2, 4]))
    G = int(rng.choice([1, 2, 4]))
    D = int(rng.choice([8, 16, 64]))
    B = int(rng.integers(1, 4))
    W = int(rng.choice([1, 5, 16, 64]))
    lens = rng.integers(0, 300, size=B)
    q_pos = None
    if rng.random() < 0.5:
        q_pos = np.array([int(rng.integers(0, max(1, L))) for L in lens], np.int32)
    case = synth.ring_case(seed, B, Hkv * G, Hkv, D, W, lens, q_pos=q_pos, causal=int(rng.integers(0, 2)),
                           softcap=float(rng.choice([0.0, 0.0, 5.0, 50.0])),
                           scale=float(rng.choice([0.0, np.float32(rng.uniform(0.05, 0.5))])))
    out, lse = _run(case)
    ref_out, ref_lse = attend(case)
    _close(out, ref_out)
    _close(lse, ref_lse)


def _paged_history(rc, W):
    """The ring case's whole token history as a paged f16 cache (block size 1, identity table)."""
    B = rc.params["num_seqs"]
    lens = rc.seq_lens
    kh, vh = rc.extra["k_history"], rc.extra["v_history"]
    Lmax = kh.shape[1]
    kc = kh.reshape(B * Lmax, 1, *kh.shape[2:])
    vc = vh.reshape(B * Lmax, 1, *vh.shape[2:])
    table = (np.arange(B)[:, None] * Lmax + np.arange(Lmax)[None, :]).astype(np.int32)
    params = dict(rc.params, block_size=1, max_blocks_per_seq=Lmax, num_blocks=B * Lmax, sliding_window=W)
    return synth.Case("paged", params, rc.q, lens, None, k_cache=kc, v_cache=vc, block_table=table)


@pytest.mark.parametrize("W,lens", [(16, [100, 7, 16, 17]), (1, [5, 1]), (64, [300, 64, 65, 3]), (50, [51, 149])])
def test_ring_equals_paged_history_with_window(W, lens):
    rc = synth.ring_case(W * 7, len(lens), 8, 2, 16, W, lens, softcap=9.0)
    out_r, lse_r = _run(rc)
    out_p, lse_p = _run(_paged_history(rc, W))
    assert np.array_equal(out_r, out_p) and np.array_equal(lse_r, lse_p)


def test_earlier_query_sees_only_resident_keys():
    """A query before the last token: its window reaches back past the ring, but only
    resident tokens (the last W) can be seen; the paged history with the window
    restricted to those tokens agrees exactly."""
    W, lens = 32, [100, 80]
    qp = np.array([90, 60], np.int32)      # windows [59, 90] and [29, 60]; resident [68, 99] and [48, 79]
    rc = synth.ring_case(5, 2, 8, 2, 16, W, lens, q_pos=qp, causal=1)
    out_r, lse_r = _run(rc)
    pc = _paged_history(rc, 0)
    # resident keys visible to the query: [max(L-W, q-W+1), q]; as a window from q that is q - (L-W) + 1 keys
    for b in range(2):
        lo = max(lens[b] - W, int(qp[b]) - W + 1)
        pcb = synth.Case("paged", dict(pc.params, num_seqs=1, sliding_window=int(qp[b]) - lo + 1), pc.q[b:b + 1],
                         pc.seq_lens[b:b + 1], qp[b:b + 1], k_cache=pc.k_cache, v_cache=pc.v_cache,
                         block_table=pc.block_table[b:b + 1])
        out_p, lse_p = _run(pcb)
        assert np.array_equal(out_r[b:b + 1], out_p) and np.array_equal(lse_r[b:b + 1], lse_p)


def test_unfilled_slots_are_never_read():
    rc = synth.ring_case(9, 3, 8, 2, 16, 40, [10, 0, 39], softcap=9.0)
    ref = _run(rc)
    for b, L in enumerate(rc.seq_lens):
        rc.k_hot[b, int(L):] = np.nan
        rc.v_hot[b, int(L):] = np.nan
    out, lse = _run(rc)
    assert np.array_equal(out, ref[0]) and np.array_equal(lse, ref[1])
    assert np.all(out[1] == 0) and np.all(lse[1] == -np.inf)


def test_ring_needs_a_window():
    rc = synth.ring_case(9, 1, 8, 2, 16, 4, [10])
    rc.params["sliding_window"] = 0
    with pytest.raises(oracle.OracleError):
        _run(rc)


# ----------------------------------------------------------- the write path

def _ring_of_history(k_hist, v_hist, lens, W):
    """The ring a token history must leave: slot t mod W holds token t for the last W
    tokens of each sequence; slots no token reached keep their initial +-300."""
    B, _, Hkv, D = k_hist.shape
    kr = np.full((B, W, Hkv, D), 300.0, np.float16)
    vr = np.full((B, W, Hkv, D), -300.0, np.float16)
    for b, L in enumerate(lens):
        for t in range(max(0, L - W), L):
            kr[b, t % W] = k_hist[b, t]
            vr[b, t % W] = v_hist[b, t]
    return kr, vr


@pytest.mark.parametrize("W,start,steps", [(4, [0, 3], 9), (16, [20, 0], 20), (1, [2, 5], 3), (7, [7, 6], 1)])
def test_ring_appends_leave_the_ring_of_the_history(W, start, steps):
    rng = np.random.default_rng(W * 31 + steps)
    B, Hkv, D = 2, 2, 16
    T = [s + steps for s in start]
    k = rng.standard_normal((B, max(T), Hkv, D)).astype(np.float16)
    v = rng.standard_normal((B, max(T), Hkv, D)).astype(np.float16)
    kr, vr = _ring_of_history(k, v, start, W)
    sl = np.array(start, np.int32)
    p = oracle.Params(B, 2 * Hkv, Hkv, D, sliding_window=W, block_size=1, max_blocks_per_seq=1, num_blocks=1)
    for i in range(steps):
        kn = np.stack([k[b, start[b] + i] for b in range(B)])
        vn = np.stack([v[b, start[b] + i] for b in range(B)])
        kr, vr, sl = oracle.append_ring_f16(p, kn, vn, kr, vr, sl)
    want_k, want_v = _ring_of_history(k, v, T, W)
    assert np.array_equal(kr.view(np.uint16), want_k.view(np.uint16))
    assert np.array_equal(vr.view(np.uint16), want_v.view(np.uint16))
    assert list(sl) == T


def test_ring_append_rejects_a_missing_window():
    p = oracle.Params(1, 2, 1, 16, sliding_window=0, block_size=1, max_blocks_per_seq=1, num_blocks=1)
    z = np.zeros((1, 1, 16), np.float16)
    with pytest.raises(oracle.OracleError):
        oracle.append_ring_f16(p, z, z, np.zeros((1, 4, 1, 16), np.float16), np.zeros((1, 4, 1, 16), np.float16),
                               np.int32([3]))
