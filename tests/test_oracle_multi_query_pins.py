"""Pins of the oracle's multi-query decode (query_len Qn > 1: Qn query rows
per sequence, query i at position q_pos[b] + i, q_pos defaulting to
L - Qn) against the dense brute force, and against Qn single-query calls
that put the query at each of those positions: the visible set, the rows and
their order are the same, so the results must agree bit for bit."""
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
    Qn = max(1, p["query_len"])
    return (out.reshape(p["num_seqs"], Qn, p["num_heads"], p["head_dim"]),
            lse.reshape(p["num_seqs"], Qn, p["num_heads"]))


def _case(seed, rng):
    Hkv = int(rng.choice([1, 2, 4]))
    G = int(rng.choice([1, 2, 4]))
    Qn = int(rng.choice([2, 3, 4, 8]))
    D = int(rng.choice([8, 16, 64]))
    B = int(rng.integers(1, 4))
    bs = int(rng.choice([1, 3, 16]))
    lens = rng.integers(0, 300, size=B)
    q_pos = None
    if rng.random() < 0.5:
        q_pos = np.array([int(rng.integers(0, max(1, L))) for L in lens], np.int32)
    return synth.paged_case(seed, B, Hkv * G, Hkv, D, bs, lens=lens, query_len=Qn, q_pos=q_pos,
                            kv_dtype=synth.F32 if rng.random() < 0.3 else synth.F16,
                            causal=int(rng.integers(0, 2)), window=int(rng.choice([0, 0, 1, 5, 64])),
                            softcap=float(rng.choice([0.0, 0.0, 5.0])),
                            scale=float(rng.choice([0.0, np.float32(rng.uniform(0.05, 0.5))])))


@pytest.mark.parametrize("seed", range(50))
def test_multi_query_matches_bruteforce(seed):
    case = _case(seed, np.random.default_rng(9000 + seed))
    out, lse = _run(case)
    ref_out, ref_lse = attend(case)
    _close(out, ref_out)
    _close(lse, ref_lse)


@pytest.mark.parametrize("seed", range(12))
def test_multi_query_equals_single_queries_at_each_position(seed):
    case = _case(seed, np.random.default_rng(9500 + seed))
    out, lse = _run(case)
    p = case.params
    B, Qn, H = p["num_seqs"], p["query_len"], p["num_heads"]
    q0 = case.q_pos if case.q_pos is not None else (case.seq_lens - Qn).astype(np.int32)
    for i in range(Qn):
        single = synth.Case("paged", dict(p, query_len=1), np.ascontiguousarray(case.q[:, i]), case.seq_lens,
                            (q0 + i).astype(np.int32), k_cache=case.k_cache, v_cache=case.v_cache,
                            block_table=case.block_table)
        o1, l1 = oracle.run(single)
        assert np.array_equal(out[:, i], o1.reshape(B, H, -1)), i
        assert np.array_equal(lse[:, i], l1.reshape(B, H)), i


def test_query_len_one_is_the_single_query_call():
    c1 = synth.paged_case(3, 2, 8, 2, 16, 4, lens=[50, 9])
    o_a, l_a = oracle.run(c1)
    c1.params["query_len"] = 0                 # 0 and 1 both mean one query
    o_b, l_b = oracle.run(c1)
    assert np.array_equal(o_a, o_b) and np.array_equal(l_a, l_b)


def test_causal_counts_grow_by_one_per_query():
    """q = 0 and V = 1 in one dim: exp(lse) is the number of visible keys, which
    grows by one from each query to the next under the causal mask."""
    c = synth.paged_case(4, 2, 4, 1, 8, 4, lens=[40, 17], query_len=5)
    c.q[:] = 0
    c.v_cache[:] = 1
    out, lse = _run(c)
    counts = np.rint(np.exp(lse)).astype(int)
    for b, L in enumerate([40, 17]):
        assert list(counts[b, :, 0]) == [L - 4 + i for i in range(5)]
    assert np.allclose(out, 1.0)


@pytest.mark.parametrize("kind,seed", [(k, s) for k in ("tiered", "tiered_f16", "ring") for s in range(8)])
def test_multi_query_other_caches_match_bruteforce(kind, seed):
    rng = np.random.default_rng(9700 + seed)
    Hkv, G, Qn = int(rng.choice([1, 2])), int(rng.choice([1, 2, 4])), int(rng.choice([2, 3, 4]))
    B, D = 2, 16
    lens = rng.integers(0, 200, size=B)
    kw = dict(query_len=Qn, causal=int(rng.integers(0, 2)), softcap=float(rng.choice([0.0, 5.0])))
    if kind == "ring":
        case = synth.ring_case(seed, B, Hkv * G, Hkv, D, int(rng.choice([5, 16, 64])), lens, **kw)
    else:
        hw = int(rng.choice([7, 32]))
        cold = np.array([max(0, int(L) - int(rng.integers(0, hw + 1))) for L in lens])
        make = synth.tiered_case if kind == "tiered" else synth.tiered_f16_case
        case = make(seed, B, Hkv * G, Hkv, D, 3, lens, cold, hw, window=int(rng.choice([0, 20])), **kw)
    out, lse = _run(case)
    ref_out, ref_lse = attend(case)
    _close(out, ref_out)
    _close(lse, ref_lse)


def _sparse_case(seed, rng):
    Hkv, G, Qn = int(rng.choice([1, 2])), int(rng.choice([1, 2, 4])), int(rng.choice([2, 3, 4, 8]))
    B, D, bs = 2, 16, int(rng.choice([4, 8]))
    SB = bs * int(rng.choice([1, 2, 4]))
    lens = rng.integers(0, 260, size=B)
    q_pos = None
    if rng.random() < 0.4:
        q_pos = np.array([int(rng.integers(0, max(1, L))) for L in lens], np.int32)
    return synth.sparse_case(seed, B, Hkv * G, Hkv, D, bs, SB, int(rng.choice([1, 3, 4])), lens, q_pos=q_pos,
                             query_len=Qn, causal=int(rng.integers(0, 2)), window=int(rng.choice([0, 0, 30])),
                             softcap=float(rng.choice([0.0, 5.0])),
                             csr_kind=str(rng.choice(["local_strided", "random"])))


@pytest.mark.parametrize("seed", range(16))
def test_multi_query_block_sparse_matches_bruteforce(seed):
    """Each query selects the blocks of its own CSR row (row q // SB of each
    head's layout); a query before position 0 (L < Qn) selects none."""
    case = _sparse_case(seed, np.random.default_rng(9800 + seed))
    out, lse = _run(case)
    ref_out, ref_lse = attend(case)
    _close(out, ref_out)
    _close(lse, ref_lse)


@pytest.mark.parametrize("seed", range(6))
def test_multi_query_block_sparse_equals_single_queries(seed):
    case = _sparse_case(seed, np.random.default_rng(9900 + seed))
    out, lse = _run(case)
    p = case.params
    B, Qn, H = p["num_seqs"], p["query_len"], p["num_heads"]
    q0 = case.q_pos if case.q_pos is not None else (case.seq_lens - Qn).astype(np.int32)
    for i in range(Qn):
        qi = (q0 + i).astype(np.int32)
        if np.any(qi < 0):
            continue   # the single-query call takes no position below 0
        single = synth.Case("sparse", dict(p, query_len=1), np.ascontiguousarray(case.q[:, i]), case.seq_lens, qi,
                            k_cache=case.k_cache, v_cache=case.v_cache, block_table=case.block_table,
                            sparse_block=case.sparse_block, num_layouts=case.num_layouts, row_ptr=case.row_ptr,
                            col_idx=case.col_idx)
        o1, l1 = oracle.run(single)
        assert np.array_equal(out[:, i], o1.reshape(B, H, -1)), i
        assert np.array_equal(lse[:, i], l1.reshape(B, H)), i


def test_multi_query_block_sparse_query_before_position_zero_sees_nothing():
    # L = 3 < Qn = 5 without q_pos: the first two queries sit at -2 and -1; non-causal
    # so that only the missing CSR row hides the keys
    c = synth.sparse_case(5, 1, 4, 2, 16, 4, 8, 2, [3], query_len=5, causal=0)
    out, lse = _run(c)
    assert np.all(lse[0, :2] == -np.inf) and np.all(out[0, :2] == 0.0)
    assert np.all(np.isfinite(lse[0, 2:]))
