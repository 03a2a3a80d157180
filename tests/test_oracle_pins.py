"""Pins of the fp64 oracle against things other than itself.

* scalar decoders against the IEEE binary16 format (numpy's float16) and
  against hand-built words / a little-endian byte view;
* the whole attention against a dense numpy/scipy brute force on a few
  hundred seeded tiny cases;
* closed forms (constant V, zero query, single key, two keys, softcap limits);
* exact invariants (block permutation, hot/cold split, ring size, GQA
  expansion, CSR duplicates and the all-columns CSR);
* visited-set probes whose counts are fixed by enumeration.
"""
import math

import numpy as np
import pytest

import oracle
import synth
from bruteforce import attend, logical_rows, scale_of, visible_matrix

TOL = 1e-12


def _close(a, b, tol=TOL):
    a, b = np.asarray(a), np.asarray(b)
    fa, fb = np.isfinite(a), np.isfinite(b)
    assert np.array_equal(fa, fb)
    assert np.array_equal(a[~fa], b[~fb])
    if fa.any():
        err = np.max(np.abs(a[fa] - b[fb]))
        assert err <= tol * max(1.0, np.max(np.abs(b[fb]))), err


def _run(case, **kw):
    out, lse = oracle.run(case, **kw)
    p = case.params
    return out.reshape(p["num_seqs"], p["num_heads"], p["head_dim"]), lse.reshape(p["num_seqs"], p["num_heads"])


# ------------------------------------------------------------------ scalars

def test_f16_decoder_matches_binary16_for_every_pattern():
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    ref = bits.view(np.float16).astype(np.float64)
    got = np.array([oracle.f16_to_f64(int(x)) for x in bits])
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan], ref[~nan])
    assert np.array_equal(np.signbit(got[~nan]), np.signbit(ref[~nan]))


def test_int8_lanes_hand_built_word():
    # bytes from least significant: 0xFF, 0x01, 0x7F, 0x80
    assert [oracle.int8_lane(0x807F01FF, i) for i in range(4)] == [-1, 1, 127, -128]
    assert [oracle.int8_lane(0x00000080, i) for i in range(4)] == [-128, 0, 0, 0]
    assert [oracle.int8_lane(0x7F000000, i) for i in range(4)] == [0, 0, 0, 127]


def test_int8_lanes_match_little_endian_byte_view():
    rng = np.random.default_rng(7)
    words = rng.integers(0, 2 ** 32, size=2000, dtype=np.uint64).astype(np.uint32)
    ref = words.astype("<u4").view("<i1").reshape(-1, 4)
    got = np.array([[oracle.int8_lane(int(w), i) for i in range(4)] for w in words])
    assert np.array_equal(got, ref)


def test_pack_int8_is_least_significant_byte_first():
    codes = np.array([[-1, 1, 127, -128, 0, 5, -5, 64]], np.int8)
    w = synth.pack_int8(codes)
    assert w.tolist() == [[0x807F01FF, 0x40FB0500]]


@pytest.mark.parametrize("q", [0, 1, 7, 100])
def test_causal_boundary_is_inclusive(q):
    L = 200
    assert oracle.key_visible(q, q, L, 1, 0)
    assert not oracle.key_visible(q + 1, q, L, 1, 0)
    assert oracle.key_visible(q + 1, q, L, 0, 0)        # without causal, later keys stay visible
    assert not oracle.key_visible(L, q, L, 0, 0)         # never past the sequence


@pytest.mark.parametrize("W", [1, 2, 5, 64])
def test_window_keeps_exactly_the_last_W_keys(W):
    L = 150
    for q in range(L):
        vis = [t for t in range(L) if oracle.key_visible(t, q, L, 1, W)]
        assert len(vis) == min(W, q + 1)
        assert vis[0] == max(0, q - W + 1) and vis[-1] == q
        # window without causal keeps the future
        vis_nc = [t for t in range(L) if oracle.key_visible(t, q, L, 0, W)]
        assert vis_nc[0] == max(0, q - W + 1) and vis_nc[-1] == L - 1


def test_ring_slots_wrap():
    assert [oracle.ring_slot(t, 4) for t in range(10)] == [0, 1, 2, 3, 0, 1, 2, 3, 0, 1]
    assert oracle.ring_slot(7680, 512) == 0 and oracle.ring_slot(8191, 512) == 511


# ------------------------------------------------------------ brute force

def _rand_common(rng):
    Hkv = int(rng.choice([1, 2, 4]))
    G = int(rng.choice([1, 2, 4]))
    D = int(rng.choice([8, 16, 64]))
    B = int(rng.integers(1, 4))
    causal = int(rng.integers(0, 2))
    window = int(rng.choice([0, 0, 1, 5, 64]))
    softcap = float(rng.choice([0.0, 0.0, 0.5, 5.0, 50.0]))
    scale = float(rng.choice([0.0, np.float32(rng.uniform(0.05, 0.5))]))
    return B, Hkv * G, Hkv, D, causal, window, softcap, scale


def _rand_qpos(rng, lens):
    if rng.random() < 0.5:
        return None
    return np.array([int(rng.integers(0, max(1, L))) if L > 0 else 0 for L in lens], np.int32)


@pytest.mark.parametrize("seed", range(100))
def test_paged_matches_bruteforce(seed):
    rng = np.random.default_rng(1000 + seed)
    B, H, Hkv, D, causal, window, softcap, scale = _rand_common(rng)
    bs = int(rng.choice([1, 3, 16]))
    lens = rng.integers(0, 300, size=B)
    if rng.random() < 0.1:
        lens[0] = 0
    dt = synth.F32 if rng.random() < 0.5 else synth.F16
    case = synth.paged_case(seed, B, H, Hkv, D, bs, lens=lens, kv_dtype=dt, permute=bool(rng.integers(0, 2)),
                            q_pos=_rand_qpos(rng, lens), causal=causal, window=window, softcap=softcap,
                            scale=scale, extra_blocks=int(rng.integers(0, 3)))
    out, lse = _run(case)
    ref_out, ref_lse = attend(case)
    _close(out, ref_out)
    _close(lse, ref_lse)


@pytest.mark.parametrize("seed", range(60))
def test_tiered_matches_bruteforce(seed):
    rng = np.random.default_rng(2000 + seed)
    B, H, Hkv, D, causal, window, softcap, scale = _rand_common(rng)
    bs = int(rng.choice([1, 3, 16]))
    hot_window = int(rng.choice([1, 7, 32, 64]))
    lens = rng.integers(0, 300, size=B)
    cold = np.array([max(0, L - int(rng.integers(0, hot_window + 1))) for L in lens])
    case = synth.tiered_case(seed, B, H, Hkv, D, bs, lens, cold, hot_window, permute=bool(rng.integers(0, 2)),
                             q_pos=_rand_qpos(rng, lens), causal=causal, window=window, softcap=softcap,
                             scale=scale)
    # some raw words so that -128 and arbitrary byte patterns occur
    flat = case.k_cold.reshape(-1)
    idx = rng.integers(0, flat.size, size=max(1, flat.size // 50))
    flat[idx] = rng.integers(0, 2 ** 32, size=idx.size, dtype=np.uint64).astype(np.uint32)
    out, lse = _run(case)
    ref_out, ref_lse = attend(case)
    _close(out, ref_out)
    _close(lse, ref_lse)


@pytest.mark.parametrize("seed", range(60))
def test_sparse_matches_bruteforce(seed):
    rng = np.random.default_rng(3000 + seed)
    B, H, Hkv, D, causal, window, softcap, scale = _rand_common(rng)
    bs = int(rng.choice([1, 2, 4]))
    SB = bs * int(rng.choice([1, 2, 4]))
    NL = int(rng.integers(1, 5))
    lens = rng.integers(1, 200, size=B)
    case = synth.sparse_case(seed, B, H, Hkv, D, bs, SB, NL, lens, q_pos=_rand_qpos(rng, lens), causal=causal,
                             window=window, softcap=softcap, scale=scale,
                             csr_kind="random" if seed % 2 else "local_strided")
    out, lse = _run(case)
    ref_out, ref_lse = attend(case)
    _close(out, ref_out)
    _close(lse, ref_lse)


# ------------------------------------------------------------- closed forms

def test_constant_values_give_that_constant():
    case = synth.paged_case(11, 2, 8, 2, 16, 4, lens=[57, 90], softcap=5.0, window=20, causal=1)
    c = np.random.default_rng(0).standard_normal((2, 16)).astype(np.float16)   # one vector per kv head
    case.v_cache[:] = c[None, None]
    out, _ = _run(case)
    G = 4
    for h in range(8):
        np.testing.assert_allclose(out[:, h], np.broadcast_to(c[h // G].astype(np.float64), (2, 16)),
                                   rtol=0, atol=1e-14)


def test_zero_query_gives_mean_and_log_count():
    case = synth.paged_case(12, 2, 4, 2, 8, 3, lens=[40, 77], window=9, q_pos=[30, 76])
    case.q[:] = 0
    out, lse = _run(case)
    for b in range(2):
        K, V = logical_rows(case, b)
        vis = visible_matrix(case, b)
        for h in range(4):
            g = h // 2
            n = int(vis[h].sum())
            assert abs(lse[b, h] - math.log(n)) <= 1e-14
            np.testing.assert_allclose(out[b, h], V[vis[h], g].mean(axis=0), rtol=0, atol=1e-14)


def test_single_visible_key():
    # window 1: only key q is visible: out = v_q, lse = s_q
    case = synth.paged_case(13, 1, 4, 1, 16, 5, lens=[33], window=1, q_pos=[20], softcap=3.0)
    out, lse = _run(case)
    K, V = logical_rows(case, 0)
    sc = scale_of(case.params)
    for h in range(4):
        s = sc * float(np.dot(case.q[0, h].astype(np.float64), K[20, 0]))
        s = 3.0 * math.tanh(s / 3.0)
        assert abs(lse[0, h] - s) <= 1e-14
        np.testing.assert_array_equal(out[0, h], V[20, 0])


def test_two_keys_logistic_weights():
    case = synth.paged_case(14, 1, 2, 1, 8, 1, lens=[2], kv_dtype=synth.F32)
    out, lse = _run(case)
    K, V = logical_rows(case, 0)
    sc = scale_of(case.params)
    for h in range(2):
        s1 = sc * float(np.dot(case.q[0, h].astype(np.float64), K[0, 0]))
        s2 = sc * float(np.dot(case.q[0, h].astype(np.float64), K[1, 0]))
        w1 = 1.0 / (1.0 + math.exp(s2 - s1))
        w2 = 1.0 / (1.0 + math.exp(s1 - s2))
        np.testing.assert_allclose(out[0, h], w1 * V[0, 0] + w2 * V[1, 0], rtol=0, atol=1e-14)
        assert abs(lse[0, h] - (max(s1, s2) + math.log1p(math.exp(-abs(s1 - s2))))) <= 1e-14


def test_softcap_limits():
    base = synth.paged_case(15, 2, 4, 2, 16, 4, lens=[50, 61])
    out0, lse0 = _run(base)
    huge = synth.paged_case(15, 2, 4, 2, 16, 4, lens=[50, 61], softcap=1e9)
    out1, lse1 = _run(huge)
    _close(out1, out0, 1e-13)
    _close(lse1, lse0, 1e-13)
    # large scores through a small cap: every capped score lies in (-cap, cap)
    cap = 2.0
    big = synth.paged_case(16, 2, 4, 2, 16, 4, lens=[50, 61], softcap=cap)
    big.q *= 1000.0
    _, lse = _run(big)
    for b, n in enumerate([50, 61]):
        assert np.all(lse[b] < math.log(n) + cap) and np.all(lse[b] > math.log(n) - cap)


def test_empty_visible_set_gives_zero_and_minus_inf():
    case = synth.paged_case(17, 2, 4, 2, 8, 4, lens=[0, 9])
    out, lse = _run(case)
    assert np.all(out[0] == 0) and np.all(lse[0] == -np.inf)
    assert np.all(np.isfinite(lse[1]))


# ------------------------------------------------------------ invariants

def test_block_permutation_is_exact():
    case = synth.paged_case(21, 3, 8, 2, 16, 4, lens=[37, 64, 5], softcap=7.0, window=30)
    out0, lse0 = _run(case)
    rng = np.random.default_rng(5)
    pi = rng.permutation(case.k_cache.shape[0])
    k = np.empty_like(case.k_cache)
    v = np.empty_like(case.v_cache)
    k[pi] = case.k_cache
    v[pi] = case.v_cache
    case.k_cache, case.v_cache, case.block_table = k, v, pi[case.block_table].astype(np.int32)
    out1, lse1 = _run(case)
    assert np.array_equal(out0, out1) and np.array_equal(lse0, lse1)


def _exact_tiered(cold, hot_window, seed=31, lens=(70, 45)):
    return synth.tiered_case(seed, 2, 8, 2, 16, 4, list(lens), list(cold), hot_window, exact=True, softcap=9.0,
                             window=50)


def test_hot_cold_split_point_is_exact_when_int8_round_trips():
    ref_out, ref_lse = _run(_exact_tiered([70, 45], 64))
    for cold in ([20, 0], [64, 10], [10, 40], [69, 44]):
        out, lse = _run(_exact_tiered(cold, 64))
        assert np.array_equal(out, ref_out) and np.array_equal(lse, ref_lse)


def test_ring_size_does_not_matter():
    ref_out, ref_lse = _run(_exact_tiered([20, 30], 64))
    for W in (50, 51, 97):                      # cold_len mod W != 0: the ring wraps
        out, lse = _run(_exact_tiered([20, 30], W))
        assert np.array_equal(out, ref_out) and np.array_equal(lse, ref_lse)


def test_tiered_equals_paged_on_the_f16_copy():
    tc = _exact_tiered([33, 12], 64)
    out_t, lse_t = _run(tc)
    # the same logical rows as an f16 paged cache, block size 1, identity table
    B, Hkv, D = 2, 2, 16
    lens = tc.seq_lens
    rows_k, rows_v = [], []
    for b in range(B):
        K, V = logical_rows(tc, b)
        rows_k.append(K)
        rows_v.append(V)
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


def test_gqa_equals_expanded_mha():
    case = synth.paged_case(41, 2, 8, 2, 16, 4, lens=[29, 44], softcap=4.0)
    out0, lse0 = _run(case)
    G = 4
    case.k_cache = np.repeat(case.k_cache, G, axis=2)
    case.v_cache = np.repeat(case.v_cache, G, axis=2)
    case.params = dict(case.params, num_kv_heads=8)
    out1, lse1 = _run(case)
    assert np.array_equal(out0, out1) and np.array_equal(lse0, lse1)


def test_csr_duplicates_carry_no_extra_mass():
    case = synth.sparse_case(51, 2, 8, 2, 16, 2, 4, 3, [90, 61], csr_kind="random")
    out0, lse0 = _run(case)
    rows = [[list(dict.fromkeys(r)) for r in lay] for lay in case.extra["rows"]]
    case.row_ptr, case.col_idx = synth.csr_from_rows(rows)
    out1, lse1 = _run(case)
    assert np.array_equal(out0, out1) and np.array_equal(lse0, lse1)


def test_all_columns_csr_equals_dense_causal():
    sp = synth.sparse_case(52, 2, 8, 2, 16, 2, 4, 2, [90, 61], window=17)
    R = sp.row_ptr.shape[1] - 1
    rows = [[list(range(r + 1)) for r in range(R)] for _ in range(2)]
    sp.row_ptr, sp.col_idx = synth.csr_from_rows(rows)
    out_s, lse_s = _run(sp)
    pc = synth.Case("paged", sp.params, sp.q, sp.seq_lens, None, k_cache=sp.k_cache, v_cache=sp.v_cache,
                    block_table=sp.block_table)
    out_p, lse_p = _run(pc)
    assert np.array_equal(out_s, out_p) and np.array_equal(lse_s, lse_p)


# ------------------------------------------------------- visited-set probes

def _onehot_values(case, lens):
    """V[t][j] = 1 iff floor(t / bs) mod D == j, written through the block table."""
    p = case.params
    bs, D = p["block_size"], p["head_dim"]
    case.v_cache[:] = 0
    for b, L in enumerate(lens):
        t = np.arange(L)
        case.v_cache[case.block_table[b, t // bs], t % bs, :, (t // bs) % D] = 1


@pytest.mark.parametrize("kind", ["paged", "sparse"])
def test_visited_counts(kind):
    lens = [203, 150]
    if kind == "paged":
        case = synth.paged_case(61, 2, 4, 2, 16, 3, lens=lens, window=100, q_pos=[180, 149])
    else:
        case = synth.sparse_case(61, 2, 4, 2, 16, 3, 6, 3, lens, q_pos=[180, 149], csr_kind="random")
    case.q[:] = 0
    _onehot_values(case, lens)
    out, lse = _run(case)
    bs, D = 3, 16
    for b, L in enumerate(lens):
        vis = visible_matrix(case, b)
        t = np.arange(L)
        for h in range(4):
            n = int(vis[h].sum())
            assert round(math.exp(lse[b, h])) == n
            want = np.bincount(((t // bs) % D)[vis[h]], minlength=D)
            assert np.array_equal(np.rint(out[b, h] * n).astype(int), want)


def test_pairs_subset_matches_full_run():
    case = synth.paged_case(71, 3, 8, 4, 16, 4, lens=[40, 12, 77])
    out, lse = oracle.run(case)
    pairs = [23, 0, 9, 9]
    o2, l2 = oracle.run(case, pairs=pairs)
    assert np.array_equal(o2, out[pairs]) and np.array_equal(l2, lse[pairs])


def _golden(name):
    import os
    path = os.path.join(os.path.dirname(__file__), "golden", name)
    rows = []
    for line in open(path):
        line = line.split("#")[0].strip()
        if line:
            rows.append(line.split())
    return rows


def test_golden_int8_words():
    for row in _golden("int8_words.txt"):
        w = int(row[0], 16)
        assert [oracle.int8_lane(w, i) for i in range(4)] == [int(x) for x in row[1:]]


def test_golden_f16_values():
    for bits, val in _golden("f16_values.txt"):
        assert oracle.f16_to_f64(int(bits, 16)) == float(val)
