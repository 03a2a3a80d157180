"""Pins of the oracle's tiered write path (quantise-on-evict append) against
what the reading and the mathematics fix, independently of the oracle's code:
numpy's own f32 -> f16 rounding, a vectorised numpy restatement of the
quantiser, its error bound, and the cache that a history of appends must leave
(built directly from the token history)."""
import os

import numpy as np
import pytest

import oracle
from bruteforce import pack_bytes, quantize_f16_rows, tiered_after_appends


def test_f32_to_f16_exact_on_every_f16_value():
    bits = np.arange(0x10000, dtype=np.uint32).astype(np.uint16)
    vals = bits.view(np.float16)
    finite = np.isfinite(vals)
    got = np.array([oracle.f32_to_f16(float(v)) for v in vals[finite].astype(np.float32)], np.uint16)
    want = vals[finite].astype(np.float32).astype(np.float16).view(np.uint16)
    # -0 and +0 both round-trip with their sign
    assert np.array_equal(got, want)


def test_f32_to_f16_ties_overflow_and_random_match_numpy():
    pos = np.arange(0x7C00, dtype=np.uint16).view(np.float16).astype(np.float64)
    mids = ((pos[:-1] + pos[1:]) / 2).astype(np.float32)        # exact in f32: ties to even
    edges = np.array([65504.0, 65519.996, 65520.0, 1e6, 2.0 ** -24, 2.0 ** -25, 3 * 2.0 ** -26,
                      2.0 ** -14, 2.0 ** -14 - 2.0 ** -30, np.inf], np.float32)
    rng = np.random.default_rng(7)
    rand = rng.integers(0, 0x7F800000, size=20000, dtype=np.uint32).view(np.float32)
    xs = np.concatenate([mids, edges, rand])
    xs = np.concatenate([xs, -xs])
    got = np.array([oracle.f32_to_f16(float(x)) for x in xs], np.uint16)
    with np.errstate(over="ignore"):   # values past the f16 range round to inf on purpose
        want = xs.astype(np.float16).view(np.uint16)
    assert np.array_equal(got, want)


def _rows(rng, n, D):
    mags = rng.choice([1.0, 1e-3, 3e-6, 100.0, 2e4], size=(n, 1))
    x = np.clip(rng.standard_normal((n, D)) * mags, -65504.0, 65504.0).astype(np.float16)   # finite f16
    x[0] = 0                                    # an all-zero row
    x[1] = 0
    x[1, 5] = np.float16(-3.0)                  # one non-zero element
    x[2] = np.float16(65504.0) * np.sign(rng.standard_normal(D)).astype(np.float16)
    return x


@pytest.mark.parametrize("D", [64, 128])
def test_quantize_row_matches_the_reading(D):
    rng = np.random.default_rng(D)
    x = _rows(rng, 300, D)
    codes, scales = quantize_f16_rows(x)
    for r in range(x.shape[0]):
        words, s = oracle.quantize_row(x[r].view(np.uint16))
        assert s == int(scales[r].view(np.uint16)), r
        assert np.array_equal(words, pack_bytes(codes[r])), r


def _golden_rows():
    path = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden", "quantizer_rows.txt")
    rows = []
    for line in open(path):
        if line.startswith("#") or not line.strip():
            continue
        name, sbits, xs, cs = (f.strip() for f in line.split("|"))
        rows.append((name, int(sbits, 16), [float(v) for v in xs.split()], [int(v) for v in cs.split()]))
    return rows


@pytest.mark.parametrize("row", _golden_rows(), ids=lambda r: r[0])
def test_quantize_row_hand_worked_ties_and_clip(row):
    """Rows worked by hand (tests/golden/quantizer_rows.txt): ties to even at
    two scales, a subnormal f16 scale whose codes clip at 127, a zero row."""
    name, sbits, xs, codes = row
    x = np.zeros(64, np.float16)
    x[:len(xs)] = np.array(xs, np.float32).astype(np.float16)
    assert np.array_equal(x[:len(xs)].astype(np.float64), np.array(xs)), "inputs must be exact f16 values"
    words, s = oracle.quantize_row(x.view(np.uint16))
    assert s == sbits, (name, hex(s))
    want = np.zeros(64, np.int64)
    want[:len(codes)] = codes
    got = [oracle.int8_lane(int(words[d // 4]), d % 4) for d in range(64)]
    assert got == want.tolist(), name


def test_quantize_row_error_bound_and_full_range():
    rng = np.random.default_rng(3)
    x = _rows(rng, 200, 128)
    for r in range(x.shape[0]):
        words, s = oracle.quantize_row(x[r].view(np.uint16))
        s = float(np.uint16(s).view(np.float16))
        i = np.array([oracle.int8_lane(int(words[d // 4]), d % 4) for d in range(128)], np.float64)
        xr = x[r].astype(np.float64)
        assert np.all(np.abs(i) <= 127)
        if s == 0.0:
            assert np.all(i == 0) and np.max(np.abs(xr)) <= 127 * 2.0 ** -25
            continue
        # i = clip(rint(fl(x / s))): |x - i s| <= s (1/2 + |x/s| 2^-24) unless |x/s| > 127.5,
        # where the code saturates at +-127 with the sign of x (only a subnormal f16 scale,
        # rounded far below max|x| / 127, gets there)
        ratio = xr / s
        inside = np.abs(ratio) <= 127.5 - 2.0 ** -10
        assert np.all(np.abs(xr - i * s)[inside] <= s * (0.5 + 2.0 ** -17))
        assert np.all(i[~inside] == 127 * np.sign(xr[~inside]))
        if s >= 2.0 ** -14:                      # a normal scale is within 2^-11 of max|x| / 127
            assert np.all(inside) and np.max(np.abs(i)) == 127


def _history(rng, B, T, Hkv, D):
    k = [(rng.standard_normal((T[b], Hkv, D)) * 2).astype(np.float16) for b in range(B)]
    v = [(rng.standard_normal((T[b], Hkv, D)) * 2).astype(np.float16) for b in range(B)]
    return k, v


@pytest.mark.parametrize("hw,bs,start,steps", [(4, 3, [0, 5], 13), (16, 16, [0, 40], 30), (8, 5, [8, 7], 1),
                                               (8, 5, [7, 0], 2), (1, 2, [0, 3], 6)])
def test_appends_leave_the_cache_of_the_history(hw, bs, start, steps):
    """Start from the cache of a first part of each history, append the rest one
    token per call, and compare with the cache of the whole history."""
    rng = np.random.default_rng(hw * 100 + bs)
    B, Hkv, D = 2, 2, 64
    T = [s + steps for s in start]
    k, v = _history(rng, B, T, Hkv, D)
    max_blocks = max(T) // bs + 2
    num_blocks = B * max_blocks
    table = rng.permutation(num_blocks).reshape(B, max_blocks).astype(np.int32)
    state = tiered_after_appends([k[b][:start[b]] for b in range(B)], [v[b][:start[b]] for b in range(B)],
                                 hw, table, bs, num_blocks)
    p = oracle.Params(B, 2 * Hkv, Hkv, D, block_size=bs, max_blocks_per_seq=max_blocks, num_blocks=num_blocks)
    kh, vh, kc, vc, ks, vs, sl, cl = state
    for i in range(steps):
        kn = np.stack([k[b][start[b] + i] for b in range(B)])
        vn = np.stack([v[b][start[b] + i] for b in range(B)])
        kh, vh, kc, vc, ks, vs, sl, cl = oracle.append_tiered_int8(p, kn, vn, kh, vh, hw, kc, vc, ks, vs,
                                                                     table, sl, cl)
    want = tiered_after_appends(k, v, hw, table, bs, num_blocks)
    names = ["k_hot", "v_hot", "k_cold", "v_cold", "k_scale", "v_scale", "seq_lens", "cold_lens"]
    for name, g, w in zip(names, (kh, vh, kc, vc, ks, vs, sl, cl), want):
        assert np.array_equal(np.asarray(g).view(np.uint8), np.asarray(w).view(np.uint8)), name


def test_append_rejects_broken_preconditions():
    B, Hkv, D, bs, hw = 1, 1, 64, 4, 4
    p = oracle.Params(B, 1, Hkv, D, block_size=bs, max_blocks_per_seq=2, num_blocks=2)
    z16 = np.zeros((B, Hkv, D), np.float16)
    hot = np.zeros((B, hw, Hkv, D), np.float16)
    cold = np.zeros((2, bs, Hkv, D // 4), np.uint32)
    sc = np.zeros((2, bs, Hkv), np.float16)
    table = np.array([[0, 1]], np.int32)
    with pytest.raises(oracle.OracleError):     # more hot tokens than the ring holds
        oracle.append_tiered_int8(p, z16, z16, hot, hot, hw, cold, cold, sc, sc, table, np.int32([5]), np.int32([0]))
    with pytest.raises(oracle.OracleError):     # eviction needs cold block 2: not in the table
        oracle.append_tiered_int8(p, z16, z16, hot, hot, hw, cold, cold, sc, sc, table, np.int32([12]), np.int32([8]))
    with pytest.raises(oracle.OracleError):     # table entry out of the pool
        oracle.append_tiered_int8(p, z16, z16, hot, hot, hw, cold, cold, sc, sc, np.array([[0, 7]], np.int32),
                                  np.int32([8]), np.int32([4]))
