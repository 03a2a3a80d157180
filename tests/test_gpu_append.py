"""GPU parity of the tiered write path (quantise-on-evict append) against the
oracle: every array of the cache bit-exact after every call (integer codes,
f16 scale bits, ring contents, lengths), then decode over the appended cache."""
import numpy as np
import pytest

import oracle
from bruteforce import tiered_after_appends
from gpu_util import compare, log

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


def _host(t, like):
    return t.cpu().numpy().view(like.dtype).reshape(like.shape)


def _tokens(rng, B, T, Hkv, D):
    """f16 token rows of mixed magnitude: ordinary, tiny (subnormal f16 scales),
    all-zero and at the f16 limit, so the scale rounding is exercised."""
    out = []
    for b in range(B):
        mags = rng.choice([1.0, 1e-5, 40.0, 3e-7], size=(T[b], Hkv, 1))
        x = np.clip(rng.standard_normal((T[b], Hkv, D)) * mags, -65504, 65504).astype(np.float16)
        if T[b] > 2:
            x[1, 0] = 0
            x[2, 0] = np.float16(65504.0)
        out.append(x)
    return out


CASES = [  # (D, Hkv, hot_window, block_size, start lengths, appends)
    (128, 8, 16, 16, [0, 20, 37], 24),
    (64, 3, 5, 3, [5, 0, 11], 13),
    (128, 20, 8, 16, [8, 3], 9),       # more kv heads than waves in a workgroup
    (64, 1, 1, 4, [0, 6], 5),          # a one-slot ring evicts on every call
]


@pytest.mark.parametrize("D,Hkv,hw,bs,start,steps", CASES)
def test_append_bit_exact_with_oracle(D, Hkv, hw, bs, start, steps):
    import int8_quantized_kv_amd as dk
    rng = np.random.default_rng(D * 1000 + Hkv * 10 + hw)
    B = len(start)
    T = [s + steps for s in start]
    k = _tokens(rng, B, T, Hkv, D)
    v = _tokens(rng, B, T, Hkv, D)
    max_blocks = max(T) // bs + 2
    num_blocks = B * max_blocks
    table = rng.permutation(num_blocks).reshape(B, max_blocks).astype(np.int32)
    state = list(tiered_after_appends([k[b][:start[b]] for b in range(B)], [v[b][:start[b]] for b in range(B)],
                                      hw, table, bs, num_blocks))
    p = oracle.Params(B, Hkv, Hkv, D, block_size=bs, max_blocks_per_seq=max_blocks, num_blocks=num_blocks)
    dstate = [_dev(a) for a in state]
    dtable = _dev(table)
    names = ["k_hot", "v_hot", "k_cold", "v_cold", "k_scale", "v_scale", "seq_lens", "cold_lens"]
    log(f"append D={D} Hkv={Hkv} hw={hw} bs={bs} start={start} steps={steps}")
    for i in range(steps):
        kn = np.stack([k[b][start[b] + i] for b in range(B)])
        vn = np.stack([v[b][start[b] + i] for b in range(B)])
        state = list(oracle.append_tiered_int8(p, kn, vn, *state[:2], hw, *state[2:6], table, *state[6:]))
        dk.dattn_append_tiered_int8(_dev(kn), _dev(vn), *dstate[:6], dtable, *dstate[6:])
        for name, want, got in zip(names, state, dstate):
            g = _host(got, np.asarray(want))
            assert np.array_equal(g.view(np.uint8), np.asarray(want).view(np.uint8)), f"{name} after call {i}"


def test_append_then_decode_matches_oracle():
    """Decode over a cache the GPU built by appending, against the oracle's decode
    over the cache the oracle built."""
    import torch
    import int8_quantized_kv_amd as dk
    rng = np.random.default_rng(11)
    B, H, Hkv, D, hw, bs, steps = 3, 16, 4, 128, 64, 16, 150
    start = [0, 30, 100]
    T = [s + steps for s in start]
    k = [(rng.standard_normal((T[b], Hkv, D))).astype(np.float16) for b in range(B)]
    v = [(rng.standard_normal((T[b], Hkv, D))).astype(np.float16) for b in range(B)]
    max_blocks = max(T) // bs + 2
    num_blocks = B * max_blocks
    table = rng.permutation(num_blocks).reshape(B, max_blocks).astype(np.int32)
    state = list(tiered_after_appends([k[b][:start[b]] for b in range(B)], [v[b][:start[b]] for b in range(B)],
                                      hw, table, bs, num_blocks))
    dstate = [_dev(a) for a in state]
    dtable = _dev(table)
    for i in range(steps):
        kn = np.stack([k[b][start[b] + i] for b in range(B)])
        vn = np.stack([v[b][start[b] + i] for b in range(B)])
        dk.dattn_append_tiered_int8(_dev(kn), _dev(vn), *dstate[:6], dtable, *dstate[6:])
    want = tiered_after_appends(k, v, hw, table, bs, num_blocks)
    for name, w, g in zip(["k_cold", "k_scale", "seq_lens", "cold_lens"], [want[2], want[4], want[6], want[7]],
                          [dstate[2], dstate[4], dstate[6], dstate[7]]):
        assert np.array_equal(_host(g, w).view(np.uint8), w.view(np.uint8)), name
    q = rng.standard_normal((B, H, D)).astype(np.float32)
    out, lse = dk.dattn_decode_tiered_int8(torch.from_numpy(q).cuda(), *dstate[:6], dtable, dstate[6], dstate[7],
                                           softcap=30.0, sliding_window=100, max_seq_len=int(want[6].max()))
    p = oracle.Params(B, H, Hkv, D, sliding_window=100, softcap=30.0, block_size=bs, max_blocks_per_seq=max_blocks,
                      num_blocks=num_blocks)
    ro, rl = oracle.decode_tiered_int8(p, q, want[0], want[1], hw, want[2], want[3], want[4], want[5], table,
                                       want[6], want[7])
    compare(out.cpu().numpy().reshape(B * H, D), lse.cpu().numpy().reshape(B * H), ro, rl,
            what="decode over the appended cache")


def test_append_leaves_broken_sequences_unchanged():
    """Sequences whose lengths or needed table entry break the preconditions are
    left as they are; the others are appended."""
    import int8_quantized_kv_amd as dk
    rng = np.random.default_rng(5)
    B, Hkv, D, hw, bs = 3, 2, 64, 4, 4
    max_blocks, num_blocks = 3, 9
    table = np.array([[0, 1, 2], [3, -1, 5], [6, 7, 8]], np.int32)
    k_hot = rng.standard_normal((B, hw, Hkv, D)).astype(np.float16)
    v_hot = rng.standard_normal((B, hw, Hkv, D)).astype(np.float16)
    cold = np.zeros((num_blocks, bs, Hkv, D // 4), np.uint32)
    sc = np.zeros((num_blocks, bs, Hkv), np.float16)
    seq = np.array([8, 8, 9], np.int32)     # b=0: full ring, evicts position 4 (block 1: fine)
    cl = np.array([4, 4, 4], np.int32)      # b=1: needs block 1 -> entry -1; b=2: 5 hot > 4
    st = [k_hot, v_hot, cold, cold.copy(), sc, sc.copy(), seq, cl]
    d = [_dev(a) for a in st]
    kn = rng.standard_normal((B, Hkv, D)).astype(np.float16)
    vn = rng.standard_normal((B, Hkv, D)).astype(np.float16)
    dk.dattn_append_tiered_int8(_dev(kn), _dev(vn), *d[:6], _dev(table), *d[6:])
    got = [_host(g, a) for g, a in zip(d, st)]
    assert list(got[6]) == [9, 8, 9] and list(got[7]) == [5, 4, 4]
    assert np.array_equal(got[0][1:].view(np.uint16), k_hot[1:].view(np.uint16))
    assert np.array_equal(got[0][0, 0].view(np.uint16), kn[0].view(np.uint16))   # slot 8 % 4 = 0


@pytest.mark.parametrize("D,Hkv,W,start,steps", [(128, 8, 16, [0, 20, 37], 24), (64, 20, 5, [3, 0], 11),
                                                 (128, 1, 1, [4, 0], 3)])
def test_ring_append_bit_exact_then_decode(D, Hkv, W, start, steps):
    import torch

    import int8_quantized_kv_amd as dk
    import synth
    rng = np.random.default_rng(D + Hkv * 7 + W)
    B = len(start)
    kr = rng.standard_normal((B, W, Hkv, D)).astype(np.float16)
    vr = rng.standard_normal((B, W, Hkv, D)).astype(np.float16)
    sl = np.array(start, np.int32)
    p = oracle.Params(B, Hkv, Hkv, D, sliding_window=W, block_size=1, max_blocks_per_seq=1, num_blocks=1)
    dkr, dvr, dsl = _dev(kr), _dev(vr), _dev(sl)
    log(f"ring append D={D} Hkv={Hkv} W={W} start={start} steps={steps}")
    for i in range(steps):
        kn = rng.standard_normal((B, Hkv, D)).astype(np.float16)
        vn = rng.standard_normal((B, Hkv, D)).astype(np.float16)
        kr, vr, sl = oracle.append_ring_f16(p, kn, vn, kr, vr, sl)
        dk.dattn_append_ring_f16(_dev(kn), _dev(vn), dkr, dvr, dsl)
        torch.cuda.synchronize()
        assert np.array_equal(_host(dkr, kr).view(np.uint16), kr.view(np.uint16)), i
        assert np.array_equal(_host(dvr, vr).view(np.uint16), vr.view(np.uint16)), i
        assert np.array_equal(dsl.cpu().numpy(), sl), i
    # decode over the appended ring
    G = 4
    q = rng.standard_normal((B, Hkv * G, D)).astype(np.float32)
    case = synth.Case("ring", dict(num_seqs=B, num_heads=Hkv * G, num_kv_heads=Hkv, head_dim=D, scale=0.0, causal=1,
                                   sliding_window=W, softcap=0.0, block_size=1, max_blocks_per_seq=1, num_blocks=1,
                                   query_len=1), q, sl, None, k_hot=kr, v_hot=vr, hot_window=W)
    out, lse = dk.dattn_decode_ring_f16(_dev(q), dkr, dvr, dsl, max_seq_len=int(sl.max()))
    torch.cuda.synchronize()
    ro, rl = oracle.run(case)
    compare(out.cpu().numpy(), lse.cpu().numpy(), ro.reshape(B, Hkv * G, D), rl.reshape(B, Hkv * G),
            what="decode over the appended ring")
