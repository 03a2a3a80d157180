"""GPU parity of multi-query decode (Qn query rows per sequence, query i at
q_pos[b] + i; the MFMA columns hold the Qn * G (query, head) pairs of a kv
head, 16 per wave) against the fp64 oracle."""
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


def _check(case, split_tokens=0, what="", **over):
    log(f"case mq {what} split_tokens={split_tokens}")
    og, lg = DeviceCase(case).run_np(split_tokens, **over)
    orf, lrf = oracle_run(case)
    return compare(og, lg, orf, lrf, what=what)


@pytest.mark.parametrize("qn", [2, 4])
@pytest.mark.parametrize("split_tokens", [0, 64])
def test_mq_paged_f16_small(qn, split_tokens):
    c = synth.paged_case(501, 4, 32, 8, 128, 16, len_range=(512, 1200), kv_dtype=synth.F16, query_len=qn)
    _check(c, split_tokens, what=f"paged f16 G4 Qn{qn}")


@pytest.mark.parametrize("G,qn", [(8, 2), (1, 16), (2, 8), (4, 3)])
def test_mq_column_limits(G, qn):
    c = synth.paged_case(502 + G, 3, 4 * G, 4, 128, 16, lens=[700, 33, 5], kv_dtype=synth.F16, query_len=qn,
                         softcap=30.0, window=200)
    _check(c, what=f"G{G} Qn{qn} window 200 cap 30")


def test_mq_paged_f32_d64():
    c = synth.paged_case(503, 2, 8, 2, 64, 5, lens=[300, 47], kv_dtype=synth.F32, query_len=3, causal=1)
    _check(c, what="paged f32 D64 bs5 Qn3")


def test_mq_sequences_shorter_than_the_queries():
    # q_pos defaults to L - Qn: queries before position 0 see nothing (causal)
    c = synth.paged_case(504, 4, 16, 4, 128, 16, lens=[2, 0, 1, 40], kv_dtype=synth.F16, query_len=4)
    _check(c, what="L < Qn")


def _rand_case(seed):
    rng = np.random.default_rng(95_000 + seed)
    D = int(rng.choice([64, 128]))
    G = int(rng.choice([1, 2, 4, 8]))
    qn = int(rng.choice([q for q in (2, 3, 4, 5, 8, 16) if q * G <= 16]))
    Hkv = int(rng.choice([1, 2, 3, 4, 8]))
    B = int(rng.integers(1, 4))
    lens = rng.integers(0, 900, size=B)
    qp = None
    if rng.random() < 0.4:
        qp = np.array([int(rng.integers(0, max(1, L))) for L in lens], np.int32)
    bs = int(rng.choice([1, 3, 16, 64]))
    return synth.paged_case(seed, B, Hkv * G, Hkv, D, bs, lens=lens, query_len=qn, q_pos=qp,
                            kv_dtype=synth.F32 if rng.random() < 0.25 else synth.F16,
                            causal=int(rng.random() < 0.85), window=int(rng.choice([0, 0, 1, 17, 200])),
                            softcap=float(rng.choice([0.0, 0.0, 5.0, 50.0])),
                            scale=float(rng.choice([0.0, np.float32(rng.uniform(0.03, 0.3))])))


@pytest.mark.parametrize("seed", range(24))
def test_mq_random_sweep(seed):
    case = _rand_case(seed)
    st = int(np.random.default_rng(seed).choice([0, 0, 16, 48, 256]))
    p = case.params
    _check(case, split_tokens=st,
           what=f"seed{seed} B{p['num_seqs']} Qn{p['query_len']} H{p['num_heads']}/{p['num_kv_heads']} "
                f"D{p['head_dim']} bs{p['block_size']} W{p['sliding_window']} cap{p['softcap']}")


def test_mq_f16_output_and_lse_only():
    import torch
    c = synth.paged_case(505, 2, 32, 8, 128, 16, lens=[900, 300], kv_dtype=synth.F16, query_len=4)
    dc = DeviceCase(c)
    o32, l32 = dc.run()
    o16, l16 = dc.run(out_dtype=torch.float16)
    o_none, l_only = dc.run(want_out=False)
    torch.cuda.synchronize()
    assert tuple(o16.shape) == (2, 4, 32, 128) and tuple(l_only.shape) == (2, 4, 32) and o_none is None
    assert torch.equal(o16, o32.to(torch.float16))
    assert torch.equal(l16, l32) and torch.equal(l_only, l32)
    orf, lrf = oracle_run(c)
    compare(o32.cpu().numpy(), l32.cpu().numpy(), orf, lrf, what="mq f32 out")


@pytest.mark.parametrize("kind", ["tiered", "tiered_f16", "ring"])
@pytest.mark.parametrize("split_tokens", [0, 48])
def test_mq_other_caches(kind, split_tokens):
    kw = dict(query_len=4, softcap=50.0)
    if kind == "ring":
        c = synth.ring_case(510, 3, 32, 8, 128, 256, [1000, 100, 257], **kw)
    else:
        make = synth.tiered_case if kind == "tiered" else synth.tiered_f16_case
        c = make(511, 2, 32, 8, 128, 16, [700, 613], [450, 420], 256, window=300, **kw)
    _check(c, split_tokens, what=f"{kind} Qn4")


@pytest.mark.parametrize("seed", range(12))
def test_mq_other_caches_sweep(seed):
    rng = np.random.default_rng(97_000 + seed)
    kind = ["tiered", "tiered_f16", "ring"][seed % 3]
    G = int(rng.choice([1, 2, 4, 8]))
    qn = int(rng.choice([q for q in (2, 3, 4, 8) if q * G <= 16]))
    Hkv = int(rng.choice([1, 2, 4, 8]))
    D = int(rng.choice([64, 128]))
    B = int(rng.integers(1, 4))
    lens = rng.integers(0, 900, size=B)
    kw = dict(query_len=qn, causal=int(rng.random() < 0.85), softcap=float(rng.choice([0.0, 5.0, 50.0])))
    if kind == "ring":
        case = synth.ring_case(seed, B, Hkv * G, Hkv, D, int(rng.choice([16, 50, 128])), lens, **kw)
    else:
        hw = int(rng.choice([16, 50, 128]))
        cold = np.array([max(0, int(L) - int(rng.integers(0, hw + 1))) for L in lens])
        make = synth.tiered_case if kind == "tiered" else synth.tiered_f16_case
        case = make(seed, B, Hkv * G, Hkv, D, int(rng.choice([5, 16])), lens, cold, hw,
                    window=int(rng.choice([0, 0, 17, 200])), **kw)
    st = int(np.random.default_rng(seed).choice([0, 0, 16, 256]))
    _check(case, st, what=f"seed{seed} {kind} B{B} Qn{qn} G{G} Hkv{Hkv} D{D}")


# More than 16 (query, head) rows per kv head: the rows are cut into blocks of
# 16, one wave each, and the row blocks of a kv head share a workgroup.
@pytest.mark.parametrize("G,qn,Hkv", [(4, 5, 8), (4, 8, 2), (4, 12, 1), (4, 16, 8), (8, 16, 4), (1, 100, 2),
                                      (2, 40, 3), (8, 9, 1), (1, 128, 1)])
@pytest.mark.parametrize("split_tokens", [0, 64])
def test_mq_row_blocks(G, qn, Hkv, split_tokens):
    c = synth.paged_case(520 + qn, 2, Hkv * G, Hkv, 128, 16, lens=[900, qn + 37], kv_dtype=synth.F16, query_len=qn,
                         softcap=30.0 if qn % 2 else 0.0, window=300 if G == 4 else 0)
    _check(c, split_tokens, what=f"rows {G * qn} G{G} Qn{qn} Hkv{Hkv}")


@pytest.mark.parametrize("kind", ["tiered", "tiered_f16", "ring"])
@pytest.mark.parametrize("split_tokens", [0, 48])
def test_mq_row_blocks_other_caches(kind, split_tokens):
    kw = dict(query_len=12, softcap=50.0)
    if kind == "ring":
        c = synth.ring_case(530, 3, 32, 8, 128, 256, [1000, 100, 257], **kw)
    else:
        make = synth.tiered_case if kind == "tiered" else synth.tiered_f16_case
        c = make(531, 2, 32, 8, 128, 16, [700, 613], [450, 420], 256, window=300, **kw)
    _check(c, split_tokens, what=f"{kind} Qn12 (48 rows)")


def test_mq_row_blocks_f32_d64_and_short_sequences():
    # q_pos defaults to L - Qn: the early queries of a short sequence see nothing
    c = synth.paged_case(532, 4, 32, 8, 64, 5, lens=[3, 0, 1, 70], kv_dtype=synth.F32, query_len=20)
    _check(c, what="paged f32 D64 Qn20 (80 rows), L < Qn")


def test_mq_row_blocks_f16_q_and_output_modes():
    import torch
    c = synth.paged_case(533, 2, 32, 8, 128, 16, lens=[900, 300], kv_dtype=synth.F16, query_len=16)
    dc = DeviceCase(c)
    q16 = dc.q.half()
    dc.q = q16.float()           # the f32 copy of f16 values: an f16 q must give the same bits
    o32, l32 = dc.run()
    o16, l16 = dc.run(out_dtype=torch.float16)
    o_none, l_only = dc.run(want_out=False)
    dc.q = q16
    oq, lq = dc.run()
    torch.cuda.synchronize()
    assert tuple(o16.shape) == (2, 16, 32, 128) and o_none is None
    assert torch.equal(o16, o32.to(torch.float16)) and torch.equal(l16, l32) and torch.equal(l_only, l32)
    assert torch.equal(oq, o32) and torch.equal(lq, l32)
    c.q = q16.float().cpu().numpy()
    orf, lrf = oracle_run(c)
    compare(o32.cpu().numpy(), l32.cpu().numpy(), orf, lrf, what="Qn16 (64 rows) f16 q")


@pytest.mark.parametrize("seed", range(16))
def test_mq_row_blocks_random_sweep(seed):
    rng = np.random.default_rng(99_000 + seed)
    kind = ["paged", "tiered", "tiered_f16", "ring"][seed % 4]
    G = int(rng.choice([1, 2, 4, 8]))
    qn = int(rng.integers(16 // G + 1, 128 // G + 1))
    Hkv = int(rng.choice([1, 2, 3, 4, 8]))
    D = int(rng.choice([64, 128]))
    B = int(rng.integers(1, 4))
    lens = rng.integers(0, 700, size=B)
    kw = dict(query_len=qn, causal=int(rng.random() < 0.85), softcap=float(rng.choice([0.0, 5.0, 50.0])))
    if kind == "paged":
        case = synth.paged_case(seed, B, Hkv * G, Hkv, D, int(rng.choice([3, 16])), lens=lens,
                                kv_dtype=synth.F32 if rng.random() < 0.25 else synth.F16,
                                window=int(rng.choice([0, 0, 17, 200])), **kw)
    elif kind == "ring":
        case = synth.ring_case(seed, B, Hkv * G, Hkv, D, int(rng.choice([16, 50, 128])), lens, **kw)
    else:
        hw = int(rng.choice([16, 50, 128]))
        cold = np.array([max(0, int(L) - int(rng.integers(0, hw + 1))) for L in lens])
        make = synth.tiered_case if kind == "tiered" else synth.tiered_f16_case
        case = make(seed, B, Hkv * G, Hkv, D, int(rng.choice([5, 16])), lens, cold, hw,
                    window=int(rng.choice([0, 0, 17, 200])), **kw)
    st = int(np.random.default_rng(seed).choice([0, 0, 16, 256]))
    _check(case, st, what=f"seed{seed} {kind} B{B} Qn{qn} G{G} rows {qn * G} Hkv{Hkv} D{D}")


# The block-sparse cache: each query takes the CSR row of its own position; the
# union list carries one mask bit per (query, head) column.
@pytest.mark.parametrize("G,qn", [(4, 4), (8, 2), (1, 16), (2, 3)])
@pytest.mark.parametrize("split_tokens", [0, 128])
def test_mq_block_sparse(G, qn, split_tokens):
    c = synth.sparse_case(540 + qn, 2, 4 * G, 4, 128, 16, 64, 4, [2000, 700], query_len=qn, softcap=30.0,
                          csr_kind="random" if qn % 2 else "local_strided")
    _check(c, split_tokens, what=f"sparse G{G} Qn{qn}")


def test_mq_block_sparse_gather_and_short_sequences():
    # block size 5 (tiles gathered row by row), sparse blocks of 10, L < Qn: the
    # first queries sit before position 0 and select no block
    c = synth.sparse_case(545, 4, 16, 4, 64, 5, 10, 3, [3, 0, 250, 41], query_len=4, causal=0, window=0)
    _check(c, what="sparse bs5 SB10 D64 non-causal, L < Qn")


@pytest.mark.parametrize("seed", range(8))
def test_mq_block_sparse_random_sweep(seed):
    rng = np.random.default_rng(98_000 + seed)
    G = int(rng.choice([1, 2, 4, 8]))
    qn = int(rng.choice([q for q in (2, 3, 4, 8, 16) if q * G <= 16]))
    Hkv = int(rng.choice([1, 2, 4, 8]))
    D = int(rng.choice([64, 128]))
    bs = int(rng.choice([5, 16, 32]))
    sb = bs * int(rng.choice([1, 2, 4]))
    B = int(rng.integers(1, 4))
    lens = rng.integers(0, 1200, size=B)
    qp = None
    if rng.random() < 0.4:
        qp = np.array([int(rng.integers(0, max(1, L))) for L in lens], np.int32)
    c = synth.sparse_case(seed, B, Hkv * G, Hkv, D, bs, sb, int(rng.choice([1, 3, 4])), lens, q_pos=qp, query_len=qn,
                          causal=int(rng.random() < 0.85), window=int(rng.choice([0, 0, 17, 300])),
                          softcap=float(rng.choice([0.0, 5.0, 50.0])),
                          csr_kind=str(rng.choice(["local_strided", "random"])))
    st = int(np.random.default_rng(seed).choice([0, 0, 64, 256]))
    _check(c, st, what=f"sparse seed{seed} B{B} Qn{qn} G{G} Hkv{Hkv} D{D} bs{bs} SB{sb}")


@pytest.mark.parametrize("G,qn,split_tokens", [(4, 8, 0), (4, 16, 128), (8, 16, 0), (1, 100, 0), (2, 40, 64)])
def test_mq_block_sparse_row_blocks(G, qn, split_tokens):
    # more than 16 rows per kv head: each row-block wave builds the union of its own columns
    c = synth.sparse_case(550 + qn, 2, 4 * G, 4, 128, 16, 64, 4, [2000, qn + 50], query_len=qn, softcap=30.0,
                          csr_kind="random" if G % 2 else "local_strided")
    _check(c, split_tokens, what=f"sparse rows {G * qn} G{G} Qn{qn}")
