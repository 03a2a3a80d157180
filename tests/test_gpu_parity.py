"""GPU parity: the HIP path through the C ABI against the fp64 oracle, element
by element, on seeded inputs that span several 16-key tiles, several KV splits
and ragged tails; plus exact invariants of the GPU path itself (block
permutation, visited-key counts) and split-count independence."""
import math

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
    dc = DeviceCase(case)
    og, lg = dc.run_np(split_tokens)
    orf, lrf = oracle_run(case)
    return compare(og, lg, orf, lrf, what=what)


# ------------------------------------------------------------ the workloads

def test_tiny_f32():
    _check(synth.workload(1), what="tiny f32 B1 H4/2 D64 L256")


def test_paged_f16_small():
    c = synth.paged_case(102, 4, 32, 8, 128, 16, len_range=(512, 1200), kv_dtype=synth.F16,
                         scale=float(np.float32(1 / math.sqrt(128))))
    _check(c, what="paged f16 B4 L512-1200")


@pytest.mark.parametrize("window", [0, 300])
def test_tiered_int8_small(window):
    c = synth.tiered_case(103, 2, 32, 8, 128, 16, [700, 613], [450, 420], 256, softcap=50.0, window=window)
    _check(c, what=f"tiered int8 B2 L700 W{window} cap50 ring-wrap")


def test_long_paged_small():
    c = synth.paged_case(104, 1, 64, 8, 128, 64, lens=[5000], kv_dtype=synth.F16)
    _check(c, what="paged f16 G8 L5000 bs64")


def test_sparse_small():
    c = synth.sparse_case(105, 2, 32, 8, 128, 64, 64, 4, [2048, 1999])
    _check(c, what="sparse local+strided L2048 SB64")


def test_sparse_random_csr_small_blocks():
    c = synth.sparse_case(106, 2, 16, 4, 64, 4, 8, 3, [300, 211], csr_kind="random", window=150, softcap=20.0)
    _check(c, what="sparse random CSR SB8 bs4")


# ------------------------------------------------------------ random sweep

def _rand_case(seed):
    rng = np.random.default_rng(50_000 + seed)
    kind = ["paged", "paged", "tiered", "sparse"][seed % 4]
    D = int(rng.choice([64, 128]))
    G = int(rng.choice([1, 2, 4, 8]))
    Hkv = int(rng.choice([1, 2, 3, 4, 8]))
    B = int(rng.integers(1, 4))
    causal = int(rng.random() < 0.8)
    window = int(rng.choice([0, 0, 1, 17, 200]))
    softcap = float(rng.choice([0.0, 0.0, 5.0, 50.0]))
    scale = float(rng.choice([0.0, np.float32(rng.uniform(0.03, 0.3))]))
    lens = rng.integers(0, 700, size=B)
    if rng.random() < 0.3:
        lens[0] = int(rng.choice([0, 1, 15, 16, 17]))
    qp = None
    if rng.random() < 0.4:
        qp = np.array([int(rng.integers(0, max(1, L))) for L in lens], np.int32)
    kw = dict(causal=causal, window=window, softcap=softcap, scale=scale, q_pos=qp)
    if kind == "paged":
        bs = int(rng.choice([1, 3, 16, 64]))
        dt = synth.F32 if rng.random() < 0.3 else synth.F16
        return synth.paged_case(seed, B, Hkv * G, Hkv, D, bs, lens=lens, kv_dtype=dt,
                                permute=bool(rng.integers(0, 2)), extra_blocks=int(rng.integers(0, 3)), **kw)
    if kind == "tiered":
        bs = int(rng.choice([1, 5, 16]))
        hw = int(rng.choice([1, 16, 50, 128]))
        cold = np.array([max(0, int(L) - int(rng.integers(0, hw + 1))) for L in lens])
        return synth.tiered_case(seed, B, Hkv * G, Hkv, D, bs, lens, cold, hw, **kw)
    bs = int(rng.choice([1, 2, 16]))
    sb = bs * int(rng.choice([1, 2, 4]))
    lens = np.maximum(lens, 1)
    if qp is not None:
        qp = np.minimum(qp, lens - 1).astype(np.int32)
        kw["q_pos"] = qp
    return synth.sparse_case(seed, B, Hkv * G, Hkv, D, bs, sb, int(rng.integers(1, 5)), lens,
                             csr_kind="random" if rng.random() < 0.5 else "local_strided", **kw)


@pytest.mark.parametrize("seed", range(48))
def test_random_sweep(seed):
    case = _rand_case(seed)
    st = int(np.random.default_rng(seed).choice([0, 0, 16, 48, 256]))
    p = case.params
    _check(case, split_tokens=st,
           what=f"seed{seed} {case.kind} B{p['num_seqs']} H{p['num_heads']}/{p['num_kv_heads']} D{p['head_dim']} "
                f"bs{p['block_size']} W{p['sliding_window']} cap{p['softcap']}")


# ---------------------------------------------------------------- edges

def test_empty_and_single_key_sequences():
    c = synth.paged_case(201, 4, 8, 2, 128, 16, lens=[0, 1, 0, 33], kv_dtype=synth.F16)
    _check(c, what="lens 0/1/0/33")


def test_all_sequences_empty():
    c = synth.paged_case(202, 2, 8, 2, 64, 16, lens=[0, 0], kv_dtype=synth.F16)
    dc = DeviceCase(c)
    out, lse = dc.run_np(max_seq_len=0)
    assert np.all(out == 0) and np.all(lse == -np.inf)


def test_query_before_end_masks_the_future():
    c = synth.paged_case(203, 2, 8, 2, 128, 16, lens=[500, 400], q_pos=[100, 399], window=64)
    _check(c, what="q_pos < L-1 with window")


def test_non_causal_window_keeps_future_keys():
    c = synth.paged_case(204, 2, 8, 2, 128, 16, lens=[500, 400], q_pos=[100, 50], causal=0, window=64)
    _check(c, what="non-causal window")


def test_int8_minus_128_codes():
    c = synth.tiered_case(205, 1, 8, 2, 128, 16, [300], [280], 32)
    rng = np.random.default_rng(0)
    for arr in (c.k_cold, c.v_cold):
        flat = arr.reshape(-1)
        idx = rng.integers(0, flat.size, size=flat.size // 8)
        flat[idx] = rng.integers(0, 2 ** 32, size=idx.size, dtype=np.uint64).astype(np.uint32)
    _check(c, what="raw int8 words incl. -128")


# ------------------------------------------------------------ invariants

def test_block_permutation_is_bit_exact_on_gpu():
    c = synth.paged_case(301, 3, 32, 8, 128, 16, lens=[700, 1300, 260], softcap=30.0)
    o1, l1 = DeviceCase(c).run_np(split_tokens=256)
    pi = np.random.default_rng(9).permutation(c.k_cache.shape[0])
    k = np.empty_like(c.k_cache)
    v = np.empty_like(c.v_cache)
    k[pi], v[pi] = c.k_cache, c.v_cache
    c.k_cache, c.v_cache, c.block_table = k, v, pi[c.block_table].astype(np.int32)
    o2, l2 = DeviceCase(c).run_np(split_tokens=256)
    assert np.array_equal(o1, o2) and np.array_equal(l1, l2)


@pytest.mark.parametrize("kind", ["paged", "tiered", "sparse"])
def test_split_count_independence(kind):
    if kind == "paged":
        c = synth.paged_case(302, 2, 32, 8, 128, 16, lens=[1500, 777])
    elif kind == "tiered":
        c = synth.tiered_case(302, 2, 32, 8, 128, 16, [1500, 777], [1200, 700], 512, softcap=50.0)
    else:
        c = synth.sparse_case(302, 2, 32, 8, 128, 16, 64, 4, [1500, 777])
    dc = DeviceCase(c)
    ref_o, ref_l = oracle_run(c)
    outs = []
    for st in (16, 64, 272, 4096):
        o, l = dc.run_np(split_tokens=st)
        compare(o, l, ref_o, ref_l, what=f"{kind} split_tokens={st}")
        outs.append(o)
    for o in outs[1:]:
        assert np.max(np.abs(o - outs[0])) <= 1e-4


def _visited_case(kind):
    lens = [1203, 650]
    if kind == "paged":
        c = synth.paged_case(401, 2, 16, 4, 128, 3, lens=lens, window=700, q_pos=[1100, 649])
    elif kind == "tiered":
        c = synth.tiered_case(401, 2, 16, 4, 128, 3, lens, [1000, 600], 256, window=700, q_pos=[1100, 649])
    else:
        c = synth.sparse_case(401, 2, 16, 4, 128, 3, 6, 3, lens, q_pos=[1100, 649], window=700, csr_kind="random")
    return c, lens


@pytest.mark.parametrize("kind", ["paged", "tiered", "sparse"])
def test_visited_key_counts_exact(kind):
    """q = 0 makes every visible key weigh the same: exp(lse) is the number of
    visible keys, exactly after rounding; with V one-hot on (block index mod D)
    the output times that number counts the visible keys of every block class."""
    from bruteforce import visible_matrix
    c, lens = _visited_case(kind)
    c.q[:] = 0
    D, bs = 128, 3
    if kind == "tiered":
        c.v_cold[:] = 0
        c.v_scale[:] = np.float16(1.0)
        c.v_hot[:] = 0
        for b, L in enumerate(lens):
            cl = int(c.cold_lens[b])
            for t in range(L):
                j = (t // bs) % D
                if t < cl:
                    blk, off = c.cold_block_table[b, t // bs], t % bs
                    c.v_cold[blk, off, :, j // 4] |= np.uint32(1 << (8 * (j % 4)))
                else:
                    c.v_hot[b, t % c.hot_window, :, :] = 0
                    c.v_hot[b, t % c.hot_window, :, j] = 1
    else:
        c.v_cache[:] = 0
        for b, L in enumerate(lens):
            t = np.arange(L)
            c.v_cache[c.block_table[b, t // bs], t % bs, :, (t // bs) % D] = 1
    out, lse = DeviceCase(c).run_np(split_tokens=64)
    for b, L in enumerate(lens):
        vis = visible_matrix(c, b)
        t = np.arange(L)
        for h in range(c.params["num_heads"]):
            n = int(vis[h].sum())
            assert round(math.exp(lse[b, h])) == n
            want = np.bincount(((t // bs) % D)[vis[h]], minlength=D)
            assert np.array_equal(np.rint(out[b, h] * n).astype(int), want), (b, h)


def test_hot_cold_split_point_on_gpu():
    ref = None
    for cold in ([700, 300], [500, 0], [650, 299], [300, 100]):
        c = synth.tiered_case(501, 2, 16, 4, 128, 16, [700, 300], cold, 512, exact=True, softcap=20.0)
        o, l = DeviceCase(c).run_np(split_tokens=128)
        if ref is None:
            ref = oracle_run(c)
        compare(o, l, *ref, what=f"exact tiered cold={cold}")


# ------------------------------------------- rows that hold no live token

def _poison_paged(k, v, table, lens, bs):
    """NaN / Inf in every pool row that holds no token of any sequence."""
    live = np.zeros(k.shape[:2], bool)
    for b, L in enumerate(lens):
        t = np.arange(int(L))
        live[table[b, t // bs], t % bs] = True
    k[~live] = np.float16(np.nan)
    v[~live] = np.float16(np.inf)


@pytest.mark.parametrize("bs", [16, 5])
def test_paged_nonlive_rows_hold_nan(bs):
    """Tiles that straddle the end of a sequence read whole rows when the block
    size is a multiple of 16: whatever the rows past the end hold must not reach
    the output (the oracle never reads them)."""
    c = synth.paged_case(120 + bs, 3, 16, 4, 128, bs, lens=[77, 300, 1], kv_dtype=synth.F16, window=0,
                         q_pos=[70, 299, 0])
    _poison_paged(c.k_cache, c.v_cache, c.block_table, c.seq_lens, bs)
    _check(c, what=f"paged f16 bs{bs} NaN/Inf outside the live rows")


def test_tiered_nonlive_rows_hold_nan():
    c = synth.tiered_case(122, 3, 16, 4, 128, 16, [700, 300, 40], [450, 260, 0], 256, softcap=30.0, window=200)
    live = np.zeros(c.k_scale.shape[:2], bool)
    for b, C in enumerate(c.cold_lens):
        t = np.arange(int(C))
        live[c.cold_block_table[b, t // 16], t % 16] = True
    c.k_scale[~live] = np.float16(np.nan)
    c.v_scale[~live] = np.float16(np.inf)
    ring_live = np.zeros(c.k_hot.shape[:2], bool)
    for b, (L, C) in enumerate(zip(c.seq_lens, c.cold_lens)):
        ring_live[b, np.arange(int(C), int(L)) % c.hot_window] = True
    c.k_hot[~ring_live] = np.float16(np.nan)
    c.v_hot[~ring_live] = np.float16(np.inf)
    _check(c, what="tiered NaN/Inf outside the live rows and ring slots")


def test_sparse_nonlive_rows_hold_nan():
    c = synth.sparse_case(123, 2, 16, 4, 128, 16, 64, 3, [1000, 333])
    _poison_paged(c.k_cache, c.v_cache, c.block_table, c.seq_lens, 16)
    _check(c, what="sparse NaN/Inf outside the live rows")


@pytest.mark.parametrize("qn", [4, 16])
def test_multi_query_nonlive_rows_hold_nan(qn):
    """The same with several queries per sequence; with 16 queries (64 rows per
    kv head) the tiles go through the shared LDS buffers of the row-block waves."""
    c = synth.paged_case(124 + qn, 3, 16, 4, 128, 16, lens=[77, 300, 1], kv_dtype=synth.F16, query_len=qn,
                         q_pos=[60, 280, 0])
    _poison_paged(c.k_cache, c.v_cache, c.block_table, c.seq_lens, 16)
    _check(c, what=f"paged f16 Qn{qn} NaN/Inf outside the live rows")
    t = synth.tiered_case(126 + qn, 3, 16, 4, 128, 16, [700, 300, 40], [450, 260, 0], 256, query_len=qn)
    live = np.zeros(t.k_scale.shape[:2], bool)
    for b, C in enumerate(t.cold_lens):
        k = np.arange(int(C))
        live[t.cold_block_table[b, k // 16], k % 16] = True
    t.k_scale[~live] = np.float16(np.nan)
    t.v_scale[~live] = np.float16(np.inf)
    ring_live = np.zeros(t.k_hot.shape[:2], bool)
    for b, (L, C) in enumerate(zip(t.seq_lens, t.cold_lens)):
        ring_live[b, np.arange(int(C), int(L)) % t.hot_window] = True
    t.k_hot[~ring_live] = np.float16(np.nan)
    t.v_hot[~ring_live] = np.float16(np.inf)
    _check(t, what=f"tiered Qn{qn} NaN/Inf outside the live rows and ring slots")


# ------------------------------------------------- NaN in a row a query uses

def _check_nan(case, split_tokens, what):
    """NaN in visible rows: the GPU gives NaN exactly where the fp64 oracle does
    (a NaN key poisons every head of its group, a NaN value element one output
    dim, a NaN int8 value scale the whole row of values); the rest matches."""
    log(f"case {case.kind} {what} split_tokens={split_tokens}")
    og, lg = DeviceCase(case).run_np(split_tokens)
    orf, lrf = oracle_run(case)
    assert np.isnan(orf).any(), f"{what}: the planted NaN reaches no oracle output"
    assert np.array_equal(np.isnan(og), np.isnan(orf)), f"{what}: NaN pattern of out differs from the oracle"
    assert np.array_equal(np.isnan(lg), np.isnan(lrf)), f"{what}: NaN pattern of lse differs from the oracle"
    ok = ~np.isnan(orf)
    err = float(np.max(np.abs(og[ok] - orf[ok])))
    assert err <= 1e-3 and err <= 1e-3 * float(np.max(np.abs(orf[ok]))), f"{what}: max abs error {err}"
    okl = ~np.isnan(lrf)
    assert float(np.max(np.abs(lg[okl] - lrf[okl]))) <= 1e-3, f"{what}: lse error"


@pytest.mark.parametrize("split_tokens", [0, 64])
def test_nan_in_live_rows_reaches_the_output(split_tokens):
    """Merging splits must not drop a piece whose running sum is NaN: only a
    piece with no visible key (l = 0 exactly) is skipped."""
    c = synth.paged_case(130, 3, 16, 4, 128, 16, lens=[300, 700, 50], kv_dtype=synth.F16)
    tb = c.block_table
    c.k_cache[tb[1, 123 // 16], 123 % 16, 2, 7] = np.float16(np.nan)    # key of seq 1, kv head 2
    c.v_cache[tb[0, 5 // 16], 5 % 16, 1, 17] = np.float16(np.nan)      # one value dim of seq 0, kv head 1
    _check_nan(c, split_tokens, "paged f16 NaN key and NaN value element")
    t = synth.tiered_case(131, 3, 16, 4, 128, 16, [700, 300, 40], [450, 260, 0], 256, softcap=30.0)
    ctb = t.cold_block_table
    t.k_scale[ctb[0, 200 // 16], 200 % 16, 3] = np.float16(np.nan)      # cold key scale, seq 0, kv head 3
    t.v_scale[ctb[1, 17 // 16], 17 % 16, 0] = np.float16(np.nan)        # cold value scale, seq 1, kv head 0
    t.k_hot[2, 33 % t.hot_window, 1, 64] = np.float16(np.nan)           # hot key, seq 2, kv head 1
    _check_nan(t, split_tokens, "tiered int8 NaN scales and NaN hot key")


@pytest.mark.parametrize("Hkv,offset", [(8, 0), (8, 1), (3, 0), (2, 1), (1, 0)])
def test_int8_scale_gathers(Hkv, offset):
    """Scale gathers of contiguous int8 tiles with odd and even kv-head counts,
    and scale arrays that start on or 2 bytes past a 4-byte boundary (offset 1),
    against the oracle."""
    import torch
    c = synth.tiered_case(150 + 2 * Hkv + offset, 3, 4 * Hkv, Hkv, 128, 16, [900, 700, 250], [700, 600, 0], 256,
                          softcap=30.0)
    dc = DeviceCase(c)
    if offset:
        for name in ("k_scale", "v_scale"):
            t = getattr(dc, name)
            buf = torch.empty(t.numel() + 1, dtype=t.dtype, device=t.device)
            v = buf[1:].view(t.shape)
            v.copy_(t)
            assert v.data_ptr() % 4 == 2
            setattr(dc, name, v)
    log(f"int8 scale gathers Hkv={Hkv} offset={offset}")
    og, lg = dc.run_np()
    ro, rl = oracle_run(c)
    compare(og, lg, ro, rl, what=f"int8 scale gathers Hkv{Hkv} offset{offset}")
