"""Seeded synthetic inputs for decode attention over paged / tiered / sparse KV caches.

This module only draws and lays out input data: random queries and caches,
block-table permutations of a shared physical pool, the symmetric int8
quantisation that produces the cold tier's stored bytes, ring placement of the
hot tier and CSR block masks.  It computes nothing of the attention itself and
is the one module that both the oracle side and the HIP side of the tests
read their inputs from.

Draw order for every case (one ``numpy.random.default_rng(seed)`` stream):
lengths -> Q -> K -> V -> block permutation -> CSR duplicates.

Cache layouts (all C-contiguous numpy arrays):
  paged pool      k_cache, v_cache  [num_blocks, block_size, Hkv, D]  f32 or f16
  block table     block_table       [B, max_blocks_per_seq]          i32 (unused entries 0)
  hot ring        k_hot, v_hot      [B, hot_window, Hkv, D]          f16
  cold pool       k_cold, v_cold    [num_cold_blocks, bs, Hkv, D/4]  u32, 4 x int8 LSB-first
  cold scales     k_scale, v_scale  [num_cold_blocks, bs, Hkv]       f16
  f16 cold pool   k_cold, v_cold    [num_cold_blocks, bs, Hkv, D]    f16 (the tiered f16 kind)
  window ring     k_hot, v_hot      [B, W, Hkv, D]                   f16 (the ring kind, W = sliding_window)
  CSR             row_ptr [NL, R+1], col_idx [NL, col_stride]        i32
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field
from typing import Optional

import numpy as np

F32, F16 = "f32", "f16"


def _params(B, H, Hkv, D, bs, max_blocks, num_blocks, scale=0.0, causal=1, window=0, softcap=0.0, query_len=1):
    return dict(num_seqs=int(B), num_heads=int(H), num_kv_heads=int(Hkv), head_dim=int(D), scale=float(scale),
                causal=int(causal), sliding_window=int(window), softcap=float(softcap), block_size=int(bs),
                max_blocks_per_seq=int(max_blocks), num_blocks=int(num_blocks), query_len=int(query_len))


@dataclass
class Case:
    """Every array a decode call needs, plus the scalar parameters."""
    kind: str                      # "paged", "tiered", "tiered_f16", "ring" or "sparse"
    params: dict
    q: np.ndarray
    seq_lens: np.ndarray
    q_pos: Optional[np.ndarray] = None
    # paged / sparse
    k_cache: Optional[np.ndarray] = None
    v_cache: Optional[np.ndarray] = None
    block_table: Optional[np.ndarray] = None
    # tiered
    k_hot: Optional[np.ndarray] = None
    v_hot: Optional[np.ndarray] = None
    hot_window: int = 0
    k_cold: Optional[np.ndarray] = None
    v_cold: Optional[np.ndarray] = None
    k_scale: Optional[np.ndarray] = None
    v_scale: Optional[np.ndarray] = None
    cold_block_table: Optional[np.ndarray] = None
    cold_lens: Optional[np.ndarray] = None
    # sparse
    sparse_block: int = 0
    num_layouts: int = 0
    row_ptr: Optional[np.ndarray] = None
    col_idx: Optional[np.ndarray] = None
    name: str = ""
    extra: dict = field(default_factory=dict)


_PARALLEL_MIN = 1 << 26   # elements; larger draws are split over child generators


def _normal(rng, shape, dtype):
    """N(0,1) draws in float32, cast (round-to-nearest-even) to the storage dtype.
    Draws of more than 2^26 elements are split (in C order) into 32 equal
    chunks, each drawn from a child generator seeded by 32 integers taken from
    `rng` (deterministic per seed, computed on 8 threads)."""
    n = int(np.prod(shape))
    if n < _PARALLEL_MIN:
        x = rng.standard_normal(shape, dtype=np.float32)
        return x if dtype == F32 else x.astype(np.float16)
    from concurrent.futures import ThreadPoolExecutor
    seeds = rng.integers(0, 2 ** 63 - 1, size=32)
    out = np.empty(shape, np.float32 if dtype == F32 else np.float16)
    flat = out.reshape(-1)
    bounds = np.linspace(0, n, 33).astype(np.int64)

    def fill(i):
        g = np.random.default_rng(int(seeds[i]))
        flat[bounds[i]:bounds[i + 1]] = g.standard_normal(int(bounds[i + 1] - bounds[i]), dtype=np.float32)

    with ThreadPoolExecutor(8) as ex:
        list(ex.map(fill, range(32)))
    return out


def pool_table(rng, lens, bs, permute=True, extra_blocks=0):
    """A shared physical pool of sum(ceil(L/bs)) (+extra) blocks; sequence b takes the
    next ceil(L_b/bs) entries of a permutation of the pool, in order."""
    lens = np.asarray(lens, np.int64)
    nblk = (lens + bs - 1) // bs
    pool = int(nblk.sum()) + int(extra_blocks)
    perm = rng.permutation(pool) if permute else np.arange(pool)
    max_blocks = max(1, int(nblk.max()) if len(lens) else 1)
    table = np.zeros((len(lens), max_blocks), np.int32)
    pos = 0
    for b, n in enumerate(nblk):
        table[b, :n] = perm[pos:pos + n]
        pos += n
    return table, max(pool, 1)


def paged_case(seed, B, H, Hkv, D, bs, lens=None, kv_dtype=F16, permute=True, q_pos=None, causal=1, window=0,
               softcap=0.0, scale=0.0, extra_blocks=0, len_range=None, name="", query_len=1) -> Case:
    """query_len > 1: q is [B, query_len, H, D], query i of sequence b at position
    q_pos[b] + i (q_pos[b] defaults to seq_lens[b] - query_len)."""
    rng = np.random.default_rng(seed)
    if lens is None:
        lo, hi = len_range
        lens = rng.integers(lo, hi + 1, size=B)
    lens = np.asarray(lens, np.int32)
    q = rng.standard_normal((B, H, D) if query_len == 1 else (B, query_len, H, D), dtype=np.float32)
    nblk = (lens.astype(np.int64) + bs - 1) // bs
    pool = max(int(nblk.sum()) + extra_blocks, 1)
    k = _normal(rng, (pool, bs, Hkv, D), kv_dtype)
    v = _normal(rng, (pool, bs, Hkv, D), kv_dtype)
    table, _ = pool_table(rng, lens, bs, permute, extra_blocks)
    qp = None if q_pos is None else np.asarray(q_pos, np.int32)
    return Case("paged", _params(B, H, Hkv, D, bs, table.shape[1], pool, scale, causal, window, softcap, query_len),
                q, lens, qp, k_cache=k, v_cache=v, block_table=table, name=name)


# ------------------------------------------------------------------ int8 tier

def quantize_rows(x: np.ndarray):
    """Symmetric per-row int8 codes of float32 rows x[..., D]:
    s32 = max|x| / 127 (f32), s = f16(s32), i = clip(rint(x / f32(s)), -127, 127);
    an all-zero row gives s = 0 and i = 0.  Returns (int8 codes, f16 scales).
    Large inputs are processed in row chunks on 8 threads (same result)."""
    x = np.asarray(x, np.float32)
    if x.size >= _PARALLEL_MIN and x.shape[0] >= 16:
        from concurrent.futures import ThreadPoolExecutor
        codes = np.empty(x.shape, np.int8)
        scales = np.empty(x.shape[:-1], np.float16)
        bounds = np.linspace(0, x.shape[0], 17).astype(int)

        def part(i):
            c, sc = _quantize(x[bounds[i]:bounds[i + 1]])
            codes[bounds[i]:bounds[i + 1]] = c
            scales[bounds[i]:bounds[i + 1]] = sc

        with ThreadPoolExecutor(8) as ex:
            list(ex.map(part, range(16)))
        return codes, scales
    return _quantize(x)


def _quantize(x):
    amax = np.max(np.abs(x), axis=-1)
    s16 = (amax / np.float32(127.0)).astype(np.float16)
    s32 = s16.astype(np.float32)
    safe = np.where(s32 > 0, s32, np.float32(1.0))
    codes = np.rint(x / safe[..., None])
    codes = np.where(s32[..., None] > 0, codes, 0)
    codes = np.clip(codes, -127, 127).astype(np.int8)
    return codes, s16


def pack_int8(codes: np.ndarray) -> np.ndarray:
    """int8 codes [..., D] -> u32 words [..., D/4]; element d is byte d%4 of word d/4,
    least-significant byte first."""
    c = np.asarray(codes, np.int8).view(np.uint8).astype(np.uint32)
    c = c.reshape(c.shape[:-1] + (c.shape[-1] // 4, 4))
    return (c[..., 0] | (c[..., 1] << 8) | (c[..., 2] << 16) | (c[..., 3] << 24)).astype(np.uint32)


def exact_rows(rng, shape):
    """Rows x = n * 2^-5 with integer |n| <= 127 and one entry of each row at +-127 * 2^-5,
    so that the f16 value, the int8 code and the f16 scale 2^-5 reproduce each other exactly."""
    n = rng.integers(-127, 128, size=shape).astype(np.float32)
    idx = rng.integers(0, shape[-1], size=shape[:-1])
    sign = np.where(rng.integers(0, 2, size=shape[:-1]) == 0, -1.0, 1.0).astype(np.float32)
    np.put_along_axis(n, idx[..., None], (127.0 * sign)[..., None], axis=-1)
    return n * np.float32(2.0 ** -5)


def tiered_case(seed, B, H, Hkv, D, bs, lens, cold_lens, hot_window, permute=True, q_pos=None, causal=1, window=0,
                softcap=0.0, scale=0.0, exact=False, extra_blocks=0, name="", query_len=1) -> Case:
    """Logical token rows K/V[b, t] are drawn first (float32 N(0,1), or ``exact_rows``); token
    t < cold_lens[b] is stored as int8 codes + f16 scale in the paged cold pool, token
    t >= cold_lens[b] as f16 in the ring at slot t mod hot_window.  Ring slots and pool rows
    that hold no live token carry large garbage, so reading one shows up in the output."""
    rng = np.random.default_rng(seed)
    lens = np.asarray(lens, np.int32)
    cold_lens = np.asarray(cold_lens, np.int32)
    assert np.all(cold_lens <= lens) and np.all(lens - cold_lens <= hot_window)
    q = rng.standard_normal((B, H, D) if query_len == 1 else (B, query_len, H, D), dtype=np.float32)
    Lmax = max(1, int(lens.max()))
    draw = exact_rows if exact else (lambda r, shp: _normal(r, shp, F32))
    k_log = draw(rng, (B, Lmax, Hkv, D))
    v_log = draw(rng, (B, Lmax, Hkv, D))
    table, pool = pool_table(rng, cold_lens, bs, permute, extra_blocks)
    # cold pool; rows no live token uses hold the code 100 with scale 1 (value 100)
    kc = np.full((pool, bs, Hkv, D), 100, np.int8)
    vc = np.full((pool, bs, Hkv, D), -100, np.int8)
    ks = np.ones((pool, bs, Hkv), np.float16)
    vs = np.ones((pool, bs, Hkv), np.float16)
    bb = np.concatenate([np.full(int(c), b) for b, c in enumerate(cold_lens)] + [np.zeros(0, int)]).astype(np.int64)
    tt = np.concatenate([np.arange(int(c)) for c in cold_lens] + [np.zeros(0, int)]).astype(np.int64)
    if bb.size:
        blk, off = table[bb, tt // bs], tt % bs
        kc[blk, off], ks[blk, off] = quantize_rows(k_log[bb, tt])
        vc[blk, off], vs[blk, off] = quantize_rows(v_log[bb, tt])
    hk = np.full((B, hot_window, Hkv, D), 300.0, np.float16)
    hv = np.full((B, hot_window, Hkv, D), -300.0, np.float16)
    hb = np.concatenate([np.full(int(L) - int(c), b) for b, (L, c) in enumerate(zip(lens, cold_lens))]
                        + [np.zeros(0, int)]).astype(np.int64)
    ht = np.concatenate([np.arange(int(c), int(L)) for L, c in zip(lens, cold_lens)] + [np.zeros(0, int)]).astype(np.int64)
    if hb.size:
        hk[hb, ht % hot_window] = k_log[hb, ht].astype(np.float16)
        hv[hb, ht % hot_window] = v_log[hb, ht].astype(np.float16)
    del k_log, v_log
    qp = None if q_pos is None else np.asarray(q_pos, np.int32)
    return Case("tiered", _params(B, H, Hkv, D, bs, table.shape[1], pool, scale, causal, window, softcap, query_len),
                q, lens, qp, k_hot=hk, v_hot=hv, hot_window=int(hot_window), k_cold=pack_int8(kc), v_cold=pack_int8(vc),
                k_scale=ks, v_scale=vs, cold_block_table=table, cold_lens=cold_lens, name=name,
                extra=dict(k_codes=kc, v_codes=vc))


def tiered_f16_case(seed, B, H, Hkv, D, bs, lens, cold_lens, hot_window, permute=True, q_pos=None, causal=1,
                    window=0, softcap=0.0, scale=0.0, extra_blocks=0, name="", query_len=1) -> Case:
    """As ``tiered_case`` with an f16 cold tier: token t < cold_lens[b] is stored as f16 in the
    paged cold pool [pool, bs, Hkv, D], token t >= cold_lens[b] as f16 in the ring at slot
    t mod hot_window.  Pool rows and ring slots that hold no live token carry +-300."""
    rng = np.random.default_rng(seed)
    lens = np.asarray(lens, np.int32)
    cold_lens = np.asarray(cold_lens, np.int32)
    assert np.all(cold_lens <= lens) and np.all(lens - cold_lens <= hot_window)
    q = rng.standard_normal((B, H, D) if query_len == 1 else (B, query_len, H, D), dtype=np.float32)
    Lmax = max(1, int(lens.max()))
    k_log = _normal(rng, (B, Lmax, Hkv, D), F16)
    v_log = _normal(rng, (B, Lmax, Hkv, D), F16)
    table, pool = pool_table(rng, cold_lens, bs, permute, extra_blocks)
    kc = np.full((pool, bs, Hkv, D), 300.0, np.float16)
    vc = np.full((pool, bs, Hkv, D), -300.0, np.float16)
    bb = np.concatenate([np.full(int(c), b) for b, c in enumerate(cold_lens)] + [np.zeros(0, int)]).astype(np.int64)
    tt = np.concatenate([np.arange(int(c)) for c in cold_lens] + [np.zeros(0, int)]).astype(np.int64)
    if bb.size:
        blk, off = table[bb, tt // bs], tt % bs
        kc[blk, off] = k_log[bb, tt]
        vc[blk, off] = v_log[bb, tt]
    hk = np.full((B, hot_window, Hkv, D), 300.0, np.float16)
    hv = np.full((B, hot_window, Hkv, D), -300.0, np.float16)
    hb = np.concatenate([np.full(int(L) - int(c), b) for b, (L, c) in enumerate(zip(lens, cold_lens))]
                        + [np.zeros(0, int)]).astype(np.int64)
    ht = np.concatenate([np.arange(int(c), int(L)) for L, c in zip(lens, cold_lens)] + [np.zeros(0, int)]).astype(np.int64)
    if hb.size:
        hk[hb, ht % hot_window] = k_log[hb, ht]
        hv[hb, ht % hot_window] = v_log[hb, ht]
    del k_log, v_log
    qp = None if q_pos is None else np.asarray(q_pos, np.int32)
    return Case("tiered_f16", _params(B, H, Hkv, D, bs, table.shape[1], pool, scale, causal, window, softcap,
                                      query_len), q, lens, qp, k_hot=hk, v_hot=hv, hot_window=int(hot_window), k_cold=kc, v_cold=vc,
                cold_block_table=table, cold_lens=cold_lens, name=name)


def ring_case(seed, B, H, Hkv, D, W, lens, q_pos=None, causal=1, softcap=0.0, scale=0.0, history=True,
              name="", query_len=1) -> Case:
    """Sliding-window ring of W slots per sequence: token t of sequence b sits at slot
    t mod W and only the last W tokens are resident.  With ``history`` the whole token
    history K/V[b, t] is drawn (float32 N(0,1) -> f16, kept in ``extra``) and its last W
    tokens are written to the ring; otherwise the resident rows are drawn directly.
    Slots that hold no resident token carry +-300."""
    rng = np.random.default_rng(seed)
    lens = np.asarray(lens, np.int32)
    q = rng.standard_normal((B, H, D) if query_len == 1 else (B, query_len, H, D), dtype=np.float32)
    hk = np.full((B, W, Hkv, D), 300.0, np.float16)
    hv = np.full((B, W, Hkv, D), -300.0, np.float16)
    extra = {}
    if history:
        Lmax = max(1, int(lens.max()))
        k_log = _normal(rng, (B, Lmax, Hkv, D), F16)
        v_log = _normal(rng, (B, Lmax, Hkv, D), F16)
        for b, L in enumerate(lens):
            t = np.arange(max(0, int(L) - W), int(L))
            hk[b, t % W] = k_log[b, t]
            hv[b, t % W] = v_log[b, t]
        extra = dict(k_history=k_log, v_history=v_log)
    else:
        full = lens >= W
        hk[full] = _normal(rng, (int(full.sum()), W, Hkv, D), F16)
        hv[full] = _normal(rng, (int(full.sum()), W, Hkv, D), F16)
        for b in np.nonzero(~full)[0]:
            L = int(lens[b])
            hk[b, :L] = rng.standard_normal((L, Hkv, D), dtype=np.float32).astype(np.float16)
            hv[b, :L] = rng.standard_normal((L, Hkv, D), dtype=np.float32).astype(np.float16)
    qp = None if q_pos is None else np.asarray(q_pos, np.int32)
    return Case("ring", _params(B, H, Hkv, D, 1, 1, 1, scale, causal, W, softcap, query_len), q, lens, qp, k_hot=hk,
                v_hot=hv, hot_window=int(W), name=name, extra=extra)


# ------------------------------------------------------------------- sparse

def csr_from_rows(rows_per_layout):
    """rows_per_layout[l][r] = list of column indices -> (row_ptr [NL, R+1], col_idx [NL, max_nnz])."""
    NL = len(rows_per_layout)
    R = len(rows_per_layout[0])
    nnz = [sum(len(r) for r in rows) for rows in rows_per_layout]
    col_stride = max(1, max(nnz))
    row_ptr = np.zeros((NL, R + 1), np.int32)
    col_idx = np.zeros((NL, col_stride), np.int32)
    for l, rows in enumerate(rows_per_layout):
        pos = 0
        for r, cols in enumerate(rows):
            row_ptr[l, r] = pos
            col_idx[l, pos:pos + len(cols)] = cols
            pos += len(cols)
        row_ptr[l, R] = pos
    return row_ptr, col_idx


def local_strided_rows(rng, R, NL, local=4, stride=8, dup_frac=0.1):
    """Row r of layout l: {r-local+1 .. r} U {j <= r : j = l (mod stride)}, sorted, then
    about dup_frac of its entries repeated at random positions.  A row whose entry count
    equals r+1 without covering 0..r gets one more repeat, so that count-based dense
    shortcuts and boolean set semantics agree on this data."""
    layouts = []
    for l in range(NL):
        rows = []
        for r in range(R):
            base = sorted(set(range(max(0, r - local + 1), r + 1)) | set(range(l % stride, r + 1, stride)))
            row = list(base)
            ndup = int(round(dup_frac * len(base)))
            for _ in range(ndup):
                row.insert(int(rng.integers(0, len(row) + 1)), int(base[rng.integers(0, len(base))]))
            if len(row) == r + 1 and set(row) != set(range(r + 1)):
                row.insert(int(rng.integers(0, len(row) + 1)), int(base[0]))
            rows.append(row)
        layouts.append(rows)
    return layouts


def random_rows(rng, R, NL, density=0.4, dup_frac=0.3, beyond=True):
    """Random CSR rows: any subset of 0..R-1 (also columns beyond the row, which the
    causal clip must drop), shuffled, with repeats."""
    layouts = []
    for _ in range(NL):
        rows = []
        for r in range(R):
            top = R if beyond else r + 1
            cols = [j for j in range(top) if rng.random() < density]
            cols += [cols[int(rng.integers(0, len(cols)))] for _ in range(int(dup_frac * len(cols)))] if cols else []
            rng.shuffle(cols)
            rows.append([int(c) for c in cols])
        layouts.append(rows)
    return layouts


def sparse_case(seed, B, H, Hkv, D, bs, sparse_block, num_layouts, lens, rows=None, permute=True, q_pos=None,
                causal=1, window=0, softcap=0.0, scale=0.0, name="", csr_kind="local_strided", query_len=1) -> Case:
    """query_len > 1: q is [B, query_len, H, D], query i of sequence b at position
    q_pos[b] + i (q_pos[b] defaults to seq_lens[b] - query_len), each with the CSR
    row of its own position."""
    rng = np.random.default_rng(seed)
    lens = np.asarray(lens, np.int32)
    q = rng.standard_normal((B, H, D) if query_len == 1 else (B, query_len, H, D), dtype=np.float32)
    nblk = (lens.astype(np.int64) + bs - 1) // bs
    pool = max(int(nblk.sum()), 1)
    k = _normal(rng, (pool, bs, Hkv, D), F16)
    v = _normal(rng, (pool, bs, Hkv, D), F16)
    table, _ = pool_table(rng, lens, bs, permute)
    R = max(1, int(math.ceil(int(lens.max()) / sparse_block)))
    if rows is None:
        rows = (local_strided_rows(rng, R, num_layouts) if csr_kind == "local_strided"
                else random_rows(rng, R, num_layouts))
    row_ptr, col_idx = csr_from_rows(rows)
    qp = None if q_pos is None else np.asarray(q_pos, np.int32)
    return Case("sparse", _params(B, H, Hkv, D, bs, table.shape[1], pool, scale, causal, window, softcap, query_len),
                q, lens,
                qp, k_cache=k, v_cache=v, block_table=table, sparse_block=int(sparse_block),
                num_layouts=int(num_layouts), row_ptr=row_ptr, col_idx=col_idx, name=name, extra=dict(rows=rows))


# ------------------------------------------------------------ the workloads

def workload(i: int, window: int = 0) -> Case:
    """The five decode workloads, seeded with their index.

    1  tiny: B=1, H=4/Hkv=2, D=64, L=256, f32 KV, bs=16, identity table, causal at 255
    2  paged f16: B=32, 32/8 heads, D=128, bs=16, L ~ U{512..4096}, permuted pool
    3  tiered: B=16, 32/8, D=128, L=8192 = 7680 int8 cold (bs=16, permuted) + 512 f16 hot
       (ring of 512), softcap 50, window 0 or 4096
    4  long paged f16: B=4, 64/8 heads, D=128, L=131072, bs=64, permuted pool
    5  block-sparse: B=8, 32/8, D=128, L=16384, SB=bs=64, 4 layouts (head % 4), last 4
       local blocks + every 8th block offset by layout, ~10% repeated columns
    """
    if i == 1:
        return paged_case(1, 1, 4, 2, 64, 16, lens=[256], kv_dtype=F32, permute=False,
                          scale=float(np.float32(1.0 / math.sqrt(64))), name="tiny_f32_B1_H4_L256")
    if i == 2:
        return paged_case(2, 32, 32, 8, 128, 16, len_range=(512, 4096), kv_dtype=F16,
                          scale=float(np.float32(1.0 / math.sqrt(128))), name="paged_f16_B32_H32x8_D128_L512-4096")
    if i == 3:
        B = 16
        return tiered_case(3, B, 32, 8, 128, 16, lens=[8192] * B, cold_lens=[7680] * B, hot_window=512,
                           softcap=50.0, window=window, scale=float(np.float32(1.0 / math.sqrt(128))),
                           name=f"tiered_int8_B16_H32x8_D128_L8192_W{window}_cap50")
    if i == 4:
        return paged_case(4, 4, 64, 8, 128, 64, lens=[131072] * 4, kv_dtype=F16,
                          scale=float(np.float32(1.0 / math.sqrt(128))), name="paged_f16_B4_H64x8_D128_L131072")
    if i == 5:
        return sparse_case(5, 8, 32, 8, 128, 64, 64, 4, lens=[16384] * 8,
                           scale=float(np.float32(1.0 / math.sqrt(128))), name="sparse_f16_B8_H32x8_D128_L16384")
    raise ValueError(i)


def ring_workload() -> Case:
    """Sliding-window ring f16: B=32, 32/8 heads, D=128, window (= ring) 4096,
    L ~ U{4096..32768} (every ring full), causal, scale 1/sqrt(128)."""
    rng = np.random.default_rng(7)
    lens = rng.integers(4096, 32769, size=32)
    return ring_case(7, 32, 32, 8, 128, 4096, lens, history=False, scale=float(np.float32(1.0 / math.sqrt(128))),
                     name="ring_f16_B32_H32x8_D128_W4096")


def multi_query_workload(query_len: int = 4) -> Case:
    """Multi-query (speculative) decode over workload 2's paged f16 cache shape:
    B=32, 32/8 heads, D=128, bs=16, L ~ U{512..4096}, permuted pool, causal; the
    last query_len tokens of each sequence are the queries."""
    return paged_case(8, 32, 32, 8, 128, 16, len_range=(512, 4096), kv_dtype=F16, query_len=query_len,
                      scale=float(np.float32(1.0 / math.sqrt(128))),
                      name=f"paged_f16_mq{query_len}_B32_H32x8_D128_L512-4096")


def sparse_multi_query_workload(query_len: int = 4) -> Case:
    """Multi-query decode over workload 5's block-sparse cache: B=8, 32/8 heads,
    D=128, L=16384, SB=bs=64, 4 layouts; the last query_len tokens are the queries,
    each with its own CSR row."""
    return sparse_case(5, 8, 32, 8, 128, 64, 64, 4, lens=[16384] * 8, query_len=query_len,
                       scale=float(np.float32(1.0 / math.sqrt(128))),
                       name=f"sparse_f16_mq{query_len}_B8_H32x8_D128_L16384")


def tiered_multi_query_workload(query_len: int = 4) -> Case:
    """Multi-query decode over the tiered int8 workload's shape: B=16, 32/8 heads,
    D=128, L=8192 = 7680 int8 cold + 512 f16 hot (ring of 512), softcap 50; the
    last query_len tokens of each sequence are the queries."""
    B = 16
    return tiered_case(11, B, 32, 8, 128, 16, lens=[8192] * B, cold_lens=[7680] * B, hot_window=512,
                       softcap=50.0, scale=float(np.float32(1.0 / math.sqrt(128))), query_len=query_len,
                       name=f"tiered_int8_mq{query_len}_B16_H32x8_D128_L8192_cap50")


def tiered_f16_workload(window: int = 0) -> Case:
    """The tiered workload's shape with an f16 cold tier: B=16, 32/8 heads, D=128,
    L=8192 = 7680 f16 cold (bs=16, permuted pool) + 512 f16 hot (ring of 512), softcap 50."""
    B = 16
    return tiered_f16_case(6, B, 32, 8, 128, 16, lens=[8192] * B, cold_lens=[7680] * B, hot_window=512,
                           softcap=50.0, window=window, scale=float(np.float32(1.0 / math.sqrt(128))),
                           name=f"tiered_f16_B16_H32x8_D128_L8192_W{window}_cap50")
