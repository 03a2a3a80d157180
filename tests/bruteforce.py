"""Dense brute-force decode attention in numpy/scipy float64, for tiny inputs only.

Written independently of the C oracle: it gathers every sequence's logical
K/V rows with numpy fancy indexing (the int8 tier through a little-endian byte
view of the packed words), builds the full boolean visibility matrix over
[0, L) with vectorised comparisons, and takes the softmax and log-sum-exp
from scipy.special.  It is the reference the oracle is pinned against.
"""
from __future__ import annotations

import numpy as np
from scipy.special import logsumexp, softmax


def scale_of(p):
    return float(p["scale"]) if p["scale"] != 0.0 else float(np.float32(1.0 / np.sqrt(p["head_dim"])))


def logical_rows(case, b):
    """float64 K, V of sequence b: [L, Hkv, D]."""
    p = case.params
    L = int(case.seq_lens[b])
    bs = p["block_size"]
    t = np.arange(L)
    if case.kind in ("paged", "sparse"):
        blk = case.block_table[b, t // bs]
        K = case.k_cache[blk, t % bs].astype(np.float64)
        V = case.v_cache[blk, t % bs].astype(np.float64)
        return K, V
    Hkv, D = p["num_kv_heads"], p["head_dim"]
    if case.kind == "ring":
        # only the last W tokens are resident; older positions get NaN rows, which the
        # visibility matrix below never selects
        W = case.hot_window
        K = np.full((L, Hkv, D), np.nan)
        V = np.full((L, Hkv, D), np.nan)
        tr = t[max(0, L - W):]
        K[tr] = case.k_hot[b, tr % W]
        V[tr] = case.v_hot[b, tr % W]
        return K, V
    c = int(case.cold_lens[b])
    if case.kind == "tiered_f16":
        tc, th = t[:c], t[c:]
        blk = case.cold_block_table[b, tc // bs]
        K = np.concatenate([case.k_cold[blk, tc % bs], case.k_hot[b, th % case.hot_window]]).astype(np.float64)
        V = np.concatenate([case.v_cold[blk, tc % bs], case.v_hot[b, th % case.hot_window]]).astype(np.float64)
        return K.reshape(L, Hkv, D), V.reshape(L, Hkv, D)
    # tiered int8
    K = np.empty((L, Hkv, D))
    V = np.empty((L, Hkv, D))
    tc = t[:c]
    blk = case.cold_block_table[b, tc // bs]
    kb = np.ascontiguousarray(case.k_cold[blk, tc % bs]).view("<i1").reshape(c, Hkv, D).astype(np.float64)
    vb = np.ascontiguousarray(case.v_cold[blk, tc % bs]).view("<i1").reshape(c, Hkv, D).astype(np.float64)
    K[:c] = kb * case.k_scale[blk, tc % bs].astype(np.float64)[..., None]
    V[:c] = vb * case.v_scale[blk, tc % bs].astype(np.float64)[..., None]
    th = t[c:]
    K[c:] = case.k_hot[b, th % case.hot_window].astype(np.float64)
    V[c:] = case.v_hot[b, th % case.hot_window].astype(np.float64)
    return K, V


def query_len(case):
    return max(1, int(case.params.get("query_len", 1)))


def visible_matrix(case, b, i=0):
    """bool [H, L]: which keys each head of query i of sequence b attends to (query i
    at position q_pos[b] + i, q_pos[b] defaulting to L - query_len)."""
    p = case.params
    H = p["num_heads"]
    L = int(case.seq_lens[b])
    q = (int(case.q_pos[b]) if case.q_pos is not None else L - query_len(case)) + i
    t = np.arange(L)
    ok = np.ones(L, bool)
    if p["causal"]:
        ok &= t <= q
    W = p["sliding_window"]
    if W > 0 and q >= W:
        ok &= t >= q - W + 1
    if case.kind == "ring":
        ok &= t >= L - case.hot_window
    vis = np.repeat(ok[None, :], H, axis=0)
    if case.kind == "sparse" and q < 0:
        vis[:] = False   # a query before position 0 has no CSR row
    elif case.kind == "sparse":
        SB = case.sparse_block
        r = q // SB
        for h in range(H):
            l = h % case.num_layouts
            cols = case.col_idx[l, case.row_ptr[l, r]:case.row_ptr[l, r + 1]]
            chosen = np.zeros(max(1, (L + SB - 1) // SB), bool)
            cols = cols[(cols >= 0) & (cols <= r) & (cols < chosen.size)]
            chosen[cols] = True
            vis[h] &= chosen[t // SB]
    return vis


def attend(case):
    """(out [B, H, D], lse [B, H]) in float64; with query_len Qn > 1,
    (out [B, Qn, H, D], lse [B, Qn, H])."""
    p = case.params
    B, H, Hkv, D = p["num_seqs"], p["num_heads"], p["num_kv_heads"], p["head_dim"]
    Qn = query_len(case)
    G = H // Hkv
    sc = scale_of(p)
    cap = float(p["softcap"])
    qs = case.q.reshape(B, Qn, H, D)
    out = np.zeros((B, Qn, H, D))
    lse = np.full((B, Qn, H), -np.inf)
    for b in range(B):
        K, V = logical_rows(case, b)
        Kh = np.repeat(K, G, axis=1).transpose(1, 0, 2)       # [H, L, D]
        Vh = np.repeat(V, G, axis=1).transpose(1, 0, 2)
        for i in range(Qn):
            vis = visible_matrix(case, b, i)
            qb = qs[b, i].astype(np.float64)                  # [H, D]
            s = sc * np.einsum("hd,hld->hl", qb, Kh)
            if cap > 0:
                s = cap * np.tanh(s / cap)
            for h in range(H):
                if not vis[h].any():
                    continue
                sv = s[h][vis[h]]
                out[b, i, h] = softmax(sv) @ Vh[h][vis[h]]
                lse[b, i, h] = logsumexp(sv)
    if Qn == 1:
        return out[:, 0], lse[:, 0]
    return out, lse


# ----------------------------------------------- the tiered write path

def quantize_f16_rows(x16):
    """The quantiser reading restated with numpy on f16 rows [..., D]: in f32,
    s32 = max|x| / 127, s = numpy's f16 rounding of s32, i = clip(rint(x / s),
    -127, 127); s == 0 gives i == 0.  Returns (int8 codes, f16 scales)."""
    x = np.asarray(x16, np.float16).astype(np.float32)
    s32 = (np.max(np.abs(x), axis=-1) / np.float32(127.0)).astype(np.float32)
    s16 = s32.astype(np.float16)
    s = s16.astype(np.float32)
    with np.errstate(divide="ignore", invalid="ignore"):
        i = np.rint((x / s[..., None]).astype(np.float32))
    i = np.where(s[..., None] > 0, i, 0.0)
    return np.clip(i, -127, 127).astype(np.int8), s16


def pack_bytes(codes):
    """int8 [..., D] -> u32 [..., D/4]: element d is byte d % 4 of word d / 4, LSB first."""
    u = np.asarray(codes, np.int8).view(np.uint8).astype(np.uint32).reshape(codes.shape[:-1] + (-1, 4))
    return u[..., 0] | (u[..., 1] << 8) | (u[..., 2] << 16) | (u[..., 3] << 24)


def tiered_after_appends(tokens_k, tokens_v, hot_window, table, bs, num_blocks):
    """The tiered cache that holds the token histories tokens_k/v[b] ([T_b, Hkv, D] f16)
    when every token was appended one at a time: the last min(T, hot_window)
    tokens sit in ring slot t mod hot_window, the older ones are int8 in the
    cold pool at row table[b][t // bs] * bs + t % bs."""
    B = len(tokens_k)
    Hkv, D = tokens_k[0].shape[1:]
    k_hot = np.zeros((B, hot_window, Hkv, D), np.float16)
    v_hot = np.zeros_like(k_hot)
    k_cold = np.zeros((num_blocks, bs, Hkv, D // 4), np.uint32)
    v_cold = np.zeros_like(k_cold)
    k_sc = np.zeros((num_blocks, bs, Hkv), np.float16)
    v_sc = np.zeros_like(k_sc)
    seq = np.zeros(B, np.int32)
    cold = np.zeros(B, np.int32)
    for b in range(B):
        T = len(tokens_k[b])
        C = max(0, T - hot_window)
        seq[b], cold[b] = T, C
        for t in range(C, T):
            k_hot[b, t % hot_window] = tokens_k[b][t]
            v_hot[b, t % hot_window] = tokens_v[b][t]
        if C:
            ck, sk = quantize_f16_rows(tokens_k[b][:C])
            cv, sv = quantize_f16_rows(tokens_v[b][:C])
            t = np.arange(C)
            blk, off = table[b, t // bs], t % bs
            k_cold[blk, off] = pack_bytes(ck)
            v_cold[blk, off] = pack_bytes(cv)
            k_sc[blk, off] = sk
            v_sc[blk, off] = sv
    return k_hot, v_hot, k_cold, v_cold, k_sc, v_sc, seq, cold
