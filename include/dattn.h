/*
 * dattn.h -- C ABI of the MI355X (gfx950) split-KV decode-attention library.
 *
 * One query token per sequence ("decode"), or a few (multi-query decode, see
 * dattn_params.query_len), with grouped-query attention (GQA): query head h
 * reads kv head h / (num_heads / num_kv_heads)
 * (doppler attention_decode_tiered_int8_f16kv.wgsl, get_kv_head_idx).
 * For every sequence b and query head h the library computes
 *
 *     out[b,h,:] = sum_t softmax_t(s_t) * v_t          lse[b,h] = ln sum_t e^{s_t}
 *     s_t        = softcap(scale * <q[b,h,:], k_t>)    over the visible keys t
 *
 * with softcap(x) = cap * tanh(x / cap) when cap > 0 (applied after scaling and
 * before masking, the order of the doppler kernels' score loop).  Visible keys
 * are t in [0, seq_lens[b]) that survive the masks of doppler's is_masked:
 * with causal, keys t > q are dropped; with a window W > 0, keys t < q-W+1 are
 * dropped once q >= W.  q is the query's absolute position: q_pos[b], or
 * seq_lens[b]-1 when q_pos is NULL.  A query with no visible key gets out = 0
 * and lse = -inf.  lse is the natural log-sum-exp of the capped scores
 * (boostr paged_attention.wgsl, paged_attention_fwd_f32's lse output).
 *
 * Caches: paged f16/f32 (dattn_decode_paged), tiered int8 cold + f16 ring
 * (dattn_decode_tiered_int8), tiered f16 cold + f16 ring
 * (dattn_decode_tiered_f16), sliding-window ring (dattn_decode_ring_f16),
 * block-sparse CSR over the paged f16 cache (dattn_decode_block_sparse).
 * Write paths: dattn_append_tiered_int8 (quantise on evict) and
 * dattn_append_ring_f16.
 *
 * Conventions shared by every entry point
 *   - All array arguments are DEVICE pointers on the current HIP device,
 *     C-contiguous, owned by the caller; the library keeps no reference after
 *     the call returns and allocates no device memory.
 *   - Work is enqueued on `stream` (a hipStream_t passed as void*, NULL = the
 *     null stream) and is asynchronous: outputs are valid once the stream has
 *     reached the enqueued work.  No host synchronisation happens inside.
 *   - Scratch memory for the split partials is the caller's `workspace`
 *     (size from dattn_workspace_size, 256-byte aligned).
 *   - Every argument the host can see is validated before any HIP call; on
 *     failure nothing is enqueued and a negative code is returned, with a
 *     message available from dattn_last_error() on the calling thread.
 *   - Device-side contents are NOT validated: block-table entries a visible
 *     token needs must lie in [0, num_blocks), seq_lens[b] <= max_seq_len,
 *     q_pos[b] >= 0, cold_lens[b] <= seq_lens[b], seq_lens[b]-cold_lens[b] <=
 *     hot_window.  Breaking these is undefined behaviour.
 *   - Concurrent calls on different streams are safe if their workspaces and
 *     outputs do not overlap.
 */
#ifndef DATTN_H
#define DATTN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* return codes */
#define DATTN_OK 0
#define DATTN_ERR_INVALID (-1)     /* an argument is out of range or inconsistent */
#define DATTN_ERR_UNSUPPORTED (-2) /* valid but not built: head_dim, GQA group, sizes */
#define DATTN_ERR_WORKSPACE (-3)   /* workspace NULL, misaligned or too small */
#define DATTN_ERR_LAUNCH (-4)      /* a HIP call failed; see dattn_last_error() */

/* storage types: paged K/V pool (kv_dtype), out (out_dtype), q (q_dtype) */
#define DATTN_F32 0
#define DATTN_F16 1

/* entry-point kinds, for dattn_workspace_size */
#define DATTN_KIND_PAGED 0
#define DATTN_KIND_TIERED_INT8 1
#define DATTN_KIND_BLOCK_SPARSE 2
#define DATTN_KIND_TIERED_F16 3
#define DATTN_KIND_RING_F16 4

/*
 * Scalar parameters (doppler attention_f16kv.wgsl Uniforms and boostr
 * PagedParams; doppler attention.js executeAttentionTieredQuant defaults).
 */
typedef struct dattn_params {
  int32_t num_seqs;           /* B >= 0 (0 enqueues nothing) */
  int32_t num_heads;          /* H >= 1 query heads */
  int32_t num_kv_heads;       /* Hkv >= 1, H % Hkv == 0; G = H/Hkv in {1, 2, 4, 8} */
  int32_t head_dim;           /* D in {64, 128} */
  float scale;                /* score scale; 0 => 1/sqrt(D) rounded to f32 */
  int32_t causal;             /* 0 or 1 */
  int32_t sliding_window;     /* W >= 0; 0 => no window */
  float softcap;              /* cap; <= 0 => no softcap */
  int32_t block_size;         /* tokens per physical block, >= 1 */
  int32_t max_blocks_per_seq; /* row stride of the block table, >= 1 */
  int32_t num_blocks;         /* physical blocks in the pool, >= 1 */
  int32_t max_seq_len;        /* host-known upper bound of seq_lens[], >= 0; sizes the grid */
  int32_t split_tokens;       /* keys per KV split (block-sparse: at most split_tokens / sparse_block
                                 union blocks per split); 0 => library choice, else a multiple of 16 */
  int32_t phases;             /* 0 (or DATTN_PHASE_ALL) => both phases; see below */
  int32_t out_dtype;          /* storage type of out: DATTN_F32 (0) or DATTN_F16, the f32
                                 result rounded to nearest even (attention.js sizes its output
                                 by the kernel variant's outputDtype, f16 or f32) */
  int32_t query_len;          /* queries per sequence, 0 or 1 => one; > 1: multi-query decode
                                 (every cache; query_len * GQA group <= 128, else
                                 DATTN_ERR_UNSUPPORTED); see dattn_decode_paged */
  int32_t q_dtype;            /* storage type of q: DATTN_F32 (0) or DATTN_F16 (converted to f32
                                 exactly); with DATTN_F16 and out_dtype DATTN_F16 this is the f16
                                 Q/K/V, f16 output variant (doppler attention_f16.wgsl) */
} dattn_params;

/*
 * Phases of one call.  A call runs two kernels on `stream`: the split kernel
 * writes one partial (m, l, acc[D]) per (sequence, head, KV split) into the
 * workspace, and the combine kernel merges the partials of every
 * (sequence, head) into out / lse with the pairwise rule of
 * SparseAttention's combine_partials (m = max(m1, m2),
 * l = l1 e^{m1-m} + l2 e^{m2-m}, acc likewise).  DATTN_PHASE_SPLIT enqueues
 * only the first kernel (out and lse are not touched and may be NULL);
 * DATTN_PHASE_COMBINE enqueues only the second and reads partials left in the
 * workspace by an earlier DATTN_PHASE_SPLIT call with identical parameters
 * (only out, lse and workspace are read from the arguments).
 * Workspace layout: acc f32 [B, H, S, D] at offset 0, then, at the next
 * 256-byte boundary, (m, l) f32 pairs [B, H, S]; m is in log2 units
 * (m_nat = m * ln 2); l == 0 marks a split with no visible key (acc unset).
 */
#define DATTN_PHASE_ALL 0
#define DATTN_PHASE_SPLIT 1
#define DATTN_PHASE_COMBINE 2

/*
 * Workspace bytes a call of `kind` with these parameters needs.
 * sparse_block is read only for DATTN_KIND_BLOCK_SPARSE.  For that kind with
 * split_tokens == 0 the split count follows the current device's CU count
 * (256 assumed when no device can be queried), so query the size with the
 * device current that the calls will run on.
 * Returns DATTN_OK and writes *bytes, or a negative code.
 */
int dattn_workspace_size(const dattn_params* p, int32_t kind, int32_t sparse_block, size_t* bytes);

/*
 * Paged cache (boostr paged_attention.wgsl: token t of sequence b lives in
 * physical block block_table[b][t / block_size] at offset t % block_size).
 *   q            [B, H, D] f32, or f16 per p->q_dtype; 16-byte aligned
 *   k_cache,
 *   v_cache      [num_blocks, block_size, Hkv, D], f32 or f16 per kv_dtype
 *   block_table  [B, max_blocks_per_seq] i32
 *   seq_lens     [B] i32
 *   q_pos        [B] i32, or NULL for seq_lens[b]-1
 *   out          [B, H, D] f32 or f16 per p->out_dtype (written), or NULL to
 *                write lse only (the split kernel still reads K and V)
 *   lse          [B, H] f32 (written), or NULL; out and lse are not both NULL
 * Multi-query decode (p->query_len = Qn > 1; doppler attention_f16kv.wgsl,
 * query rows at abs_query = query_pos + start_pos): q is [B, Qn, H, D], query
 * i of sequence b sits at position q_pos[b] + i (q_pos NULL: seq_lens[b] - Qn,
 * the last Qn tokens of the cache) with its own causal / window bound; out is
 * [B, Qn, H, D] and lse [B, Qn, H].  The Qn * G (query, head) rows of a kv
 * head (at most 128) are taken 16 at a time by the waves of one workgroup,
 * which sweep the same keys side by side, so each K/V row is fetched from HBM
 * about once per (sequence, kv head) for all of them.  The tiered and
 * window-ring entry points take query_len the same way, and so does the
 * block-sparse one, whose waves each build the block union of their own 16
 * rows.
 */
int dattn_decode_paged(const dattn_params* p, const void* q, const void* k_cache, const void* v_cache,
                       int32_t kv_dtype, const int32_t* block_table, const int32_t* seq_lens,
                       const int32_t* q_pos, void* out, float* lse, void* workspace, size_t workspace_bytes,
                       void* stream);

/*
 * Tiered cache (doppler attention_decode_tiered_int8_f16kv.wgsl and
 * attention.js executeAttentionTieredQuant / executeAttentionTiered):
 * tokens t < cold_lens[b] are int8 in a paged cold pool, tokens
 * t >= cold_lens[b] are f16 in a per-sequence ring at slot t % hot_window.
 *   k_hot, v_hot          [B, hot_window, Hkv, D] f16 (bit patterns)
 *   hot_window            ring slots, >= 1
 *   k_cold, v_cold        [num_blocks, block_size, Hkv, D/4] u32; element d of a
 *                         row is byte d%4 of word d/4, least-significant byte
 *                         first, two's complement (read_cold_k / read_cold_v)
 *   k_scale, v_scale      [num_blocks, block_size, Hkv] f16 (bit patterns);
 *                         the value of element d is int8 * f32(scale)
 *   cold_block_table      [B, max_blocks_per_seq] i32 (block_size, num_blocks and
 *                         max_blocks_per_seq in p describe the cold pool)
 *   seq_lens, cold_lens   [B] i32
 *   q_pos, out, lse       as for dattn_decode_paged
 */
int dattn_decode_tiered_int8(const dattn_params* p, const void* q, const uint16_t* k_hot,
                             const uint16_t* v_hot, int32_t hot_window, const uint32_t* k_cold,
                             const uint32_t* v_cold, const uint16_t* k_scale, const uint16_t* v_scale,
                             const int32_t* cold_block_table, const int32_t* seq_lens, const int32_t* cold_lens,
                             const int32_t* q_pos, void* out, float* lse, void* workspace,
                             size_t workspace_bytes, void* stream);

/*
 * dattn_decode_tiered_int8 for callers that cannot allocate device memory
 * (code under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc): the same arguments without the workspace.  The split partials go
 * to a static scratch array inside the library, 32 MiB on each device (held
 * from the first call on that device until the process ends).  A call whose
 * partials need more (dattn_workspace_size with DATTN_KIND_TIERED_INT8 above
 * 32 MiB) returns DATTN_ERR_UNSUPPORTED before anything is enqueued.  The call
 * allocates nothing; the caller still provides q, the cache arrays, out and
 * lse.  Every call on a device uses that device's one scratch array: calls
 * that overlap on one device (other streams, other host threads) race and
 * give wrong results; calls ordered on one stream are safe.  Nothing in the
 * scratch needs clearing between calls (each call writes every partial it
 * reads).  The first call on a device looks up the scratch's device address
 * (hipGetSymbolAddress) with that device current.
 */
int dattn_decode_tiered_int8_static(const dattn_params* p, const void* q, const uint16_t* k_hot,
                                    const uint16_t* v_hot, int32_t hot_window, const uint32_t* k_cold,
                                    const uint32_t* v_cold, const uint16_t* k_scale, const uint16_t* v_scale,
                                    const int32_t* cold_block_table, const int32_t* seq_lens,
                                    const int32_t* cold_lens, const int32_t* q_pos, void* out, float* lse,
                                    void* stream);

/*
 * Tiered cache with an f16 cold tier (attention.js executeAttentionTiered:
 * f16 hot and cold buffers, the cold tier paged through a page table by
 * default, the hot tier a ring): tokens t < cold_lens[b] are f16 rows of a
 * paged cold pool, tokens t >= cold_lens[b] f16 rows of the ring at slot
 * t % hot_window, exactly as for dattn_decode_tiered_int8.
 *   k_hot, v_hot          [B, hot_window, Hkv, D] f16 (bit patterns)
 *   hot_window            ring slots, >= 1
 *   k_cold, v_cold        [num_blocks, block_size, Hkv, D] f16 (bit patterns)
 *   cold_block_table      [B, max_blocks_per_seq] i32 (block_size, num_blocks and
 *                         max_blocks_per_seq in p describe the cold pool)
 *   seq_lens, cold_lens   [B] i32
 *   q_pos, out, lse       as for dattn_decode_paged
 * Workspace size: kind DATTN_KIND_TIERED_F16.
 */
int dattn_decode_tiered_f16(const dattn_params* p, const void* q, const uint16_t* k_hot, const uint16_t* v_hot,
                            int32_t hot_window, const uint16_t* k_cold, const uint16_t* v_cold,
                            const int32_t* cold_block_table, const int32_t* seq_lens, const int32_t* cold_lens,
                            const int32_t* q_pos, void* out, float* lse, void* workspace, size_t workspace_bytes,
                            void* stream);

/*
 * Sliding-window ring f16 cache (doppler attention_f16kv.wgsl, get_kv_pos
 * with the ring layout): each sequence owns W = p->sliding_window slots and
 * token t lives at slot t % W, so only the last W tokens,
 * [max(0, seq_lens[b] - W), seq_lens[b]), are resident; the visible keys are
 * those resident keys that pass the causal / window masks (a query before the
 * last token cannot see keys the ring has already overwritten).
 *   k_ring, v_ring  [B, W, Hkv, D] f16 (bit patterns); W = p->sliding_window >= 1
 *   seq_lens        [B] i32, tokens written so far (may exceed W)
 *   q_pos, out, lse as for dattn_decode_paged
 * block_size, max_blocks_per_seq and num_blocks in p are ignored.  Workspace
 * size: kind DATTN_KIND_RING_F16.
 */
int dattn_decode_ring_f16(const dattn_params* p, const void* q, const uint16_t* k_ring, const uint16_t* v_ring,
                          const int32_t* seq_lens, const int32_t* q_pos, void* out, float* lse, void* workspace,
                          size_t workspace_bytes, void* stream);

/*
 * Block-sparse selection over the paged f16 cache (com.microsoft.SparseAttention
 * sparse-attention.wgsl.jinja, attention pass): head h uses CSR layout
 * h % num_layouts; row r = q / sparse_block lists the sparse blocks (of
 * sparse_block consecutive keys) the query may see; columns > r are ignored
 * and a repeated column counts once.  Keys inside a chosen block still pass
 * the causal / window masks.
 *   sparse_block  keys per sparse block, a multiple of block_size
 *   row_ptr       [num_layouts, row_stride] i32, row_stride = rows + 1
 *   col_idx       [num_layouts, col_stride] i32
 *   other arrays  as for dattn_decode_paged with kv_dtype = DATTN_F16
 * Needs q / sparse_block < row_stride - 1 (rows beyond select nothing).
 * Multi-query decode (p->query_len = Qn > 1): query i at position q_pos[b] + i
 * takes the CSR row of its own position; a query before position 0 selects
 * no block.
 */
int dattn_decode_block_sparse(const dattn_params* p, const void* q, const uint16_t* k_cache,
                              const uint16_t* v_cache, const int32_t* block_table, const int32_t* seq_lens,
                              const int32_t* q_pos, int32_t sparse_block, int32_t num_layouts,
                              const int32_t* row_ptr, int32_t row_stride, const int32_t* col_idx,
                              int32_t col_stride, void* out, float* lse, void* workspace, size_t workspace_bytes,
                              void* stream);

/*
 * Write path of the tiered cache: append one token per sequence (the step
 * that produces the data dattn_decode_tiered_int8 reads).  For every
 * sequence b with L = seq_lens[b], C = cold_lens[b]:
 *   - if the ring is full (L - C == hot_window), the oldest hot token
 *     (absolute position C, ring slot C % hot_window) is quantised into the
 *     cold tier at position C (block cold_block_table[b][C / block_size],
 *     offset C % block_size) and cold_lens[b] becomes C + 1;
 *   - the new token k_new[b], v_new[b] goes to ring slot L % hot_window and
 *     seq_lens[b] becomes L + 1.
 * The ring slot and cold-row conventions are those of the tiered decode
 * (doppler attention_decode_tiered_int8_f16kv.wgsl get_hot_pos and
 * read_cold_k; attention.js pages the cold tier).  The quantiser is not on
 * the pages; it follows the tiered workload's description (f16 scale =
 * max|x| / 127 per (token, kv head)), every decision in f32:
 * s = f16(max|x| / 127) rounded to nearest even,
 * code = clamp(rint(x / s), -127, 127), an all-zero row giving s = 0.
 *   k_new, v_new          [B, Hkv, D] f16 (bit patterns), read
 *   k_hot, v_hot          [B, hot_window, Hkv, D] f16, updated
 *   k_cold, v_cold        [num_blocks, block_size, Hkv, D/4] u32, updated
 *   k_scale, v_scale      [num_blocks, block_size, Hkv] f16, updated
 *   cold_block_table      [B, max_blocks_per_seq] i32; the entry for the block
 *                         of position C must be allocated before an eviction
 *   seq_lens, cold_lens   [B] i32 on the device, advanced in place
 * Reads num_seqs, num_kv_heads, head_dim (64 or 128), block_size,
 * max_blocks_per_seq and num_blocks from p.  Needs no workspace.  A sequence
 * whose device state breaks 0 <= C <= L, L - C <= hot_window, or whose
 * needed table entry is outside [0, num_blocks), is left unchanged.
 * Overlapping calls on the same cache race.
 */
int dattn_append_tiered_int8(const dattn_params* p, const uint16_t* k_new, const uint16_t* v_new, uint16_t* k_hot,
                             uint16_t* v_hot, int32_t hot_window, uint32_t* k_cold, uint32_t* v_cold,
                             uint16_t* k_scale, uint16_t* v_scale, const int32_t* cold_block_table,
                             int32_t* seq_lens, int32_t* cold_lens, void* stream);

/*
 * Write path of the window ring: append one token per sequence.  The new
 * token k_new[b], v_new[b] goes to slot seq_lens[b] % W (W =
 * p->sliding_window >= 1), overwriting the token that leaves the window, and
 * seq_lens[b] becomes seq_lens[b] + 1 (the slot rule of
 * dattn_decode_ring_f16).
 *   k_new, v_new    [B, Hkv, D] f16 (bit patterns), read
 *   k_ring, v_ring  [B, W, Hkv, D] f16, updated
 *   seq_lens        [B] i32 on the device, advanced in place
 * Reads num_seqs, num_kv_heads, head_dim (64 or 128) and sliding_window from
 * p.  Needs no workspace.  A sequence with a negative length is left
 * unchanged.  Overlapping calls on the same ring race.
 */
int dattn_append_ring_f16(const dattn_params* p, const uint16_t* k_new, const uint16_t* v_new, uint16_t* k_ring,
                          uint16_t* v_ring, int32_t* seq_lens, void* stream);

/*
 * Measurement helper, not part of the attention method: a plain streaming
 * read of `bytes` bytes (a multiple of 16, src 16-byte aligned) with 128-bit
 * nontemporal loads (4 workgroups of 1024 threads per CU).  It gives the
 * measured read ceiling that kernel rates are reported against.  *sink
 * (device, 4 bytes) is written only if the data fold to one particular 32-bit
 * value.  Enqueued on `stream`.
 */
int dattn_stream_read(const void* src, size_t bytes, uint32_t* sink, void* stream);

/* Message for the last non-zero return on this thread ("" if none). */
const char* dattn_last_error(void);

/* Library version string. */
const char* dattn_version(void);

#ifdef __cplusplus
}
#endif

#endif /* DATTN_H */
