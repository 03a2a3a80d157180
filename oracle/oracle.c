/*
 * oracle.c -- plain, slow fp64 CPU oracle for single-query (decode) GQA
 * attention over a paged f16/f32 KV cache, a tiered int8-cold / f16-hot
 * cache, a tiered f16-cold / f16-hot cache, and a block-sparse (CSR)
 * selection over the paged cache.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the product library calls, links or
 * includes this file; it exists so that the HIP path can be compared against
 * an obviously correct definition.  It shares no header, helper, table or
 * constant with the GPU code.
 *
 * What it computes (for every requested (sequence b, query head h)):
 *
 *   g   = h / (H / Hkv)                       GQA head map, doppler
 *                                             attention_decode_tiered_int8_f16kv.wgsl,
 *                                             get_kv_head_idx
 *   q   = q_pos[b] if given, else L-1         the absolute query position
 *                                             (start_pos in the doppler kernels;
 *                                             total-1 in SparseAttention decode)
 *   V   = { t in [0,L) : visible(t) }         is_masked in the doppler kernels:
 *                                             causal drops t > q; a window W > 0
 *                                             drops t < q-W+1 once q >= W
 *   s_t = scale * sum_d q[b,h,d] * k_t[d]     then s_t <- cap*tanh(s_t/cap) when
 *                                             cap > 0 (score, softcap, then mask:
 *                                             the order of the doppler kernels)
 *   out = sum_t e^{s_t-M} v_t / sum_t e^{s_t-M},  M = max_t s_t
 *   lse = M + ln(sum_t e^{s_t-M})             boostr paged_attention.wgsl, the
 *                                             lse write of paged_attention_fwd_f32
 *   empty V: out = 0, lse = -inf.
 *
 * Multi-query decode (query_len = Qn > 1): q holds Qn query rows per
 * sequence, [B, Qn, H, D]; query i of sequence b sits at absolute position
 * q0 + i with q0 = q_pos[b], or L - Qn when q_pos is not given (the queries
 * are the last Qn tokens of the cache), and each query has its own visible
 * set (doppler attention_f16kv.wgsl: abs_query = query_pos + start_pos in
 * is_masked).  Outputs are [B, Qn, H, D] and [B, Qn, H].
 *
 * The softmax is evaluated as the plain two-pass definition (max, then
 * exp-sum and weighted sum), in double precision, with no online rescaling.
 *
 * Where k_t and v_t come from:
 *   paged:  block p = block_table[b][t / bs], offset o = t % bs, row
 *           cache[p][o][g][0..D) (boostr paged_attention.wgsl, the k_base /
 *           v_base indexing of paged_attention_fwd_f32), stored f32 or f16.
 *   tiered: t < cold_len[b]: the same paged map through cold_block_table, the
 *           row holds D/4 u32 words, element d is byte (d % 4) of word d / 4,
 *           least-significant byte first, two's complement, times the f16
 *           scale of (p, o, g) (doppler attention_decode_tiered_int8_f16kv.wgsl,
 *           read_cold_k / read_cold_v);
 *           t >= cold_len[b]: hot ring slot t mod hot_window of
 *           hot[b][slot][g][0..D) in f16 (get_hot_pos, with the hot tier's
 *           first absolute position equal to cold_len[b]).
 *   tiered f16: as tiered, but the cold row is D f16 values, the paged
 *           layout of the paged cache read through cold_block_table
 *           (attention.js executeAttentionTiered: f16 hot and cold buffers,
 *           the cold tier paged by default).
 *   window ring: a per-sequence ring of W = sliding_window slots holding
 *           the last W tokens, token t at slot t mod W (doppler
 *           attention_f16kv.wgsl, get_kv_pos with the ring layout); only
 *           t in [max(0, L-W), L) is resident, so the visible set is
 *           intersected with that range (the kv_start / kv_len range of the
 *           same kernel).
 *   sparse: the paged cache, and t is visible to head h only if its sparse
 *           block j = t / SB is a column of row r = q / SB of CSR layout
 *           (h mod NL) and j <= r; repeated columns count once
 *           (com.microsoft.SparseAttention sparse-attention.wgsl.jinja, the
 *           slot-resolution loop of the attention pass).
 *
 * The write path (orc_append_tiered_int8) appends one token per sequence to
 * the tiered cache: when the hot ring already holds hot_window tokens, the
 * oldest hot token (absolute position cold_len[b], ring slot
 * cold_len[b] mod hot_window) is first quantised into the paged cold tier at
 * position cold_len[b] and cold_len[b] grows by one; the new token then goes
 * to ring slot seq_len[b] mod hot_window and seq_len[b] grows by one.  The
 * quantiser is not on the pages; it is the one the tiered workload's data is
 * described with (a per-(token, kv head) f16 scale max|x|/127), read as:
 * s32 = max|x| / 127 in f32, s = s32 rounded to f16 (nearest even),
 * i = clamp(rint(x / f32(s)), -127, 127) in f32, an all-zero row giving
 * s = 0 and i = 0.
 *
 * The window ring's write path (orc_append_ring_f16) stores the new token at
 * slot seq_len[b] mod W, overwriting the token that leaves the window.
 *
 * Every function validates its inputs enough never to read out of bounds and
 * returns a negative code otherwise.
 */
#include <float.h>
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

#define ORC_OK 0
#define ORC_EINVAL (-1)
#define ORC_ENOMEM (-5)

enum { ORC_F32 = 0, ORC_F16 = 1 };

typedef struct {
  int32_t num_seqs;
  int32_t num_heads;
  int32_t num_kv_heads;
  int32_t head_dim;
  float scale;            /* 0 => 1/sqrt(head_dim), rounded to f32 */
  int32_t causal;
  int32_t sliding_window; /* 0 => no window */
  float softcap;          /* <= 0 => no softcap */
  int32_t block_size;
  int32_t max_blocks_per_seq;
  int32_t num_blocks;     /* rows of the physical pool, for bounds checks */
  int32_t query_len;      /* queries per sequence; 0 or 1 => one */
} orc_params;

/* ---------------------------------------------------------------- scalars */

/* IEEE 754 binary16 -> double, from the format's definition: 1 sign bit,
 * 5 exponent bits (bias 15), 10 fraction bits; exponent 0 is subnormal,
 * exponent 31 is inf/NaN. */
double orc_f16_to_f64(uint16_t bits) {
  int sign = (bits >> 15) & 1;
  int e = (bits >> 10) & 31;
  int m = bits & 1023;
  double v;
  if (e == 0)
    v = ldexp((double)m, -24);
  else if (e == 31)
    v = m ? NAN : INFINITY;
  else
    v = ldexp((double)(1024 + m), e - 25);
  return sign ? -v : v;
}

/* Byte `lane` (0..3) of a packed word, least-significant byte first, read as
 * two's complement (doppler read_cold_k: shift by 8*lane, mask 0xff, subtract
 * 256 from values >= 128). */
int32_t orc_int8_lane(uint32_t word, int32_t lane) {
  uint32_t byte = (word >> (8u * (uint32_t)lane)) & 0xffu;
  return byte >= 128u ? (int32_t)byte - 256 : (int32_t)byte;
}

/* Visibility of absolute key t to a query at absolute position q in a
 * sequence of length L (doppler is_masked, plus the sequence bound). */
int32_t orc_key_visible(int64_t t, int64_t q, int64_t L, int32_t causal, int32_t window) {
  if (t < 0 || t >= L) return 0;
  if (causal && t > q) return 0;
  if (window > 0 && q >= window && t < q - window + 1) return 0;
  return 1;
}

/* Hot-ring slot of absolute position t (doppler get_hot_pos with the hot
 * tier starting at absolute position cold_len). */
int64_t orc_ring_slot(int64_t t, int32_t hot_window) { return t % hot_window; }

static double orc_scale(const orc_params* p) {
  if (p->scale != 0.0f) return (double)p->scale;
  return (double)(float)(1.0 / sqrt((double)p->head_dim));
}

/* ------------------------------------------------------------ row sources */

typedef struct {
  const orc_params* p;
  const void* k;
  const void* v;
  int32_t dtype;
  const int32_t* block_table;
} paged_src;

typedef struct {
  const orc_params* p;
  const uint16_t* k_hot;
  const uint16_t* v_hot;
  int32_t hot_window;
  const uint32_t* k_cold;
  const uint32_t* v_cold;
  const uint16_t* k_scale;
  const uint16_t* v_scale;
  const int32_t* cold_block_table;
  const int32_t* cold_lens;
} tiered_src;

typedef void (*row_fn)(const void* src, int32_t b, int32_t g, int64_t t, int32_t is_v, double* dst);

/* Physical row index (p*bs + o) of logical token t of sequence b. */
static int64_t paged_row(const orc_params* p, const int32_t* table, int32_t b, int64_t t) {
  int64_t blk = table[(int64_t)b * p->max_blocks_per_seq + t / p->block_size];
  return blk * p->block_size + t % p->block_size;
}

static void paged_fetch(const void* vsrc, int32_t b, int32_t g, int64_t t, int32_t is_v, double* dst) {
  const paged_src* s = (const paged_src*)vsrc;
  const orc_params* p = s->p;
  int64_t base = (paged_row(p, s->block_table, b, t) * p->num_kv_heads + g) * p->head_dim;
  const void* cache = is_v ? s->v : s->k;
  for (int32_t d = 0; d < p->head_dim; ++d) {
    if (s->dtype == ORC_F32)
      dst[d] = (double)((const float*)cache)[base + d];
    else
      dst[d] = orc_f16_to_f64(((const uint16_t*)cache)[base + d]);
  }
}

static void tiered_fetch(const void* vsrc, int32_t b, int32_t g, int64_t t, int32_t is_v, double* dst) {
  const tiered_src* s = (const tiered_src*)vsrc;
  const orc_params* p = s->p;
  int32_t D = p->head_dim;
  if (t < s->cold_lens[b]) {
    int64_t row = paged_row(p, s->cold_block_table, b, t) * p->num_kv_heads + g;
    const uint32_t* words = (is_v ? s->v_cold : s->k_cold) + row * (D / 4);
    double sc = orc_f16_to_f64((is_v ? s->v_scale : s->k_scale)[row]);
    for (int32_t d = 0; d < D; ++d) dst[d] = (double)orc_int8_lane(words[d / 4], d % 4) * sc;
  } else {
    int64_t slot = orc_ring_slot(t, s->hot_window);
    const uint16_t* hot = is_v ? s->v_hot : s->k_hot;
    int64_t base = (((int64_t)b * s->hot_window + slot) * p->num_kv_heads + g) * D;
    for (int32_t d = 0; d < D; ++d) dst[d] = orc_f16_to_f64(hot[base + d]);
  }
}

/* Tiered f16: paged f16 cold rows through cold_block_table, then the ring. */
static void tiered_f16_fetch(const void* vsrc, int32_t b, int32_t g, int64_t t, int32_t is_v, double* dst) {
  const tiered_src* s = (const tiered_src*)vsrc;
  const orc_params* p = s->p;
  int32_t D = p->head_dim;
  const uint16_t* rows;
  int64_t base;
  const int32_t in_cold = t < s->cold_lens[b];
  if (in_cold) {
    rows = (const uint16_t*)(is_v ? (const void*)s->v_cold : (const void*)s->k_cold);
    base = (paged_row(p, s->cold_block_table, b, t) * p->num_kv_heads + g) * D;
  } else {
    rows = is_v ? s->v_hot : s->k_hot;
    base = (((int64_t)b * s->hot_window + orc_ring_slot(t, s->hot_window)) * p->num_kv_heads + g) * D;
  }
  for (int32_t d = 0; d < D; ++d) dst[d] = orc_f16_to_f64(rows[base + d]);
}

/* Window ring: ring[b][t mod W][g][0..D) in f16. */
typedef struct {
  const orc_params* p;
  const uint16_t* k;
  const uint16_t* v;
  int32_t ring;
} ring_src;

static void ring_fetch(const void* vsrc, int32_t b, int32_t g, int64_t t, int32_t is_v, double* dst) {
  const ring_src* s = (const ring_src*)vsrc;
  const orc_params* p = s->p;
  const int64_t base = (((int64_t)b * s->ring + t % s->ring) * p->num_kv_heads + g) * p->head_dim;
  const uint16_t* rows = is_v ? s->v : s->k;
  for (int32_t d = 0; d < p->head_dim; ++d) dst[d] = orc_f16_to_f64(rows[base + d]);
}

/* -------------------------------------------------------------- attention */

/* Attention of one query head over an explicit list of visible tokens. */
/* q row `qrow` (flat index into [B, Qn, H]) of sequence b and query head h. */
static int head_attend(const orc_params* p, const float* q, int64_t qrow, int32_t b, int32_t h, const int64_t* toks,
                       int64_t n, row_fn fetch, const void* src, double* out, double* lse) {
  int32_t D = p->head_dim;
  int32_t g = h / (p->num_heads / p->num_kv_heads);
  double scale = orc_scale(p);
  double cap = (double)p->softcap;
  if (n == 0) {
    for (int32_t d = 0; d < D; ++d) out[d] = 0.0;
    *lse = -INFINITY;
    return ORC_OK;
  }
  double* qv = (double*)malloc(sizeof(double) * D);
  double* row = (double*)malloc(sizeof(double) * D);
  double* acc = (double*)calloc(D, sizeof(double));
  double* s = (double*)malloc(sizeof(double) * n);
  if (!qv || !row || !acc || !s) {
    free(qv), free(row), free(acc), free(s);
    return ORC_ENOMEM;
  }
  for (int32_t d = 0; d < D; ++d) qv[d] = (double)q[qrow * D + d];

  /* pass 1: scores, then their maximum */
  double M = -INFINITY;
  for (int64_t i = 0; i < n; ++i) {
    fetch(src, b, g, toks[i], 0, row);
    double dot = 0.0;
    for (int32_t d = 0; d < D; ++d) dot += qv[d] * row[d];
    double x = scale * dot;
    if (cap > 0.0) x = cap * tanh(x / cap);
    s[i] = x;
    if (x > M) M = x;
  }
  /* pass 2: normaliser and weighted sum of values */
  double ell = 0.0;
  for (int64_t i = 0; i < n; ++i) {
    double w = exp(s[i] - M);
    ell += w;
    fetch(src, b, g, toks[i], 1, row);
    for (int32_t d = 0; d < D; ++d) acc[d] += w * row[d];
  }
  for (int32_t d = 0; d < D; ++d) out[d] = acc[d] / ell;
  *lse = M + log(ell);
  free(qv), free(row), free(acc), free(s);
  return ORC_OK;
}

static int check_common(const orc_params* p) {
  if (!p) return ORC_EINVAL;
  if (p->num_seqs < 0 || p->num_heads <= 0 || p->num_kv_heads <= 0 || p->head_dim <= 0) return ORC_EINVAL;
  if (p->num_heads % p->num_kv_heads) return ORC_EINVAL;
  if (p->block_size <= 0 || p->max_blocks_per_seq < 0 || p->num_blocks < 0) return ORC_EINVAL;
  if (p->sliding_window < 0 || p->query_len < 0) return ORC_EINVAL;
  return ORC_OK;
}

/* Every table entry a sequence of length `len` uses must name a pool row. */
static int check_table(const orc_params* p, const int32_t* table, int32_t b, int64_t len) {
  if (len <= 0) return ORC_OK;
  int64_t nblk = (len + p->block_size - 1) / p->block_size;
  if (nblk > p->max_blocks_per_seq) return ORC_EINVAL;
  for (int64_t j = 0; j < nblk; ++j) {
    int32_t e = table[(int64_t)b * p->max_blocks_per_seq + j];
    if (e < 0 || e >= p->num_blocks) return ORC_EINVAL;
  }
  return ORC_OK;
}

static int32_t queries(const orc_params* p) { return p->query_len > 1 ? p->query_len : 1; }

/* Absolute position of query i of sequence b. */
static int64_t query_pos(const orc_params* p, const int32_t* q_pos, const int32_t* seq_lens, int32_t b, int32_t i) {
  return (q_pos ? (int64_t)q_pos[b] : (int64_t)seq_lens[b] - queries(p)) + i;
}

/* Sparse selection for one head: sel[j] = 1 iff block j <= r is a column of
 * row r of layout (h mod NL). */
typedef struct {
  int32_t sparse_block, num_layouts, row_stride, col_stride;
  const int32_t* row_ptr;
  const int32_t* col_idx;
} sparse_csr;

static int sparse_select(const sparse_csr* c, int32_t h, int64_t q, unsigned char* sel, int64_t nsel) {
  memset(sel, 0, (size_t)nsel);
  if (q < 0) return ORC_OK;   /* a query before position 0 has no CSR row: it selects no block */
  int64_t r = q / c->sparse_block;
  if (r + 1 >= c->row_stride) return ORC_EINVAL;
  int32_t layout = h % c->num_layouts;
  const int32_t* rp = c->row_ptr + (int64_t)layout * c->row_stride;
  int32_t start = rp[r], end = rp[r + 1];
  if (start < 0 || end < start || end > c->col_stride) return ORC_EINVAL;
  for (int32_t e = start; e < end; ++e) {
    int32_t j = c->col_idx[(int64_t)layout * c->col_stride + e];
    if (j >= 0 && j <= r && j < nsel) sel[j] = 1;
  }
  return ORC_OK;
}

/* Shared driver: for each requested flat pair b*H+h, enumerate the visible
 * tokens and attend.  pairs == NULL means every pair in order.  resident > 0
 * keeps only the last `resident` tokens of each sequence (a ring). */
static int run_pairs(const orc_params* p, const float* q, const int32_t* seq_lens, const int32_t* q_pos,
                     const sparse_csr* csr, int32_t resident, row_fn fetch, const void* src, const int32_t* pairs,
                     int32_t npairs, int32_t nthreads, double* out, double* lse) {
  const int32_t Qn = queries(p);
  int64_t total = (int64_t)p->num_seqs * Qn * p->num_heads;
  if (!pairs) npairs = (int32_t)total;
  for (int32_t i = 0; i < npairs; ++i)
    if (pairs && (pairs[i] < 0 || pairs[i] >= total)) return ORC_EINVAL;
  int rc = ORC_OK;
#ifdef _OPENMP
  if (nthreads <= 0) nthreads = omp_get_max_threads();
#pragma omp parallel for schedule(dynamic, 1) num_threads(nthreads)
#endif
  for (int32_t i = 0; i < npairs; ++i) {
    int32_t flat = pairs ? pairs[i] : i;   /* (b * Qn + query) * H + h */
    int32_t h = flat % p->num_heads, bq = flat / p->num_heads;
    int32_t b = bq / Qn, qi = bq % Qn;
    int64_t L = seq_lens[b];
    int64_t qp = query_pos(p, q_pos, seq_lens, b, qi);
    int64_t* toks = (int64_t*)malloc(sizeof(int64_t) * (size_t)(L > 0 ? L : 1));
    unsigned char* sel = NULL;
    int local = toks ? ORC_OK : ORC_ENOMEM;
    int64_t nblk = csr ? (L + csr->sparse_block - 1) / csr->sparse_block : 0;
    if (local == ORC_OK && csr) {
      sel = (unsigned char*)malloc((size_t)(nblk > 0 ? nblk : 1));
      local = sel ? sparse_select(csr, h, qp, sel, nblk) : ORC_ENOMEM;
    }
    int64_t n = 0;
    if (local == ORC_OK) {
      for (int64_t t = 0; t < L; ++t) {
        if (resident > 0 && t < L - resident) continue;
        if (!orc_key_visible(t, qp, L, p->causal, p->sliding_window)) continue;
        if (csr && !sel[t / csr->sparse_block]) continue;
        toks[n++] = t;
      }
      local = head_attend(p, q, flat, b, h, toks, n, fetch, src, out + (int64_t)i * p->head_dim, lse + i);
    }
    free(toks);
    free(sel);
    if (local != ORC_OK) {
#ifdef _OPENMP
#pragma omp critical
#endif
      rc = local;
    }
  }
  return rc;
}

/* Paged f32/f16 cache.  out is [npairs][D], lse is [npairs]. */
int orc_decode_paged(const orc_params* p, const float* q, const void* k_cache, const void* v_cache,
                     int32_t kv_dtype, const int32_t* block_table, const int32_t* seq_lens,
                     const int32_t* q_pos, const int32_t* pairs, int32_t npairs, int32_t nthreads,
                     double* out, double* lse) {
  int rc = check_common(p);
  if (rc) return rc;
  if (kv_dtype != ORC_F32 && kv_dtype != ORC_F16) return ORC_EINVAL;
  for (int32_t b = 0; b < p->num_seqs; ++b) {
    if (seq_lens[b] < 0) return ORC_EINVAL;
    if ((rc = check_table(p, block_table, b, seq_lens[b]))) return rc;
  }
  paged_src src = {p, k_cache, v_cache, kv_dtype, block_table};
  return run_pairs(p, q, seq_lens, q_pos, NULL, 0, paged_fetch, &src, pairs, npairs, nthreads, out, lse);
}

/* Tiered cache: paged int8 cold history + f16 hot ring. */
int orc_decode_tiered_int8(const orc_params* p, const float* q, const uint16_t* k_hot, const uint16_t* v_hot,
                           int32_t hot_window, const uint32_t* k_cold, const uint32_t* v_cold,
                           const uint16_t* k_scale, const uint16_t* v_scale, const int32_t* cold_block_table,
                           const int32_t* seq_lens, const int32_t* cold_lens, const int32_t* q_pos,
                           const int32_t* pairs, int32_t npairs, int32_t nthreads, double* out, double* lse) {
  int rc = check_common(p);
  if (rc) return rc;
  if (p->head_dim % 4 || hot_window <= 0) return ORC_EINVAL;
  for (int32_t b = 0; b < p->num_seqs; ++b) {
    if (seq_lens[b] < 0 || cold_lens[b] < 0 || cold_lens[b] > seq_lens[b]) return ORC_EINVAL;
    if (seq_lens[b] - cold_lens[b] > hot_window) return ORC_EINVAL;
    if ((rc = check_table(p, cold_block_table, b, cold_lens[b]))) return rc;
  }
  tiered_src src = {p, k_hot, v_hot, hot_window, k_cold, v_cold, k_scale, v_scale, cold_block_table, cold_lens};
  return run_pairs(p, q, seq_lens, q_pos, NULL, 0, tiered_fetch, &src, pairs, npairs, nthreads, out, lse);
}

/* Tiered cache with an f16 cold tier: paged f16 cold history + f16 hot ring.
 * k_cold / v_cold are [num_blocks, block_size, Hkv, D] f16 bit patterns. */
int orc_decode_tiered_f16(const orc_params* p, const float* q, const uint16_t* k_hot, const uint16_t* v_hot,
                          int32_t hot_window, const uint16_t* k_cold, const uint16_t* v_cold,
                          const int32_t* cold_block_table, const int32_t* seq_lens, const int32_t* cold_lens,
                          const int32_t* q_pos, const int32_t* pairs, int32_t npairs, int32_t nthreads, double* out,
                          double* lse) {
  int rc = check_common(p);
  if (rc) return rc;
  if (hot_window <= 0) return ORC_EINVAL;
  for (int32_t b = 0; b < p->num_seqs; ++b) {
    if (seq_lens[b] < 0 || cold_lens[b] < 0 || cold_lens[b] > seq_lens[b]) return ORC_EINVAL;
    if (seq_lens[b] - cold_lens[b] > hot_window) return ORC_EINVAL;
    if ((rc = check_table(p, cold_block_table, b, cold_lens[b]))) return rc;
  }
  /* the cold words/scales fields carry the f16 rows; the scales are unused */
  tiered_src src = {p, k_hot, v_hot, hot_window, (const uint32_t*)(const void*)k_cold,
                    (const uint32_t*)(const void*)v_cold, NULL, NULL, cold_block_table, cold_lens};
  return run_pairs(p, q, seq_lens, q_pos, NULL, 0, tiered_f16_fetch, &src, pairs, npairs, nthreads, out, lse);
}

/* Sliding-window ring f16 cache: ring [B, W, Hkv, D], W = sliding_window >= 1;
 * token t of sequence b at slot t mod W, the last W tokens resident. */
int orc_decode_ring_f16(const orc_params* p, const float* q, const uint16_t* k_ring, const uint16_t* v_ring,
                        const int32_t* seq_lens, const int32_t* q_pos, const int32_t* pairs, int32_t npairs,
                        int32_t nthreads, double* out, double* lse) {
  int rc = check_common(p);
  if (rc) return rc;
  if (p->sliding_window <= 0) return ORC_EINVAL;
  for (int32_t b = 0; b < p->num_seqs; ++b)
    if (seq_lens[b] < 0) return ORC_EINVAL;
  ring_src src = {p, k_ring, v_ring, p->sliding_window};
  return run_pairs(p, q, seq_lens, q_pos, NULL, p->sliding_window, ring_fetch, &src, pairs, npairs, nthreads, out,
                   lse);
}

/* Block-sparse CSR selection over the paged f16 cache. */
int orc_decode_block_sparse(const orc_params* p, const float* q, const uint16_t* k_cache, const uint16_t* v_cache,
                            const int32_t* block_table, const int32_t* seq_lens, const int32_t* q_pos,
                            int32_t sparse_block, int32_t num_layouts, const int32_t* row_ptr, int32_t row_stride,
                            const int32_t* col_idx, int32_t col_stride, const int32_t* pairs, int32_t npairs,
                            int32_t nthreads, double* out, double* lse) {
  int rc = check_common(p);
  if (rc) return rc;
  if (sparse_block <= 0 || sparse_block % p->block_size || num_layouts <= 0 || row_stride < 2 || col_stride < 0)
    return ORC_EINVAL;
  for (int32_t b = 0; b < p->num_seqs; ++b) {
    if (seq_lens[b] < 0) return ORC_EINVAL;
    if ((rc = check_table(p, block_table, b, seq_lens[b]))) return rc;
  }
  paged_src src = {p, k_cache, v_cache, ORC_F16, block_table};
  sparse_csr csr = {sparse_block, num_layouts, row_stride, col_stride, row_ptr, col_idx};
  return run_pairs(p, q, seq_lens, q_pos, &csr, 0, paged_fetch, &src, pairs, npairs, nthreads, out, lse);
}

int orc_max_threads(void) {
#ifdef _OPENMP
  return omp_get_max_threads();
#else
  return 1;
#endif
}

/* ------------------------------------------------------- the write path */

/* f32 -> IEEE binary16 bits, rounded to nearest, ties to even, from the
 * format's definition: the value is scaled so that one unit is the f16 step
 * at its exponent (2^-24 below 2^-14, 2^(e-10) in [2^e, 2^(e+1))) and rounded
 * with rint; a carry into the next binade or past 65504 is handled
 * explicitly.  Every f32 is exact in double, so the scaling is exact. */
uint16_t orc_f32_to_f16(float f) {
  double v = (double)f;
  if (isnan(v)) return 0x7e00;
  const uint16_t sign = signbit(v) ? 0x8000 : 0;
  v = fabs(v);
  if (isinf(v)) return sign | 0x7c00;
  if (v < ldexp(1.0, -14)) {                 /* subnormal result (or zero) */
    const double r = rint(ldexp(v, 24));     /* r == 1024 is the smallest normal */
    return sign | (uint16_t)r;
  }
  int e;
  frexp(v, &e);
  e -= 1;                                    /* v in [2^e, 2^(e+1)) */
  double r = rint(ldexp(v, 10 - e));         /* in [1024, 2048] */
  if (r == 2048.0) {
    r = 1024.0;
    e += 1;
  }
  if (e > 15) return sign | 0x7c00;
  return sign | (uint16_t)((e + 15) << 10) | (uint16_t)(r - 1024.0);
}

/* One row of D f16 values -> D/4 packed words (element d is byte d % 4 of
 * word d / 4, least-significant byte first, two's complement) and its f16
 * scale, with the quantiser reading above; every step on floats is an f32
 * operation. */
void orc_quantize_row(const uint16_t* x, int32_t D, uint32_t* words, uint16_t* scale) {
  float amax = 0.0f;
  for (int32_t d = 0; d < D; ++d) {
    const float v = (float)orc_f16_to_f64(x[d]);
    if (fabsf(v) > amax) amax = fabsf(v);
  }
  const float s32 = amax / 127.0f;
  const uint16_t s16 = orc_f32_to_f16(s32);
  const float s = (float)orc_f16_to_f64(s16);
  for (int32_t w = 0; w < D / 4; ++w) words[w] = 0u;
  for (int32_t d = 0; d < D; ++d) {
    int32_t i = 0;
    if (s > 0.0f) {
      const float r = rintf((float)orc_f16_to_f64(x[d]) / s);
      i = r > 127.0f ? 127 : (r < -127.0f ? -127 : (int32_t)r);
    }
    words[d / 4] |= ((uint32_t)(uint8_t)(int8_t)i) << (8 * (d % 4));
  }
  *scale = s16;
}

/* Append one token per sequence (k_new, v_new [B][Hkv][D] f16) to the tiered
 * cache, updating seq_lens and cold_lens in place.  Returns ORC_EINVAL, with
 * nothing written, if a sequence breaks 0 <= cold_len <= seq_len,
 * seq_len - cold_len <= hot_window, or needs a cold block-table entry that is
 * out of range. */
int orc_append_tiered_int8(const orc_params* p, const uint16_t* k_new, const uint16_t* v_new, uint16_t* k_hot,
                           uint16_t* v_hot, int32_t hot_window, uint32_t* k_cold, uint32_t* v_cold,
                           uint16_t* k_scale, uint16_t* v_scale, const int32_t* cold_block_table,
                           int32_t* seq_lens, int32_t* cold_lens) {
  const int32_t B = p->num_seqs, Hkv = p->num_kv_heads, D = p->head_dim, bs = p->block_size;
  if (B < 0 || Hkv < 1 || D < 4 || D % 4 || bs < 1 || hot_window < 1 || p->max_blocks_per_seq < 1 ||
      p->num_blocks < 1)
    return ORC_EINVAL;
  for (int32_t b = 0; b < B; ++b) {
    const int64_t L = seq_lens[b], C = cold_lens[b];
    if (C < 0 || C > L || L - C > hot_window || L >= INT32_MAX) return ORC_EINVAL;
    if (L - C == hot_window) {
      if (C / bs >= p->max_blocks_per_seq) return ORC_EINVAL;
      const int32_t blk = cold_block_table[(size_t)b * p->max_blocks_per_seq + C / bs];
      if (blk < 0 || blk >= p->num_blocks) return ORC_EINVAL;
    }
  }
  for (int32_t b = 0; b < B; ++b) {
    int64_t L = seq_lens[b], C = cold_lens[b];
    if (L - C == hot_window) {               /* ring full: evict position C */
      const int64_t slot = orc_ring_slot(C, hot_window);
      const int64_t blk = cold_block_table[(size_t)b * p->max_blocks_per_seq + C / bs];
      const int64_t row = blk * bs + C % bs;
      for (int32_t g = 0; g < Hkv; ++g) {
        const size_t hot = (((size_t)b * hot_window + slot) * Hkv + g) * D;
        const size_t cold = ((size_t)row * Hkv + g);
        orc_quantize_row(k_hot + hot, D, k_cold + cold * (D / 4), k_scale + cold);
        orc_quantize_row(v_hot + hot, D, v_cold + cold * (D / 4), v_scale + cold);
      }
      C += 1;
    }
    const int64_t slot = orc_ring_slot(L, hot_window);
    for (int32_t g = 0; g < Hkv; ++g) {
      const size_t hot = (((size_t)b * hot_window + slot) * Hkv + g) * D;
      const size_t src = ((size_t)b * Hkv + g) * D;
      memcpy(k_hot + hot, k_new + src, (size_t)D * sizeof(uint16_t));
      memcpy(v_hot + hot, v_new + src, (size_t)D * sizeof(uint16_t));
    }
    seq_lens[b] = (int32_t)(L + 1);
    cold_lens[b] = (int32_t)C;
  }
  return ORC_OK;
}

/* Window-ring write path: the new token of sequence b goes to slot
 * seq_len[b] mod W (W = sliding_window), overwriting the token W positions
 * older -- the one that leaves the window -- and seq_len[b] grows by one
 * (the slot rule of doppler attention_f16kv.wgsl, get_kv_pos with the ring
 * layout).  Refuses the call, nothing written, if W < 1 or a seq_len is
 * negative. */
int orc_append_ring_f16(const orc_params* p, const uint16_t* k_new, const uint16_t* v_new, uint16_t* k_ring,
                        uint16_t* v_ring, int32_t* seq_lens) {
  const int32_t B = p->num_seqs, Hkv = p->num_kv_heads, D = p->head_dim, W = p->sliding_window;
  if (B < 0 || Hkv < 1 || D < 1 || W < 1) return ORC_EINVAL;
  for (int32_t b = 0; b < B; ++b)
    if (seq_lens[b] < 0 || seq_lens[b] >= INT32_MAX) return ORC_EINVAL;
  for (int32_t b = 0; b < B; ++b) {
    const int64_t L = seq_lens[b];
    const int64_t slot = L % W;
    for (int32_t g = 0; g < Hkv; ++g) {
      const size_t dst = (((size_t)b * W + slot) * Hkv + g) * D;
      const size_t src = ((size_t)b * Hkv + g) * D;
      memcpy(k_ring + dst, k_new + src, (size_t)D * sizeof(uint16_t));
      memcpy(v_ring + dst, v_new + src, (size_t)D * sizeof(uint16_t));
    }
    seq_lens[b] = (int32_t)(L + 1);
  }
  return ORC_OK;
}
