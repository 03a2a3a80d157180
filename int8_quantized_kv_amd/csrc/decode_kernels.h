// decode_kernels.h -- gfx950 split-KV decode attention kernels.
//
// Work decomposition ("flash decoding"): one wavefront owns one
// (sequence b, kv head, KV split) and reads each visible K/V row of its split
// exactly once for the whole GQA group of G query heads.  A workgroup holds
// `waves` such wavefronts: the kv heads blockIdx.z*waves .. +waves-1 of the same
// (sequence, split), so they share the block-table indices staged in LDS.
// Each wavefront leaves an unnormalised partial (m, l, acc[D]) per query
// head; a second kernel merges the partials of the splits with the pairwise
// rule of SparseAttention's combine_partials
// (m = max(m1, m2), d = d1 e^{m1-m} + d2 e^{m2-m}), extended to acc.
//
// Inside a wavefront, keys are processed in tiles of 16; both products of a
// tile run on the matrix cores and the VALU only unpacks, masks and exponentiates:
//   QK^T  as S^T = K . Q^T with v_mfma_f32_16x16x32_f16 (A = 16 keys x 32 dims
//         of K, B = 32 dims x 16 heads of Q^T).  Q is f32, so it enters as an
//         f16 hi/lo pair (q = hi + lo) and the two products are accumulated in
//         f32; f16 and int8 keys are exact in f16.  f32 caches use
//         v_mfma_f32_16x16x4_f32 instead.  The scores land as
//         lane l <-> head l%16, keys 4*(l/16)+e (e<4).
//   softmax online, in the log2 domain, per head (one head per lane column).
//   PV    as O = P . V with 16x16x16 products, one per 16 output dims.  The
//         score layout above is exactly the A operand (rows = heads, k = keys
//         4*(l/16)+e), so the probabilities never move between lanes.  Lane l
//         reads keys 4*(l/16)+e, dims (D/16)*(l%16) + [0, D/16) of V and
//         regroups them in registers into B operands (n-tile t = dims
//         (D/16)*c + t of column c).  f16 V uses f16 products with p as an f16
//         hi/lo pair; int8 V becomes exact bf16 integers, and the value scale
//         goes with p (p * scale as a bf16 hi/lo pair, which keeps f32 range);
//         f32 V uses v_mfma_f32_16x16x4_f32 with p as is.  The accumulator
//         holds heads 4*(l/16)+e, dims (D/16)*(l%16)+t, so a partial needs no
//         cross-lane reduction.
// Loads are 128-bit where the row allows; each K instruction reads whole
// 64-byte pieces of 16 K rows, each V instruction (D/2) contiguous bytes of
// 4 V rows per 16 lanes.
//
// Caches: paged (f16 or f32 pool through a block table), tiered (a paged int8
// or f16 cold tier below cold_lens[b], then an f16 ring), window ring (the
// tiered path with no cold tier: the last hot_window tokens), block-sparse
// (the union of the GQA group's CSR rows over the paged f16 pool).  With
// several queries per sequence the 16 score columns hold (query, head)
// pairs -- column r is query r / G, head r % G -- and each lane masks its
// column with its own query's causal / window bound.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

#include "fastdiv.h"

namespace dattn {

typedef _Float16 h8 __attribute__((ext_vector_type(8)));
typedef _Float16 h2 __attribute__((ext_vector_type(2)));
typedef float f4 __attribute__((ext_vector_type(4)));
typedef uint32_t u4 __attribute__((ext_vector_type(4)));
typedef uint32_t u2v __attribute__((ext_vector_type(2)));
typedef _Float16 h4 __attribute__((ext_vector_type(4)));
typedef short s4 __attribute__((ext_vector_type(4)));
typedef float f2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf8 __attribute__((ext_vector_type(8)));
typedef short s8v __attribute__((ext_vector_type(8)));

constexpr int kTile = 16;          // keys per tile
#ifndef DATTN_MAX_THREADS
#define DATTN_MAX_THREADS 256
#endif
#ifndef DATTN_PIPE
#define DATTN_PIPE 2
#endif
constexpr int kPipe = DATTN_PIPE;  // tile buffers: kPipe-1 tiles of loads in flight
constexpr float kSlack = 8.0f;     // lazy max: raise m only when a tile exceeds it by > 2^8
constexpr float kLn2 = 0.69314718055994531f;

// Kernel arguments (one struct for every kind; unused fields are zero).
struct DecodeArgs {
  const void* q;             // [B, H, D] (or [B, qn, H, D]) f32, or f16 when q_f16
  const void* k;             // paged pool [NB, bs, Hkv, D] (f16/f32) or cold words [NB, bs, Hkv, D/4]
  const void* v;
  const uint16_t* k_scale;   // cold scales [NB, bs, Hkv]
  const uint16_t* v_scale;
  const uint16_t* k_hot;     // hot ring [B, hw, Hkv, D]
  const uint16_t* v_hot;
  const int32_t* table;      // [B, max_blocks]
  const int32_t* seq_lens;
  const int32_t* cold_lens;
  const int32_t* q_pos;      // may be null
  const int32_t* row_ptr;    // sparse CSR
  const int32_t* col_idx;
  float* part_acc;           // [B, H, S, D] (static splits) or [slots, H, D] (balanced)
  float2* part_ml;           // [B, H, S] or [slots, H]  (m in log2 units, l)
  int32_t* sched;            // balanced: N, C, P[0..B]
  int32_t num_seqs, num_heads, num_kv_heads, max_blocks, num_splits, split_tokens;
  int32_t causal, window, hot_window;
  int32_t ring;   // 1: the ring holds only the last hot_window tokens (no cold tier)
  int32_t qn;         // queries per sequence (multi-query decode), >= 1
  int32_t grp;        // GQA group size H / Hkv
  int32_t heads_out;  // qn * num_heads: rows per slot of the partials and of out
  int32_t rbk;        // multi-query: blocks of 16 (query, head) columns per kv head, one wave each
  int32_t tile_lds;   // bytes of shared-tile buffers at the start of dynamic LDS (rbk > 1), else 0
  int32_t q_f16;      // 1: q holds f16 values (converted to f32 exactly)
  int32_t sparse_block, num_layouts, row_stride, col_stride, sparse_nblk;
  float qmul;    // scale * log2(e) without softcap, 2 log2(e) * scale / cap with softcap
  float capl2;   // cap * log2(e), 0 without softcap
  FastDiv bs, hw, sb;
};

// ----------------------------------------------------------------- helpers

template <int I, int N, class F>
__device__ __forceinline__ void static_for(F&& f) {
  if constexpr (I < N) {
    f(std::integral_constant<int, I>{});
    static_for<I + 1, N>(f);
  }
}

// Value of lane `H` of this lane's 16-lane row (DPP row_newbcast).
template <int H>
__device__ __forceinline__ float row_bcast(float x) {
  return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), 0x150 + H, 0xF,
                                                              0xF, false));
}

__device__ __forceinline__ float shfl_xor_f(float x, int m) { return __shfl_xor(x, m, 64); }

// Reductions over the four 16-lane rows (lanes l, l^16, l^32, l^48) with the
// gfx950 row swaps: v_permlane32_swap exchanges the upper half of its first
// operand with the lower half of its second, v_permlane16_swap the odd rows of
// the first with the even rows of the second, so with both operands equal to x
// the two results hold x of lane l and of its partner at distance 32 (16).
__device__ __forceinline__ void swap32(float x, float& a, float& b) {
  const auto r = __builtin_amdgcn_permlane32_swap(__builtin_bit_cast(uint32_t, x), __builtin_bit_cast(uint32_t, x),
                                                  false, false);
  a = __builtin_bit_cast(float, (uint32_t)r[0]);
  b = __builtin_bit_cast(float, (uint32_t)r[1]);
}
__device__ __forceinline__ void swap16(float x, float& a, float& b) {
  const auto r = __builtin_amdgcn_permlane16_swap(__builtin_bit_cast(uint32_t, x), __builtin_bit_cast(uint32_t, x),
                                                  false, false);
  a = __builtin_bit_cast(float, (uint32_t)r[0]);
  b = __builtin_bit_cast(float, (uint32_t)r[1]);
}
__device__ __forceinline__ float rows_max(float x) {
  float a, b;
  swap32(x, a, b);
  x = a > b ? a : b;
  swap16(x, a, b);
  return a > b ? a : b;
}
__device__ __forceinline__ float rows_sum(float x) {
  float a, b;
  swap32(x, a, b);
  x = a + b;
  swap16(x, a, b);
  return a + b;
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// Softcapped score in log2 units from y = 2 log2(e) x (x = scaled score / cap):
// cap log2(e) tanh(x) = capl2 - 2 capl2 / (2^y + 1), which saturates correctly
// at y = +-inf.
__device__ __forceinline__ float softcap_l2(float y, float capl2) {
  return __builtin_fmaf(-2.0f * capl2, __builtin_amdgcn_rcpf(fast_exp2(y) + 1.0f), capl2);
}

// Visible absolute key range [lo, hi] of sequence b (hi < lo when empty):
// causal keeps t <= q, a window W keeps t >= q-W+1 once q >= W
// (doppler is_masked), and keys exist only below seq_lens[b] -- in a window
// ring only the last hot_window of them (the ring layout's kv_start).
// With qn queries per sequence, query i sits at q0 + i (q0 = q_pos[b], or
// L - qn) and the range is the union over the queries.
__device__ __forceinline__ void visible_range(const DecodeArgs& a, int b, int& lo, int& hi, int& qpos) {
  int L = a.seq_lens[b];
  int q = a.q_pos ? a.q_pos[b] : L - a.qn;
  hi = a.causal ? min(q + a.qn - 1, L - 1) : L - 1;
  lo = (a.window > 0 && q >= a.window) ? q - a.window + 1 : 0;
  if (a.ring) lo = max(lo, L - a.hot_window);   // older tokens were overwritten
  qpos = q;
}

// int8 x 8 (two LSB-first words, two's complement) -> exact f16 x 8.
// Bias each byte by 128 (xor 0x80), place it in the low mantissa byte of
// 1024.0h (0x64xx) with one byte permute per pair, and subtract 1152:
// (1024 + i + 128) - 1152 = i exactly.  v_perm_b32 picks bytes of {S0, S1}
// (S1 = bytes 0-3, S0 = bytes 4-7); S0 = 0x64646464 supplies the 0x64 bytes.
__device__ __forceinline__ h2 i8pair_to_h2(uint32_t biased, uint32_t sel) {
  const h2 v = __builtin_bit_cast(h2, __builtin_amdgcn_perm(0x64646464u, biased, sel));
  return v - h2{(_Float16)1152.0f, (_Float16)1152.0f};
}
__device__ __forceinline__ h8 i8x8_to_h8(uint32_t w0, uint32_t w1) {
  const uint32_t x0 = w0 ^ 0x80808080u, x1 = w1 ^ 0x80808080u;
  const h2 a = i8pair_to_h2(x0, 0x04010400u);   // bytes 0, 1
  const h2 b = i8pair_to_h2(x0, 0x04030402u);   // bytes 2, 3
  const h2 c = i8pair_to_h2(x1, 0x04010400u);
  const h2 d = i8pair_to_h2(x1, 0x04030402u);
  return h8{a.x, a.y, b.x, b.y, c.x, c.y, d.x, d.y};
}

__device__ __forceinline__ float h2f(uint16_t bits) { return (float)__builtin_bit_cast(_Float16, bits); }

// p = hi + lo with hi, lo in f16 (about 22 significant bits while p stays in
// f16 range; p <= 2^8 here).
__device__ __forceinline__ void split_f16(const float (&p)[4], h4& hi, h4& lo) {
  // pairs converted at once (round to nearest even, as one at a time)
  const h2 h01 = __builtin_convertvector(f2{p[0], p[1]}, h2);
  const h2 h23 = __builtin_convertvector(f2{p[2], p[3]}, h2);
  const h2 l01 = __builtin_convertvector(f2{p[0] - (float)h01[0], p[1] - (float)h01[1]}, h2);
  const h2 l23 = __builtin_convertvector(f2{p[2] - (float)h23[0], p[3] - (float)h23[1]}, h2);
  hi = __builtin_shufflevector(h01, h23, 0, 1, 2, 3);
  lo = __builtin_shufflevector(l01, l23, 0, 1, 2, 3);
}

// Four floats rounded to bf16 (round to nearest even), as an MFMA operand.
// Whole vectors are bit-cast: this clang reads element 0 when
// __builtin_bit_cast is applied to an element of an ext_vector lvalue.
__device__ __forceinline__ s4 pack_bf16(float a, float b, float c, float d) {
  const uint32_t x = __builtin_bit_cast(uint32_t, __builtin_convertvector(f2{a, b}, bf2));
  const uint32_t y = __builtin_bit_cast(uint32_t, __builtin_convertvector(f2{c, d}, bf2));
  return __builtin_bit_cast(s4, u2v{x, y});
}
__device__ __forceinline__ float bf16_bits_to_f32(short h) {
  return __builtin_bit_cast(float, (uint32_t)(uint16_t)h << 16);
}
// q = hi + lo with hi, lo in bf16: about 16 significant bits over the whole
// f32 exponent range (q - hi is exact in f32).
__device__ __forceinline__ void split_bf16(const float (&q)[4], s4& hi, s4& lo) {
  hi = pack_bf16(q[0], q[1], q[2], q[3]);
  lo = pack_bf16(q[0] - bf16_bits_to_f32(hi[0]), q[1] - bf16_bits_to_f32(hi[1]), q[2] - bf16_bits_to_f32(hi[2]),
                 q[3] - bf16_bits_to_f32(hi[3]));
}

// Byte `byte` of w as a signed integer, converted exactly to f32 (the
// compiler selects v_cvt_f32_i32 with a sign-extended byte operand).
__device__ __forceinline__ float i8_at(uint32_t w, int byte) { return (float)(int8_t)(w >> (8 * byte)); }

// ------------------------------------------------------------ Q fragments
//
// Q is read raw at kernel start (before any K/V load, so that waiting for it
// never waits for K/V) and converted once the first K/V tiles are in flight.

// f16 MFMA path.  Slab c (32 dims of the contraction) of lane l covers 8
// dims that depend on how the keys are stored, so that every K load reads 64
// contiguous bytes of a row: f16 rows use dims 32c + 8g + [0, 8) (g = l/16);
// int8 rows, loaded 16 dims per lane, use 64(c/2) + 16g + 8(c%2) + [0, 8).
// The K fragments of a store and the Q fragments must use the same map.
template <bool I8MAP>
__device__ __forceinline__ int qdim(int c, int g) {
  return I8MAP ? 64 * (c >> 1) + 16 * g + 8 * (c & 1) : 32 * c + 8 * g;
}

// Half `i` (0: low, 1: high) of the 32-bit pattern in w, as a float.
__device__ __forceinline__ float half_at(float w, int i) {
  const uint32_t u = __builtin_bit_cast(uint32_t, w);
  return (float)__builtin_bit_cast(_Float16, (uint16_t)(i ? u >> 16 : u & 0xFFFFu));
}

template <int D>
struct QRaw16 {
  f4 x[D / 16];
};
template <int D>
struct QF16 {
  h8 hi[D / 32], lo[D / 32];
};

// Row of q (in units of D) for MFMA column j of kv head kvh.  One query per
// sequence: column j < G is head kvh*G + j.  With qn queries (MQ), column
// j < grp*qn is query j / grp, head kvh*grp + j % grp, of q [B, qn, H, D];
// the wave of row block rb holds columns 16*rb + [0, 16).  Columns beyond
// those read row 0 of the group (their Q is zeroed).
template <int G, bool MQ>
__device__ __forceinline__ size_t q_row(const DecodeArgs& a, int b, int kvh, int j) {
  if constexpr (MQ) {
    const int jj = j < a.grp * a.qn ? j : 0;
    const int i = jj / a.grp;
    return ((size_t)b * a.qn + i) * a.num_heads + (size_t)kvh * a.grp + (jj - i * a.grp);
  } else {
    return (size_t)b * a.num_heads + (size_t)kvh * G + (j < G ? j : 0);
  }
}

template <int D, int G, bool I8MAP, bool MQ = false>
__device__ __forceinline__ void load_q_raw16(const DecodeArgs& a, int b, int kvh, int lane, QRaw16<D>& r,
                                             int col0 = 0) {
  const int j = col0 + (lane & 15), g = lane >> 4;
  const size_t row = q_row<G, MQ>(a, b, kvh, j) * D;
  if (a.q_f16) {   // the 8 halves stay raw in x[2c] until convert_q
    const _Float16* qrow = (const _Float16*)a.q + row;
#pragma unroll
    for (int c = 0; c < D / 32; ++c) {
      r.x[2 * c] = __builtin_bit_cast(f4, *(const u4*)(qrow + qdim<I8MAP>(c, g)));
      r.x[2 * c + 1] = f4{0.f, 0.f, 0.f, 0.f};   // defined on both paths: keeps r in registers
    }
  } else {
    const float* qrow = (const float*)a.q + row;
#pragma unroll
    for (int c = 0; c < D / 32; ++c) {
      const int d0 = qdim<I8MAP>(c, g);
      r.x[2 * c] = *(const f4*)(qrow + d0);
      r.x[2 * c + 1] = *(const f4*)(qrow + d0 + 4);
    }
  }
}

template <int D, int G, bool MQ = false>
__device__ __forceinline__ void convert_q(const DecodeArgs& a, int lane, const QRaw16<D>& r, QF16<D>& qf,
                                          int col0 = 0) {
  const bool live = col0 + (lane & 15) < (MQ ? a.grp * a.qn : G);
#pragma unroll
  for (int c = 0; c < D / 32; ++c) {
    const f4 x0 = r.x[2 * c], x1 = r.x[2 * c + 1];
    const float f[8] = {x0.x, x0.y, x0.z, x0.w, x1.x, x1.y, x1.z, x1.w};
    const float w[4] = {x0.x, x0.y, x0.z, x0.w};   // the raw halves, two per word, when q is f16
    float x[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) x[e] = a.q_f16 ? half_at(w[e >> 1], e & 1) : f[e];
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const float v = live ? x[e] * a.qmul : 0.0f;
      const _Float16 h = (_Float16)v;
      qf.hi[c][e] = h;
      qf.lo[c][e] = (_Float16)(v - (float)h);
    }
  }
}

// Q fragments built in the int8 order, moved into the f16 order in registers
// (the tiered sweep's change from cold to hot keys).  Number the 8-dim pieces
// p = dim / 8: the int8 order puts p = 8(c/2) + 2g + c%2 in slab c of lane row
// g, the f16 order p = 4c + g.  Writing g = 2a + b and c = 2x + y, the f16
// order's (a, b, x, y) holds the int8 order's piece at row 2y + a, slab
// 2x + b: exchanging the row's low bit with the slab's low bit
// (v_permlane16_swap between slabs 2x and 2x+1), then the row's high bit with
// the slab's low bit (v_permlane32_swap) gives it.
template <int D>
__device__ __forceinline__ void q_i8_to_f16_order(QF16<D>& qf) {
  auto swaps = [](h8& lo_slab, h8& hi_slab) {
    u4 A = __builtin_bit_cast(u4, lo_slab), B = __builtin_bit_cast(u4, hi_slab);
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const auto r = __builtin_amdgcn_permlane16_swap(A[k], B[k], false, false);
      A[k] = r[0];
      B[k] = r[1];
    }
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const auto r = __builtin_amdgcn_permlane32_swap(A[k], B[k], false, false);
      A[k] = r[0];
      B[k] = r[1];
    }
    lo_slab = __builtin_bit_cast(h8, A);
    hi_slab = __builtin_bit_cast(h8, B);
  };
#pragma unroll
  for (int x = 0; x < D / 64; ++x) {
    swaps(qf.hi[2 * x], qf.hi[2 * x + 1]);
    swaps(qf.lo[2 * x], qf.lo[2 * x + 1]);
  }
}

// f32 MFMA path (16x16x4): slab c of lane l is dim 16*(c/4) + 4*(l/16) + c%4.
template <int D>
struct QRaw32 {
  f4 x[D / 16];
};
template <int D>
struct QF32 {
  float v[D / 4];
};

template <int D, int G, bool MQ = false>
__device__ __forceinline__ void load_q_raw32(const DecodeArgs& a, int b, int kvh, int lane, QRaw32<D>& r,
                                             int col0 = 0) {
  const int j = col0 + (lane & 15), g = lane >> 4;
  const size_t row = q_row<G, MQ>(a, b, kvh, j) * D;
  if (a.q_f16) {   // 4 halves raw in the low half of x[m] until convert_q
    const _Float16* qrow = (const _Float16*)a.q + row;
#pragma unroll
    for (int m = 0; m < D / 16; ++m) {
      const u2v w = *(const u2v*)(qrow + 16 * m + 4 * g);
      const uint32_t w0 = w.x, w1 = w.y;   // bit casts take whole values, not vector elements
      r.x[m] = f4{__builtin_bit_cast(float, w0), __builtin_bit_cast(float, w1), 0.0f, 0.0f};
    }
  } else {
    const float* qrow = (const float*)a.q + row;
#pragma unroll
    for (int m = 0; m < D / 16; ++m) r.x[m] = *(const f4*)(qrow + 16 * m + 4 * g);
  }
}

template <int D, int G, bool MQ = false>
__device__ __forceinline__ void convert_q(const DecodeArgs& a, int lane, const QRaw32<D>& r, QF32<D>& qf,
                                          int col0 = 0) {
  const bool live = col0 + (lane & 15) < (MQ ? a.grp * a.qn : G);
#pragma unroll
  for (int m = 0; m < D / 16; ++m) {
    const f4 y = r.x[m];   // the raw halves, two per word in .x and .y, when q is f16
    const f4 x = a.q_f16 ? f4{half_at(y.x, 0), half_at(y.x, 1), half_at(y.y, 0), half_at(y.y, 1)} : y;
    qf.v[4 * m + 0] = live ? x.x * a.qmul : 0.0f;
    qf.v[4 * m + 1] = live ? x.y * a.qmul : 0.0f;
    qf.v[4 * m + 2] = live ? x.z * a.qmul : 0.0f;
    qf.v[4 * m + 3] = live ? x.w * a.qmul : 0.0f;
  }
}

// ------------------------------------------------------- K / V fragments
//
// A tile has 16 keys.  K lane l holds key l%16 (row l%16 of the MFMA A
// operand).  V lane l holds keys 4*(l/16) + e (e < 4), dims (D/16)*(l%16) +
// [0, D/16): the k range of the lane in the B operand of the PV products, for
// the output column l%16 of every n-tile.  Every key of the tile is named by a
// physical row index r of its pool, whose kv-head rows sit at element
// (r*Hkv + kvh) * RE.

template <int D>
struct Lay {
  static constexpr int NT = D / 16;   // PV n-tiles = V dims per lane and key
};

// Per-lane constants of one wavefront.
struct LaneGeo {
  int g;      // lane / 16: keys 4g + e of the score and V layouts
  int kkey;   // lane % 16: K row of the lane, PV output column
  __device__ __forceinline__ void init(int lane) {
    g = lane >> 4;
    kkey = lane & 15;
  }
};

// Rows of one tile, for the general path (one row per key the lane touches).
struct TileRows {
  uint32_t krow;      // row of key kkey
  uint32_t srow[4];   // rows of keys 4g + e
  uint32_t xrow;      // row of key 4g + kkey%4 (whose per-token scales the lane loads)
};

template <int N>
struct WordVec {
  typedef uint32_t T __attribute__((ext_vector_type(N)));
};
template <>
struct WordVec<1> {
  typedef uint32_t T;
};
template <class T>
__device__ __forceinline__ uint32_t word_at(const T& x, int i) {
  if constexpr (std::is_same_v<T, uint32_t>)
    return x;
  else
    return x[i];
}

// K/V rows are read once per call: every load of them is nontemporal (the
// "nt" streaming policy), which measured 5-10% faster than default caching
// on every workload.
template <class T>
__device__ __forceinline__ T ntload(const void* p) {
  return __builtin_nontemporal_load((const T*)p);
}
// Loads of a contiguous tile: a wave-uniform base (SGPRs, recomputed per
// tile) plus a loop-invariant 32-bit per-lane byte offset plus an immediate,
// which is global_load's saddr form.  `tie` makes the offset a value of the
// tile (an empty asm that only names the base): otherwise the 64-bit sum of
// the pointer and the zero-extended offset is hoisted out of the loop and
// every load pays a 64-bit VALU add of the tile offset.
__device__ __forceinline__ uint32_t tie(uint32_t off, const void* base) {
  asm("" : "+v"(off) : "s"(base));
  return off;
}
template <class T>
__device__ __forceinline__ T load_at(const char* base, uint32_t off, uint32_t imm = 0) {
  return __builtin_nontemporal_load((const T*)(base + off + imm));
}
// A wave-uniform global pointer the compiler cannot re-associate with a
// per-lane offset (base + k*stride + off would otherwise become
// (base + off) + k*stride, a 64-bit VALU add per load).  It keeps the global
// address space, so that the loads stay global (not flat) loads.
typedef const __attribute__((address_space(1))) char* gptr;
__device__ __forceinline__ gptr sbase(const char* p) {
  gptr g = (gptr)p;
  asm("" : "+s"(g));
  return g;
}
template <class T>
__device__ __forceinline__ T load_at(gptr base, uint32_t off, uint32_t imm = 0) {
  return __builtin_nontemporal_load((const __attribute__((address_space(1))) T*)(base + off + imm));
}

// ---- f16 rows of D halves (paged pool or hot ring)
template <int D>
struct StoreF16 {
  static constexpr int RE = D;  // elements per kv-head row
  static constexpr int NT = Lay<D>::NT;
  static constexpr bool kScaled = false;
  static constexpr bool kPairScales = false;
  static constexpr bool kSanRows = true;   // sanitize() zeroes V rows (pv<SAN> would on every tile)
  using VW = typename WordVec<D / 32>::T;   // D/16 halves of one V row
  struct KFrag {
    u4 r[D / 32];
  };
  struct VFrag {
    VW r[4];
  };
  const _Float16* kbase;
  const _Float16* vbase;
  int Hkv, kvh;

  __device__ __forceinline__ const _Float16* krow_ptr(const _Float16* base, uint32_t row) const {
    return base + (size_t)(row * (uint32_t)Hkv + (uint32_t)kvh) * RE;
  }
  __device__ __forceinline__ void load(const TileRows& tr, const LaneGeo& lg, KFrag& k, VFrag& v) const {
    const _Float16* kr = krow_ptr(kbase, tr.krow) + 8 * lg.g;
#pragma unroll
    for (int c = 0; c < D / 32; ++c) k.r[c] = ntload<u4>(kr + 32 * c);
#pragma unroll
    for (int e = 0; e < 4; ++e) v.r[e] = ntload<VW>(krow_ptr(vbase, tr.srow[e]) + NT * lg.kkey);
  }
  // rows row0 .. row0+15: uniform base plus per-lane constant byte offsets
  __device__ __forceinline__ void load_tile(uint32_t row0, const LaneGeo& lg, KFrag& k, VFrag& v) const {
    const size_t rs = (size_t)(uint32_t)Hkv * (RE * 2);   // bytes per row of the pool
    const char* kt = (const char*)kbase + row0 * rs;
    const char* vt = (const char*)vbase + row0 * rs;
    const uint32_t ko = tie(((uint32_t)(lg.kkey * Hkv + kvh) * RE + 8 * lg.g) * 2, kt);
    const uint32_t vo = tie(((uint32_t)(4 * lg.g * Hkv + kvh) * RE + NT * lg.kkey) * 2, vt);
#pragma unroll
    for (int c = 0; c < D / 32; ++c) k.r[c] = load_at<u4>(kt, ko, 64 * c);
#pragma unroll
    for (int e = 0; e < 4; ++e) v.r[e] = load_at<VW>(sbase(vt + e * rs), vo);
  }
  template <int P = 0>
  __device__ __forceinline__ f4 scores(const KFrag& k, const QF16<D>& q) const {
    f4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int c = 0; c < D / 32; ++c) {
      h8 a = __builtin_bit_cast(h8, k.r[c]);
      acc = __builtin_amdgcn_mfma_f32_16x16x32_f16(a, q.hi[c], acc, 0, 0, 0);
      acc = __builtin_amdgcn_mfma_f32_16x16x32_f16(a, q.lo[c], acc, 0, 0, 0);
    }
    return acc;
  }
  // o[t] += P . V for n-tile t: the B operand of lane l is the halves of
  // dim (D/16)*(l%16) + t of its four keys, two keys per dword (one byte
  // permute each: low halves for even t, high halves for odd t).
  // With SAN the rows of keys outside the key range (kvalid false: p = 0,
  // contents unknown) are zeroed first, so that no Inf or NaN they may hold
  // reaches the sum.
  // V rows of keys outside the key range (kvalid false) zeroed.
  __device__ __forceinline__ void sanitize(VFrag& v, const bool (&kvalid)[4]) const {
#pragma unroll
    for (int e = 0; e < 4; ++e) v.r[e] = kvalid[e] ? v.r[e] : VW{};
  }
  // W32 (multi-query sweeps, where the matrix cores are busy): one 16x16x32
  // product per n-tile instead of two 16x16x16 ones -- k slots 8g + [0, 4)
  // carry p_hi and 8g + [4, 8) p_lo, each against the same four V values, and
  // on gfx950 the K = 32 product takes the cycles of a K = 16 one.  Measured:
  // sixteen queries per sequence 78.3 -> 75.2 us; the one-query sweeps, which
  // wait on memory, gain nothing (and the tiered cache lost 2% at W = 4096).
  template <bool SAN, int P = 0, bool W32 = false>
  __device__ __forceinline__ void pv(const KFrag&, const VFrag& v_in, const float (&p)[4], const bool (&valid)[4],
                                     f4 (&o)[NT]) const {
    VFrag v = v_in;
    if constexpr (SAN) sanitize(v, valid);
    h4 hi, lo;
    split_f16(p, hi, lo);
    const h8 a = __builtin_shufflevector(hi, lo, 0, 1, 2, 3, 4, 5, 6, 7);
#pragma unroll
    for (int t = 0; t < NT; ++t) {
      const uint32_t sel = (t & 1) ? 0x07060302u : 0x05040100u;
      const uint32_t b01 = __builtin_amdgcn_perm(word_at(v.r[1], t >> 1), word_at(v.r[0], t >> 1), sel);
      const uint32_t b23 = __builtin_amdgcn_perm(word_at(v.r[3], t >> 1), word_at(v.r[2], t >> 1), sel);
      const h4 b = __builtin_bit_cast(h4, u2v{b01, b23});
      if constexpr (W32) {
        o[t] = __builtin_amdgcn_mfma_f32_16x16x32_f16(a, __builtin_shufflevector(b, b, 0, 1, 2, 3, 0, 1, 2, 3), o[t],
                                                      0, 0, 0);
      } else {
        o[t] = __builtin_amdgcn_mfma_f32_16x16x16f16(hi, b, o[t], 0, 0, 0);
        o[t] = __builtin_amdgcn_mfma_f32_16x16x16f16(lo, b, o[t], 0, 0, 0);
      }
    }
  }
};

// ---- f32 rows (QK^T on MFMA 16x16x4 f32: slab c of lane l is dim 16*(c/4) + 4*(l/16) + c%4)
template <int D>
struct StoreF32 {
  static constexpr int RE = D;
  static constexpr int NT = Lay<D>::NT;
  static constexpr bool kScaled = false;
  static constexpr bool kPairScales = false;
  static constexpr bool kSanRows = true;
  struct KFrag {
    f4 r[D / 16];
  };
  struct VFrag {
    f4 r[4][D / 64];   // D/16 floats of each of the lane's four keys
  };
  const float* kbase;
  const float* vbase;
  int Hkv, kvh;

  __device__ __forceinline__ const float* row_ptr(const float* base, uint32_t row) const {
    return base + (size_t)(row * (uint32_t)Hkv + (uint32_t)kvh) * RE;
  }
  __device__ __forceinline__ void load(const TileRows& tr, const LaneGeo& lg, KFrag& k, VFrag& v) const {
    const float* kr = row_ptr(kbase, tr.krow);
#pragma unroll
    for (int m = 0; m < D / 16; ++m) k.r[m] = ntload<f4>(kr + 16 * m + 4 * lg.g);
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const float* vr = row_ptr(vbase, tr.srow[e]) + NT * lg.kkey;
#pragma unroll
      for (int h = 0; h < D / 64; ++h) v.r[e][h] = ntload<f4>(vr + 4 * h);
    }
  }
  __device__ __forceinline__ void load_tile(uint32_t row0, const LaneGeo& lg, KFrag& k, VFrag& v) const {
    const size_t rs = (size_t)(uint32_t)Hkv * (RE * 4);
    const char* kt = (const char*)kbase + row0 * rs;
    const char* vt = (const char*)vbase + row0 * rs;
    const uint32_t ko = tie(((uint32_t)(lg.kkey * Hkv + kvh) * RE + 4 * lg.g) * 4, kt);
    const uint32_t vo = tie(((uint32_t)(4 * lg.g * Hkv + kvh) * RE + NT * lg.kkey) * 4, vt);
#pragma unroll
    for (int m = 0; m < D / 16; ++m) k.r[m] = load_at<f4>(kt, ko, 64 * m);
#pragma unroll
    for (int e = 0; e < 4; ++e)
#pragma unroll
      for (int h = 0; h < D / 64; ++h) v.r[e][h] = load_at<f4>(sbase(vt + e * rs), vo, 16 * h);
  }
  template <int P = 0>
  __device__ __forceinline__ f4 scores(const KFrag& k, const QF32<D>& q) const {
    f4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int m = 0; m < D / 16; ++m) {
      acc = __builtin_amdgcn_mfma_f32_16x16x4f32(k.r[m].x, q.v[4 * m + 0], acc, 0, 0, 0);
      acc = __builtin_amdgcn_mfma_f32_16x16x4f32(k.r[m].y, q.v[4 * m + 1], acc, 0, 0, 0);
      acc = __builtin_amdgcn_mfma_f32_16x16x4f32(k.r[m].z, q.v[4 * m + 2], acc, 0, 0, 0);
      acc = __builtin_amdgcn_mfma_f32_16x16x4f32(k.r[m].w, q.v[4 * m + 3], acc, 0, 0, 0);
    }
    return acc;
  }
  // One 16x16x4 product per (key e, n-tile t): A = p of key 4*(l/16)+e for
  // head l%16 (k = l/16), B = that key's dim (D/16)*(l%16) + t.
  __device__ __forceinline__ void sanitize(VFrag& v, const bool (&kvalid)[4]) const {
#pragma unroll
    for (int e = 0; e < 4; ++e)
#pragma unroll
      for (int h = 0; h < D / 64; ++h) v.r[e][h] = kvalid[e] ? v.r[e][h] : f4{0.f, 0.f, 0.f, 0.f};
  }
  template <bool SAN, int P = 0, bool W32 = false>
  __device__ __forceinline__ void pv(const KFrag&, const VFrag& v_in, const float (&p)[4], const bool (&valid)[4],
                                     f4 (&o)[NT]) const {
    VFrag v = v_in;
    if constexpr (SAN) sanitize(v, valid);
#pragma unroll
    for (int e = 0; e < 4; ++e)
#pragma unroll
      for (int t = 0; t < NT; ++t)
        o[t] = __builtin_amdgcn_mfma_f32_16x16x4f32(p[e], v.r[e][t >> 2][t & 3], o[t], 0, 0, 0);
  }
};

// ---- int8 rows of D/4 words + one f16 scale per (row, kv head)
//
// Scales travel in groups: lane r of 16-lane row g holds, for r in [0, 4), the
// K scale of key 4g + r of a tile A; [4, 8) the V scale of that key; [8, 12)
// and [12, 16) the same for a tile B.  scores<P> and pv<SAN, P> take tile P's
// (0: A, 1: B) from lanes 8P + e and 8P + 4 + e of the row with a DPP row
// broadcast.  Contiguous tiles load the scales of two consecutive tiles with
// one 2-byte gather (measured: the two gathers per tile the scales used to
// cost were ~4% of the tiered kernel's time); the gather path loads tile A's
// K and V scales with one.  SCW (the host checks that the kv-head count is
// even and both scale arrays are 4-byte aligned): each lane gathers the 4-byte
// word holding its kv head's scale and its neighbour's, and keeps its half by
// the kv head's parity; measured, 2-byte gathers cost more (tiered split
// kernel 52.7 against 51.9 us).
template <int D, bool SCW = false>
struct StoreI8 {
  static constexpr int RE = D / 4;
  static constexpr int NT = Lay<D>::NT;
  static constexpr bool kScaled = true;
  static constexpr bool kPairScales = true;
  static constexpr bool kSanRows = false;   // codes are finite; pv<SAN> zeroes the scaled p instead
  using VW = typename WordVec<D / 64>::T;   // D/16 codes of one V row
  struct KFrag {
    u4 r[D / 64];
    uint16_t sc;   // this lane's entry of a scale group (above)
  };
  struct VFrag {
    VW r[4];
  };
  const uint32_t* kbase;
  const uint32_t* vbase;
  const uint16_t* ksc;
  const uint16_t* vsc;
  int Hkv, kvh;

  __device__ __forceinline__ uint32_t rk(uint32_t row) const { return row * (uint32_t)Hkv + (uint32_t)kvh; }
  __device__ __forceinline__ void load(const TileRows& tr, const LaneGeo& lg, KFrag& k, VFrag& v) const {
    const uint32_t* kr = kbase + (size_t)rk(tr.krow) * RE;
#pragma unroll
    for (int c2 = 0; c2 < D / 64; ++c2) k.r[c2] = ntload<u4>(kr + 16 * c2 + 4 * lg.g);
    k.sc = ntload<uint16_t>(((lg.kkey & 4) ? vsc : ksc) + rk(tr.xrow));   // tile A of a group
#pragma unroll
    for (int e = 0; e < 4; ++e) v.r[e] = ntload<VW>(vbase + (size_t)rk(tr.srow[e]) * RE + (NT / 4) * lg.kkey);
  }
  // K and V codes of rows row0 .. row0+15 (the scales come from load_scales)
  __device__ __forceinline__ void load_tile(uint32_t row0, const LaneGeo& lg, KFrag& k, VFrag& v) const {
    const size_t r0 = (size_t)row0 * (uint32_t)Hkv;
    const size_t rs = (size_t)(uint32_t)Hkv * (RE * 4);   // bytes per row of the pool
    const char* kt = (const char*)(kbase + r0 * RE);
    const char* vt = (const char*)(vbase + r0 * RE);
    const uint32_t ko = tie(((uint32_t)(lg.kkey * Hkv + kvh) * RE + 4 * lg.g) * 4, kt);
    const uint32_t vo = tie(((uint32_t)(4 * lg.g * Hkv + kvh) * RE + (NT / 4) * lg.kkey) * 4, vt);
#pragma unroll
    for (int c2 = 0; c2 < D / 64; ++c2) k.r[c2] = load_at<u4>(kt, ko, 64 * c2);
#pragma unroll
    for (int e = 0; e < 4; ++e) v.r[e] = load_at<VW>(sbase(vt + e * rs), vo);
  }
  // The scale group of the 16-row tiles starting at rows rowA and rowB.
  __device__ __forceinline__ void load_scales(uint32_t rowA, uint32_t rowB, const LaneGeo& lg, KFrag& k) const {
    const int r = lg.kkey;
    const size_t row = (size_t)((r & 8) ? rowB : rowA) + 4 * lg.g + (r & 3);
    const uint16_t* rs = ((r & 4) ? vsc : ksc) + row * (uint32_t)Hkv;   // the row's scales
    if constexpr (SCW) {
      const uint32_t w = ntload<uint32_t>(rs + (kvh & ~1));
      k.sc = (uint16_t)(w >> (16 * (kvh & 1)));
    } else {
      k.sc = ntload<uint16_t>(rs + kvh);
    }
  }
  template <int P = 0>
  __device__ __forceinline__ f4 scores(const KFrag& k, const QF16<D>& q) const {
    f4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int c2 = 0; c2 < D / 64; ++c2) {
      h8 a0 = i8x8_to_h8(k.r[c2].x, k.r[c2].y);
      h8 a1 = i8x8_to_h8(k.r[c2].z, k.r[c2].w);
      acc = __builtin_amdgcn_mfma_f32_16x16x32_f16(a0, q.hi[2 * c2], acc, 0, 0, 0);
      acc = __builtin_amdgcn_mfma_f32_16x16x32_f16(a0, q.lo[2 * c2], acc, 0, 0, 0);
      acc = __builtin_amdgcn_mfma_f32_16x16x32_f16(a1, q.hi[2 * c2 + 1], acc, 0, 0, 0);
      acc = __builtin_amdgcn_mfma_f32_16x16x32_f16(a1, q.lo[2 * c2 + 1], acc, 0, 0, 0);
    }
    // key scale of key 4g + e of tile P sits in lane 8P + e of the row
    const float s = h2f(k.sc);
    acc[0] *= row_bcast<8 * P + 0>(s);
    acc[1] *= row_bcast<8 * P + 1>(s);
    acc[2] *= row_bcast<8 * P + 2>(s);
    acc[3] *= row_bcast<8 * P + 3>(s);
    return acc;
  }
  // The value scale of each key goes with p (A = p * scale as a bf16 hi/lo
  // pair); B = the lane's four codes of dim (D/16)*(l%16) + t, exact in bf16.
  // With SAN, q of keys outside the key range is set to 0 (their scale may be
  // anything); codes are finite whatever the bytes.
  template <bool SAN, int P = 0, bool W32 = false>
  __device__ __forceinline__ void pv(const KFrag& k, const VFrag& v, const float (&p)[4], const bool (&valid)[4],
                                     f4 (&o)[NT]) const {
    const float s = h2f(k.sc);   // value scale of key 4g + e of tile P: lane 8P + 4 + e of the row
    float q[4] = {p[0] * row_bcast<8 * P + 4>(s), p[1] * row_bcast<8 * P + 5>(s), p[2] * row_bcast<8 * P + 6>(s),
                  p[3] * row_bcast<8 * P + 7>(s)};
    if constexpr (SAN) {
#pragma unroll
      for (int e = 0; e < 4; ++e) q[e] = valid[e] ? q[e] : 0.0f;
    }
    s4 hi, lo;
    split_bf16(q, hi, lo);
    const bf8 a = __builtin_bit_cast(bf8, __builtin_shufflevector(hi, lo, 0, 1, 2, 3, 4, 5, 6, 7));
#pragma unroll
    for (int t = 0; t < NT; ++t) {
      const int w = t >> 2, byte = t & 3;
      const s4 b = pack_bf16(i8_at(word_at(v.r[0], w), byte), i8_at(word_at(v.r[1], w), byte),
                             i8_at(word_at(v.r[2], w), byte), i8_at(word_at(v.r[3], w), byte));
      if constexpr (W32) {   // as StoreF16::pv: p_hi and p_lo in the two k halves of one K = 32 product
        const s8v bb = __builtin_shufflevector(b, b, 0, 1, 2, 3, 0, 1, 2, 3);
        o[t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, __builtin_bit_cast(bf8, bb), o[t], 0, 0, 0);
      } else {
        o[t] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(hi, b, o[t], 0, 0, 0);
        o[t] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(lo, b, o[t], 0, 0, 0);
      }
    }
  }
};

// ------------------------------------------------------- position -> row maps
//
// A map turns a position of the sweep (an absolute key, or a slot of the
// sparse union list) into a physical row and says which (position, head)
// pairs are visible.  When the map is contiguous (`contig`), every tile of 16
// positions starting at a multiple of 16 is 16 consecutive rows of one
// physical block, and `tile_row0` gives the first row of the tile, clamped
// into the tiles the sweep may touch so that it always names an allocated
// block; rows of invisible keys are then read but masked.  Otherwise `row`
// gives each key's row, clamped to a visible key.

// Paged: key t lives in block tbl[t / bs - blk0] (LDS), offset t % bs.
struct PagedMap {
  const int32_t* tbl;
  int blk0, lo, hi;        // [lo, hi]: keys this sweep may touch and see
  FastDiv bs;
  bool contig;             // bs % 16 == 0
  __device__ __forceinline__ uint32_t row(int t) const {
    t = min(max(t, lo), hi);
    const uint32_t blk = fdiv((uint32_t)t, bs);
    return (uint32_t)tbl[blk - blk0] * bs.d + ((uint32_t)t - blk * bs.d);
  }
  __device__ __forceinline__ uint32_t tile_row0(int t0) const {
    t0 = min(max(t0, lo & ~15), hi & ~15);
    const uint32_t blk = fdiv((uint32_t)t0, bs);
    const uint32_t phys = (uint32_t)__builtin_amdgcn_readfirstlane(tbl[blk - blk0]);
    return phys * bs.d + ((uint32_t)t0 - blk * bs.d);
  }
  __device__ __forceinline__ bool visible(int t, int) const { return t >= lo && t <= hi; }
  // the tile of keys [t0, t0 + 16) holds keys outside [lo, hi] (wave-uniform)
  __device__ __forceinline__ bool tile_edge(int t0) const { return t0 < lo || t0 + (kTile - 1) > hi; }
  // valid: (key t0 + 4g + e, head lane%16) takes part; kvalid: that key is
  // inside [lo, hi], so its row holds cache data (one unsigned compare each)
  __device__ __forceinline__ void tile_valid(int t0, const LaneGeo& lg, bool (&valid)[4], bool (&kvalid)[4]) const {
    const uint32_t rel = (uint32_t)(t0 + 4 * lg.g - lo), span = (uint32_t)(hi - lo);
#pragma unroll
    for (int e = 0; e < 4; ++e) kvalid[e] = valid[e] = rel + e <= span;
  }
};

// Hot ring: key t of sequence b at row b*hw + t % hw.
struct RingMap {
  int b, lo, hi;
  FastDiv hw;
  bool contig;             // hw % 16 == 0
  __device__ __forceinline__ uint32_t row(int t) const {
    t = min(max(t, lo), hi);
    return (uint32_t)b * hw.d + fmod_((uint32_t)t, hw);
  }
  __device__ __forceinline__ uint32_t tile_row0(int t0) const {
    t0 = min(max(t0, lo & ~15), hi & ~15);
    return (uint32_t)b * hw.d + fmod_((uint32_t)t0, hw);
  }
  __device__ __forceinline__ bool visible(int t, int) const { return t >= lo && t <= hi; }
  __device__ __forceinline__ bool tile_edge(int t0) const { return t0 < lo || t0 + (kTile - 1) > hi; }
  __device__ __forceinline__ void tile_valid(int t0, const LaneGeo& lg, bool (&valid)[4], bool (&kvalid)[4]) const {
    const uint32_t rel = (uint32_t)(t0 + 4 * lg.g - lo), span = (uint32_t)(hi - lo);
#pragma unroll
    for (int e = 0; e < 4; ++e) kvalid[e] = valid[e] = rel + e <= span;
  }
};

// Sparse: slot s -> union entry e = s / SB = (block << 16) | head mask (LDS),
// key t = block*SB + s % SB, then the paged map through the global table.
struct SparseMap {
  const uint32_t* list;
  const int32_t* table_row;
  int slot_end, lo, hi;
  FastDiv bs, sb;
  bool contig;             // sb % 16 == 0 and bs % 16 == 0
  uint32_t gmask;          // bits of the G heads of the group
  __device__ __forceinline__ void resolve(int slot, int& t, uint32_t& mask) const {
    const int s = min(slot, slot_end - 1);
    const uint32_t e = fdiv((uint32_t)s, sb);
    const uint32_t ent = list[e];
    t = (int)((ent >> 16) * sb.d + ((uint32_t)s - e * sb.d));
    mask = slot < slot_end ? (ent & 0xFFFFu) : 0u;
  }
  __device__ __forceinline__ uint32_t key_row(int t) const {
    t = min(max(t, lo), hi);
    const uint32_t blk = fdiv((uint32_t)t, bs);
    return (uint32_t)table_row[blk] * bs.d + ((uint32_t)t - blk * bs.d);
  }
  __device__ __forceinline__ uint32_t row(int slot) const {
    int t;
    uint32_t mk;
    resolve(slot, t, mk);
    return key_row(t);
  }
  // slots past the end fall back to the last tile; keys of a block outside
  // [lo, hi] to the tile of lo or hi, whose paged block is allocated
  __device__ __forceinline__ uint32_t tile_row0(int s0) const {
    int t;
    uint32_t mk;
    resolve(min(s0, slot_end - 16), t, mk);
    t = __builtin_amdgcn_readfirstlane(t);
    t = min(max(t, lo & ~15), hi & ~15);
    const uint32_t blk = fdiv((uint32_t)t, bs);
    const uint32_t phys = (uint32_t)__builtin_amdgcn_readfirstlane(table_row[blk]);
    return phys * bs.d + ((uint32_t)t - blk * bs.d);
  }
  __device__ __forceinline__ bool visible(int slot, int head) const {
    int t;
    uint32_t mk;
    resolve(slot, t, mk);
    return ((mk >> head) & 1u) && t >= lo && t <= hi;
  }
  __device__ __forceinline__ bool tile_edge(int) const { return true; }   // every tile is sanitized
  // A contiguous tile lies in one union entry: resolve it once.  valid adds
  // the head mask (lane%16 is the head in the score layout); kvalid is the
  // key range alone (slots past the end have no key: never valid).
  __device__ __forceinline__ void tile_valid(int s0, const LaneGeo& lg, bool (&valid)[4], bool (&kvalid)[4]) const {
    if (contig) {
      int t;
      uint32_t mk;
      resolve(s0, t, mk);
      t = __builtin_amdgcn_readfirstlane(t);
      mk = (uint32_t)__builtin_amdgcn_readfirstlane((int)mk);
      const bool head_on = (mk >> lg.kkey) & 1u;
      const bool live = s0 < slot_end;
      const uint32_t rel = (uint32_t)(t + 4 * lg.g - lo), span = (uint32_t)(hi - lo);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        kvalid[e] = live && rel + e <= span;
        valid[e] = head_on && kvalid[e];
      }
    } else {
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        valid[e] = visible(s0 + 4 * lg.g + e, lg.kkey);
        kvalid[e] = valid[e];   // rows are clamped to visible keys: only p is masked
      }
    }
  }
};

// Several queries per sequence: the lane's score column is one (query, head)
// pair, whose CSR row is its query's; the union list carries one mask bit per
// column, and the lane also masks keys outside its query's bounds [qlo, qhi].
struct SparseMapMQ : SparseMap {
  int qlo, qhi;
  __device__ __forceinline__ void tile_valid(int s0, const LaneGeo& lg, bool (&valid)[4], bool (&kvalid)[4]) const {
    if (contig) {
      int t;
      uint32_t mk;
      resolve(s0, t, mk);
      t = __builtin_amdgcn_readfirstlane(t);
      mk = (uint32_t)__builtin_amdgcn_readfirstlane((int)mk);
      const bool head_on = (mk >> lg.kkey) & 1u;
      const bool live = s0 < slot_end;
      const uint32_t rel = (uint32_t)(t + 4 * lg.g - lo), span = (uint32_t)(hi - lo);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int k = t + 4 * lg.g + e;
        kvalid[e] = live && rel + e <= span;
        valid[e] = head_on && kvalid[e] && k >= qlo && k <= qhi;
      }
    } else {
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        int t;
        uint32_t mk;
        resolve(s0 + 4 * lg.g + e, t, mk);
        valid[e] = ((mk >> lg.kkey) & 1u) && t >= lo && t <= hi && t >= qlo && t <= qhi;
        kvalid[e] = valid[e];
      }
    }
  }
};

// ------------------------------------------------- online softmax state

// Where the partial (acc[D], (m, l)) of heads kvh*G + h, h < G, goes.
struct PartialDst {
  float* acc;            // head 0's acc row
  size_t acc_hstride;    // floats between consecutive heads
  float2* ml;            // head 0's (m, l)
  size_t ml_hstride;
};

// Static splits: partials [B, H, S, D] and [B, H, S] (H -> qn*H with several
// queries per sequence; G is the GQA group, the column count of one query).
__device__ __forceinline__ PartialDst split_dst(const DecodeArgs& a, int b, int kvh, int G, int split, int D) {
  const size_t S = (size_t)a.num_splits;
  const size_t head0 = (size_t)b * a.heads_out + (size_t)kvh * G;
  return PartialDst{a.part_acc + (head0 * S + split) * D, S * D, a.part_ml + head0 * S + split, S};
}

// Balanced schedule: partials [slots, H, D] and [slots, H].
__device__ __forceinline__ PartialDst slot_dst(const DecodeArgs& a, int slot, int kvh, int G, int D) {
  const size_t head0 = (size_t)slot * a.heads_out + (size_t)kvh * G;
  return PartialDst{a.part_acc + head0 * D, (size_t)D, a.part_ml + head0, 1};
}

template <int D, int G, bool CAP>
struct Online {
  static constexpr int NT = Lay<D>::NT;
  float m;       // running max (log2 units) of head lane%16 -- equal in all rows
  float l;       // denominator part of (head lane%16, keys of row lane/16)
  float c_last;  // correction factor of the last tile (1 when m did not move)
  f4 o[NT];      // o[t][e]: PV sum of head 4*(lane/16)+e, dim NT*(lane%16)+t

  __device__ __forceinline__ void init() {
    m = -__builtin_inff();
    l = 0.f;
#pragma unroll
    for (int t = 0; t < NT; ++t) o[t] = f4{0.f, 0.f, 0.f, 0.f};
  }

  // raw: this lane's 4 scores (already multiplied by qmul and any int8 key
  // scale); valid: which of keys 4*(lane/16)+e take part.  Returns p[4] in
  // the score layout, which is the A operand of the PV products, updates m
  // and l, and says whether the accumulator must be rescaled (rescale()).
  __device__ __forceinline__ bool softmax_tile(float capl2, const f4& raw, const bool (&valid)[4], float (&p)[4]) {
    float s[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      float x = raw[e];
      if constexpr (CAP) x = softcap_l2(x, capl2);
      s[e] = valid[e] ? x : -__builtin_inff();
    }
    const float mx = rows_max(fmaxf(fmaxf(s[0], s[1]), fmaxf(s[2], s[3])));
    const float m_new = (mx > m + kSlack) ? mx : m;
    const float c = (m_new == m) ? 1.0f : fast_exp2(m - m_new);
    m = m_new;
    const float m_use = (m == -__builtin_inff()) ? 0.0f : m;
#pragma unroll
    for (int e = 0; e < 4; ++e) p[e] = fast_exp2(s[e] - m_use);
    l = l * c + ((p[0] + p[1]) + (p[2] + p[3]));
    c_last = c;
    return __builtin_amdgcn_ballot_w64(c != 1.0f) != 0;
  }

  // Rescale the accumulator after softmax_tile returned true: row 4g+e of it
  // is head 4g+e, whose factor lane 4g+e holds.
  __device__ __forceinline__ void rescale(int lane) {
    const int g = lane >> 4;
    float ce[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) ce[e] = __shfl(c_last, 4 * g + e, 64);
#pragma unroll
    for (int t = 0; t < NT; ++t)
#pragma unroll
      for (int e = 0; e < 4; ++e) o[t][e] *= ce[e];
  }

  // Write the partial of heads kvh*G + [0, G): head 4g+e's dims
  // NT*(lane%16) + [0, NT) from the lanes of row g, (m, l) from lanes h < G.
  __device__ __forceinline__ void finish(const PartialDst& dst, int lane) {
    const float lt = rows_sum(l);
    const int g = lane >> 4, c = lane & 15;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int h = 4 * g + e;
      if (h < G) {
        float* out = dst.acc + h * dst.acc_hstride + NT * c;
#pragma unroll
        for (int t4 = 0; t4 < NT / 4; ++t4)
          *(f4*)(out + 4 * t4) = f4{o[4 * t4][e], o[4 * t4 + 1][e], o[4 * t4 + 2][e], o[4 * t4 + 3][e]};
      }
    }
    if (lane < G) dst.ml[lane * dst.ml_hstride] = make_float2(m, lt);
  }
  // Several queries per sequence: column r < grp*qn is query r / grp, head
  // r % grp, stored at row (r / grp) * H + r % grp of the partials; this
  // wave holds columns col0 + [0, 16).
  __device__ __forceinline__ void finish_mq(const PartialDst& dst, int lane, int grp, int qn, int H, int col0) {
    const float lt = rows_sum(l);
    const int g = lane >> 4, c = lane & 15, ncols = grp * qn;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int r = col0 + 4 * g + e;
      if (r < ncols) {
        const int i = r / grp;
        float* out = dst.acc + (size_t)(i * H + r - i * grp) * dst.acc_hstride + NT * c;
#pragma unroll
        for (int t4 = 0; t4 < NT / 4; ++t4)
          *(f4*)(out + 4 * t4) = f4{o[4 * t4][e], o[4 * t4 + 1][e], o[4 * t4 + 2][e], o[4 * t4 + 3][e]};
      }
    }
    if (lane < 16 && col0 + lane < ncols) {
      const int r = col0 + lane, i = r / grp;
      dst.ml[(size_t)(i * H + r - i * grp) * dst.ml_hstride] = make_float2(m, lt);
    }
  }
};

template <int G>
__device__ __forceinline__ void write_empty(const PartialDst& dst, int lane) {
  if (lane < G) dst.ml[lane * dst.ml_hstride] = make_float2(-__builtin_inff(), 0.f);
}

__device__ __forceinline__ void write_empty_mq(const PartialDst& dst, int lane, int grp, int qn, int H, int col0) {
  if (lane < 16 && col0 + lane < grp * qn) {
    const int r = col0 + lane, i = r / grp;
    dst.ml[(size_t)(i * H + r - i * grp) * dst.ml_hstride] = make_float2(-__builtin_inff(), 0.f);
  }
}

// Several queries per sequence over a paged or ring map: the keys a lane's
// score column sees in a sweep over [lo, hi] are [max(lo, qlo), min(hi, qhi)],
// so key t0 + 4g + e takes part iff (unsigned)(t0 + off + e) <= span, one
// compare per key (off = 4g - the range's first key; an empty range never
// matches, as t0 + 2^30 + e stays far from 0).
template <class M>
constexpr bool kRangeMap = std::is_same_v<M, PagedMap> || std::is_same_v<M, RingMap>;
struct ColRange {
  int off;
  uint32_t span;
  __device__ __forceinline__ void init(int lo, int hi, int qlo, int qhi, int g) {
    const int vlo = max(lo, qlo), vhi = min(hi, qhi);
    off = vhi >= vlo ? 4 * g - vlo : (1 << 30);
    span = vhi >= vlo ? (uint32_t)(vhi - vlo) : 0u;
  }
  __device__ __forceinline__ void valid(int t0, bool (&v)[4]) const {
    const uint32_t x = (uint32_t)t0 + (uint32_t)off;   // modulo 2^32, as the compares expect
#pragma unroll
    for (int e = 0; e < 4; ++e) v[e] = x + (uint32_t)e <= span;
  }
};

// ------------------------------------------------------------ tile engine
//
// Sweep positions [tfirst, tend) in tiles of 16 keeping NBUF-1 tiles of loads
// in flight while one tile is computed.  Every issue in the steady state is
// unconditional (the wait-count pass would otherwise merge counter states at
// the join and wait for the prefetched tiles as well); tiles past the end load
// the last tile again (a cache hit) and are never consumed.  With FAST (a
// contiguous map) every tile is read as 16 consecutive rows from a
// wave-uniform address, rows of invisible keys included, so their V is
// zeroed before the product; otherwise each lane gathers its rows, clamped to
// visible keys.  Masking is branch-free (a branch around the accumulating
// products costs accumulator copies at the join).  The Q fragments are
// prepared after the first loads are on their way.

//
// MQ (several queries per sequence): each lane's score column belongs to one
// query, whose visible keys are [qlo, qhi]; keys outside are masked per lane.
template <int D, int G, bool CAP, int NBUF, bool FAST, bool MQ = false, class Store, class Map, class QF, class QPrep>
__device__ __forceinline__ void run_tiles(const DecodeArgs& a, const Store& st, const Map& map, QF& qf,
                                          QPrep&& prep_q, const LaneGeo& lg, Online<D, G, CAP>& on, int tfirst,
                                          int tend, int lane, int qlo = 0, int qhi = 0) {
  using KFrag = typename Store::KFrag;
  using VFrag = typename Store::VFrag;
  KFrag kb[NBUF];
  VFrag vb[NBUF];
  // Scaled rows with two buffers: slot 0 loads the scale group of its tile and
  // the next one (slot 1's); slot 1 gets a copy when slot 0 is consumed, before
  // slot 0 is refilled.
  constexpr bool PAIR = FAST && Store::kPairScales && NBUF == 2;
  ColRange cr;
  if constexpr (MQ && kRangeMap<Map>) cr.init(map.lo, map.hi, qlo, qhi, lg.g);
  auto issue = [&](int t0, auto slotc) {
    constexpr int slot = decltype(slotc)::value;
    if constexpr (FAST) {
      const uint32_t row0 = map.tile_row0(t0);
      st.load_tile(row0, lg, kb[slot], vb[slot]);
      if constexpr (PAIR) {
        if constexpr (slot == 0) st.load_scales(row0, map.tile_row0(t0 + kTile), lg, kb[0]);
      } else if constexpr (Store::kPairScales) {
        st.load_scales(row0, row0, lg, kb[slot]);
      }
    } else {
      TileRows tr;
      tr.krow = map.row(t0 + lg.kkey);
#pragma unroll
      for (int e = 0; e < 4; ++e) tr.srow[e] = map.row(t0 + 4 * lg.g + e);
      if constexpr (Store::kScaled) {
        const int x = lg.kkey & 3;
        tr.xrow = (x & 2) ? ((x & 1) ? tr.srow[3] : tr.srow[2]) : ((x & 1) ? tr.srow[1] : tr.srow[0]);
      }
      st.load(tr, lg, kb[slot], vb[slot]);
    }
  };
  auto consume = [&](int t0, auto slotc) {
    constexpr int slot = decltype(slotc)::value;
    constexpr int PS = PAIR ? slot : 0;   // which tile of the scale group
    const f4 raw = st.template scores<PS>(kb[slot], qf);
    if constexpr (PAIR) {
      if constexpr (slot == 0) kb[1].sc = kb[0].sc;
    }
    bool valid[4], kvalid[4];
    map.tile_valid(t0, lg, valid, kvalid);
    if constexpr (MQ && kRangeMap<Map>) {
      cr.valid(t0, valid);
    } else if constexpr (MQ) {
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int t = t0 + 4 * lg.g + e;
        valid[e] = valid[e] && t >= qlo && t <= qhi;
      }
    }
    float p[4];
    if (on.softmax_tile(a.capl2, raw, valid, p)) on.rescale(lane);
    if constexpr (FAST && Store::kSanRows) {
      // only a tile at the sweep's edge reads rows outside the key range
      if (map.tile_edge(t0)) st.sanitize(vb[slot], kvalid);
      st.template pv<false, PS, MQ>(kb[slot], vb[slot], p, kvalid, on.o);
    } else {
      st.template pv<FAST, PS, MQ>(kb[slot], vb[slot], p, kvalid, on.o);
    }
  };

  if (tfirst >= tend) {
    prep_q(qf);
    return;
  }
  const int ntiles = (tend - tfirst + kTile - 1) / kTile;
  static_for<0, NBUF - 1>([&](auto u) { issue(tfirst + decltype(u)::value * kTile, u); });
  prep_q(qf);
  int i = 0;
  for (; i + NBUF <= ntiles; i += NBUF) {
    static_for<0, NBUF>([&](auto u) {
      constexpr int U = decltype(u)::value;
      const int t = tfirst + (i + U) * kTile;
      issue(t + (NBUF - 1) * kTile, std::integral_constant<int, (U + NBUF - 1) % NBUF>{});
      consume(t, u);
    });
  }
  // fewer than NBUF tiles remain; their loads are already in flight
  static_for<0, NBUF - 1>([&](auto u) {
    constexpr int U = decltype(u)::value;
    if (i + U < ntiles) consume(tfirst + (i + U) * kTile, u);
  });
}

// ------------------------------------------------------------ shared tiles
//
// Multi-query decode with more than 16 (query, head) columns per kv head: the
// RBK row-block waves of a kv head sit in one workgroup and need the same
// tiles.  Fetching every tile in every wave would leave each wave's stream
// latency-bound at a quarter of the streams.  Instead wave w fetches a 1/RBK
// share of each tile (1 KB blocks j*RBK + w of 16-byte chunks) into
// registers, NS tiles ahead, and writes it into one of two LDS buffers just
// before the tile is used; after a barrier every wave reads its MFMA
// fragments from the buffer.  Each byte is fetched once per workgroup and
// each wave keeps 4-8 KB of loads in flight, as the one-query kernels do.
// A buffer holds the 16 K rows, the 16 V rows and, for int8 rows, the 16 K
// and 16 V scales; chunk c of row r sits at position r*CPR + (c ^ (r % CPR))
// (CPR chunks per row) so that the fragment reads of 16 rows fall into
// distinct banks.  Contiguous tiles only.
template <class Store>
struct ShareGeo;
template <int D>
struct ShareGeo<StoreF16<D>> {
  static constexpr int RB = 2 * D;   // bytes per row
  static constexpr bool kScaled = false;
};
template <int D, bool SCW>
struct ShareGeo<StoreI8<D, SCW>> {
  static constexpr int RB = D;
  static constexpr bool kScaled = true;
};

template <class Store, int RBK>
struct Share {
  static constexpr int RB = ShareGeo<Store>::RB;
  static constexpr bool kScaled = ShareGeo<Store>::kScaled;
  static constexpr int CPR = RB / 16;                  // 16-byte chunks per row
  static constexpr int KCH = 16 * CPR;                 // chunks of the K rows (a multiple of 64)
  static constexpr int NBLK = 2 * KCH / 64;            // 1 KB blocks per tile
  static constexpr int PER = (NBLK + RBK - 1) / RBK;   // blocks per wave
  static constexpr int NS = 2;                         // tiles of shares in flight
  static constexpr int kScaleOff = 2 * KCH * 16;
  static constexpr int kBytes = kScaleOff + (kScaled ? 64 : 0);
  struct Regs {
    u4 r[PER];
    uint16_t sc;
  };
  __device__ static __forceinline__ int pos(int row, int chunk) { return row * CPR + (chunk ^ (row & (CPR - 1))); }

  // Block j of wave wv: j*RBK + wv, wrapped into the tile's NBLK blocks (both
  // powers of two), so every load and store is unconditional: with fewer
  // blocks than waves, two waves move the same block (equal bytes to equal
  // addresses).  Likewise every lane moves one scale (lane % 32 < 16: K).
  __device__ static __forceinline__ int block(int j, int wv) { return (j * RBK + wv) & (NBLK - 1); }
  __device__ static __forceinline__ void load(const Store& st, uint32_t row0, int wv, int lane, Regs& s) {
    const uint32_t rs = (uint32_t)st.Hkv * RB;   // bytes per row of the pool
    const size_t head = (size_t)row0 * rs + (size_t)st.kvh * RB;
    const char* kt = (const char*)st.kbase + head;
    const char* vt = (const char*)st.vbase + head;
#pragma unroll
    for (int j = 0; j < PER; ++j) {
      const int blk = block(j, wv);
      const int q = (blk & (NBLK / 2 - 1)) * 64 + lane;   // chunk within the K (or V) rows
      const int row = q / CPR, c = (q & (CPR - 1)) ^ (row & (CPR - 1));
      const char* base = blk >= NBLK / 2 ? vt : kt;
      s.r[j] = load_at<u4>(base, tie((uint32_t)row * rs + 16u * (uint32_t)c, base));
    }
    if constexpr (kScaled) {
      const uint16_t* sc = (lane & 16) ? st.vsc : st.ksc;
      s.sc = ntload<uint16_t>(sc + ((size_t)row0 + (lane & 15)) * (uint32_t)st.Hkv + st.kvh);
    }
  }
  __device__ static __forceinline__ void store(const Regs& s, int wv, int lane, char* buf) {
#pragma unroll
    for (int j = 0; j < PER; ++j) *(u4*)(buf + 16 * (block(j, wv) * 64 + lane)) = s.r[j];
    if constexpr (kScaled) *(uint16_t*)(buf + kScaleOff + 2 * (lane & 31)) = s.sc;
  }
  // the fragments Store::load_tile would have loaded
  __device__ static __forceinline__ void read(const char* buf, const LaneGeo& lg, typename Store::KFrag& k,
                                              typename Store::VFrag& v) {
    constexpr int KQ = RB / 64;   // 16-byte K pieces per lane
#pragma unroll
    for (int c = 0; c < KQ; ++c) k.r[c] = *(const u4*)(buf + 16 * pos(lg.kkey, lg.g + 4 * c));
    using VW = std::remove_reference_t<decltype(v.r[0])>;
    constexpr int VB = sizeof(VW);   // V bytes per lane and key
    const int vbyte = VB * lg.kkey;
#pragma unroll
    for (int e = 0; e < 4; ++e)
      v.r[e] = *(const VW*)(buf + 16 * (KCH + pos(4 * lg.g + e, vbyte / 16)) + (vbyte & 15));
    if constexpr (kScaled) {   // tile A of a scale group: K scales, then V scales at +32 bytes
      const int key = 4 * lg.g + (lg.kkey & 3);
      k.sc = *(const uint16_t*)(buf + kScaleOff + ((lg.kkey & 4) ? 32 : 0) + 2 * key);
    }
  }
};

// The sweep of run_tiles (contiguous tiles, several queries) through shared
// tiles; ring holds two buffers of Share::kBytes.  Every wave of the
// workgroup calls it with the same range: each tile costs one barrier.
template <int D, int G, bool CAP, int RBK, class Store, class Map, class QF, class QPrep>
__device__ __forceinline__ void run_tiles_shared(const DecodeArgs& a, const Store& st, const Map& map, QF& qf,
                                                 QPrep&& prep_q, const LaneGeo& lg, Online<D, G, CAP>& on,
                                                 int tfirst, int tend, int lane, int qlo, int qhi, int wv,
                                                 char* ring) {
  using SH = Share<Store, RBK>;
  constexpr int NS = SH::NS;
  typename SH::Regs sh[NS];
  ColRange cr;
  if constexpr (kRangeMap<Map>) cr.init(map.lo, map.hi, qlo, qhi, lg.g);
  auto issue = [&](int t0, auto slotc) { SH::load(st, map.tile_row0(t0), wv, lane, sh[decltype(slotc)::value]); };
  auto consume = [&](int t0, int i, auto slotc) {
    constexpr int slot = decltype(slotc)::value;
    char* buf = ring + (i & 1) * SH::kBytes;
    SH::store(sh[slot], wv, lane, buf);   // the other waves left this buffer two barriers ago
    issue(t0 + NS * kTile, slotc);
    __syncthreads();
    typename Store::KFrag kf;
    typename Store::VFrag vf;
    SH::read(buf, lg, kf, vf);
    const f4 raw = st.scores(kf, qf);
    bool valid[4], kvalid[4];
    map.tile_valid(t0, lg, valid, kvalid);
    if constexpr (kRangeMap<Map>) {
      cr.valid(t0, valid);
    } else {
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int t = t0 + 4 * lg.g + e;
        valid[e] = valid[e] && t >= qlo && t <= qhi;
      }
    }
    float p[4];
    if (on.softmax_tile(a.capl2, raw, valid, p)) on.rescale(lane);
    if constexpr (Store::kSanRows) {
      if (map.tile_edge(t0)) st.sanitize(vf, kvalid);
      st.template pv<false, 0, true>(kf, vf, p, kvalid, on.o);
    } else {
      st.template pv<true, 0, true>(kf, vf, p, kvalid, on.o);
    }
  };

  if (tfirst >= tend) {
    prep_q(qf);
    return;
  }
  const int ntiles = (tend - tfirst + kTile - 1) / kTile;
  static_for<0, NS>([&](auto u) { issue(tfirst + decltype(u)::value * kTile, u); });
  prep_q(qf);
  int i = 0;
  for (; i + NS <= ntiles; i += NS) {
    static_for<0, NS>([&](auto u) {
      constexpr int U = decltype(u)::value;
      consume(tfirst + (i + U) * kTile, i + U, u);
    });
  }
  static_for<0, NS - 1>([&](auto u) {
    constexpr int U = decltype(u)::value;
    if (i + U < ntiles) consume(tfirst + (i + U) * kTile, i + U, u);
  });
  __syncthreads();   // every wave is done with the buffers
}

// One sweep of a segment: through shared tiles by the RBK row-block waves of
// the kv head (RBK > 1: multi-query kernels built for contiguous tiles, with
// 2 * Share::kBytes of LDS at the start of dynamic LDS), else each wave on
// its own.
template <int D, int G, bool CAP, bool FM, bool MQ, int RBK, class Store, class Map, class QF, class QPrep>
__device__ __forceinline__ void sweep(const DecodeArgs& a, const Store& st, const Map& map, QF& qf, QPrep&& prep_q,
                                      const LaneGeo& lg, Online<D, G, CAP>& on, int tfirst, int tend, int lane,
                                      int qlo, int qhi, int col0, char* ring) {
  if constexpr (RBK > 1) {
    static_assert(MQ && FM, "shared tiles are built for contiguous multi-query sweeps");
    const int wv = __builtin_amdgcn_readfirstlane((col0 >> 4) & (RBK - 1));   // row block of this wave
    run_tiles_shared<D, G, CAP, RBK>(a, st, map, qf, prep_q, lg, on, tfirst, tend, lane, qlo, qhi, wv, ring);
  } else {
    run_tiles<D, G, CAP, kPipe, FM, MQ>(a, st, map, qf, prep_q, lg, on, tfirst, tend, lane, qlo, qhi);
  }
}

// ---------------------------------------------------------------- kernels
//
// FM (chosen by the host): every cache the kernel sweeps is contiguous in
// 16-row tiles -- paged block size, hot-ring size and sparse block all
// multiples of 16 -- so tiles are read with uniform-base loads.  Kernels are
// instantiated once per FM value instead of branching at run time: holding
// both sweep loops in one function costs the register allocator dozens of
// VGPRs.

// Stage block-table entries [blk0, blk0 + n) of sequence b into LDS, once
// every wave of the workgroup is done with the previous contents.
__device__ __forceinline__ void stage_table(const DecodeArgs& a, int b, int blk0, int n, int32_t* lds) {
  __syncthreads();
  const int32_t* src = a.table + (size_t)b * a.max_blocks + blk0;
  for (int i = threadIdx.x; i < n; i += blockDim.x) lds[i] = src[i];
  __syncthreads();
}

// Blocks holding keys [t0, t1).
__device__ __forceinline__ void table_span(const DecodeArgs& a, int t0, int t1, int& blk0, int& n) {
  blk0 = 0;
  n = 0;
  if (t0 < t1) {
    blk0 = (int)fdiv((uint32_t)t0, a.bs);
    n = (int)fdiv((uint32_t)(t1 - 1), a.bs) - blk0 + 1;
  }
}

// Several queries per sequence: the visible keys [qlo, qhi] of the query whose
// (query, head) pair is this lane's score column (column r = col0 + lane % 16:
// query r / grp); an unused column (r >= grp * qn) sees nothing.
__device__ __forceinline__ void query_bounds(const DecodeArgs& a, int b, int lane, int col0, int& qlo, int& qhi) {
  const int L = a.seq_lens[b];
  const int c = col0 + (lane & 15);
  const int q = (a.q_pos ? a.q_pos[b] : L - a.qn) + c / a.grp;
  qhi = a.causal ? min(q, L - 1) : L - 1;
  qlo = (a.window > 0 && q >= a.window) ? q - a.window + 1 : 0;
  if (c >= a.grp * a.qn) qlo = qhi + 1;
}

// Sweep keys [tb, te) of sequence b for one kv head of a paged cache and write
// the partial to dst.  Every wave of the workgroup calls it with the same
// (b, tb, te): the block-table staging is shared.  MQ: several queries per
// sequence (G = 16 columns, a.grp * a.qn of them used); the lane's query
// bounds [qlo, qhi] mask its column.
template <int D, int G, bool CAP, class T, bool FM, bool MQ = false, int RBK = 1>
__device__ __forceinline__ void paged_segment(const DecodeArgs& a, int b, int kvh, int lane, int tb, int te,
                                              int32_t* lds_tbl, const PartialDst& dst, int col0 = 0,
                                              char* ring = nullptr) {
  using QRaw = std::conditional_t<std::is_same_v<T, float>, QRaw32<D>, QRaw16<D>>;
  QRaw qraw;
  if (tb < te) {
    if constexpr (std::is_same_v<T, float>)
      load_q_raw32<D, G, MQ>(a, b, kvh, lane, qraw, col0);
    else
      load_q_raw16<D, G, false, MQ>(a, b, kvh, lane, qraw, col0);
  }
  int blk0, nblk;
  table_span(a, tb, te, blk0, nblk);
  stage_table(a, b, blk0, nblk, lds_tbl);
  if (tb >= te) {
    if constexpr (MQ)
      write_empty_mq(dst, lane, a.grp, a.qn, a.num_heads, col0);
    else
      write_empty<G>(dst, lane);
    return;
  }
  int qlo = 0, qhi = 0;
  if constexpr (MQ) query_bounds(a, b, lane, col0, qlo, qhi);
  LaneGeo lg;
  lg.init(lane);
  PagedMap map{lds_tbl, blk0, tb, te - 1, a.bs, FM};
  Online<D, G, CAP> on;
  on.init();
  if constexpr (std::is_same_v<T, float>) {
    QF32<D> qf;
    StoreF32<D> st{(const float*)a.k, (const float*)a.v, a.num_kv_heads, kvh};
    run_tiles<D, G, CAP, kPipe, FM, MQ>(a, st, map, qf, [&](QF32<D>& q) { convert_q<D, G, MQ>(a, lane, qraw, q, col0); },
                                        lg, on, tb & ~(kTile - 1), te, lane, qlo, qhi);
  } else {
    QF16<D> qf;
    StoreF16<D> st{(const _Float16*)a.k, (const _Float16*)a.v, a.num_kv_heads, kvh};
    sweep<D, G, CAP, FM, MQ, RBK>(a, st, map, qf, [&](QF16<D>& q) { convert_q<D, G, MQ>(a, lane, qraw, q, col0); }, lg,
                             on, tb & ~(kTile - 1), te, lane, qlo, qhi, col0, ring);
  }
  if constexpr (MQ)
    on.finish_mq(dst, lane, a.grp, a.qn, a.num_heads, col0);
  else
    on.finish(dst, lane);
}

// The same for the tiered cache: keys below cold_lens[b] from the paged cold
// pool (int8 words with f16 scales, or f16 rows when CF16), the rest from the
// f16 ring.
// C: cold_lens[b] (0 for the window ring, which has no cold tier).  SCW: the
// int8 scales are gathered as 4-byte words (StoreI8).
template <int D, int G, bool CAP, bool FM, bool CF16, bool MQ = false, int RBK = 1, bool SCW = false>
__device__ __forceinline__ void tiered_segment(const DecodeArgs& a, int b, int kvh, int lane, int tb, int te, int C,
                                               int32_t* lds_tbl, const PartialDst& dst, int col0 = 0,
                                               char* ring = nullptr) {
  const int ce = min(te, C);   // cold part [tb, ce)
  const int hb = max(tb, C);   // hot part  [hb, te)
  QRaw16<D> qraw;              // int8 cold keys use the int8 dim map, f16 keys the f16 one
  if (tb < ce)
    load_q_raw16<D, G, !CF16, MQ>(a, b, kvh, lane, qraw, col0);
  else if (tb < te)
    load_q_raw16<D, G, false, MQ>(a, b, kvh, lane, qraw, col0);
  int blk0, nblk;
  table_span(a, tb, ce, blk0, nblk);
  stage_table(a, b, blk0, nblk, lds_tbl);
  if (tb >= te) {
    if constexpr (MQ)
      write_empty_mq(dst, lane, a.grp, a.qn, a.num_heads, col0);
    else
      write_empty<G>(dst, lane);
    return;
  }
  int qlo = 0, qhi = 0;
  if constexpr (MQ) query_bounds(a, b, lane, col0, qlo, qhi);
  LaneGeo lg;
  lg.init(lane);
  QF16<D> qf;
  Online<D, G, CAP> on;
  on.init();
  if (tb < ce) {
    PagedMap map{lds_tbl, blk0, tb, ce - 1, a.bs, FM};
    if constexpr (CF16) {
      StoreF16<D> st{(const _Float16*)a.k, (const _Float16*)a.v, a.num_kv_heads, kvh};
      sweep<D, G, CAP, FM, MQ, RBK>(a, st, map, qf, [&](QF16<D>& q) { convert_q<D, G, MQ>(a, lane, qraw, q, col0); },
                               lg, on, tb & ~(kTile - 1), ce, lane, qlo, qhi, col0, ring);
    } else {
      StoreI8<D, SCW> st{(const uint32_t*)a.k, (const uint32_t*)a.v, a.k_scale, a.v_scale, a.num_kv_heads, kvh};
      sweep<D, G, CAP, FM, MQ, RBK>(a, st, map, qf, [&](QF16<D>& q) { convert_q<D, G, MQ>(a, lane, qraw, q, col0); },
                               lg, on, tb & ~(kTile - 1), ce, lane, qlo, qhi, col0, ring);
    }
  } else {
    // no cold keys: Q in the f16 order now, so that the raw Q is dead in both sweeps
    convert_q<D, G, MQ>(a, lane, qraw, qf, col0);
  }
  if (hb < te) {
    RingMap map{b, hb, te - 1, a.hw, FM};
    StoreF16<D> st{(const _Float16*)a.k_hot, (const _Float16*)a.v_hot, a.num_kv_heads, kvh};
    const bool had_cold = !CF16 && tb < ce;   // Q was converted in the int8 order
    sweep<D, G, CAP, FM, MQ, RBK>(a, st, map, qf,
                             [&](QF16<D>& q) {
                               if (had_cold) q_i8_to_f16_order<D>(q);
                             },
                             lg, on, hb & ~(kTile - 1), te, lane, qlo, qhi, col0, ring);
  }
  if constexpr (MQ)
    on.finish_mq(dst, lane, a.grp, a.qn, a.num_heads, col0);
  else
    on.finish(dst, lane);
}

// The wave's kv head and first score column.  One query per sequence: wave v
// of workgroup z is kv head z*waves + v.  Several queries (MQ): the (kv head,
// row block) pairs are numbered kv-head-major, a.rbk row blocks of 16
// columns per kv head, so the row blocks of a kv head sit in one workgroup
// and sweep the same keys side by side.
template <bool MQ>
__device__ __forceinline__ void wave_head(const DecodeArgs& a, int& kvh, int& col0) {
  const int v = blockIdx.z * (blockDim.x >> 6) + (threadIdx.x >> 6);
  if constexpr (MQ) {
    kvh = v / a.rbk;
    col0 = 16 * (v - kvh * a.rbk);
  } else {
    kvh = v;
    col0 = 0;
  }
}

// Multi-query workgroups hold up to 8 row-block waves of one kv head.
#define DATTN_BOUNDS(MQ) __launch_bounds__((MQ) ? 2 * DATTN_MAX_THREADS : DATTN_MAX_THREADS)

// Static splits: workgroup (split, b, z) sweeps keys [split*T, (split+1)*T)
// of sequence b for its waves' kv heads.
template <int D, int G, bool CAP, class T, bool FM, bool MQ = false, int RBK = 1>
__global__ DATTN_BOUNDS(MQ) __attribute__((amdgpu_waves_per_eu(2))) void paged_split_kernel(DecodeArgs a) {
  extern __shared__ int32_t lds_all[];
  int32_t* lds_tbl = MQ ? lds_all + a.tile_lds / 4 : lds_all;
  const int split = blockIdx.x, b = blockIdx.y;
  const int lane = threadIdx.x & 63;
  int kvh, col0;
  wave_head<MQ>(a, kvh, col0);
  int lo, hi, qp;
  visible_range(a, b, lo, hi, qp);
  const int tb = max(split * a.split_tokens, lo);
  const int te = min((split + 1) * a.split_tokens, hi + 1);
  paged_segment<D, G, CAP, T, FM, MQ, RBK>(a, b, kvh, lane, tb, te, lds_tbl,
                                      split_dst(a, b, kvh, MQ ? a.grp : G, split, D), col0, (char*)lds_all);
}

template <int D, int G, bool CAP, bool FM, bool CF16, bool MQ = false, int RBK = 1, bool SCW = false>
__global__ DATTN_BOUNDS(MQ) __attribute__((amdgpu_waves_per_eu(2))) void tiered_split_kernel(DecodeArgs a) {
  extern __shared__ int32_t lds_all[];
  int32_t* lds_tbl = MQ ? lds_all + a.tile_lds / 4 : lds_all;
  const int split = blockIdx.x, b = blockIdx.y;
  const int lane = threadIdx.x & 63;
  int kvh, col0;
  wave_head<MQ>(a, kvh, col0);
  int lo, hi, qp;
  visible_range(a, b, lo, hi, qp);
  const int tb = max(split * a.split_tokens, lo);
  const int te = min((split + 1) * a.split_tokens, hi + 1);
  tiered_segment<D, G, CAP, FM, CF16, MQ, RBK, SCW>(a, b, kvh, lane, tb, te, a.cold_lens ? a.cold_lens[b] : 0, lds_tbl,
                                          split_dst(a, b, kvh, MQ ? a.grp : G, split, D), col0, (char*)lds_all);
}

// ------------------------------------------------------- balanced schedule
//
// The visible keys of sequence b are cut into 16-key tiles aligned to
// absolute positions.  Each tile costs units in proportion to the bytes it
// reads: 1 for a paged tile or an int8 cold tile, 2 for an f16 hot-ring tile
// of the int8 tiered cache (16 rows of 2*D halves against 16 rows of 2*D
// bytes); every tile of the f16 tiered cache costs 1, as in the paged cache;
// each sequence adds a fixed start-up cost.
// b owns units [P[b], P[b+1]) of the concatenation over all sequences (N
// units in all).  Worker w of a kv-head group (blockIdx.x) owns units
// [w*C, min((w+1)*C, N)) with C = ceil(N / gridDim.x) and sweeps the tiles
// whose first unit lies there, so every worker streams about the same number
// of bytes whatever the length mix, and the grid is one round of resident
// workgroups.  A worker's range can cross sequence boundaries; its piece of
// sequence b (possibly empty, when its range lies inside one hot tile) is
// partial slot w + b, which no other (worker, sequence) pair shares because
// each boundary along the concatenation advances w, b or both.  Worker 0 of
// group 0 leaves N, C and P in the schedule area of the workspace for the
// combine kernel.

// Tiles of sequence b and the unit cost of each.  A sequence with visible
// keys also costs kSeqUnits up front, the start-up of a segment (table
// staging, Q, the first dependent loads), so that a worker which starts a
// second sequence is given fewer tiles.
#ifndef DATTN_SEQ_UNITS
#define DATTN_SEQ_UNITS 4
#endif
constexpr int kSeqUnits = DATTN_SEQ_UNITS;
// A sequence of the int8 tiered cache whose visible keys reach both tiers
// also costs kTransUnits between its last cold tile and its first hot tile:
// the worker that crosses the boundary drains its load pipeline, reloads Q
// in the f16 dims order and refills the pipeline from the ring.
#ifndef DATTN_TRANS_UNITS
#define DATTN_TRANS_UNITS 2
#endif
constexpr int kTransUnits = DATTN_TRANS_UNITS;

// KIND 2 and 8: tiered int8 (8 gathers the scales as words); 6: the same with
// several queries per sequence.
constexpr bool kind_i8(int K) { return K == 2 || K == 6 || K == 8; }
constexpr bool kind_mq(int K) { return K >= 4 && K <= 7; }

template <int KIND>
struct SeqCost {
  int lo, hi, base;   // visible keys [lo, hi]; tile i starts at key base + 16i
  int ntiles, ncold;  // tiles < ncold cost 1 unit, the others 2 (int8 tiered only)
  int head;           // start-up units (0 for a sequence with no visible key)
  int trans;          // units between the cold and the hot tiles (int8 tiered only)
  int cold;           // cold_lens[b] for the tiered kinds (0 without a cold tier), else 0
  static constexpr bool kTiered = kind_i8(KIND) || KIND == 3 || KIND == 7;
  __device__ __forceinline__ void init(const DecodeArgs& a, int b) {
    int q, l, h;
    visible_range(a, b, l, h, q);
    init_vals(l, h, kTiered && a.cold_lens ? a.cold_lens[b] : 0);
  }
  __device__ __forceinline__ void init_vals(int l, int h, int c) {
    lo = l;
    hi = h;
    cold = c;
    base = lo & ~(kTile - 1);
    ntiles = hi < lo ? 0 : (hi >> 4) - (lo >> 4) + 1;
    ncold = ntiles;
    if constexpr (kind_i8(KIND)) ncold = min(ntiles, max(0, (cold - base + kTile - 1) / kTile));
    head = ntiles > 0 ? kSeqUnits : 0;
    trans = kind_i8(KIND) && ncold > 0 && ntiles > ncold ? kTransUnits : 0;
  }
  __device__ __forceinline__ int units() const { return head + ncold + trans + 2 * (ntiles - ncold); }
  // first tile whose first unit is >= u (0 <= u <= units())
  __device__ __forceinline__ int tile_at(int u) const {
    u = max(u - head, 0);
    return u <= ncold ? u : ncold + max(0, u - ncold - trans + 1) / 2;
  }
};

// Batches of at most kStashSeqs sequences keep each sequence's visible range
// and cold length in LDS (three arrays of stash_stride(B) entries after P), so
// that a worker starting a sequence does not read them from memory again: one
// dependent round trip less before its first tiles.
constexpr int kStashSeqs = 256;
__host__ __device__ constexpr int stash_stride(int B) { return B <= kStashSeqs ? (B + 3) & ~3 : 0; }
__host__ __device__ constexpr int prefix_stride(int B) { return (B + 4) & ~3; }

// P[0..B] (exclusive prefix of unit counts) into LDS, and the stash when B is
// small enough; returns N = P[B].
template <int KIND>
__device__ __forceinline__ int unit_prefix(const DecodeArgs& a, int32_t* P) {
  const int B = a.num_seqs;
  const int ss = stash_stride(B);
  int32_t* stash = P + prefix_stride(B);
  if (threadIdx.x < 64) {
    const int lane = threadIdx.x;
    int run = 0;
    for (int base = 0; base < B; base += 64) {
      const int b = base + lane;
      int c = 0;
      if (b < B) {
        SeqCost<KIND> sc;
        sc.init(a, b);
        c = sc.units();
        if (ss) {
          stash[b] = sc.lo;
          stash[ss + b] = sc.hi;
          stash[2 * ss + b] = sc.cold;
        }
      }
      int x = c;
#pragma unroll
      for (int o = 1; o < 64; o <<= 1) {
        const int y = __shfl_up(x, o, 64);
        if (lane >= o) x += y;
      }
      if (b < B) P[b] = run + x - c;
      run += __shfl(x, 63, 64);
    }
    if (lane == 0) P[B] = run;
  }
  __syncthreads();
  return P[B];
}

// KIND: 0 paged f16, 1 paged f32, 2 tiered int8, 3 tiered f16 (and the window
// ring); 4, 5, 6, 7: paged f16, paged f32, tiered int8, tiered f16 with
// several queries per sequence (G = 16 columns per wave, a.rbk waves per kv
// head).  Registers are capped for two
// waves per SIMD: measured, a third wave (with Q moved to LDS to make room)
// and a third tile of loads in flight per wave are both slower -- about
// 32 KiB of loads in flight per SIMD is what HBM rewards here.
template <int D, int G, bool CAP, int KIND, bool FM, int RBK = 1>
__global__ DATTN_BOUNDS(kind_mq(KIND)) __attribute__((amdgpu_waves_per_eu(2)))
void balanced_kernel(DecodeArgs a) {
  extern __shared__ int32_t lds_all[];
  int32_t* lds = kind_mq(KIND) ? lds_all + a.tile_lds / 4 : lds_all;
  char* ring = (char*)lds_all;
  const int B = a.num_seqs;
  int32_t* P = lds;
  const int ss = stash_stride(B);
  const int32_t* stash = lds + prefix_stride(B);
  int32_t* tbl = lds + prefix_stride(B) + 3 * ss;
  const int w = blockIdx.x, nw = gridDim.x;
  const int lane = threadIdx.x & 63;
  int kvh, col0;
  wave_head<kind_mq(KIND)>(a, kvh, col0);
  const int N = unit_prefix<KIND>(a, P);
  const int C = (N + nw - 1) / nw;
  if (w == 0 && blockIdx.z == 0) {
    for (int i = threadIdx.x; i <= B; i += blockDim.x) a.sched[2 + i] = P[i];
    if (threadIdx.x == 0) {
      a.sched[0] = N;
      a.sched[1] = C;
    }
  }
  int x0 = w * C;
  const int x1 = min(x0 + C, N);
  if (x0 >= x1) return;
  int b = 0, top = B - 1;   // last b with P[b] <= x0
  while (b < top) {
    const int mid = (b + top + 1) >> 1;
    if (P[mid] <= x0)
      b = mid;
    else
      top = mid - 1;
  }
  while (x0 < x1) {
    while (P[b + 1] <= x0) ++b;
    const int seg_end = min(x1, P[b + 1]);
    SeqCost<KIND> sc;
    if (ss)
      sc.init_vals(stash[b], stash[ss + b], stash[2 * ss + b]);
    else
      sc.init(a, b);
    const int tb = max(sc.lo, sc.base + kTile * sc.tile_at(x0 - P[b]));
    const int te = min(sc.hi + 1, sc.base + kTile * sc.tile_at(seg_end - P[b]));
    const PartialDst dst = slot_dst(a, w + b, kvh, kind_mq(KIND) ? a.grp : G, D);
    if constexpr (KIND == 2)
      tiered_segment<D, G, CAP, FM, false>(a, b, kvh, lane, tb, te, sc.cold, tbl, dst);
    else if constexpr (KIND == 8)
      tiered_segment<D, G, CAP, FM, false, false, 1, true>(a, b, kvh, lane, tb, te, sc.cold, tbl, dst);
    else if constexpr (KIND == 3)
      tiered_segment<D, G, CAP, FM, true>(a, b, kvh, lane, tb, te, sc.cold, tbl, dst);
    else if constexpr (KIND == 1)
      paged_segment<D, G, CAP, float, FM>(a, b, kvh, lane, tb, te, tbl, dst);
    else if constexpr (KIND == 4)
      paged_segment<D, G, CAP, _Float16, FM, true, RBK>(a, b, kvh, lane, tb, te, tbl, dst, col0, ring);
    else if constexpr (KIND == 5)
      paged_segment<D, G, CAP, float, FM, true>(a, b, kvh, lane, tb, te, tbl, dst, col0, ring);
    else if constexpr (KIND == 6)
      tiered_segment<D, G, CAP, FM, false, true, RBK>(a, b, kvh, lane, tb, te, sc.cold, tbl, dst, col0, ring);
    else if constexpr (KIND == 7)
      tiered_segment<D, G, CAP, FM, true, true, RBK>(a, b, kvh, lane, tb, te, sc.cold, tbl, dst, col0, ring);
    else
      paged_segment<D, G, CAP, _Float16, FM>(a, b, kvh, lane, tb, te, tbl, dst);
    x0 = seg_end;
    ++b;
  }
}

// Block-sparse: each wave builds the union of the CSR rows of its G heads in
// LDS (a G-bit head mask per sparse block, then the blocks with a non-zero
// mask compacted in increasing order), takes the slice of that list its
// split owns and sweeps its keys.
template <int D, int G, bool CAP, bool FM, bool MQ = false>
__global__ DATTN_BOUNDS(MQ) __attribute__((amdgpu_waves_per_eu(2))) void sparse_split_kernel(DecodeArgs a) {
  extern __shared__ uint32_t lds_sp[];
  const int split = blockIdx.x, b = blockIdx.y;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  int kvh, col0;   // several queries: each wave builds the union of its own 16 columns
  wave_head<MQ>(a, kvh, col0);
  const int nb = a.sparse_nblk;
  uint32_t* mask = lds_sp + (size_t)wave * 2 * nb;
  uint32_t* list = mask + nb;
  int lo, hi, qp;
  visible_range(a, b, lo, hi, qp);
  QRaw16<D> qraw;
  load_q_raw16<D, G, false, MQ>(a, b, kvh, lane, qraw, col0);
  for (int i = lane; i < nb; i += 64) mask[i] = 0u;
  __syncthreads();
  // Column j (a head of the group, or with several queries the (query c / grp,
  // head c % grp) pair of column c = col0 + j) selects the blocks of the CSR
  // row of its query's position in its head's layout; a query before
  // position 0 selects none.
  // Two dependent round trips for all columns at once: lane j < ncols reads
  // its row's bounds, then every lane reads one column index of every row per
  // pass (rows longer than 64 entries take more passes).
  const int ncols = MQ ? min(16, a.grp * a.qn - col0) : G;
  int rstart = 0, rlen = 0, rrow = 0, rlay = 0;   // lane j: column j's CSR row
  if (lo <= hi && lane < ncols) {
    const int c = col0 + lane;
    const int qj = MQ ? qp + c / a.grp : max(qp, 0);
    const uint32_t r = qj >= 0 ? fdiv((uint32_t)qj, a.sb) : 0u;
    if (qj >= 0 && (int)r + 1 < a.row_stride) {
      const int head = MQ ? kvh * a.grp + c % a.grp : kvh * G + lane;
      rlay = head % a.num_layouts;
      const int32_t* rp = a.row_ptr + (size_t)rlay * a.row_stride;
      rstart = max(rp[r], 0);
      rlen = max(min(rp[r + 1], a.col_stride) - rstart, 0);
      rrow = (int)r;
    }
  }
  int maxlen = rlen;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) maxlen = max(maxlen, __shfl_xor(maxlen, o, 64));
  constexpr int kCols = MQ ? 16 : G;
  for (int off = 0; off < maxlen; off += 64) {
    int cj[kCols];
#pragma unroll
    for (int j = 0; j < kCols; ++j) {
      const int st = __shfl(rstart, j, 64), ln = __shfl(rlen, j, 64), ly = __shfl(rlay, j, 64);
      const int e = off + lane;
      cj[j] = (j < ncols && e < ln) ? a.col_idx[(size_t)ly * a.col_stride + st + e] : -1;
    }
#pragma unroll
    for (int j = 0; j < kCols; ++j) {
      const int r = __shfl(rrow, j, 64);
      if (cj[j] >= 0 && cj[j] <= r && cj[j] < nb) atomicOr(&mask[cj[j]], 1u << j);
    }
  }
  __syncthreads();
  int count = 0;
  for (int base = 0; base < nb; base += 64) {
    const int c = base + lane;
    const uint32_t mk = c < nb ? mask[c] : 0u;
    const uint64_t bal = __builtin_amdgcn_ballot_w64(mk != 0u);
    const int before = __builtin_popcountll(bal & ((1ull << lane) - 1ull));
    if (mk) list[count + before] = ((uint32_t)c << 16) | mk;
    count += __builtin_popcountll(bal);
  }
  __syncthreads();
  const PartialDst dst = split_dst(a, b, kvh, MQ ? a.grp : G, split, D);
  const int e0 = (int)((int64_t)split * count / a.num_splits);
  const int e1 = (int)((int64_t)(split + 1) * count / a.num_splits);
  if (e0 >= e1 || lo > hi) {
    if constexpr (MQ)
      write_empty_mq(dst, lane, a.grp, a.qn, a.num_heads, col0);
    else
      write_empty<G>(dst, lane);
    return;
  }
  LaneGeo lg;
  lg.init(lane);
  const SparseMap smap{list, a.table + (size_t)b * a.max_blocks, e1 * (int)a.sb.d, lo, hi, a.bs, a.sb,
                       FM, (1u << G) - 1u};
  QF16<D> qf;
  StoreF16<D> st{(const _Float16*)a.k, (const _Float16*)a.v, a.num_kv_heads, kvh};
  Online<D, G, CAP> on;
  on.init();
  auto prep = [&](QF16<D>& q) { convert_q<D, G, MQ>(a, lane, qraw, q, col0); };
  if constexpr (MQ) {
    // the map applies each lane's query bounds to the resolved key positions
    SparseMapMQ map{smap, 0, 0};
    query_bounds(a, b, lane, col0, map.qlo, map.qhi);
    run_tiles<D, G, CAP, kPipe, FM>(a, st, map, qf, prep, lg, on, e0 * (int)a.sb.d, map.slot_end, lane);
    on.finish_mq(dst, lane, a.grp, a.qn, a.num_heads, col0);
  } else {
    run_tiles<D, G, CAP, kPipe, FM>(a, st, smap, qf, prep, lg, on, e0 * (int)a.sb.d, smap.slot_end, lane);
    on.finish(dst, lane);
  }
}

// ------------------------------------------------------------------ combine
//
// Merge the partials of one (sequence, head): M = max m_s,
// l = sum l_s 2^{m_s - M}, out = sum acc_s 2^{m_s - M} / l, lse = (M + log2 l) ln 2.
// One workgroup per (sequence, head).  Partials with l = 0 exactly (no
// visible key) are skipped; any other l, NaN included, is merged, so a NaN
// that reached a partial from a visible K, V or Q value reaches out and lse as
// it does in the plain definition.  out is f32, or f16 rounded to nearest even
// from the f32 result; with out == nullptr only lse is written (acc is then
// not read).

struct OutRow {
  void* p;     // first element of the (sequence, head) row, or nullptr
  bool f16;
  __device__ __forceinline__ void store(int d, float x) const {
    if (f16)
      ((_Float16*)p)[d] = (_Float16)x;
    else
      ((float*)p)[d] = x;
  }
  // Elements d .. d + 3 (d a multiple of 4): one 8- or 16-byte store when the
  // row is aligned to it (the output's base address decides it for every row).
  __device__ __forceinline__ void store4(int d, f4 x) const {
    if (f16) {
      const h4 y = {(_Float16)x[0], (_Float16)x[1], (_Float16)x[2], (_Float16)x[3]};
      if (((uintptr_t)p & 7) == 0) {
        *(h4*)((_Float16*)p + d) = y;
      } else {
#pragma unroll
        for (int e = 0; e < 4; ++e) ((_Float16*)p)[d + e] = y[e];
      }
    } else {
      if (((uintptr_t)p & 15) == 0) {
        *(f4*)((float*)p + d) = x;
      } else {
#pragma unroll
        for (int e = 0; e < 4; ++e) ((float*)p)[d + e] = x[e];
      }
    }
  }
};

__device__ __forceinline__ OutRow out_row(void* out, bool f16, int bh, int D) {
  if (!out) return OutRow{nullptr, f16};
  return OutRow{f16 ? (void*)((_Float16*)out + (size_t)bh * D) : (void*)((float*)out + (size_t)bh * D), f16};
}

template <int D, class Loc>
__device__ __forceinline__ void merge_partials(const Loc& loc, int n, const OutRow out, float* __restrict__ lse_out) {
  // 256 threads: slot group sg = tid / 32 takes partials sg, sg + 8, ... and
  // folds them in with a running max (the rule above, one partial at a
  // time), loading four partials at once; thread c of a group owns dims
  // 4c + 128j.  The eight groups are then merged through LDS.  (m, l) and acc
  // are loaded together, so the merge waits on one round of loads.
  constexpr int NJ = D / 128 > 0 ? D / 128 : 1;
  constexpr int DC = D >= 128 ? 32 : D / 4;   // threads per group carrying dims
  constexpr int U = 4;                        // partials per group per round
  __shared__ float red[8][D];
  __shared__ float redm[8], redl[8];
  const int tid = threadIdx.x, sg = tid >> 5, c = tid & 31;
  float m = -__builtin_inff(), L = 0.f;
  f4 o[NJ];
#pragma unroll
  for (int j = 0; j < NJ; ++j) o[j] = f4{0.f, 0.f, 0.f, 0.f};
  for (int s0 = sg; s0 < n; s0 += 8 * U) {
    float2 v[U];
    f4 x[U][NJ];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int s = s0 + 8 * u;
      v[u] = s < n ? loc.ml(s) : make_float2(-__builtin_inff(), 0.f);
      if (s < n && c < DC && out.p) {
        const float* row = loc.acc(s);
#pragma unroll
        for (int j = 0; j < NJ; ++j) x[u][j] = *(const f4*)(row + 128 * j + 4 * c);
      }
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      if (v[u].y != 0.f) {   // skipped: empty pieces (their acc is never read into the sum)
        const float m_new = fmaxf(m, v[u].x);
        const float ca = fast_exp2(m - m_new), cb = fast_exp2(v[u].x - m_new);
        L = L * ca + v[u].y * cb;
        if (c < DC) {
#pragma unroll
          for (int j = 0; j < NJ; ++j) o[j] = o[j] * ca + x[u][j] * cb;
        }
        m = m_new;
      }
    }
  }
  if (c < DC) {
#pragma unroll
    for (int j = 0; j < NJ; ++j) *(f4*)&red[sg][128 * j + 4 * c] = o[j];
  }
  if (c == 0) {
    redm[sg] = m;
    redl[sg] = L;
  }
  __syncthreads();
  float M = -__builtin_inff();
#pragma unroll
  for (int g = 0; g < 8; ++g) M = redl[g] != 0.f ? fmaxf(M, redm[g]) : M;
  float wg[8], Lt = 0.f;
#pragma unroll
  for (int g = 0; g < 8; ++g) {
    wg[g] = redl[g] != 0.f ? fast_exp2(redm[g] - M) : 0.f;
    Lt += redl[g] * wg[g];
  }
  if (out.p) {
    for (int d = tid; d < D; d += 256) {
      float ot = 0.f;
#pragma unroll
      for (int g = 0; g < 8; ++g) ot += red[g][d] * wg[g];
      out.store(d, Lt != 0.f ? ot / Lt : 0.f);
    }
  }
  if (tid == 0 && lse_out) *lse_out = Lt != 0.f ? (M + __builtin_log2f(Lt)) * kLn2 : -__builtin_inff();
}

// The same merge by 32 threads for one row with few partials: the partials
// are folded in one at a time with a running max, four loads in flight;
// thread c owns dims 4c + 128j.  No LDS and no barrier.
template <int D, class Loc>
__device__ __forceinline__ void merge_row(const Loc& loc, int n, const OutRow out, float* __restrict__ lse_out,
                                          int c) {
  constexpr int NJ = D / 128 > 0 ? D / 128 : 1;
  constexpr int DC = D >= 128 ? 32 : D / 4;
  constexpr int U = 4;
  float m = -__builtin_inff(), L = 0.f;
  f4 o[NJ];
#pragma unroll
  for (int j = 0; j < NJ; ++j) o[j] = f4{0.f, 0.f, 0.f, 0.f};
  // Loads without branches: past the last partial a lane reloads it (weighted
  // out below), and lanes beyond the row's dims (D = 64) reload dims 0..3.
  const int cl = c < DC ? c : 0;
  for (int s0 = 0; s0 < n; s0 += U) {
    float2 v[U];
    f4 x[U][NJ];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int s = min(s0 + u, n - 1);
      v[u] = loc.ml(s);
      if (out.p) {
        const float* row = loc.acc(s);
#pragma unroll
        for (int j = 0; j < NJ; ++j) x[u][j] = *(const f4*)(row + 128 * j + 4 * cl);
      }
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      if (s0 + u < n && v[u].y != 0.f) {
        const float m_new = fmaxf(m, v[u].x);
        const float ca = fast_exp2(m - m_new), cb = fast_exp2(v[u].x - m_new);
        L = L * ca + v[u].y * cb;
#pragma unroll
        for (int j = 0; j < NJ; ++j) o[j] = o[j] * ca + x[u][j] * cb;
        m = m_new;
      }
    }
  }
  if (out.p && c < DC) {
#pragma unroll
    for (int j = 0; j < NJ; ++j) {
      f4 y;
#pragma unroll
      for (int e = 0; e < 4; ++e) y[e] = L != 0.f ? o[j][e] / L : 0.f;
      out.store4(128 * j + 4 * c, y);
    }
  }
  if (c == 0 && lse_out) *lse_out = L != 0.f ? (m + __builtin_log2f(L)) * kLn2 : -__builtin_inff();
}

// Static splits of at most kShortRow pieces per row take the row-group combine.
constexpr int kShortRow = 16;

// Static splits: partials of (b, h) at [bh, s] for s < S.
struct SplitLoc {
  const float* acc0;
  const float2* ml0;
  int D;
  __device__ __forceinline__ float2 ml(int s) const { return ml0[s]; }
  __device__ __forceinline__ const float* acc(int s) const { return acc0 + (size_t)s * D; }
};

template <int D>
__global__ __launch_bounds__(256) void combine_kernel(const float* __restrict__ part_acc,
                                                      const float2* __restrict__ part_ml, void* __restrict__ out,
                                                      int out_f16, float* __restrict__ lse, int S, int nbh) {
  const int bh = blockIdx.x;
  const SplitLoc loc{part_acc + (size_t)bh * S * D, part_ml + (size_t)bh * S, D};
  merge_partials<D>(loc, S, out_row(out, out_f16 != 0, bh, D), lse ? lse + bh : nullptr);
}

// Balanced schedule: the partials of (b, h) sit in slots w + b for the
// workers w whose unit range meets b's, at [slot, h] (an empty piece has l = 0).
struct SlotLoc {
  const float* acc0;   // slot (w0 + b), head h
  const float2* ml0;
  int H, D;
  __device__ __forceinline__ float2 ml(int s) const { return ml0[(size_t)s * H]; }
  __device__ __forceinline__ const float* acc(int s) const { return acc0 + (size_t)s * H * D; }
};

// Row bh = (b, h): its n partials from the schedule (C units per worker, the
// unit prefix P at sched[2 ..]): workers w0 .. w1 meet sequence b, and their
// pieces of it sit in slots w0 + b .. w1 + b.
__device__ __forceinline__ SlotLoc balanced_row(const float* part_acc, const float2* part_ml,
                                                const int32_t* __restrict__ sched, int H, int D, int bh, int& n) {
  const int b = bh / H, h = bh - b * H;
  const int C = sched[1];
  const int p0 = sched[2 + b], p1 = sched[3 + b];
  n = 0;
  size_t slot0 = 0;
  if (p1 > p0 && C > 0) {
    const int w0 = p0 / C, w1 = (p1 - 1) / C;
    n = w1 - w0 + 1;
    slot0 = (size_t)(w0 + b);
  }
  return SlotLoc{part_acc + (slot0 * H + h) * D, part_ml + slot0 * H + h, H, D};
}

template <int D>
__global__ __launch_bounds__(256) void combine_balanced_kernel(const float* __restrict__ part_acc,
                                                               const float2* __restrict__ part_ml,
                                                               const int32_t* __restrict__ sched,
                                                               void* __restrict__ out, int out_f16,
                                                               float* __restrict__ lse, int H, int nbh) {
  const int bh = blockIdx.x;
  int n;
  const SlotLoc loc = balanced_row(part_acc, part_ml, sched, H, D, bh, n);
  merge_partials<D>(loc, n, out_row(out, out_f16 != 0, bh, D), lse ? lse + bh : nullptr);
}

// One wave per row, for rows with few partials: the wave's 64 / (D/4) lane
// groups (D/4 lanes of four dims each) fold the partials h, h + groups, ...
// with a running max, four loads in flight, then the groups are merged with
// row swaps (permlane32, and permlane16 for D = 64).  The merge of two states
// is symmetric, so both partners end with the same bits.  No LDS, no barrier.
template <int D, class Loc>
__device__ __forceinline__ void merge_row_wave(const Loc& loc, int n, const OutRow out, float* __restrict__ lse_out,
                                               int lane) {
  static_assert(D == 64 || D == 128, "one wave per row covers D = 64 or 128");
  constexpr int DL = D / 4;        // lanes per group
  constexpr int NG = 64 / DL;      // groups per wave
  constexpr int U = 4;
  const int h = lane / DL, c = lane % DL;
  float m = -__builtin_inff(), L = 0.f;
  f4 o = {0.f, 0.f, 0.f, 0.f};
  for (int s0 = h; s0 < n; s0 += NG * U) {
    float2 v[U];
    f4 x[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {   // past the last partial a lane reloads it, weighted out below
      const int s = min(s0 + NG * u, n - 1);
      v[u] = loc.ml(s);
      if (out.p) x[u] = *(const f4*)(loc.acc(s) + 4 * c);
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      if (s0 + NG * u < n && v[u].y != 0.f) {   // skipped: empty pieces
        const float m_new = fmaxf(m, v[u].x);
        const float ca = fast_exp2(m - m_new), cb = fast_exp2(v[u].x - m_new);
        L = L * ca + v[u].y * cb;
        if (out.p) o = o * ca + x[u] * cb;
        m = m_new;
      }
    }
  }
  auto merge = [&](auto swap) {
    float m1, m2, l1, l2;
    swap(m, m1, m2);
    swap(L, l1, l2);
    float a[4], b[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) swap(o[e], a[e], b[e]);
    const float M = fmaxf(m1, m2);
    const float Mu = M == -__builtin_inff() ? 0.0f : M;
    const float ca = fast_exp2(m1 - Mu), cb = fast_exp2(m2 - Mu);
    L = l1 * ca + l2 * cb;
#pragma unroll
    for (int e = 0; e < 4; ++e) o[e] = a[e] * ca + b[e] * cb;
    m = M;
  };
  merge([](float x, float& a, float& b) { swap32(x, a, b); });
  if constexpr (NG == 4) merge([](float x, float& a, float& b) { swap16(x, a, b); });
  if (h == 0 && out.p) {
    f4 y;
#pragma unroll
    for (int e = 0; e < 4; ++e) y[e] = L != 0.f ? o[e] / L : 0.f;
    out.store4(4 * c, y);
  }
  if (lane == 0 && lse_out) *lse_out = L != 0.f ? (m + __builtin_log2f(L)) * kLn2 : -__builtin_inff();
}

// Balanced schedule, one wave per (sequence, head) row, four rows per
// workgroup; for calls whose rows have few partials.
template <int D>
__global__ __launch_bounds__(256) void combine_balanced_wave_kernel(const float* __restrict__ part_acc,
                                                                    const float2* __restrict__ part_ml,
                                                                    const int32_t* __restrict__ sched,
                                                                    void* __restrict__ out, int out_f16,
                                                                    float* __restrict__ lse, int H, int nbh) {
  const int bh = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (bh >= nbh) return;
  int n;
  const SlotLoc loc = balanced_row(part_acc, part_ml, sched, H, D, bh, n);
  merge_row_wave<D>(loc, n, out_row(out, out_f16 != 0, bh, D), lse ? lse + bh : nullptr, threadIdx.x & 63);
}

// Balanced schedule, two rows per wave (eight per workgroup), each merged by
// its own 32 lanes; for many rows of about four partials or fewer, which one
// round of loads covers.
template <int D>
__global__ __launch_bounds__(256) void combine_balanced_half_kernel(const float* __restrict__ part_acc,
                                                                    const float2* __restrict__ part_ml,
                                                                    const int32_t* __restrict__ sched,
                                                                    void* __restrict__ out, int out_f16,
                                                                    float* __restrict__ lse, int H, int nbh) {
  const int bh = blockIdx.x * 8 + (threadIdx.x >> 5);
  if (bh >= nbh) return;
  int n;
  const SlotLoc loc = balanced_row(part_acc, part_ml, sched, H, D, bh, n);
  merge_row<D>(loc, n, out_row(out, out_f16 != 0, bh, D), lse ? lse + bh : nullptr, threadIdx.x & 31);
}

// Static splits with at most kShortRow splits: eight rows per workgroup, each
// merged by its own 32 threads.
template <int D>
__global__ __launch_bounds__(256) void combine_rows_kernel(const float* __restrict__ part_acc,
                                                           const float2* __restrict__ part_ml, void* __restrict__ out,
                                                           int out_f16, float* __restrict__ lse, int S, int nbh) {
  const int row = blockIdx.x * 8 + (threadIdx.x >> 5);
  if (row >= nbh) return;
  const SplitLoc loc{part_acc + (size_t)row * S * D, part_ml + (size_t)row * S, D};
  merge_row<D>(loc, S, out_row(out, out_f16 != 0, row, D), lse ? lse + row : nullptr, threadIdx.x & 31);
}

}  // namespace dattn
