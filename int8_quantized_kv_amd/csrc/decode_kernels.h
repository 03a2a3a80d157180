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
// Inside a wavefront, keys are processed in tiles of 16:
//   QK^T  on the matrix cores as S^T = K . Q^T with v_mfma_f32_16x16x32_f16
//         (A = 16 keys x 32 dims of K, B = 32 dims x 16 heads of Q^T).  Q is
//         f32, so it enters as an f16 hi/lo pair (q = hi + lo) and the two
//         products are accumulated in f32; f16 and int8 keys are exact in f16.
//         f32 caches use v_mfma_f32_16x16x4_f32 instead.
//         The output lands as lane l <-> head l%16, keys 4*(l/16)+e (e<4).
//   softmax online, in the log2 domain, per head (one head per lane column).
//   PV    on the VALU: lane l owns 8 output dims and a group of keys of the
//         tile; the probabilities of those keys sit in lane (16*(l/16) + head)
//         of the same row, so one DPP row broadcast per (head, key) delivers
//         them without touching LDS.
// Loads are 128-bit and each instruction reads whole 64-byte pieces of K
// rows (16 keys per instruction) or whole V rows (4 keys per instruction).
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

constexpr int kTile = 16;          // keys per tile
constexpr float kSlack = 8.0f;     // lazy max: raise m only when a tile exceeds it by > 2^8
constexpr float kLn2 = 0.69314718055994531f;

// Kernel arguments (one struct for every kind; unused fields are zero).
struct DecodeArgs {
  const float* q;            // [B, H, D]
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
  float* part_acc;           // [B, H, S, D]
  float2* part_ml;           // [B, H, S]  (m in log2 units, l)
  int32_t num_heads, num_kv_heads, max_blocks, num_splits, split_tokens;
  int32_t causal, window, hot_window;
  int32_t sparse_block, num_layouts, row_stride, col_stride, sparse_nblk, blocks_per_split;
  float qmul;    // scale * log2(e) without softcap, scale / cap with softcap
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

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// tanh(x) = 1 - 2 / (e^{2x} + 1); saturates correctly at +-inf.
__device__ __forceinline__ float fast_tanh(float x) {
  float e = fast_exp2(x * 2.8853900817779268f);
  return 1.0f - 2.0f * __builtin_amdgcn_rcpf(e + 1.0f);
}

// Visible absolute key range [lo, hi] of sequence b (hi < lo when empty):
// causal keeps t <= q, a window W keeps t >= q-W+1 once q >= W
// (doppler is_masked), and keys exist only below seq_lens[b].
__device__ __forceinline__ void visible_range(const DecodeArgs& a, int b, int& lo, int& hi, int& qpos) {
  int L = a.seq_lens[b];
  int q = a.q_pos ? a.q_pos[b] : L - 1;
  hi = a.causal ? min(q, L - 1) : L - 1;
  lo = (a.window > 0 && q >= a.window) ? q - a.window + 1 : 0;
  qpos = q;
}

// int8 x 8 (two LSB-first words, two's complement) -> exact f16 x 8.
// Bias each byte by 128, drop it into the mantissa of 1024.0h (0x6400) and
// subtract 1152: (1024 + i + 128) - 1152 = i exactly.
__device__ __forceinline__ h2 i8pair_to_h2(uint32_t lo_byte_word) {
  h2 v = __builtin_bit_cast(h2, lo_byte_word | 0x64006400u);
  return v - h2{(_Float16)1152.0f, (_Float16)1152.0f};
}
__device__ __forceinline__ h8 i8x8_to_h8(uint32_t w0, uint32_t w1) {
  uint32_t x0 = w0 ^ 0x80808080u, x1 = w1 ^ 0x80808080u;
  h2 a = i8pair_to_h2((x0 & 0xFFu) | ((x0 & 0xFF00u) << 8));
  h2 b = i8pair_to_h2(((x0 >> 16) & 0xFFu) | ((x0 >> 8) & 0xFF0000u));
  h2 c = i8pair_to_h2((x1 & 0xFFu) | ((x1 & 0xFF00u) << 8));
  h2 d = i8pair_to_h2(((x1 >> 16) & 0xFFu) | ((x1 >> 8) & 0xFF0000u));
  return h8{a.x, a.y, b.x, b.y, c.x, c.y, d.x, d.y};
}

__device__ __forceinline__ float h2f(uint16_t bits) { return (float)__builtin_bit_cast(_Float16, bits); }

// ------------------------------------------------------------ Q fragments

// f16 MFMA path: slab c (32 dims) of lane l covers dims
// 64*(c/2) + 16*(l/16) + 8*(c%2) + [0, 8); the K fragments use the same map.
template <int D>
struct QF16 {
  h8 hi[D / 32], lo[D / 32];
};

template <int D, int G>
__device__ __forceinline__ void load_q_f16(const DecodeArgs& a, int b, int kvh, int lane, QF16<D>& qf) {
  const int j = lane & 15, g = lane >> 4;
  const float* qrow = a.q + ((size_t)b * a.num_heads + (size_t)kvh * G + (j < G ? j : 0)) * D;
#pragma unroll
  for (int c = 0; c < D / 32; ++c) {
    const int d0 = 64 * (c >> 1) + 16 * g + 8 * (c & 1);
    f4 x0 = *(const f4*)(qrow + d0), x1 = *(const f4*)(qrow + d0 + 4);
    float x[8] = {x0.x, x0.y, x0.z, x0.w, x1.x, x1.y, x1.z, x1.w};
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      float v = j < G ? x[e] * a.qmul : 0.0f;
      _Float16 h = (_Float16)v;
      qf.hi[c][e] = h;
      qf.lo[c][e] = (_Float16)(v - (float)h);
    }
  }
}

// f32 MFMA path (16x16x4): slab c of lane l is dim 16*(c/4) + 4*(l/16) + c%4.
template <int D>
struct QF32 {
  float v[D / 4];
};

template <int D, int G>
__device__ __forceinline__ void load_q_f32(const DecodeArgs& a, int b, int kvh, int lane, QF32<D>& qf) {
  const int j = lane & 15, g = lane >> 4;
  const float* qrow = a.q + ((size_t)b * a.num_heads + (size_t)kvh * G + (j < G ? j : 0)) * D;
#pragma unroll
  for (int m = 0; m < D / 16; ++m) {
    f4 x = *(const f4*)(qrow + 16 * m + 4 * g);
    qf.v[4 * m + 0] = j < G ? x.x * a.qmul : 0.0f;
    qf.v[4 * m + 1] = j < G ? x.y * a.qmul : 0.0f;
    qf.v[4 * m + 2] = j < G ? x.z * a.qmul : 0.0f;
    qf.v[4 * m + 3] = j < G ? x.w * a.qmul : 0.0f;
  }
}

// ------------------------------------------------------- K / V fragments
//
// A tile has 16 keys.  K lane l holds key l%16; V lane l holds keys
// 4*(l/16) + vsub*NTV + e (e < NTV) and dims 8*vdim + [0, 8) where, for
// DPR = D/8 lanes per V row, vdim = (l%16) % DPR and vsub = (l%16) / DPR.

template <int D>
struct Lay {
  static constexpr int DPR = D / 8;
  static constexpr int NTV = D / 32;
};

// f16 rows (paged pool or hot ring)
template <int D>
struct KF16 {
  u4 r[D / 32];
};
template <int D>
__device__ __forceinline__ void load_k_f16(const _Float16* row, int g, KF16<D>& k) {
#pragma unroll
  for (int c2 = 0; c2 < D / 64; ++c2) {
    const u4* p = (const u4*)(row + 64 * c2 + 16 * g);
    k.r[2 * c2] = __builtin_nontemporal_load(p);
    k.r[2 * c2 + 1] = __builtin_nontemporal_load(p + 1);
  }
}
template <int D>
__device__ __forceinline__ f4 scores_f16(const KF16<D>& k, const QF16<D>& q) {
  f4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int c = 0; c < D / 32; ++c) {
    h8 a = __builtin_bit_cast(h8, k.r[c]);
    acc = __builtin_amdgcn_mfma_f32_16x16x32_f16(a, q.hi[c], acc, 0, 0, 0);
    acc = __builtin_amdgcn_mfma_f32_16x16x32_f16(a, q.lo[c], acc, 0, 0, 0);
  }
  return acc;
}

// int8 cold rows: D/4 words, lane loads the 16 bytes of dims 64*c2 + 16*g + [0,16)
template <int D>
struct KI8 {
  u4 r[D / 64];
};
template <int D>
__device__ __forceinline__ void load_k_i8(const uint32_t* row, int g, KI8<D>& k) {
#pragma unroll
  for (int c2 = 0; c2 < D / 64; ++c2) k.r[c2] = __builtin_nontemporal_load((const u4*)(row + 16 * c2 + 4 * g));
}
template <int D>
__device__ __forceinline__ f4 scores_i8(const KI8<D>& k, const QF16<D>& q) {
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
  return acc;
}

// f32 rows
template <int D>
struct KF32 {
  f4 r[D / 16];
};
template <int D>
__device__ __forceinline__ void load_k_f32(const float* row, int g, KF32<D>& k) {
#pragma unroll
  for (int m = 0; m < D / 16; ++m) k.r[m] = __builtin_nontemporal_load((const f4*)(row + 16 * m + 4 * g));
}
template <int D>
__device__ __forceinline__ f4 scores_f32(const KF32<D>& k, const QF32<D>& q) {
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

// V pieces: 8 dims of one key.
struct VF16 {
  u4 r;
};
struct VI8 {
  u2v r;
};
struct VF32 {
  f4 a, b;
};
__device__ __forceinline__ void load_vrow(const _Float16* p, VF16& v) { v.r = __builtin_nontemporal_load((const u4*)p); }
__device__ __forceinline__ void load_vrow(const uint32_t* p, VI8& v) { v.r = __builtin_nontemporal_load((const u2v*)p); }
__device__ __forceinline__ void load_vrow(const float* p, VF32& v) {
  v.a = __builtin_nontemporal_load((const f4*)p);
  v.b = __builtin_nontemporal_load((const f4*)p + 1);
}

template <int G>
__device__ __forceinline__ void pv_acc(const VF16& v, const float (&w)[G], float (&acc)[G][8]) {
  h8 x = __builtin_bit_cast(h8, v.r);
#pragma unroll
  for (int h = 0; h < G; ++h)
#pragma unroll
    for (int d = 0; d < 8; ++d) acc[h][d] = __builtin_fmaf(w[h], (float)x[d], acc[h][d]);
}
template <int G>
__device__ __forceinline__ void pv_acc(const VI8& v, const float (&w)[G], float (&acc)[G][8]) {
  h8 x = i8x8_to_h8(v.r.x, v.r.y);
#pragma unroll
  for (int h = 0; h < G; ++h)
#pragma unroll
    for (int d = 0; d < 8; ++d) acc[h][d] = __builtin_fmaf(w[h], (float)x[d], acc[h][d]);
}
template <int G>
__device__ __forceinline__ void pv_acc(const VF32& v, const float (&w)[G], float (&acc)[G][8]) {
  float x[8] = {v.a.x, v.a.y, v.a.z, v.a.w, v.b.x, v.b.y, v.b.z, v.b.w};
#pragma unroll
  for (int h = 0; h < G; ++h)
#pragma unroll
    for (int d = 0; d < 8; ++d) acc[h][d] = __builtin_fmaf(w[h], x[d], acc[h][d]);
}

// ------------------------------------------------- online softmax state

template <int D, int G>
struct Online {
  float m;            // running max (log2 units) of head lane%16 -- equal in all rows
  float l;            // denominator part of (head lane%16, keys of row lane/16)
  float acc[G][8];    // PV part of (dims 8*vdim.., keys of this lane)

  __device__ __forceinline__ void init() {
    m = -__builtin_inff();
    l = 0.f;
#pragma unroll
    for (int h = 0; h < G; ++h)
#pragma unroll
      for (int d = 0; d < 8; ++d) acc[h][d] = 0.f;
  }

  // raw: this lane's 4 scores (already multiplied by qmul and any int8 key
  // scale); valid: which of keys 4*(lane/16)+e take part.  Returns p[4] and
  // rescales the state; the caller then broadcasts p to the PV lanes.
  __device__ __forceinline__ void softmax_tile(const DecodeArgs& a, const f4& raw, const bool (&valid)[4],
                                               float (&p)[4]) {
    float s[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      float x = raw[e];
      if (a.capl2 > 0.f) x = a.capl2 * fast_tanh(x);
      s[e] = valid[e] ? x : -__builtin_inff();
    }
    float mx = fmaxf(fmaxf(s[0], s[1]), fmaxf(s[2], s[3]));
    mx = fmaxf(mx, shfl_xor_f(mx, 16));
    mx = fmaxf(mx, shfl_xor_f(mx, 32));
    const float m_new = (mx > m + kSlack) ? mx : m;
    const float c = (m_new == m) ? 1.0f : fast_exp2(m - m_new);
    m = m_new;
    const float m_use = (m == -__builtin_inff()) ? 0.0f : m;
#pragma unroll
    for (int e = 0; e < 4; ++e) p[e] = fast_exp2(s[e] - m_use);
    l = l * c + ((p[0] + p[1]) + (p[2] + p[3]));
    if (__builtin_amdgcn_ballot_w64(c != 1.0f)) {
      static_for<0, G>([&](auto hc) {
        constexpr int h = decltype(hc)::value;
        const float ch = row_bcast<h>(c);
#pragma unroll
        for (int d = 0; d < 8; ++d) acc[h][d] *= ch;
      });
    }
  }

  // p of keys 4*(lane/16) + e for every head h < G, as seen by this lane.
  __device__ __forceinline__ static void broadcast(const float (&p)[4], float (&pb)[4][G]) {
    static_for<0, G>([&](auto hc) {
      constexpr int h = decltype(hc)::value;
#pragma unroll
      for (int e = 0; e < 4; ++e) pb[e][h] = row_bcast<h>(p[e]);
    });
  }

  // Reduce across lanes and write the split partial of heads kvh*G + [0, G).
  __device__ __forceinline__ void finish(const DecodeArgs& a, int b, int kvh, int split, int lane) {
    float lt = l + shfl_xor_f(l, 16);
    lt += shfl_xor_f(lt, 32);
#pragma unroll
    for (int h = 0; h < G; ++h)
#pragma unroll
      for (int d = 0; d < 8; ++d) {
        float x = acc[h][d];
        if constexpr (Lay<D>::DPR < 16) x += shfl_xor_f(x, 8);
        x += shfl_xor_f(x, 16);
        x += shfl_xor_f(x, 32);
        acc[h][d] = x;
      }
    const size_t S = (size_t)a.num_splits;
    const size_t head0 = (size_t)b * a.num_heads + (size_t)kvh * G;
    if (lane < Lay<D>::DPR) {
#pragma unroll
      for (int h = 0; h < G; ++h) {
        float* dst = a.part_acc + ((head0 + h) * S + split) * D + 8 * lane;
        *(f4*)dst = f4{acc[h][0], acc[h][1], acc[h][2], acc[h][3]};
        *(f4*)(dst + 4) = f4{acc[h][4], acc[h][5], acc[h][6], acc[h][7]};
      }
    }
    if (lane < G) a.part_ml[(head0 + lane) * S + split] = make_float2(m, lt);
  }
};

template <int G>
__device__ __forceinline__ void write_empty(const DecodeArgs& a, int b, int kvh, int split, int lane) {
  if (lane < G) {
    const size_t head0 = (size_t)b * a.num_heads + (size_t)kvh * G;
    a.part_ml[(head0 + lane) * (size_t)a.num_splits + split] = make_float2(-__builtin_inff(), 0.f);
  }
}

// ------------------------------------------------------------ tile engine
//
// Process tiles t0 = tfirst, tfirst+16, ... < tend over "positions" (absolute
// keys, or slots of the sparse union list).  The policy object maps a
// position to a row pointer and says whether (position, head) is visible.

template <int D, int G, class Policy>
__device__ __forceinline__ void run_tiles(const DecodeArgs& a, Policy& pol, Online<D, G>& st, int tfirst, int tend,
                                          int lane) {
  using KFrag = typename Policy::KFrag;
  using VFrag = typename Policy::VFrag;
  constexpr int NTV = Lay<D>::NTV;
  constexpr int DPR = Lay<D>::DPR;
  const int g = lane >> 4;
  const int vdim = (lane & 15) % DPR;
  const int vsub = (lane & 15) / DPR;

  KFrag kb[2];
  VFrag vb[2][NTV];
  auto issue = [&](int t0, int slot) {
    pol.load_k(t0 + (lane & 15), g, kb[slot]);
#pragma unroll
    for (int e = 0; e < NTV; ++e) pol.load_v(t0 + 4 * g + vsub * NTV + e, vdim, vb[slot][e]);
  };
  auto consume = [&](int t0, int slot) {
    f4 raw = pol.scores(kb[slot], t0 + 4 * g);
    bool valid[4];
    const int head = lane & 15;
#pragma unroll
    for (int e = 0; e < 4; ++e) valid[e] = pol.visible(t0 + 4 * g + e, head);
    float p[4];
    st.softmax_tile(a, raw, valid, p);
    float pb[4][G];
    Online<D, G>::broadcast(p, pb);
#pragma unroll
    for (int e = 0; e < NTV; ++e) {
      float w[G];
#pragma unroll
      for (int h = 0; h < G; ++h) {
        float x = pb[e][h];
        if constexpr (NTV < 4) x = vsub ? pb[NTV + e][h] : x;
        w[h] = x;
      }
      pol.scale_v(t0 + 4 * g + vsub * NTV + e, w);
      pv_acc<G>(vb[slot][e], w, st.acc);
    }
  };

  if (tfirst >= tend) return;
  issue(tfirst, 0);
  int t0 = tfirst;
  for (;;) {
    const int t1 = t0 + kTile;
    if (t1 < tend) issue(t1, 1);
    consume(t0, 0);
    if (t1 >= tend) break;
    const int t2 = t1 + kTile;
    if (t2 < tend) issue(t2, 0);
    consume(t1, 1);
    if (t2 >= tend) break;
    t0 = t2;
  }
}

// ------------------------------------------------------------- policies

// Position = absolute key; rows of a paged pool through the block table
// staged in LDS (entries blk0 .. blk0+n-1).
template <int D, class T>
struct PagedPolicy {
  using KFrag = std::conditional_t<std::is_same_v<T, float>, KF32<D>, KF16<D>>;
  using VFrag = std::conditional_t<std::is_same_v<T, float>, VF32, VF16>;
  const T* kpool;
  const T* vpool;
  const int32_t* tbl;   // LDS
  int blk0, kvh, Hkv, lo, hi;  // clamp / visibility range [lo, hi]
  FastDiv bs;
  QF16<D> qh;
  QF32<D> qf;

  __device__ __forceinline__ size_t row_off(int t) const {
    t = min(max(t, lo), hi);
    const uint32_t blk = fdiv((uint32_t)t, bs);
    const uint32_t off = (uint32_t)t - blk * bs.d;
    const int32_t phys = tbl[blk - blk0];
    return ((size_t)((uint32_t)phys * bs.d + off) * Hkv + kvh) * D;
  }
  __device__ __forceinline__ void load_k(int t, int g, KFrag& k) const {
    if constexpr (std::is_same_v<T, float>)
      load_k_f32<D>(kpool + row_off(t), g, k);
    else
      load_k_f16<D>(kpool + row_off(t), g, k);
  }
  __device__ __forceinline__ void load_v(int t, int vdim, VFrag& v) const {
    load_vrow(vpool + row_off(t) + 8 * vdim, v);
  }
  __device__ __forceinline__ f4 scores(const KFrag& k, int) const {
    if constexpr (std::is_same_v<T, float>)
      return scores_f32<D>(k, qf);
    else
      return scores_f16<D>(k, qh);
  }
  __device__ __forceinline__ bool visible(int t, int) const { return t >= lo && t <= hi; }
  template <int G>
  __device__ __forceinline__ void scale_v(int, float (&)[G]) const {}
};

// Cold tier: int8 rows through the staged cold table, f16 scales per (row, kvh).
template <int D>
struct ColdPolicy {
  using KFrag = KI8<D>;
  using VFrag = VI8;
  const uint32_t* kw;
  const uint32_t* vw;
  const uint16_t* ks;
  const uint16_t* vs;
  const int32_t* tbl;
  int blk0, kvh, Hkv, lo, hi;
  FastDiv bs;
  QF16<D> qh;

  __device__ __forceinline__ size_t rowkv(int t) const {  // (phys row)*Hkv + kvh
    t = min(max(t, lo), hi);
    const uint32_t blk = fdiv((uint32_t)t, bs);
    const uint32_t off = (uint32_t)t - blk * bs.d;
    return (size_t)((uint32_t)tbl[blk - blk0] * bs.d + off) * Hkv + kvh;
  }
  __device__ __forceinline__ void load_k(int t, int g, KFrag& k) const { load_k_i8<D>(kw + rowkv(t) * (D / 4), g, k); }
  __device__ __forceinline__ void load_v(int t, int vdim, VFrag& v) const {
    load_vrow(vw + rowkv(t) * (D / 4) + 2 * vdim, v);
  }
  __device__ __forceinline__ f4 scores(const KFrag& k, int t4) const {
    f4 r = scores_i8<D>(k, qh);
#pragma unroll
    for (int e = 0; e < 4; ++e) r[e] *= h2f(ks[rowkv(t4 + e)]);
    return r;
  }
  __device__ __forceinline__ bool visible(int t, int) const { return t >= lo && t <= hi; }
  template <int G>
  __device__ __forceinline__ void scale_v(int t, float (&w)[G]) const {
    const float sc = h2f(vs[rowkv(t)]);
#pragma unroll
    for (int h = 0; h < G; ++h) w[h] *= sc;
  }
};

// Hot tier: f16 ring, key t at slot t mod hot_window (doppler get_hot_pos).
template <int D>
struct HotPolicy {
  using KFrag = KF16<D>;
  using VFrag = VF16;
  const _Float16* kh;
  const _Float16* vh;
  int b, kvh, Hkv, lo, hi;
  FastDiv hw;
  QF16<D> qh;

  __device__ __forceinline__ size_t row_off(int t) const {
    t = min(max(t, lo), hi);
    const uint32_t slot = fmod_((uint32_t)t, hw);
    return (((size_t)b * hw.d + slot) * Hkv + kvh) * D;
  }
  __device__ __forceinline__ void load_k(int t, int g, KFrag& k) const { load_k_f16<D>(kh + row_off(t), g, k); }
  __device__ __forceinline__ void load_v(int t, int vdim, VFrag& v) const { load_vrow(vh + row_off(t) + 8 * vdim, v); }
  __device__ __forceinline__ f4 scores(const KFrag& k, int) const { return scores_f16<D>(k, qh); }
  __device__ __forceinline__ bool visible(int t, int) const { return t >= lo && t <= hi; }
  template <int G>
  __device__ __forceinline__ void scale_v(int, float (&)[G]) const {}
};

// Sparse: position = slot in the union list of selected sparse blocks of the
// GQA group (entry = (block << 16) | head mask), then the paged f16 pool
// through the global block table.
template <int D>
struct SparsePolicy {
  using KFrag = KF16<D>;
  using VFrag = VF16;
  const _Float16* kpool;
  const _Float16* vpool;
  const int32_t* table_row;   // global, this sequence
  const uint32_t* list;       // LDS
  int slot_end, kvh, Hkv, lo, hi;
  FastDiv bs, sb;
  QF16<D> qh;

  __device__ __forceinline__ void resolve(int slot, int& t, uint32_t& mask) const {
    const int s = min(slot, slot_end - 1);
    const uint32_t e = fdiv((uint32_t)s, sb);
    const uint32_t ent = list[e];
    t = (int)((ent >> 16) * sb.d + ((uint32_t)s - e * sb.d));
    mask = slot < slot_end ? (ent & 0xFFFFu) : 0u;
  }
  __device__ __forceinline__ size_t row_off(int slot) const {
    int t;
    uint32_t mk;
    resolve(slot, t, mk);
    t = min(max(t, lo), hi);
    const uint32_t blk = fdiv((uint32_t)t, bs);
    const uint32_t off = (uint32_t)t - blk * bs.d;
    return ((size_t)((uint32_t)table_row[blk] * bs.d + off) * Hkv + kvh) * D;
  }
  __device__ __forceinline__ void load_k(int s, int g, KFrag& k) const { load_k_f16<D>(kpool + row_off(s), g, k); }
  __device__ __forceinline__ void load_v(int s, int vdim, VFrag& v) const { load_vrow(vpool + row_off(s) + 8 * vdim, v); }
  __device__ __forceinline__ f4 scores(const KFrag& k, int) const { return scores_f16<D>(k, qh); }
  __device__ __forceinline__ bool visible(int slot, int head) const {
    int t;
    uint32_t mk;
    resolve(slot, t, mk);
    return ((mk >> head) & 1u) && t >= lo && t <= hi;
  }
  template <int G>
  __device__ __forceinline__ void scale_v(int, float (&)[G]) const {}
};

// ---------------------------------------------------------------- kernels

// Stage block-table entries [blk0, blk0 + n) of sequence b into LDS.
__device__ __forceinline__ void stage_table(const DecodeArgs& a, int b, int blk0, int n, int32_t* lds) {
  const int32_t* src = a.table + (size_t)b * a.max_blocks + blk0;
  for (int i = threadIdx.x; i < n; i += blockDim.x) lds[i] = src[i];
  __syncthreads();
}

template <int D, int G, class T>
__global__ __launch_bounds__(256) void paged_split_kernel(DecodeArgs a) {
  extern __shared__ int32_t lds_tbl[];
  const int split = blockIdx.x, b = blockIdx.y;
  const int lane = threadIdx.x & 63;
  const int kvh = blockIdx.z * (blockDim.x >> 6) + (threadIdx.x >> 6);
  int lo, hi, qp;
  visible_range(a, b, lo, hi, qp);
  const int tb = max(split * a.split_tokens, lo);
  const int te = min((split + 1) * a.split_tokens, hi + 1);   // [tb, te)
  int blk0 = 0, nblk = 0;
  if (tb < te) {
    blk0 = (int)fdiv((uint32_t)tb, a.bs);
    nblk = (int)fdiv((uint32_t)(te - 1), a.bs) - blk0 + 1;
  }
  stage_table(a, b, blk0, nblk, lds_tbl);
  if (tb >= te) {
    write_empty<G>(a, b, kvh, split, lane);
    return;
  }
  PagedPolicy<D, T> pol;
  pol.kpool = (const T*)a.k;
  pol.vpool = (const T*)a.v;
  pol.tbl = lds_tbl;
  pol.blk0 = blk0;
  pol.kvh = kvh;
  pol.Hkv = a.num_kv_heads;
  pol.lo = tb;
  pol.hi = te - 1;
  pol.bs = a.bs;
  if constexpr (std::is_same_v<T, float>)
    load_q_f32<D, G>(a, b, kvh, lane, pol.qf);
  else
    load_q_f16<D, G>(a, b, kvh, lane, pol.qh);
  Online<D, G> st;
  st.init();
  const int tfirst = tb & ~(kTile - 1);
  run_tiles<D, G>(a, pol, st, tfirst, te, lane);
  st.finish(a, b, kvh, split, lane);
}

template <int D, int G>
__global__ __launch_bounds__(256) void tiered_split_kernel(DecodeArgs a) {
  extern __shared__ int32_t lds_tbl[];
  const int split = blockIdx.x, b = blockIdx.y;
  const int lane = threadIdx.x & 63;
  const int kvh = blockIdx.z * (blockDim.x >> 6) + (threadIdx.x >> 6);
  int lo, hi, qp;
  visible_range(a, b, lo, hi, qp);
  const int C = a.cold_lens[b];
  const int tb = max(split * a.split_tokens, lo);
  const int te = min((split + 1) * a.split_tokens, hi + 1);
  const int ce = min(te, C);          // cold part [tb, ce)
  const int hb = max(tb, C);          // hot part  [hb, te)
  int blk0 = 0, nblk = 0;
  if (tb < ce) {
    blk0 = (int)fdiv((uint32_t)tb, a.bs);
    nblk = (int)fdiv((uint32_t)(ce - 1), a.bs) - blk0 + 1;
  }
  stage_table(a, b, blk0, nblk, lds_tbl);
  if (tb >= te) {
    write_empty<G>(a, b, kvh, split, lane);
    return;
  }
  QF16<D> qh;
  load_q_f16<D, G>(a, b, kvh, lane, qh);
  Online<D, G> st;
  st.init();
  if (tb < ce) {
    ColdPolicy<D> pol;
    pol.kw = (const uint32_t*)a.k;
    pol.vw = (const uint32_t*)a.v;
    pol.ks = a.k_scale;
    pol.vs = a.v_scale;
    pol.tbl = lds_tbl;
    pol.blk0 = blk0;
    pol.kvh = kvh;
    pol.Hkv = a.num_kv_heads;
    pol.lo = tb;
    pol.hi = ce - 1;
    pol.bs = a.bs;
    pol.qh = qh;
    run_tiles<D, G>(a, pol, st, tb & ~(kTile - 1), ce, lane);
  }
  if (hb < te) {
    HotPolicy<D> pol;
    pol.kh = (const _Float16*)a.k_hot;
    pol.vh = (const _Float16*)a.v_hot;
    pol.b = b;
    pol.kvh = kvh;
    pol.Hkv = a.num_kv_heads;
    pol.lo = hb;
    pol.hi = te - 1;
    pol.hw = a.hw;
    pol.qh = qh;
    run_tiles<D, G>(a, pol, st, hb & ~(kTile - 1), te, lane);
  }
  st.finish(a, b, kvh, split, lane);
}

// Block-sparse: each wave builds the union of the CSR rows of its G heads in
// LDS (a G-bit head mask per sparse block, then the blocks with a non-zero
// mask compacted in increasing order), takes the slice of that list its
// split owns and sweeps its keys.
template <int D, int G>
__global__ __launch_bounds__(256) void sparse_split_kernel(DecodeArgs a) {
  extern __shared__ uint32_t lds_sp[];
  const int split = blockIdx.x, b = blockIdx.y;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int kvh = blockIdx.z * (blockDim.x >> 6) + wave;
  const int nb = a.sparse_nblk;
  uint32_t* mask = lds_sp + (size_t)wave * 2 * nb;
  uint32_t* list = mask + nb;
  int lo, hi, qp;
  visible_range(a, b, lo, hi, qp);
  for (int i = lane; i < nb; i += 64) mask[i] = 0u;
  __syncthreads();
  const uint32_t r = fdiv((uint32_t)max(qp, 0), a.sb);
  if (lo <= hi && (int)r + 1 < a.row_stride) {
    for (int j = 0; j < G; ++j) {
      const int layout = (kvh * G + j) % a.num_layouts;
      const int32_t* rp = a.row_ptr + (size_t)layout * a.row_stride;
      const int start = max(rp[r], 0);
      const int end = min(rp[r + 1], a.col_stride);
      const int32_t* cols = a.col_idx + (size_t)layout * a.col_stride;
      for (int e = start + lane; e < end; e += 64) {
        const int c = cols[e];
        if (c >= 0 && c <= (int)r && c < nb) atomicOr(&mask[c], 1u << j);
      }
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
  const int e0 = split * a.blocks_per_split;
  const int e1 = min(e0 + a.blocks_per_split, count);
  if (e0 >= e1 || lo > hi) {
    write_empty<G>(a, b, kvh, split, lane);
    return;
  }
  SparsePolicy<D> pol;
  pol.kpool = (const _Float16*)a.k;
  pol.vpool = (const _Float16*)a.v;
  pol.table_row = a.table + (size_t)b * a.max_blocks;
  pol.list = list;
  pol.slot_end = e1 * (int)a.sb.d;
  pol.kvh = kvh;
  pol.Hkv = a.num_kv_heads;
  pol.lo = lo;
  pol.hi = hi;
  pol.bs = a.bs;
  pol.sb = a.sb;
  load_q_f16<D, G>(a, b, kvh, lane, pol.qh);
  Online<D, G> st;
  st.init();
  run_tiles<D, G>(a, pol, st, e0 * (int)a.sb.d, pol.slot_end, lane);
  st.finish(a, b, kvh, split, lane);
}

// Merge the split partials of one (sequence, head): 4 waves stride over the
// splits, lane owns dims lane + 64*j.
template <int D>
__global__ __launch_bounds__(256) void combine_kernel(const float* __restrict__ part_acc,
                                                      const float2* __restrict__ part_ml, float* __restrict__ out,
                                                      float* __restrict__ lse, int S) {
  constexpr int NJ = D / 64;
  __shared__ float red[4][D];
  __shared__ float redl[4], redm[4];
  const size_t bh = blockIdx.x;
  const int w = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const float2* ml = part_ml + bh * S;
  float M = -__builtin_inff();
  for (int s = threadIdx.x; s < S; s += 256) {
    float2 v = ml[s];
    if (v.y > 0.f) M = fmaxf(M, v.x);
  }
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) M = fmaxf(M, shfl_xor_f(M, o));
  if (lane == 0) redm[w] = M;
  __syncthreads();
  M = fmaxf(fmaxf(redm[0], redm[1]), fmaxf(redm[2], redm[3]));
  float L = 0.f, o[NJ];
#pragma unroll
  for (int j = 0; j < NJ; ++j) o[j] = 0.f;
  for (int s = w; s < S; s += 4) {
    const float2 v = ml[s];
    if (v.y > 0.f) {
      const float wt = fast_exp2(v.x - M);
      L += wt * v.y;
      const float* row = part_acc + (bh * S + s) * D;
#pragma unroll
      for (int j = 0; j < NJ; ++j) o[j] += wt * row[lane + 64 * j];
    }
  }
#pragma unroll
  for (int j = 0; j < NJ; ++j) red[w][lane + 64 * j] = o[j];
  if (lane == 0) redl[w] = L;
  __syncthreads();
  if (w == 0) {
    const float Lt = (redl[0] + redl[1]) + (redl[2] + redl[3]);
#pragma unroll
    for (int j = 0; j < NJ; ++j) {
      const int d = lane + 64 * j;
      const float ot = (red[0][d] + red[1][d]) + (red[2][d] + red[3][d]);
      out[bh * D + d] = Lt > 0.f ? ot / Lt : 0.f;
    }
    if (lane == 0 && lse) lse[bh] = Lt > 0.f ? (M + __builtin_log2f(Lt)) * kLn2 : -__builtin_inff();
  }
}

}  // namespace dattn
