// append_kernel.h -- gfx950 write paths: append one token per sequence to the
// tiered cache's f16 hot ring, first moving the oldest hot token to the paged
// int8 cold tier when the ring is full (quantise on evict); and append one
// token per sequence to a window ring.
//
// The ring and the paged cold tier are the layouts the tiered decode reads
// (doppler attention_decode_tiered_int8_f16kv.wgsl: hot slot = absolute
// position mod hot_window, cold rows of D/4 words holding four two's-complement
// bytes each, least-significant first, with one f16 scale per (token, kv
// head); attention.js pages the cold tier through its own block table).  The
// quantiser itself is not on the pages; it follows the description of the
// tiered workload's data (scale = max|x| / 127 per (token, kv head)), with
// every decision taken in f32: s = f16(max|x| / 127) rounded to nearest even,
// code = clamp(rint(x / s), -127, 127), an all-zero row giving s = 0.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace dattn {

struct AppendArgs {
  const uint16_t* k_new;   // [B, Hkv, D] f16
  const uint16_t* v_new;
  uint16_t* k_hot;         // [B, hot_window, Hkv, D] f16
  uint16_t* v_hot;
  uint32_t* k_cold;        // [num_blocks, bs, Hkv, D/4] u32
  uint32_t* v_cold;
  uint16_t* k_scale;       // [num_blocks, bs, Hkv] f16
  uint16_t* v_scale;
  const int32_t* table;    // [B, max_blocks]
  int32_t* seq_lens;       // [B], advanced by one
  int32_t* cold_lens;      // [B], advanced by one when a token is evicted
  int32_t num_kv_heads, block_size, max_blocks, num_blocks, hot_window;
};

// Quantise one f16 row of D values held by the wave's first D/4 lanes, four
// consecutive elements per lane (x), into one packed word per lane and the
// row's f16 scale.
template <int D>
__device__ __forceinline__ void quantize_row_wave(const float (&x)[4], int lane, uint32_t& word, uint16_t& scale) {
  float amax = 0.0f;
  if (lane < D / 4) amax = fmaxf(fmaxf(fabsf(x[0]), fabsf(x[1])), fmaxf(fabsf(x[2]), fabsf(x[3])));
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) amax = fmaxf(amax, __shfl_xor(amax, o, 64));
  const float s32 = __fdiv_rn(amax, 127.0f);
  const _Float16 s16 = (_Float16)s32;       // round to nearest even
  const float s = (float)s16;
  word = 0u;
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    int i = 0;
    if (s > 0.0f) {
      const float r = rintf(__fdiv_rn(x[e], s));
      i = r > 127.0f ? 127 : (r < -127.0f ? -127 : (int)r);
    }
    word |= ((uint32_t)(uint8_t)(int8_t)i) << (8 * e);
  }
  scale = __builtin_bit_cast(uint16_t, s16);
}

__device__ __forceinline__ void unpack4_f16(uint2 w, float (&x)[4]) {
  x[0] = (float)__builtin_bit_cast(_Float16, (uint16_t)(w.x & 0xFFFFu));
  x[1] = (float)__builtin_bit_cast(_Float16, (uint16_t)(w.x >> 16));
  x[2] = (float)__builtin_bit_cast(_Float16, (uint16_t)(w.y & 0xFFFFu));
  x[3] = (float)__builtin_bit_cast(_Float16, (uint16_t)(w.y >> 16));
}

// One workgroup per sequence, one wave per kv head (strided when Hkv exceeds
// the waves); lane l < D/4 owns elements 4l .. 4l+3 of every row it touches.
// A sequence whose lengths or cold block-table entry break the preconditions
// is left unchanged.  The rows of the first kv head a wave handles are loaded
// while the block-table entry is still in flight (their addresses depend only
// on the lengths), so a call costs two dependent memory round trips, not three.
template <int D>
__global__ __launch_bounds__(1024) void append_tiered_int8_kernel(AppendArgs a) {
  const int b = blockIdx.x;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, waves = blockDim.x >> 6;
  const int64_t L = a.seq_lens[b], C = a.cold_lens[b];
  const int hw = a.hot_window, bs = a.block_size, Hkv = a.num_kv_heads;
  if (!(C >= 0 && C <= L && L - C <= hw && L < 0x7FFFFFFF)) return;   // uniform over the workgroup
  const bool evict = L - C == hw;
  const int64_t bi = C / bs;
  int32_t blk = 0;
  if (evict) blk = bi < a.max_blocks ? a.table[(int64_t)b * a.max_blocks + bi] : -1;
  const int64_t slot_old = C % hw, slot_new = L % hw;
  const int c0 = 4 * lane;
  const bool row_lane = lane < D / 4;
  auto hot_at = [&](int64_t slot, int g) { return (((int64_t)b * hw + slot) * Hkv + g) * D + c0; };
  auto new_at = [&](int g) { return ((int64_t)b * Hkv + g) * D + c0; };
  uint2 hk = {0u, 0u}, hv = {0u, 0u}, nk = {0u, 0u}, nv = {0u, 0u};
  if (wave < Hkv && row_lane) {
    if (evict) {
      hk = *(const uint2*)(a.k_hot + hot_at(slot_old, wave));
      hv = *(const uint2*)(a.v_hot + hot_at(slot_old, wave));
    }
    nk = *(const uint2*)(a.k_new + new_at(wave));
    nv = *(const uint2*)(a.v_new + new_at(wave));
  }
  if (evict && (blk < 0 || blk >= a.num_blocks)) return;   // uniform over the workgroup
  const int64_t row = (int64_t)blk * bs + C % bs;
  for (int g = wave; g < Hkv; g += waves) {
    if (g != wave && row_lane) {
      if (evict) {
        hk = *(const uint2*)(a.k_hot + hot_at(slot_old, g));
        hv = *(const uint2*)(a.v_hot + hot_at(slot_old, g));
      }
      nk = *(const uint2*)(a.k_new + new_at(g));
      nv = *(const uint2*)(a.v_new + new_at(g));
    }
    if (evict) {
      const int64_t cold = row * Hkv + g;
      float xk[4], xv[4];
      unpack4_f16(hk, xk);
      unpack4_f16(hv, xv);
      uint32_t wk, wv;
      uint16_t sk, sv;
      quantize_row_wave<D>(xk, lane, wk, sk);
      quantize_row_wave<D>(xv, lane, wv, sv);
      if (row_lane) {
        a.k_cold[cold * (D / 4) + lane] = wk;
        a.v_cold[cold * (D / 4) + lane] = wv;
      }
      if (lane == 0) {
        a.k_scale[cold] = sk;
        a.v_scale[cold] = sv;
      }
    }
    // the new token goes to slot L mod hw (the evicted slot when the ring was
    // full: its old contents are already in registers)
    if (row_lane) {
      *(uint2*)(a.k_hot + hot_at(slot_new, g)) = nk;
      *(uint2*)(a.v_hot + hot_at(slot_new, g)) = nv;
    }
  }
  __syncthreads();   // every thread has read seq_lens[b] and cold_lens[b]
  if (threadIdx.x == 0) {
    a.seq_lens[b] = (int32_t)(L + 1);
    a.cold_lens[b] = (int32_t)(evict ? C + 1 : C);
  }
}

// Window-ring write path: the new token of sequence b goes to slot
// seq_lens[b] mod W, overwriting the token that leaves the window, and
// seq_lens[b] grows by one.  One workgroup per sequence, a wave per kv head
// (strided), lane l < D/4 copying elements 4l .. 4l+3.  A negative length
// leaves the sequence unchanged.
template <int D>
__global__ __launch_bounds__(1024) void append_ring_f16_kernel(const uint16_t* k_new, const uint16_t* v_new,
                                                               uint16_t* k_ring, uint16_t* v_ring, int32_t* seq_lens,
                                                               int Hkv, int W) {
  const int b = blockIdx.x;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, waves = blockDim.x >> 6;
  const int64_t L = seq_lens[b];
  if (L < 0 || L >= 0x7FFFFFFF) return;   // uniform over the workgroup
  const int64_t slot = L % W;
  if (lane < D / 4) {
    for (int g = wave; g < Hkv; g += waves) {
      const int64_t src = ((int64_t)b * Hkv + g) * D + 4 * lane;
      const int64_t dst = (((int64_t)b * W + slot) * Hkv + g) * D + 4 * lane;
      *(uint2*)(k_ring + dst) = *(const uint2*)(k_new + src);
      *(uint2*)(v_ring + dst) = *(const uint2*)(v_new + src);
    }
  }
  __syncthreads();   // every thread has read seq_lens[b]
  if (threadIdx.x == 0) seq_lens[b] = (int32_t)(L + 1);
}

}  // namespace dattn
