// kernel_table.h -- host handles of the split kernels.  The instances of
// one (head_dim, softcap) pair live in their own translation unit
// (kernels.hip built with -DDATTN_D and -DDATTN_CAP) so that the four units
// compile in parallel.
#pragma once

namespace dattn {

enum SplitKind : int {
  kPagedF16 = 0,   // static splits, paged f16 cache
  kPagedF32,       // static splits, paged f32 cache
  kTiered,         // static splits, int8 cold pool + f16 hot ring
  kSparse,         // static splits over the CSR union, paged f16 cache
  kBalF16,         // balanced schedule, paged f16
  kBalF32,         // balanced schedule, paged f32
  kBalTiered,      // balanced schedule, tiered
  kTieredF16,      // static splits, f16 cold pool + f16 hot ring
  kBalTieredF16,   // balanced schedule, tiered f16
  kPagedF16MQ,     // static splits, paged f16, several queries per sequence (G = 16 columns)
  kPagedF32MQ,
  kBalF16MQ,       // balanced schedule, the same
  kBalF32MQ,
  kTieredMQ,       // static splits, tiered int8, several queries per sequence
  kTieredF16MQ,    // static splits, tiered f16 / window ring, several queries per sequence
  kBalTieredMQ,    // balanced schedule, the same
  kBalTieredF16MQ,
  kSparseMQ,       // static splits over the CSR union, several queries per sequence
  kTieredW,        // static splits, tiered int8, scales gathered as 4-byte words (even Hkv, aligned scales)
  kBalTieredW,     // balanced schedule, the same
};

// Split kernel for (kind, GQA group G in {1, 2, 4, 8}, contiguous 16-row
// tiles); the multi-query kinds take G = 16.  nullptr for an unknown pair.
void* split_kernel_d64_cap0(int kind, int G, bool contig);
void* split_kernel_d64_cap1(int kind, int G, bool contig);
void* split_kernel_d128_cap0(int kind, int G, bool contig);
void* split_kernel_d128_cap1(int kind, int G, bool contig);

inline void* split_kernel(int kind, int D, bool cap, int G, bool contig) {
  if (D == 64) return cap ? split_kernel_d64_cap1(kind, G, contig) : split_kernel_d64_cap0(kind, G, contig);
  return cap ? split_kernel_d128_cap1(kind, G, contig) : split_kernel_d128_cap0(kind, G, contig);
}

// Multi-query kernels (kPagedF16MQ, kBalF16MQ, kTieredMQ, kTieredF16MQ,
// kBalTieredMQ, kBalTieredF16MQ) for contiguous tiles whose rbk in {2, 4, 8}
// row-block waves per kv head share each tile through LDS (2 * 64 * D bytes
// at the start of dynamic LDS).  nullptr for other kinds.
void* shared_kernel_d64_cap0(int kind, int rbk);
void* shared_kernel_d64_cap1(int kind, int rbk);
void* shared_kernel_d128_cap0(int kind, int rbk);
void* shared_kernel_d128_cap1(int kind, int rbk);

inline void* shared_kernel(int kind, int D, bool cap, int rbk) {
  if (D == 64) return cap ? shared_kernel_d64_cap1(kind, rbk) : shared_kernel_d64_cap0(kind, rbk);
  return cap ? shared_kernel_d128_cap1(kind, rbk) : shared_kernel_d128_cap0(kind, rbk);
}

}  // namespace dattn
