// kernels.hip -- the split-kernel instances of one (head_dim, softcap) pair,
// chosen with -DDATTN_D=<64|128> -DDATTN_CAP=<0|1>; with -DDATTN_SHARED=1 the
// multi-query instances whose row-block waves share tiles through LDS.
#include "decode_kernels.h"
#include "kernel_table.h"

#if !defined(DATTN_D) || !defined(DATTN_CAP)
#error "kernels.hip is built with -DDATTN_D=<64|128> -DDATTN_CAP=<0|1>"
#endif

namespace dattn {
namespace {

#if !DATTN_SHARED
template <int G, bool FM>
void* instance(int kind) {
  constexpr int D = DATTN_D;
  constexpr bool CAP = DATTN_CAP != 0;
  if constexpr (G == 16) {   // multi-query kinds only
    switch (kind) {
      case kPagedF16MQ: return (void*)&paged_split_kernel<D, 16, CAP, _Float16, FM, true>;
      case kPagedF32MQ: return (void*)&paged_split_kernel<D, 16, CAP, float, FM, true>;
      case kBalF16MQ: return (void*)&balanced_kernel<D, 16, CAP, 4, FM>;
      case kBalF32MQ: return (void*)&balanced_kernel<D, 16, CAP, 5, FM>;
      case kTieredMQ: return (void*)&tiered_split_kernel<D, 16, CAP, FM, false, true>;
      case kTieredF16MQ: return (void*)&tiered_split_kernel<D, 16, CAP, FM, true, true>;
      case kBalTieredMQ: return (void*)&balanced_kernel<D, 16, CAP, 6, FM>;
      case kBalTieredF16MQ: return (void*)&balanced_kernel<D, 16, CAP, 7, FM>;
      case kSparseMQ: return (void*)&sparse_split_kernel<D, 16, CAP, FM, true>;
      default: return nullptr;
    }
  } else {
    switch (kind) {
      case kPagedF16: return (void*)&paged_split_kernel<D, G, CAP, _Float16, FM>;
      case kPagedF32: return (void*)&paged_split_kernel<D, G, CAP, float, FM>;
      case kTiered: return (void*)&tiered_split_kernel<D, G, CAP, FM, false>;
      case kTieredF16: return (void*)&tiered_split_kernel<D, G, CAP, FM, true>;
      case kSparse: return (void*)&sparse_split_kernel<D, G, CAP, FM>;
      case kBalF16: return (void*)&balanced_kernel<D, G, CAP, 0, FM>;
      case kBalF32: return (void*)&balanced_kernel<D, G, CAP, 1, FM>;
      case kBalTiered: return (void*)&balanced_kernel<D, G, CAP, 2, FM>;
      case kBalTieredF16: return (void*)&balanced_kernel<D, G, CAP, 3, FM>;
      case kTieredW: return (void*)&tiered_split_kernel<D, G, CAP, FM, false, false, 1, true>;
      case kBalTieredW: return (void*)&balanced_kernel<D, G, CAP, 8, FM>;
      default: return nullptr;
    }
  }
}

#endif

#if DATTN_SHARED
// Multi-query kinds over contiguous tiles whose RBK row-block waves per kv
// head share each tile through LDS.
template <int RBK>
void* shared_instance(int kind) {
  constexpr int D = DATTN_D;
  constexpr bool CAP = DATTN_CAP != 0;
  switch (kind) {
    case kPagedF16MQ: return (void*)&paged_split_kernel<D, 16, CAP, _Float16, true, true, RBK>;
    case kBalF16MQ: return (void*)&balanced_kernel<D, 16, CAP, 4, true, RBK>;
    case kTieredMQ: return (void*)&tiered_split_kernel<D, 16, CAP, true, false, true, RBK>;
    case kTieredF16MQ: return (void*)&tiered_split_kernel<D, 16, CAP, true, true, true, RBK>;
    case kBalTieredMQ: return (void*)&balanced_kernel<D, 16, CAP, 6, true, RBK>;
    case kBalTieredF16MQ: return (void*)&balanced_kernel<D, 16, CAP, 7, true, RBK>;
    default: return nullptr;
  }
}
#else
template <bool FM>
void* by_group(int kind, int G) {
  switch (G) {
    case 1: return instance<1, FM>(kind);
    case 2: return instance<2, FM>(kind);
    case 4: return instance<4, FM>(kind);
    case 8: return instance<8, FM>(kind);
    case 16: return instance<16, FM>(kind);
    default: return nullptr;
  }
}

#endif

}  // namespace

#if DATTN_SHARED
#define DATTN_NAME2(d, c) shared_kernel_d##d##_cap##c
#define DATTN_NAME(d, c) DATTN_NAME2(d, c)

void* DATTN_NAME(DATTN_D, DATTN_CAP)(int kind, int rbk) {
  switch (rbk) {
    case 2: return shared_instance<2>(kind);
    case 4: return shared_instance<4>(kind);
    case 8: return shared_instance<8>(kind);
    default: return nullptr;
  }
}
#else
#define DATTN_NAME2(d, c) split_kernel_d##d##_cap##c
#define DATTN_NAME(d, c) DATTN_NAME2(d, c)

void* DATTN_NAME(DATTN_D, DATTN_CAP)(int kind, int G, bool contig) {
  return contig ? by_group<true>(kind, G) : by_group<false>(kind, G);
}
#endif

}  // namespace dattn
