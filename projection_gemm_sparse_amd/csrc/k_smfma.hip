// k_smfma.hip -- small-M matrix-core kernel instantiations (bf16, gate/up
// and block-scaled weights).
#include "kernels.h"
#include "smfma.hpp"
#include "../../include/fusedproj.h"

namespace {

// Two token halves: up to 12 tokens the loads of each step go in turn
// (first half, weights, second half), above that every activation first.
constexpr int kSmfmaInterleaveMaxM = 12;

template <int KT>
const void* smfma_kt(bool pairs, int mt, int64_t M, int tt) {
  if (tt == 2) {
    if (pairs || mt > 16) return nullptr;
    if (mt == 16)
      return M <= kSmfmaInterleaveMaxM
                 ? reinterpret_cast<const void*>(&fp::smfma_kernel<KT, false, 2, false, 2>)
                 : reinterpret_cast<const void*>(&fp::smfma_kernel<KT, false, 2, true, 2>);
    return reinterpret_cast<const void*>(&fp::smfma_kernel<KT, false, 1, true, 2>);
  }
  if (tt != 1) return nullptr;
  if (mt == 24)
    return pairs ? nullptr : reinterpret_cast<const void*>(&fp::smfma_kernel<KT, false, 3>);
  if (mt == 16) {
    if (pairs) return nullptr;
    return M <= kSmfmaInterleaveMaxM
               ? reinterpret_cast<const void*>(&fp::smfma_kernel<KT, false, 2, false>)
               : reinterpret_cast<const void*>(&fp::smfma_kernel<KT, false, 2>);
  }
  return pairs ? reinterpret_cast<const void*>(&fp::smfma_kernel<KT, true>)
               : reinterpret_cast<const void*>(&fp::smfma_kernel<KT, false>);
}

template <int FMT, int MH>
const void* smfma_mx_kt(int kt) {
  switch (kt) {
    case 4: return reinterpret_cast<const void*>(&fp::smfma_mx_kernel<4, FMT, MH>);
    case 8: return reinterpret_cast<const void*>(&fp::smfma_mx_kernel<8, FMT, MH>);
    case 16: return reinterpret_cast<const void*>(&fp::smfma_mx_kernel<16, FMT, MH>);
    default: return nullptr;
  }
}

template <int MH>
const void* smfma_mx_fmt(int32_t dtype, int kt) {
  return dtype == FP_MXFP8   ? smfma_mx_kt<8, MH>(kt)
         : dtype == FP_MXFP4 ? smfma_mx_kt<4, MH>(kt)
         : dtype == FP_NVFP4 ? smfma_mx_kt<fp::kFmtNv4, MH>(kt)
                             : nullptr;
}

}  // namespace

namespace fpk {

const void* smfma(int kt, bool pairs, int mt, int64_t M, int tt) {
  switch (kt) {
    case 4: return smfma_kt<4>(pairs, mt, M, tt);
    case 8: return smfma_kt<8>(pairs, mt, M, tt);
    case 16: return smfma_kt<16>(pairs, mt, M, tt);
    default: return nullptr;
  }
}

const void* smfma_mx(int32_t dtype, int mh, int kt) {
  return mh == 1 ? smfma_mx_fmt<1>(dtype, kt) : mh == 2 ? smfma_mx_fmt<2>(dtype, kt) : nullptr;
}

}  // namespace fpk
