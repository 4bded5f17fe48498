// Device helpers shared by the GEMMs that read a frozen weight: the absmax of
// the 64-element block holding a given element, for both NF4 storages.
#pragma once
#include "common.h"
#include "kernels.h"

namespace lsf {

// NF4_DQ: 8-bit code times the group's scale plus the group's offset (groups
// of 256 blocks).
__device__ __forceinline__ float dq_absmax(const WeightRef& w, int64_t block) {
  const float2 so = reinterpret_cast<const float2*>(w.dq2)[block >> 8];
  return dq_absmax_value(w.absq[block], so.x, so.y);
}

__device__ __forceinline__ float block_absmax(const WeightRef& w, int64_t elem) {
  const int64_t b = elem >> 6;
  return (w.fmt == FMT_NF4_DQ) ? dq_absmax(w, b) : w.absmax[b];
}

// The same with the storage known at compile time.
template <int FMT>
__device__ __forceinline__ float block_absmax_t(const WeightRef& w, int64_t elem) {
  const int64_t b = elem >> 6;
  if constexpr (FMT == FMT_NF4_DQ) return dq_absmax(w, b);
  else return w.absmax[b];
}

}  // namespace lsf
