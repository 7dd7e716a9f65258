// Device helpers shared by the attention kernels (decode and prefill).
#pragma once
#include "common.h"

namespace cdb {

// Sum of the split partials of one projection output element.
__device__ __forceinline__ float qkv_at(const float* qkv, int sk, int rows, int ld, int b, int col) {
  return sum_splits(qkv + (long)b * ld + col, (long)rows * ld, sk);
}

}  // namespace cdb
