// Device helpers shared by the attention kernels (decode and prefill).
#pragma once
#include "common.h"

namespace cdb {

// Sum over the 16 lanes of a row (lanes 16k .. 16k+15), result in every lane:
// DPP quad_perm [1,0,3,2] and [2,3,0,1] sum each quad, row_half_mirror adds
// the mirrored quad of the same 8 lanes, row_mirror the mirrored 8 lanes.
__device__ __forceinline__ float sum16(float v) {
  v += __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, v), 0xB1, 0xF, 0xF, false));
  v += __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, v), 0x4E, 0xF, 0xF, false));
  v += __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, v), 0x141, 0xF, 0xF, false));
  v += __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, v), 0x140, 0xF, 0xF, false));
  return v;
}

// Sum of the split partials of one projection output element.
__device__ __forceinline__ float qkv_at(const float* qkv, int sk, int rows, int ld, int b, int col) {
  return sum_splits(qkv + (long)b * ld + col, (long)rows * ld, sk);
}

}  // namespace cdb
