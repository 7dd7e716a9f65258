// Device helpers shared by the CDB kernels (gfx950, wave64).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));

// Raw storage of one bfloat16 value.
struct bf16_t {
  uint16_t u;
};

__device__ __forceinline__ float bf16_to_f32(uint16_t u) {
  return __builtin_bit_cast(float, (uint32_t)u << 16);
}

// Round to nearest, ties to even; NaN stays a quiet NaN.
// Two floats to packed bf16 (lo in bits 0..15) with the hardware conversion
// (v_cvt_pk_bf16_f32, round to nearest even): one instruction where
// f32_to_bf16 below takes five; the same bits for every non-NaN input.
typedef __bf16 bf16x2v_t __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint32_t cvt_bf16x2(float lo, float hi) {
  const bf16x2v_t v = {(__bf16)lo, (__bf16)hi};
  return __builtin_bit_cast(uint32_t, v);
}

__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
  uint32_t u = __builtin_bit_cast(uint32_t, f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return (uint16_t)((u >> 16) | 0x40u);
  u += 0x7fffu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

// Element traits: how one 16-byte load maps to MFMA operands.
//  bf16: 8 elements per 16 B; one v_mfma_f32_16x16x32_bf16 per fragment
//        pair (lane l holds row l%16, k = 8*(l/16) .. +8 of a 32-wide step).
//  f32:  4 elements per 16 B; four v_mfma_f32_16x16x4_f32 per fragment
//        pair, MFMA i using element i (k = 4*(l/16) + i of a 16-wide step).
// Both produce the same 16x16 accumulator layout: lane l holds rows
// 4*(l/16) .. +4 of column l%16.
template <typename T> struct Elt;
template <> struct Elt<float> {
  typedef float raw;
  static constexpr int VEC = 4;
  static constexpr int KSTEP = 16;
  __device__ static __forceinline__ float to_f32(float v) { return v; }
  __device__ static __forceinline__ float from_f32(float v) { return v; }
  __device__ static __forceinline__ void mma(f32x4_t& acc, const uint4& a, const uint4& b) {
    acc = __builtin_amdgcn_mfma_f32_16x16x4f32(__builtin_bit_cast(float, a.x), __builtin_bit_cast(float, b.x), acc, 0, 0, 0);
    acc = __builtin_amdgcn_mfma_f32_16x16x4f32(__builtin_bit_cast(float, a.y), __builtin_bit_cast(float, b.y), acc, 0, 0, 0);
    acc = __builtin_amdgcn_mfma_f32_16x16x4f32(__builtin_bit_cast(float, a.z), __builtin_bit_cast(float, b.z), acc, 0, 0, 0);
    acc = __builtin_amdgcn_mfma_f32_16x16x4f32(__builtin_bit_cast(float, a.w), __builtin_bit_cast(float, b.w), acc, 0, 0, 0);
  }
};
template <> struct Elt<bf16_t> {
  typedef uint16_t raw;
  static constexpr int VEC = 8;
  static constexpr int KSTEP = 32;
  __device__ static __forceinline__ float to_f32(uint16_t v) { return bf16_to_f32(v); }
  __device__ static __forceinline__ uint16_t from_f32(float v) { return f32_to_bf16(v); }
  __device__ static __forceinline__ void mma(f32x4_t& acc, const uint4& a, const uint4& b) {
    acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, a), __builtin_bit_cast(bf16x8_t, b), acc, 0, 0, 0);
  }
};

// 16-byte load through a global-address-space pointer: a plain global load
// (counted on the vector-memory counter only), never a flat one.
__device__ __forceinline__ uint4 ldg_u4(const void* p) {
  typedef uint32_t u32x4_ld __attribute__((ext_vector_type(4)));
  const u32x4_ld v = *(const __attribute__((address_space(1))) u32x4_ld*)p;
  return make_uint4(v.x, v.y, v.z, v.w);
}

// 16-byte non-temporal load: for data read once per step and far larger
// than the caches (the KV stream of decode attention), so it does not
// displace reusable lines.
__device__ __forceinline__ uint4 ldg_nt_u4(const void* p) {
  typedef uint32_t u32x4_ld __attribute__((ext_vector_type(4)));
  const u32x4_ld v = __builtin_nontemporal_load((const __attribute__((address_space(1))) u32x4_ld*)p);
  return make_uint4(v.x, v.y, v.z, v.w);
}

// Sum of p[s * stride] for s = 0 .. n-1, added in that order (so the result
// is the plain sequential sum), with the loads issued eight at a time: the
// split-K partials of one element are independent, and a one-at-a-time loop
// would wait a full memory round trip per split.
template <int R = 8>
__device__ __forceinline__ float sum_splits(const float* p, long stride, int n) {
  float v = 0.f;
  for (int s = 0; s < n; s += R) {
    float t[R];
#pragma unroll
    for (int u = 0; u < R; u++) t[u] = p[(long)min(s + u, n - 1) * stride];
#pragma unroll
    for (int u = 0; u < R; u++)
      if (s + u < n) v += t[u];
  }
  return v;
}

// Unpack a 16-byte vector of VEC elements into floats.
__device__ __forceinline__ void unpack16(const uint4& v, float* out, float) {
  out[0] = __builtin_bit_cast(float, v.x);
  out[1] = __builtin_bit_cast(float, v.y);
  out[2] = __builtin_bit_cast(float, v.z);
  out[3] = __builtin_bit_cast(float, v.w);
}
__device__ __forceinline__ void unpack16(const uint4& v, float* out, bf16_t) {
  const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
  for (int i = 0; i < 4; i++) {
    out[2 * i] = __builtin_bit_cast(float, w[i] << 16);
    out[2 * i + 1] = __builtin_bit_cast(float, w[i] & 0xffff0000u);
  }
}

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
  return v;
}

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, 64));
  return v;
}

// Sum over a 256-thread block; every thread gets the result.  `red` needs 4
// floats of LDS.  Fixed order, so the result is deterministic.
__device__ __forceinline__ float block_sum256(float v, float* red) {
  v = wave_sum(v);
  const int w = threadIdx.x >> 6;
  __syncthreads();
  if ((threadIdx.x & 63) == 0) red[w] = v;
  __syncthreads();
  return (red[0] + red[1]) + (red[2] + red[3]);
}

__device__ __forceinline__ float silu_f(float z) { return z / (1.0f + __expf(-z)); }

__device__ __forceinline__ int ld_nvalid(const int* p, int dflt) { return p ? *p : dflt; }

// Fragment-packed activations, the A-operand layout of the decode GEMMs
// (rows <= 64): an [rows][K] matrix stored as tiles of 16 rows x one MFMA
// k-step (KS columns), tile (row tile, k-step) holding 64 pieces of VEC
// elements where piece l is row l % 16, columns (l / 16) * VEC .. + VEC --
// exactly one lane's operand, so a wave reads a tile as one contiguous
// kilobyte.  Element offset of (m, k):
template <typename T>
__device__ __forceinline__ long apack_off(int m, int k, int K) {
  constexpr int VEC = Elt<T>::VEC, KS = Elt<T>::KSTEP;
  const int ks = k / KS, kin = k - ks * KS;
  return ((long)((m >> 4) * (K / KS) + ks) * 64 + (m & 15) + 16 * (kin / VEC)) * VEC + (kin % VEC);
}

// Sum over the 16 lanes of a row (lanes 16k .. 16k+15), result in every lane:
// DPP quad_perm [1,0,3,2] and [2,3,0,1] sum each quad, row_half_mirror adds
// the mirrored quad of the same 8 lanes, row_mirror the mirrored 8 lanes
// (each step adds a pair in both orders, so all 16 lanes hold the same bits).
__device__ __forceinline__ float sum16(float v) {
  v += __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, v), 0xB1, 0xF, 0xF, false));
  v += __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, v), 0x4E, 0xF, 0xF, false));
  v += __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, v), 0x141, 0xF, 0xF, false));
  v += __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, v), 0x140, 0xF, 0xF, false));
  return v;
}

// Sum over the wave in a fixed order: each 16-lane row by DPP, then the four
// rows' sums read out as scalars and added in row order -- the same value in
// every lane, without the LDS round trips of cross-row shuffles.
__device__ __forceinline__ float wave_sum_dpp(float v) {
  const int t = __builtin_bit_cast(int, sum16(v));
  const float r0 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(t, 0));
  const float r1 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(t, 16));
  const float r2 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(t, 32));
  const float r3 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(t, 48));
  return ((r0 + r1) + r2) + r3;
}

// Deferred RMSNorm scale.  A residual projection that completes the
// residual stream also writes, per row, the sums of x^2 over each group of
// 8 outputs (ss[m][0..n)); the consumer of the unscaled input g * x
// multiplies its own outputs by 1 / sqrt(sum / H + eps), which is the norm's
// 1 / rms(x) since a GEMM is linear in each row.  The wave-wide form: lane l
// adds parts l, l + 64, ... (n <= 256, all four loads issued at once), then
// wave_sum_dpp.
__device__ __forceinline__ float rstd_from_parts_wave(const float* ss, int n, int m, int H, float eps) {
  const int lane = threadIdx.x & 63;
  float v[4];
#pragma unroll
  for (int u = 0; u < 4; u++) v[u] = lane + 64 * u < n ? ss[(long)m * n + lane + 64 * u] : 0.f;
  const float s = wave_sum_dpp(((v[0] + v[1]) + v[2]) + v[3]);
  return 1.0f / sqrtf(s / (float)H + eps);
}

__device__ __forceinline__ float ld_f32(float v) { return v; }
__device__ __forceinline__ float ld_f32(uint16_t v) { return bf16_to_f32(v); }

// Device-side descriptor errors.  Indices read from device memory (slots,
// sequence ids, positions, depths, block ids, token ids) and device row
// counts are clamped into their buffers so every access stays in bounds; a
// kernel that had to clamp also sets one of these bits in the context's
// error word, which cdb_sync reports (and clears) as CDB_EINVAL.
enum { ERR_SLOT = 1, ERR_SEQ = 2, ERR_POS = 4, ERR_DEPTH = 8, ERR_BLOCK = 16, ERR_TOKEN = 32, ERR_COUNT = 64 };

__device__ __forceinline__ void flag_err(int* err, int bit) {
  if (err) atomicOr(err, bit);
}

// v clamped into [lo, hi]; a value outside sets `bit` in *err.
__device__ __forceinline__ int clamp_chk(int v, int lo, int hi, int* err, int bit) {
  if (v < lo || v > hi) {
    flag_err(err, bit);
    v = v < lo ? lo : hi;
  }
  return v;
}
