// LDS-tiled MFMA GEMM for many rows: C[M][N] = A[M][K] . W[N][K]^T in bf16
// with fp32 accumulation (prefill chunks of up to thousands of tokens, large
// decode batches).  Above a few hundred rows the projections stop being
// weight-streaming and become dense contractions, so here operand reuse is
// what matters:
//  - one workgroup (4 waves, 2 x 2) owns a BM x BN output tile; each k-tile of
//    64 is copied once from global memory into LDS (16-byte loads: A in rows
//    of 128 contiguous bytes, W as whole one-kilobyte fragment-packed tiles)
//    and read from there by the waves as MFMA fragments, so every A byte is
//    fetched once per N-tile and every W byte once per M-tile;
//  - LDS is double-buffered and the next k-tile's global loads are in flight
//    in registers while the MFMAs of the current one run: one barrier per
//    k-tile;
//  - LDS rows are padded by 16 bytes so the 16-byte fragment reads of eight
//    consecutive rows fall in distinct banks;
//  - tiles are ordered so that each XCD (blockIdx % 8) takes a contiguous
//    range of tiles, walked in groups of 8 M-tiles with M fastest: the
//    workgroups resident on one XCD at a time share their A and W tiles in
//    that XCD's L2;
//  - epilogues from registers: store fp32 / bf16, residual add into the fp32
//    stream through the slot table, and SwiGLU, for which each wave's column
//    fragments are laid out as gate columns followed by the up columns of
//    the same outputs, so silu(gate) * up is formed without any exchange.
// K must be a multiple of 32; a final half k-tile is zero-filled.
#include "common.h"
#include "kernels.h"

namespace cdb {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

// 16-byte load through a global-address-space pointer (a plain global load,
// not a flat one, so it only counts against the vector-memory counter)
__device__ __forceinline__ u32x4 ldg16(const uint16_t* p) {
  return *(const __attribute__((address_space(1))) u32x4*)p;
}

template <int BM, int BN, int WM, int WN, int EPI>
__global__ __launch_bounds__(256) void k_gemm_tiled(GemmArgs g) {
  constexpr int BK = 64, LDK = BK + 8;
  constexpr int WAVES_N = BN / WN;
  constexpr int FM = WM / 16, FN = WN / 16;
  constexpr int A_CH = BM * (BK / 8) / 256;      // 16-byte chunks per thread per k-tile
  constexpr int B_CH = BN * (BK / 8) / 256;
  constexpr bool SWI = (EPI == EPI_SWIGLU);
  constexpr int OUT_BN = SWI ? BN / 2 : BN;
  static_assert((BM / WM) * (BN / WN) == 4, "four waves");
  static_assert(!SWI || (FN % 2 == 0), "SwiGLU pairs column fragments");
  __shared__ __align__(16) uint16_t As[2][BM * LDK];
  __shared__ __align__(16) uint16_t Bs[2][BN * LDK];

  const int m_valid = min(ld_nvalid(g.n_valid, g.M), g.M);
  const int n_tiles = (g.N + OUT_BN - 1) / OUT_BN;
  const int m_tiles = g.m_tiles;
  const int total = m_tiles * n_tiles;
  int vid = blockIdx.x;
  if ((total & 7) == 0) vid = (blockIdx.x & 7) * (total >> 3) + (blockIdx.x >> 3);
  constexpr int GM = 8;
  const int grp = vid / (GM * n_tiles);
  const int first_m = grp * GM;
  const int gsz = min(GM, m_tiles - first_m);
  const int in = vid - grp * GM * n_tiles;
  const int m_tile = first_m + in % gsz;
  const int n_tile = in / gsz;
  const int m0 = m_tile * BM;
  if (m0 >= m_valid) return;                     // uniform per workgroup

  const int tid = threadIdx.x;
  const int lane = tid & 63, w = tid >> 6;
  const int r16 = lane & 15, g4 = lane >> 4;
  const int wm0 = (w / WAVES_N) * WM, wn0 = (w % WAVES_N) * WN;

  const uint16_t* A = (const uint16_t*)g.A;
  const uint16_t* W = (const uint16_t*)g.W;
  // chunk i of this thread: tile row (tid / 8) + 32 i, k offset 8 (tid % 8)
  const int kc = (tid & 7) * 8;
  long a_off[A_CH];
#pragma unroll
  for (int i = 0; i < A_CH; i++) {
    const int m = min(m0 + (tid >> 3) + 32 * i, g.M - 1);
    a_off[i] = (long)m * g.lda + kc;
  }
  // W tile from the fragment-packed weights: the BN x 64 tile is BN/16 row
  // tiles x 2 k-steps of one-kilobyte packed tiles; chunk i of this thread is
  // piece (tid % 64) of packed tile (tid / 64) + 4 i, so each wave reads one
  // packed tile contiguously.  Packed tile t -> virtual row tile t / 2,
  // k-step t % 2; piece p -> LDS row 16 (t / 2) + p % 16, column
  // 32 (t % 2) + 8 (p / 16).
  const int ksteps = g.K / 32;
  long b_off[B_CH];
  int b_lds[B_CH], b_ks[B_CH];
#pragma unroll
  for (int i = 0; i < B_CH; i++) {
    const int t = (tid >> 6) + 4 * i, piece = tid & 63;
    const int vt = t >> 1, ks = t & 1;              // virtual row tile, k-step within the k-tile
    int wt;                                          // weight row tile
    if (SWI) {
      const int wn = (16 * vt) / WN, j = ((16 * vt) % WN) / 16;
      const int outt = ((n_tile * OUT_BN + wn * (WN / 2)) >> 4) + (j % (FN / 2));
      wt = min(outt, (g.N - 1) >> 4) + (j >= FN / 2 ? (g.up_off >> 4) : 0);
    } else {
      wt = min(((n_tile * BN) >> 4) + vt, (g.N - 1) >> 4);
    }
    b_off[i] = ((long)wt * ksteps * 64 + piece) * 8;
    b_ks[i] = ks;
    b_lds[i] = (16 * vt + (piece & 15)) * LDK + 32 * ks + 8 * (piece >> 4);
  }

  f32x4_t acc[FM][FN];
#pragma unroll
  for (int i = 0; i < FM; i++)
#pragma unroll
    for (int j = 0; j < FN; j++) acc[i][j] = (f32x4_t){0.f, 0.f, 0.f, 0.f};

  // Global loads of k-tile kt into registers.  A half k-tile at the end of
  // K (K % 64 == 32) reads the previous 32 columns (A) or the previous
  // k-step (W) instead, and those chunks are stored to LDS as zeros (the
  // choice is made at the store, after the loads have landed, so the loads
  // stay in flight).
  u32x4 ra[A_CH], rb[B_CH];
  uint32_t amask = ~0u, bmask[B_CH];
#define CDB_TILE_LOAD(kt)                                                        \
  {                                                                              \
    const int k0_ = (kt) * BK;                                                   \
    const bool kin_ = k0_ + kc < g.K;                                            \
    amask = kin_ ? ~0u : 0u;                                                     \
    const int kk_ = kin_ ? k0_ : k0_ - 32;                                       \
    _Pragma("unroll") for (int i = 0; i < A_CH; i++)                             \
      ra[i] = ldg16(A + a_off[i] + kk_);                                         \
    _Pragma("unroll") for (int i = 0; i < B_CH; i++) {                           \
      const int st_ = 2 * (kt) + b_ks[i];                                        \
      bmask[i] = st_ < ksteps ? ~0u : 0u;                                        \
      rb[i] = ldg16(W + b_off[i] + (long)min(st_, ksteps - 1) * 512);            \
    }                                                                            \
    __builtin_amdgcn_sched_barrier(0);                                           \
  }
#define CDB_TILE_STORE(buf)                                                      \
  {                                                                              \
    _Pragma("unroll") for (int i = 0; i < A_CH; i++)                             \
      *(u32x4*)&As[buf][((tid >> 3) + 32 * i) * LDK + kc] = ra[i] & amask;       \
    _Pragma("unroll") for (int i = 0; i < B_CH; i++)                             \
      *(u32x4*)&Bs[buf][b_lds[i]] = rb[i] & bmask[i];                            \
  }

  const int nk = (g.K + BK - 1) / BK;
  CDB_TILE_LOAD(0);
  CDB_TILE_STORE(0);
  __syncthreads();
  for (int kt = 0; kt < nk; kt++) {
    const int buf = kt & 1;
    const bool more = kt + 1 < nk;
    CDB_TILE_LOAD(more ? kt + 1 : kt);           // last iteration: a harmless reload
#pragma unroll
    for (int s = 0; s < BK / 32; s++) {
      const int koff = 32 * s + 8 * g4;
      bf16x8_t af[FM], bfr[FN];
#pragma unroll
      for (int i = 0; i < FM; i++) af[i] = *(const bf16x8_t*)&As[buf][(wm0 + 16 * i + r16) * LDK + koff];
#pragma unroll
      for (int j = 0; j < FN; j++) bfr[j] = *(const bf16x8_t*)&Bs[buf][(wn0 + 16 * j + r16) * LDK + koff];
#pragma unroll
      for (int i = 0; i < FM; i++)
#pragma unroll
        for (int j = 0; j < FN; j++)
          acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af[i], bfr[j], acc[i][j], 0, 0, 0);
    }
    if (more) CDB_TILE_STORE(buf ^ 1);
    __syncthreads();
  }
#undef CDB_TILE_LOAD
#undef CDB_TILE_STORE

  // ---- epilogues: lane holds rows 4*g4 + r of column r16 of each fragment ----
  if (SWI) {
#pragma unroll
    for (int i = 0; i < FM; i++)
#pragma unroll
      for (int j = 0; j < FN / 2; j++)
#pragma unroll
        for (int r = 0; r < 4; r++) {
          const int m = m0 + wm0 + 16 * i + 4 * g4 + r;
          const int n = n_tile * OUT_BN + (wn0 / 2) + 16 * j + r16;
          if (m >= m_valid || n >= g.N) continue;
          const float gt = acc[i][j][r], up = acc[i][j + FN / 2][r];
          ((uint16_t*)g.C)[(long)m * g.ldc + n] = f32_to_bf16(silu_f(gt) * up);
        }
  } else {
#pragma unroll
    for (int i = 0; i < FM; i++)
#pragma unroll
      for (int j = 0; j < FN; j++)
#pragma unroll
        for (int r = 0; r < 4; r++) {
          const int m = m0 + wm0 + 16 * i + 4 * g4 + r;
          const int n = n_tile * BN + wn0 + 16 * j + r16;
          if (m >= m_valid || n >= g.N) continue;
          const float v = acc[i][j][r];
          if (EPI == EPI_STORE_F32) {
            ((float*)g.C)[(long)m * g.ldc + n] = v;
          } else if (EPI == EPI_STORE_T) {
            ((uint16_t*)g.C)[(long)m * g.ldc + n] = f32_to_bf16(v);
          } else {  // EPI_RESID
            const int rr = g.slot ? min(max(g.slot[m], 0), g.slot_max - 1) : m;
            float* dst = (float*)g.C + (long)rr * g.ldc + n;
            *dst = *dst + v;
          }
        }
  }
}

template <int BM, int BN, int WM, int WN, int EPI>
static int tiled_one(GemmArgs g, hipStream_t st) {
  constexpr int OUT_BN = (EPI == EPI_SWIGLU) ? BN / 2 : BN;
  g.m_tiles = (g.M + BM - 1) / BM;
  const int n_tiles = (g.N + OUT_BN - 1) / OUT_BN;
  hipLaunchKernelGGL((k_gemm_tiled<BM, BN, WM, WN, EPI>), dim3(g.m_tiles * n_tiles), dim3(256), 0, st, g);
  return hipGetLastError() == hipSuccess ? 0 : -1;
}

template <int BM, int BN, int WM, int WN>
static int tiled_epi(int epi, const GemmArgs& g, hipStream_t st) {
  switch (epi) {
    case EPI_STORE_F32: return tiled_one<BM, BN, WM, WN, EPI_STORE_F32>(g, st);
    case EPI_STORE_T: return tiled_one<BM, BN, WM, WN, EPI_STORE_T>(g, st);
    case EPI_RESID: return tiled_one<BM, BN, WM, WN, EPI_RESID>(g, st);
    case EPI_SWIGLU: return tiled_one<BM, BN, WM, WN, EPI_SWIGLU>(g, st);
    default: return -2;
  }
}

bool gemm_tiled_supported(int dtype, int epi) {
  return dtype == 1 && (epi == EPI_STORE_F32 || epi == EPI_STORE_T || epi == EPI_RESID || epi == EPI_SWIGLU);
}

// 128 x 128 tiles, waves of 64 x 64 (two workgroups per CU).  Measured on
// MI355X at 8192 rows, this beat 256 x 128 tiles with 128 x 64 waves (one
// workgroup per CU) on every projection shape of the Ouro-like core.
int gemm_tiled_launch(int epi, const GemmArgs& g, hipStream_t st) {
  if (g.K % 32 || g.M <= 0 || g.N <= 0) return -2;
  return tiled_epi<128, 128, 64, 64>(epi, g, st);
}

}  // namespace cdb
