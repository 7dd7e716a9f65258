// LDS-tiled MFMA GEMM for many rows: C[M][N] = A[M][K] . W[N][K]^T in bf16
// with fp32 accumulation (prefill chunks of up to thousands of tokens, large
// decode batches).  Above a few hundred rows the projections stop being
// weight-streaming and become dense contractions, so here operand reuse and
// keeping the matrix cores fed are what matter:
//  - one workgroup (4 waves, 2 x 2 of 64 x 64) owns a 128 x 128 output tile;
//    each k-tile of 64 is copied once from global memory into LDS and read
//    from there by the waves as MFMA fragments, so every A byte is fetched
//    once per N-tile and every W byte once per M-tile;
//  - the copies are direct global -> LDS loads (global_load_lds_dwordx4:
//    lane l of an instruction writes 16 bytes at the instruction's LDS base
//    + 16 l): no register staging, no LDS store instructions.  LDS is double
//    buffered; the next k-tile's loads are in flight while the current one
//    feeds the MFMAs, and each wave waits only for its own previous loads
//    (vmcnt) before the barrier.  The loads are issued from inline assembly
//    and their waits placed by hand, because the compiler cannot tell the
//    two buffers apart and would otherwise wait for every outstanding load;
//  - A sits in LDS row-major, 128 bytes per row, with 16-byte chunk c of
//    row r stored in slot c ^ (r & 7): each lane fetches the global chunk
//    that belongs in its slot (rows stay 128-byte coalesced), and the
//    fragment reads of eight consecutive rows fall in distinct banks;
//  - W is already fragment-packed in memory (one kilobyte per 16 rows x one
//    k-step) and is kept packed in LDS, so a wave's fragment read is one
//    contiguous kilobyte;
//  - tiles are ordered so that each XCD (blockIdx % 8) takes a contiguous
//    range of tiles, walked in groups of 8 M-tiles with M fastest: the
//    workgroups resident on one XCD at a time share their A and W tiles in
//    that XCD's L2;
//  - epilogues from registers: store fp32 / bf16, residual add into the fp32
//    stream through the slot table, and SwiGLU, for which each wave's column
//    fragments are laid out as gate columns followed by the up columns of
//    the same outputs, so silu(gate) * up is formed without any exchange.
// K must be a multiple of 32; a final half k-tile runs one MFMA k-step.
#include "common.h"
#include "kernels.h"

namespace cdb {

typedef __attribute__((address_space(3))) void lds_void;

// Direct 16-byte global -> LDS load: this lane's 16 bytes at gptr go to LDS
// byte offset lds_base + 16 * lane (lds_base wave-uniform, through M0).
// M0 is reserved (it cannot be named as a clobber); the compiler uses it for
// nothing else in this kernel (checked in the generated assembly), and each
// load sets it itself.
__device__ __forceinline__ void lds_dma16(const void* gptr, uint32_t lds_base) {
  asm volatile("s_mov_b32 m0, %1\n\tglobal_load_lds_dwordx4 %0, off" ::"v"(gptr), "s"(lds_base) : "memory");
}

__device__ __forceinline__ uint32_t lds_offset(const void* p) { return (uint32_t)(uintptr_t)(lds_void*)p; }

// s_waitcnt with vmcnt = n and the other counters left alone (gfx9 encoding)
#define CDB_WAIT_VM(n) __builtin_amdgcn_s_waitcnt(0x0F70 | ((n)&15))

template <int EPI>
__global__ __launch_bounds__(256) void k_gemm_tiled(GemmArgs g) {
  constexpr int BM = 128, BN = 128, WM = 64, WN = 64;
  constexpr int FM = WM / 16, FN = WN / 16;
  constexpr bool SWI = (EPI == EPI_SWIGLU);
  constexpr int OUT_BN = SWI ? BN / 2 : BN;
  constexpr int LOADS = 8;                       // direct loads per wave per k-tile (4 A + 4 W)
  __shared__ __align__(16) uint16_t As0[BM * 64], As1[BM * 64];
  __shared__ __align__(16) uint16_t Bs0[16 * 512], Bs1[16 * 512];

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
  const int wm0 = (w >> 1) * WM, wn0 = (w & 1) * WN;
  const int ksteps = g.K / 32;
  const int nk = (g.K + 63) / 64;
  const bool half_last = (g.K & 63) != 0;        // the last k-tile holds one k-step

  const uint16_t* A = (const uint16_t*)g.A;
  const uint16_t* W = (const uint16_t*)g.W;
  // A: instruction i of wave w fills LDS chunks q = (4w + i) * 64 + lane:
  // row q / 8, slot q % 8, holding global chunk (slot ^ (row & 7)).
  const uint16_t* asrc[4];
  int a_chunk[4];
#pragma unroll
  for (int i = 0; i < 4; i++) {
    const int q = (4 * w + i) * 64 + lane, r = q >> 3, c = (q & 7) ^ (r & 7);
    asrc[i] = A + (long)min(m0 + r, g.M - 1) * g.lda;
    a_chunk[i] = c;
  }
  // W: instruction i of wave w copies packed tile t = 4w + i (virtual row tile
  // t / 2, k-step t % 2 of the k-tile), piece `lane`.
  const uint16_t* bsrc[4];
  int b_ks[4];
#pragma unroll
  for (int i = 0; i < 4; i++) {
    const int t = 4 * w + i, vt = t >> 1;
    int wt;
    if (SWI) {
      const int wn = (16 * vt) / WN, j = ((16 * vt) % WN) / 16;
      const int outt = ((n_tile * OUT_BN + wn * (WN / 2)) >> 4) + (j % (FN / 2));
      wt = min(outt, (g.N - 1) >> 4) + (j >= FN / 2 ? (g.up_off >> 4) : 0);
    } else {
      wt = min(((n_tile * BN) >> 4) + vt, (g.N - 1) >> 4);
    }
    bsrc[i] = W + ((long)wt * ksteps * 64 + lane) * 8;
    b_ks[i] = t & 1;
  }

  // k-tile kt into buffers (AS, BS).  Chunks past K (second half of a half
  // k-tile) are loaded from the first half instead: valid memory, never used.
#define CDB_TILE_ISSUE(kt, AS, BS)                                                               \
  {                                                                                              \
    const int k0_ = (kt) * 64;                                                                   \
    _Pragma("unroll") for (int i = 0; i < 4; i++) {                                              \
      const int c_ = (k0_ + a_chunk[i] * 8 < g.K) ? a_chunk[i] : (a_chunk[i] & 3);               \
      lds_dma16(asrc[i] + k0_ + c_ * 8, __builtin_amdgcn_readfirstlane(lds_offset(&AS[(4 * w + i) * 512]))); \
    }                                                                                            \
    _Pragma("unroll") for (int i = 0; i < 4; i++) {                                              \
      const int st_ = min(2 * (kt) + b_ks[i], ksteps - 1);                                       \
      lds_dma16(bsrc[i] + (long)st_ * 512, __builtin_amdgcn_readfirstlane(lds_offset(&BS[(4 * w + i) * 512]))); \
    }                                                                                            \
  }
#define CDB_TILE_COMPUTE(AS, BS, nsub)                                                           \
  _Pragma("unroll") for (int s = 0; s < 2; s++) {                                                \
    if (s < (nsub)) {                                                                            \
      bf16x8_t af[FM], bfr[FN];                                                                  \
      _Pragma("unroll") for (int i = 0; i < FM; i++) {                                           \
        const int r = wm0 + 16 * i + r16, c = 4 * s + g4;                                        \
        af[i] = *(const bf16x8_t*)&AS[r * 64 + ((c ^ (r & 7)) * 8)];                             \
      }                                                                                          \
      _Pragma("unroll") for (int j = 0; j < FN; j++)                                             \
        bfr[j] = *(const bf16x8_t*)&BS[((((wn0 >> 4) + j) * 2) + s) * 512 + lane * 8];           \
      _Pragma("unroll") for (int i = 0; i < FM; i++)                                             \
        _Pragma("unroll") for (int j = 0; j < FN; j++)                                           \
          acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af[i], bfr[j], acc[i][j], 0, 0, 0);\
    }                                                                                            \
  }
#define CDB_TILE_STEP(KT, CA, CB, NA, NB, NSUB)                                                  \
  {                                                                                              \
    if ((KT) + 1 < nk) {                                                                         \
      CDB_TILE_ISSUE((KT) + 1, NA, NB)                                                           \
      CDB_WAIT_VM(LOADS);                        /* this wave's loads of tile KT have landed */  \
    } else {                                                                                     \
      CDB_WAIT_VM(0);                                                                            \
    }                                                                                            \
    __syncthreads();                             /* every wave's loads of tile KT are in LDS */  \
    CDB_TILE_COMPUTE(CA, CB, NSUB)                                                               \
    __syncthreads();                             /* buffers of tile KT free for tile KT + 2 */   \
  }

  f32x4_t acc[FM][FN];
#pragma unroll
  for (int i = 0; i < FM; i++)
#pragma unroll
    for (int j = 0; j < FN; j++) acc[i][j] = (f32x4_t){0.f, 0.f, 0.f, 0.f};

  // Full k-tiles in pairs (buffer 0 then 1), straight-line so that the
  // accumulators keep one register assignment through the loop (a branch on
  // the buffer parity made the compiler copy every accumulator once per
  // k-tile), then at most one more full tile and the final half tile.
  const int nkf = g.K / 64;
  CDB_TILE_ISSUE(0, As0, Bs0)
  int kt = 0;
  for (; kt + 2 <= nkf; kt += 2) {
    CDB_TILE_STEP(kt, As0, Bs0, As1, Bs1, 2)
    CDB_TILE_STEP(kt + 1, As1, Bs1, As0, Bs0, 2)
  }
  if (kt < nkf) {
    CDB_TILE_STEP(kt, As0, Bs0, As1, Bs1, 2)
    if (half_last) CDB_TILE_STEP(kt + 1, As1, Bs1, As0, Bs0, 1)
  } else if (half_last) {
    CDB_TILE_STEP(kt, As0, Bs0, As1, Bs1, 1)
  }
#undef CDB_TILE_ISSUE
#undef CDB_TILE_COMPUTE
#undef CDB_TILE_STEP

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

template <int EPI>
static int tiled_one(GemmArgs g, hipStream_t st) {
  constexpr int OUT_BN = (EPI == EPI_SWIGLU) ? 64 : 128;
  g.m_tiles = (g.M + 127) / 128;
  const int n_tiles = (g.N + OUT_BN - 1) / OUT_BN;
  hipLaunchKernelGGL((k_gemm_tiled<EPI>), dim3(g.m_tiles * n_tiles), dim3(256), 0, st, g);
  return hipGetLastError() == hipSuccess ? 0 : -1;
}

bool gemm_tiled_supported(int dtype, int epi) {
  return dtype == 1 && (epi == EPI_STORE_F32 || epi == EPI_STORE_T || epi == EPI_RESID || epi == EPI_SWIGLU);
}

// 128 x 128 tiles, waves of 64 x 64 (two workgroups per CU).
int gemm_tiled_launch(int epi, const GemmArgs& g, hipStream_t st) {
  if (g.K % 32 || g.M <= 0 || g.N <= 0 || g.N % 16 || (epi == EPI_SWIGLU && g.up_off % 16)) return -2;
  switch (epi) {
    case EPI_STORE_F32: return tiled_one<EPI_STORE_F32>(g, st);
    case EPI_STORE_T: return tiled_one<EPI_STORE_T>(g, st);
    case EPI_RESID: return tiled_one<EPI_RESID>(g, st);
    case EPI_SWIGLU: return tiled_one<EPI_SWIGLU>(g, st);
    default: return -2;
  }
}

}  // namespace cdb
