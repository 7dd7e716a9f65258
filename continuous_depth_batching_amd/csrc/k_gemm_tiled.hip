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
// byte offset lds_base + 16 * lane (lds_base wave-uniform).  The instruction
// takes the LDS base in M0; the "{m0}" operand constraint hands lds_base to
// the compiler, which writes M0 itself and knows it is in use.
__device__ __forceinline__ void lds_dma16(const void* gptr, uint32_t lds_base) {
  asm volatile("global_load_lds_dwordx4 %0, off" ::"v"(gptr), "{m0}"(lds_base) : "memory");
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
  const int ksteps = g.K / 32;                   // packed weight row stride (whole K)
  // split over K (grid y, EPI_PARTIAL): split s takes k-tiles of 64 from
  // s * per on; the host makes every split non-empty and only the last one
  // can end in a half k-tile
  const int split = blockIdx.y;
  const int per = (((g.K + 63) / 64) + g.SK - 1) / g.SK;
  const int kbase = split * per * 64;
  const int Kloc = min(g.K - kbase, per * 64);
  const int nk = (Kloc + 63) / 64;
  const bool half_last = (Kloc & 63) != 0;       // the last k-tile holds one k-step

  const uint16_t* A = (const uint16_t*)g.A + kbase;
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
    bsrc[i] = W + ((long)wt * ksteps * 64 + lane) * 8 + (long)(kbase / 32) * 512;
    b_ks[i] = t & 1;
  }
  const int ksteps_loc = kbase / 32 + (Kloc + 31) / 32;   // k-steps up to this split's end

  // k-tile kt into buffers (AS, BS).  Chunks past K (second half of a half
  // k-tile) are loaded from the first half instead: valid memory, never used.
#define CDB_TILE_ISSUE(kt, AS, BS)                                                               \
  {                                                                                              \
    const int k0_ = (kt) * 64;                                                                   \
    _Pragma("unroll") for (int i = 0; i < 4; i++) {                                              \
      const int c_ = (k0_ + a_chunk[i] * 8 < Kloc) ? a_chunk[i] : (a_chunk[i] & 3);              \
      lds_dma16(asrc[i] + k0_ + c_ * 8, __builtin_amdgcn_readfirstlane(lds_offset(&AS[(4 * w + i) * 512]))); \
    }                                                                                            \
    _Pragma("unroll") for (int i = 0; i < 4; i++) {                                              \
      const int st_ = min(2 * (kt) + b_ks[i], ksteps_loc - kbase / 32 - 1);                      \
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
  const int nkf = Kloc / 64;
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
  } else if (EPI == EPI_RESID) {
    // per row tile: the residual rows of the lane's 4 output rows, then its
    // 16 residual values, then the adds and stores -- three memory round
    // trips per row tile instead of two dependent ones per element, and few
    // enough live registers to keep two workgroups per CU (valid rows have
    // distinct residual rows).  The loads are unconditional (an invalid
    // element reads row 0 / the last column, never used): a branch per load
    // would make the compiler wait for every earlier load before each one.
#pragma unroll
    for (int i = 0; i < FM; i++) {
      int rr[4];
#pragma unroll
      for (int r = 0; r < 4; r++) {
        const int m = m0 + wm0 + 16 * i + 4 * g4 + r;
        const int sl = g.slot ? min(max(g.slot[min(m, g.M - 1)], 0), g.slot_max - 1) : m;
        if (g.slot && m < m_valid && sl != g.slot[min(m, g.M - 1)]) flag_err(g.err, ERR_SLOT);
        rr[r] = m < m_valid ? sl : -1;
      }
      float old[FN][4];
#pragma unroll
      for (int j = 0; j < FN; j++)
#pragma unroll
        for (int r = 0; r < 4; r++) {
          const int n = min(n_tile * BN + wn0 + 16 * j + r16, g.N - 1);
          old[j][r] = ((const float*)g.C)[(long)max(rr[r], 0) * g.ldc + n];
        }
#pragma unroll
      for (int j = 0; j < FN; j++)
#pragma unroll
        for (int r = 0; r < 4; r++) {
          const int n = n_tile * BN + wn0 + 16 * j + r16;
          if (rr[r] >= 0 && n < g.N) ((float*)g.C)[(long)rr[r] * g.ldc + n] = old[j][r] + acc[i][j][r];
        }
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
          } else if (EPI == EPI_PARTIAL) {
            g.partial[((long)split * g.M + m) * g.N + n] = v;
          } else {
            ((uint16_t*)g.C)[(long)m * g.ldc + n] = f32_to_bf16(v);
          }
        }
  }
}

// Large-tile variant for chunks with enough 256 x 256 output tiles to give
// every CU one workgroup: four waves of 128 x 128, one wave per SIMD, with
// v_mfma_f32_32x32x16_bf16.  On this chip the 16x16x32 bf16 MFMA issues at
// about half the rate of the 32x32x16 one, and with 64 x 64 wave tiles the
// LDS fragment reads, not the MFMAs, set the pace; a 128 x 128 wave tile
// reads half as many fragment bytes per MFMA.  The 256 accumulators of a
// lane fill the accumulation registers, so the register budget allows one
// wave per SIMD (amdgpu_waves_per_eu(1)).  With no second workgroup on the
// CU to cover memory latency, k-tiles of 32 go through a four-buffer LDS
// ring (4 x 32 KB), loaded three tiles ahead, with one barrier per k-tile:
// it publishes tile kt and also certifies that every wave has finished
// tile kt - 1, whose buffer then takes tile kt + 3.
//  - A rows: 64 bytes (four 16-byte chunks) per row, chunk c of row r in
//    slot c ^ ((r / 4) % 4), so the fragment reads of 16 consecutive rows
//    cover all banks;
//  - W: the packed 16-column tiles of the k-step, one kilobyte each;
//  - fragments (32x32x16 lane map): A lane l takes row l % 32 of its 32-row
//    tile, chunk 2s + l / 32 for the 16-wide step s of the k-tile; W lane l
//    takes output column l % 32, piece (col % 16) + 16 (2s + l / 32) of its
//    packed tile.  Accumulator element e of lane l is row
//    8 (e / 4) + 4 (l / 32) + e % 4, column l % 32.
// K % 32 == 0 (every k-tile is whole).
#define CDB_WAIT_VM6(n) __builtin_amdgcn_s_waitcnt(0x0F70 | ((n)&15) | (((n) >> 4) << 14))

template <int EPI>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(1, 1))) void k_gemm_big(GemmArgs g) {
  constexpr int BM = 256, BN = 256, WM = 128, WN = 128;
  constexpr int TM = WM / 32, TN = WN / 32;
  constexpr bool SWI = (EPI == EPI_SWIGLU);
  constexpr int OUT_BN = SWI ? BN / 2 : BN;
  constexpr int NBUF = 5;                        // 5 x 32 KB: the whole LDS
  constexpr int LOADS = 8;                       // direct loads per wave per k-tile (4 A + 4 W)
  constexpr int ABUF = BM * 32, BBUF = 16 * 512; // bf16 elements per buffer
  __shared__ __align__(16) uint16_t As[NBUF * ABUF];
  __shared__ __align__(16) uint16_t Bs[NBUF * BBUF];

  const int m_valid = min(ld_nvalid(g.n_valid, g.M), g.M);
  const int n_tiles = (g.N + OUT_BN - 1) / OUT_BN;
  const int m_tiles = g.m_tiles;
  const int total = m_tiles * n_tiles;
  int vid = blockIdx.x;
  if ((total & 7) == 0) vid = (blockIdx.x & 7) * (total >> 3) + (blockIdx.x >> 3);
  constexpr int GM = 4;
  const int grp = vid / (GM * n_tiles);
  const int first_m = grp * GM;
  const int gsz = min(GM, m_tiles - first_m);
  const int in = vid - grp * GM * n_tiles;
  const int m_tile = first_m + in % gsz;
  const int n_tile = in / gsz;
  const int m0 = m_tile * BM;
  if (m0 >= m_valid) return;                     // uniform per workgroup

  const int tid = threadIdx.x;
  const int lane = tid & 63, w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int l32 = lane & 31, h2 = lane >> 5;
  const int wm0 = (w >> 1) * WM, wn0 = (w & 1) * WN;
  const int nk = g.K / 32;

  const uint16_t* A = (const uint16_t*)g.A;
  const uint16_t* W = (const uint16_t*)g.W;
  // A: instruction i of wave w fills chunks q = (4w + i) * 64 + lane of the
  // buffer: row q / 4 = (4w + i) * 16 + lane / 4, slot lane % 4, holding
  // global chunk slot ^ ((row / 4) % 4) = (lane % 4) ^ ((lane / 16) % 4)
  const int a_row0 = m0 + 64 * w + (lane >> 2);
  const int a_chunk = (lane & 3) ^ ((lane >> 4) & 3);
  // W: instruction i of wave w copies packed tile vt = 4w + i of the k-step
  auto w_tile = [&](int i) -> int {
    const int vt = 4 * w + i;
    if (SWI) {
      const int wn = (16 * vt) / WN, j = ((16 * vt) % WN) / 16;
      const int outt = ((n_tile * OUT_BN + wn * (WN / 2)) >> 4) + (j % (WN / 32));
      return min(outt, (g.N - 1) >> 4) + (j >= WN / 32 ? (g.up_off >> 4) : 0);
    }
    return min(((n_tile * BN) >> 4) + vt, (g.N - 1) >> 4);
  };
  const uint32_t as_base = lds_offset(As), bs_base = lds_offset(Bs);
  auto issue = [&](int kt) {
    const int b = kt % NBUF;
#pragma unroll
    for (int i = 0; i < 4; i++) {
      const uint16_t* src = A + (long)min(a_row0 + 16 * i, g.M - 1) * g.lda + kt * 32 + a_chunk * 8;
      lds_dma16(src, __builtin_amdgcn_readfirstlane(as_base + 2 * (b * ABUF + (4 * w + i) * 512)));
    }
#pragma unroll
    for (int i = 0; i < 4; i++) {
      const long tile = ((long)w_tile(i) * nk + kt) * 512;
      lds_dma16(W + tile + lane * 8, __builtin_amdgcn_readfirstlane(bs_base + 2 * (b * BBUF + (4 * w + i) * 512)));
    }
  };

  typedef float f32x16_t __attribute__((ext_vector_type(16)));
  f32x16_t acc[TM][TN];
#pragma unroll
  for (int i = 0; i < TM; i++)
#pragma unroll
    for (int j = 0; j < TN; j++)
#pragma unroll
      for (int e = 0; e < 16; e++) acc[i][j][e] = 0.f;

  // Fragments of tile kt + 1 are read from LDS while the MFMAs of tile kt
  // run (two register sets, the loop unrolled by two so they alternate
  // without copies); the scheduling groups interleave one fragment read
  // with two MFMAs so the reads stay ahead of their use.
#define CDB_BIG_READ(kt, fa, fb)                                                                 \
  {                                                                                              \
    const uint16_t* AS_ = As + ((kt) % NBUF) * ABUF;                                       \
    const uint16_t* BS_ = Bs + ((kt) % NBUF) * BBUF;                                       \
    _Pragma("unroll") for (int s = 0; s < 2; s++) {                                              \
      _Pragma("unroll") for (int i = 0; i < TM; i++) {                                           \
        const int r = wm0 + 32 * i + l32, c = 2 * s + h2;                                        \
        fa[s][i] = *(const bf16x8_t*)&AS_[r * 32 + ((c ^ ((r >> 2) & 3)) * 8)];                  \
      }                                                                                          \
      _Pragma("unroll") for (int j = 0; j < TN; j++) {                                           \
        const int col = wn0 + 32 * j + l32;                                                      \
        fb[s][j] = *(const bf16x8_t*)&BS_[(col >> 4) * 512 + ((col & 15) + 16 * (2 * s + h2)) * 8]; \
      }                                                                                          \
    }                                                                                            \
  }
#define CDB_BIG_MMA_STEP(fa, fb, s)                                                              \
  _Pragma("unroll") for (int i = 0; i < TM; i++)                                                 \
    _Pragma("unroll") for (int j = 0; j < TN; j++)                                               \
      acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa[s][i], fb[s][j], acc[i][j], 0, 0, 0);
  // Iteration kt: make tile kt + 1 visible (this wave's loads of it landed,
  // then the barrier); run tile kt's MFMAs on (ca, cb) while reading tile
  // kt + 1's fragments into (na, nb), and after the first half of them
  // refill the buffer of tile kt - 1 with tile kt + 4 (the load issue then
  // overlaps the MFMAs already in the pipe).  Past the last tile the reads
  // fetch a stale buffer that is never used, which keeps every iteration
  // the same straight-line code.
#define CDB_BIG_ITER(kt, ca, cb, na, nb)                                                         \
  {                                                                                              \
    if ((kt) + 1 < nk) {                                                                         \
      if ((kt) + 3 < nk) CDB_WAIT_VM6(2 * LOADS);                                                \
      else if ((kt) + 2 < nk) CDB_WAIT_VM6(LOADS);                                               \
      else CDB_WAIT_VM6(0);                                                                      \
      __syncthreads();                                                                           \
    }                                                                                            \
    CDB_BIG_READ((kt) + 1, na, nb)                                                               \
    CDB_BIG_MMA_STEP(ca, cb, 0)                                                                  \
    _Pragma("unroll") for (int q = 0; q < 16; q++) {                                             \
      __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);                                         \
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);                                         \
    }                                                                                            \
    if ((kt) + 4 < nk) issue((kt) + 4);                                                          \
    CDB_BIG_MMA_STEP(ca, cb, 1)                                                                  \
  }

  bf16x8_t fa0[2][TM], fb0[2][TN], fa1[2][TM], fb1[2][TN];
  issue(0);
  if (nk > 1) issue(1);
  if (nk > 2) issue(2);
  if (nk > 3) issue(3);
  if (nk > 3) CDB_WAIT_VM6(3 * LOADS);
  else if (nk > 2) CDB_WAIT_VM6(2 * LOADS);
  else if (nk > 1) CDB_WAIT_VM6(LOADS);
  else CDB_WAIT_VM6(0);
  __syncthreads();
  CDB_BIG_READ(0, fa0, fb0)
  int kt = 0;
  for (; kt + 2 <= nk; kt += 2) {
    CDB_BIG_ITER(kt, fa0, fb0, fa1, fb1)
    CDB_BIG_ITER(kt + 1, fa1, fb1, fa0, fb0)
  }
  if (kt < nk) CDB_BIG_ITER(kt, fa0, fb0, fa1, fb1)
#undef CDB_BIG_READ
#undef CDB_BIG_MMA_STEP
#undef CDB_BIG_ITER

  // ---- epilogues from registers ----
  if (SWI) {
#pragma unroll
    for (int i = 0; i < TM; i++)
#pragma unroll
      for (int j = 0; j < TN / 2; j++) {
#pragma unroll
        for (int e = 0; e < 16; e++) {
          const int m = m0 + wm0 + 32 * i + 8 * (e >> 2) + 4 * h2 + (e & 3);
          const int n = n_tile * OUT_BN + (wn0 / 2) + 32 * j + l32;
          if (m >= m_valid || n >= g.N) continue;
          const float gt = acc[i][j][e], up = acc[i][j + TN / 2][e];
          ((uint16_t*)g.C)[(long)m * g.ldc + n] = f32_to_bf16(silu_f(gt) * up);
        }
      }
  } else if (EPI == EPI_RESID) {
    // residual rows read a 32 x 32 tile at a time (16 loads in flight, then
    // the adds and stores), not one dependent round trip per element
#pragma unroll
    for (int i = 0; i < TM; i++)
#pragma unroll
      for (int j = 0; j < TN; j++) {
        // unconditional loads (an invalid element reads row 0 / the last
        // column, never used), so no branch makes the compiler wait for
        // every earlier load
        float* dst[16];
        float old[16];
        bool ok[16];
#pragma unroll
        for (int e = 0; e < 16; e++) {
          const int m = m0 + wm0 + 32 * i + 8 * (e >> 2) + 4 * h2 + (e & 3);
          const int n = n_tile * BN + wn0 + 32 * j + l32;
          ok[e] = m < m_valid && n < g.N;
          const int rr = !ok[e] ? 0 : (g.slot ? clamp_chk(g.slot[min(m, g.M - 1)], 0, g.slot_max - 1, g.err, ERR_SLOT) : m);
          dst[e] = (float*)g.C + (long)rr * g.ldc + min(n, g.N - 1);
          old[e] = *dst[e];
        }
#pragma unroll
        for (int e = 0; e < 16; e++)
          if (ok[e]) *dst[e] = old[e] + acc[i][j][e];
      }
  } else {
#pragma unroll
    for (int i = 0; i < TM; i++)
#pragma unroll
      for (int j = 0; j < TN; j++) {
#pragma unroll
        for (int e = 0; e < 16; e++) {
          const int m = m0 + wm0 + 32 * i + 8 * (e >> 2) + 4 * h2 + (e & 3);
          const int n = n_tile * BN + wn0 + 32 * j + l32;
          if (m >= m_valid || n >= g.N) continue;
          const float v = acc[i][j][e];
          if (EPI == EPI_STORE_F32) {
            ((float*)g.C)[(long)m * g.ldc + n] = v;
          } else {
            ((uint16_t*)g.C)[(long)m * g.ldc + n] = f32_to_bf16(v);
          }
        }
      }
  }
}
#undef CDB_WAIT_VM6

// Wide-tile variant for short reductions into many columns (the Ouro-like
// QKV and gate/up prefill projections, K = 2048): 256 x 128 output tiles,
// four waves of 128 x 64 (16x16x32 MFMAs), k-tiles of 32 in two LDS buffers
// (48 KB per workgroup, so two or three workgroups share a CU).  Against the
// 128 x 128 kernel each fragment read from LDS feeds 1.33x the MFMAs and
// each staged byte 1.33x the output, which is where that kernel loses its
// time; the arithmetic per output is the same (same MFMA, same k order), so
// the two kernels produce the same bits.  Two loop forms:
//  - PF = false: tile kt + 1's loads in flight while tile kt's fragments are
//    read and multiplied, two barriers per tile (165 registers, so three
//    workgroups fit a CU by LDS);
//  - PF = true: also tile kt + 1's fragments read during tile kt's MFMAs
//    (two register sets), one barrier per tile (it publishes tile kt + 1 and
//    certifies that every wave has read tile kt's fragments, whose buffer
//    then takes tile kt + 2); 243 registers, two workgroups per CU.
// Measured at 8192 rows against the 128 x 128 kernel, TFLOP/s: 8192 x 6144 x
// 2048 1,062 -> 1,154 (PF 1,169), 8192 x 11264 x 2048 893 -> 1,084 (PF 989),
// 8192 x 2048 x 2048 879 -> 931 (PF 1,009), 8192 x 2048 x 5632 1,127 -> 1,122
// (PF 1,217), 8192 x 6144 x 8192 1,202 -> 1,153 (PF 1,071): the prefetching
// form wins on grids of two workgroups per CU, the other on larger grids,
// where a third workgroup per CU hides more.
//  - A rows: 64 bytes per row, chunk c of row r in slot c ^ ((r / 4) % 4)
//    (as the 256 x 256 kernel), so the fragment reads of 16 rows cover all
//    banks; W: the packed 16-column tiles of the k-step;
//  - SwiGLU: each wave's four column tiles are the gate columns of 32
//    outputs followed by the up columns of the same outputs (64 outputs per
//    workgroup), so silu(gate) * up is formed from registers;
//  - residual add: a row tile's 16 residual values loaded first,
//    unconditionally, then added and stored (as the 128 x 128 kernel).
// K % 32 == 0.
template <int EPI, bool PF>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2))) void k_gemm_wide(GemmArgs g) {
  constexpr int BM = 256, BN = 128, WM = 128, WN = 64, FM = WM / 16, FN = WN / 16;
  constexpr bool SWI = (EPI == EPI_SWIGLU);
  constexpr int OUT_BN = SWI ? BN / 2 : BN;
  constexpr int LOADS = 6;                       // direct loads per wave per k-tile (4 A + 2 W)
  constexpr int ABUF = BM * 32, BBUF = (BN / 16) * 512;   // bf16 elements per buffer
  __shared__ __align__(16) uint16_t As[2 * ABUF];
  __shared__ __align__(16) uint16_t Bs[2 * BBUF];

  const int m_valid = min(ld_nvalid(g.n_valid, g.M), g.M);
  const int n_tiles = (g.N + OUT_BN - 1) / OUT_BN;
  const int m_tiles = g.m_tiles;
  const int total = m_tiles * n_tiles;
  int vid = blockIdx.x;
  if ((total & 7) == 0) vid = (blockIdx.x & 7) * (total >> 3) + (blockIdx.x >> 3);
  constexpr int GM = 4;
  const int grp = vid / (GM * n_tiles);
  const int first_m = grp * GM;
  const int gsz = min(GM, m_tiles - first_m);
  const int in = vid - grp * GM * n_tiles;
  const int m_tile = first_m + in % gsz;
  const int n_tile = in / gsz;
  const int m0 = m_tile * BM;
  if (m0 >= m_valid) return;                     // uniform per workgroup

  const int tid = threadIdx.x;
  const int lane = tid & 63, w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int r16 = lane & 15, g4 = lane >> 4;
  const int wm0 = (w >> 1) * WM, wn0 = (w & 1) * WN;
  const int nk = g.K / 32;
  const uint16_t* A = (const uint16_t*)g.A;
  const uint16_t* W = (const uint16_t*)g.W;
  // A: instruction i of wave w fills chunks q = (4w + i) * 64 + lane of the
  // buffer: row q / 4 = (4w + i) * 16 + lane / 4, slot lane % 4, holding
  // global chunk slot ^ ((row / 4) % 4) = (lane % 4) ^ (lane / 16)
  const int a_row0 = m0 + 64 * w + (lane >> 2);
  const int a_chunk = (lane & 3) ^ (lane >> 4);
  // W: instruction i of wave w copies packed column tile t = 2w + i of the
  // workgroup (for SwiGLU: wave t / 4's tile t % 4, gate then up)
  const uint16_t* bsrc[2];
#pragma unroll
  for (int i = 0; i < 2; i++) {
    const int t = 2 * w + i;
    int wt;
    if (SWI) {
      const int wn = t / FN, j = t % FN;
      const int outt = ((n_tile * OUT_BN + wn * (WN / 2)) >> 4) + (j % (FN / 2));
      wt = min(outt, (g.N - 1) >> 4) + (j >= FN / 2 ? (g.up_off >> 4) : 0);
    } else {
      wt = min(((n_tile * BN) >> 4) + t, (g.N - 1) >> 4);
    }
    bsrc[i] = W + ((long)wt * nk * 64 + lane) * 8;
  }
  const uint32_t as_base = lds_offset(As), bs_base = lds_offset(Bs);
  auto issue = [&](int kt) {
    const int b = kt & 1;
#pragma unroll
    for (int i = 0; i < 4; i++) {
      const uint16_t* src = A + (long)min(a_row0 + 16 * i, g.M - 1) * g.lda + kt * 32 + a_chunk * 8;
      lds_dma16(src, __builtin_amdgcn_readfirstlane(as_base + 2 * (b * ABUF + (4 * w + i) * 512)));
    }
#pragma unroll
    for (int i = 0; i < 2; i++)
      lds_dma16(bsrc[i] + (long)kt * 512, __builtin_amdgcn_readfirstlane(bs_base + 2 * (b * BBUF + (2 * w + i) * 512)));
  };

  f32x4_t acc[FM][FN];
#pragma unroll
  for (int i = 0; i < FM; i++)
#pragma unroll
    for (int j = 0; j < FN; j++) acc[i][j] = (f32x4_t){0.f, 0.f, 0.f, 0.f};
  // this wave's fragments of tile kt from its LDS buffer
  auto rd = [&](int kt, bf16x8_t (&af)[FM], bf16x8_t (&bfr)[FN]) __attribute__((always_inline)) {
    const uint16_t* AS = As + (kt & 1) * ABUF;
    const uint16_t* BS = Bs + (kt & 1) * BBUF;
#pragma unroll
    for (int j = 0; j < FN; j++) bfr[j] = *(const bf16x8_t*)&BS[((wn0 >> 4) + j) * 512 + lane * 8];
#pragma unroll
    for (int i = 0; i < FM; i++) {
      const int r = wm0 + 16 * i + r16;
      af[i] = *(const bf16x8_t*)&AS[r * 32 + ((g4 ^ ((r >> 2) & 3)) * 8)];
    }
  };
  auto mma = [&](bf16x8_t (&af)[FM], bf16x8_t (&bfr)[FN]) __attribute__((always_inline)) {
#pragma unroll
    for (int i = 0; i < FM; i++)
#pragma unroll
      for (int j = 0; j < FN; j++) acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af[i], bfr[j], acc[i][j], 0, 0, 0);
  };
  if constexpr (!PF) {
    // tile kt + 1's loads are in flight while tile kt feeds the MFMAs; each
    // wave waits only for its own loads of tile kt (vmcnt), then the barrier
    // makes every wave's loads visible; the second barrier frees the buffer
    issue(0);
    for (int kt = 0; kt < nk; kt++) {
      if (kt + 1 < nk) {
        issue(kt + 1);
        CDB_WAIT_VM(LOADS);
      } else {
        CDB_WAIT_VM(0);
      }
      __syncthreads();
      // one A fragment at a time, so the register count stays low enough
      // for three workgroups per CU
      const uint16_t* AS = As + (kt & 1) * ABUF;
      const uint16_t* BS = Bs + (kt & 1) * BBUF;
      bf16x8_t bfr[FN];
#pragma unroll
      for (int j = 0; j < FN; j++) bfr[j] = *(const bf16x8_t*)&BS[((wn0 >> 4) + j) * 512 + lane * 8];
#pragma unroll
      for (int i = 0; i < FM; i++) {
        const int r = wm0 + 16 * i + r16;
        const bf16x8_t af = *(const bf16x8_t*)&AS[r * 32 + ((g4 ^ ((r >> 2) & 3)) * 8)];
#pragma unroll
        for (int j = 0; j < FN; j++) acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af, bfr[j], acc[i][j], 0, 0, 0);
      }
      __syncthreads();
    }
  } else {
    // tiles kt + 1 (loads landed, fragments being read) and kt + 2 (loads in
    // flight) overlap tile kt's MFMAs; the loop is unrolled by two so the
    // two fragment register sets alternate without copies
    bf16x8_t fa0[FM], fb0[FN], fa1[FM], fb1[FN];
    issue(0);
    if (nk > 1) issue(1);
    if (nk > 1) CDB_WAIT_VM(LOADS);
    else CDB_WAIT_VM(0);
    __syncthreads();
    rd(0, fa0, fb0);
    auto iter = [&](int kt, bf16x8_t (&ca)[FM], bf16x8_t (&cb)[FN], bf16x8_t (&na)[FM],
                    bf16x8_t (&nb)[FN]) __attribute__((always_inline)) {
      if (kt + 1 < nk) {
        CDB_WAIT_VM(0);                          // this wave's loads of tile kt + 1 landed
        __syncthreads();                         // ... every wave's; tile kt's fragments all read
        if (kt + 2 < nk) issue(kt + 2);          // into tile kt's buffer
        rd(kt + 1, na, nb);
      }
      mma(ca, cb);
    };
    int kt = 0;
    for (; kt + 2 <= nk; kt += 2) {
      iter(kt, fa0, fb0, fa1, fb1);
      iter(kt + 1, fa1, fb1, fa0, fb0);
    }
    if (kt < nk) iter(kt, fa0, fb0, fa1, fb1);
  }

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
  } else if (EPI == EPI_RESID) {
#pragma unroll
    for (int i = 0; i < FM; i++) {
      int rr[4];
#pragma unroll
      for (int r = 0; r < 4; r++) {
        const int m = m0 + wm0 + 16 * i + 4 * g4 + r;
        const int sl = g.slot ? min(max(g.slot[min(m, g.M - 1)], 0), g.slot_max - 1) : m;
        if (g.slot && m < m_valid && sl != g.slot[min(m, g.M - 1)]) flag_err(g.err, ERR_SLOT);
        rr[r] = m < m_valid ? sl : -1;
      }
      float old[FN][4];
#pragma unroll
      for (int j = 0; j < FN; j++)
#pragma unroll
        for (int r = 0; r < 4; r++) {
          const int n = min(n_tile * BN + wn0 + 16 * j + r16, g.N - 1);
          old[j][r] = ((const float*)g.C)[(long)max(rr[r], 0) * g.ldc + n];
        }
#pragma unroll
      for (int j = 0; j < FN; j++)
#pragma unroll
        for (int r = 0; r < 4; r++) {
          const int n = n_tile * BN + wn0 + 16 * j + r16;
          if (rr[r] >= 0 && n < g.N) ((float*)g.C)[(long)rr[r] * g.ldc + n] = old[j][r] + acc[i][j][r];
        }
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
          if (EPI == EPI_STORE_F32) ((float*)g.C)[(long)m * g.ldc + n] = v;
          else ((uint16_t*)g.C)[(long)m * g.ldc + n] = f32_to_bf16(v);
        }
  }
}

template <int EPI>
static int wide_one(GemmArgs g, hipStream_t st) {
  constexpr int OUT_BN = (EPI == EPI_SWIGLU) ? 64 : 128;
  g.m_tiles = (g.M + 255) / 256;
  const int n_tiles = (g.N + OUT_BN - 1) / OUT_BN;
  const int wgs = g.m_tiles * n_tiles;
  // the prefetching form on grids of at most two workgroups per CU
  if (wgs <= 512) hipLaunchKernelGGL((k_gemm_wide<EPI, true>), dim3(wgs), dim3(256), 0, st, g);
  else hipLaunchKernelGGL((k_gemm_wide<EPI, false>), dim3(wgs), dim3(256), 0, st, g);
  return hipGetLastError() == hipSuccess ? 0 : -1;
}

template <int EPI>
static int big_one(GemmArgs g, hipStream_t st) {
  constexpr int OUT_BN = (EPI == EPI_SWIGLU) ? 128 : 256;
  g.m_tiles = (g.M + 255) / 256;
  const int n_tiles = (g.N + OUT_BN - 1) / OUT_BN;
  hipLaunchKernelGGL((k_gemm_big<EPI>), dim3(g.m_tiles * n_tiles), dim3(256), 0, st, g);
  return hipGetLastError() == hipSuccess ? 0 : -1;
}

template <int EPI>
static int tiled_one(GemmArgs g, hipStream_t st) {
  constexpr int OUT_BN = (EPI == EPI_SWIGLU) ? 64 : 128;
  g.m_tiles = (g.M + 127) / 128;
  const int n_tiles = (g.N + OUT_BN - 1) / OUT_BN;
  hipLaunchKernelGGL((k_gemm_tiled<EPI>), dim3(g.m_tiles * n_tiles, g.SK), dim3(256), 0, st, g);
  return hipGetLastError() == hipSuccess ? 0 : -1;
}

bool gemm_tiled_supported(int dtype, int epi) {
  return dtype == 1 && (epi == EPI_STORE_F32 || epi == EPI_STORE_T || epi == EPI_RESID || epi == EPI_SWIGLU ||
                        epi == EPI_PARTIAL);
}

// 128 x 128 tiles, waves of 64 x 64 (two workgroups per CU).
int gemm_tiled_launch(int epi, const GemmArgs& g, hipStream_t st) {
  if (g.K % 32 || g.M <= 0 || g.N <= 0 || g.N % 16 || (epi == EPI_SWIGLU && g.up_off % 16)) return -2;
  // K splits only with partial outputs; every split must own at least one
  // k-tile of 64 (the host passes the split count this rule gives)
  const int nkt = (g.K + 63) / 64;
  if (g.SK < 1 || (g.SK > 1 && epi != EPI_PARTIAL) || (epi == EPI_PARTIAL && !g.partial)) return -2;
  if (g.SK > 1 && ((nkt + g.SK - 1) / g.SK) * (g.SK - 1) >= nkt) return -2;
  switch (epi) {
    case EPI_PARTIAL: return tiled_one<EPI_PARTIAL>(g, st);
    case EPI_STORE_F32: return tiled_one<EPI_STORE_F32>(g, st);
    case EPI_STORE_T: return tiled_one<EPI_STORE_T>(g, st);
    case EPI_RESID: return tiled_one<EPI_RESID>(g, st);
    case EPI_SWIGLU: return tiled_one<EPI_SWIGLU>(g, st);
    default: return -2;
  }
}

// 256 x 256 tiles, waves of 128 x 128 with 32x32x16 MFMAs (one workgroup per CU).
int gemm_big_launch(int epi, const GemmArgs& g, hipStream_t st) {
  if (g.K % 32 || g.M <= 0 || g.N <= 0 || g.N % 16 || (epi == EPI_SWIGLU && g.up_off % 16)) return -2;
  switch (epi) {
    case EPI_STORE_F32: return big_one<EPI_STORE_F32>(g, st);
    case EPI_STORE_T: return big_one<EPI_STORE_T>(g, st);
    case EPI_RESID: return big_one<EPI_RESID>(g, st);
    case EPI_SWIGLU: return big_one<EPI_SWIGLU>(g, st);
    default: return -2;
  }
}

// 256 x 128 tiles, waves of 128 x 64 (two or three workgroups per CU).
int gemm_wide_launch(int epi, const GemmArgs& g, hipStream_t st) {
  if (g.K % 32 || g.M <= 0 || g.N <= 0 || g.N % 16 || (epi == EPI_SWIGLU && g.up_off % 16)) return -2;
  switch (epi) {
    case EPI_STORE_F32: return wide_one<EPI_STORE_F32>(g, st);
    case EPI_STORE_T: return wide_one<EPI_STORE_T>(g, st);
    case EPI_RESID: return wide_one<EPI_RESID>(g, st);
    case EPI_SWIGLU: return wide_one<EPI_SWIGLU>(g, st);
    default: return -2;
  }
}

}  // namespace cdb
