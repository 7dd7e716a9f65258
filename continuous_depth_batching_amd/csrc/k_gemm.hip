// MFMA GEMM for the core and boundary projections: C[M][N] = A[M][K] . W[N][K]^T
// (weights in [out][in] layout), fp32 accumulation, fused epilogues.
//
// Design (decode-shaped GEMMs are weight-streaming, HBM-bound below M ~ 300):
//  - one workgroup = 4 waves computes a (16*MW) x (16*NW) output tile; the
//    four waves split the workgroup's K range four ways and their partial
//    tiles are summed through LDS in fixed wave order;
//  - grid.y splits K across SK workgroups when the N-tiles alone cannot fill
//    256 CUs; each split writes its fp32 partial tile (EPI_PARTIAL) and the
//    consumer — the residual-add + RMSNorm kernel that runs next anyway —
//    sums the splits in split order, so no workgroup waits on another and
//    results do not depend on arrival order;
//  - operands go straight from global memory into MFMA fragments (16 B per
//    lane per fragment); weights are streamed exactly once per M-tile, and
//    the M-tiles of one N-tile are placed on the same XCD so the second read
//    hits that XCD's L2;
//  - epilogues: store fp32, store T, residual add into the fp32 loop state
//    through the slot table, SwiGLU (gate and up tiles of the same columns),
//    per-tile (max, index) partials of the greedy argmax over the vocabulary
//    (reduced by k_argmax_reduce; lowest index among equal maxima).
#include "common.h"
#include "kernels.h"

namespace cdb {

template <typename T, int MW, int NW, int EPI>
__global__ __launch_bounds__(256) void k_gemm(GemmArgs g) {
  typedef typename Elt<T>::raw raw;
  constexpr int VEC = Elt<T>::VEC;
  constexpr int KSTEP = Elt<T>::KSTEP;
  constexpr bool SWI = (EPI == EPI_SWIGLU);
  constexpr int NWX = SWI ? 2 * NW : NW;      // weight row blocks per wave
  constexpr int MT = 16 * MW, NT = 16 * NW, NTX = 16 * NWX;
  constexpr int UNR = (MW + NWX) >= 6 ? 2 : ((MW + NWX) >= 3 ? 4 : 8);
  extern __shared__ float lds[];               // [4][MT][NTX]; lds[0] doubles as a flag

  const int n_tiles_n = (g.N + NT - 1) / NT;
  const int n_tiles = n_tiles_n * g.m_tiles;
  // XCD-aware order: consecutive virtual ids run on one XCD (blockIdx % 8)
  int bid = blockIdx.x;
  int vid = bid;
  if ((n_tiles & 7) == 0) vid = (bid & 7) * (n_tiles >> 3) + (bid >> 3);
  const int m_tile = vid % g.m_tiles;           // M fastest: same N-tile, same XCD
  const int n_tile = vid / g.m_tiles;
  const int split = blockIdx.y;
  const int n0 = n_tile * NT, m0 = m_tile * MT;
  const int m_valid = min(ld_nvalid(g.n_valid, g.M), g.M);
  if (m0 >= m_valid) return;                    // every split of this tile returns

  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int r16 = lane & 15, g4 = lane >> 4;
  const int nsteps = g.K / KSTEP;
  const int s0 = (int)((long)split * nsteps / g.SK), s1 = (int)((long)(split + 1) * nsteps / g.SK);
  const int ws0 = s0 + (s1 - s0) * w / 4, ws1 = s0 + (s1 - s0) * (w + 1) / 4;

  const raw* A = (const raw*)g.A;
  const raw* W = (const raw*)g.W;
  const raw* arow[MW];
#pragma unroll
  for (int i = 0; i < MW; i++) {
    int m = m0 + 16 * i + r16;
    m = m < g.M ? m : g.M - 1;
    arow[i] = A + (long)m * g.lda + g4 * VEC;
  }
  // weight fragments: packed tile (row tile, k-step) piece `lane`
  const raw* wrow[NWX];
#pragma unroll
  for (int j = 0; j < NWX; j++) {
    int nt = min((n0 >> 4) + (j % NW), (g.N - 1) >> 4);
    if (SWI && j >= NW) nt += g.up_off >> 4;     // up rows follow the gate rows
    wrow[j] = W + ((long)nt * nsteps * 64 + lane) * VEC;
  }

  f32x4_t acc[MW][NWX];
#pragma unroll
  for (int i = 0; i < MW; i++)
#pragma unroll
    for (int j = 0; j < NWX; j++) acc[i][j] = (f32x4_t){0.f, 0.f, 0.f, 0.f};

  int s = ws0;
  for (; s + UNR <= ws1; s += UNR) {
    uint4 a[UNR][MW], b[UNR][NWX];
#pragma unroll
    for (int u = 0; u < UNR; u++) {
      const long k = (long)(s + u) * KSTEP;
#pragma unroll
      for (int j = 0; j < NWX; j++) b[u][j] = *(const uint4*)(wrow[j] + (long)(s + u) * 64 * VEC);
#pragma unroll
      for (int i = 0; i < MW; i++) a[u][i] = *(const uint4*)(arow[i] + k);
    }
#pragma unroll
    for (int u = 0; u < UNR; u++)
#pragma unroll
      for (int i = 0; i < MW; i++)
#pragma unroll
        for (int j = 0; j < NWX; j++) Elt<T>::mma(acc[i][j], a[u][i], b[u][j]);
  }
  for (; s < ws1; s++) {
    const long k = (long)s * KSTEP;
    uint4 a[MW], b[NWX];
#pragma unroll
    for (int j = 0; j < NWX; j++) b[j] = *(const uint4*)(wrow[j] + (long)s * 64 * VEC);
#pragma unroll
    for (int i = 0; i < MW; i++) a[i] = *(const uint4*)(arow[i] + k);
#pragma unroll
    for (int i = 0; i < MW; i++)
#pragma unroll
      for (int j = 0; j < NWX; j++) Elt<T>::mma(acc[i][j], a[i], b[j]);
  }

  // ---- sum the four waves' partial tiles (fixed order) ----
  float* red = lds;                              // [4][MT][NTX]
#pragma unroll
  for (int i = 0; i < MW; i++)
#pragma unroll
    for (int j = 0; j < NWX; j++)
#pragma unroll
      for (int r = 0; r < 4; r++) {
        const int row = 16 * i + 4 * g4 + r, col = 16 * j + r16;
        red[(w * MT + row) * NTX + col] = acc[i][j][r];
      }
  __syncthreads();
  constexpr int PER = (MT * NTX + 255) / 256;
  float v[PER];
#pragma unroll
  for (int p = 0; p < PER; p++) {
    const int e = threadIdx.x + 256 * p;
    v[p] = 0.f;
    if (e < MT * NTX)
      v[p] = (red[e] + red[MT * NTX + e]) + (red[2 * MT * NTX + e] + red[3 * MT * NTX + e]);
  }

  // ---- epilogues ----
  if (EPI == EPI_STORE_F32 || EPI == EPI_STORE_T || EPI == EPI_RESID || EPI == EPI_PARTIAL) {
#pragma unroll
    for (int p = 0; p < PER; p++) {
      const int e = threadIdx.x + 256 * p;
      const int row = e / NT, col = e % NT;
      const int m = m0 + row, n = n0 + col;
      if (e >= MT * NT || n >= g.N || m >= m_valid) continue;
      if (EPI == EPI_STORE_F32) {
        ((float*)g.C)[(long)m * g.ldc + n] = v[p];
      } else if (EPI == EPI_PARTIAL) {
        g.partial[((long)split * g.M + m) * g.N + n] = v[p];
      } else if (EPI == EPI_STORE_T) {
        ((raw*)g.C)[(long)m * g.ldc + n] = Elt<T>::from_f32(v[p]);
      } else {
        const int r = g.slot ? clamp_chk(g.slot[m], 0, g.slot_max - 1, g.err, ERR_SLOT) : m;
        float* dst = (float*)g.C + (long)r * g.ldc + n;
        *dst = *dst + v[p];
      }
    }
  } else if (EPI == EPI_SWIGLU) {
    // v holds tile elements e = row*NTX + col with col < NT gate, col >= NT up
    __syncthreads();
#pragma unroll
    for (int p = 0; p < PER; p++) {
      const int e = threadIdx.x + 256 * p;
      if (e < MT * NTX) red[e] = v[p];
    }
    __syncthreads();
    for (int e = threadIdx.x; e < MT * NT; e += 256) {
      const int row = e / NT, col = e % NT;
      const int m = m0 + row, n = n0 + col;
      if (n >= g.N || m >= m_valid) continue;
      const float gt = red[row * NTX + col], up = red[row * NTX + NT + col];
      ((raw*)g.C)[(long)m * g.ldc + n] = Elt<T>::from_f32(silu_f(gt) * up);
    }
  } else if (EPI == EPI_ARGMAX) {
    // optional logits, then per-row (max, index) of this tile's columns
    __syncthreads();
#pragma unroll
    for (int p = 0; p < PER; p++) {
      const int e = threadIdx.x + 256 * p;
      if (e < MT * NT) {
        red[e] = v[p];
        const int m = m0 + e / NT, n = n0 + e % NT;
        if (g.C && m < m_valid && n < g.N) ((float*)g.C)[(long)m * g.ldc + n] = v[p];
      }
    }
    __syncthreads();
    if (threadIdx.x < MT) {
      const int row = threadIdx.x;
      float best = -INFINITY;
      int bi = -1;
      for (int c = 0; c < NT; c++) {
        const int n = n0 + c;
        const float x = red[row * NT + c];
        if (n < g.N && (bi < 0 || x > best)) { best = x; bi = n; }
      }
      g.amax_val[(long)(m0 + row) * n_tiles_n + n_tile] = best;
      g.amax_idx[(long)(m0 + row) * n_tiles_n + n_tile] = bi;
    }
  }
}

// Greedy argmax of each row from the per-tile partials: larger value wins,
// equal values keep the lower index (an order-independent combine, so the
// block reduction is deterministic).
__global__ __launch_bounds__(256) void k_argmax_reduce(ArgmaxArgs a) {
  __shared__ float sv[256];
  __shared__ int si[256];
  const int m = blockIdx.x;
  if (m >= min(ld_nvalid(a.n_valid, a.rows), a.rows)) return;
  float best = -INFINITY;
  int bi = -1;
  for (int t = threadIdx.x; t < a.n_tiles; t += 256) {
    const float x = a.val[(long)m * a.n_tiles + t];
    const int ix = a.idx[(long)m * a.n_tiles + t];
    if (bi < 0 || x > best || (x == best && ix < bi)) { best = x; bi = ix; }
  }
  sv[threadIdx.x] = best;
  si[threadIdx.x] = bi;
  __syncthreads();
  for (int o = 128; o > 0; o >>= 1) {
    if (threadIdx.x < o) {
      const float x = sv[threadIdx.x + o];
      const int ix = si[threadIdx.x + o];
      if (ix >= 0 && (si[threadIdx.x] < 0 || x > sv[threadIdx.x] || (x == sv[threadIdx.x] && ix < si[threadIdx.x]))) {
        sv[threadIdx.x] = x;
        si[threadIdx.x] = ix;
      }
    }
    __syncthreads();
  }
  if (threadIdx.x == 0) a.tok_out[m] = si[0];
}

int argmax_reduce_launch(const ArgmaxArgs& a, hipStream_t st) {
  if (a.rows <= 0) return 0;
  hipLaunchKernelGGL(k_argmax_reduce, dim3(a.rows), dim3(256), 0, st, a);
  return hipGetLastError() == hipSuccess ? 0 : -1;
}

template <typename T, int MW, int NW, int EPI>
static int launch_one(const GemmArgs& g, hipStream_t st) {
  constexpr int NWX = (EPI == EPI_SWIGLU) ? 2 * NW : NW;
  constexpr int MT = 16 * MW, NT = 16 * NW, NTX = 16 * NWX;
  const size_t lds = (size_t)4 * MT * NTX * sizeof(float);
  const int n_tiles_n = (g.N + NT - 1) / NT;
  dim3 grid(n_tiles_n * g.m_tiles, g.SK);
  hipLaunchKernelGGL((k_gemm<T, MW, NW, EPI>), grid, dim3(256), lds, st, g);
  return hipGetLastError() == hipSuccess ? 0 : -1;
}

template <typename T, int EPI>
static int dispatch_mw_nw(int MW, int NW, const GemmArgs& g, hipStream_t st) {
#define CDB_GEMM_CASE(mw, nw) if (MW == mw && NW == nw) return launch_one<T, mw, nw, EPI>(g, st);
  CDB_GEMM_CASE(1, 1)
  CDB_GEMM_CASE(2, 1)
  CDB_GEMM_CASE(4, 1)
  CDB_GEMM_CASE(4, 2)
  CDB_GEMM_CASE(4, 4)
#undef CDB_GEMM_CASE
  return -2;
}

int gemm_launch(int dtype, int epi, int MW, int NW, GemmArgs g, hipStream_t st) {
  if (epi == EPI_SWIGLU && NW > 2) return -2;
  const int MT = 16 * MW;
  g.m_tiles = (g.M + MT - 1) / MT;
#define CDB_EPI(T)                                                                  \
  switch (epi) {                                                                    \
    case EPI_STORE_F32: return dispatch_mw_nw<T, EPI_STORE_F32>(MW, NW, g, st);     \
    case EPI_STORE_T: return dispatch_mw_nw<T, EPI_STORE_T>(MW, NW, g, st);         \
    case EPI_RESID: return dispatch_mw_nw<T, EPI_RESID>(MW, NW, g, st);             \
    case EPI_SWIGLU: return dispatch_mw_nw<T, EPI_SWIGLU>(MW, NW, g, st);           \
    case EPI_ARGMAX: return dispatch_mw_nw<T, EPI_ARGMAX>(MW, NW, g, st);           \
    case EPI_PARTIAL: return dispatch_mw_nw<T, EPI_PARTIAL>(MW, NW, g, st);         \
  }
  if (dtype == 0) { CDB_EPI(float) } else { CDB_EPI(bf16_t) }
#undef CDB_EPI
  return -2;
}

}  // namespace cdb

// ---------------------------------------------------------------------------
// Decode GEMM (M <= 64): weight streaming, one memory round trip per wave.
//
// A workgroup owns 64 weight rows (4 row tiles of 16) and 4*KW*nb consecutive
// MFMA k-steps; wave w takes KW*nb of them, for all four row tiles, in nb
// batches of KW (nb = 1 unless K is very long).  Every load of a batch — the
// wave's activation fragments (MW tiles of 16 rows, L2-resident and re-read
// by every workgroup) and its 4*KW packed weight tiles (one contiguous
// kilobyte each) — is issued before the batch's first MFMA, so a wave waits
// for memory once per batch.  In the decode core step the activations come
// fragment-packed from their producers (norm, attention, SwiGLU), so an
// activation fragment is one contiguous kilobyte as well.  The four waves' partial tiles are summed
// through LDS in wave order; wave j then finishes row tile j: fp32 split
// partials [SK][M][N] (EPI_PARTIAL; the consumer adds the splits in order) or
// per-16-column (max, index) of the greedy argmax (EPI_ARGMAX, SK == 1).
namespace cdb {

template <typename T, int MW, int KW, int EPI>
__global__ __launch_bounds__(256) void k_gemm_dec(GemmArgs g) {
  typedef typename Elt<T>::raw raw;
  constexpr int VEC = Elt<T>::VEC, KS = Elt<T>::KSTEP;
  constexpr int NTW = 4;                             // row tiles per workgroup (and per wave)
  __shared__ f32x4_t red[4][MW * NTW][64];

  const int n_tiles = (g.N + 63) / 64;
  const int n_tile = blockIdx.x % n_tiles;
  const int split = blockIdx.x / n_tiles;
  const int m0 = blockIdx.y * 16 * MW;               // this workgroup's block of 16 * MW rows
  // row blocks past the first one check the row count first and skip when
  // it holds no valid row (the first block never waits for it)
  if (blockIdx.y > 0 && m0 >= ld_nvalid(g.n_valid, g.M)) return;
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int r16 = lane & 15, g4 = lane >> 4;
  const int nsteps = g.K / KS;
  const int nb = max(g.dec_batches, 1);
  const int s0 = (split * 4 + w) * KW * nb;          // this wave's first k-step

  const raw* A = (const raw*)g.A;
  const raw* W = (const raw*)g.W;
  // activation fragment of row tile i at k-step st: arow[i] + st * a_step
  // (rows past M re-read row M - 1; their outputs are never stored)
  const raw* arow[MW];
  const long a_step = g.a_packed ? 64L * VEC : KS;
#pragma unroll
  for (int i = 0; i < MW; i++) {
    const int m = min(m0 + 16 * i + r16, g.M - 1);
    arow[i] = g.a_packed ? A + ((long)(m >> 4) * nsteps * 64 + (m & 15) + 16 * g4) * VEC
                         : A + (long)m * g.lda + g4 * VEC;
  }
  const raw* wt[NTW];
#pragma unroll
  for (int j = 0; j < NTW; j++) {
    const int nt = min(n_tile * NTW + j, (g.N - 1) >> 4);
    wt[j] = W + ((long)nt * nsteps * 64 + lane) * VEC;
  }

  f32x4_t acc[MW][NTW];
#pragma unroll
  for (int i = 0; i < MW; i++)
#pragma unroll
    for (int j = 0; j < NTW; j++) acc[i][j] = (f32x4_t){0.f, 0.f, 0.f, 0.f};
  int m_valid = g.M;
  for (int b = 0; b < nb; b++) {
    const int sb = s0 + b * KW;
    // all loads of the batch first (k-steps past the end re-read the last one and are skipped)
    uint4 av[KW][MW], wv[KW][NTW];
#pragma unroll
    for (int t = 0; t < KW; t++) {
      const int st = min(sb + t, nsteps - 1);
#pragma unroll
      for (int j = 0; j < NTW; j++) wv[t][j] = ldg_u4(wt[j] + (long)st * 64 * VEC);
#pragma unroll
      for (int i = 0; i < MW; i++) av[t][i] = ldg_u4(arow[i] + (long)st * a_step);
    }
    // the row count is needed only by the stores: its load goes out behind the batch
    if (b == 0) m_valid = min(ld_nvalid(g.n_valid, g.M), g.M);
    __builtin_amdgcn_sched_barrier(0);               // keep every load ahead of the MFMAs
    if (sb + KW <= nsteps) {
#pragma unroll
      for (int t = 0; t < KW; t++)
#pragma unroll
        for (int i = 0; i < MW; i++)
#pragma unroll
          for (int j = 0; j < NTW; j++) Elt<T>::mma(acc[i][j], av[t][i], wv[t][j]);
    } else {
      // the batch runs past the last k-step: those steps multiply a zeroed activation fragment
#pragma unroll
      for (int t = 0; t < KW; t++) {
        const uint32_t keep = (sb + t < nsteps) ? ~0u : 0u;
#pragma unroll
        for (int i = 0; i < MW; i++) {
          const uint4 a = make_uint4(av[t][i].x & keep, av[t][i].y & keep, av[t][i].z & keep, av[t][i].w & keep);
#pragma unroll
          for (int j = 0; j < NTW; j++) Elt<T>::mma(acc[i][j], a, wv[t][j]);
        }
      }
    }
  }

  // sum the four waves' tiles in wave order; wave j finishes row tile j
#pragma unroll
  for (int i = 0; i < MW; i++)
#pragma unroll
    for (int j = 0; j < NTW; j++) red[w][i * NTW + j][lane] = acc[i][j];
  __syncthreads();
  f32x4_t sum[MW];
#pragma unroll
  for (int i = 0; i < MW; i++) {
    sum[i] = red[0][i * NTW + w][lane];
#pragma unroll
    for (int v = 1; v < 4; v++) sum[i] += red[v][i * NTW + w][lane];
  }

  const int ncol = n_tile * 64 + 16 * w + r16;
  if (EPI == EPI_PARTIAL) {
    if (ncol < g.N) {
#pragma unroll
      for (int i = 0; i < MW; i++)
#pragma unroll
        for (int r = 0; r < 4; r++) {
          const int m = m0 + 16 * i + 4 * g4 + r;
          if (m < m_valid) g.partial[((long)split * g.M + m) * g.N + ncol] = sum[i][r];
        }
    }
  } else {  // EPI_ARGMAX (SK == 1): per row, max over this row tile's 16 columns
    const int tile16 = (n_tile * 64 + 16 * w) / 16;
    const int n_t16 = (g.N + 15) / 16;
#pragma unroll
    for (int i = 0; i < MW; i++)
#pragma unroll
      for (int r = 0; r < 4; r++) {
        const int m = m0 + 16 * i + 4 * g4 + r;
        float v = sum[i][r];
        int ix = ncol;
        if (ncol >= g.N) { v = -INFINITY; ix = 0x7fffffff; }
        if (g.C && m < m_valid && ncol < g.N) ((float*)g.C)[(long)m * g.ldc + ncol] = v;
#pragma unroll
        for (int o = 8; o > 0; o >>= 1) {
          const float v2 = __shfl_xor(v, o, 16);
          const int i2 = __shfl_xor(ix, o, 16);
          if (v2 > v || (v2 == v && i2 < ix)) { v = v2; ix = i2; }
        }
        if (r16 == 0 && m < m_valid && tile16 < n_t16) {
          g.amax_val[(long)m * n_t16 + tile16] = v;
          g.amax_idx[(long)m * n_t16 + tile16] = ix;
        }
      }
  }
}

template <typename T, int MW, int KW, int EPI>
static int dec_one(const GemmArgs& g, hipStream_t st) {
  const int n_tiles = (g.N + 63) / 64;
  const int m_blocks = (g.M + 16 * MW - 1) / (16 * MW);
  hipLaunchKernelGGL((k_gemm_dec<T, MW, KW, EPI>), dim3(n_tiles * g.SK, m_blocks), dim3(256), 0, st, g);
  return hipGetLastError() == hipSuccess ? 0 : -1;
}

template <typename T, int EPI>
static int dec_kw(int MW, int KW, const GemmArgs& g, hipStream_t st) {
#define CDB_DEC_CASE(mw, kw) if (MW == mw && KW == kw) return dec_one<T, mw, kw, EPI>(g, st);
  CDB_DEC_CASE(1, 2) CDB_DEC_CASE(1, 4) CDB_DEC_CASE(1, 8)
  CDB_DEC_CASE(2, 2) CDB_DEC_CASE(2, 4) CDB_DEC_CASE(2, 6)
  CDB_DEC_CASE(4, 2) CDB_DEC_CASE(4, 4)
#undef CDB_DEC_CASE
  return -2;
}

// k-steps per wave: the largest allowed for this row-tile count (register
// budget) that still gives at least `target` workgroups, else the smallest.
int dec_wave_steps(int MW, int M, int N, int K, int dtype) {
  const int ks = dtype == 0 ? 16 : 32;
  const int nsteps = K / ks;
  const int n_tiles = (N + 63) / 64;
  const int m_blocks = (M + 16 * MW - 1) / (16 * MW);   // workgroups along the rows
  const int target = M <= 16 ? 512 : 256;
  const int opts1[3] = {8, 4, 2}, opts2[3] = {6, 4, 2}, opts4[2] = {4, 2};
  const int* opts = MW == 1 ? opts1 : (MW == 2 ? opts2 : opts4);
  const int nopt = MW == 4 ? 2 : 3;
  for (int o = 0; o < nopt; o++) {
    const int sk = (nsteps + 4 * opts[o] - 1) / (4 * opts[o]);
    if ((long)n_tiles * sk * m_blocks >= target) return opts[o];
  }
  return opts[nopt - 1];
}

int gemm_dec_launch(int dtype, int epi, int MW, int KW, const GemmArgs& g, hipStream_t st) {
  // up to 256 rows; the LM head (argmax, no split partials) up to 1024
  if (g.M < 1 || g.M > (epi == EPI_ARGMAX ? 1024 : 256) || (MW == 1 && g.M > 16) || (MW == 2 && g.M > 64)) return -2;
  const int per_split = 4 * KW * std::max(g.dec_batches, 1);
  if (g.SK != (g.K / (dtype == 0 ? 16 : 32) + per_split - 1) / per_split) return -2;
  if (epi == EPI_ARGMAX && g.SK != 1) return -2;
  if (dtype == 0) {
    if (epi == EPI_PARTIAL) return dec_kw<float, EPI_PARTIAL>(MW, KW, g, st);
    if (epi == EPI_ARGMAX) return dec_kw<float, EPI_ARGMAX>(MW, KW, g, st);
  } else {
    if (epi == EPI_PARTIAL) return dec_kw<bf16_t, EPI_PARTIAL>(MW, KW, g, st);
    if (epi == EPI_ARGMAX) return dec_kw<bf16_t, EPI_ARGMAX>(MW, KW, g, st);
  }
  return -2;
}

// Decode gate/up projection fused with SwiGLU (M <= 64), no K split.
//
// The split decode GEMM above writes fp32 partials that a SwiGLU kernel then
// sums; here one workgroup owns 32 outputs for the whole reduction: the
// packed tiles of gate rows 2t, 2t+1 and up rows 2t, 2t+1 (16 rows each),
// with wave w taking a contiguous quarter of the k-steps in batches of KW.
// The next batch's loads are issued before the current batch's MFMAs, with no
// branch between them, so the compiler's waits count only the older batch
// (steps past the wave's range re-read its last step, a cache hit, and are
// multiplied as zeros).  The four waves' tiles are summed through LDS in
// wave order; wave w then finishes gate tile w & 1 with the up tile of the
// same columns for row tiles (w >> 1) + 2q, and writes silu(gate) * up.
// Against split GEMM + SwiGLU at M = 64 on the Ouro-like MLP: 14.7 vs
// 19.9 us; fewer workgroups (F / 32), but no partials and one launch less.
// With g.ss the input rows are g * x without their RMSNorm scale: each wave
// forms the scale of 4 * MW of the workgroup's rows from the producer's
// partial sums of squares (loads issued ahead of the first weight batch,
// summed while it is in flight) and the epilogue applies it to gate and up
// before the SwiGLU.  SS = 1 takes up to 256 partials per row (per 8
// columns, from the fused residual projections), SS = 2 up to 16 (per 256
// columns, from the deferred residual add): one load per lane and row.
template <typename T, int MW, int KW, int SS>
__global__ __launch_bounds__(256) void k_gemm_dec_glu(GemmArgs g) {
  typedef typename Elt<T>::raw raw;
  constexpr int VEC = Elt<T>::VEC, KS = Elt<T>::KSTEP, NTW = 4;
  __shared__ f32x4_t red[4][MW * NTW][64];
  const int n_tile = blockIdx.x;
  const int m0 = blockIdx.y * 16 * MW;               // this workgroup's block of 16 * MW rows
  if (blockIdx.y > 0 && m0 >= ld_nvalid(g.n_valid, g.M)) return;   // an empty later row block
  const int lane = threadIdx.x & 63, r16 = lane & 15, g4 = lane >> 4;
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);   // wave-uniform: scalar loop control
  const int nsteps = g.K / KS;
  const int per_w = (nsteps + 3) / 4;
  const int sbeg = w * per_w, send = min(sbeg + per_w, nsteps);
  const raw* A = (const raw*)g.A;
  const raw* W = (const raw*)g.W;
  const long a_step = g.a_packed ? 64L * VEC : KS;
  const raw* arow[MW];
#pragma unroll
  for (int i = 0; i < MW; i++) {
    const int m = min(m0 + 16 * i + r16, g.M - 1);
    arow[i] = g.a_packed ? A + ((long)(m >> 4) * nsteps * 64 + (m & 15) + 16 * g4) * VEC
                         : A + (long)m * g.lda + g4 * VEC;
  }
  const raw* wt[NTW];
#pragma unroll
  for (int j = 0; j < NTW; j++) {
    const int nt = (j < 2 ? 0 : (g.up_off >> 4)) + 2 * n_tile + (j & 1);
    wt[j] = W + ((long)nt * nsteps * 64 + lane) * VEC;
  }
  f32x4_t acc[MW][NTW];
#pragma unroll
  for (int i = 0; i < MW; i++)
#pragma unroll
    for (int j = 0; j < NTW; j++) acc[i][j] = (f32x4_t){0.f, 0.f, 0.f, 0.f};
  uint4 av0[KW][MW], wv0[KW][NTW], av1[KW][MW], wv1[KW][NTW];
  const int last = max(send - 1, 0);
  auto load = [&](uint4 (&av)[KW][MW], uint4 (&wv)[KW][NTW], int sb) __attribute__((always_inline)) {
#pragma unroll
    for (int t = 0; t < KW; t++) {
      const int st = min(sb + t, last);
#pragma unroll
      for (int j = 0; j < NTW; j++) wv[t][j] = ldg_u4(wt[j] + (long)st * 64 * VEC);
#pragma unroll
      for (int i = 0; i < MW; i++) av[t][i] = ldg_u4(arow[i] + (long)st * a_step);
    }
  };
  // row scales (SS: the input rows lack them): the 16-lane group g4 of wave
  // w takes the MW rows from 4 * MW * w + MW * g4, lane r16 adding parts
  // r16, r16 + 16, ... (<= 256 parts) before a DPP sum over the group.  The
  // loads go out ahead of the first two weight batches, so the wait before
  // the sums leaves the batches in flight.
  constexpr int RPW = 4 * MW, PPL = SS == 1 ? kMaxSsParts / 16 : 1;   // SS 2: at most 16 parts per row
  __shared__ float rs[16 * MW];
  const int nss = g.ss_n;
  float sv[MW][PPL];
  if constexpr (SS) {
#pragma unroll
    for (int j = 0; j < MW; j++) {
      const int m = min(m0 + RPW * w + MW * g4 + j, g.M - 1);
#pragma unroll
      for (int u = 0; u < PPL; u++) sv[j][u] = g.ss[(long)m * nss + min(r16 + 16 * u, nss - 1)];
    }
  }
  __builtin_amdgcn_sched_barrier(0);
  auto compute = [&](uint4 (&av)[KW][MW], uint4 (&wv)[KW][NTW], int sb) __attribute__((always_inline)) {
    if (sb + KW <= send) {
#pragma unroll
      for (int t = 0; t < KW; t++)
#pragma unroll
        for (int i = 0; i < MW; i++)
#pragma unroll
          for (int j = 0; j < NTW; j++) Elt<T>::mma(acc[i][j], av[t][i], wv[t][j]);
    } else {
#pragma unroll
      for (int t = 0; t < KW; t++) {
        const uint32_t keep = (sb + t < send) ? ~0u : 0u;
#pragma unroll
        for (int i = 0; i < MW; i++) {
          const uint4 a = make_uint4(av[t][i].x & keep, av[t][i].y & keep, av[t][i].z & keep, av[t][i].w & keep);
#pragma unroll
          for (int j = 0; j < NTW; j++) Elt<T>::mma(acc[i][j], a, wv[t][j]);
        }
      }
    }
  };
  // the row scales: SS = 1 sums its 16 loads per lane and row up front (so
  // their registers are free for the loop), SS = 2 after the loop, when its
  // one load per lane and row has long landed
  auto row_scales = [&]() __attribute__((always_inline)) {
#pragma unroll
    for (int j = 0; j < MW; j++) {
      float t = 0.f;
#pragma unroll
      for (int u = 0; u < PPL; u++) t += r16 + 16 * u < nss ? sv[j][u] : 0.f;
      t = sum16(t);
      if (r16 == 0) rs[RPW * w + MW * g4 + j] = 1.0f / sqrtf(t / (float)g.ss_h + g.eps);
    }
  };
  if constexpr (SS == 1) {
    // both buffers in flight before the sums wait for the row-scale loads
    load(av0, wv0, sbeg);
    load(av1, wv1, sbeg + KW);
    __builtin_amdgcn_sched_barrier(0);
    row_scales();
    for (int sb = sbeg; sb < send; sb += 2 * KW) {
      compute(av0, wv0, sb);
      load(av0, wv0, sb + 2 * KW);
      __builtin_amdgcn_sched_barrier(0);
      compute(av1, wv1, sb + KW);
      load(av1, wv1, sb + 3 * KW);
      __builtin_amdgcn_sched_barrier(0);
    }
  } else {
    load(av0, wv0, sbeg);
    for (int sb = sbeg; sb < send; sb += 2 * KW) {
      load(av1, wv1, sb + KW);
      __builtin_amdgcn_sched_barrier(0);
      compute(av0, wv0, sb);
      load(av0, wv0, sb + 2 * KW);
      __builtin_amdgcn_sched_barrier(0);
      compute(av1, wv1, sb + KW);
    }
    if constexpr (SS == 2) row_scales();
  }
  const int m_valid = min(ld_nvalid(g.n_valid, g.M), g.M);
#pragma unroll
  for (int i = 0; i < MW; i++)
#pragma unroll
    for (int j = 0; j < NTW; j++) red[w][i * NTW + j][lane] = acc[i][j];
  __syncthreads();
  const int c = w & 1;
  const int f = n_tile * 32 + 16 * c + r16;
#pragma unroll
  for (int q = 0; q < (MW + 1) / 2; q++) {
    const int i = (w >> 1) + 2 * q;
    if (i >= MW) break;
    f32x4_t gt = red[0][i * NTW + c][lane], up = red[0][i * NTW + 2 + c][lane];
#pragma unroll
    for (int v = 1; v < 4; v++) {
      gt += red[v][i * NTW + c][lane];
      up += red[v][i * NTW + 2 + c][lane];
    }
#pragma unroll
    for (int r = 0; r < 4; r++) {
      const int m = m0 + 16 * i + 4 * g4 + r;
      if (m < m_valid) {
        const long oi = g.a_packed ? apack_off<T>(m, f, g.N) : (long)m * g.ldc + f;
        if constexpr (SS) {
          const float sc = rs[16 * i + 4 * g4 + r];
          ((raw*)g.C)[oi] = Elt<T>::from_f32(silu_f(gt[r] * sc) * (up[r] * sc));
        } else {
          ((raw*)g.C)[oi] = Elt<T>::from_f32(silu_f(gt[r]) * up[r]);
        }
      }
    }
  }
}

// Decode residual projection with the next norm's row statistics, no K split.
//
// The split decode GEMM leaves fp32 partials that the following norm kernel
// adds to the residual stream before it normalises the row.  Here one
// workgroup owns 8 outputs n for the whole reduction (wave w takes a
// contiguous quarter of the k-steps; loads double-buffered in batches of KW),
// so the epilogue holds final values: x = resid[slot(m)][n] + acc is written
// back, and for the next RMSNorm (gain g) the unscaled input g[n] * x goes
// out fragment-packed together with sum_n x^2 over the workgroup's 8
// outputs.  The norm's 1 / rms(x) needs the whole row, so the consumer GEMM
// applies it to its outputs instead (a GEMM is linear in each row); that
// saves a launch and the partials' round trip through HBM.  Eight outputs
// (half a packed weight tile: each lane's 16 bytes lie in the half's own
// 128-byte lines) give N / 8 workgroups, so every CU streams; 16 outputs
// per workgroup left half the CUs idle at N = 2048 (O 5.7 -> 5.3 us, down
// 9.4 -> 8.9 us at one row).  Load order: slots, both weight batches, then
// the residual values (their wait for the slots overlaps the batches'
// flight).  Wave w < MW finishes row tile w.  (Eight or sixteen waves per
// workgroup, on eighths or sixteenths of the k-steps, were slower.)
//
// NSP > 0 (the O projection of a batch of one or a few rows whose attention
// ran split over the context): A is not read from memory but formed here
// from the attention's split partials (max, sum, output of every split),
// merged the way the split merge kernel merges them (the same sums in split
// order, the same rounding of the result), which saves that kernel's launch.
// Each wave merges the A pieces of its own quarter of the k-steps, one per
// lane (a 16-byte piece: one row, VEC consecutive columns of one head),
// issuing those loads before its weight batches, and passes them to the
// MFMA lanes through LDS.  Every workgroup merges the whole row again, which
// its L2 serves.  Measured at context 1024: one row 1.219 -> 1.181 ms per
// step; with two pieces per lane (two rows) no gain, with four or eight
// (four and eight rows) 8-10% slower, so the host takes this form only
// where a lane merges one piece.
template <typename T, int MW, int KW, int NSP>
__global__ __launch_bounds__(256) void k_gemm_dec_res(GemmArgs g) {
  typedef typename Elt<T>::raw raw;
  constexpr int VEC = Elt<T>::VEC, KS = Elt<T>::KSTEP;
  constexpr bool MG = NSP > 0;
  __shared__ f32x4_t red[4][MW][64];
  __shared__ uint4 pcs[MG ? 4 : 1][MG ? kMergePieces : 1];
  // eight outputs: half of the 16-row weight tile n_tile (lanes of MFMA
  // columns 8..15 re-read the rows of columns 0..7 and are not stored)
  const int n_tile = blockIdx.x >> 1;
  const int c16 = (blockIdx.x & 1) * 8 + (threadIdx.x & 7);   // this lane's row of the weight tile
  const int m0 = blockIdx.y * 16 * MW;
  if (blockIdx.y > 0 && m0 >= ld_nvalid(g.n_valid, g.M)) return;   // an empty later row block
  const int lane = threadIdx.x & 63, r16 = lane & 15, g4 = lane >> 4;
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int nsteps = g.K / KS;
  const int per_w = (nsteps + 3) / 4;
  const int sbeg = w * per_w, send = min(sbeg + per_w, nsteps);
  const raw* A = (const raw*)g.A;
  const raw* W = (const raw*)g.W;
  const raw* arow[MW];
#pragma unroll
  for (int i = 0; i < MW; i++) {
    const int m = min(m0 + 16 * i + r16, g.M - 1);
    arow[i] = MG ? nullptr : A + ((long)(m >> 4) * nsteps * 64 + (m & 15) + 16 * g4) * VEC;
  }
  const raw* wt = W + ((long)n_tile * nsteps * 64 + c16 + 16 * g4) * VEC;

  // epilogue operands: the rows of tile min(w, MW - 1) this lane finishes
  // (waves past MW load them too and skip the epilogue), the gain of its column
  const int ti = min(w, MW - 1);
  const int n = n_tile * 16 + c16;
  const bool own = r16 < 8;
  float* X = (float*)g.C;
  int srow[4];
#pragma unroll
  for (int r = 0; r < 4; r++) {
    const int m = min(m0 + 16 * ti + 4 * g4 + r, g.M - 1);
    srow[r] = g.slot ? g.slot[m] : m;
  }
  const float gn = (g.gain ? g.gain : (const float*)X)[n];
  __builtin_amdgcn_sched_barrier(0);

  f32x4_t acc[MW];
#pragma unroll
  for (int i = 0; i < MW; i++) acc[i] = (f32x4_t){0.f, 0.f, 0.f, 0.f};
  uint4 av0[KW][MW], wv0[KW], av1[KW][MW], wv1[KW];
  const int last = max(send - 1, 0);
  // merged pieces: piece p of this wave is row p % mr, k-step sbeg + (p / mr) / 4,
  // columns VEC * ((p / mr) % 4) of that step
  const int mr = min(g.M, 16);
  auto a_frag = [&](int st) __attribute__((always_inline)) -> uint4 {
    return pcs[w][min(r16, mr - 1) + mr * (4 * (st - sbeg) + g4)];
  };
  auto load = [&](uint4 (&av)[KW][MW], uint4 (&wv)[KW], int sb) __attribute__((always_inline)) {
#pragma unroll
    for (int t = 0; t < KW; t++) {
      const int st = min(sb + t, last);
      wv[t] = ldg_u4(wt + (long)st * 64 * VEC);
      if constexpr (!MG) {
#pragma unroll
        for (int i = 0; i < MW; i++) av[t][i] = ldg_u4(arow[i] + (long)st * 64 * VEC);
      }
    }
  };
  auto compute = [&](uint4 (&av)[KW][MW], uint4 (&wv)[KW], int sb) __attribute__((always_inline)) {
    if constexpr (MG) {
#pragma unroll
      for (int t = 0; t < KW; t++) av[t][0] = a_frag(min(sb + t, last));
    }
    if (sb + KW <= send) {
#pragma unroll
      for (int t = 0; t < KW; t++)
#pragma unroll
        for (int i = 0; i < MW; i++) Elt<T>::mma(acc[i], av[t][i], wv[t]);
    } else {
#pragma unroll
      for (int t = 0; t < KW; t++) {
        const uint32_t keep = (sb + t < send) ? ~0u : 0u;
#pragma unroll
        for (int i = 0; i < MW; i++) {
          const uint4 a = make_uint4(av[t][i].x & keep, av[t][i].y & keep, av[t][i].z & keep, av[t][i].w & keep);
          Elt<T>::mma(acc[i], a, wv[t]);
        }
      }
    }
  };
  // the merge's loads go out first (its math then waits for them only), then
  // the weight batches, whose flight the merge math overlaps
  // this lane's piece p = lane (at most 64 per wave; clamped into the wave's
  // pieces and k-steps, an unused lane's loads are never stored)
  const int npc = MG ? mr * max(send - sbeg, 0) * 4 : 0;
  float sm[MG ? NSP : 1], sl[MG ? NSP : 1], ov[MG ? NSP : 1][VEC];
  if constexpr (MG) {
    const int p = min(lane, max(npc - 1, 0));
    const int r = p % mr, tq = p / mr;
    const int c0 = min(sbeg + (tq >> 2), nsteps - 1) * KS + (tq & 3) * VEC;
    const int hd = g.attn_hd, ns = g.attn_ns;
    const float* pb = g.attn_part + ((long)r * g.attn_nh + c0 / hd) * ns * (hd + 2);
#pragma unroll
    for (int u = 0; u < NSP; u++) {
      // a split's record starts 8-byte aligned (hd + 2 floats, hd % VEC == 0)
      const float* ps = pb + (long)min(u, ns - 1) * (hd + 2);
      const float2 st2 = *(const float2*)ps;
      sm[u] = st2.x;
      sl[u] = st2.y;
#pragma unroll
      for (int e = 0; e < VEC; e += 2) {
        const float2 o2 = *(const float2*)(ps + 2 + c0 % hd + e);
        ov[u][e] = o2.x;
        ov[u][e + 1] = o2.y;
      }
    }
  }
  __builtin_amdgcn_sched_barrier(0);
  load(av0, wv0, sbeg);
  load(av1, wv1, sbeg + KW);
  __builtin_amdgcn_sched_barrier(0);
  // residual values (slots clamped silently here; a valid row's bad slot is
  // reported at its store)
  float xo[4];
#pragma unroll
  for (int r = 0; r < 4; r++) xo[r] = X[(long)min(max(srow[r], 0), g.slot_max - 1) * g.ldc + n];
  __builtin_amdgcn_sched_barrier(0);
  if constexpr (MG) {
    // max over the splits, then sum and output in split order; a split with
    // no positions (max -inf) adds nothing
    const int ns = g.attn_ns;
    float mm = -INFINITY;
#pragma unroll
    for (int u = 0; u < NSP; u++)
      if (u < ns) mm = fmaxf(mm, sm[u]);
    float ll = 0.f, oo[VEC];
#pragma unroll
    for (int e = 0; e < VEC; e++) oo[e] = 0.f;
#pragma unroll
    for (int u = 0; u < NSP; u++) {
      if (u >= ns || sm[u] == -INFINITY) continue;
      const float f = __expf(sm[u] - mm);
      ll += sl[u] * f;
#pragma unroll
      for (int e = 0; e < VEC; e++) oo[e] += ov[u][e] * f;
    }
    raw pv[VEC];
#pragma unroll
    for (int e = 0; e < VEC; e++) pv[e] = Elt<T>::from_f32(oo[e] / ll);
    uint4 pu;
    __builtin_memcpy(&pu, pv, sizeof(pu));
    if (lane < npc) pcs[w][lane] = pu;
    __syncthreads();
  }
  for (int sb = sbeg; sb < send; sb += 2 * KW) {
    compute(av0, wv0, sb);
    load(av0, wv0, sb + 2 * KW);
    __builtin_amdgcn_sched_barrier(0);
    compute(av1, wv1, sb + KW);
    load(av1, wv1, sb + 3 * KW);
    __builtin_amdgcn_sched_barrier(0);
  }
  const int m_valid = min(ld_nvalid(g.n_valid, g.M), g.M);
#pragma unroll
  for (int i = 0; i < MW; i++) red[w][i][lane] = acc[i];
  __syncthreads();
  if (w >= MW) return;
  f32x4_t sum = red[0][w][lane];
#pragma unroll
  for (int v = 1; v < 4; v++) sum += red[v][w][lane];
#pragma unroll
  for (int r = 0; r < 4; r++) {
    const int m = m0 + 16 * w + 4 * g4 + r;
    float x = 0.f;
    if (m < m_valid && own) {
      const int row = g.slot ? clamp_chk(srow[r], 0, g.slot_max - 1, g.err, ERR_SLOT) : m;
      x = xo[r] + sum[r];
      X[(long)row * g.ldc + n] = x;
      if (g.gain) ((raw*)g.Y)[apack_off<T>(m, n, g.N)] = Elt<T>::from_f32(gn * x);
    }
    float q = x * x;
#pragma unroll
    for (int o = 8; o > 0; o >>= 1) q += __shfl_xor(q, o, 16);
    if (g.gain && r16 == 0 && m < m_valid) g.ss_out[(long)m * gridDim.x + blockIdx.x] = q;
  }
}

template <typename T, int MW, int KW, int NSP>
static int res_one(const GemmArgs& g, hipStream_t st) {
  const dim3 grid(g.N / 8, (g.M + 16 * MW - 1) / (16 * MW)), block(256);
  hipLaunchKernelGGL((k_gemm_dec_res<T, MW, KW, NSP>), grid, block, 0, st, g);
  return hipGetLastError() == hipSuccess ? 0 : -1;
}

template <typename T>
static int res_kw(int MW, int KW, const GemmArgs& g, hipStream_t st) {
  if (g.attn_part) {                              // merged attention splits (one row tile)
    if (MW != 1 || KW != 8) return -2;
    if (g.attn_ns <= 8) return res_one<T, 1, 8, 8>(g, st);
    return res_one<T, 1, 8, 16>(g, st);
  }
#define CDB_RES_CASE(mw, kw) if (MW == mw && KW == kw) return res_one<T, mw, kw, 0>(g, st);
  CDB_RES_CASE(1, 8) CDB_RES_CASE(2, 8) CDB_RES_CASE(4, 4)
#undef CDB_RES_CASE
  return -2;
}

int gemm_res_merge_pieces(int dtype, int M, int K) {
  const int ks = dtype == 0 ? 16 : 32;
  const int per_w = (K / ks + 3) / 4;
  return std::min(M, 16) * per_w * 4;
}

int gemm_dec_res_launch(int dtype, int MW, int KW, const GemmArgs& g, hipStream_t st) {
  if (g.M < 1 || g.M > 256 || (MW < 4 && g.M > 16 * MW) || g.N < 16 || g.N % 16) return -2;
  if (!g.C || g.slot_max < (g.slot ? 1 : g.M) || (g.gain && (!g.Y || !g.ss_out))) return -2;
  if (g.attn_part) {
    const int vec = dtype == 0 ? 4 : 8;
    if (g.M > 16 || g.attn_ns < 2 || g.attn_ns > 16 || g.attn_hd < vec || g.attn_hd % vec || g.attn_nh < 1 ||
        g.K != g.attn_nh * g.attn_hd || g.K % (dtype == 0 ? 16 : 32) ||
        gemm_res_merge_pieces(dtype, g.M, g.K) > kMergePieces)
      return -2;
  } else if (!g.a_packed) {
    return -2;
  }
  return dtype == 0 ? res_kw<float>(MW, KW, g, st) : res_kw<bf16_t>(MW, KW, g, st);
}

template <typename T, int SS>
static int glu_mw(const GemmArgs& g, hipStream_t st) {
  const int rb = g.M <= 16 ? 16 : (g.M <= 32 ? 32 : 64);   // rows per workgroup
  const dim3 grid(g.N / 32, (g.M + rb - 1) / rb), block(256);
  if (g.M <= 16) hipLaunchKernelGGL((k_gemm_dec_glu<T, 1, 2, SS>), grid, block, 0, st, g);
  else if (g.M <= 32) hipLaunchKernelGGL((k_gemm_dec_glu<T, 2, 2, SS>), grid, block, 0, st, g);
  else hipLaunchKernelGGL((k_gemm_dec_glu<T, 4, 1, SS>), grid, block, 0, st, g);
  return hipGetLastError() == hipSuccess ? 0 : -1;
}

int gemm_dec_glu_launch(int dtype, const GemmArgs& g, hipStream_t st) {
  if (g.M < 1 || g.M > 256 || g.N % 32 || g.up_off % 16 || g.up_off < g.N) return -2;
  if (g.ss && (g.ss_n < 1 || g.ss_n > kMaxSsParts || !g.a_packed)) return -2;
  if (g.ss && g.ss_n <= 16) return dtype == 0 ? glu_mw<float, 2>(g, st) : glu_mw<bf16_t, 2>(g, st);
  if (g.ss) return dtype == 0 ? glu_mw<float, 1>(g, st) : glu_mw<bf16_t, 1>(g, st);
  return dtype == 0 ? glu_mw<float, 0>(g, st) : glu_mw<bf16_t, 0>(g, st);
}

// Row-major [rows][cols] -> fragment-packed: piece e = (tile, lane) of 16
// bytes holds row 16 * (tile / ksteps) + lane % 16, columns
// KS * (tile % ksteps) + VEC * (lane / 16) .. + VEC.
template <typename T>
__global__ __launch_bounds__(256) void k_pack_weight(const void* src, void* dst, int rows, int cols) {
  typedef typename Elt<T>::raw raw;
  constexpr int VEC = Elt<T>::VEC, KS = Elt<T>::KSTEP;
  const int ksteps = cols / KS;
  const long pieces = (long)(rows / 16) * ksteps * 64;
  for (long e = blockIdx.x * 256L + threadIdx.x; e < pieces; e += (long)gridDim.x * 256) {
    const long tile = e >> 6;
    const int lane = (int)(e & 63);
    const int n = (int)(tile / ksteps) * 16 + (lane & 15);
    const int k = (int)(tile % ksteps) * KS + (lane >> 4) * VEC;
    *(uint4*)((raw*)dst + e * VEC) = *(const uint4*)((const raw*)src + (long)n * cols + k);
  }
}

int pack_weight_launch(int dtype, const void* src, void* dst, int rows, int cols, hipStream_t st) {
  const int ks = dtype == 0 ? 16 : 32;
  if (rows <= 0 || cols <= 0 || rows % 16 || cols % ks) return -2;
  const long pieces = (long)(rows / 16) * (cols / ks) * 64;
  const int blocks = (int)std::min<long>((pieces + 255) / 256, 8192);
  if (dtype == 0) hipLaunchKernelGGL(k_pack_weight<float>, dim3(blocks), dim3(256), 0, st, src, dst, rows, cols);
  else hipLaunchKernelGGL(k_pack_weight<bf16_t>, dim3(blocks), dim3(256), 0, st, src, dst, rows, cols);
  return hipGetLastError() == hipSuccess ? 0 : -1;
}

// SwiGLU of split partials of the fused gate/up projection:
// out[m][j] = silu(sum_s P[s][m][j]) * sum_s P[s][m][F + j]
template <typename T, int R>
__global__ __launch_bounds__(256) void k_swiglu(SwigluArgs a) {
  typedef typename Elt<T>::raw raw;
  const int m = blockIdx.y;
  if (m >= min(ld_nvalid(a.n_valid, a.rows), a.rows)) return;
  const int j = blockIdx.x * 256 + threadIdx.x;
  if (j >= a.F) return;
  const float* p = a.part + (long)m * (2L * a.F);
  const long stride = (long)a.rows * (2L * a.F);
  // R splits' loads in flight per round (R = 4 when that covers the count)
  const float gt = sum_splits<R>(p + j, stride, a.sk);
  const float up = sum_splits<R>(p + a.F + j, stride, a.sk);
  const long oi = a.packed ? apack_off<T>(m, j, a.F) : (long)m * a.ldo + j;
  ((raw*)a.out)[oi] = Elt<T>::from_f32(silu_f(gt) * up);
}

int swiglu_launch(int dtype, const SwigluArgs& a, hipStream_t st) {
  dim3 grid((a.F + 255) / 256, a.rows);
  const bool r4 = a.sk <= 4;
  if (dtype == 0) {
    if (r4) hipLaunchKernelGGL((k_swiglu<float, 4>), grid, dim3(256), 0, st, a);
    else hipLaunchKernelGGL((k_swiglu<float, 8>), grid, dim3(256), 0, st, a);
  } else {
    if (r4) hipLaunchKernelGGL((k_swiglu<bf16_t, 4>), grid, dim3(256), 0, st, a);
    else hipLaunchKernelGGL((k_swiglu<bf16_t, 8>), grid, dim3(256), 0, st, a);
  }
  return hipGetLastError() == hipSuccess ? 0 : -1;
}

}  // namespace cdb
