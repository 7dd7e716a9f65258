// MFMA GEMM for the core and boundary projections: C[M][N] = A[M][K] . W[N][K]^T
// (weights in [out][in] layout), fp32 accumulation, fused epilogues.
//
// Design (decode-shaped GEMMs are weight-streaming, HBM-bound below M ~ 300):
//  - one workgroup = 4 waves computes a (16*MW) x (16*NW) output tile; the
//    four waves split the workgroup's K range four ways and their partial
//    tiles are summed through LDS in fixed wave order;
//  - grid.y splits K across SK workgroups when the N-tiles alone cannot fill
//    256 CUs; the last workgroup to finish a tile (integer counter) sums the
//    SK partials in split order and runs the epilogue, so results do not
//    depend on arrival order;
//  - operands go straight from global memory into MFMA fragments (16 B per
//    lane per fragment); weights are streamed exactly once per M-tile, and
//    the M-tiles of one N-tile are placed on the same XCD so the second read
//    hits that XCD's L2;
//  - epilogues: store fp32, store T, residual add into the fp32 loop state
//    through the slot table, SwiGLU (gate and up tiles of the same columns),
//    and greedy argmax over the vocabulary (lowest index among equal maxima).
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
  const int tile = n_tile * g.m_tiles + m_tile;
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
  const raw* wrow[NWX];
#pragma unroll
  for (int j = 0; j < NWX; j++) {
    int n = n0 + 16 * (j % NW) + r16;
    n = n < g.N ? n : g.N - 1;
    if (SWI && j >= NW) n += g.up_off;           // up rows follow the gate rows
    wrow[j] = W + (long)n * g.ldw + g4 * VEC;
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
      for (int j = 0; j < NWX; j++) b[u][j] = *(const uint4*)(wrow[j] + k);
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
    for (int j = 0; j < NWX; j++) b[j] = *(const uint4*)(wrow[j] + k);
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

  // ---- split-K across workgroups: last arriver reduces in split order ----
  if (g.SK > 1) {
    float* part = g.partial + ((long)tile * g.SK) * (MT * NTX);
#pragma unroll
    for (int p = 0; p < PER; p++) {
      const int e = threadIdx.x + 256 * p;
      if (e < MT * NTX) part[(long)split * MT * NTX + e] = v[p];
    }
    __threadfence();
    __syncthreads();                             // red[] fully consumed into v[]
    int* flag = (int*)lds;
    if (threadIdx.x == 0) {
      const int old = atomicAdd(&g.counters[tile], 1);
      flag[0] = (old == g.SK - 1);
      if (old == g.SK - 1) g.counters[tile] = 0;   // self-reset for the next launch
    }
    __syncthreads();
    if (!flag[0]) return;
    __threadfence();
#pragma unroll
    for (int p = 0; p < PER; p++) {
      const int e = threadIdx.x + 256 * p;
      float t = 0.f;
      if (e < MT * NTX)
        for (int q = 0; q < g.SK; q++) t += __builtin_nontemporal_load(part + (long)q * MT * NTX + e);
      v[p] = t;
    }
  }

  // ---- epilogues ----
  if (EPI == EPI_STORE_F32 || EPI == EPI_STORE_T || EPI == EPI_RESID) {
#pragma unroll
    for (int p = 0; p < PER; p++) {
      const int e = threadIdx.x + 256 * p;
      const int row = e / NT, col = e % NT;
      const int m = m0 + row, n = n0 + col;
      if (e >= MT * NT || n >= g.N || m >= m_valid) continue;
      if (EPI == EPI_STORE_F32) {
        ((float*)g.C)[(long)m * g.ldc + n] = v[p];
      } else if (EPI == EPI_STORE_T) {
        ((raw*)g.C)[(long)m * g.ldc + n] = Elt<T>::from_f32(v[p]);
      } else {
        const int r = g.slot ? min(max(g.slot[m], 0), g.slot_max - 1) : m;
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
    // optional logits, then per-row (max, index) of this tile's columns;
    // the last tile of an M-tile scans the per-tile results in column order
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
    __threadfence();
    __syncthreads();                             // red[] read by the row scans above
    int* flag = (int*)lds;
    if (threadIdx.x == 0) {
      const int old = atomicAdd(&g.counters2[m_tile], 1);
      flag[0] = (old == n_tiles_n - 1);
      if (old == n_tiles_n - 1) g.counters2[m_tile] = 0;
    }
    __syncthreads();
    if (!flag[0]) return;
    __threadfence();
    if (threadIdx.x < MT) {
      const int m = m0 + threadIdx.x;
      if (m < m_valid) {
        float best = -INFINITY;
        int bi = -1;
        for (int t = 0; t < n_tiles_n; t++) {
          const float x = __builtin_nontemporal_load(g.amax_val + (long)m * n_tiles_n + t);
          const int ix = __builtin_nontemporal_load(g.amax_idx + (long)m * n_tiles_n + t);
          if (bi < 0 || x > best) { best = x; bi = ix; }
        }
        g.tok_out[m] = bi;
      }
    }
  }
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
  }
  if (dtype == 0) { CDB_EPI(float) } else { CDB_EPI(bf16_t) }
#undef CDB_EPI
  return -2;
}

}  // namespace cdb
