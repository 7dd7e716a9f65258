// Prefill-side attention kernels: the rotary table, the K/V write of a
// prompt chunk, and causal attention of the chunk over the paged cache at one
// plane (full depth, "Depth-adaptive Inference of Looped Language Models via
// Continuous Depth Batching", App. A.1 "Chunked prefill").
#include <algorithm>

#include "common.h"
#include "kernels.h"
#include "attn_common.h"

namespace cdb {

// Rotary table: entry (pos, i) = (cos, sin) of pos * theta^(-2i/hd), the
// angle formed and evaluated in double and rounded once to float.  Every
// kernel that rotates q or k reads it instead of evaluating the angle.
__global__ void k_rope_table(float2* t, int rows, int hd, double theta) {
  const int half = hd / 2;
  const long n = (long)rows * half;
  for (long e = blockIdx.x * (long)blockDim.x + threadIdx.x; e < n; e += (long)gridDim.x * blockDim.x) {
    const int pos = (int)(e / half), i = (int)(e % half);
    const double ang = (double)pos * pow(theta, -(2.0 * (double)i) / (double)hd);
    t[e] = make_float2((float)cos(ang), (float)sin(ang));
  }
}

// K/V of a prompt chunk into the cache: one workgroup per row, each thread
// a group of four consecutive elements (16-byte loads of the fp32 split
// partials, one rotary pair of groups per thread for K).
template <typename T, int HD>
__global__ __launch_bounds__(256) void k_kv_write(KvWriteArgs a) {
  typedef typename Elt<T>::raw raw;
  constexpr int HALF = HD / 2, G = HALF / 4;     // groups of four per half
  static_assert(HALF % 4 == 0, "head_dim");
  const int r = blockIdx.x;
  if (r >= a.rows) return;
  const int p = min(max(a.pos[r], 0), a.max_pos - 1);
  const int seq = min(max(a.seq[r], 0), a.max_seqs - 1);
  const int Q = a.nh * HD;
  const int blk = min(max(a.btab[(long)seq * a.bt_stride + (p >> 4)], 0), a.num_blocks - 1), off = p & 15;
  const float* row = a.qkv + (long)r * a.ldq;
  const long split = (long)a.rows * a.ldq;
  auto load4 = [&](int col) -> float4 {          // the splits of four columns, summed in split order
    float4 v = *(const float4*)(row + col);
    for (int sp = 1; sp < a.qkv_sk; sp++) {
      const float4 w = *(const float4*)(row + sp * split + col);
      v.x += w.x; v.y += w.y; v.z += w.z; v.w += w.w;
    }
    return v;
  };
  auto store4 = [&](void* pool, long idx, float e0, float e1, float e2, float e3) {
    raw* d = (raw*)pool + idx;
    if (sizeof(raw) == 2) {
      *(uint2*)d = make_uint2(cvt_bf16x2(e0, e1), cvt_bf16x2(e2, e3));
    } else {
      *(float4*)d = make_float4(e0, e1, e2, e3);
    }
  };
  for (int t = threadIdx.x; t < a.nh * G; t += blockDim.x) {   // K: rotate-half pairs (i, i + HALF)
    const int h = t / G, i0 = (t % G) * 4;
    const float4 lo = load4(Q + h * HD + i0), hi = load4(Q + h * HD + HALF + i0);
    const float4 c01 = *(const float4*)(a.rope + (long)p * HALF + i0);      // (cos, sin) of i0, i0 + 1
    const float4 c23 = *(const float4*)(a.rope + (long)p * HALF + i0 + 2);  // of i0 + 2, i0 + 3
    const long idx = ((((long)blk * a.nh + h) * a.planes + a.plane) * 16 + off) * HD + i0;
    store4(a.kpool, idx, lo.x * c01.x - hi.x * c01.y, lo.y * c01.z - hi.y * c01.w,
           lo.z * c23.x - hi.z * c23.y, lo.w * c23.z - hi.w * c23.w);
    store4(a.kpool, idx + HALF, hi.x * c01.x + lo.x * c01.y, hi.y * c01.z + lo.y * c01.w,
           hi.z * c23.x + lo.z * c23.y, hi.w * c23.z + lo.w * c23.w);
  }
  for (int t = threadIdx.x; t < Q / 4; t += blockDim.x) {      // V
    const int h = (4 * t) / HD, i0 = (4 * t) % HD;
    const float4 v = load4(2 * Q + 4 * t);
    const long idx = ((((long)blk * a.nh + h) * a.planes + a.plane) * 16 + off) * HD + i0;
    store4(a.vpool, idx, v.x, v.y, v.z, v.w);
  }
}

template <typename T, int HD>
static int kvw_one(const KvWriteArgs& a, hipStream_t st) {
  if (a.rows <= 0) return 0;
  hipLaunchKernelGGL((k_kv_write<T, HD>), dim3(a.rows), dim3(256), 0, st, a);
  return hipGetLastError() == hipSuccess ? 0 : -1;
}

int kv_write_launch(int dtype, int hd, const KvWriteArgs& a, hipStream_t st) {
  if (dtype == 0) {
    if (hd == 64) return kvw_one<float, 64>(a, st);
    if (hd == 32) return kvw_one<float, 32>(a, st);
    if (hd == 16) return kvw_one<float, 16>(a, st);
  } else {
    if (hd == 128) return kvw_one<bf16_t, 128>(a, st);
    if (hd == 96) return kvw_one<bf16_t, 96>(a, st);
    if (hd == 64) return kvw_one<bf16_t, 64>(a, st);
    if (hd == 16) return kvw_one<bf16_t, 16>(a, st);
  }
  return -2;
}

}  // namespace cdb

// ---------------------------------------------------------------------------
// Prefill attention (full depth, App. A.1 "Chunked prefill"): the queries of
// one prompt chunk attend causally to every cached position of their
// sequence at one plane (prompt positions all have e_j = r_max, so at loop d
// the depth-indexed read plane is d for every position; the single-slot
// cache has one plane).  K/V of the chunk were written by k_kv_write.
//
// One workgroup per (tile of up to 32 consecutive query tokens of one
// sequence, head).  Key/value blocks of 64 positions are staged in LDS once
// and shared by the tile's 32 queries, so each K/V byte is read once per
// tile instead of once per query.
namespace cdb {

template <typename T, int HD>
__global__ __launch_bounds__(256) void k_attn_prefill(PrefillAttnArgs a) {
  typedef typename Elt<T>::raw raw;
  constexpr int QT = 32, KB = 64;
  constexpr int HALF = HD / 2;
  __shared__ float qs[QT][HD + 1];
  __shared__ float ks[KB][HD + 1];
  __shared__ float vs[KB][HD + 1];
  __shared__ float ps[QT][KB + 1];
  __shared__ float mrow[QT], lrow[QT], corr[QT];
  __shared__ int blk_s[KB / 16];

  const int tile = blockIdx.x / a.nh, h = blockIdx.x % a.nh;
  const int2 td = a.tiles[tile];                   // (first row, rows)
  const int r0 = td.x, nq = td.y;
  const int seq = min(max(a.seq[r0], 0), a.max_seqs - 1);
  const int* bt = a.btab + (long)seq * a.bt_stride;
  const int pmax = min(a.pos[r0 + nq - 1], a.max_pos - 1);

  // rotated, scaled queries of the tile
  for (int e = threadIdx.x; e < QT * HD; e += 256) {
    const int qi = e / HD, i = e % HD;
    float v = 0.f;
    if (qi < nq) {
      const int r = r0 + qi;
      const int p = min(max(a.pos[r], 0), a.max_pos - 1);
      const int ii = i < HALF ? i : i - HALF, ip = i < HALF ? i + HALF : i - HALF;
      const float2 cs = a.rope[(long)p * HALF + ii];
      const float c = cs.x, s = cs.y;
      const float x = qkv_at(a.qkv, a.qkv_sk, a.rows, a.ldq, r, h * HD + i);
      const float y = qkv_at(a.qkv, a.qkv_sk, a.rows, a.ldq, r, h * HD + ip);
      v = ((i < HALF) ? (x * c - y * s) : (x * c + y * s)) * a.scale;
    }
    qs[qi][i] = v;
  }
  if (threadIdx.x < QT) { mrow[threadIdx.x] = -INFINITY; lrow[threadIdx.x] = 0.f; }
  // output accumulators: thread t owns query row t / 8 and 16 dims ((t % 8) * HD/8 ..)
  constexpr int DPT = HD / 8;
  const int oq = threadIdx.x >> 3, od0 = (threadIdx.x & 7) * DPT;
  float o[DPT];
#pragma unroll
  for (int k = 0; k < DPT; k++) o[k] = 0.f;

  const raw* kp = (const raw*)a.kpool;
  const raw* vp = (const raw*)a.vpool;
  for (int j0 = 0; j0 <= pmax; j0 += KB) {
    __syncthreads();
    if (threadIdx.x < KB / 16) {
      const int lb = (j0 >> 4) + threadIdx.x;
      blk_s[threadIdx.x] = (j0 + 16 * threadIdx.x <= pmax) ? min(max(bt[lb], 0), a.num_blocks - 1) : 0;
    }
    __syncthreads();
    // stage K and V of positions j0 .. j0+KB-1 (16 B per load)
    constexpr int EPL = 16 / sizeof(raw);
    for (int e = threadIdx.x; e < KB * (HD / EPL); e += 256) {
      const int jj = e / (HD / EPL), c = (e % (HD / EPL)) * EPL;
      const int j = j0 + jj;
      float kf[EPL], vf[EPL];
      if (j <= pmax) {
        const long idx = ((((long)blk_s[jj >> 4] * a.nh + h) * a.planes + a.plane) * 16 + (j & 15)) * HD + c;
        unpack16(*(const uint4*)(kp + idx), kf, T());
        unpack16(*(const uint4*)(vp + idx), vf, T());
      } else {
#pragma unroll
        for (int k = 0; k < EPL; k++) { kf[k] = 0.f; vf[k] = 0.f; }
      }
#pragma unroll
      for (int k = 0; k < EPL; k++) { ks[jj][c + k] = kf[k]; vs[jj][c + k] = vf[k]; }
    }
    __syncthreads();
    // scores: thread t computes query t / 8, keys (t % 8) + 8k
    {
      const int qi = threadIdx.x >> 3, kk0 = threadIdx.x & 7;
      const int pq = (qi < nq) ? a.pos[r0 + qi] : -1;
      float sc[KB / 8];
#pragma unroll
      for (int k = 0; k < KB / 8; k++) sc[k] = 0.f;
      for (int i = 0; i < HD; i++) {
        const float qv = qs[qi][i];
#pragma unroll
        for (int k = 0; k < KB / 8; k++) sc[k] += qv * ks[kk0 + 8 * k][i];
      }
      float mx = -INFINITY;
#pragma unroll
      for (int k = 0; k < KB / 8; k++) {
        const int j = j0 + kk0 + 8 * k;
        if (j > pq) sc[k] = -INFINITY;              // causal (and padding rows)
        mx = fmaxf(mx, sc[k]);
      }
#pragma unroll
      for (int off = 4; off > 0; off >>= 1) mx = fmaxf(mx, __shfl_xor(mx, off, 8));
      const float m_old = mrow[qi];
      const float m_new = fmaxf(m_old, mx);
      float sum = 0.f;
#pragma unroll
      for (int k = 0; k < KB / 8; k++) {
        const float p = (m_new == -INFINITY) ? 0.f : __expf(sc[k] - m_new);
        ps[qi][kk0 + 8 * k] = p;
        sum += p;
      }
#pragma unroll
      for (int off = 4; off > 0; off >>= 1) sum += __shfl_xor(sum, off, 8);
      __syncthreads();                              // every lane of the row read m_old
      if (kk0 == 0) {
        const float cf = (m_old == -INFINITY) ? 0.f : __expf(m_old - m_new);
        corr[qi] = cf;
        lrow[qi] = lrow[qi] * cf + sum;
        mrow[qi] = m_new;
      }
    }
    __syncthreads();
    {
      const float cf = corr[oq];
#pragma unroll
      for (int k = 0; k < DPT; k++) o[k] *= cf;
      for (int jj = 0; jj < KB; jj++) {
        const float p = ps[oq][jj];
#pragma unroll
        for (int k = 0; k < DPT; k++) o[k] += p * vs[jj][od0 + k];
      }
    }
  }
  __syncthreads();
  if (oq < nq) {
    const float inv = 1.f / lrow[oq];
    raw* out = (raw*)a.out + (long)(r0 + oq) * a.ldo + h * HD + od0;
#pragma unroll
    for (int k = 0; k < DPT; k++) out[k] = Elt<T>::from_f32(o[k] * inv);
  }
}

// K / V of one 64-key block for the MFMA prefill kernels (expanded inside
// them: they name the kernel's staging registers, masks and LDS tiles).
// Loads of the block's K rows and V key pairs into registers; the block's
// four 16-position pages are looked up once per block (the same for the whole
// workgroup, so scalar loads and scalar address arithmetic); a page past the
// tile's last position re-reads the last page, so every load stays inside a
// page of this sequence, and the chunks of positions past pmax are zeroed
// when stored to LDS, via the masks.
__device__ __forceinline__ long pf_sel4(long p0, long p1, long p2, long p3, int i) {
  long r = p0;                                   // selects, not branches: i differs across lanes
  r = (i == 1) ? p1 : r;
  r = (i == 2) ? p2 : r;
  r = (i == 3) ? p3 : r;
  return r;
}
#define CDB_PF_LOAD(j0)                                                                  \
  {                                                                                      \
    const int pg0 = (j0) >> 4;                                                           \
    const long o0 = page_off(pg0), o1 = page_off(pg0 + 1), o2 = page_off(pg0 + 2), o3 = page_off(pg0 + 3); \
    _Pragma("unroll") for (int c = 0; c < KCH; c++) {                                    \
      const int e = min(tid + 256 * c, NKC - 1);                                         \
      const int row = e / (HD / 8);                                                      \
      /* head_dim 128: chunk c covers rows 16c .. 16c + 15, one page for the workgroup */ \
      const long po = HD == 128 ? pf_sel4(o0, o1, o2, o3, c) : pf_sel4(o0, o1, o2, o3, row >> 4); \
      kr[c] = *(gu32x4*)(kp + po + (row & 15) * HD + (e % (HD / 8)) * 8);               \
    }                                                                                    \
    _Pragma("unroll") for (int c = 0; c < VCH; c++) {                                    \
      const int e = min(tid + 256 * c, NVC - 1);                                         \
      const int row = 2 * (e % (KB / 2)), col = (e / (KB / 2)) * 8;                      \
      const uint16_t* vrow = vp + pf_sel4(o0, o1, o2, o3, row >> 4) + (row & 15) * HD + col; \
      vr[c][0] = *(gu32x4*)vrow;                                                         \
      vr[c][1] = *(gu32x4*)(vrow + HD);                                                  \
    }                                                                                    \
  }
// masks of a block reaching past pmax: chunks of positions j0 + row > pmax
#define CDB_PF_MASKS(j0)                                                                 \
  {                                                                                      \
    _Pragma("unroll") for (int c = 0; c < KCH; c++) {                                    \
      const int e = tid + 256 * c;                                                       \
      kmask[c] = (e < NKC && (j0) + e / (HD / 8) <= pmax) ? ~0u : 0u;                    \
    }                                                                                    \
    _Pragma("unroll") for (int c = 0; c < VCH; c++) {                                    \
      const int e = tid + 256 * c;                                                       \
      const int j = (j0) + 2 * (e % (KB / 2));                                           \
      vmask[c][0] = (e < NVC && j <= pmax) ? ~0u : 0u;                                   \
      vmask[c][1] = (e < NVC && j + 1 <= pmax) ? ~0u : 0u;                               \
    }                                                                                    \
  }
#define CDB_PF_STORE()                                                                   \
  {                                                                                      \
    _Pragma("unroll") for (int c = 0; c < KCH; c++) {                                    \
      const int e = tid + 256 * c;                                                       \
      if (e < NKC) *(u32x4*)&Ks[(e / (HD / 8)) * LDKS + (e % (HD / 8)) * 8] = kr[c] & kmask[c]; \
    }                                                                                    \
    _Pragma("unroll") for (int c = 0; c < VCH; c++) {                                    \
      const int e = tid + 256 * c;                                                       \
      if (e < NVC) {                                                                     \
        const int kpair = e % (KB / 2), col = (e / (KB / 2)) * 8;                        \
        const u32x4 a0 = vr[c][0] & vmask[c][0], a1 = vr[c][1] & vmask[c][1];           \
        _Pragma("unroll") for (int q = 0; q < 4; q++) {  /* byte permutes: low / high halves */ \
          *(uint32_t*)&Vt[(col + 2 * q) * LDV + 2 * kpair] = __builtin_amdgcn_perm(a1[q], a0[q], 0x05040100u); \
          *(uint32_t*)&Vt[(col + 2 * q + 1) * LDV + 2 * kpair] = __builtin_amdgcn_perm(a1[q], a0[q], 0x07060302u); \
        }                                                                                \
      }                                                                                  \
    }                                                                                    \
  }


// MFMA variant for bf16 (flash-attention style).  One workgroup per (tile of
// up to 64 QG consecutive query tokens of one sequence, head); wave w owns
// queries 64g + 16w .. 64g + 16w + 15 for g < QG (QG = 1: the 128-row tiles
// take the 32x32x16 kernel below).  Per key block of 64:
//  - S^T = K Q^T with v_mfma_f32_16x16x32_bf16 (A = K rows from LDS, B = the
//    wave's rotated, scaled queries held in registers), so each lane ends up
//    with 16 scores of ONE query (keys 16t + 4(l/16) + r);
//  - online softmax in base 2 (log2 e folded into the query scale): row
//    max / sum over the lane's 16 values and the 4 lanes sharing the query;
//  - O^T += V^T P^T with the same MFMA: the probabilities, rounded to bf16,
//    are already laid out as its B operand (the 32 keys of a step are taken
//    in a fixed permutation that A and B share), V is staged transposed in
//    LDS so its A operand is two 8-byte reads.
// Keys past the tile's last position are staged as zeros (their pages may
// hold anything); the next block's K/V are loaded into registers while the
// current one is computed.  The register budget is held to two waves per
// SIMD: the softmax and staging VALU work of one wave then overlaps the
// MFMAs of the other.  The VALU work per block is kept small: the causal
// mask is applied only in blocks that reach past the tile's first position,
// probabilities are rounded to bf16 by the hardware conversion, and V is
// transposed with byte permutes, no row is ever all-masked (so no selects
// guard the exponentials), and the accumulators are rescaled only when some
// row's max moved.  With QG = 2 (two groups of 16 queries per wave, 128-row
// tiles) every K and V fragment read from LDS fed both groups, halving the
// staging, fragment reads and barriers per query.  Measured on 16 heads of
// an 8192-token causal chunk: 1.01 ms without the register cap, 0.89 with
// it, 0.62 with the first VALU savings as well (heaviest tiles first), 0.55
// in a later build, 0.50 with QG = 2, 0.48 with the select-free softmax;
// same results bit for bit throughout.
template <int HD>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2))) void k_attn_prefill_mfma(PrefillAttnArgs a) {
  constexpr int QG = 1;                          // groups of 16 queries per wave
  constexpr int QT = 64 * QG, KB = 64;
  // row pitches in bf16 elements; K rows of head_dim 128 are padded by 16
  // (288 B), measured 8-13% faster than a 272-B pitch (304, 320 and 352 B
  // were slower than both): the K fragment reads meet fewer LDS bank
  // conflicts
  constexpr int LDQ = HD + 8, LDKS = HD + (HD == 128 ? 16 : 8), LDV = KB + 4;
  constexpr int HALF = HD / 2;
  constexpr int DS = HD / 32;                    // 32-wide steps over head dims
  constexpr int DT = HD / 16;                    // 16-wide output dim tiles
  constexpr int NKC = KB * (HD / 8);             // K chunks (16 B) per block
  constexpr int KCH = (NKC + 255) / 256;
  constexpr int NVC = (KB / 2) * (HD / 8);       // V (key pair, 8 dims) items per block
  constexpr int VCH = (NVC + 255) / 256;
  static_assert(HD % 32 == 0, "head_dim");
  __shared__ __align__(16) uint16_t Qs[QT * LDQ];
  __shared__ __align__(16) uint16_t Ks[KB * LDKS];
  __shared__ __align__(16) uint16_t Vt[HD * LDV];

  const int tile = blockIdx.x / a.nh, h = blockIdx.x % a.nh;
  const int2 td = a.tiles[tile];
  const int r0 = td.x, nq = td.y;
  const int seq = min(max(a.seq[r0], 0), a.max_seqs - 1);
  const int* bt = a.btab + (long)seq * a.bt_stride;
  const int pmax = min(a.pos[r0 + nq - 1], a.max_pos - 1);
  const int pmin = min(max(a.pos[r0], 0), a.max_pos - 1);   // the tile's first (smallest) position
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int r16 = lane & 15, g4 = lane >> 4;
  const float qscale = a.scale * 1.4426950408889634f;   // scores in log2 units

  // rotated, scaled queries of the tile -> LDS (bf16)
  for (int e = tid; e < QT * HALF; e += 256) {
    const int qi = e / HALF, i = e % HALF;
    float o0 = 0.f, o1 = 0.f;
    if (qi < nq) {
      const int r = r0 + qi;
      const float2 cs = a.rope[(long)min(max(a.pos[r], 0), a.max_pos - 1) * HALF + i];
      const float c = cs.x, sn = cs.y;
      const float x = qkv_at(a.qkv, a.qkv_sk, a.rows, a.ldq, r, h * HD + i);
      const float y = qkv_at(a.qkv, a.qkv_sk, a.rows, a.ldq, r, h * HD + i + HALF);
      o0 = (x * c - y * sn) * qscale;
      o1 = (y * c + x * sn) * qscale;
    }
    Qs[qi * LDQ + i] = f32_to_bf16(o0);
    Qs[qi * LDQ + i + HALF] = f32_to_bf16(o1);
  }

  typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
  typedef __attribute__((address_space(1))) const u32x4 gu32x4;
  const uint16_t* kp = (const uint16_t*)a.kpool;
  const uint16_t* vp = (const uint16_t*)a.vpool;
  // K / V of one key block in registers (CDB_PF_LOAD / MASKS / STORE)
  u32x4 kr[KCH], vr[VCH][2];
  uint32_t kmask[KCH], vmask[VCH][2];
  const int last_page = pmax >> 4;
  auto page_off = [&](int pg) -> long {
    const int blk = min(max(bt[min(pg, last_page)], 0), a.num_blocks - 1);
    return (((long)blk * a.nh + h) * a.planes + a.plane) * 16 * HD;
  };
  // this lane's query of group g within the tile: 64 g + 16 w + r16
  int myq[QG], pq[QG];
  float m_run[QG], l_run[QG];
  f32x4_t oacc[QG][DT];
#pragma unroll
  for (int g = 0; g < QG; g++) {
    myq[g] = 64 * g + 16 * w + r16;
    // rows past the tile (zero queries, never stored) mask like the tile's
    // last row, so every row sees key 0 in the first block and no row's
    // running max is ever -inf
    pq[g] = (myq[g] < nq) ? a.pos[r0 + myq[g]] : pmax;
    m_run[g] = -INFINITY;
    l_run[g] = 0.f;
#pragma unroll
    for (int d = 0; d < DT; d++) oacc[g][d] = (f32x4_t){0.f, 0.f, 0.f, 0.f};
  }

  CDB_PF_LOAD(0);
  __syncthreads();                                 // Qs complete
  bf16x8_t qf[QG][DS];
#pragma unroll
  for (int g = 0; g < QG; g++)
#pragma unroll
    for (int s = 0; s < DS; s++) qf[g][s] = *(const bf16x8_t*)&Qs[myq[g] * LDQ + 32 * s + 8 * g4];

  for (int j0 = 0; j0 <= pmax; j0 += KB) {
    __syncthreads();                               // previous block's readers are done
    if (j0 + KB - 1 <= pmax) {                     // every key valid: no masking work
#pragma unroll
      for (int c = 0; c < KCH; c++) kmask[c] = ~0u;
#pragma unroll
      for (int c = 0; c < VCH; c++) { vmask[c][0] = ~0u; vmask[c][1] = ~0u; }
      CDB_PF_STORE();
    } else {
      CDB_PF_MASKS(j0);
      CDB_PF_STORE();
    }
    __syncthreads();
    if (j0 + KB <= pmax) CDB_PF_LOAD(j0 + KB);
    // S^T tiles: keys 16t + 4*g4 + r, query r16 of each group (one K
    // fragment read feeds the QG groups' MFMAs)
    f32x4_t st[QG][4];
#pragma unroll
    for (int t = 0; t < 4; t++) {
#pragma unroll
      for (int g = 0; g < QG; g++) st[g][t] = (f32x4_t){0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int s = 0; s < DS; s++) {
        const bf16x8_t kf = *(const bf16x8_t*)&Ks[(16 * t + r16) * LDKS + 32 * s + 8 * g4];
#pragma unroll
        for (int g = 0; g < QG; g++) st[g][t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kf, qf[g][s], st[g][t], 0, 0, 0);
      }
    }
    bf16x8_t pbf[QG][2];
#pragma unroll
    for (int g = 0; g < QG; g++) {
      // causal mask, needed only by a block reaching past the tile's first
      // position (every earlier block is visible to all of the tile's
      // queries; rows past the tile hold zero queries and are never stored)
      if (j0 + KB - 1 > pmin) {
#pragma unroll
        for (int t = 0; t < 4; t++)
#pragma unroll
          for (int r = 0; r < 4; r++) {
            const int j = j0 + 16 * t + 4 * g4 + r;
            if (j > pq[g]) st[g][t][r] = -INFINITY;
          }
      }
      float mx = -INFINITY;
#pragma unroll
      for (int t = 0; t < 4; t++)
#pragma unroll
        for (int r = 0; r < 4; r++) mx = fmaxf(mx, st[g][t][r]);
      mx = fmaxf(mx, __shfl_xor(mx, 16, 64));
      mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
      // m_new is finite (key 0 is visible to every row in the first block),
      // so no select guards the exponentials; in the first block
      // m_run = -inf gives corr = 0, which scales the zero accumulators
      const float m_new = fmaxf(m_run[g], mx);
      const float corr = __builtin_amdgcn_exp2f(m_run[g] - m_new);
      float sum = 0.f;
      uint32_t pk[4][2];                            // bf16 pairs of each tile's 4 probabilities
#pragma unroll
      for (int t = 0; t < 4; t++) {
        float p[4];
#pragma unroll
        for (int r = 0; r < 4; r++) {
          p[r] = __builtin_amdgcn_exp2f(st[g][t][r] - m_new);
          sum += p[r];
        }
        pk[t][0] = cvt_bf16x2(p[0], p[1]);
        pk[t][1] = cvt_bf16x2(p[2], p[3]);
      }
      sum += __shfl_xor(sum, 16, 64);
      sum += __shfl_xor(sum, 32, 64);
      l_run[g] = l_run[g] * corr + sum;
      m_run[g] = m_new;
      // the accumulator rescale only when some row's max moved (corr = 1
      // leaves the values unchanged; once the running maxima settle most
      // blocks skip it)
      if (__ballot(corr != 1.f)) {
#pragma unroll
        for (int d = 0; d < DT; d++) oacc[g][d] *= corr;
      }
#pragma unroll
      for (int hh = 0; hh < 2; hh++) {
        const u32x4 pb = {pk[2 * hh][0], pk[2 * hh][1], pk[2 * hh + 1][0], pk[2 * hh + 1][1]};
        pbf[g][hh] = __builtin_bit_cast(bf16x8_t, pb);
      }
    }
    // O^T += V^T P^T over two 32-key steps (keys 32h + 4*g4 + {0..3} and
    // 32h + 16 + 4*g4 + {0..3}); one V fragment read feeds the QG groups
#pragma unroll
    for (int hh = 0; hh < 2; hh++) {
#pragma unroll
      for (int d = 0; d < DT; d++) {
        const uint16_t* vrow = &Vt[(16 * d + r16) * LDV + 32 * hh + 4 * g4];
        const uint2 v0 = *(const uint2*)vrow;
        const uint2 v1 = *(const uint2*)(vrow + 16);
        const u32x4 va = {v0.x, v0.y, v1.x, v1.y};
#pragma unroll
        for (int g = 0; g < QG; g++)
          oacc[g][d] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, va), pbf[g][hh], oacc[g][d], 0, 0, 0);
      }
    }
  }
#pragma unroll
  for (int g = 0; g < QG; g++) {
    if (myq[g] < nq) {
      const float inv = 1.f / l_run[g];
      uint16_t* out = (uint16_t*)a.out + (long)(r0 + myq[g]) * a.ldo + h * HD;
#pragma unroll
      for (int d = 0; d < DT; d++) {
        const uint32_t lo = (uint32_t)f32_to_bf16(oacc[g][d][0] * inv) | ((uint32_t)f32_to_bf16(oacc[g][d][1] * inv) << 16);
        const uint32_t hi = (uint32_t)f32_to_bf16(oacc[g][d][2] * inv) | ((uint32_t)f32_to_bf16(oacc[g][d][3] * inv) << 16);
        *(uint2*)(out + 16 * d + 4 * g4) = make_uint2(lo, hi);
      }
    }
  }
}

// 32x32x16 form of the 128-row tiles (head dims 96 and 128): wave w owns
// queries 32w .. 32w + 31 of the tile, and every product is one
// v_mfma_f32_32x32x16_bf16, which issues at about twice the rate of the
// 16x16x32 one on this chip.  Per key block of 64:
//  - S^T = K Q^T as two 32-key tiles (A = 32 K rows from LDS, B = the lane's
//    query, 16 head dims per step): lane l holds 32 scores of query l % 32,
//    keys 32t + 8(e / 4) + 4(l / 32) + e % 4;
//  - the softmax as in the 16x16x32 kernel (base 2, no all-masked row, the
//    rescale only when a row's max moved); a query's row spans lanes l and
//    l ^ 32;
//  - O^T += V^T P^T in four 16-key steps: virtual key 8(l / 32) + i of step
//    s is key 32(s / 2) + 8(s % 2) + 4(l / 32) + i for i < 4 and that + 12
//    otherwise, in both operands (the V^T operand is two 8-byte reads), so
//    two consecutive steps take the keys of a 32-key step of the 16x16x32
//    kernel in its order;
//  - the row sums in that kernel's order as well.
// The same staging and masks as the 16x16x32 kernel (K rows padded by 8
// elements at both head dims), and with the same key order in every sum the
// outputs are bit for bit that kernel's (GPU test on the model's prefill at
// 64- and 128-row tiles).  Against the 128-row tiles of that kernel (two
// groups of 16 queries per wave), first version: 16 heads of 128, one
// 8192-token prompt 0.472 -> 0.473-0.481 ms, two of 4096 0.296-0.299 ->
// 0.288-0.291 ms, four of 4096 0.593 -> 0.583-0.586 ms; 55 heads of 96, two
// of 4096 0.893-0.900 -> 0.733-0.747 ms.
template <int HD>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2))) void k_attn_prefill_m32(PrefillAttnArgs a) {
  constexpr int QT = 128, KB = 64;
  // K rows padded by 8 elements for both head dims (for 128: 0.458-0.464 ms
  // on an 8192-token chunk against 0.468 with 16, as the 16x16x32 kernel
  // pads; 24 the same as 8, 32 slower)
  constexpr int LDQ = HD + 8, LDKS = HD + 8, LDV = KB + 4;
  constexpr int HALF = HD / 2;
  constexpr int DS = HD / 16;                    // 16-wide steps over head dims
  constexpr int DT = HD / 32;                    // 32-wide output dim tiles
  constexpr int NKC = KB * (HD / 8);
  constexpr int KCH = (NKC + 255) / 256;
  constexpr int NVC = (KB / 2) * (HD / 8);
  constexpr int VCH = (NVC + 255) / 256;
  static_assert(HD % 32 == 0, "head_dim");
  typedef float f32x16_t __attribute__((ext_vector_type(16)));
  __shared__ __align__(16) uint16_t Qs[QT * LDQ];
  __shared__ __align__(16) uint16_t Ks[KB * LDKS];
  __shared__ __align__(16) uint16_t Vt[HD * LDV];

  const int tile = blockIdx.x / a.nh, h = blockIdx.x % a.nh;
  const int2 td = a.tiles[tile];
  const int r0 = td.x, nq = td.y;
  const int seq = min(max(a.seq[r0], 0), a.max_seqs - 1);
  const int* bt = a.btab + (long)seq * a.bt_stride;
  const int pmax = min(a.pos[r0 + nq - 1], a.max_pos - 1);
  const int pmin = min(max(a.pos[r0], 0), a.max_pos - 1);
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int l32 = lane & 31, h2 = lane >> 5;
  const float qscale = a.scale * 1.4426950408889634f;   // scores in log2 units

  // rotated, scaled queries of the tile -> LDS (bf16)
  for (int e = tid; e < QT * HALF; e += 256) {
    const int qi = e / HALF, i = e % HALF;
    float o0 = 0.f, o1 = 0.f;
    if (qi < nq) {
      const int r = r0 + qi;
      const float2 cs = a.rope[(long)min(max(a.pos[r], 0), a.max_pos - 1) * HALF + i];
      const float c = cs.x, sn = cs.y;
      const float x = qkv_at(a.qkv, a.qkv_sk, a.rows, a.ldq, r, h * HD + i);
      const float y = qkv_at(a.qkv, a.qkv_sk, a.rows, a.ldq, r, h * HD + i + HALF);
      o0 = (x * c - y * sn) * qscale;
      o1 = (y * c + x * sn) * qscale;
    }
    Qs[qi * LDQ + i] = f32_to_bf16(o0);
    Qs[qi * LDQ + i + HALF] = f32_to_bf16(o1);
  }

  typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
  typedef __attribute__((address_space(1))) const u32x4 gu32x4;
  const uint16_t* kp = (const uint16_t*)a.kpool;
  const uint16_t* vp = (const uint16_t*)a.vpool;
  u32x4 kr[KCH], vr[VCH][2];
  uint32_t kmask[KCH], vmask[VCH][2];
  const int last_page = pmax >> 4;
  auto page_off = [&](int pg) -> long {
    const int blk = min(max(bt[min(pg, last_page)], 0), a.num_blocks - 1);
    return (((long)blk * a.nh + h) * a.planes + a.plane) * 16 * HD;
  };
  // this lane's query; rows past the tile mask like its last row
  const int myq = 32 * w + l32;
  const int pq = (myq < nq) ? a.pos[r0 + myq] : pmax;
  float m_run = -INFINITY, l_run = 0.f;
  f32x16_t oacc[DT];
#pragma unroll
  for (int d = 0; d < DT; d++)
#pragma unroll
    for (int e = 0; e < 16; e++) oacc[d][e] = 0.f;

  CDB_PF_LOAD(0);
  __syncthreads();                                 // Qs complete
  bf16x8_t qf[DS];
#pragma unroll
  for (int s = 0; s < DS; s++) qf[s] = *(const bf16x8_t*)&Qs[myq * LDQ + 16 * s + 8 * h2];

  for (int j0 = 0; j0 <= pmax; j0 += KB) {
    __syncthreads();                               // previous block's readers are done
    if (j0 + KB - 1 <= pmax) {
#pragma unroll
      for (int c = 0; c < KCH; c++) kmask[c] = ~0u;
#pragma unroll
      for (int c = 0; c < VCH; c++) { vmask[c][0] = ~0u; vmask[c][1] = ~0u; }
      CDB_PF_STORE();
    } else {
      CDB_PF_MASKS(j0);
      CDB_PF_STORE();
    }
    __syncthreads();
    if (j0 + KB <= pmax) CDB_PF_LOAD(j0 + KB);
    f32x16_t st[2];
#pragma unroll
    for (int t = 0; t < 2; t++) {
#pragma unroll
      for (int e = 0; e < 16; e++) st[t][e] = 0.f;
#pragma unroll
      for (int s = 0; s < DS; s++) {
        const bf16x8_t kf = *(const bf16x8_t*)&Ks[(32 * t + l32) * LDKS + 16 * s + 8 * h2];
        st[t] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf, qf[s], st[t], 0, 0, 0);
      }
    }
    if (j0 + KB - 1 > pmin) {                      // the causal mask, only where it can bite
#pragma unroll
      for (int t = 0; t < 2; t++)
#pragma unroll
        for (int e = 0; e < 16; e++) {
          const int j = j0 + 32 * t + 8 * (e >> 2) + 4 * h2 + (e & 3);
          if (j > pq) st[t][e] = -INFINITY;
        }
    }
    float mx = -INFINITY;
#pragma unroll
    for (int t = 0; t < 2; t++)
#pragma unroll
      for (int e = 0; e < 16; e++) mx = fmaxf(mx, st[t][e]);
    mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
    const float m_new = fmaxf(m_run, mx);
    const float corr = __builtin_amdgcn_exp2f(m_run - m_new);
    // the row sum in the 16x16x32 kernel's order: lane h2 forms the sums of
    // that kernel's key groups h2 (keys 16u + 4h2 + r) and 2 + h2 (16u + 8 +
    // 4h2 + r), each over u then r, and the lanes combine them as its
    // shuffles do
    float pr[2][16];
#pragma unroll
    for (int t = 0; t < 2; t++)
#pragma unroll
      for (int e = 0; e < 16; e++) pr[t][e] = __builtin_amdgcn_exp2f(st[t][e] - m_new);
    float s_lo = 0.f, s_hi = 0.f;
#pragma unroll
    for (int u = 0; u < 4; u++)
#pragma unroll
      for (int r = 0; r < 4; r++) {
        s_lo += pr[u >> 1][8 * (u & 1) + r];
        s_hi += pr[u >> 1][8 * (u & 1) + 4 + r];
      }
    s_lo += __shfl_xor(s_lo, 32, 64);
    s_hi += __shfl_xor(s_hi, 32, 64);
    const float sum = s_lo + s_hi;
    // B operand of PV step s (16 keys): tile s / 2, virtual key 8h2 + i =
    // key 8(s % 2) + 4h2 + i (i < 4) or 16 + 8(s % 2) + 4h2 + i - 4 of the
    // tile, the key order of the 16x16x32 kernel's 32-key steps
    bf16x8_t pf[4];
#pragma unroll
    for (int s = 0; s < 4; s++) {
      const float* q0 = &pr[s >> 1][4 * (s & 1)];
      const float* q1 = &pr[s >> 1][8 + 4 * (s & 1)];
      const u32x4 pb = {cvt_bf16x2(q0[0], q0[1]), cvt_bf16x2(q0[2], q0[3]), cvt_bf16x2(q1[0], q1[1]),
                        cvt_bf16x2(q1[2], q1[3])};
      pf[s] = __builtin_bit_cast(bf16x8_t, pb);
    }
    l_run = l_run * corr + sum;
    m_run = m_new;
    if (__ballot(corr != 1.f)) {
#pragma unroll
      for (int d = 0; d < DT; d++) oacc[d] *= corr;
    }
#pragma unroll
    for (int s = 0; s < 4; s++) {
#pragma unroll
      for (int d = 0; d < DT; d++) {
        const uint16_t* vrow = &Vt[(32 * d + l32) * LDV + 32 * (s >> 1) + 8 * (s & 1) + 4 * h2];
        const uint2 v0 = *(const uint2*)vrow;
        const uint2 v1 = *(const uint2*)(vrow + 16);
        const u32x4 va = {v0.x, v0.y, v1.x, v1.y};
        oacc[d] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, va), pf[s], oacc[d], 0, 0, 0);
      }
    }
  }
  // lane holds query myq, head dims 32d + 8(e / 4) + 4h2 + e % 4
  if (myq < nq) {
    const float inv = 1.f / l_run;
    uint16_t* out = (uint16_t*)a.out + (long)(r0 + myq) * a.ldo + h * HD;
#pragma unroll
    for (int d = 0; d < DT; d++)
#pragma unroll
      for (int g = 0; g < 4; g++) {
        const uint32_t lo = (uint32_t)f32_to_bf16(oacc[d][4 * g] * inv) | ((uint32_t)f32_to_bf16(oacc[d][4 * g + 1] * inv) << 16);
        const uint32_t hi = (uint32_t)f32_to_bf16(oacc[d][4 * g + 2] * inv) | ((uint32_t)f32_to_bf16(oacc[d][4 * g + 3] * inv) << 16);
        *(uint2*)(out + 32 * d + 8 * g + 4 * h2) = make_uint2(lo, hi);
      }
  }
}
#undef CDB_PF_LOAD
#undef CDB_PF_MASKS
#undef CDB_PF_STORE

template <int HD>
static int pfm_one(const PrefillAttnArgs& a, hipStream_t st) {
  if constexpr (HD != 64) {
    if (a.tile_rows == 128) {
      hipLaunchKernelGGL((k_attn_prefill_m32<HD>), dim3(a.n_tiles * a.nh), dim3(256), 0, st, a);
      return hipGetLastError() == hipSuccess ? 0 : -1;
    }
  }
  if (a.tile_rows != 64) return -2;
  hipLaunchKernelGGL((k_attn_prefill_mfma<HD>), dim3(a.n_tiles * a.nh), dim3(256), 0, st, a);
  return hipGetLastError() == hipSuccess ? 0 : -1;
}

// Query rows per prefill tile.  The bf16 MFMA kernel has 64-row tiles (one
// group of 16 queries per wave); for head dims 96 and 128 the 32x32x16
// kernel takes 128-row tiles (32 queries per wave), with the same bits.
// Larger tiles pay where each tile's key range is long; otherwise they
// lose, with half the workgroups (and a tile's first queries also walk the
// last, masked, block of its later ones).  Measured, 64-row tiles against
// the 32x32x16 kernel: 16 heads of 128, four prompts of 4096 0.633-0.650 ->
// 0.583-0.586 ms, eight of 2048 0.421 -> 0.419-0.422, four of 2048 0.210 ->
// 0.216, eight of 1024 0.155 -> 0.171; 55 heads of 96, sixteen of 1024
// 0.846-0.856 -> 0.790-0.799 ms, eight of 1024 0.392-0.397 -> 0.387-0.388,
// sixteen of 512 0.309-0.312 -> 0.336, thirty-two of 256 0.268-0.272 ->
// 0.313; earlier, a 1,234-token chunk continuing a prompt at position 8192
// (160 workgroups of 128 rows) lost 5 ms over a 9,426-token prompt's 96
// layer passes.  So 128-row tiles go, at head dim 128, to chunks whose
// 64-row tiles reach 3072 keys on average with at least 768 workgroups, or
// 2048 keys with at least 1024, and at head dim 96 (cheaper per score, so
// the 32x32x16 MFMAs gain more) to chunks of at least 512 keys on average
// and 1024 workgroups.
int attn_prefill_tile_rows(int dtype, int hd, double mean_keys, long wg128, int force) {
  if (dtype != 1 || !(hd == 64 || hd == 96 || hd == 128)) return 32;
  if (hd == 64) return 64;
  if (force == 64 || force == 128) return force;
  if (hd == 96) return (mean_keys >= 512.0 && wg128 >= 1024) ? 128 : 64;
  return ((mean_keys >= 3072.0 && wg128 >= 768) || (mean_keys >= 2048.0 && wg128 >= 1024)) ? 128 : 64;
}

template <typename T, int HD>
static int pf_one(const PrefillAttnArgs& a, hipStream_t st) {
  hipLaunchKernelGGL((k_attn_prefill<T, HD>), dim3(a.n_tiles * a.nh), dim3(256), 0, st, a);
  return hipGetLastError() == hipSuccess ? 0 : -1;
}

int rope_table_launch(float2* table, int rows, int head_dim, float theta, hipStream_t st) {
  const long n = (long)rows * (head_dim / 2);
  const int blocks = (int)std::min<long>((n + 255) / 256, 4096);
  hipLaunchKernelGGL(k_rope_table, dim3(std::max(blocks, 1)), dim3(256), 0, st, table, rows, head_dim, (double)theta);
  return hipGetLastError() == hipSuccess ? 0 : -1;
}

int attn_prefill_launch(int dtype, int hd, const PrefillAttnArgs& a, hipStream_t st) {
  if (a.n_tiles <= 0) return 0;
  if (dtype == 0) {
    if (hd == 64) return pf_one<float, 64>(a, st);
    if (hd == 32) return pf_one<float, 32>(a, st);
    if (hd == 16) return pf_one<float, 16>(a, st);
  } else {
    if (hd == 128) return pfm_one<128>(a, st);
    if (hd == 96) return pfm_one<96>(a, st);
    if (hd == 64) return pfm_one<64>(a, st);
    if (hd == 16) return pf_one<bf16_t, 16>(a, st);
  }
  return -2;
}

}  // namespace cdb
