// Ragged decode attention over the paged, depth-indexed KV cache.
//
// Row b (sequence seq[b], position p = pos[b], loop step d) attends to
// positions 0..p of its sequence.  Depth-indexed cache: earlier position j
// is read at plane min(d, e_j) — what a last-exited copy of the token's
// final KV into its skipped slots would hold ("Depth-adaptive Inference of
// Looped Language Models via Continuous Depth Batching", §4.2 and Fig. 2
// right); the row itself is read at plane d.  Single-slot cache: every
// position is read from the one plane (latest state).
//
// Work split: one workgroup per (row, head, split); the splits cut the
// row's context into n_split equal ranges (flash-decoding).  Each 16-lane
// group of a wave owns one position at a time: its lanes load 16 B of K and
// 16 B of V each (one 256-B K row and one V row per group for head_dim 128
// in bf16), reduce the q.k partial dot over the group, and keep an online
// softmax.  K/V are streamed straight into registers: with multi-head KV
// there is no reuse across rows or heads, so staging through LDS would only
// add traffic; LDS holds the rotated query and the cross-group merge.
// Partial (max, sum, o) of the splits are merged by the last workgroup of a
// (row, head) to arrive, in split order (deterministic).
//
// With write_kv the workgroup whose range holds p rotates this row's new k,
// stores k and v at plane d (or the single plane), and attends to them from
// registers (rounded to the cache type first, as a later reader sees them).
#include "common.h"
#include "kernels.h"

namespace cdb {

__device__ __forceinline__ void rope_angle(int pos, int i, int hd, float theta, float& c, float& s) {
  // angle = pos * theta^(-2i/hd), formed and evaluated in double, rounded once
  const double inv = pow((double)theta, -(2.0 * (double)i) / (double)hd);
  const double ang = (double)pos * inv;
  c = (float)cos(ang);
  s = (float)sin(ang);
}

template <typename T, int HD>
__global__ __launch_bounds__(256) void k_attn(AttnArgs a) {
  typedef typename Elt<T>::raw raw;
  constexpr int EPL = 16 / sizeof(raw);          // elements per lane (one 16-B load)
  constexpr int LP = HD / EPL;                    // active lanes per 16-lane group
  static_assert(LP <= 16 && HD % EPL == 0, "head_dim");
  constexpr int HALF = HD / 2;
  __shared__ float q_s[HD];
  __shared__ float kself[HD], vself[HD];
  __shared__ float gm[17], gl[17];
  __shared__ float go[17][HD];
  __shared__ int flag;

  const int bh = blockIdx.x;
  const int b = bh / a.nh, h = bh % a.nh;
  const int sp = blockIdx.y;
  const int n_valid = ld_nvalid(a.n_valid, a.rows);
  if (b >= n_valid) return;
  // indices read from device memory are clamped into their buffers
  const int p = min(max(a.pos[b], 0), a.max_pos - 1);
  const int seq = min(max(a.seq[b], 0), a.max_seqs - 1);
  const int d = min(max(a.depth ? a.depth[b] : a.depth_uniform, 1), a.planes > 1 ? a.planes : 0x7fffffff);
  const int ctx = p + 1;
  const int chunk = (ctx + a.n_split - 1) / a.n_split;
  const int j0 = sp * chunk;
  const int j1 = min(ctx, j0 + chunk);
  const bool has_self = a.write_kv && (p >= j0 && p < j1);
  const int jend = a.write_kv ? min(j1, p) : j1;  // positions read from the cache
  const int* bt = a.btab + (long)seq * a.bt_stride;
  const long plane_d = (a.planes > 1) ? (long)(d - 1) * a.plane_stride : 0;

  // rotated query (and, for the self split, rotated k and v)
  const float* qrow = a.qkv + (long)b * a.ldq + h * HD;
  const int Q = a.nh * HD;
  if (threadIdx.x < HD) {
    const int i = threadIdx.x;
    const int ii = i < HALF ? i : i - HALF;
    float c, s;
    rope_angle(p, ii, HD, a.theta, c, s);
    const float x = qrow[i], y = (i < HALF) ? qrow[i + HALF] : qrow[i - HALF];
    q_s[i] = (i < HALF) ? (x * c - y * s) : (x * c + y * s);
    if (has_self) {
      const float* krow = qrow + Q;
      const float* vrow = qrow + 2 * Q;
      const float kx = krow[i], ky = (i < HALF) ? krow[i + HALF] : krow[i - HALF];
      const float kr = (i < HALF) ? (kx * c - ky * s) : (kx * c + ky * s);
      const raw kq = Elt<T>::from_f32(kr), vq = Elt<T>::from_f32(vrow[i]);
      kself[i] = Elt<T>::to_f32(kq);
      vself[i] = Elt<T>::to_f32(vq);
      const int blk = min(max(bt[p >> 4], 0), a.num_blocks - 1), off = p & 15;
      const long idx = plane_d + (((long)blk * a.nh + h) * 16 + off) * HD + i;
      ((raw*)a.kpool)[idx] = kq;
      ((raw*)a.vpool)[idx] = vq;
    }
  }
  __syncthreads();

  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int c = lane & 15;                        // lane within the group
  const int grp = w * 4 + (lane >> 4);            // 0..15
  const bool act = c < LP;
  float qv[EPL];
#pragma unroll
  for (int e = 0; e < EPL; e++) qv[e] = act ? q_s[c * EPL + e] * a.scale : 0.f;

  float m_run = -INFINITY, l_run = 0.f;
  float o[EPL];
#pragma unroll
  for (int e = 0; e < EPL; e++) o[e] = 0.f;

  const raw* kp = (const raw*)a.kpool;
  const raw* vp = (const raw*)a.vpool;
  constexpr int U = 4;
  for (int jb = j0 + grp; jb < jend; jb += 16 * U) {
    uint4 kk[U], vv[U];
    bool ok[U];
#pragma unroll
    for (int u = 0; u < U; u++) {
      const int j = jb + 16 * u;
      ok[u] = j < jend;
      const int jj = ok[u] ? j : j0;
      const int blk = min(max(bt[jj >> 4], 0), a.num_blocks - 1), off = jj & 15;
      long plane = 0;
      if (a.planes > 1) {
        const int e = max((int)a.emap[(long)blk * 16 + off], 1);
        plane = (long)((e < d ? e : d) - 1) * a.plane_stride;
      }
      const long idx = plane + (((long)blk * a.nh + h) * 16 + off) * HD + c * EPL;
      if (act) {
        kk[u] = *(const uint4*)(kp + idx);
        vv[u] = *(const uint4*)(vp + idx);
      } else {
        kk[u] = make_uint4(0, 0, 0, 0);
        vv[u] = make_uint4(0, 0, 0, 0);
      }
    }
#pragma unroll
    for (int u = 0; u < U; u++) {
      float kf[EPL], vf[EPL];
      unpack16(kk[u], kf, T());
      unpack16(vv[u], vf, T());
      float sdot = 0.f;
#pragma unroll
      for (int e = 0; e < EPL; e++) sdot += qv[e] * kf[e];
#pragma unroll
      for (int off = 8; off > 0; off >>= 1) sdot += __shfl_xor(sdot, off, 16);
      if (ok[u]) {
        const float m_new = fmaxf(m_run, sdot);
        const float corr = __expf(m_run - m_new);
        const float pj = __expf(sdot - m_new);
        l_run = l_run * corr + pj;
#pragma unroll
        for (int e = 0; e < EPL; e++) o[e] = o[e] * corr + pj * vf[e];
        m_run = m_new;
      }
    }
  }

  // merge the 16 groups (+ the self position) in fixed order
  if (c == 0) { gm[grp] = m_run; gl[grp] = l_run; }
  if (act) {
#pragma unroll
    for (int e = 0; e < EPL; e++) go[grp][c * EPL + e] = o[e];
  }
  if (threadIdx.x == 0) {
    if (has_self) {
      float sdot = 0.f;
      for (int i = 0; i < HD; i++) sdot += q_s[i] * a.scale * kself[i];
      gm[16] = sdot;
      gl[16] = 1.f;
    } else {
      gm[16] = -INFINITY;
      gl[16] = 0.f;
    }
  }
  __syncthreads();
  float M = -INFINITY;
  for (int g = 0; g < 17; g++) M = fmaxf(M, gm[g]);
  float L = 0.f, O = 0.f;
  const int i = threadIdx.x;
  if (M != -INFINITY) {
    for (int g = 0; g < 16; g++) {
      const float f = __expf(gm[g] - M);
      L += gl[g] * f;
      if (i < HD) O += go[g][i] * f;
    }
    if (has_self) {
      const float f = __expf(gm[16] - M);
      L += f;
      if (i < HD) O += vself[i] * f;
    }
  }
  raw* out = (raw*)a.out + (long)b * a.ldo + h * HD;
  if (a.n_split == 1) {
    if (i < HD) out[i] = Elt<T>::from_f32(O / L);
    return;
  }
  // split partials; the last workgroup of this (row, head) merges them
  float* part = a.part + ((long)bh * a.n_split + sp) * (HD + 2);
  if (i < HD) part[2 + i] = O;
  if (i == 0) { part[0] = M; part[1] = L; }
  __threadfence();
  __syncthreads();
  if (threadIdx.x == 0) {
    const int old = atomicAdd(&a.counters[bh], 1);
    flag = (old == a.n_split - 1);
    if (old == a.n_split - 1) a.counters[bh] = 0;
  }
  __syncthreads();
  if (!flag) return;
  __threadfence();
  const float* pb = a.part + (long)bh * a.n_split * (HD + 2);
  float MM = -INFINITY;
  for (int s = 0; s < a.n_split; s++) MM = fmaxf(MM, __builtin_nontemporal_load(pb + (long)s * (HD + 2)));
  float LL = 0.f, OO = 0.f;
  for (int s = 0; s < a.n_split; s++) {
    const float ms = __builtin_nontemporal_load(pb + (long)s * (HD + 2));
    if (ms == -INFINITY) continue;
    const float f = __expf(ms - MM);
    LL += __builtin_nontemporal_load(pb + (long)s * (HD + 2) + 1) * f;
    if (i < HD) OO += __builtin_nontemporal_load(pb + (long)s * (HD + 2) + 2 + i) * f;
  }
  if (i < HD) out[i] = Elt<T>::from_f32(OO / LL);
}

template <typename T, int HD>
__global__ __launch_bounds__(256) void k_kv_write(KvWriteArgs a) {
  typedef typename Elt<T>::raw raw;
  constexpr int HALF = HD / 2;
  const int r = blockIdx.x;
  if (r >= a.rows) return;
  const int p = min(max(a.pos[r], 0), a.max_pos - 1);
  const int seq = min(max(a.seq[r], 0), a.max_seqs - 1);
  const int Q = a.nh * HD;
  const int blk = min(max(a.btab[(long)seq * a.bt_stride + (p >> 4)], 0), a.num_blocks - 1), off = p & 15;
  const float* krow = a.qkv + (long)r * a.ldq + Q;
  const float* vrow = krow + Q;
  for (int t = threadIdx.x; t < Q; t += blockDim.x) {
    const int h = t / HD, i = t % HD;
    const int ii = i < HALF ? i : i - HALF;
    float c, s;
    rope_angle(p, ii, HD, a.theta, c, s);
    const float x = krow[t], y = (i < HALF) ? krow[t + HALF] : krow[t - HALF];
    const float kr = (i < HALF) ? (x * c - y * s) : (x * c + y * s);
    const long idx = (long)a.plane * a.plane_stride + (((long)blk * a.nh + h) * 16 + off) * HD + i;
    ((raw*)a.kpool)[idx] = Elt<T>::from_f32(kr);
    ((raw*)a.vpool)[idx] = Elt<T>::from_f32(vrow[t]);
  }
}

template <typename T, int HD>
static int attn_one(const AttnArgs& a, hipStream_t st) {
  dim3 grid(a.rows * a.nh, a.n_split);
  hipLaunchKernelGGL((k_attn<T, HD>), grid, dim3(256), 0, st, a);
  return hipGetLastError() == hipSuccess ? 0 : -1;
}

int attn_launch(int dtype, int hd, const AttnArgs& a, hipStream_t st) {
  if (dtype == 0) {
    if (hd == 64) return attn_one<float, 64>(a, st);
    if (hd == 32) return attn_one<float, 32>(a, st);
    if (hd == 16) return attn_one<float, 16>(a, st);
  } else {
    if (hd == 128) return attn_one<bf16_t, 128>(a, st);
    if (hd == 96) return attn_one<bf16_t, 96>(a, st);
    if (hd == 64) return attn_one<bf16_t, 64>(a, st);
    if (hd == 16) return attn_one<bf16_t, 16>(a, st);
  }
  return -2;
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
