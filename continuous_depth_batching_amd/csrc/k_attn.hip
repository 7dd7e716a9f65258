// Ragged decode attention over the paged, depth-indexed KV cache.
//
// Row b (sequence seq[b], position p = pos[b], loop step d) attends to
// positions 0..p of its sequence.  Depth-indexed cache: earlier position j
// is read at plane min(d, e_j) — what a last-exited copy of the token's
// final KV into its skipped slots would hold ("Depth-adaptive Inference of
// Looped Language Models via Continuous Depth Batching", §4.2 and Fig. 2
// right); the row itself is read at plane d.  With that copy made
// explicitly at exit (no depth map passed) every earlier position is read at
// plane d.  Single-slot cache: every position is read from the one plane
// (latest state).
//
// Work split: one workgroup per (row, head, split); the splits cut the
// row's context into n_split equal ranges (flash-decoding).  A workgroup has
// 16 or 32 16-lane groups (256 or 512 threads); each group owns one position
// at a time: its lanes load 16 B of K and 16 B of V each (one 256-B K row and
// one V row per group for head_dim 128 in bf16), reduce the q.k partial dot
// over the group, and keep an online softmax.  K/V are streamed straight into registers: with multi-head KV
// there is no reuse across rows or heads, so staging through LDS would only
// add traffic; LDS holds the rotated query and the cross-group merge.  The
// K/V loads are non-temporal: the stream is read once per step and is far
// larger than L2 and the Infinity Cache, and keeping it out of them raises
// the read rate by about 13% (5.2 -> 5.9 TB/s at 64 rows x 1024 positions).
// With several splits each workgroup writes its partial (max, sum, o) and
// k_attn_merge combines them in split order (deterministic, no workgroup
// waits on another).
//
// With write_kv the workgroup whose range holds p rotates this row's new k,
// stores k and v at plane d (or the single plane), and attends to them from
// registers (rounded to the cache type first, as a later reader sees them).
#include "common.h"
#include "kernels.h"
#include "attn_common.h"

namespace cdb {

template <typename T, int HD, int NT>
__global__ __launch_bounds__(NT) void k_attn(AttnArgs a) {
  typedef typename Elt<T>::raw raw;
  constexpr int EPL = 16 / sizeof(raw);          // elements per lane (one 16-B load)
  constexpr int LP = HD / EPL;                    // active lanes per 16-lane group
  constexpr int NG = NT / 16;                     // 16-lane groups (position streams)
  static_assert(LP <= 16 && HD % EPL == 0, "head_dim");
  constexpr int HALF = HD / 2;
  __shared__ float q_s[HD];
  __shared__ float kself[HD], vself[HD];
  __shared__ float gm[NG + 1], gl[NG + 1];
  __shared__ float go[NG + 1][HD];

  const int bh = blockIdx.x;
  const int b = bh / a.nh, h = bh % a.nh;
  const int sp = blockIdx.y;
  // The row's indices are read together with the valid count (b < rows and
  // every row array holds at least rows entries), one memory round trip.
  const int pos_b = a.pos[b], seq_b = a.seq[b];
  const int dep_b = a.depth ? a.depth[b] : a.depth_uniform;
  const int n_valid = ld_nvalid(a.n_valid, a.rows);
  if (bh == 0 && sp == 0 && threadIdx.x == 0 && n_valid > a.rows) flag_err(a.err, ERR_COUNT);
  if (b >= n_valid) return;
  // indices read from device memory are clamped into their buffers (and a
  // clamp is reported through the error word)
  const int p = clamp_chk(pos_b, 0, a.max_pos - 1, a.err, ERR_POS);
  const int seq = clamp_chk(seq_b, 0, a.max_seqs - 1, a.err, ERR_SEQ);
  const int d = min(clamp_chk(dep_b, 1, a.r_max, a.err, ERR_DEPTH), a.planes > 1 ? a.planes : 0x7fffffff);
  const int ctx = p + 1;
  const int chunk = (ctx + a.n_split - 1) / a.n_split;
  const int j0 = sp * chunk;
  const int j1 = min(ctx, j0 + chunk);
  const bool has_self = a.write_kv && (p >= j0 && p < j1);
  const int jend = a.write_kv ? min(j1, p) : j1;  // positions read from the cache
  const int* bt = a.btab + (long)seq * a.bt_stride;
  const int plane_d = (a.planes > 1) ? d - 1 : 0;

  // rotated query (and, for the self split, rotated k and v).  Rows whose
  // QKV input is still unscaled (deferred RMSNorm) get the row's 1 / rms
  // here; the waves holding query lanes form it after issuing their
  // projection loads, so one wait covers both.
  const int Q = a.nh * HD;
  if ((int)(threadIdx.x & ~63) < HD) {
    const int i = min((int)threadIdx.x, HD - 1);
    const int ii = i < HALF ? i : i - HALF;
    const int ip = i < HALF ? i + HALF : i - HALF;
    const float2 cs = a.rope[(long)p * HALF + ii];
    const float c = cs.x, s = cs.y;
    const int qc = h * HD;
    const float x0 = qkv_at(a.qkv, a.qkv_sk, a.rows, a.ldq, b, qc + i);
    const float y0 = qkv_at(a.qkv, a.qkv_sk, a.rows, a.ldq, b, qc + ip);
    float kx0 = 0.f, ky0 = 0.f, vx0 = 0.f;
    if (has_self) {
      kx0 = qkv_at(a.qkv, a.qkv_sk, a.rows, a.ldq, b, Q + qc + i);
      ky0 = qkv_at(a.qkv, a.qkv_sk, a.rows, a.ldq, b, Q + qc + ip);
      vx0 = qkv_at(a.qkv, a.qkv_sk, a.rows, a.ldq, b, 2 * Q + qc + i);
    }
    const float rsc = a.ss ? rstd_from_parts_wave(a.ss, a.ss_n, b, a.ss_h, a.eps) : 1.0f;
    if (threadIdx.x < HD) {
      const float x = rsc * x0, y = rsc * y0;
      q_s[i] = (i < HALF) ? (x * c - y * s) : (x * c + y * s);
      if (has_self) {
        const float kx = rsc * kx0, ky = rsc * ky0, vx = rsc * vx0;
        const float kr = (i < HALF) ? (kx * c - ky * s) : (kx * c + ky * s);
        const raw kq = Elt<T>::from_f32(kr), vq = Elt<T>::from_f32(vx);
        kself[i] = Elt<T>::to_f32(kq);
        vself[i] = Elt<T>::to_f32(vq);
        const int blk = clamp_chk(bt[p >> 4], 0, a.num_blocks - 1, a.err, ERR_BLOCK), off = p & 15;
        const long idx = ((((long)blk * a.nh + h) * a.planes + plane_d) * 16 + off) * HD + i;
        ((raw*)a.kpool)[idx] = kq;
        ((raw*)a.vpool)[idx] = vq;
      }
    }
  }

  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int c = lane & 15;                        // lane within the group
  const int grp = w * 4 + (lane >> 4);            // 0..NG-1
  const bool act = c < LP;

  float m_run = -INFINITY, l_run = 0.f;
  float o[EPL];
#pragma unroll
  for (int e = 0; e < EPL; e++) o[e] = 0.f;

  const raw* kp = (const raw*)a.kpool;
  const raw* vp = (const raw*)a.vpool;
  constexpr int U = 4;
  // The block ids and read planes of a segment of positions are staged in
  // LDS first, so every K/V address comes from LDS instead of two dependent
  // global loads (block table, then depth map).
  // The first segment is staged before the barrier that also publishes the
  // rotated query, so its loads overlap the query's.
  constexpr int SEG = 4096;
  __shared__ int blk_s[SEG / 16 + 1];
  __shared__ uint8_t pl_s[SEG];
  auto stage = [&](int seg0) {
    const int seg1 = min(jend, seg0 + SEG);
    const int b0 = seg0 >> 4;
    for (int j = seg0 + threadIdx.x; j < seg1; j += NT) {
      const int blk = clamp_chk(bt[j >> 4], 0, a.num_blocks - 1, a.err, ERR_BLOCK);
      int pl = 0;
      if (a.planes > 1 && a.emap) {
        const int e = max((int)a.emap[(long)blk * 16 + (j & 15)], 1);
        pl = (e < d ? e : d) - 1;
      } else if (a.planes > 1) {
        pl = d - 1;                               // explicit copies: the reader's own plane
      }
      pl_s[j - seg0] = (uint8_t)pl;
      if ((j & 15) == 0 || j == seg0) blk_s[(j >> 4) - b0] = blk;
    }
  };
  stage(j0);
  __syncthreads();
  float qv[EPL];
#pragma unroll
  for (int e = 0; e < EPL; e++) qv[e] = act ? q_s[c * EPL + e] * a.scale : 0.f;
  for (int seg0 = j0; seg0 < jend; seg0 += SEG) {
    const int seg1 = min(jend, seg0 + SEG);
    const int b0 = seg0 >> 4;
    if (seg0 != j0) {
      __syncthreads();                            // the previous segment's readers are done
      stage(seg0);
      __syncthreads();
    }
    // Software-pipelined over batches of U positions: the K/V loads of the
    // next batch are in flight while the current batch is scored (ping-pong
    // registers).  Positions past the segment load a valid row of it and are
    // masked out of the softmax.
    uint4 kk[2][U], vv[2][U];
    bool ok[2][U];
#define CDB_ATTN_LOAD(buf, jbase)                                                        \
    _Pragma("unroll") for (int u = 0; u < U; u++) {                                      \
      const int j = (jbase) + NG * u;                                                    \
      ok[buf][u] = j < seg1;                                                             \
      const int jj = ok[buf][u] ? j : seg0;                                              \
      const int blk = blk_s[(jj >> 4) - b0], off = jj & 15;                              \
      const long idx = ((((long)blk * a.nh + h) * a.planes + pl_s[jj - seg0]) * 16 + off) * HD + c * EPL; \
      if (act) {                                                                         \
        kk[buf][u] = ldg_nt_u4(kp + idx);                                                \
        vv[buf][u] = ldg_nt_u4(vp + idx);                                                \
      } else {                                                                           \
        kk[buf][u] = make_uint4(0, 0, 0, 0);                                             \
        vv[buf][u] = make_uint4(0, 0, 0, 0);                                             \
      }                                                                                  \
    }
#define CDB_ATTN_SCORE(buf)                                                              \
    {                                                                                    \
      float sc[U];                                                                       \
      _Pragma("unroll") for (int u = 0; u < U; u++) {                                    \
        float kf[EPL];                                                                   \
        unpack16(kk[buf][u], kf, T());                                                   \
        float sdot = 0.f;                                                                \
        _Pragma("unroll") for (int e = 0; e < EPL; e++) sdot += qv[e] * kf[e];           \
        const float sd = sum16(sdot);                                                    \
        sc[u] = ok[buf][u] ? sd : -INFINITY;                                             \
      }                                                                                  \
      float mb = sc[0];                                                                  \
      _Pragma("unroll") for (int u = 1; u < U; u++) mb = fmaxf(mb, sc[u]);               \
      if (mb > -INFINITY) {                                                              \
        const float m_new = fmaxf(m_run, mb);                                            \
        const float corr = __expf(m_run - m_new);                                        \
        l_run *= corr;                                                                   \
        _Pragma("unroll") for (int e = 0; e < EPL; e++) o[e] *= corr;                    \
        _Pragma("unroll") for (int u = 0; u < U; u++) {                                  \
          float vf[EPL];                                                                 \
          unpack16(vv[buf][u], vf, T());                                                 \
          const float pj = __expf(sc[u] - m_new);                                        \
          l_run += pj;                                                                   \
          _Pragma("unroll") for (int e = 0; e < EPL; e++) o[e] += pj * vf[e];            \
        }                                                                                \
        m_run = m_new;                                                                   \
      }                                                                                  \
    }
    int jb = seg0 + grp;
    CDB_ATTN_LOAD(0, jb)
    for (; jb < seg1; jb += 2 * NG * U) {
      CDB_ATTN_LOAD(1, jb + NG * U)
      CDB_ATTN_SCORE(0)
      if (jb + NG * U >= seg1) break;
      CDB_ATTN_LOAD(0, jb + 2 * NG * U)
      CDB_ATTN_SCORE(1)
    }
#undef CDB_ATTN_LOAD
#undef CDB_ATTN_SCORE
  }

  // merge the NG groups (+ the self position) in fixed order
  if (c == 0) { gm[grp] = m_run; gl[grp] = l_run; }
  if (act) {
#pragma unroll
    for (int e = 0; e < EPL; e++) go[grp][c * EPL + e] = o[e];
  }
  if (threadIdx.x == 0) {
    if (has_self) {
      float sdot = 0.f;
      for (int i = 0; i < HD; i++) sdot += q_s[i] * a.scale * kself[i];
      gm[NG] = sdot;
      gl[NG] = 1.f;
    } else {
      gm[NG] = -INFINITY;
      gl[NG] = 0.f;
    }
  }
  __syncthreads();
  float M = -INFINITY;
  for (int g = 0; g < NG + 1; g++) M = fmaxf(M, gm[g]);
  float L = 0.f, O = 0.f;
  const int i = threadIdx.x;
  if (M != -INFINITY) {
    for (int g = 0; g < NG; g++) {
      const float f = __expf(gm[g] - M);
      L += gl[g] * f;
      if (i < HD) O += go[g][i] * f;
    }
    if (has_self) {
      const float f = __expf(gm[NG] - M);
      L += f;
      if (i < HD) O += vself[i] * f;
    }
  }
  if (a.n_split == 1) {
    if (i < HD) {
      const long oi = a.out_packed ? apack_off<T>(b, h * HD + i, a.nh * HD) : (long)b * a.ldo + h * HD + i;
      ((raw*)a.out)[oi] = Elt<T>::from_f32(O / L);
    }
    return;
  }
  float* part = a.part + ((long)bh * a.n_split + sp) * (HD + 2);
  if (i < HD) part[2 + i] = O;
  if (i == 0) { part[0] = M; part[1] = L; }
}

template <typename T, int HD, int R>
__global__ __launch_bounds__(HD) void k_attn_merge(AttnArgs a) {
  typedef typename Elt<T>::raw raw;
  const int bh = blockIdx.x;
  const int b = bh / a.nh, h = bh % a.nh;
  if (b >= min(ld_nvalid(a.n_valid, a.rows), a.rows)) return;
  const int i = threadIdx.x;
  const int ns = min(a.n_split, R);              // R >= n_split (launch)
  const float* pb = a.part + (long)bh * a.n_split * (HD + 2);
  // one round of loads: this thread's output element of every split (past
  // the split count the last split is re-read and not used), and the
  // (max, sum) of every split into LDS
  float ov[R];
#pragma unroll
  for (int u = 0; u < R; u++) ov[u] = pb[(long)min(u, ns - 1) * (HD + 2) + 2 + i];
  __shared__ float sm[R], sl[R];
  for (int s = i; s < ns; s += HD) {
    sm[s] = pb[(long)s * (HD + 2)];
    sl[s] = pb[(long)s * (HD + 2) + 1];
  }
  __syncthreads();
  float MM = -INFINITY;
  for (int s = 0; s < ns; s++) MM = fmaxf(MM, sm[s]);
  float LL = 0.f, OO = 0.f;
#pragma unroll
  for (int u = 0; u < R; u++) {                  // in split order
    if (u >= ns || sm[u] == -INFINITY) continue;
    const float f = __expf(sm[u] - MM);
    LL += sl[u] * f;
    OO += ov[u] * f;
  }
  const long oi = a.out_packed ? apack_off<T>(b, h * HD + i, a.nh * HD) : (long)b * a.ldo + h * HD + i;
  ((raw*)a.out)[oi] = Elt<T>::from_f32(OO / LL);
}

template <typename T, int HD>
static int attn_one(const AttnArgs& a, hipStream_t st) {
  dim3 grid(a.rows * a.nh, a.n_split);
  // 32 position streams per workgroup when the grid is small (at most two
  // workgroups per CU) and the rows are not so few that each stream gets a
  // handful of positions: B = 4..32 at context 1024 1-1.6% faster; B = 1, 2
  // and grids of 1024 workgroups and more keep 16 streams
  if (a.rows >= 4 && (long)a.rows * a.nh * a.n_split <= 512)
    hipLaunchKernelGGL((k_attn<T, HD, 512>), grid, dim3(512), 0, st, a);
  else
    hipLaunchKernelGGL((k_attn<T, HD, 256>), grid, dim3(256), 0, st, a);
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
static int merge_one(const AttnArgs& a, hipStream_t st) {
  const dim3 grid(a.rows * a.nh), block(HD);
  if (a.n_split <= 8) hipLaunchKernelGGL((k_attn_merge<T, HD, 8>), grid, block, 0, st, a);
  else if (a.n_split <= 16) hipLaunchKernelGGL((k_attn_merge<T, HD, 16>), grid, block, 0, st, a);
  else hipLaunchKernelGGL((k_attn_merge<T, HD, 32>), grid, block, 0, st, a);
  return hipGetLastError() == hipSuccess ? 0 : -1;
}

int attn_merge_launch(int dtype, int hd, const AttnArgs& a, hipStream_t st) {
  if (dtype == 0) {
    if (hd == 64) return merge_one<float, 64>(a, st);
    if (hd == 32) return merge_one<float, 32>(a, st);
    if (hd == 16) return merge_one<float, 16>(a, st);
  } else {
    if (hd == 128) return merge_one<bf16_t, 128>(a, st);
    if (hd == 96) return merge_one<bf16_t, 96>(a, st);
    if (hd == 64) return merge_one<bf16_t, 64>(a, st);
    if (hd == 16) return merge_one<bf16_t, 16>(a, st);
  }
  return -2;
}

}  // namespace cdb
