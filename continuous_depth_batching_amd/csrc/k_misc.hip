// Row-wise kernels of the CDB path: RMSNorm, the lookahead gate with stream
// compaction, coda preparation, token bookkeeping, prelude embedding,
// prefill setup and small row movers.
//
// "Depth-adaptive Inference of Looped Language Models via Continuous Depth
// Batching": the gate and its one-step lookahead (§4.3; §7 "Designing exit
// gates": earliest exit after step 2); the recurrent and coda queues and the
// refill of freed core slots (§4.1, Alg. 2); exit depths of cached positions
// feed the depth-indexed read rule (§4.2); prefill positions are at full
// depth (App. A.1).
#include "common.h"
#include "kernels.h"

namespace cdb {

// Exclusive prefix count of `f` over a 256-thread block (wave ballots).
__device__ __forceinline__ int block_rank256(bool f, int* wt, int& total) {
  const unsigned long long bal = __ballot(f);
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int in_wave = __popcll(bal & ((1ull << lane) - 1ull));
  __syncthreads();
  if (lane == 0) wt[w] = __popcll(bal);
  __syncthreads();
  int base = 0;
  for (int i = 0; i < w; i++) base += wt[i];
  total = wt[0] + wt[1] + wt[2] + wt[3];
  return base + in_wave;
}

// ---------------------------------------------------- residual add + RMSNorm
// x = resid + sum of split partials (fixed split order; written back), then
// y = g * x / sqrt(mean(x^2) + eps) in fp32, stored in the GEMM input type.
// The loads that need neither the row count nor the slot map (the gain and
// the first round of partials) are issued before those two are read, so the
// kernel waits on two memory round trips, not four.
template <typename T, int MAXV, int SB>
__global__ __launch_bounds__(256) void k_rmsnorm(NormArgs a) {
  typedef typename Elt<T>::raw raw;
  __shared__ float red[4];
  const int b = blockIdx.x;
  const int H4 = a.H >> 2;                       // H is a multiple of 16
  const bool has_part = a.part != nullptr && a.part_sk > 0;
  // first SB splits' partials of row b (b < rows <= part_rows, so in bounds
  // whatever the valid count; loads past the split count re-read the last split)
  float4 pv[SB][MAXV];
  auto load_round = [&](int s0) {
#pragma unroll
    for (int u = 0; u < SB; u++) {
      const int s = min(s0 + u, a.part_sk - 1);
      const float4* p = (const float4*)(a.part + ((long)s * a.part_rows + b) * a.H);
#pragma unroll
      for (int k = 0; k < MAXV; k++) {
        const int i = threadIdx.x + 256 * k;
        pv[u][k] = i < H4 ? p[i] : make_float4(0.f, 0.f, 0.f, 0.f);
      }
    }
  };
  if (has_part) load_round(0);
  float4 gv[MAXV];
  const float4* g4 = (const float4*)a.gain;
#pragma unroll
  for (int k = 0; k < MAXV; k++) {
    const int i = threadIdx.x + 256 * k;
    gv[k] = (a.out && i < H4) ? g4[i] : make_float4(0.f, 0.f, 0.f, 0.f);
  }
  const int nv = ld_nvalid(a.n_valid, a.rows);
  const int n = min(nv, a.rows);
  if (b == 0 && threadIdx.x == 0 && nv > a.rows) flag_err(a.err, ERR_COUNT);
  raw* out = a.out ? (raw*)a.out + (a.packed ? 0L : (long)b * a.ldo) : nullptr;
  // output element i of this row (row-major, or the decode GEMMs' packed layout)
  auto oi = [&](int i) -> long { return a.packed ? apack_off<T>(b, i, a.H) : (long)i; };
  if (b >= n) {
    if (out)
      for (int i = threadIdx.x; i < a.H; i += 256) out[oi(i)] = Elt<T>::from_f32(0.f);
    return;
  }
  const int r = a.slot ? clamp_chk(a.slot[b], 0, a.x_rows - 1, a.err, ERR_SLOT) : b;
  float4* x = (float4*)(a.x + (long)r * a.ldx);
  // MAXV float4 per thread hold the row (H <= MAXV * 1024)
  float4 xv[MAXV];
#pragma unroll
  for (int k = 0; k < MAXV; k++) {
    const int i = threadIdx.x + 256 * k;
    xv[k] = i < H4 ? x[i] : make_float4(0.f, 0.f, 0.f, 0.f);
  }
  if (has_part) {
    // partials added in split order, SB splits' loads in flight at a time
    for (int s0 = 0;;) {
#pragma unroll
      for (int u = 0; u < SB; u++) {
        if (s0 + u < a.part_sk) {
#pragma unroll
          for (int k = 0; k < MAXV; k++) {
            xv[k].x += pv[u][k].x; xv[k].y += pv[u][k].y; xv[k].z += pv[u][k].z; xv[k].w += pv[u][k].w;
          }
        }
      }
      s0 += SB;
      if (s0 >= a.part_sk) break;
      load_round(s0);
    }
#pragma unroll
    for (int k = 0; k < MAXV; k++) {
      const int i = threadIdx.x + 256 * k;
      if (i < H4) x[i] = xv[k];
    }
  }
  if (!out) return;
  float ss = 0.f;
#pragma unroll
  for (int k = 0; k < MAXV; k++) ss += xv[k].x * xv[k].x + xv[k].y * xv[k].y + xv[k].z * xv[k].z + xv[k].w * xv[k].w;
  ss = block_sum256(ss, red);
  const float rstd = 1.0f / sqrtf(ss / (float)a.H + a.eps);
#pragma unroll
  for (int k = 0; k < MAXV; k++) {
    const int i = threadIdx.x + 256 * k;
    if (i < H4) {
      const float4 gg = gv[k];
      raw* o = out + oi(4 * i);                  // four consecutive columns stay adjacent in both layouts
      o[0] = Elt<T>::from_f32(xv[k].x * rstd * gg.x);
      o[1] = Elt<T>::from_f32(xv[k].y * rstd * gg.y);
      o[2] = Elt<T>::from_f32(xv[k].z * rstd * gg.z);
      o[3] = Elt<T>::from_f32(xv[k].w * rstd * gg.w);
    }
  }
}

// The same norm for decode batches (few rows): one 1024-thread workgroup per
// row, each thread holding E2 pairs of columns, so the residual row, every
// split partial (up to 24) and the gain are in flight at once -- one memory
// round trip -- instead of rounds of split loads per thread.  Same sums in
// the same order (residual, then the splits in split order, per element);
// the sum of squares is reduced over the block in a fixed order.
template <typename T, int E2, int SBW>
__global__ __launch_bounds__(1024) void k_rmsnorm_wide(NormArgs a) {
  typedef typename Elt<T>::raw raw;
  __shared__ float red[16];
  const int b = blockIdx.x;
  const int H2 = a.H >> 1;
  const bool has_part = a.part != nullptr && a.part_sk > 0;
  // the SBW >= part_sk split partials, unconditional loads (past the split
  // count they re-read the last split and are not added)
  float2 pv[SBW][E2];
  if (has_part) {
#pragma unroll
    for (int u = 0; u < SBW; u++) {
      const float2* p = (const float2*)(a.part + ((long)min(u, a.part_sk - 1) * a.part_rows + b) * a.H);
#pragma unroll
      for (int k = 0; k < E2; k++) {
        const int i = threadIdx.x + 1024 * k;
        pv[u][k] = i < H2 ? p[i] : make_float2(0.f, 0.f);
      }
    }
  }
  float2 gv[E2];
#pragma unroll
  for (int k = 0; k < E2; k++) {
    const int i = threadIdx.x + 1024 * k;
    gv[k] = (a.out && i < H2) ? ((const float2*)a.gain)[i] : make_float2(0.f, 0.f);
  }
  const int nv = ld_nvalid(a.n_valid, a.rows);
  const int n = min(nv, a.rows);
  if (b == 0 && threadIdx.x == 0 && nv > a.rows) flag_err(a.err, ERR_COUNT);
  raw* out = a.out ? (raw*)a.out + (a.packed ? 0L : (long)b * a.ldo) : nullptr;
  auto oi = [&](int i) -> long { return a.packed ? apack_off<T>(b, i, a.H) : (long)i; };
  if (b >= n) {
    if (out)
      for (int i = threadIdx.x; i < a.H; i += 1024) out[oi(i)] = Elt<T>::from_f32(0.f);
    return;
  }
  const int r = a.slot ? clamp_chk(a.slot[b], 0, a.x_rows - 1, a.err, ERR_SLOT) : b;
  float2* x = (float2*)(a.x + (long)r * a.ldx);
  float2 xv[E2];
#pragma unroll
  for (int k = 0; k < E2; k++) {
    const int i = threadIdx.x + 1024 * k;
    xv[k] = i < H2 ? x[i] : make_float2(0.f, 0.f);
  }
  if (has_part) {
#pragma unroll
    for (int u = 0; u < SBW; u++) {
      if (u < a.part_sk) {
#pragma unroll
        for (int k = 0; k < E2; k++) { xv[k].x += pv[u][k].x; xv[k].y += pv[u][k].y; }
      }
    }
#pragma unroll
    for (int k = 0; k < E2; k++) {
      const int i = threadIdx.x + 1024 * k;
      if (i < H2) x[i] = xv[k];
    }
  }
  if (!out) return;
  float ss = 0.f;
#pragma unroll
  for (int k = 0; k < E2; k++) ss += xv[k].x * xv[k].x + xv[k].y * xv[k].y;
  ss = wave_sum(ss);
  const int wv = threadIdx.x >> 6;
  if ((threadIdx.x & 63) == 0) red[wv] = ss;
  __syncthreads();
  float tot = 0.f;
#pragma unroll
  for (int i = 0; i < 16; i++) tot += red[i];
  const float rstd = 1.0f / sqrtf(tot / (float)a.H + a.eps);
#pragma unroll
  for (int k = 0; k < E2; k++) {
    const int i = threadIdx.x + 1024 * k;
    if (i < H2) {
      raw* o = out + oi(2 * i);                  // two consecutive columns stay adjacent in both layouts
      o[0] = Elt<T>::from_f32(xv[k].x * rstd * gv[k].x);
      o[1] = Elt<T>::from_f32(xv[k].y * rstd * gv[k].y);
    }
  }
}

// Residual add with the next RMSNorm deferred (decode batches that take
// the split projections): one thread per column, a workgroup per (256
// columns, row), so the add is spread over H / 256 workgroups per row
// instead of one workgroup holding the whole row for its sum of squares.
// The residual row plus every split are in flight at once; the sums are
// the norm kernel's (residual, then the splits in split order), so the
// residual stream is the same bit for bit.  The row statistics leave as one
// sum of x^2 per workgroup (wave sums, then the four waves in order), and
// the consumer applies 1 / rms from the row's H / 256 sums.
template <typename T, int SBW>
__global__ __launch_bounds__(256) void k_resid_defer(NormArgs a) {
  typedef typename Elt<T>::raw raw;
  const int m = blockIdx.y;
  const int n = blockIdx.x * 256 + threadIdx.x;
  const bool in = n < a.H;
  const int nc = min(n, a.H - 1);
  float pv[SBW];
#pragma unroll
  for (int u = 0; u < SBW; u++) pv[u] = a.part[((long)min(u, a.part_sk - 1) * a.part_rows + m) * a.H + nc];
  const float gn = a.gain[nc];
  const int nv = ld_nvalid(a.n_valid, a.rows);
  if (m == 0 && blockIdx.x == 0 && threadIdx.x == 0 && nv > a.rows) flag_err(a.err, ERR_COUNT);
  raw* out = (raw*)a.out;
  const long si = (long)m * gridDim.x + blockIdx.x;
  if (m >= min(nv, a.rows)) {                    // uniform per workgroup
    if (in) out[apack_off<T>(m, n, a.H)] = Elt<T>::from_f32(0.f);
    if (threadIdx.x == 0) a.ss_out[si] = 0.f;
    return;
  }
  const int r = a.slot ? clamp_chk(a.slot[m], 0, a.x_rows - 1, a.err, ERR_SLOT) : m;
  float* xp = a.x + (long)r * a.ldx;
  float x = xp[nc];
#pragma unroll
  for (int u = 0; u < SBW; u++)
    if (u < a.part_sk) x += pv[u];
  if (in) {
    xp[n] = x;
    out[apack_off<T>(m, n, a.H)] = Elt<T>::from_f32(gn * x);
  }
  __shared__ float red[4];
  const float q = wave_sum(in ? x * x : 0.f);
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = q;
  __syncthreads();
  if (threadIdx.x == 0) a.ss_out[si] = ((red[0] + red[1]) + red[2]) + red[3];
}

template <typename T>
static void resid_defer_one(const NormArgs& a, hipStream_t st) {
  const dim3 grid((a.H + 255) / 256, a.rows);
  const int sk = a.part_sk;
  if (sk <= 4) hipLaunchKernelGGL((k_resid_defer<T, 4>), grid, dim3(256), 0, st, a);
  else if (sk <= 8) hipLaunchKernelGGL((k_resid_defer<T, 8>), grid, dim3(256), 0, st, a);
  else if (sk <= 16) hipLaunchKernelGGL((k_resid_defer<T, 16>), grid, dim3(256), 0, st, a);
  else hipLaunchKernelGGL((k_resid_defer<T, 24>), grid, dim3(256), 0, st, a);
}

int resid_defer_launch(int dtype, const NormArgs& a, hipStream_t st) {
  if (a.rows <= 0) return 0;
  if (!a.part || a.part_sk < 1 || a.part_sk > 24 || a.part_rows < a.rows || !a.gain || !a.out || !a.ss_out ||
      !a.packed || a.H % 32 || a.H > 4096)
    return -2;
  if (dtype == 0) resid_defer_one<float>(a, st);
  else resid_defer_one<bf16_t>(a, st);
  return hipGetLastError() == hipSuccess ? 0 : -1;
}

template <typename T, int MAXV>
static void norm_sb(const NormArgs& a, hipStream_t st) {
  const int sk = a.part ? a.part_sk : 1;
  if (MAXV > 2 || sk <= 4) hipLaunchKernelGGL((k_rmsnorm<T, MAXV, 4>), dim3(a.rows), dim3(256), 0, st, a);
  else if (sk <= 8) hipLaunchKernelGGL((k_rmsnorm<T, MAXV, 8>), dim3(a.rows), dim3(256), 0, st, a);
  else if (sk <= 12) hipLaunchKernelGGL((k_rmsnorm<T, MAXV, 12>), dim3(a.rows), dim3(256), 0, st, a);
  else hipLaunchKernelGGL((k_rmsnorm<T, MAXV, 16>), dim3(a.rows), dim3(256), 0, st, a);
}

template <typename T>
static void norm_one(const NormArgs& a, hipStream_t st) {
  if (a.H <= 1024) norm_sb<T, 1>(a, st);
  else if (a.H <= 2048) norm_sb<T, 2>(a, st);
  else norm_sb<T, 6>(a, st);
}

template <typename T, int E2, int SB>
static void norm_wide_one(const NormArgs& a, hipStream_t st) {
  if constexpr (E2 * SB <= 32)     // only the forms norm_launch selects (no register spills)
    hipLaunchKernelGGL((k_rmsnorm_wide<T, E2, SB>), dim3(a.rows), dim3(1024), 0, st, a);
}

template <typename T, int E2>
static void norm_wide_sb(const NormArgs& a, hipStream_t st) {
  const int sk = a.part ? a.part_sk : 0;
  if (sk <= 4) norm_wide_one<T, E2, 4>(a, st);
  else if (sk <= 8) norm_wide_one<T, E2, 8>(a, st);
  else if (sk <= 12) norm_wide_one<T, E2, 12>(a, st);
  else if (sk <= 16) norm_wide_one<T, E2, 16>(a, st);
  else norm_wide_one<T, E2, 24>(a, st);
}

template <typename T>
static void norm_wide(const NormArgs& a, hipStream_t st) {
  const int e2 = (a.H / 2 + 1023) / 1024;
  if (e2 <= 1) norm_wide_sb<T, 1>(a, st);
  else if (e2 == 2) norm_wide_sb<T, 2>(a, st);
  else norm_wide_sb<T, 3>(a, st);
}

int norm_launch(int dtype, const NormArgs& a, hipStream_t st) {
  if (a.rows <= 0) return 0;
  if (a.H > 6144) return -2;
  // decode-sized batches take the 1024-thread form (all loads in one round)
  // where its partials fit the register budget of 16 waves per workgroup
  // (at most 32 float2 of partials per thread)
  const int sk = a.part ? a.part_sk : 0;
  const int sbw = sk <= 4 ? 4 : (sk <= 8 ? 8 : (sk <= 12 ? 12 : (sk <= 16 ? 16 : 24)));
  const bool wide = a.rows <= 256 && sk <= 24 && ((a.H / 2 + 1023) / 1024) * sbw <= 32;
  if (dtype == 0) wide ? norm_wide<float>(a, st) : norm_one<float>(a, st);
  else wide ? norm_wide<bf16_t>(a, st) : norm_one<bf16_t>(a, st);
  return hipGetLastError() == hipSuccess ? 0 : -1;
}

// ------------------------------------------------- gate + stream compaction
// Block b evaluates the gate of a valid row that does not leave now: the
// linear gate z_b = gate_w . RMSNorm(h_b) + bias, or (kind 1, loops >= 2)
// the convergence value z_b = |h_b - h_prev_b| / |h_b|; the last block to
// arrive partitions the rows (stable): continuing rows move to the front
// with depth + 1 (exit_at = depth + 1 when the gate fired), leaving rows
// append to the exit queue.
__global__ __launch_bounds__(256) void k_gate_compact(GateArgs a) {
  __shared__ float red[4];
  __shared__ int wt[4];
  __shared__ int flag;
  const int b = blockIdx.x;
  const int nv = *a.n_valid;
  const int n = min(nv, a.rows_pad);
  if (b == 0 && threadIdx.x == 0 && nv > a.rows_pad) flag_err(a.err, ERR_COUNT);
  if (b < n && a.gate_enabled && a.depth[b] != a.exit_at[b] && (a.kind == 0 || a.depth[b] >= 2)) {
    const int sl = clamp_chk(a.slot[b], 0, a.n_slots - 1, a.err, ERR_SLOT);
    const float* x = a.state + (long)sl * a.H;
    float s1 = 0.f, s2 = 0.f;
    if (a.kind == 0) {
      for (int i = threadIdx.x; i < a.H; i += 256) {
        const float v = x[i];
        s2 += v * v;
        s1 += v * a.gate_w[i];
      }
    } else {
      const float* xp = a.prev + (long)sl * a.H;
      for (int i = threadIdx.x; i < a.H; i += 256) {
        const float v = x[i], dv = v - xp[i];
        s2 += v * v;
        s1 += dv * dv;
      }
    }
    s2 = block_sum256(s2, red);
    s1 = block_sum256(s1, red);
    if (threadIdx.x == 0)
      a.z[b] = a.kind == 0 ? s1 / sqrtf(s2 / (float)a.H + a.eps) + a.bias : sqrtf(s1) / sqrtf(s2);
  }
  __threadfence();
  __syncthreads();
  if (threadIdx.x == 0) {
    const int old = atomicAdd(a.counter, 1);
    flag = (old == (int)gridDim.x - 1);
    if (flag) *a.counter = 0;
  }
  __syncthreads();
  if (!flag) return;
  __threadfence();

  int cont_base = 0, exit_base = *a.q_n, fired_base = 0, n_exit = 0, next_base = 0;
  for (int c0 = 0; c0 < n; c0 += 256) {
    const int r = c0 + threadIdx.x;
    const bool valid = r < n;
    int sl = 0, sq = 0, ps = 0, d = 0, ea = 0;
    if (valid) { sl = a.slot[r]; sq = a.seq[r]; ps = a.pos[r]; d = a.depth[r]; ea = a.exit_at[r]; }
    const bool ex = valid && d == ea;
    bool fire = false;
    if (valid && !ex && a.gate_enabled) {
      if (a.kind == 0) fire = __builtin_nontemporal_load(a.z + r) > a.threshold;
      else fire = d >= 2 && __builtin_nontemporal_load(a.z + r) < a.tau;
    }
    const bool cont = valid && !ex;
    const int new_exit = fire ? d + 1 : ea;
    const bool next = cont && new_exit == d + 1;     // leaves after the next step
    int tc, te, tf, tn;
    const int rc = block_rank256(cont, wt, tc);
    const int re = block_rank256(ex, wt, te);
    block_rank256(fire, wt, tf);
    const int rn = block_rank256(next, wt, tn);
    __syncthreads();                                 // all rows of this chunk read
    if (cont) {
      const int o = cont_base + rc;
      a.slot[o] = sl; a.seq[o] = sq; a.pos[o] = ps;
      a.depth[o] = d + 1;
      a.exit_at[o] = new_exit;
    }
    if (ex) {
      const int o = exit_base + re;
      if (o < a.q_cap) { a.q_slot[o] = sl; a.q_seq[o] = sq; a.q_pos[o] = ps; a.q_depth[o] = d; }
      else flag_err(a.err, ERR_COUNT);
    }
    if (next) a.fired_seq[next_base + rn] = sq;
    cont_base += tc; exit_base += te; fired_base += tf; next_base += tn; n_exit += te;
    __syncthreads();
  }
  if (threadIdx.x == 0) {
    *a.n_valid = cont_base;
    *a.q_n = min(exit_base, a.q_cap);
    a.counts[0] = cont_base;
    a.counts[1] = n_exit;
    a.counts[2] = fired_base;
    a.counts[3] = next_base;
  }
}

int gate_compact_launch(const GateArgs& a, hipStream_t st) {
  hipLaunchKernelGGL(k_gate_compact, dim3(a.rows_pad), dim3(256), 0, st, a);
  return hipGetLastError() == hipSuccess ? 0 : -1;
}

// ------------------------------------------------------------- coda prep
__global__ __launch_bounds__(256) void k_coda_prep(CodaPrepArgs a) {
  const int r = blockIdx.x;
  const int qn = *a.q_n;
  if (r == 0 && threadIdx.x == 0 && qn > a.rows_pad) flag_err(a.err, ERR_COUNT);
  if (r >= qn) return;
  const int sl = clamp_chk(a.q_slot[r], 0, a.n_slots - 1, a.err, ERR_SLOT);
  const int sq = clamp_chk(a.q_seq[r], 0, a.max_seqs - 1, a.err, ERR_SEQ);
  const int ps = clamp_chk(a.q_pos[r], 0, a.max_pos - 1, a.err, ERR_POS);
  const float* x = a.state + (long)sl * a.H;
  float* y = a.resid + (long)r * a.H;
  for (int i = threadIdx.x; i < a.H; i += 256) {
    const float v = x[i];
    y[i] = v;
    if (a.states_out) a.states_out[(long)r * a.H + i] = v;
  }
  if (threadIdx.x == 0) {
    const int blk = clamp_chk(a.btab[(long)sq * a.bt_stride + (ps >> 4)], 0, a.num_blocks - 1, a.err, ERR_BLOCK);
    a.emap[(long)blk * 16 + (ps & 15)] = (uint8_t)a.q_depth[r];
    a.pos1[r] = ps + 1;
  }
}

int coda_prep_launch(const CodaPrepArgs& a, hipStream_t st) {
  hipLaunchKernelGGL(k_coda_prep, dim3(a.rows_pad), dim3(256), 0, st, a);
  return hipGetLastError() == hipSuccess ? 0 : -1;
}

// One workgroup per (exit row, core layer): the row's K and V at plane e - 1
// of its (block, offset), for every head, into planes e .. planes - 1, in
// 16-byte pieces ("Depth-adaptive Inference of Looped Language Models via
// Continuous Depth Batching", §4.2: the skipped depth slots of a token hold
// the KV of its last loop).
__global__ __launch_bounds__(256) void k_kv_exit_copy(KvExitCopyArgs a) {
  const int r = blockIdx.x, l = blockIdx.y;
  if (r >= min(*a.q_n, a.rows_pad)) return;
  const int e = clamp_chk(a.q_depth[r], 1, a.planes, a.err, ERR_DEPTH);
  if (e >= a.planes) return;
  const int sq = clamp_chk(a.q_seq[r], 0, a.max_seqs - 1, a.err, ERR_SEQ);
  const int ps = clamp_chk(a.q_pos[r], 0, a.max_pos - 1, a.err, ERR_POS);
  const int blk = clamp_chk(a.btab[(long)sq * a.bt_stride + (ps >> 4)], 0, a.num_blocks - 1, a.err, ERR_BLOCK);
  const int pieces = a.hd * a.el / 16;          // 16-byte pieces of one K (or V) row
  const int fill = a.planes - e;
  const int total = 2 * a.nh * fill * pieces;
  char* kb = (char*)a.kpool + (long)l * a.layer_elems * a.el;
  char* vb = (char*)a.vpool + (long)l * a.layer_elems * a.el;
  for (int i = threadIdx.x; i < total; i += 256) {
    const int c = i % pieces;
    const int t = i / pieces;
    const int p = t % fill;
    const int h = (t / fill) % a.nh;
    char* base = (t / fill) / a.nh ? vb : kb;
    const long row0 = (((long)blk * a.nh + h) * a.planes) * 16 + (ps & 15);   // plane 0 of this (block, head, offset)
    const long src = (row0 + (long)(e - 1) * 16) * a.hd * a.el + 16L * c;
    const long dst = (row0 + (long)(e + p) * 16) * a.hd * a.el + 16L * c;
    *(uint4*)(base + dst) = *(const uint4*)(base + src);
  }
}

int kv_exit_copy_launch(const KvExitCopyArgs& a, hipStream_t st) {
  if (a.rows_pad < 1 || a.n_core < 1 || (a.hd * a.el) % 16) return -2;
  hipLaunchKernelGGL(k_kv_exit_copy, dim3(a.rows_pad, a.n_core), dim3(256), 0, st, a);
  return hipGetLastError() == hipSuccess ? 0 : -1;
}

// ---------------------------------------------------------- bookkeeping
__global__ __launch_bounds__(256) void k_book(BookArgs a) {
  __shared__ int wt[4];
  const int nr = a.n_rows ? *a.n_rows : a.host_rows;
  const int n = min(nr, a.rows_cap);
  if (threadIdx.x == 0 && nr > a.rows_cap) flag_err(a.err, ERR_COUNT);
  int c_base = 0;
  const int d_base = a.d_n ? *a.d_n : 0;
  for (int c0 = 0; c0 < n; c0 += 256) {
    const int r = c0 + threadIdx.x;
    const bool valid = r < n;
    int sl = 0, sq = 0, ps = 0, t = 0;
    bool cont = false;
    if (valid) {
      sl = a.r_slot[r];
      sq = clamp_chk(a.r_seq[r], 0, a.max_seqs - 1, a.err, ERR_SEQ);
      ps = a.r_pos[r];
      t = a.tok[r];
      const int e = a.r_depth ? a.r_depth[r] : a.depth_uniform;
      const int idx = a.n_gen[sq];                // one row per sequence in a batch
      if (idx >= 0 && idx < a.max_out) {
        a.tokens_out[(long)sq * a.max_out + idx] = t;
        a.exits_out[(long)sq * a.max_out + idx] = e;
      }
      a.n_gen[sq] = idx + 1;
      cont = idx + 1 < a.n_out[sq];
      if (a.tokens_rows_out) a.tokens_rows_out[r] = t;
    }
    int tot;
    const int rk = block_rank256(cont, wt, tot);
    if (cont) {
      const int o = c_base + rk;
      a.c_slot[o] = sl; a.c_seq[o] = sq; a.c_pos[o] = ps + 1; a.c_tok[o] = t;
      const int od = d_base + o;
      if (a.d_n && od < a.d_cap) {
        a.d_slot[od] = sl; a.d_seq[od] = sq; a.d_pos[od] = ps + 1;
        a.d_depth[od] = 1; a.d_exit_at[od] = a.r_max;
      } else if (a.d_n) {
        flag_err(a.err, ERR_COUNT);
      }
    }
    c_base += tot;
  }
  if (threadIdx.x == 0) {
    *a.c_n = c_base;
    if (a.d_n) *a.d_n = min(d_base + c_base, a.d_cap);
    if (a.q_n_reset) *a.q_n_reset = 0;
  }
}

int book_launch(const BookArgs& a, hipStream_t st) {
  hipLaunchKernelGGL(k_book, dim3(1), dim3(256), 0, st, a);
  return hipGetLastError() == hipSuccess ? 0 : -1;
}

// ------------------------------------------------------ prelude embedding
template <typename raw>
__global__ __launch_bounds__(256) void k_prelude_embed(PreludeEmbedArgs a) {
  const int r = blockIdx.x;
  if (r >= *a.c_n) return;
  const int sl = clamp_chk(a.c_slot[r], 0, a.n_slots - 1, a.err, ERR_SLOT);
  float* x = a.state + (long)sl * a.H;
  if (a.pre_out && a.inject) {
    const float* e = a.pre_out + (long)r * a.H;
    float* inj = a.inject + (long)sl * a.H;
    for (int i = threadIdx.x; i < a.H; i += 256) { inj[i] = e[i]; x[i] = 0.f; }
  } else if (a.pre_out) {
    const float* e = a.pre_out + (long)r * a.H;
    for (int i = threadIdx.x; i < a.H; i += 256) x[i] = e[i];
  } else {
    const int tok = clamp_chk(a.c_tok[r], 0, a.vocab - 1, a.err, ERR_TOKEN);
    const raw* e = (const raw*)a.embed + (long)tok * a.H;
    for (int i = threadIdx.x; i < a.H; i += 256) x[i] = ld_f32(e[i]);
  }
  if (threadIdx.x == 0) {
    const int sq = clamp_chk(a.c_seq[r], 0, a.max_seqs - 1, a.err, ERR_SEQ);
    const int ps = clamp_chk(a.c_pos[r], 0, a.max_pos - 1, a.err, ERR_POS);
    const int blk = clamp_chk(a.btab[(long)sq * a.bt_stride + (ps >> 4)], 0, a.num_blocks - 1, a.err, ERR_BLOCK);
    a.emap[(long)blk * 16 + (ps & 15)] = (uint8_t)a.r_max;
  }
}

int prelude_embed_launch(const PreludeEmbedArgs& a, hipStream_t st) {
  if (a.dtype == 0) hipLaunchKernelGGL(k_prelude_embed<float>, dim3(a.rows_pad), dim3(256), 0, st, a);
  else hipLaunchKernelGGL(k_prelude_embed<uint16_t>, dim3(a.rows_pad), dim3(256), 0, st, a);
  return hipGetLastError() == hipSuccess ? 0 : -1;
}

// ---------------------------------------------------------- prefill setup
template <typename raw>
__global__ __launch_bounds__(256) void k_prefill_setup(PrefillSetupArgs a) {
  __shared__ int s_i;
  const int t = blockIdx.x;
  if (threadIdx.x == 0) {
    int lo = 0, hi = a.n_seqs - 1;                // last i with cu[i] <= t
    while (lo < hi) {
      const int mid = (lo + hi + 1) >> 1;
      if (a.cu[mid] <= t) lo = mid; else hi = mid - 1;
    }
    s_i = lo;
  }
  __syncthreads();
  const int i = s_i;
  const int sq = clamp_chk(a.seq[i], 0, a.max_seqs - 1, a.err, ERR_SEQ);
  const int ps = clamp_chk(a.start_pos[i] + (t - a.cu[i]), 0, a.max_pos - 1, a.err, ERR_POS);
  const int tok = clamp_chk(a.tokens[t], 0, a.vocab - 1, a.err, ERR_TOKEN);
  const raw* e = (const raw*)a.embed + (long)tok * a.H;
  float* x = a.resid + (long)t * a.H;
  for (int k = threadIdx.x; k < a.H; k += 256) x[k] = ld_f32(e[k]);
  if (threadIdx.x == 0) {
    a.tok_seq[t] = sq;
    a.tok_pos[t] = ps;
    const int blk = clamp_chk(a.btab[(long)sq * a.bt_stride + (ps >> 4)], 0, a.num_blocks - 1, a.err, ERR_BLOCK);
    a.emap[(long)blk * 16 + (ps & 15)] = (uint8_t)a.r_max;
  }
  if (t == 0 && threadIdx.x == 0) {               // final tokens of prompts ending here
    int nf = 0;
    for (int s = 0; s < a.n_seqs; s++) {
      if (!a.is_final[s]) continue;
      const int last = a.cu[s + 1] - 1;
      a.f_idx[nf] = last;
      a.f_slot[nf] = a.slot[s];
      a.f_seq[nf] = a.seq[s];
      a.f_pos[nf] = a.start_pos[s] + (last - a.cu[s]);
      nf++;
    }
    *a.f_n = nf;
  }
}

int prefill_setup_launch(const PrefillSetupArgs& a, hipStream_t st) {
  if (a.dtype == 0) hipLaunchKernelGGL(k_prefill_setup<float>, dim3(a.n_tokens), dim3(256), 0, st, a);
  else hipLaunchKernelGGL(k_prefill_setup<uint16_t>, dim3(a.n_tokens), dim3(256), 0, st, a);
  return hipGetLastError() == hipSuccess ? 0 : -1;
}

// ------------------------------------------------------------ row movers
__global__ __launch_bounds__(256) void k_gather_rows(GatherRowsArgs a) {
  const int r = blockIdx.x;
  if (r >= (a.n ? *a.n : a.rows)) return;
  const int src = clamp_chk(a.idx[r], 0, a.x_rows - 1, a.err, ERR_COUNT);
  const float* x = a.x + (long)src * a.ldx;
  float* y = a.out + (long)r * a.ldo;
  for (int i = threadIdx.x; i < a.H; i += 256) y[i] = x[i];
}

int gather_rows_launch(const GatherRowsArgs& a, hipStream_t st) {
  if (a.rows <= 0) return 0;
  hipLaunchKernelGGL(k_gather_rows, dim3(a.rows), dim3(256), 0, st, a);
  return hipGetLastError() == hipSuccess ? 0 : -1;
}

__global__ __launch_bounds__(256) void k_add_rows(AddRowsArgs a) {
  const int r = blockIdx.x;
  if (r >= ld_nvalid(a.n_valid, a.rows)) return;
  const int sl = a.slot ? clamp_chk(a.slot[r], 0, a.n_slots - 1, a.err, ERR_SLOT) : r;
  float* x = a.x + (long)sl * a.H;
  const float* y = a.y + (long)sl * a.H;
  for (int i = threadIdx.x; i < a.H; i += 256) x[i] += y[i];
}

__global__ __launch_bounds__(256) void k_save_rows(AddRowsArgs a) {
  const int r = blockIdx.x;
  if (r >= ld_nvalid(a.n_valid, a.rows)) return;
  const int sl = a.slot ? clamp_chk(a.slot[r], 0, a.n_slots - 1, a.err, ERR_SLOT) : r;
  const float* src = a.y + (long)sl * a.H;
  float* dst = a.x + (long)sl * a.H;
  for (int i = threadIdx.x; i < a.H; i += 256) dst[i] = src[i];
}

int save_rows_launch(const AddRowsArgs& a, hipStream_t st) {
  if (a.rows <= 0) return 0;
  hipLaunchKernelGGL(k_save_rows, dim3(a.rows), dim3(256), 0, st, a);
  return hipGetLastError() == hipSuccess ? 0 : -1;
}

int add_rows_launch(const AddRowsArgs& a, hipStream_t st) {
  if (a.rows <= 0) return 0;
  hipLaunchKernelGGL(k_add_rows, dim3(a.rows), dim3(256), 0, st, a);
  return hipGetLastError() == hipSuccess ? 0 : -1;
}

template <typename raw>
__global__ __launch_bounds__(256) void k_embed_tok(EmbedTokArgs a) {
  const int r = blockIdx.x;
  if (r >= (a.n ? *a.n : a.rows)) return;
  const int tok = clamp_chk(a.tok[r], 0, a.vocab - 1, a.err, ERR_TOKEN);
  const raw* e = (const raw*)a.embed + (long)tok * a.H;
  float* y = a.out + (long)r * a.ldo;
  for (int i = threadIdx.x; i < a.H; i += 256) y[i] = ld_f32(e[i]);
}

int embed_tok_launch(const EmbedTokArgs& a, hipStream_t st) {
  if (a.rows <= 0) return 0;
  if (a.dtype == 0) hipLaunchKernelGGL(k_embed_tok<float>, dim3(a.rows), dim3(256), 0, st, a);
  else hipLaunchKernelGGL(k_embed_tok<uint16_t>, dim3(a.rows), dim3(256), 0, st, a);
  return hipGetLastError() == hipSuccess ? 0 : -1;
}

}  // namespace cdb
