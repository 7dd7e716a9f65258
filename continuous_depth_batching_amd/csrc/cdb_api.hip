// Host side of the C ABI declared in include/cdb.h: argument validation,
// workspace carving, and the kernel sequences of each stage.
//
// Stage sequences ("Depth-adaptive Inference of Looped Language Models via
// Continuous Depth Batching", §4.1 and Alg. 1 / Alg. 2):
//   core step  : per core layer  norm -> QKV -> attention(+K/V write) ->
//                O + residual -> norm -> gate/up + SwiGLU -> down + residual
//   gate       : gate + stream compaction into the recurrent / coda queues
//   boundary   : coda (depth map, coda layers, final norm, LM head, argmax)
//                then prelude of the successor tokens into the core batch
//   prefill    : embedding (+ prelude layers), r_max loops of the core over
//                the chunk with K/V written to every plane, coda layers, LM
//                head for final prompt tokens only, prelude of first tokens
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <string>
#include <array>
#include <vector>

#include "../../include/cdb.h"
#include "kernels.h"
#include <cstdlib>
#include <mutex>

using namespace cdb;

namespace {

thread_local std::string g_err;

int fail(int code, const char* fmt, ...) __attribute__((format(printf, 2, 3)));
int fail(int code, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_err = buf;
  return code;
}

#define HIPCHK(x)                                                                     \
  do {                                                                                \
    hipError_t e_ = (x);                                                              \
    if (e_ != hipSuccess) return fail(CDB_EHIP, "%s: %s", #x, hipGetErrorString(e_)); \
  } while (0)
#define LCHK(x)                                                                       \
  do {                                                                                \
    int r_ = (x);                                                                     \
    if (r_ == -2) return fail(CDB_EINVAL, "unsupported shape in %s", #x);             \
    if (r_ != 0) return fail(CDB_EHIP, "launch failed in %s: %s", #x,                 \
                             hipGetErrorString(hipGetLastError()));                   \
  } while (0)

constexpr size_t kPartialCap = 32u << 20;     // split-K partial tiles (bytes)
constexpr int kDecM = 256;                     // decode GEMM: rows up to this (64-row blocks above 64)
constexpr int kDecSK = 24;                     // decode GEMM: most K splits at 64 rows
constexpr int kDecPartRows = kDecSK * 64;      // split partial buffers hold SK x M <= this many rows

// Decode layers whose O / down projections complete the residual stream and
// hand the next norm's input unscaled (k_gemm_dec_res) need F % 32 == 0 (the
// gate/up kernel takes the scale) and at most kMaxSsParts row-scale
// partials (one per 8 outputs) per row.
bool fused_norm_dims(const cdb_dims& d) {
  return d.hidden % 16 == 0 && d.hidden / 8 <= kMaxSsParts && d.ffn % 32 == 0;
}

bool is_pow2(int x) { return x > 0 && (x & (x - 1)) == 0; }

// Context splits of decode attention: about 256 workgroups in all (one per
// CU).  Each split adds a fixed prologue and a partial to merge, so small
// batches take fewer, longer splits than a multiple of the CU count would
// ask for (measured at context 1024: 256 against 512 workgroups, B = 1
// 1.41 -> 1.35 ms, B = 16 1.91 -> 1.88; 128 was slower at B = 4).
// `target` (at most 256, so the count never exceeds what the workspace was
// sized for) is the workgroup count aimed at.
int attn_splits(int rows_pad, int nh, int target = 256) {
  const int wg = rows_pad * nh;
  int s = (std::min(target, 256) + wg - 1) / wg;
  return std::max(1, std::min(32, s));
}

struct Work {  // carved workspace
  float* resid_b;  void* act;  void* act_f;  void* act2;  float* ss_a;  float* ss_m;  float* qkv;  long qkv_rows;  float* resid_p;  float* inj_p;
  int* tok_seq;  int* tok_pos;
  int* f_n;  int* f_idx;  int* f_slot;  int* f_seq;  int* f_pos;
  int* tok_rows;  int* c_n;  int* c_slot;  int* c_seq;  int* c_pos;  int* c_tok;  int* pos1;
  float* z;  float* partial;  float* part_gu;  float* amax_val;  int* amax_idx;
  int* pf_tiles;  int pf_tiles_cap;
  int* gate_counter;  int* err;  float* attn_part;
  float2* rope;  int rope_rows;       // cos / sin of position x frequency, [rope_rows][head_dim / 2]
  size_t counters_bytes;  char* counters_base;
};

size_t carve(const cdb_dims& d, int max_rows, int max_T, int max_ctx, char* base, Work* w) {
  const size_t el = d.dtype == CDB_BF16 ? 2 : 4;
  const long H = d.hidden, Q = (long)d.n_heads * d.head_dim, F = d.ffn, V = d.vocab;
  // (activation rows rounded up to whole 64-row tiles: the packed layout of
  // the decode GEMM inputs holds 16-row tiles)
  const long maxM = std::max<long>(std::max(max_rows, max_T), ((long)max_rows + 63) / 64 * 64);
  const long ldact = std::max(H, Q);
  const long rows64 = ((long)max_rows + 63) / 64 * 64;
  size_t off = 0;
  auto take = [&](size_t bytes) -> char* {
    off = (off + 255) & ~(size_t)255;
    char* p = base ? base + off : nullptr;
    off += bytes;
    return p;
  };
  Work t{};
  t.resid_b = (float*)take(sizeof(float) * max_rows * H);
  t.act = take(el * maxM * ldact);
  t.act_f = take(el * maxM * F);
  // deferred-norm decode layers (fused residual projections): the MLP input
  // g * x beside the attention output, and the per-8-column sums of x^2
  // that finish the attention and MLP norms
  const bool fusable = fused_norm_dims(d);
  const long frows = std::min<long>(rows64, kDecM);
  t.act2 = take(fusable ? el * frows * H : 0);
  t.ss_a = (float*)take(fusable ? 4L * frows * (H / 8) : 0);
  t.ss_m = (float*)take(fusable ? 4L * frows * (H / 8) : 0);
  t.qkv_rows = std::max<long>(maxM, kDecPartRows);
  t.qkv = (float*)take(sizeof(float) * t.qkv_rows * 3 * Q);
  t.resid_p = (float*)take(sizeof(float) * (long)max_T * H);
  t.inj_p = (float*)take(d.inject ? sizeof(float) * (long)max_T * H : 0);
  t.pf_tiles_cap = max_T / 32 + std::max(max_rows, 1024) + 1;
  t.pf_tiles = (int*)take(8L * t.pf_tiles_cap);
  t.tok_seq = (int*)take(4L * max_T);
  t.tok_pos = (int*)take(4L * max_T);
  t.f_n = (int*)take(4);
  t.f_idx = (int*)take(4L * max_rows);
  t.f_slot = (int*)take(4L * max_rows);
  t.f_seq = (int*)take(4L * max_rows);
  t.f_pos = (int*)take(4L * max_rows);
  t.tok_rows = (int*)take(4L * max_rows);
  t.c_n = (int*)take(4);
  t.c_slot = (int*)take(4L * max_rows);
  t.c_seq = (int*)take(4L * max_rows);
  t.c_pos = (int*)take(4L * max_rows);
  t.c_tok = (int*)take(4L * max_rows);
  t.pos1 = (int*)take(4L * max_rows);
  t.z = (float*)take(4L * std::max(max_rows, 1024));
  t.partial = (float*)take(std::max<size_t>(kPartialCap, sizeof(float) * kDecPartRows * H));
  // split gate/up partials: only where the fused decode gate/up kernel cannot
  // run (F not a multiple of 32, possible in fp32 only)
  t.part_gu = (float*)take(F % 32 ? sizeof(float) * kDecPartRows * 2 * F : 0);
  const long vt = (V + 15) / 16;
  t.amax_val = (float*)take(4L * rows64 * vt);
  t.amax_idx = (int*)take(4L * rows64 * vt);
  long apart = 0;
  for (int r = 1; r <= max_rows; r *= 2) apart = std::max(apart, (long)r * d.n_heads * attn_splits(r, d.n_heads));
  t.attn_part = (float*)take(4L * apart * (d.head_dim + 2));
  t.rope_rows = std::max(max_ctx, 1);
  t.rope = (float2*)take(8L * t.rope_rows * (d.head_dim / 2));
  // the gate's arrival counter (zeroed once at init, self-resetting
  // afterwards) and the descriptor error word
  off = (off + 255) & ~(size_t)255;
  const size_t cstart = off;
  t.gate_counter = (int*)take(64);
  t.err = (int*)take(64);             // descriptor error word (cdb_sync reports and clears it)
  t.counters_base = base ? base + cstart : nullptr;
  t.counters_bytes = off - cstart;
  if (w) *w = t;
  return off + 256;
}

enum { CLS_ATTN, CLS_QKV, CLS_O, CLS_GU, CLS_DOWN, CLS_LMHEAD, CLS_NORM, CLS_GATE, CLS_BOUNDARY,
       CLS_PF_ATTN, CLS_PF_GEMM, CLS_OTHER, NCLS };
const char* kClsNames[NCLS] = {"attn", "gemm_qkv", "gemm_o", "gemm_gu", "gemm_down", "lm_head", "norm", "gate",
                               "boundary", "prefill_attn", "prefill_gemm", "other"};

struct ProfRec { int cls; hipEvent_t a, b; };

struct Ctx {
  bool prof = false;
  bool big_tiles = true;                // 256 x 256 GEMM allowed (CDB_TILE256=0 turns it off)
  bool wide_tiles = true;               // 256 x 128 GEMM allowed (CDB_TILE_WIDE=0 turns it off)
  // decode batches up to these many rows take the fused residual
  // projections for O and down (CDB_FUSE_O_ROWS / CDB_FUSE_DOWN_ROWS)
  // (O: 16; at 32 rows the split O with the deferred residual add measured
  // 2.390 against 2.399 ms per step)
  int fuse_o_rows = 16, fuse_down_rows = 16;
  // larger decode batches up to this many rows add the split projections'
  // partials with the norm deferred to the consumer (CDB_DEFER_NORM_ROWS;
  // measured: B = 48 / 64 / 128 1.5 / 1.1 / 0.4% faster steps, B = 256
  // 0.2% slower)
  int defer_norm_rows = 128;
  // the fused O projection merges split attention partials itself instead
  // of a merge kernel (CDB_FOLD_MERGE=0 turns it off)
  bool fold_merge = true;
  // workgroups the decode attention's context splits aim at (CDB_ATTN_WGS,
  // at most 256)
  int attn_wgs = 256;
  // prefill attention tile rows: 0 = by the chunk's key ranges, 64 / 128
  // forced (CDB_PF_TILE_ROWS); pf_qt is the current chunk's choice
  int pf_tile_rows = 0, pf_qt = 64;
  bool capturing = false;
  std::vector<int> pf_tiles_host[4];   // (first row, rows) pairs; a ring so an
  int pf_ring = 0;                      // upload never reads a buffer being refilled
  int n_pf_tiles = 0;
  std::vector<ProfRec> recs;
  std::vector<hipEvent_t> pool;
  double tot_ms[NCLS] = {};
  long long cnt[NCLS] = {};
  cdb_dims d;
  cdb_weights w;
  std::vector<cdb_layer> pre, core, coda;
  cdb_kv kv;
  cdb_pools pools;
  cdb_seqs seqs;
  hipStream_t st;
  Work ws;
  int Q, el, max_T;
  long core_layer_elems;    // elements of one core layer's K (or V) pool
  int core_planes;
};

hipEvent_t ev_get(Ctx& c) {
  if (!c.pool.empty()) { hipEvent_t e = c.pool.back(); c.pool.pop_back(); return e; }
  hipEvent_t e = nullptr;
  if (hipEventCreate(&e) != hipSuccess) return nullptr;
  return e;
}

// Records a start/stop event pair around one launch while profiling is on.
struct Prof {
  Ctx& c; int cls; hipEvent_t a = nullptr;
  Prof(Ctx& cc, int k) : c(cc), cls(k) {
    if (c.prof && (a = ev_get(c))) (void)hipEventRecord(a, c.st);
  }
  ~Prof() {
    if (!a) return;
    hipEvent_t b = ev_get(c);
    if (!b) { c.pool.push_back(a); return; }
    (void)hipEventRecord(b, c.st);
    c.recs.push_back({cls, a, b});
  }
};

int check_dims(const cdb_dims* d) {
  if (!d) return fail(CDB_EINVAL, "dims is NULL");
  if (d->dtype != CDB_FP32 && d->dtype != CDB_BF16) return fail(CDB_EINVAL, "dtype %d", d->dtype);
  if (d->kv_layout != CDB_KV_DEPTH && d->kv_layout != CDB_KV_SINGLE && d->kv_layout != CDB_KV_FIRST_SHARED &&
      d->kv_layout != CDB_KV_DEPTH_COPY)
    return fail(CDB_EINVAL, "kv_layout %d", d->kv_layout);
  if (d->kv_layout == CDB_KV_FIRST_SHARED && d->r_max < 2)
    return fail(CDB_EINVAL, "first-then-shared KV needs r_max >= 2 (r_max %d)", d->r_max);
  if (d->vocab <= 0 || d->hidden <= 0 || d->n_heads <= 0 || d->ffn <= 0 || d->n_core <= 0)
    return fail(CDB_EINVAL, "non-positive dimension");
  if (d->n_prelude < 0 || d->n_coda < 0) return fail(CDB_EINVAL, "negative layer count");
  if (d->r_max < 1 || d->r_max > 255) return fail(CDB_EINVAL, "r_max %d outside 1..255", d->r_max);
  if (d->gate_kind != CDB_GATE_LINEAR && d->gate_kind != CDB_GATE_CONVERGENCE)
    return fail(CDB_EINVAL, "gate_kind %d", d->gate_kind);
  const int hd = d->head_dim;
  const bool hd_ok = d->dtype == CDB_FP32 ? (hd == 16 || hd == 32 || hd == 64)
                                          : (hd == 16 || hd == 64 || hd == 96 || hd == 128);
  if (!hd_ok) return fail(CDB_EINVAL, "head_dim %d not supported for dtype %d", hd, d->dtype);
  const int kstep = d->dtype == CDB_BF16 ? 32 : 16;
  const int Q = d->n_heads * hd;
  if (d->hidden % kstep || Q % kstep || d->ffn % kstep)
    return fail(CDB_EINVAL, "hidden (%d), heads*head_dim (%d) and ffn (%d) must be multiples of %d",
                d->hidden, Q, d->ffn, kstep);
  if (d->hidden % 16 || d->ffn % 16 || Q % 16 || d->vocab % 16) return fail(CDB_EINVAL, "dimensions must be multiples of 16");
  if (d->hidden > 6144) return fail(CDB_EINVAL, "hidden %d > 6144", d->hidden);
  return CDB_OK;
}

// GEMM tile choice for an M x N x K product.  split_ok: the product may be
// split over K into EPI_PARTIAL partials that the next residual+norm kernel
// reduces (O and down projections); others run unsplit.
void pick_gemm(int dtype, int M, int N, int K, int epi, bool split_ok, int& MW, int& NW, int& SK) {
  const int kstep = dtype == CDB_BF16 ? 32 : 16;
  const bool swi = epi == EPI_SWIGLU;
  MW = M <= 16 ? 1 : (M <= 32 ? 2 : 4);
  if (M <= 64) NW = 1;
  else if (M <= 256) NW = swi ? 1 : 2;
  else NW = swi ? 2 : 4;
  const int m_tiles = (M + 16 * MW - 1) / (16 * MW);
  const int n_tiles = (N + 16 * NW - 1) / (16 * NW);
  const int tiles = m_tiles * n_tiles;
  SK = 1;
  if (split_ok) {
    SK = std::max(1, std::min(8, (512 + tiles - 1) / tiles));
    const int steps = K / kstep;
    while (SK > 1 && steps / SK < 8) SK--;
    while (SK > 1 && (size_t)SK * M * N * 4 > kPartialCap) SK--;
  }
}

// LDS-tiled MFMA kernel for dense-contraction shapes: enough rows that its
// 128 x 128 tile grid alone gives every CU a workgroup, no split over K.
bool use_tiled(int dtype, int epi, int M, int N, int SK) {
  if (SK != 1 || M < 256 || !gemm_tiled_supported(dtype, epi)) return false;
  const int out_bn = epi == EPI_SWIGLU ? 64 : 128;
  return ((M + 127) / 128) * ((N + out_bn - 1) / out_bn) >= 256;
}

// 256 x 256 tiles with 32x32x16 MFMAs (one workgroup per CU): ahead of the
// 128 x 128 kernel on long reductions (K >= 4096) when its grid covers the
// CUs at least twice, so the exposed prologue and epilogue of a workgroup
// are amortised (measured: +21% at 8000 x 5280 x 5280, +6% at
// 8192 x 6144 x 8192; level at K = 2048 for QKV and for the residual-add
// projections, behind for gate/up).  The two kernels produce the same bits.
bool use_big(int epi, int M, int N, int K) {
  const int out_bn = epi == EPI_SWIGLU ? 128 : 256;
  return K >= 4096 && (long)((M + 255) / 256) * ((N + out_bn - 1) / out_bn) >= 512;
}

// 256 x 128 tiles (waves of 128 x 64): ahead of the 128 x 128 kernel on the
// Ouro-like prefill projections at 8192 rows (QKV +10%, gate/up +21%, O
// +15%, down +8%), behind at K = 8192; used below K = 8192 with a grid of at
// least one workgroup per CU (the 256 x 256 kernel, where it applies, comes
// first).  The two kernels produce the same bits.
bool use_wide(int epi, int M, int N, int K) {
  if (epi != EPI_STORE_F32 && epi != EPI_STORE_T && epi != EPI_SWIGLU && epi != EPI_RESID) return false;
  const int out_bn = epi == EPI_SWIGLU ? 64 : 128;
  return K < 8192 && (long)((M + 255) / 256) * ((N + out_bn - 1) / out_bn) >= 256;
}

int gemm(Ctx& c, int cls, int epi, const void* A, int lda, const void* W, int M, int N, int K,
         const int* n_valid, void* C, int ldc, const int* slot, int slot_max, int up_off, int MW, int NW, int SK) {
  GemmArgs g{};
  g.A = A; g.lda = lda; g.W = W; g.M = M; g.N = N; g.K = K;
  g.n_valid = n_valid; g.SK = SK; g.partial = c.ws.partial;
  g.C = C; g.ldc = ldc; g.slot = slot; g.slot_max = slot_max; g.up_off = up_off;
  g.amax_val = c.ws.amax_val; g.amax_idx = c.ws.amax_idx; g.err = c.ws.err;
  Prof pr(c, cls);
  if (use_tiled(c.d.dtype, epi, M, N, SK)) {
    if (c.big_tiles && use_big(epi, M, N, K)) LCHK(gemm_big_launch(epi, g, c.st));
    else if (c.wide_tiles && use_wide(epi, M, N, K)) LCHK(gemm_wide_launch(epi, g, c.st));
    else LCHK(gemm_tiled_launch(epi, g, c.st));
  } else {
    LCHK(gemm_launch(c.d.dtype, epi, MW, NW, g, c.st));
  }
  return CDB_OK;
}

// Decode batches above the weight-streaming kernels' 256 rows (bf16): the
// LDS-tiled MFMA kernel with 128 x 128 tiles, split over K into fp32
// partials until the grid has at least 256 workgroups (one per CU), within
// the partial buffer (rows of SK x M).  Every split owns whole k-tiles of 64.
// Returns 0 when the tiled kernel does not apply.
int tiled_decode_splits(const Ctx& c, int M, int N, int K, long cap_rows) {
  if (c.d.dtype != CDB_BF16 || M <= kDecM) return 0;
  const int tiles = ((M + 127) / 128) * ((N + 127) / 128);
  const int nkt = (K + 63) / 64;
  int sk = 1;
  while (tiles * sk < 256 && sk < nkt && (long)(sk + 1) * M <= cap_rows) sk++;
  const int per = (nkt + sk - 1) / sk;
  return (nkt + per - 1) / per;                  // the splits that own k-tiles
}

int gemm_auto(Ctx& c, int cls, int epi, const void* A, int lda, const void* W, int M, int N, int K,
              const int* n_valid, void* C, int ldc, int up_off) {
  int MW, NW, SK;
  pick_gemm(c.d.dtype, M, N, K, epi, false, MW, NW, SK);
  return gemm(c, cls, epi, A, lda, W, M, N, K, n_valid, C, ldc, nullptr, 0, up_off, MW, NW, 1);
}

// Decode GEMM (M <= kDecM): fp32 split partials [SK][M][N] into `part`.
// Steps per wave from dec_wave_steps; batches per wave raised until the
// split partials fit their buffers (SK x M <= kDecPartRows, SK <= kDecSK).
struct DecPlan { int MW, KW, nb, SK; };

DecPlan dec_plan(int dtype, int M, int N, int K) {
  DecPlan p;
  const int kstep = dtype == CDB_BF16 ? 32 : 16;
  const int nsteps = K / kstep;
  // row tiles per workgroup: 32-row blocks up to 64 rows where the grid of
  // both row blocks stays within 1024 workgroups, so the second block's
  // weight reads meet the first block's in L2 (at 64 rows on the Ouro-like
  // widths each wave then takes more k-steps, so fewer splits and partials:
  // QKV 12.2 -> 11.9 us, O 7.7 -> 7.4, down 12.2 -> 10.7, the step 3.621 ->
  // 3.534 ms; on the Huginn-like widths, grids of 1,100-4,000 workgroups,
  // the core stages took 6.5% longer with them; 16-row blocks at 64 rows
  // 3.618 ms, and 32-row blocks at 128 / 256 rows within 0.5%)
  p.MW = M <= 16 ? 1 : (M <= 32 ? 2 : 4);
  if (M <= 64) {
    const int kw2 = dec_wave_steps(2, M, N, K, dtype);
    const int sk2 = (nsteps + 4 * kw2 - 1) / (4 * kw2);
    if ((long)((N + 63) / 64) * sk2 * ((M + 31) / 32) <= 1024) p.MW = 2;
  }
  p.KW = dec_wave_steps(p.MW, M, N, K, dtype);
  p.nb = 1;
  for (;;) {
    const int per = 4 * p.KW * p.nb;
    p.SK = (nsteps + per - 1) / per;
    if ((long)p.SK * M <= kDecPartRows && p.SK <= kDecSK) break;
    p.nb++;
  }
  return p;
}

int gemm_dec(Ctx& c, int cls, const void* A, int lda, bool a_packed, const void* W, int M, int N, int K,
             const int* n_valid, float* part, int& sk_out) {
  const DecPlan p = dec_plan(c.d.dtype, M, N, K);
  GemmArgs g{};
  g.A = A; g.lda = lda; g.a_packed = a_packed ? 1 : 0; g.W = W; g.M = M; g.N = N; g.K = K; g.n_valid = n_valid;
  g.SK = p.SK; g.dec_batches = p.nb;
  g.partial = part; g.err = c.ws.err;
  sk_out = g.SK;
  Prof pr(c, cls);
  LCHK(gemm_dec_launch(c.d.dtype, EPI_PARTIAL, p.MW, p.KW, g, c.st));
  return CDB_OK;
}

// LDS-tiled GEMM split over K into fp32 partials [SK][M][N] at `part`.
int gemm_tiled_split(Ctx& c, int cls, const void* A, int lda, const void* W, int M, int N, int K,
                     const int* n_valid, float* part, int SK) {
  GemmArgs g{};
  g.A = A; g.lda = lda; g.W = W; g.M = M; g.N = N; g.K = K; g.n_valid = n_valid; g.SK = SK;
  g.partial = part; g.err = c.ws.err;
  Prof pr(c, cls);
  LCHK(gemm_tiled_launch(EPI_PARTIAL, g, c.st));
  return CDB_OK;
}

// What the next norm still has to do: add the split partials of a projection
// to the residual stream (part), or -- after a fused residual projection --
// nothing but the row scale, whose sums of squares are at ss (the GEMM input
// g * x is already in place).
struct Pending {
  const float* part = nullptr;
  int sk = 0, rows = 0;
  const float* ss = nullptr;
  int ss_n = 0;                         // row-scale partials per row at ss
};

// resid[slot] += W x (residual projection): split over K into partials when
// that fills the GPU better; the partials become `pend` for the next norm.
int resid_proj(Ctx& c, int cls, const void* A, int lda, const void* W, int M, int N, int K, const int* n_valid,
               float* resid, int ld_resid, const int* slot, int slot_max, bool allow_split, Pending& pend,
               bool decode = false) {
  const int tsk = decode && allow_split ? tiled_decode_splits(c, M, N, K, (long)(kPartialCap / (4L * N))) : 0;
  if (tsk) {
    int e = gemm_tiled_split(c, cls, A, lda, W, M, N, K, n_valid, c.ws.partial, tsk);
    if (e) return e;
    pend.part = c.ws.partial;
    pend.sk = tsk;
    pend.rows = M;
    return CDB_OK;
  }
  int MW, NW, SK;
  pick_gemm(c.d.dtype, M, N, K, EPI_RESID, allow_split, MW, NW, SK);
  if (SK > 1) {
    int e = gemm(c, cls, EPI_PARTIAL, A, lda, W, M, N, K, n_valid, nullptr, 0, nullptr, 0, 0, MW, NW, SK);
    if (e) return e;
    pend.part = c.ws.partial;
    pend.sk = SK;
    pend.rows = M;
    return CDB_OK;
  }
  pend = Pending();
  return gemm(c, cls, EPI_RESID, A, lda, W, M, N, K, n_valid, resid, ld_resid, slot, slot_max, 0, MW, NW, 1);
}

// Decode residual projection without a K split: resid[slot] += A W^T, and
// with `gain` (the next norm's) the next GEMM input gain * x into `y` plus
// its row-scale partials into `ss` (pend.ss).
// attn (optional): A is instead merged from these split attention partials
struct AttnSplits { const float* part; int ns; int hd; int nh; };

int gemm_res(Ctx& c, int cls, const void* A, const void* W, int M, int N, int K, const int* n_valid, float* resid,
             int ld_resid, const int* slot, int slot_max, const float* gain, void* y, float* ss, Pending& pend,
             const AttnSplits* attn = nullptr) {
  GemmArgs g{};
  g.A = A; g.a_packed = 1; g.W = W; g.M = M; g.N = N; g.K = K; g.n_valid = n_valid; g.SK = 1;
  if (attn) { g.attn_part = attn->part; g.attn_ns = attn->ns; g.attn_hd = attn->hd; g.attn_nh = attn->nh; }
  g.C = resid; g.ldc = ld_resid; g.slot = slot; g.slot_max = slot_max; g.err = c.ws.err;
  g.gain = gain; g.Y = gain ? y : nullptr; g.ss_out = gain ? ss : nullptr;
  const int MW = M <= 16 ? 1 : (M <= 32 ? 2 : 4);
  const int KW = MW == 4 ? 4 : 8;
  Prof pr(c, cls);
  LCHK(gemm_dec_res_launch(c.d.dtype, MW, KW, g, c.st));
  pend = Pending();
  pend.ss = gain ? ss : nullptr;
  pend.ss_n = N / 8;
  return CDB_OK;
}

// residual add of pending partials (+ RMSNorm into act when gain is given,
// fragment-packed for a decode GEMM when `packed`)
int norm_step(Ctx& c, float* resid, int ld, const int* slot, int slot_max, const int* n_valid, int rows,
              const float* gain, Pending& pend, bool packed = false) {
  if (pend.ss) return fail(CDB_ESTATE, "internal: deferred norm left pending");
  if (!gain && !pend.part) return CDB_OK;
  NormArgs na{};
  na.x = resid; na.ldx = ld; na.slot = slot; na.x_rows = slot_max; na.n_valid = n_valid; na.rows = rows;
  na.H = c.d.hidden; na.gain = gain; na.eps = c.d.rms_eps;
  na.out = gain ? c.ws.act : nullptr; na.ldo = std::max(c.d.hidden, c.Q);
  na.part = pend.part; na.part_sk = pend.sk; na.part_rows = pend.rows;
  na.packed = packed ? 1 : 0; na.err = c.ws.err;
  Prof pr(c, CLS_NORM);
  LCHK(norm_launch(c.d.dtype, na, c.st));
  pend = Pending();
  return CDB_OK;
}

// residual add of pending split partials with the next norm deferred: the
// GEMM input gain * x into act (fragment-packed) and its row-scale partials
// into ss (pend.ss), as after a fused residual projection
int resid_defer(Ctx& c, float* resid, int ld, const int* slot, int slot_max, const int* n_valid, int rows,
                const float* gain, float* ss, Pending& pend) {
  NormArgs na{};
  na.x = resid; na.ldx = ld; na.slot = slot; na.x_rows = slot_max; na.n_valid = n_valid; na.rows = rows;
  na.H = c.d.hidden; na.gain = gain; na.eps = c.d.rms_eps;
  na.out = c.ws.act; na.ldo = c.d.hidden; na.packed = 1;
  na.part = pend.part; na.part_sk = pend.sk; na.part_rows = pend.rows; na.err = c.ws.err; na.ss_out = ss;
  Prof pr(c, CLS_NORM);
  LCHK(resid_defer_launch(c.d.dtype, na, c.st));
  pend = Pending();
  pend.ss = ss;
  pend.ss_n = resid_defer_parts(c.d.hidden);
  return CDB_OK;
}

// One transformer block on rows of an fp32 residual stream.
struct LayerRun {
  const cdb_layer* L;
  float* resid; int ld_resid; const int* slot; int slot_max;
  const int* n_valid; int rows;
  const int* seq; const int* pos;
  const int* depth; int depth_uniform;
  void* kbase; void* vbase; int planes;   // layer base [num_blocks][nh][planes][16][hd]
  bool decode;            // true: K/V of each row written by attention (rows are distinct sequences)
  int plane_write;        // prefill: plane index written for all rows
  const float* next_gain; // the next layer's attention-norm gain (NULL: last layer of the run)
};

int run_layer(Ctx& c, const LayerRun& r, Pending& pend) {
  const cdb_dims& d = c.d;
  const int H = d.hidden, Q = c.Q, F = d.ffn;
  const int ldact = std::max(H, Q);
  const bool pf = !r.decode;
  const bool dec = r.rows <= kDecM;             // weight-streaming decode GEMMs
  // decode: the producers write the GEMM inputs fragment-packed (the prefill
  // attention writes row-major, so prefill keeps row-major throughout)
  const bool pk = dec && r.decode;
  // fused residual projections (O, down): small decode batches, where the
  // unsplit GEMM's activation re-reads are cheap and launches dominate
  const bool fuse_o = pk && r.rows <= c.fuse_o_rows;
  const bool fuse_down = pk && r.rows <= c.fuse_down_rows;
  // split O / down with the following norm deferred to its consumer
  const bool defer_o = pk && !fuse_o && r.rows <= c.defer_norm_rows;
  const bool defer_down = pk && !fuse_down && r.rows <= c.defer_norm_rows && r.next_gain;
  const float* ss_attn = pend.ss;     // this layer's QKV input waits for its row scale
  const int ss_attn_n = pend.ss_n;
  pend.ss = nullptr;
  int e = ss_attn ? CDB_OK
                  : norm_step(c, r.resid, r.ld_resid, r.slot, r.slot_max, r.n_valid, r.rows, r.L->attn_norm, pend, pk);
  if (e) return e;
  int qkv_sk = 1;
  const int qkv_tsk = r.decode ? tiled_decode_splits(c, r.rows, 3 * Q, H, c.ws.qkv_rows) : 0;
  if (dec) {
    e = gemm_dec(c, pf ? CLS_PF_GEMM : CLS_QKV, c.ws.act, ldact, pk, r.L->wqkv, r.rows, 3 * Q, H, r.n_valid,
                 c.ws.qkv, qkv_sk);
  } else if (qkv_tsk) {
    e = gemm_tiled_split(c, CLS_QKV, c.ws.act, ldact, r.L->wqkv, r.rows, 3 * Q, H, r.n_valid, c.ws.qkv, qkv_tsk);
    qkv_sk = qkv_tsk;
  } else {
    e = gemm_auto(c, pf ? CLS_PF_GEMM : CLS_QKV, EPI_STORE_F32, c.ws.act, ldact, r.L->wqkv, r.rows, 3 * Q, H,
                  r.n_valid, c.ws.qkv, 3 * Q, 0);
  }
  if (e) return e;
  const int max_pos = c.kv.max_blocks_per_seq * 16;
  if (!r.decode) {
    KvWriteArgs kw{c.ws.qkv, 3 * Q, qkv_sk, r.rows, r.seq, r.pos, r.kbase, r.vbase, r.planes, r.plane_write,
                   c.kv.block_table, c.kv.max_blocks_per_seq, c.kv.num_blocks, c.kv.max_seqs, max_pos,
                   d.n_heads, c.ws.rope};
    Prof pr(c, CLS_PF_ATTN);
    LCHK(kv_write_launch(d.dtype, d.head_dim, kw, c.st));
  }
  if (!r.decode) {
    PrefillAttnArgs pa{};
    pa.qkv = c.ws.qkv; pa.ldq = 3 * Q; pa.qkv_sk = qkv_sk; pa.rows = r.rows;
    pa.seq = r.seq; pa.pos = r.pos;
    pa.tiles = (const int2*)c.ws.pf_tiles; pa.n_tiles = c.n_pf_tiles; pa.tile_rows = c.pf_qt;
    pa.kpool = r.kbase; pa.vpool = r.vbase; pa.planes = r.planes; pa.plane = r.plane_write;
    pa.btab = c.kv.block_table; pa.bt_stride = c.kv.max_blocks_per_seq;
    pa.num_blocks = c.kv.num_blocks; pa.max_seqs = c.kv.max_seqs; pa.max_pos = max_pos;
    pa.nh = d.n_heads; pa.scale = 1.0f / sqrtf((float)d.head_dim); pa.rope = c.ws.rope;
    pa.out = c.ws.act; pa.ldo = ldact;
    Prof pr(c, CLS_PF_ATTN);
    LCHK(attn_prefill_launch(d.dtype, d.head_dim, pa, c.st));
  }
  AttnArgs aa{};
  aa.qkv = c.ws.qkv; aa.ldq = 3 * Q; aa.qkv_sk = qkv_sk; aa.n_valid = r.n_valid; aa.rows = r.rows;
  aa.seq = r.seq; aa.pos = r.pos; aa.depth = r.depth; aa.depth_uniform = r.depth_uniform;
  aa.kpool = r.kbase; aa.vpool = r.vbase; aa.planes = r.planes;
  // explicit last-exited copies: no depth map, every position at the reader's plane
  aa.emap = d.kv_layout == CDB_KV_DEPTH_COPY ? nullptr : c.kv.exit_depth;
  aa.btab = c.kv.block_table; aa.bt_stride = c.kv.max_blocks_per_seq;
  aa.num_blocks = c.kv.num_blocks; aa.max_seqs = c.kv.max_seqs; aa.max_pos = max_pos;
  aa.nh = d.n_heads; aa.scale = 1.0f / sqrtf((float)d.head_dim); aa.rope = c.ws.rope;
  aa.n_split = r.decode ? attn_splits(r.rows, d.n_heads, c.attn_wgs) : 1;
  aa.write_kv = r.decode ? 1 : 0;
  aa.part = c.ws.attn_part;
  aa.out = c.ws.act; aa.ldo = ldact; aa.out_packed = pk ? 1 : 0;
  aa.r_max = r.decode ? d.r_max : 0x7fffffff; aa.err = c.ws.err;
  aa.ss = ss_attn; aa.ss_n = ss_attn_n; aa.ss_h = H; aa.eps = d.rms_eps;
  // the fused O projection takes the split merge when its A pieces fit
  const int vec = d.dtype == 0 ? 4 : 8;
  const bool fold = fuse_o && c.fold_merge && aa.n_split > 1 && aa.n_split <= 16 && r.rows <= 16 &&
                    d.head_dim % vec == 0 && gemm_res_merge_pieces(d.dtype, r.rows, Q) <= kMergePieces;
  if (r.decode) {
    Prof pr(c, CLS_ATTN);
    LCHK(attn_launch(d.dtype, d.head_dim, aa, c.st));
    if (aa.n_split > 1 && !fold) LCHK(attn_merge_launch(d.dtype, d.head_dim, aa, c.st));
  }
  if (fuse_o) {
    const AttnSplits as{c.ws.attn_part, aa.n_split, d.head_dim, d.n_heads};
    e = gemm_res(c, CLS_O, c.ws.act, r.L->wo, r.rows, H, Q, r.n_valid, r.resid, r.ld_resid, r.slot, r.slot_max,
                 r.L->mlp_norm, c.ws.act2, c.ws.ss_m, pend, fold ? &as : nullptr);
  } else if (dec) {
    int sk;
    e = gemm_dec(c, pf ? CLS_PF_GEMM : CLS_O, c.ws.act, ldact, pk, r.L->wo, r.rows, H, Q, r.n_valid, c.ws.partial, sk);
    pend.part = c.ws.partial; pend.sk = sk; pend.rows = r.rows;
  } else {
    e = resid_proj(c, pf ? CLS_PF_GEMM : CLS_O, c.ws.act, ldact, r.L->wo, r.rows, H, Q, r.n_valid, r.resid,
                   r.ld_resid, r.slot, r.slot_max, true, pend, r.decode);
  }
  if (e) return e;
  if (defer_o) {
    e = resid_defer(c, r.resid, r.ld_resid, r.slot, r.slot_max, r.n_valid, r.rows, r.L->mlp_norm, c.ws.ss_m, pend);
    if (e) return e;
  }
  const float* ss_mlp = (fuse_o || defer_o) ? pend.ss : nullptr;   // the MLP input waits for its row scale
  const int ss_mlp_n = pend.ss_n;
  pend.ss = nullptr;
  if (!fuse_o && !defer_o)
    e = norm_step(c, r.resid, r.ld_resid, r.slot, r.slot_max, r.n_valid, r.rows, r.L->mlp_norm, pend, pk);
  if (e) return e;
  if (dec && F % 32 == 0) {
    // gate/up and SwiGLU in one kernel, no K split (activations in and out
    // in the same layout: fragment-packed in the decode core step)
    GemmArgs g{};
    g.A = fuse_o ? c.ws.act2 : c.ws.act; g.lda = ldact; g.a_packed = pk ? 1 : 0; g.W = r.L->wgu; g.M = r.rows;
    g.N = F; g.K = H;
    g.n_valid = r.n_valid; g.up_off = F; g.C = c.ws.act_f; g.ldc = F; g.SK = 1; g.err = c.ws.err;
    g.ss = ss_mlp; g.ss_n = ss_mlp_n; g.ss_h = H; g.eps = d.rms_eps;
    Prof pr(c, pf ? CLS_PF_GEMM : CLS_GU);
    LCHK(gemm_dec_glu_launch(d.dtype, g, c.st));
  } else if (dec) {
    int sk;
    e = gemm_dec(c, pf ? CLS_PF_GEMM : CLS_GU, c.ws.act, ldact, pk, r.L->wgu, r.rows, 2 * F, H, r.n_valid,
                 c.ws.part_gu, sk);
    if (e) return e;
    SwigluArgs sa{c.ws.part_gu, sk, r.rows, F, r.n_valid, c.ws.act_f, F, pk ? 1 : 0};
    Prof pr(c, pf ? CLS_PF_GEMM : CLS_GU);
    LCHK(swiglu_launch(d.dtype, sa, c.st));
  } else {
    e = gemm_auto(c, pf ? CLS_PF_GEMM : CLS_GU, EPI_SWIGLU, c.ws.act, ldact, r.L->wgu, r.rows, F, H, r.n_valid,
                  c.ws.act_f, F, F);
    if (e) return e;
  }
  if (fuse_down) {
    return gemm_res(c, CLS_DOWN, c.ws.act_f, r.L->wd, r.rows, H, F, r.n_valid, r.resid, r.ld_resid, r.slot,
                    r.slot_max, r.next_gain, c.ws.act, c.ws.ss_a, pend);
  }
  if (dec) {
    int sk;
    e = gemm_dec(c, pf ? CLS_PF_GEMM : CLS_DOWN, c.ws.act_f, F, pk, r.L->wd, r.rows, H, F, r.n_valid, c.ws.partial,
                 sk);
    pend.part = c.ws.partial; pend.sk = sk; pend.rows = r.rows;
    if (e || !defer_down) return e;
    return resid_defer(c, r.resid, r.ld_resid, r.slot, r.slot_max, r.n_valid, r.rows, r.next_gain, c.ws.ss_a, pend);
  }
  return resid_proj(c, pf ? CLS_PF_GEMM : CLS_DOWN, c.ws.act_f, F, r.L->wd, r.rows, H, F, r.n_valid, r.resid,
                    r.ld_resid, r.slot, r.slot_max, true, pend, r.decode);
}

size_t bnd_layer_stride(const Ctx& c) {
  return (size_t)c.kv.num_blocks * c.d.n_heads * 16 * c.d.head_dim;
}

void* bnd_pool(const Ctx& c, void* base, int layer) {
  return (char*)base + (size_t)layer * bnd_layer_stride(c) * c.el;
}

// Boundary layers (prelude layers are 0..n_prelude-1, coda layers follow);
// leaves the residual stream complete (pending partials flushed).
int run_bnd_layers(Ctx& c, const std::vector<cdb_layer>& Ls, int layer0, float* resid, const int* n_valid,
                   int rows, const int* seq, const int* pos, bool decode) {
  Pending pend;
  for (size_t i = 0; i < Ls.size(); i++) {
    LayerRun r{};
    r.L = &Ls[i]; r.resid = resid; r.ld_resid = c.d.hidden; r.slot = nullptr; r.slot_max = rows;
    r.n_valid = n_valid; r.rows = rows; r.seq = seq; r.pos = pos; r.depth = nullptr; r.depth_uniform = 1;
    r.kbase = bnd_pool(c, c.kv.bnd_k, layer0 + (int)i); r.vbase = bnd_pool(c, c.kv.bnd_v, layer0 + (int)i);
    r.planes = 1; r.decode = decode; r.plane_write = 0;
    r.next_gain = i + 1 < Ls.size() ? Ls[i + 1].attn_norm : nullptr;
    int e = run_layer(c, r, pend);
    if (e) return e;
  }
  return norm_step(c, resid, c.d.hidden, nullptr, rows, n_valid, rows, nullptr, pend);
}

// Final norm + LM head + greedy argmax for rows of resid_b (n valid rows on the device).
int lm_head_argmax(Ctx& c, const int* n_valid, int rows, float* logits_out) {
  const int H = c.d.hidden, V = c.d.vocab;
  const int ldact = std::max(H, c.Q);
  Pending none;
  // final norm into the fragment-packed layout, then the weight-streaming LM
  // head for any bucket (row blocks of 64 along the grid; blocks past the
  // row count return at once), so the LM head weights stream once per call
  int e = norm_step(c, c.ws.resid_b, H, nullptr, rows, n_valid, rows, c.w.final_norm, none, true);
  if (e) return e;
  // one split: every wave covers H / 4 of the reduction in batches of KW
  GemmArgs g{};
  g.A = c.ws.act; g.lda = ldact; g.a_packed = 1; g.W = c.w.lm_head; g.M = rows; g.N = V; g.K = H;
  g.n_valid = n_valid; g.SK = 1; g.C = logits_out; g.ldc = V;
  g.amax_val = c.ws.amax_val; g.amax_idx = c.ws.amax_idx; g.err = c.ws.err;
  const int MW = rows <= 16 ? 1 : (rows <= 32 ? 2 : 4);
  const int KW = MW == 4 ? 4 : (MW == 2 ? 6 : 8);   // instantiated (MW, KW) pairs
  const int nsteps = H / (c.d.dtype == CDB_BF16 ? 32 : 16);
  g.dec_batches = (nsteps + 4 * KW - 1) / (4 * KW);
  {
    Prof pr(c, CLS_LMHEAD);
    LCHK(gemm_dec_launch(c.d.dtype, EPI_ARGMAX, MW, KW, g, c.st));
  }
  ArgmaxArgs am{c.ws.amax_val, c.ws.amax_idx, (V + 15) / 16, n_valid, rows, c.ws.tok_rows};
  Prof pr(c, CLS_LMHEAD);
  LCHK(argmax_reduce_launch(am, c.st));
  return CDB_OK;
}

// Successor tokens of rows that produced a token: bookkeeping, then prelude.
int produce_and_prelude(Ctx& c, const int* n_rows, int host_rows, int rows_pad, const int* r_slot,
                        const int* r_seq, const int* r_pos, const int* r_depth, int depth_uniform,
                        const int* tok, const cdb_core_desc* core, int* q_n_reset, int* tokens_rows_out) {
  BookArgs b{};
  b.n_rows = n_rows; b.host_rows = host_rows; b.rows_cap = rows_pad; b.r_slot = r_slot; b.r_seq = r_seq; b.r_pos = r_pos;
  b.r_depth = r_depth; b.depth_uniform = depth_uniform; b.tok = tok;
  b.tokens_out = c.seqs.tokens_out; b.exits_out = c.seqs.exits_out; b.n_gen = c.seqs.n_gen;
  b.n_out = c.seqs.n_out; b.max_out = c.seqs.max_out; b.max_seqs = c.kv.max_seqs;
  b.c_n = c.ws.c_n; b.c_slot = c.ws.c_slot; b.c_seq = c.ws.c_seq; b.c_pos = c.ws.c_pos; b.c_tok = c.ws.c_tok;
  if (core) {
    b.d_n = core->n_valid; b.d_slot = core->slot; b.d_seq = core->seq; b.d_pos = core->pos;
    b.d_depth = core->depth; b.d_exit_at = core->exit_at; b.d_cap = core->cap;
  }
  b.r_max = c.d.r_max; b.q_n_reset = q_n_reset; b.tokens_rows_out = tokens_rows_out; b.err = c.ws.err;
  { Prof pr(c, CLS_BOUNDARY); LCHK(book_launch(b, c.st)); }
  const int max_pos = c.kv.max_blocks_per_seq * 16;
  const float* pre_out = nullptr;
  if (c.d.inject || c.d.n_prelude > 0) {
    EmbedTokArgs et{c.ws.c_tok, c.ws.c_n, rows_pad, c.w.embed, c.d.dtype, c.d.hidden, c.d.vocab, c.ws.resid_b,
                    c.d.hidden, c.ws.err};
    LCHK(embed_tok_launch(et, c.st));
    int e = run_bnd_layers(c, c.pre, 0, c.ws.resid_b, c.ws.c_n, rows_pad, c.ws.c_seq, c.ws.c_pos, true);
    if (e) return e;
    pre_out = c.ws.resid_b;
  }
  PreludeEmbedArgs p{};
  p.c_n = c.ws.c_n; p.c_slot = c.ws.c_slot; p.c_seq = c.ws.c_seq; p.c_pos = c.ws.c_pos; p.c_tok = c.ws.c_tok;
  p.rows_pad = rows_pad; p.embed = c.w.embed; p.dtype = c.d.dtype; p.H = c.d.hidden; p.vocab = c.d.vocab;
  p.n_slots = c.pools.n_slots; p.state = c.pools.state; p.pre_out = pre_out;
  p.inject = c.d.inject ? c.pools.inject : nullptr;
  p.emap = c.kv.exit_depth; p.btab = c.kv.block_table; p.bt_stride = c.kv.max_blocks_per_seq; p.r_max = c.d.r_max;
  p.num_blocks = c.kv.num_blocks; p.max_seqs = c.kv.max_seqs; p.max_pos = max_pos; p.err = c.ws.err;
  { Prof pr(c, CLS_BOUNDARY); LCHK(prelude_embed_launch(p, c.st)); }
  return CDB_OK;
}

int check_core(const Ctx& c, const cdb_core_desc* core, int rows_pad) {
  if (!core || !core->n_valid || !core->slot || !core->seq || !core->pos || !core->depth || !core->exit_at)
    return fail(CDB_EINVAL, "core descriptor has a NULL array");
  if (!is_pow2(rows_pad) || rows_pad > c.pools.max_rows || rows_pad > core->cap)
    return fail(CDB_EINVAL, "rows_pad %d must be a power of two <= max_rows %d and <= cap %d", rows_pad,
                c.pools.max_rows, core->cap);
  return CDB_OK;
}

}  // namespace

extern "C" {

const char* cdb_version(void) { return "cdb-mi355x 0.1 (gfx950)"; }

const char* cdb_last_error(void) { return g_err.c_str(); }

const char* cdb_strerror(int code) {
  switch (code) {
    case CDB_OK: return "ok";
    case CDB_EINVAL: return "invalid argument";
    case CDB_EHIP: return "HIP error";
    case CDB_ENOMEM: return "workspace too small";
    case CDB_ESTATE: return "bad state";
  }
  return "unknown error";
}

size_t cdb_workspace_bytes(const cdb_dims* dims, int32_t max_rows, int32_t max_prefill_tokens, int32_t max_context) {
  if (check_dims(dims) != CDB_OK || max_rows <= 0 || max_prefill_tokens <= 0) return 0;
  return carve(*dims, max_rows, max_prefill_tokens, max_context, nullptr, nullptr);
}

}  // extern "C"

namespace {

// Workspace of contexts made by cdb_init_static: a file-scope device array,
// one copy per GPU, held until the process ends.  Host code never uses the
// array's name as an address (in host code it is only a stand-in for the
// symbol): the device address of each GPU's copy comes from
// hipGetSymbolAddress, fetched once per device by the first cdb_init_static
// on it with that device current.
constexpr size_t kStaticScratchBytes = 128u << 20;
static __device__ __align__(256) char scratch[kStaticScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

int init_ctx(const cdb_dims* dims, const cdb_weights* w, const cdb_kv* kv, const cdb_pools* pools,
             const cdb_seqs* seqs, void* stream, void** out, bool static_ws) {
  g_err.clear();
  if (!out) return fail(CDB_EINVAL, "out is NULL");
  *out = nullptr;
  int e = check_dims(dims);
  if (e) return e;
  if (!w || !kv || !pools || !seqs) return fail(CDB_EINVAL, "NULL descriptor");
  const cdb_dims& d = *dims;
  if (!w->embed || !w->final_norm || !w->lm_head || !w->gate_w || (d.n_core && !w->core) ||
      (d.n_prelude && !w->prelude) || (d.n_coda && !w->coda))
    return fail(CDB_EINVAL, "NULL weight pointer");
  auto check_layers = [&](const cdb_layer* L, int n) {
    for (int i = 0; i < n; i++)
      if (!L[i].attn_norm || !L[i].wqkv || !L[i].wo || !L[i].mlp_norm || !L[i].wgu || !L[i].wd) return false;
    return true;
  };
  if (!check_layers(w->core, d.n_core) || !check_layers(w->prelude, d.n_prelude) || !check_layers(w->coda, d.n_coda))
    return fail(CDB_EINVAL, "NULL layer weight pointer");
  if (kv->block_size != 16) return fail(CDB_EINVAL, "block_size must be 16");
  if (kv->num_blocks <= 0 || !kv->core_k || !kv->core_v || !kv->exit_depth || !kv->block_table ||
      kv->max_seqs <= 0 || kv->max_blocks_per_seq <= 0)
    return fail(CDB_EINVAL, "bad KV descriptor");
  if ((d.n_prelude + d.n_coda) > 0 && (!kv->bnd_k || !kv->bnd_v)) return fail(CDB_EINVAL, "boundary KV pools missing");
  if (!pools->state || pools->n_slots <= 0 || (!static_ws && !pools->workspace) || pools->max_rows <= 0 ||
      pools->max_rows > 1024 || !is_pow2(pools->max_rows) || pools->max_prefill_tokens <= 0)
    return fail(CDB_EINVAL, "bad pools descriptor (max_rows must be a power of two in 1..1024)");
  if (static_ws && pools->workspace)
    return fail(CDB_EINVAL, "cdb_init_static takes no workspace (pools->workspace must be NULL)");
  if (d.inject && !pools->inject) return fail(CDB_EINVAL, "inject model needs an injection pool");
  if (d.gate_kind == CDB_GATE_CONVERGENCE && !pools->prev_state)
    return fail(CDB_EINVAL, "the convergence gate needs a previous-state pool");
  if (((uintptr_t)pools->workspace) & 255) return fail(CDB_EINVAL, "workspace must be 256-byte aligned");
  if (pools->max_context < kv->max_blocks_per_seq * 16)
    return fail(CDB_EINVAL, "max_context %d < max_blocks_per_seq * 16 = %d", pools->max_context,
                kv->max_blocks_per_seq * 16);
  const size_t need = carve(d, pools->max_rows, pools->max_prefill_tokens, pools->max_context, nullptr, nullptr);
  char* ws_base = (char*)pools->workspace;
  if (static_ws) {
    if (need > kStaticScratchBytes)
      return fail(CDB_ENOMEM, "cdb_init_static: these maxima need %zu bytes of workspace, more than the library's "
                  "static scratch of %zu bytes; use cdb_init with a caller workspace", need, kStaticScratchBytes);
    int dev = 0;
    HIPCHK(hipGetDevice(&dev));
    if (dev < 0 || dev >= kMaxDevices) return fail(CDB_EINVAL, "device %d beyond %d", dev, kMaxDevices);
    std::lock_guard<std::mutex> lk(g_scratch_mu);
    if (!g_scratch_ptr[dev]) {
      void* p = nullptr;
      HIPCHK(hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)));
      if (!p) return fail(CDB_EHIP, "hipGetSymbolAddress returned NULL for the static scratch");
      g_scratch_ptr[dev] = p;
    }
    ws_base = (char*)g_scratch_ptr[dev];
  } else if (pools->workspace_bytes < need) {
    return fail(CDB_ENOMEM, "workspace %zu bytes < %zu required", pools->workspace_bytes, need);
  }
  if (!seqs->tokens_out || !seqs->exits_out || !seqs->n_gen || !seqs->n_out || seqs->max_out <= 0)
    return fail(CDB_EINVAL, "bad seqs descriptor");
  Ctx* c = new (std::nothrow) Ctx();
  if (!c) return fail(CDB_ENOMEM, "host allocation failed");
  c->d = d;
  {
    const char* v = getenv("CDB_TILE256");
    c->big_tiles = !(v && v[0] == '0');
    if ((v = getenv("CDB_TILE_WIDE"))) c->wide_tiles = v[0] != '0';
    if ((v = getenv("CDB_FUSE_O_ROWS"))) c->fuse_o_rows = atoi(v);
    if ((v = getenv("CDB_FUSE_DOWN_ROWS"))) c->fuse_down_rows = atoi(v);
    if ((v = getenv("CDB_DEFER_NORM_ROWS"))) c->defer_norm_rows = atoi(v);
    if (!fused_norm_dims(d)) c->fuse_o_rows = c->fuse_down_rows = c->defer_norm_rows = 0;
    if ((v = getenv("CDB_FOLD_MERGE"))) c->fold_merge = v[0] != '0';
    if ((v = getenv("CDB_ATTN_WGS"))) c->attn_wgs = std::max(1, std::min(256, atoi(v)));
    if ((v = getenv("CDB_PF_TILE_ROWS"))) c->pf_tile_rows = atoi(v);
  }
  c->w = *w;
  c->pre.assign(w->prelude, w->prelude + d.n_prelude);
  c->core.assign(w->core, w->core + d.n_core);
  c->coda.assign(w->coda, w->coda + d.n_coda);
  c->w.prelude = c->pre.data();
  c->w.core = c->core.data();
  c->w.coda = c->coda.data();
  c->kv = *kv;
  c->pools = *pools;
  c->seqs = *seqs;
  c->st = (hipStream_t)stream;
  c->Q = d.n_heads * d.head_dim;
  c->el = d.dtype == CDB_BF16 ? 2 : 4;
  c->max_T = pools->max_prefill_tokens;
  c->core_planes = (d.kv_layout == CDB_KV_DEPTH || d.kv_layout == CDB_KV_DEPTH_COPY) ? d.r_max
                   : (d.kv_layout == CDB_KV_FIRST_SHARED ? 2 : 1);
  c->core_layer_elems = (long)kv->num_blocks * d.n_heads * c->core_planes * 16 * d.head_dim;
  if (static_ws) {
    c->pools.workspace = ws_base;
    c->pools.workspace_bytes = kStaticScratchBytes;
  }
  carve(d, pools->max_rows, pools->max_prefill_tokens, pools->max_context, ws_base, &c->ws);
  // the static scratch keeps whatever the last context on this GPU left in
  // it: clear the carved region, as a fresh caller workspace would be
  hipError_t he = static_ws ? hipMemsetAsync(ws_base, 0, need, c->st)
                            : hipMemsetAsync(c->ws.counters_base, 0, c->ws.counters_bytes, c->st);
  if (he != hipSuccess) {
    delete c;
    return fail(CDB_EHIP, "hipMemsetAsync: %s", hipGetErrorString(he));
  }
  if (rope_table_launch(c->ws.rope, c->ws.rope_rows, d.head_dim, d.rope_theta, c->st)) {
    delete c;
    return fail(CDB_EHIP, "rope table: %s", hipGetErrorString(hipGetLastError()));
  }
  *out = c;
  return CDB_OK;
}

}  // namespace

extern "C" {

int cdb_init(const cdb_dims* dims, const cdb_weights* w, const cdb_kv* kv, const cdb_pools* pools,
             const cdb_seqs* seqs, void* stream, void** out) {
  return init_ctx(dims, w, kv, pools, seqs, stream, out, false);
}

int cdb_init_static(const cdb_dims* dims, const cdb_weights* w, const cdb_kv* kv, const cdb_pools* pools,
                    const cdb_seqs* seqs, void* stream, void** out) {
  return init_ctx(dims, w, kv, pools, seqs, stream, out, true);
}

int cdb_pack_weight(int32_t dtype, const void* src, void* dst, int32_t rows, int32_t cols, void* stream) {
  if (dtype != CDB_FP32 && dtype != CDB_BF16) return fail(CDB_EINVAL, "bad dtype %d", dtype);
  if (!src || !dst) return fail(CDB_EINVAL, "NULL matrix pointer");
  const int ks = dtype == CDB_BF16 ? 32 : 16;
  if (rows <= 0 || cols <= 0 || rows % 16 || cols % ks)
    return fail(CDB_EINVAL, "matrix [%d][%d]: rows must be a multiple of 16 and cols of %d", rows, cols, ks);
  const size_t bytes = (size_t)rows * cols * (dtype == CDB_BF16 ? 2 : 4);
  if ((const char*)src < (const char*)dst + bytes && (const char*)dst < (const char*)src + bytes)
    return fail(CDB_EINVAL, "source and destination overlap");
  if (pack_weight_launch(dtype, src, dst, rows, cols, (hipStream_t)stream))
    return fail(CDB_EHIP, "pack launch: %s", hipGetErrorString(hipGetLastError()));
  return CDB_OK;
}

int cdb_core_step(void* ctx, const cdb_core_desc* core, int32_t rows_pad) {
  if (!ctx) return fail(CDB_ESTATE, "NULL context");
  Ctx& c = *(Ctx*)ctx;
  int e = check_core(c, core, rows_pad);
  if (e) return e;
  if (c.d.gate_kind == CDB_GATE_CONVERGENCE) {    // h_{d-1} for the convergence gate
    AddRowsArgs sv{c.pools.prev_state, c.pools.state, c.d.hidden, core->slot, core->n_valid, rows_pad,
                   c.pools.n_slots, c.ws.err};
    LCHK(save_rows_launch(sv, c.st));
  }
  if (c.d.inject) {
    AddRowsArgs ar{c.pools.state, c.pools.inject, c.d.hidden, core->slot, core->n_valid, rows_pad, c.pools.n_slots,
                   c.ws.err};
    LCHK(add_rows_launch(ar, c.st));
  }
  const size_t layer_bytes = (size_t)c.core_layer_elems * c.el;
  Pending pend;
  for (int l = 0; l < c.d.n_core; l++) {
    LayerRun r{};
    r.L = &c.core[l];
    r.resid = c.pools.state; r.ld_resid = c.d.hidden; r.slot = core->slot; r.slot_max = c.pools.n_slots;
    r.n_valid = core->n_valid; r.rows = rows_pad; r.seq = core->seq; r.pos = core->pos;
    r.depth = core->depth; r.depth_uniform = 1;
    r.kbase = (char*)c.kv.core_k + (size_t)l * layer_bytes;
    r.vbase = (char*)c.kv.core_v + (size_t)l * layer_bytes;
    r.planes = c.core_planes;
    r.decode = true;
    r.next_gain = l + 1 < c.d.n_core ? c.core[l + 1].attn_norm : nullptr;
    e = run_layer(c, r, pend);
    if (e) return e;
  }
  return norm_step(c, c.pools.state, c.d.hidden, core->slot, c.pools.n_slots, core->n_valid, rows_pad, nullptr, pend);
}

int cdb_gate_compact(void* ctx, const cdb_core_desc* core, int32_t rows_pad, int32_t gate_enabled,
                     cdb_exit_queue* exits, const cdb_compact_out* out) {
  if (!ctx) return fail(CDB_ESTATE, "NULL context");
  Ctx& c = *(Ctx*)ctx;
  int e = check_core(c, core, rows_pad);
  if (e) return e;
  if (!exits || !exits->n || !exits->slot || !exits->seq || !exits->pos || !exits->depth || exits->cap < rows_pad)
    return fail(CDB_EINVAL, "bad exit queue (cap must be >= rows_pad)");
  if (!out || !out->counts || !out->fired_seq) return fail(CDB_EINVAL, "bad compact outputs");
  GateArgs g{};
  g.state = c.pools.state; g.H = c.d.hidden; g.n_slots = c.pools.n_slots;
  g.gate_w = c.w.gate_w; g.bias = c.d.gate_bias; g.threshold = c.d.gate_threshold; g.eps = c.d.rms_eps;
  g.kind = c.d.gate_kind; g.prev = c.pools.prev_state; g.tau = c.d.conv_threshold;
  g.gate_enabled = gate_enabled; g.n_valid = core->n_valid;
  g.slot = core->slot; g.seq = core->seq; g.pos = core->pos; g.depth = core->depth; g.exit_at = core->exit_at;
  g.rows_pad = rows_pad; g.z = c.ws.z; g.counter = c.ws.gate_counter;
  g.q_n = exits->n; g.q_slot = exits->slot; g.q_seq = exits->seq; g.q_pos = exits->pos; g.q_depth = exits->depth;
  g.q_cap = exits->cap; g.counts = out->counts; g.fired_seq = out->fired_seq; g.err = c.ws.err;
  { Prof pr(c, CLS_GATE); LCHK(gate_compact_launch(g, c.st)); }
  if (out->host_counts) HIPCHK(hipMemcpyAsync(out->host_counts, out->counts, 4 * sizeof(int), hipMemcpyDeviceToHost, c.st));
  if (out->host_fired)
    HIPCHK(hipMemcpyAsync(out->host_fired, out->fired_seq, rows_pad * sizeof(int), hipMemcpyDeviceToHost, c.st));
  if (out->event) HIPCHK(hipEventRecord((hipEvent_t)out->event, c.st));
  return CDB_OK;
}

int cdb_boundary(void* ctx, cdb_exit_queue* exits, const cdb_core_desc* core, const cdb_boundary_desc* bd) {
  if (!ctx) return fail(CDB_ESTATE, "NULL context");
  Ctx& c = *(Ctx*)ctx;
  if (!bd || !is_pow2(bd->rows_pad) || bd->rows_pad > c.pools.max_rows)
    return fail(CDB_EINVAL, "boundary rows_pad must be a power of two <= max_rows");
  if (!exits || !exits->n || exits->cap < bd->rows_pad) return fail(CDB_EINVAL, "bad exit queue");
  if (!core || !core->n_valid) return fail(CDB_EINVAL, "bad core descriptor");
  const int rows = bd->rows_pad;
  const int max_pos = c.kv.max_blocks_per_seq * 16;
  CodaPrepArgs cp{exits->n, exits->slot, exits->seq, exits->pos, exits->depth, rows, c.pools.state, c.d.hidden,
                  c.pools.n_slots, c.ws.resid_b, bd->exit_states_out, c.ws.pos1, c.kv.exit_depth,
                  c.kv.block_table, c.kv.max_blocks_per_seq, c.kv.num_blocks, c.kv.max_seqs, max_pos, c.ws.err};
  { Prof pr(c, CLS_BOUNDARY); LCHK(coda_prep_launch(cp, c.st)); }
  if (c.d.kv_layout == CDB_KV_DEPTH_COPY && c.d.n_core > 0 && c.core_planes > 1) {
    // the last-exited copy: planes above each exit depth get the last loop's K/V
    KvExitCopyArgs kc{exits->n, exits->seq, exits->pos, exits->depth, rows, c.kv.core_k, c.kv.core_v,
                      c.core_layer_elems, c.d.n_core, c.core_planes, c.d.n_heads, c.d.head_dim, (int)c.el,
                      c.kv.block_table, c.kv.max_blocks_per_seq, c.kv.num_blocks, c.kv.max_seqs, max_pos, c.ws.err};
    Prof pr(c, CLS_BOUNDARY);
    LCHK(kv_exit_copy_launch(kc, c.st));
  }
  int e = run_bnd_layers(c, c.coda, c.d.n_prelude, c.ws.resid_b, exits->n, rows, exits->seq, exits->pos, true);
  if (e) return e;
  e = lm_head_argmax(c, exits->n, rows, bd->logits_out);
  if (e) return e;
  return produce_and_prelude(c, exits->n, 0, rows, exits->slot, exits->seq, exits->pos, exits->depth, 0,
                             c.ws.tok_rows, core, exits->n, bd->tokens_out_rows);
}

int cdb_prefill(void* ctx, const cdb_prefill_desc* pd, const cdb_core_desc* core) {
  if (!ctx) return fail(CDB_ESTATE, "NULL context");
  Ctx& c = *(Ctx*)ctx;
  if (!pd || pd->n_seqs <= 0 || pd->n_tokens <= 0 || pd->n_tokens > c.max_T || !pd->tokens || !pd->cu_seqlens ||
      !pd->seq || !pd->start_pos || !pd->slot || !pd->is_final || !pd->host_cu_seqlens || !pd->host_start_pos ||
      !pd->host_is_final)
    return fail(CDB_EINVAL, "bad prefill descriptor");
  if (!core || !core->n_valid) return fail(CDB_EINVAL, "bad core descriptor");
  const int* hcu = pd->host_cu_seqlens;
  if (hcu[0] != 0 || hcu[pd->n_seqs] != pd->n_tokens) return fail(CDB_EINVAL, "cu_seqlens must run 0..n_tokens");
  int n_final = 0;
  for (int i = 0; i < pd->n_seqs; i++) {
    if (hcu[i + 1] <= hcu[i]) return fail(CDB_EINVAL, "empty sequence %d in prefill chunk", i);
    n_final += pd->host_is_final[i] ? 1 : 0;
  }
  if (n_final > c.pools.max_rows) return fail(CDB_EINVAL, "%d final prompts > max_rows", n_final);
  const int T = pd->n_tokens, H = c.d.hidden, R = c.d.r_max;
  const int max_pos = c.kv.max_blocks_per_seq * 16;
  // query tiles of up to qt consecutive tokens of one sequence, the longest
  // key ranges first: a causal tile's cost grows with its last position, and
  // starting the heavy tiles early keeps them out of the launch's tail
  double key_sum = 0.0;                           // mean key range of the chunk's 64-row tiles
  long n64 = 0, n128 = 0;
  for (int i = 0; i < pd->n_seqs; i++) {
    for (int r = hcu[i]; r < hcu[i + 1]; r += 64, n64++)
      key_sum += pd->host_start_pos[i] + (r - hcu[i]) + std::min(64, hcu[i + 1] - r);
    n128 += (hcu[i + 1] - hcu[i] + 127) / 128;
  }
  const int qt = attn_prefill_tile_rows(c.d.dtype, c.d.head_dim, n64 ? key_sum / n64 : 0.0, n128 * c.d.n_heads,
                                        c.pf_tile_rows);
  c.pf_qt = qt;
  std::vector<int>& tl = c.pf_tiles_host[c.pf_ring];
  c.pf_ring = (c.pf_ring + 1) & 3;
  tl.clear();
  std::vector<std::array<int, 3>> order;          // (last position, first row, rows)
  for (int i = 0; i < pd->n_seqs; i++)
    for (int r = hcu[i]; r < hcu[i + 1]; r += qt) {
      const int n = std::min(qt, hcu[i + 1] - r);
      order.push_back({pd->host_start_pos[i] + (r - hcu[i]) + n - 1, r, n});
    }
  std::stable_sort(order.begin(), order.end(), [](const std::array<int, 3>& x, const std::array<int, 3>& y) {
    return x[0] > y[0];
  });
  for (const auto& o : order) {
    tl.push_back(o[1]);
    tl.push_back(o[2]);
  }
  c.n_pf_tiles = (int)tl.size() / 2;
  if (c.n_pf_tiles > c.ws.pf_tiles_cap) return fail(CDB_EINVAL, "too many prefill tiles");
  HIPCHK(hipMemcpyAsync(c.ws.pf_tiles, tl.data(), sizeof(int) * tl.size(), hipMemcpyHostToDevice, c.st));
  PrefillSetupArgs ps{};
  ps.tokens = pd->tokens; ps.cu = pd->cu_seqlens; ps.seq = pd->seq; ps.start_pos = pd->start_pos;
  ps.is_final = pd->is_final; ps.n_seqs = pd->n_seqs; ps.n_tokens = T;
  ps.tok_seq = c.ws.tok_seq; ps.tok_pos = c.ws.tok_pos;
  ps.embed = c.w.embed; ps.dtype = c.d.dtype; ps.H = H; ps.vocab = c.d.vocab; ps.resid = c.ws.resid_p;
  ps.emap = c.kv.exit_depth; ps.btab = c.kv.block_table; ps.bt_stride = c.kv.max_blocks_per_seq; ps.r_max = R;
  ps.num_blocks = c.kv.num_blocks; ps.max_seqs = c.kv.max_seqs; ps.max_pos = max_pos; ps.slot = pd->slot;
  ps.f_n = c.ws.f_n; ps.f_idx = c.ws.f_idx; ps.f_slot = c.ws.f_slot; ps.f_seq = c.ws.f_seq; ps.f_pos = c.ws.f_pos;
  ps.err = c.ws.err;
  LCHK(prefill_setup_launch(ps, c.st));
  int e = run_bnd_layers(c, c.pre, 0, c.ws.resid_p, nullptr, T, c.ws.tok_seq, c.ws.tok_pos, false);
  if (e) return e;
  if (c.d.inject) {
    HIPCHK(hipMemcpyAsync(c.ws.inj_p, c.ws.resid_p, sizeof(float) * (size_t)T * H, hipMemcpyDeviceToDevice, c.st));
    HIPCHK(hipMemsetAsync(c.ws.resid_p, 0, sizeof(float) * (size_t)T * H, c.st));
  }
  const size_t layer_bytes = (size_t)c.core_layer_elems * c.el;
  Pending pend;
  for (int depth = 1; depth <= R; depth++) {
    if (c.d.inject) {
      e = norm_step(c, c.ws.resid_p, H, nullptr, T, nullptr, T, nullptr, pend);
      if (e) return e;
      AddRowsArgs ar{c.ws.resid_p, c.ws.inj_p, H, nullptr, nullptr, T, T, c.ws.err};
      LCHK(add_rows_launch(ar, c.st));
    }
    for (int l = 0; l < c.d.n_core; l++) {
      LayerRun r{};
      r.L = &c.core[l];
      r.resid = c.ws.resid_p; r.ld_resid = H; r.slot = nullptr; r.slot_max = T;
      r.n_valid = nullptr; r.rows = T; r.seq = c.ws.tok_seq; r.pos = c.ws.tok_pos;
      r.depth = nullptr; r.depth_uniform = depth;
      r.kbase = (char*)c.kv.core_k + (size_t)l * layer_bytes;
      r.vbase = (char*)c.kv.core_v + (size_t)l * layer_bytes;
      r.planes = c.core_planes;
      r.decode = false; r.plane_write = std::min(depth, c.core_planes) - 1;
      e = run_layer(c, r, pend);
      if (e) return e;
    }
  }
  e = norm_step(c, c.ws.resid_p, H, nullptr, T, nullptr, T, nullptr, pend);
  if (e) return e;
  e = run_bnd_layers(c, c.coda, c.d.n_prelude, c.ws.resid_p, nullptr, T, c.ws.tok_seq, c.ws.tok_pos, false);
  if (e) return e;
  if (n_final == 0) return CDB_OK;
  int rows = 1;
  while (rows < n_final) rows *= 2;
  GatherRowsArgs gr{c.ws.resid_p, H, c.ws.f_idx, c.ws.f_n, rows, H, T, c.ws.resid_b, H, c.ws.err};
  LCHK(gather_rows_launch(gr, c.st));
  e = lm_head_argmax(c, c.ws.f_n, rows, pd->logits_out);
  if (e) return e;
  return produce_and_prelude(c, c.ws.f_n, 0, rows, c.ws.f_slot, c.ws.f_seq, c.ws.f_pos, nullptr, R, c.ws.tok_rows,
                             core, nullptr, nullptr);
}

int cdb_profile(void* ctx, int32_t enable) {
  if (!ctx) return fail(CDB_ESTATE, "NULL context");
  Ctx& c = *(Ctx*)ctx;
  if (enable) {
    for (int i = 0; i < NCLS; i++) { c.tot_ms[i] = 0; c.cnt[i] = 0; }
  }
  c.prof = enable != 0;
  return CDB_OK;
}

int cdb_profile_read(void* ctx, const char* cls, double* total_ms, int64_t* launches) {
  if (!ctx) return fail(CDB_ESTATE, "NULL context");
  Ctx& c = *(Ctx*)ctx;
  int k = -1;
  for (int i = 0; i < NCLS; i++)
    if (cls && strcmp(cls, kClsNames[i]) == 0) k = i;
  if (k < 0) return fail(CDB_EINVAL, "unknown kernel class '%s'", cls ? cls : "(null)");
  HIPCHK(hipStreamSynchronize(c.st));
  for (const ProfRec& r : c.recs) {
    float ms = 0.f;
    HIPCHK(hipEventElapsedTime(&ms, r.a, r.b));
    c.tot_ms[r.cls] += ms;
    c.cnt[r.cls] += 1;
    c.pool.push_back(r.a);
    c.pool.push_back(r.b);
  }
  c.recs.clear();
  if (total_ms) *total_ms = c.tot_ms[k];
  if (launches) *launches = c.cnt[k];
  return CDB_OK;
}

int cdb_graph_begin(void* ctx) {
  if (!ctx) return fail(CDB_ESTATE, "NULL context");
  Ctx& c = *(Ctx*)ctx;
  if (c.capturing) return fail(CDB_ESTATE, "already capturing");
  if (c.prof) return fail(CDB_ESTATE, "profiling is on; turn it off before capturing");
  HIPCHK(hipStreamBeginCapture(c.st, hipStreamCaptureModeRelaxed));
  c.capturing = true;
  return CDB_OK;
}

int cdb_graph_end(void* ctx, void** graph) {
  if (!ctx || !graph) return fail(CDB_EINVAL, "NULL argument");
  Ctx& c = *(Ctx*)ctx;
  *graph = nullptr;
  if (!c.capturing) return fail(CDB_ESTATE, "not capturing");
  c.capturing = false;
  hipGraph_t g = nullptr;
  HIPCHK(hipStreamEndCapture(c.st, &g));
  hipGraphExec_t ge = nullptr;
  hipError_t e = hipGraphInstantiate(&ge, g, nullptr, nullptr, 0);
  (void)hipGraphDestroy(g);
  if (e != hipSuccess) return fail(CDB_EHIP, "hipGraphInstantiate: %s", hipGetErrorString(e));
  *graph = ge;
  return CDB_OK;
}

int cdb_graph_launch(void* ctx, void* graph) {
  if (!ctx || !graph) return fail(CDB_EINVAL, "NULL argument");
  Ctx& c = *(Ctx*)ctx;
  HIPCHK(hipGraphLaunch((hipGraphExec_t)graph, c.st));
  return CDB_OK;
}

void cdb_graph_destroy(void* graph) {
  if (graph) (void)hipGraphExecDestroy((hipGraphExec_t)graph);
}

int cdb_sync(void* ctx) {
  if (!ctx) return fail(CDB_ESTATE, "NULL context");
  Ctx& c = *(Ctx*)ctx;
  if (c.capturing) return fail(CDB_ESTATE, "cdb_sync while capturing a graph");
  int err = 0;
  HIPCHK(hipMemcpyAsync(&err, c.ws.err, sizeof(int), hipMemcpyDeviceToHost, c.st));
  HIPCHK(hipStreamSynchronize(c.st));
  if (err) {
    HIPCHK(hipMemsetAsync(c.ws.err, 0, sizeof(int), c.st));
    HIPCHK(hipStreamSynchronize(c.st));
    std::string what;
    const char* names[] = {"slot", "sequence id", "position", "depth outside [1, r_max]", "block id", "token id",
                           "row count beyond the launch rows or a queue's capacity"};
    for (int i = 0; i < 7; i++)
      if (err & (1 << i)) what += std::string(what.empty() ? "" : ", ") + names[i];
    return fail(CDB_EINVAL, "a kernel clamped an out-of-range descriptor value (%s); results of the affected rows "
                "since the previous cdb_sync are not valid", what.c_str());
  }
  return CDB_OK;
}

void cdb_destroy(void* ctx) {
  if (!ctx) return;
  Ctx* c = (Ctx*)ctx;
  for (const ProfRec& r : c->recs) { (void)hipEventDestroy(r.a); (void)hipEventDestroy(r.b); }
  for (hipEvent_t e : c->pool) (void)hipEventDestroy(e);
  delete c;
}

}  // extern "C"
