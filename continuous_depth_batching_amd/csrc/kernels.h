// Internal launch interface of the CDB kernels (not part of the C ABI).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace cdb {

enum { EPI_STORE_F32 = 0, EPI_STORE_T = 1, EPI_RESID = 2, EPI_SWIGLU = 3, EPI_ARGMAX = 4, EPI_PARTIAL = 5 };

struct GemmArgs {
  const void* A; int lda;        // T [M][lda]
  const void* W;                 // T [N (+up rows)][K], fragment-packed (tiles of 16 x KSTEP)
  int M, N, K;                   // M = launch rows (bucket), N outputs, K reduction
  const int* n_valid;            // rows >= *n_valid skipped (NULL: all M)
  int SK;                        // workgroups splitting K
  int dec_batches;               // decode GEMM: batches of KW k-steps per wave (>= 1)
  int a_packed;                  // decode GEMM: A fragment-packed (apack_off) instead of row-major
  int m_tiles;                   // set by gemm_launch
  float* partial;                // EPI_PARTIAL: [SK][M][N] fp32 split partials
  void* C; int ldc;              // output (fp32 / T / residual base)
  const int* slot;               // EPI_RESID: row -> residual row (NULL: identity)
  int slot_max;                  // residual rows available (clamp for slot[])
  int up_off;                    // EPI_SWIGLU: row offset of the up rows in W
  float* amax_val; int* amax_idx;// EPI_ARGMAX per-(row, N-tile) partials
  int* err;                      // descriptor error word (EPI_RESID slots)
  // residual projection with the next norm's statistics (k_gemm_dec_res):
  // C is the fp32 residual stream, Y receives gain * x fragment-packed
  // ([M][N]), ss_out the per-8-column sums of x^2 ([M][N / 8]); no Y or
  // ss_out when gain is NULL
  const float* gain; void* Y; float* ss_out;
  // consumer side (gate/up): the rows of A still lack their RMSNorm scale,
  // 1 / sqrt(sum_k ss[m][k] / ss_h + eps) over ss_n partials (NULL: scale 1)
  const float* ss; int ss_n; int ss_h; float eps;
  // residual projection whose A is the merge of split attention partials
  // ([M * attn_nh][attn_ns][attn_hd + 2]: max, sum, output of each split;
  // K = attn_nh * attn_hd); NULL: A is read from g.A
  const float* attn_part; int attn_ns; int attn_hd; int attn_nh;
};

// dtype 0 = fp32, 1 = bf16.  Returns 0, -1 on launch failure, -2 on an
// unsupported tile shape.
int gemm_launch(int dtype, int epi, int MW, int NW, GemmArgs g, hipStream_t st);
// row-major [rows][cols] -> fragment-packed (rows % 16 == 0, cols % KSTEP == 0)
int pack_weight_launch(int dtype, const void* src, void* dst, int rows, int cols, hipStream_t st);

// Decode GEMM (M <= 64), EPI_PARTIAL or EPI_ARGMAX; grid = ceil(N/64) * SK.
// LDS-tiled MFMA GEMM (bf16, many rows; EPI_STORE_F32 / STORE_T / RESID / SWIGLU),
// 128 x 128 output tiles.  K % 32 == 0.
bool gemm_tiled_supported(int dtype, int epi);
int gemm_tiled_launch(int epi, const GemmArgs& g, hipStream_t st);
// 256 x 256 tiles of 128 x 128 waves with 32x32x16 MFMAs; same epilogues and limits.
int gemm_big_launch(int epi, const GemmArgs& g, hipStream_t st);
// 256 x 128 tiles of 128 x 64 waves with 16x16x32 MFMAs (EPI_STORE_F32 /
// STORE_T / RESID / SWIGLU, no split); the same bits as the 128 x 128 kernel.
int gemm_wide_launch(int epi, const GemmArgs& g, hipStream_t st);

// Decode GEMM (M <= 256): MW row tiles of 16 per workgroup (row blocks of
// 16 * MW rows along the grid's y; MW = 1 up to 16 rows, 2 up to 64, 4 up to
// 256), KW k-steps per wave batch,
// g.SK == ceil(K / KSTEP / (4 * KW * g.dec_batches)).
int gemm_dec_launch(int dtype, int epi, int MW, int KW, const GemmArgs& g, hipStream_t st);
int dec_wave_steps(int MW, int M, int N, int K, int dtype);
// Decode gate/up projection with SwiGLU, no K split (M <= 256): g.W holds the
// gate rows [0, N) and the up rows [g.up_off, g.up_off + N), g.N = F outputs
// (F % 32 == 0), g.C = silu(gate) * up as T; A and C are both
// fragment-packed when g.a_packed, else row-major (g.lda, g.ldc).
int gemm_dec_glu_launch(int dtype, const GemmArgs& g, hipStream_t st);
// Decode residual projection, no K split (M <= 256, N % 16 == 0): for 8
// outputs per workgroup, C[slot(m)][n] += (A W^T)[m][n]; then, with g.gain,
// Y = gain * x fragment-packed and ss_out[m][n / 8] = sum of x^2 over the
// workgroup's 8 outputs (the next norm without its row scale).
// With g.attn_part (M <= 16, MW 1, KW 8, 2..16 splits) A is merged from the
// attention's split partials in the kernel instead (no merge kernel).
int gemm_dec_res_launch(int dtype, int MW, int KW, const GemmArgs& g, hipStream_t st);
// A pieces one wave merges for that form (at most kMergePieces: one per lane)
int gemm_res_merge_pieces(int dtype, int M, int K);
constexpr int kMergePieces = 64;
// the largest row-scale partial count a consumer takes (ss_n)
constexpr int kMaxSsParts = 256;

struct SwigluArgs {
  const float* part; int sk; int rows; int F;   // partials [sk][rows][2F]
  const int* n_valid;
  void* out; int ldo;                            // T [rows][ldo]
  int packed;                                    // out fragment-packed ([rows][F], apack_off)
};
int swiglu_launch(int dtype, const SwigluArgs& a, hipStream_t st);

struct ArgmaxArgs {
  const float* val; const int* idx; int n_tiles;
  const int* n_valid; int rows;
  int* tok_out;
};
int argmax_reduce_launch(const ArgmaxArgs& a, hipStream_t st);

// Residual add + RMSNorm: x = resid[slot] + sum_s part[s][row] (when part
// is given; x is written back), then out = g * x / sqrt(mean(x^2) + eps)
// (when out is given).
struct NormArgs {
  float* x; int ldx;             // fp32 rows (through slot when given)
  const int* slot; int x_rows;   // slot NULL: identity; x_rows clamps slot[]
  const int* n_valid; int rows;  // rows >= *n_valid are written as zeros
  int H;
  const float* gain;             // [H]
  float eps;
  void* out; int ldo;            // T [rows][ldo] or NULL
  const float* part; int part_sk; int part_rows; // split partials [sk][part_rows][H] or NULL
  int packed;                    // out fragment-packed ([rows][H], apack_off)
  int* err;                      // descriptor error word
  float* ss_out;                 // resid_defer_launch: sums of x^2 per 256 columns [rows][resid_defer_parts(H)]
};
int norm_launch(int dtype, const NormArgs& a, hipStream_t st);
// Residual add of split partials with the RMSNorm deferred to the consumer:
// x = x + the splits (in split order), out = gain * x fragment-packed and
// ss_out[m][c] = sum of x^2 over columns 256c .. 256c + 255; the consumer
// (the gate/up kernel with a row scale, the decode attention) forms
// 1 / rms(x) from the resid_defer_parts(H) sums.  Rows >= *n_valid get
// zeros.  Needs gain, out, ss_out, packed, H % 32 == 0, H <= 4096 and
// part_sk <= 24.
int resid_defer_launch(int dtype, const NormArgs& a, hipStream_t st);
inline int resid_defer_parts(int H) { return (H + 255) / 256; }

struct AttnArgs {
  const float* qkv; int ldq;     // fp32 [qkv_sk][rows][3Q] split partials of the projections (pre-rotary)
  int qkv_sk;                    // number of splits summed on load
  const int* n_valid; int rows;
  const int* seq; const int* pos;
  const int* depth; int depth_uniform;  // per-row loop step (NULL: uniform)
  void* kpool; void* vpool;      // this layer's base: [num_blocks][nh][planes][16][hd]
  int planes;                    // r_max (depth-indexed) or 1
  const uint8_t* emap;           // [num_blocks][16]; NULL: every earlier position at the reader's plane
  const int* btab; int bt_stride;
  int num_blocks, max_seqs, max_pos;   // clamps for indices read from device memory
  int nh; float scale;
  const float2* rope;            // [max_pos][head_dim / 2] cos / sin of the rotary angles
  int n_split;
  int write_kv;                  // 1: rotate and store this row's K/V, attend to it from registers
  float* part;                   // split partials [rows*nh][n_split][hd+2] (n_split > 1)
  void* out; int ldo;            // T [rows][ldo] (n_split == 1)
  int out_packed;                // out fragment-packed ([rows][nh * hd], apack_off)
  int r_max;                     // loop steps: depth outside [1, r_max] is a descriptor error
  int* err;                      // descriptor error word
  // rows of qkv still lacking their RMSNorm scale: q, k and v of row b are
  // multiplied by 1 / sqrt(sum_k ss[b][k] / ss_h + eps) (NULL: scale 1)
  const float* ss; int ss_n; int ss_h; float eps;
};
int attn_launch(int dtype, int head_dim, const AttnArgs& a, hipStream_t st);
// merges the n_split partials of each (row, head) in split order
int attn_merge_launch(int dtype, int head_dim, const AttnArgs& a, hipStream_t st);

struct PrefillAttnArgs {         // tiled causal attention over one plane (prefill)
  const float* qkv; int ldq; int qkv_sk; int rows;
  const int* seq; const int* pos;  // per row
  const int2* tiles; int n_tiles;  // (first row, rows <= tile_rows): consecutive tokens of one sequence
  int tile_rows;                   // attn_prefill_tile_rows of this launch
  void* kpool; void* vpool; int planes; int plane;
  const int* btab; int bt_stride;
  int num_blocks, max_seqs, max_pos;
  int nh; float scale;
  const float2* rope;              // [max_pos][head_dim / 2] cos / sin
  void* out; int ldo;
};
int attn_prefill_launch(int dtype, int head_dim, const PrefillAttnArgs& a, hipStream_t st);
// Query rows per tile for a chunk whose 64-row tiles attend to mean_keys
// cached positions on average and whose 128-row tiles would make wg128
// workgroups (tiles x heads); 128-row tiles (the 32x32x16 kernel, head dims
// 96 and 128) where the key ranges are long and the grid stays large.
// force = 64 or 128 overrides that choice where both forms exist.
int attn_prefill_tile_rows(int dtype, int head_dim, double mean_keys, long wg128, int force);

struct KvWriteArgs {              // prefill: rotate and store K/V of every row
  const float* qkv; int ldq; int qkv_sk;
  int rows;
  const int* seq; const int* pos;
  void* kpool; void* vpool; int planes; int plane;   // layer base, layout as AttnArgs
  const int* btab; int bt_stride;
  int num_blocks, max_seqs, max_pos;
  int nh;
  const float2* rope;            // [max_pos][head_dim / 2]
};
int kv_write_launch(int dtype, int head_dim, const KvWriteArgs& a, hipStream_t st);
// cos / sin of pos * theta^(-2i/hd) for pos < rows, i < hd/2 (angles formed in double)
int rope_table_launch(float2* table, int rows, int head_dim, float theta, hipStream_t st);

struct GateArgs {
  const float* state; int H; int n_slots;
  const float* gate_w; float bias, threshold, eps;
  int kind;                      // 0 linear (z > threshold), 1 convergence (depth >= 2, c < tau)
  const float* prev; float tau;  // convergence: state before the step [n_slots][H], threshold
  int gate_enabled;
  int* n_valid;                  // in: rows; out: continuing rows
  int* slot; int* seq; int* pos; int* depth; int* exit_at;   // compacted in place
  int rows_pad;
  float* z;                      // [rows_pad] scratch
  int* counter;                  // arrival counter (self-resetting)
  int* q_n; int* q_slot; int* q_seq; int* q_pos; int* q_depth; int q_cap;
  int* counts; int* fired_seq;
  int* err;                      // descriptor error word
};
int gate_compact_launch(const GateArgs& a, hipStream_t st);

struct CodaPrepArgs {            // exit rows: write e into the depth map, copy state rows
  const int* q_n; const int* q_slot; const int* q_seq; const int* q_pos; const int* q_depth;
  int rows_pad;
  const float* state; int H; int n_slots;
  float* resid;                  // [rows_pad][H]
  float* states_out;             // optional
  int* pos1;                     // [rows_pad] pos + 1 (successor position)
  uint8_t* emap; const int* btab; int bt_stride;
  int num_blocks, max_seqs, max_pos;
  int* err;                      // descriptor error word
};
int coda_prep_launch(const CodaPrepArgs& a, hipStream_t st);

// Last-exited copy on exit (explicit depth-indexed cache): for every exit
// row r < *q_n with exit depth e < planes, in every core layer, the K and V
// rows of its position at plane e - 1 are copied into planes e .. planes - 1.
struct KvExitCopyArgs {
  const int* q_n; const int* q_seq; const int* q_pos; const int* q_depth;
  int rows_pad;
  void* kpool; void* vpool; long layer_elems;   // core pools, elements per layer
  int n_core, planes, nh, hd, el;               // el: bytes per element
  const int* btab; int bt_stride;
  int num_blocks, max_seqs, max_pos;
  int* err;
};
int kv_exit_copy_launch(const KvExitCopyArgs& a, hipStream_t st);

// One workgroup: for each produced token (row r < *n_rows, or host_rows):
// n_gen[seq]++, tokens_out / exits_out, and for sequences still generating
// the successor enters the continuing list (c_*) and the core batch.
struct BookArgs {
  const int* n_rows; int host_rows; int rows_cap;
  const int* r_slot; const int* r_seq; const int* r_pos;
  const int* r_depth; int depth_uniform;     // exit depth of the pass (NULL: uniform)
  const int* tok;
  int* tokens_out; int* exits_out; int* n_gen; const int* n_out; int max_out; int max_seqs;
  int* c_n; int* c_slot; int* c_seq; int* c_pos; int* c_tok;   // continuing rows
  int* d_n; int* d_slot; int* d_seq; int* d_pos; int* d_depth; int* d_exit_at; int d_cap;
  int r_max;
  int* q_n_reset;                            // exit queue count to zero (NULL: none)
  int* tokens_rows_out;                      // optional
  int* err;                                  // descriptor error word
};
int book_launch(const BookArgs& a, hipStream_t st);

// Prelude of the successor tokens: state[c_slot[r]] = embed[c_tok[r]] (or,
// with pre_out, inject = pre_out row and state = 0) and the depth map of the
// new position = r_max, for r < *c_n.
struct PreludeEmbedArgs {
  const int* c_n; const int* c_slot; const int* c_seq; const int* c_pos; const int* c_tok;
  int rows_pad;
  const void* embed; int dtype; int H; int vocab; int n_slots;
  float* state;
  const float* pre_out; float* inject;
  uint8_t* emap; const int* btab; int bt_stride; int r_max;
  int num_blocks, max_seqs, max_pos;
  int* err;                      // descriptor error word
};
int prelude_embed_launch(const PreludeEmbedArgs& a, hipStream_t st);

struct PrefillSetupArgs {        // per-token sequence/position, depth map = r_max, embedding
  const int* tokens; const int* cu; const int* seq; const int* start_pos; const int* is_final;
  int n_seqs, n_tokens;
  int* tok_seq; int* tok_pos;
  const void* embed; int dtype; int H; int vocab; float* resid;
  uint8_t* emap; const int* btab; int bt_stride; int r_max;
  int num_blocks, max_seqs, max_pos;
  const int* slot;
  int* f_n; int* f_idx; int* f_slot; int* f_seq; int* f_pos;   // final tokens of the chunk
  int* err;                      // descriptor error word
};
int prefill_setup_launch(const PrefillSetupArgs& a, hipStream_t st);

struct GatherRowsArgs {          // out[r] = x[idx[r]] for r < *n (or rows)
  const float* x; int ldx; const int* idx; const int* n; int rows; int H; int x_rows;
  float* out; int ldo;
  int* err;                      // descriptor error word
};
int gather_rows_launch(const GatherRowsArgs& a, hipStream_t st);

struct AddRowsArgs {             // x[slot[r]] += y[slot[r]] (injection) for r < *n_valid
  float* x; const float* y; int H; const int* slot; const int* n_valid; int rows; int n_slots;
  int* err;                      // descriptor error word
};
int add_rows_launch(const AddRowsArgs& a, hipStream_t st);
// dst[slot[r]] = src[slot[r]] for r < *n_valid (the loop state before a core step)
int save_rows_launch(const AddRowsArgs& a, hipStream_t st);

struct EmbedTokArgs {            // out[r] = embed[tok[r]] for r < *n
  const int* tok; const int* n; int rows;
  const void* embed; int dtype; int H; int vocab;
  float* out; int ldo;
  int* err;                      // descriptor error word
};
int embed_tok_launch(const EmbedTokArgs& a, hipStream_t st);

}  // namespace cdb
