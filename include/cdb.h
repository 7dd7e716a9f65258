/*
 * cdb.h — C ABI of the continuous-depth-batching (CDB) hot path on MI355X.
 *
 * The operations follow "Depth-adaptive Inference of Looped Language Models
 * via Continuous Depth Batching" (arXiv 2608.09444):
 *   - §2 Problem Setup: a looped LM = prelude, a shared core looped up to
 *     r_max times per token, coda; every token leaves the core at its own
 *     depth.
 *   - §4.1 Stage-wise Scheduling and Alg. 1 / Alg. 2 (App. A.3): prefill,
 *     prelude, recurrent-core and coda stages run as separate batches; a
 *     core batch mixes tokens at different loop depths.
 *   - §4.2 Depth-aware KV Cache and Fig. 2 (right): depth-indexed cache with
 *     r_max slots per (core layer, token) and last-exited semantics, or a
 *     shared single slot per (core layer, token).
 *   - §4.3 Asynchronous Scheduling: lookahead gate — the exit signal after
 *     step r decides participation in step r+2.
 *   - App. A.1: chunked prefill at full depth; paged KV in 16-token blocks.
 *
 * Conventions for every call
 *   - All pointers in descriptor structs are DEVICE pointers unless marked
 *     "host".  The caller allocates and owns every buffer; buffers must
 *     outlive the context.  The library allocates no device memory.
 *   - Every call is asynchronous and ordered on the stream given to
 *     cdb_init; nothing synchronises unless stated.  One context per stream;
 *     a context is not thread-safe.
 *   - Return value: CDB_OK (0) or a negative error code.  Argument errors are
 *     detected on the host before anything is enqueued (CDB_EINVAL,
 *     CDB_ENOMEM); launch failures return CDB_EHIP.  Values the kernels
 *     read from device memory (slot, sequence, position, depth, block and
 *     token ids, row counts of the queues) are clamped into their buffers,
 *     so a bad value never makes an access out of bounds; a kernel that had
 *     to clamp sets the context's device error word, and the next cdb_sync
 *     returns CDB_EINVAL naming what was out of range (the rows concerned
 *     hold wrong results).  No C++ exception crosses the ABI.
 *     cdb_last_error() returns a message for the last failure.
 *   - Results are deterministic: the same inputs and bucket give bitwise
 *     identical outputs (no floating-point atomics; fixed reduction order).
 *
 * Layouts (row-major, element type T = float for CDB_FP32 and bfloat16 for
 * CDB_BF16; H = hidden, Q = n_heads*head_dim, F = ffn, V = vocab):
 *   - projection matrices, logically [out][in]: wqkv [3Q][H] (rows q, then
 *     k, then v; head h occupies rows h*head_dim..), wo [H][Q], wgu [2F][H]
 *     (rows 0..F-1 gate, F..2F-1 up), wd [H][F], lm_head [V][H], are passed
 *     FRAGMENT-PACKED, as written by cdb_pack_weight: the matrix is cut into
 *     tiles of 16 rows x KS columns (KS = 32 for bf16, 16 for fp32), tiles
 *     ordered by row tile, then column tile; a tile is 64 pieces of 16 bytes,
 *     piece l holding row (l % 16) and columns (l / 16) * (KS / 4) .. +KS/4
 *     of the tile.  Piece l is exactly what lane l of a wave feeds one matrix
 *     instruction, so a wave reads each tile as one contiguous kilobyte.
 *     embed [V][H] stays row-major; norm gains and the gate vector are float [H].
 *   - core KV pools: T [n_core][num_blocks][n_heads][planes][block][head_dim]
 *     with planes = r_max (CDB_KV_DEPTH, CDB_KV_DEPTH_COPY), 1
 *     (CDB_KV_SINGLE) or 2 (CDB_KV_FIRST_SHARED: the first loop's private
 *     plane, then one plane every later loop overwrites; "Depth-adaptive
 *     Inference of Looped Language Models via Continuous Depth Batching",
 *     App. E.1).  Loop d writes plane min(d, planes) - 1 and reads earlier
 *     position j at plane min(d, e_j, planes) - 1 (e_j from the exit-depth
 *     map).  CDB_KV_DEPTH_COPY is the last-exited cache of §4.2 made
 *     explicit: when a token leaves after loop e < r_max, cdb_boundary
 *     copies the K/V it wrote in loop e into planes e .. r_max - 1 of every
 *     core layer, and loop d reads every earlier position at plane d - 1
 *     without the depth map (the same values as CDB_KV_DEPTH reads): the planes of
 *     one (block, head) are adjacent, so the per-position plane choices of a
 *     reader stay within one window of planes*block*head_dim elements;
 *     boundary (prelude + coda layer) pools: T [n_prelude+n_coda][num_blocks]
 *     [n_heads][block][head_dim], prelude layers first.
 *   - exit-depth map: uint8 [num_blocks][block]: e_j of cached position j
 *     (r_max for prompt positions and for the token currently in flight).
 *   - block table: int32 [max_seqs][max_blocks_per_seq], physical block of
 *     each logical block of a sequence.
 *   - loop-state pool: float [n_slots][H]; injection pool (inject models):
 *     float [n_slots][H].
 */
#ifndef CDB_H
#define CDB_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

enum {
  CDB_OK = 0,
  CDB_EINVAL = -1, /* bad dimension, pointer, bucket, depth or layout      */
  CDB_EHIP = -2,   /* a HIP launch or API call failed                      */
  CDB_ENOMEM = -3, /* the caller's workspace is smaller than required      */
  CDB_ESTATE = -4  /* call out of order (e.g. context not initialised)     */
};

enum { CDB_FP32 = 0, CDB_BF16 = 1 };
enum { CDB_KV_DEPTH = 0, CDB_KV_SINGLE = 1, CDB_KV_FIRST_SHARED = 2, CDB_KV_DEPTH_COPY = 3 };
enum { CDB_GATE_LINEAR = 0, CDB_GATE_CONVERGENCE = 1 };

/* Model shape and fixed scalars.  Linear gate: z = gate_w . RMSNorm(h) +
 * gate_bias with a unit-gain norm; the gate fires when z > gate_threshold.
 * Convergence gate (the training-free criterion of the paper's Section 7
 * gating experiments): after loop d >= 2 it fires when
 * |h_d - h_{d-1}|_2 / |h_d|_2 < conv_threshold (h the loop state; needs
 * cdb_pools.prev_state).  Either way a firing after loop d makes the token
 * leave after loop d + 1 (the lookahead of §4.3). */
typedef struct cdb_dims {
  int32_t vocab, hidden, n_heads, head_dim, ffn;
  int32_t n_prelude, n_core, n_coda;
  int32_t r_max;     /* maximum loop count (1..255)                           */
  int32_t dtype;     /* CDB_FP32 or CDB_BF16: weights, KV, GEMM inputs        */
  int32_t kv_layout; /* CDB_KV_DEPTH, CDB_KV_SINGLE, CDB_KV_FIRST_SHARED or
                        CDB_KV_DEPTH_COPY                                     */
  int32_t inject;    /* 1: core input = h + e every loop, h starts at 0       */
  int32_t gate_kind; /* CDB_GATE_LINEAR or CDB_GATE_CONVERGENCE               */
  float rms_eps, rope_theta, gate_bias, gate_threshold;
  float conv_threshold; /* convergence gate threshold tau                     */
} cdb_dims;

/* One transformer block (device pointers, layouts above). */
typedef struct cdb_layer {
  const float* attn_norm;
  const void* wqkv;
  const void* wo;
  const float* mlp_norm;
  const void* wgu;
  const void* wd;
} cdb_layer;

typedef struct cdb_weights {
  const void* embed;
  const cdb_layer* prelude; /* host array [n_prelude] (copied by cdb_init)    */
  const cdb_layer* core;    /* host array [n_core]                            */
  const cdb_layer* coda;    /* host array [n_coda]                            */
  const float* final_norm;
  const void* lm_head;
  const float* gate_w;
} cdb_weights;

typedef struct cdb_kv {
  int32_t block_size;          /* must be 16                                  */
  int32_t num_blocks;
  void* core_k;
  void* core_v;
  void* bnd_k;                 /* may be NULL when n_prelude + n_coda == 0    */
  void* bnd_v;
  uint8_t* exit_depth;
  const int32_t* block_table;
  int32_t max_seqs, max_blocks_per_seq;
} cdb_kv;

/* Per-sequence generation state on the device.  tokens_out[seq][i] receives
 * the i-th generated token (i = 0 from prefill, then one per coda) and
 * exits_out[seq][i] the exit depth of the decode pass that produced token
 * i (r_max for i = 0).  n_gen[seq] counts generated tokens (the caller
 * zeroes it when it admits the sequence); n_out[seq] is the number to
 * generate (no EOS).  A sequence with n_gen == n_out gets no successor. */
typedef struct cdb_seqs {
  int32_t* tokens_out;         /* [max_seqs][max_out]                         */
  int32_t* exits_out;          /* [max_seqs][max_out]                         */
  int32_t* n_gen;              /* [max_seqs]                                  */
  const int32_t* n_out;        /* [max_seqs]                                  */
  int32_t max_out;
} cdb_seqs;

typedef struct cdb_pools {
  float* state;                /* [n_slots][H]                                */
  float* inject;               /* [n_slots][H] or NULL                        */
  float* prev_state;           /* [n_slots][H]: state before the last core
                                  step (convergence gate), else NULL          */
  int32_t n_slots;
  void* workspace;             /* cdb_workspace_bytes() bytes, 256-B aligned  */
  size_t workspace_bytes;
  int32_t max_rows;            /* largest core / boundary bucket              */
  int32_t max_prefill_tokens;  /* largest prefill chunk (M)                   */
  int32_t max_context;         /* longest sequence (positions)                */
} cdb_pools;

/* A core batch (the recurrent queue Q_R of §4.1) at fixed device addresses.
 * Rows 0..*n_valid-1 are valid; row b is the token of sequence seq[b] at
 * position pos[b] whose loop state lives in state[slot[b]], running loop
 * step depth[b] (1-based) with scheduled exit exit_at[b] (r_max unless the
 * lookahead gate fired).  The arrays hold cap entries. */
typedef struct cdb_core_desc {
  int32_t* n_valid;            /* device scalar                               */
  int32_t* slot;
  int32_t* seq;
  int32_t* pos;
  int32_t* depth;
  int32_t* exit_at;
  int32_t cap;
} cdb_core_desc;

/* The coda queue Q_C (exited tokens) at fixed device addresses; rows append
 * at *n and cdb_boundary consumes all of them. */
typedef struct cdb_exit_queue {
  int32_t* n;                  /* device scalar                               */
  int32_t* slot;
  int32_t* seq;
  int32_t* pos;
  int32_t* depth;              /* exit depth e                                */
  int32_t cap;
} cdb_exit_queue;

/* Gate + compaction outputs besides the queues.  counts[0] = rows that
 * continue, counts[1] = rows that exited this step, counts[2] = rows whose
 * gate fired this step, counts[3] = rows that will leave after the NEXT
 * step (the lookahead of §4.3: those that fired now, and those that reach
 * r_max next).  fired_seq lists the sequences of the counts[3] rows in row
 * order, so a host scheduler knows one step ahead which sequences the next
 * core step hands to the coda and need not wait for that step to finish.
 * When host_counts / host_fired are non-NULL (host pinned memory) they
 * receive async copies and `event` (a hipEvent_t, may be NULL) is recorded
 * after them. */
typedef struct cdb_compact_out {
  int32_t* counts;             /* device [4]                                  */
  int32_t* fired_seq;          /* device [cap]: sequences leaving next step   */
  int32_t* host_counts;        /* host pinned [4] or NULL                     */
  int32_t* host_fired;         /* host pinned [cap] or NULL                   */
  void* event;                 /* hipEvent_t or NULL                          */
} cdb_compact_out;

/* A prefill chunk: tokens of n sequences packed back to back (App. A.1).
 * Sequence i contributes tokens[cu_seqlens[i]..cu_seqlens[i+1]) at
 * positions start_pos[i].. of sequence seq[i]; when is_final[i] is 1 its
 * prompt ends in this chunk, the first generated token is written to
 * tokens_out[seq][0] and the token enters the core batch (prelude) with
 * loop state slot[i].  All arrays are device arrays of n (cu_seqlens n+1)
 * entries, except the host copies (all three required) used for
 * validation, launch shapes and the order of the attention tiles. */
typedef struct cdb_prefill_desc {
  int32_t n_seqs, n_tokens;
  const int32_t* tokens;       /* [n_tokens]                                  */
  const int32_t* cu_seqlens;   /* [n_seqs+1]                                  */
  const int32_t* seq;
  const int32_t* start_pos;
  const int32_t* slot;
  const int32_t* is_final;
  const int32_t* host_cu_seqlens; /* host copy of cu_seqlens                  */
  const int32_t* host_start_pos;  /* host copy of start_pos                   */
  const int32_t* host_is_final;   /* host copy of is_final                    */
  float* logits_out;           /* optional [n_seqs][V] logits of final tokens */
} cdb_prefill_desc;

/* Boundary batch: coda for every row of the exit queue, then prelude for
 * the successor token of each sequence with n_gen < n_out (appended to the
 * core batch at depth 1, exit_at r_max, position pos+1, same slot).
 * rows_pad bounds the exit-queue length (launch shape).  exit_states_out
 * and logits_out are optional debug outputs ([rows][H], [rows][V]) in exit
 * queue order. */
typedef struct cdb_boundary_desc {
  int32_t rows_pad;
  float* exit_states_out;      /* optional                                    */
  float* logits_out;           /* optional                                    */
  int32_t* tokens_out_rows;    /* optional [rows]: the token each row produced*/
} cdb_boundary_desc;

/* Rewrite a row-major matrix src [rows][cols] (device memory, element type
 * of dtype) into the fragment-packed layout above at dst (device memory of
 * the same size, not overlapping src), enqueued on stream.  rows must be a
 * multiple of 16 and cols a multiple of KS (32 bf16 / 16 fp32), else
 * CDB_EINVAL.  Every projection matrix handed to cdb_init goes through it. */
int cdb_pack_weight(int32_t dtype, const void* src, void* dst, int32_t rows,
                    int32_t cols, void* stream);

/* Bytes of workspace a context needs for these maxima. */
size_t cdb_workspace_bytes(const cdb_dims* dims, int32_t max_rows,
                           int32_t max_prefill_tokens, int32_t max_context);

/* Create a context.  Validates every shape and pointer on the host, copies
 * the layer-pointer arrays, zeroes the workspace's self-resetting counters
 * on `stream` (hipStream_t; NULL = default stream).  *out = NULL on error.
 * The environment variable CDB_TILE256=0, read here, keeps the context off
 * the 256 x 256 prefill GEMM (the 128 x 128 kernel then takes every tiled
 * projection; both give the same bits), CDB_TILE_WIDE=0 likewise off the
 * 256 x 128 one.  CDB_FUSE_O_ROWS and
 * CDB_FUSE_DOWN_ROWS (defaults 16 and 16; 0 turns the path off) set the
 * largest decode batch whose attention-output and down projections complete
 * the residual stream themselves and leave the following RMSNorm's 1 / rms
 * to the next GEMM's consumer (the same function; the next GEMM's input is
 * rounded to bf16 before the row scale is applied instead of after).
 * CDB_DEFER_NORM_ROWS (default 128; 0 turns it off) sets the largest decode
 * batch above those whose split O and down partials are added to the
 * residual stream by a separate kernel that likewise leaves 1 / rms to the
 * consumer.  CDB_FOLD_MERGE=0 keeps the split-attention merge kernel where that O
 * projection would otherwise merge the splits itself (batches whose merged
 * attention row is one 16-byte piece per lane of the projection's waves,
 * e.g. one row at 16 heads of 128; the same bits either way).
 * CDB_ATTN_WGS (at most 256, the default) sets the workgroup count that
 * the decode attention's context splits aim at.
 * CDB_PF_TILE_ROWS=64 or 128 fixes the query rows per prefill attention
 * tile (bf16, head dims 96 and 128), which otherwise follow the chunk's key
 * ranges (the same bits either way). */
int cdb_init(const cdb_dims* dims, const cdb_weights* w, const cdb_kv* kv,
             const cdb_pools* pools, const cdb_seqs* seqs, void* stream,
             void** out);

/* cdb_init for callers that cannot allocate device memory (code under HIP
 * graph capture, serving loops and harnesses that forbid hipMalloc): the
 * context's workspace is the library's own static device array of
 * 128 MiB per GPU (held until the process ends) instead of
 * pools->workspace, which must be NULL (workspace_bytes is ignored).  No
 * hipMalloc, hipFree or other device allocation is made; the device
 * address of the array is looked up once per GPU.  Returns CDB_ENOMEM when
 * cdb_workspace_bytes() of these maxima exceeds 128 MiB (e.g. the
 * Ouro-like model fits 256 decode rows with 16-token prefill chunks, or 64
 * rows with 1024-token chunks; larger maxima need cdb_init).  The array is cleared here, so a
 * new context starts as from a zeroed caller workspace.  Every context made
 * this way on one GPU shares that GPU's array: only one may be in use at a
 * time; calls on two such contexts that overlap race (wrong results, no
 * out-of-bounds access).  Everything else is as cdb_init. */
int cdb_init_static(const cdb_dims* dims, const cdb_weights* w, const cdb_kv* kv,
                    const cdb_pools* pools, const cdb_seqs* seqs, void* stream, void** out);

/* Full-depth prefill of one chunk (App. A.1, "Chunked prefill"; Alg. 1
 * FullDepthForward; prefill always runs at r_max).  Writes K/V of every
 * core plane 1..r_max (one plane if single-slot), the exit-depth map (r_max)
 * of the chunk's positions, boundary-layer K/V; for sequences whose prompt
 * ends here computes logits of the final position only (App. A.5), writes
 * the first token (n_gen becomes 1), and appends the prelude of that token
 * to `core` when n_out > 1. */
int cdb_prefill(void* ctx, const cdb_prefill_desc* d, const cdb_core_desc* core);

/* One recurrent-core step (§4.1 "recurrent items ready for their next loop
 * step"; Alg. 2 Core) for rows 0..*n_valid-1 of `core`, each at its own
 * depth.  rows_pad (a power of two, >= *n_valid, <= max_rows) fixes the
 * launch shape.  Reads earlier positions at plane min(depth, e_j) of the
 * depth-indexed cache (equivalent to the last-exited copy of §4.2) or the
 * single plane; writes this row's K/V at plane depth (or the single plane)
 * and updates state[slot] in place. */
int cdb_core_step(void* ctx, const cdb_core_desc* core, int32_t rows_pad);

/* Lookahead gate and stream compaction after a core step (§4.3; Alg. 2
 * Gate).  For each valid row: if depth == exit_at the row leaves (appended
 * to `exits` in row order); otherwise, when gate_enabled, z is evaluated
 * and z > threshold sets exit_at = depth + 1.  Continuing rows are
 * compacted to the front of `core` in row order with depth + 1; *n_valid
 * becomes their count. */
int cdb_gate_compact(void* ctx, const cdb_core_desc* core, int32_t rows_pad,
                     int32_t gate_enabled, cdb_exit_queue* exits,
                     const cdb_compact_out* out);

/* Coda + prelude boundary (Alg. 2 Coda and Prelude; §2: prelude and coda
 * run once per token).  Consumes the whole exit queue (resets *exits->n to
 * 0): writes e into the exit-depth map at (seq, pos), runs coda layers,
 * final norm, LM head and greedy argmax (lowest index among equal maxima),
 * stores the token at tokens_out[seq][n_gen[seq]++] (and e at exits_out),
 * and preludes the token at pos+1 into `core` when n_gen < n_out. */
int cdb_boundary(void* ctx, cdb_exit_queue* exits, const cdb_core_desc* core,
                 const cdb_boundary_desc* d);

/* Kernel timing with HIP events on the context's stream.  While enabled,
 * every kernel class (see cdb_profile_read) gets a start and stop event
 * around each launch; this adds event records to the stream and is meant
 * for measurement passes.  enable = 0 stops recording and keeps totals;
 * enable = 1 clears the totals and starts recording. */
int cdb_profile(void* ctx, int32_t enable);

/* Synchronises the stream, folds the recorded events into totals, and
 * returns the summed duration (ms) and the launch count of one kernel
 * class: "attn", "gemm_qkv", "gemm_o", "gemm_gu", "gemm_down", "lm_head",
 * "norm", "gate", "boundary", "prefill_attn", "prefill_gemm", "other". */
int cdb_profile_read(void* ctx, const char* kernel_class, double* total_ms, int64_t* launches);

/* HIP graphs (§4.3 and App. A.5 of the pages: static buffers, captured
 * stage graphs per power-of-two bucket).  cdb_graph_begin starts capturing
 * the context's stream; the library calls that follow (cdb_core_step,
 * cdb_gate_compact, cdb_boundary with fixed descriptors) are recorded
 * instead of run; cdb_graph_end instantiates them into *graph (an opaque
 * handle).  cdb_graph_launch replays the graph on the context's stream:
 * every buffer address is fixed at capture and every count lives in device
 * memory, so a replay computes on the current contents.  The library
 * records no memset into a graph.  Profiling must be off while capturing.
 * cdb_prefill is not capturable (its launch shapes depend on host data). */
int cdb_graph_begin(void* ctx);
int cdb_graph_end(void* ctx, void** graph);
int cdb_graph_launch(void* ctx, void* graph);
void cdb_graph_destroy(void* graph);

/* Wait for all work of the context's stream, then read and clear the
 * device error word: CDB_EINVAL (message in cdb_last_error) when a kernel
 * since the previous cdb_sync clamped an out-of-range descriptor value --
 * a depth outside [1, r_max], a slot, sequence, position, block or token id
 * outside its buffer, or a device row count above the launch rows or a
 * queue's capacity (such rows are dropped).  CDB_ESTATE while capturing. */
int cdb_sync(void* ctx);

void cdb_destroy(void* ctx);

const char* cdb_strerror(int code);

/* Message of the last error on this thread (empty when none). */
const char* cdb_last_error(void);

/* Library version string. */
const char* cdb_version(void);

#ifdef __cplusplus
}
#endif
#endif /* CDB_H */
