/*
 * spear.h - C ABI of libspear, the compensated 4-bit linear layer on AMD
 * Instinct MI355X (gfx950).
 *
 * The layer computes, per token m (one row of x),
 *
 *     y[m] = dequant(W_q) x[m] + g(x[m]) * B (A x[m]),
 *     g(x) = sigmoid(w_g . x + b_g),
 *
 * where dequant(W_q)[n][k] = (q[n][k] - z[n][k/G]) * s[n][k/G] is the 4-bit
 * weight with fp16 scale s and zero-point z per output row and group of G
 * input columns, and A (r x K), B (N x r) form a low-rank error compensator.
 *
 * Source: "SPEAR: A System for Post-Quantization Error-Adaptive Recovery
 * Enabling Efficient Low-Bit LLM Serving", explanation pages on gist.science
 * (paper 2606.11244), English page, Technical Summary:
 *   - 2.1 A "Input-Adaptive Error Compensators": the compensator projects x
 *     to rank r with A, applies an input-dependent gate and projects back
 *     with B; the effective weight is W + alpha B diag(gamma(Ax)) A.  This
 *     library takes W as the dequantized 4-bit weight, alpha = 1 (folded into
 *     B) and the gate as one scalar per token, sigmoid(w_g . x + b_g).
 *   - 2.2 A "Phase-Aware Adaptive Kernel Fusion Dispatch": decode (few
 *     tokens, memory-bound) runs the compensator inside the low-bit product
 *     kernel; prefill (many tokens, compute-bound) runs it as a separate
 *     kernel that overlaps the product.
 *   - 2.2 C "SLO-Constrained EC-Aware Chunk Scheduling": pick the largest
 *     prefill chunk whose table-predicted latency meets the latency target.
 *
 * Conventions shared by every call:
 *   - Device pointers are HIP device memory owned by the caller.  The library
 *     allocates no device memory and copies nothing between host and device.
 *   - Every compute call is asynchronous on the stream(s) it is given and
 *     never synchronises.  A stream argument is a hipStream_t passed as a
 *     void pointer; NULL is the null stream.
 *   - Arguments are validated on the host before anything is launched.  On
 *     any error nothing is launched, the outputs are untouched and
 *     spear_last_error() describes the problem for the calling thread.
 *   - y must not alias any input.
 *   - Element types: x, y, A, B and w_g share the activation type
 *     (SPEAR_F16 or SPEAR_BF16); scales and zero-points are always fp16.
 *     Arithmetic is fp32 throughout; only y is rounded (round to nearest
 *     even) to the activation type.
 */
#ifndef SPEAR_H
#define SPEAR_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum spear_status {
  SPEAR_OK = 0,
  SPEAR_ERR_INVALID_ARGUMENT = 1, /* null/misaligned pointer, bad shape or enum */
  SPEAR_ERR_UNSUPPORTED = 2,      /* valid request outside what the kernels cover */
  SPEAR_ERR_WORKSPACE = 3,        /* workspace missing or smaller than required */
  SPEAR_ERR_HIP = 4               /* the HIP runtime reported an error */
} spear_status_t;

typedef enum spear_dtype { SPEAR_F16 = 0, SPEAR_BF16 = 1 } spear_dtype_t;

typedef void *spear_stream_t; /* a hipStream_t */

/*
 * One compensated 4-bit layer.  All pointers are device memory.
 *
 *   N, K        output and input features.  K % 32 == 0 (the packed rows are
 *               consumed in 16-byte pieces), K <= SPEAR_MAX_K; N >= 1.
 *   group_size  G: columns per scale/zero-point group.  G == K means one
 *               group per output row (per-channel).  Otherwise G % 128 == 0
 *               and K % G == 0.
 *   qweight     int32, SPEAR_QWEIGHT_WORDS(N, K) words, 16-byte aligned, in
 *               the tiled order.  Eight unsigned codes (0..15) per word along
 *               K, lowest nibble first: code k = 8j+i of row n is bits
 *               4i..4i+3 of that row's word j.  The words are stored by
 *               blocks of 16 rows (N padded with zero words to a multiple of
 *               16): inside a block, piece P (words 4P..4P+3, codes
 *               32P..32P+31) of rows 0..15, then piece P+1 of rows 0..15, and
 *               so on.  Word j of row n is thus at word index
 *                 (n / 16) * 2K + (j / 4) * 64 + (n % 16) * 4 + j % 4,
 *               and each 128-code tile of a row block is 1 KB in the order a
 *               64-lane wave loads it.  spear_pack_int4 (from codes) and
 *               spear_tile_int4 (from row-after-row words) produce it.
 *   scales      fp16 bit patterns [N][K/G], row-major (16-byte alignment is
 *               not required, but it is the fast path).
 *   zeros       fp16 bit patterns [N][K/G]: the zero-point as a code value
 *               (not pre-multiplied by the scale).
 *   rank        r >= 0.  r == 0 is the plain 4-bit product: A, B and w_gate
 *               are then ignored and may be NULL.  r <= SPEAR_MAX_RANK.
 *   A           [r][K] activation type, row-major (the down-projection).
 *   B           [N][r] activation type, row-major (the up-projection).
 *   w_gate      [K] activation type (gate weights).
 *   b_gate      gate bias; +INFINITY gives g == 1 and -INFINITY gives g == 0
 *               exactly (for finite w_gate . x).
 *   rank_gate   optional per-rank gate (see spear_rank_gate_t); r > 0 only.
 */
/*
 * The pages' per-rank gate (2.1 A: the compensator applies an input-adaptive
 * gate gamma(A x) to each of the r rank components, with a strength alpha).
 * gamma is read as a bottleneck MLP r -> hidden -> r:
 *
 *     t = A x,  gamma(t) = sigmoid(W2 relu(W1 t + b1) + b2),
 *     y = dequant(W_q) x + alpha * B (gamma(t) * t)      (elementwise product)
 *
 * All arrays are fp32 device memory: W1 [hidden][r], b1 [hidden],
 * W2 [r][hidden], b2 [r], row-major.  1 <= hidden <= SPEAR_MAX_GATE_HIDDEN.
 * The struct itself is host memory, read during the call only.
 */
#define SPEAR_MAX_GATE_HIDDEN 64
typedef struct spear_rank_gate {
  int32_t hidden;
  const float *W1;
  const float *b1;
  const float *W2;
  const float *b2;
  float alpha;
} spear_rank_gate_t;

typedef struct spear_layer {
  int32_t N, K, group_size;
  const int32_t *qweight;
  const uint16_t *scales;
  const uint16_t *zeros;
  int32_t rank;
  const void *A;
  const void *B;
  const void *w_gate;
  float b_gate;
  /* NULL: the scalar gate sigmoid(w_gate . x + b_gate).  Otherwise the
   * per-rank gate above, and w_gate / b_gate are ignored (may be NULL). */
  const spear_rank_gate_t *rank_gate;
} spear_layer_t;

#define SPEAR_MAX_RANK 128
#define SPEAR_MAX_K 131072
#define SPEAR_MAX_DECODE_M 128  /* 1..32: per-row-group kernels (but see below); 33..128: the wide-tile kernel */

/*
 * Workspace bytes that spear_linear_decode, spear_linear_prefill and
 * spear_linear need for this layer for any call with 1..M tokens.
 * Returns 0 when the layer or M is invalid.  The workspace is caller-owned
 * device memory, 256-byte aligned, and must be ZEROED ONCE before its first
 * use; every call leaves it ready for the next one.  One workspace may serve
 * several layers if it is at least the largest of their sizes: its counters
 * sit at fixed offsets and every other byte is rewritten by a call before
 * the call reads it.  Calls that may run concurrently (different streams)
 * need different workspaces.
 *
 * Compensated layers need a workspace for every call.  For a layer with
 * r == 0 it is optional, except for decode calls that take the tile launch
 * with K-splits (spear_linear_plan: SPEAR_PATH_DECODE_WIDE, k_splits > 1),
 * whose partial tiles it holds; a rank-0 layer's size can exceed that of a
 * compensated layer of the same shape, whose producers may leave its tiles
 * fewer K-splits.  Otherwise prefill uses it to split K across workgroups when
 * the output has few 128 x 128 tiles (small M), and decode uses it to
 * split K across the workgroups of each 128-row output tile where the
 * thresholds of spear_set_decode_split_min_m and _min_k ask for that.  Decode takes that split launch
 * only when the workspace given is at least this size for the call's M;
 * with a smaller (or no) workspace it runs the unsplit launch.
 */
size_t spear_workspace_bytes(const spear_layer_t *layer, int32_t M);

/* Words of qweight for an N x K layer: rows padded to a multiple of 16. */
#define SPEAR_QWEIGHT_WORDS(N, K) ((((int64_t)(N) + 15) / 16) * 16 * ((int64_t)(K) / 8))

/*
 * Pack 4-bit codes (the pages' 4-bit weight, Problem Statement and 2.1 A):
 * q uint8 [N][K] (device, row-major; only the low 4 bits of each byte are
 * used) -> qweight, SPEAR_QWEIGHT_WORDS(N, K) int32 words (device, 16-byte
 * aligned, written in full including the zero padding rows) in the tiled
 * order described at spear_layer_t.  K % 32 == 0.  Bit-exact.
 * Not a step of the layer itself: the packing done once per layer.
 * Asynchronous on stream; the caller owns both buffers.
 */
spear_status_t spear_pack_int4(const uint8_t *q, int32_t *qweight, int64_t N, int64_t K,
                               spear_stream_t stream);

/*
 * Reorder words packed row after row (int32 [N][K/8], the same eight codes
 * per word, lowest nibble first, 16-byte aligned) into the tiled order:
 * qweight as for spear_pack_int4.  For loading weights that were packed
 * elsewhere.  K % 32 == 0; the two buffers must not overlap.  Bit-exact.
 */
spear_status_t spear_tile_int4(const int32_t *words, int32_t *qweight, int64_t N, int64_t K,
                               spear_stream_t stream);

/*
 * Decode path (2.2 A, decode phase): one fused kernel launch for 1 <= M <= 128
 * tokens.  Up to 32 tokens, workgroups own groups of 16 to 128 output rows
 * over all of K (or K-splits, see below); from 33 tokens on, workgroups own
 * tiles of 128 output rows over a K-split each and stream x through LDS, so
 * that each staged activation fragment feeds many rows, and the last split to
 * finish a tile sums its partials in split order and adds the compensator.
 * The tile launch also serves 17..32 tokens on layers of at most 64 tiles of
 * 128 rows for which the split thresholds below want a K-split but no
 * split-K launch shape fits (long K with group-wise scales, e.g. K = 28672 at
 * G = 128, or a rank-64 compensator at K = 8192 past 16 tokens); there the
 * whole-K row groups would each stream all of x.  spear_linear_plan reports
 * which launch a call takes.  (With the tile launch: with the per-rank
 * gate, or with K-splits over more than 128 tiles, two more launches on the
 * same stream do that: one forms the compensator's gated sums, a finish
 * kernel adds them and the partials.)
 * x [M][K] and y [M][N] are row-major activation-type device arrays, x and y
 * 16-byte aligned.  The gate, A x and the gated B (A x) term are computed in
 * the same launch as the 4-bit product and added before y is rounded.
 * M == 0 is a no-op.  Where the split thresholds ask for it (see
 * spear_set_decode_split_min_m) and the workspace has
 * spear_workspace_bytes(layer, M) bytes, the launch splits
 * K across the workgroups of each 128-row output tile (the last split to
 * finish a tile sums the tile's partials in split order and applies the
 * compensator); the result differs from the unsplit launch only in the
 * order of fp32 additions.
 */
spear_status_t spear_linear_decode(const spear_layer_t *layer, spear_dtype_t dtype,
                                   const void *x, void *y, int32_t M, void *workspace,
                                   size_t workspace_bytes, spear_stream_t stream);

/*
 * For callers that cannot allocate device memory: code under HIP graph
 * capture, tight serving loops, harnesses that forbid allocation.  The same
 * call as spear_linear_decode, without a workspace argument: its workspace
 * is a device array of SPEAR_NOALLOC_SCRATCH_BYTES held by the library, one
 * per GPU (the GPU current when the call is made, which must be the stream's),
 * for as long as the process runs.  Nothing is allocated, by the call or by
 * its set-up (the first call on a GPU finds the array's address and clears
 * its counters with a kernel on `stream`).  Every call on one GPU shares that
 * array: calls that overlap on one GPU (concurrent streams) race and must not
 * be issued; stream-ordered calls are fine, as each call leaves the counters
 * at zero for the next.  A call whose workspace need exceeds the array
 * returns SPEAR_ERR_WORKSPACE; a split-K launch whose partial tiles do not
 * fit runs the unsplit launch instead (never at the sizes the library
 * supports: the largest need is below 16.2 MiB).
 */
#define SPEAR_NOALLOC_SCRATCH_BYTES (17u << 20)
spear_status_t spear_linear_decode_noalloc(const spear_layer_t *layer, spear_dtype_t dtype,
                                           const void *x, void *y, int32_t M,
                                           spear_stream_t stream);

/*
 * Prefill path (2.2 A, prefill phase): any M >= 1.  The 4-bit product is an
 * MFMA GEMM over LDS-staged dequantized tiles; the compensator's thin
 * products (gate, A x, scaled by the gate) are added in the GEMM tiles'
 * epilogue before y is rounded once.  Two schedules:
 *   aux_stream == NULL (or equal to main_stream): serial, all on main_stream:
 *     the compensator kernels, then the GEMM.
 *   aux_stream given: concurrent.  With the scalar gate and an unsplit GEMM
 *     (enough 128x128 output tiles), the compensator runs as producer
 *     workgroups inside the GEMM launch on main_stream, dispatched ahead of
 *     the tiles; each tile waits for them (bounded by the decode spin limit,
 *     see spear_set_decode_spin_limit) before its epilogue and computes the
 *     sums of its own tokens if the wait expires (bit 0 of the workspace
 *     flags).  aux_stream is then not used.  Otherwise (per-rank gate, or a
 *     K-split GEMM at few tiles with K > 16384) the compensator kernels run on
 *     aux_stream beside the GEMM and a finish kernel adds their term after
 *     the join.
 * In both schedules, a K-split GEMM (few output tiles) with the scalar gate
 * and K <= 16384 runs as two launches on main_stream: the compensator's
 * producers inside the GEMM launch, ahead of its tiles, and a finish kernel
 * that sums the splits and adds the compensator's term.
 * When the call returns, work on aux_stream is ordered after main_stream's
 * prior work and main_stream's later work is ordered after all of it.
 */
spear_status_t spear_linear_prefill(const spear_layer_t *layer, spear_dtype_t dtype,
                                    const void *x, void *y, int32_t M, void *workspace,
                                    size_t workspace_bytes, spear_stream_t main_stream,
                                    spear_stream_t aux_stream);

/*
 * Phase-aware dispatch (2.2 A): M <= spear_get_decode_max_m() goes to the
 * decode path on main_stream, larger M to the prefill path.  One mixed case
 * is split: when the prefill's last 128-token tile row would hold only
 * r = M mod 128 <= 32 tokens after at least 8 full tile rows (a prefill
 * chunk with a few decode tokens appended), the first M - r tokens take the
 * prefill path and the last r the decode path, one after the other on
 * main_stream (r must also be within the decode threshold, and the
 * workspace large enough for both; spear_workspace_bytes(layer, M) is).
 * Every argument is validated before anything is launched.
 */
spear_status_t spear_linear(const spear_layer_t *layer, spear_dtype_t dtype, const void *x,
                            void *y, int32_t M, void *workspace, size_t workspace_bytes,
                            spear_stream_t main_stream, spear_stream_t aux_stream);

/*
 * Static graph of layer calls (2.2 A, prefill phase: the compensator runs as
 * a separate kernel beside the GEMM in a static graph, so no host launch
 * overhead sits between the kernels).  The library captures a sequence of
 * spear_linear calls into one HIP graph it holds; each prefill call's
 * compensator kernels go on the graph's own aux branch (forked from and
 * joined back into the main chain), decode calls are single launches.
 * Calls run in the order they were added.  Every pointer given to
 * spear_graph_add (x, y, the layer's arrays, the workspace) is baked into the
 * graph: each launch reads and writes those same buffers, which must stay
 * allocated until the graph is destroyed; their contents may change between
 * launches.  Two launches of one graph, or of graphs that share a workspace,
 * must be ordered (the same stream, or events).
 *
 *   spear_graph_begin   starts a graph (creates the library's capture and aux
 *                       streams, default priority); *graph receives the handle.
 *   spear_graph_add     validates and appends one spear_linear call, with the
 *                       same arguments and checks (nothing runs yet).  An
 *                       invalid call returns its error and adds nothing.
 *   spear_graph_end     instantiates the graph; after it only launch and
 *                       destroy are valid.
 *   spear_graph_launch  runs the whole graph once on `stream`, asynchronously.
 *   spear_graph_destroy releases the graph (any state; NULL is a no-op).
 * The graph is host-side state owned by the caller through the handle.
 */
typedef struct spear_graph *spear_graph_t;
spear_status_t spear_graph_begin(spear_graph_t *graph);
spear_status_t spear_graph_add(spear_graph_t graph, const spear_layer_t *layer,
                               spear_dtype_t dtype, const void *x, void *y, int32_t M,
                               void *workspace, size_t workspace_bytes);
spear_status_t spear_graph_end(spear_graph_t graph);
spear_status_t spear_graph_launch(spear_graph_t graph, spear_stream_t stream);
spear_status_t spear_graph_destroy(spear_graph_t graph);

/* Dispatch threshold for spear_linear, 1..SPEAR_MAX_DECODE_M (default 64). Process-wide. */
spear_status_t spear_set_decode_max_m(int32_t m);
int32_t spear_get_decode_max_m(void);

/*
 * When decode considers the split-K launch: for layers with
 * K >= spear_get_decode_split_min_k() (>= 1, default 8192), from
 * M = spear_get_decode_split_min_m() tokens on (1..33, default 16; 33 switches
 * the split off; these thresholds concern calls of at most 32 tokens), and, for layers
 * with K at least twice the column threshold, from an eighth of the token
 * threshold on but never below 2 tokens (M >= max(2, ceil(min_m / 8)); with
 * the defaults, M >= 2 from K = 16384).
 * Process-wide.  Set them before sizing workspaces: spear_workspace_bytes
 * includes the split launch's partial tiles only for the calls it applies to.
 */
spear_status_t spear_set_decode_split_min_m(int32_t m);
int32_t spear_get_decode_split_min_m(void);
spear_status_t spear_set_decode_split_min_k(int32_t k);
int32_t spear_get_decode_split_min_k(void);

/*
 * How long a decode launch's consumer workgroups wait for its compensator
 * producers: at most `polls` reads of the producers' count (default 2^20,
 * about a second).  If the wait expires, the workgroup computes the sums
 * A x and w_g . x itself from A, w_g and x, so the output is the same up to
 * the order of fp32 additions, and bit 0 of the workspace flags is set (see
 * spear_workspace_flags).  0 makes every consumer compute them itself without
 * waiting (for tests of that path; it is slow).  Process-wide; read when a
 * call is issued (a captured graph keeps the value it was captured with).
 */
spear_status_t spear_set_decode_spin_limit(uint32_t polls);
uint32_t spear_get_decode_spin_limit(void);

/*
 * Chunk selector (2.2 C), host only: among n candidate prefill chunk sizes
 * with predicted step latencies pred_ms (host arrays), return the largest
 * chunk whose prediction is <= budget_ms (compared in float).  If none fits,
 * return the smallest chunk and set *violated = 1 (else 0; violated may be
 * NULL).  Returns -1 for invalid arguments (n < 1, NULL arrays, a chunk < 1).
 */
int32_t spear_select_chunk(const int32_t *chunks, const float *pred_ms, int32_t n,
                           float budget_ms, int32_t *violated);

/*
 * Which launch a call takes, computed on the host without launching anything
 * (the same planning that spear_linear, spear_linear_decode and
 * spear_linear_prefill run).  For inspection and tests; the compute calls do
 * not need it.
 */
typedef enum spear_path {
  SPEAR_PATH_NONE = 0,          /* M == 0: nothing is launched */
  SPEAR_PATH_DECODE = 1,        /* fused decode, one workgroup per group of output rows */
  SPEAR_PATH_DECODE_SPLIT = 2,  /* fused decode, K split across each 128-row tile's workgroups */
  SPEAR_PATH_PREFILL = 3,       /* the prefill GEMM path */
  SPEAR_PATH_DECODE_WIDE = 4,   /* fused decode with 128-row tiles over K-splits: 33..128 tokens (and 17..32 on long-K layers) */
  SPEAR_PATH_PREFILL_DECODE_TAIL = 5 /* spear_linear only: prefill for M - r tokens, then decode for
                                        the last r (the plan describes the prefill launch) */
} spear_path_t;

typedef struct spear_plan {
  int32_t path;                /* a spear_path_t */
  int32_t workgroups;          /* of the main launch (decode: producers included) */
  int32_t waves_per_workgroup; /* of the main launch */
  int32_t producers;           /* decode: compensator workgroups of the launch (0 at rank 0) */
  int32_t k_splits;            /* splits of K in the main product (1: none) */
  size_t workspace_bytes;      /* the least workspace this call accepts (0: none needed) */
} spear_plan_t;

/*
 * Plan of spear_linear (phase = 0), spear_linear_decode (1) or
 * spear_linear_prefill (2) for this layer, M tokens and a workspace of
 * workspace_bytes (0: no workspace) into *plan (host memory).  Returns the
 * status the call itself would return for a valid x and y.
 */
spear_status_t spear_linear_plan(const spear_layer_t *layer, int32_t M, size_t workspace_bytes,
                                 int32_t phase, spear_plan_t *plan);

/* Static description of a status code. */
const char *spear_status_string(spear_status_t status);

/* Detail of the last error reported to the calling thread ("" if none). */
const char *spear_last_error(void);

/*
 * Sticky error word of a workspace (device pointer), copied to *flags
 * (host) with a synchronous read on `stream`.  Bit 0 set: a decode launch
 * gave up waiting for its compensator producers (bounded wait, see
 * spear_set_decode_spin_limit) and computed their sums itself; its output is
 * still complete.  The bit stays set until the caller clears the word.
 * Diagnostic only; this call synchronises the stream.
 */
spear_status_t spear_workspace_flags(const void *workspace, uint32_t *flags,
                                     spear_stream_t stream);

/* Library version: major * 10000 + minor * 100 + patch. */
int32_t spear_version(void);

#ifdef __cplusplus
}
#endif

#endif /* SPEAR_H */
