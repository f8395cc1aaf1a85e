/*
 * qgemm.h - block-quantised (GGUF Q4_0 / Q8_0) weight x activation products
 * for AMD MI355X (gfx950).  Plain C ABI: no C++ or framework types cross it.
 *
 * Sources for what each call computes (the pages this library follows):
 *   [ENG]  "Engine and kernels" (Pooled engine page): "What it runs" (GGUF
 *          Q4_0 / Q8_0 blocks of 32 weights + one f16 scale), "Kernel
 *          families" (cooperative GEMV, batched GEMV twins, fused gate/up with
 *          SiLU, 16-column prefill GEMM, MoE, GPU sampling), "What each trick
 *          bought" (Reading weights: dequantise in registers, f16 scales,
 *          load-time repack into separate weight and scale arrays; Fewer
 *          passes: y += W.x into the residual, GPU argmax with lowest-index
 *          ties; Batching and prefill: split-K pinned per shape; Speculation:
 *          drafts over a prefix of the vocabulary rows), "Correctness and
 *          portability" (no f16 accumulation).
 *   [ARCH] "Architecture" (Pooled architecture page): "One token, end to end"
 *          (LM head over all vocabulary rows, greedy sampling on the GPU),
 *          "Prefill" (16 columns per pass), "Memory and caching" (Q4_0 / Q8_0
 *          repacked on the way into separate nibble and scale arrays).
 *   [MOE]  "A 235B model in a browser window": experts stacked by role (all
 *          gate matrices in one tensor, all up in a second, all down in a
 *          third), each expert a gated FFN of three matrices.
 *
 * Conventions for every call:
 *   - A matrix W has `rows` outputs and `cols` inputs; cols % 32 == 0.
 *     Row r of the GGUF tensor is cols/32 consecutive blocks.
 *   - Activations are f32 column-major: column j of X starts at X + j*ldx.
 *     X (and x) must be 16-byte aligned with ldx a multiple of 4 (columns are
 *     read as whole 16-byte vectors); Y and H need 4-byte alignment only;
 *     ldx >= cols, ldy >= rows.
 *   - Arithmetic: weights are dequantised exactly in registers; every sum and
 *     every scale multiply is f32, nothing is accumulated in f16 [ENG
 *     Correctness and portability].  Activations are f32 and keep f32 range:
 *     products of 1..8 columns (GEMV, gate/up, LM head, MoE experts) carry
 *     each activation as a pair of f16 values under a power of two chosen
 *     per 128 values of a column (any finite f32 magnitude; error <= 2^-22
 *     of the value plus 2^-39 of the largest magnitude among its 128).  Only the 16-column prefill GEMM rounds its activation
 *     operands to f16 (round to nearest even, relative error <= 2^-11, so
 *     |x| must stay below 65504 there).  Results are bitwise reproducible
 *     run to run: all reductions (split-K included) have a fixed order per
 *     shape.
 *   - Pointers named qs, d, X, Y, H, x, out_*, ws, blocks are DEVICE
 *     pointers; `stream` is a hipStream_t passed as void* (NULL = the null
 *     stream).  Calls are asynchronous on that stream; a device fault shows
 *     up at the caller's next synchronisation.  All argument checks run on
 *     the host before any HIP call, so every error code below can be
 *     produced without a GPU.  Nothing throws across the ABI.
 *   - Memory is owned by the caller.  The library allocates nothing.
 *   - Workspace (`ws`, `ws_bytes`): device memory sized by the matching
 *     *_ws_bytes query, 256-byte aligned.  Its first QG_WS_SYNC_BYTES bytes
 *     are counters through which workgroups of one call find the last of
 *     them to finish: they must be zero before the first call, and every
 *     call that completes leaves them zero again.  The rest is scratch that
 *     each call writes before reading.  So one workspace (as large as the
 *     largest query) may serve any sequence of calls, of any entry point and
 *     shape, issued in order on one stream.  Two calls that may overlap in
 *     time (different streams) must not share a workspace: they would race.
 */
#ifndef QGEMM_H
#define QGEMM_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Bytes of counters at the start of every workspace (see Conventions). */
#define QG_WS_SYNC_BYTES 262144u

/* Bytes of the library-owned scratch of lmhead_argmax_noalloc (per GPU). */
#define QG_NOALLOC_SCRATCH_BYTES (2u << 20)

/* Largest k of lmhead_topk. */
#define QG_TOPK_MAX 16

/* GGUF tensor type ids, so a GGUF reader can pass them through. */
enum { QG_Q4_0 = 2, QG_Q8_0 = 8 };
/* Source block types qg_requant_q8_0 converts (GGUF type ids). */
enum { QG_Q4_1 = 3, QG_Q5_0 = 6, QG_Q5_1 = 7, QG_Q4_K = 12, QG_Q5_K = 13, QG_Q6_K = 14 };

enum {
  QG_OK = 0,
  QG_EINVAL = -1,       /* null pointer, bad enum, overlap of output and input */
  QG_ESHAPE = -2,       /* sizes: cols % 32, non-positive sizes, ncols, n_rows, top_k */
  QG_EALIGN = -3,       /* pointer or leading dimension alignment */
  QG_EUNSUPPORTED = -4, /* valid request this build does not serve */
  QG_EWORKSPACE = -5,   /* ws NULL or smaller than the query says */
  QG_EHIP = -6          /* a HIP launch reported an error */
};

/* Text for a status code (static storage). */
const char *qg_strerror(int status);

/* Name and text of the last HIP error behind a QG_EHIP on the calling
 * thread (thread-local storage, valid until the next failing call). */
const char *qg_last_hip_error(void);

/* Measurement aid, not part of the product path  [ARCH: the pages time a
 * plain copy at load and quote their GEMV against the streaming limit they
 * measure]: reads every byte of [p, p + bytes) once, as the product kernels
 * stream weights (nontemporal 16-byte loads, one contiguous run per wave),
 * and computes nothing from it, so its rate is a measured read ceiling.
 * p: device pointer, 16-byte aligned; bytes: a multiple of 16, > 0; sink: a
 * device uint32 the kernel may write (almost never does).  Asynchronous on
 * `stream`.  Errors: QG_EINVAL (null), QG_EALIGN, QG_ESHAPE, QG_EHIP. */
int qg_read_probe(const void *p, size_t bytes, uint32_t *sink, void *stream);

/* Measurement aid: the memory clock (kHz) and bus width (bits) the HIP
 * runtime reports for `device`, from which a peak HBM rate follows (two
 * transfers per clock: 2 * clock * width / 8 bytes per second), to cross-
 * check a published peak.  Host only.  Errors: QG_EINVAL (null pointer),
 * QG_EHIP (no such device). */
int qg_device_memory(int32_t device, int32_t *clock_khz, int32_t *bus_bits);

/* ------------------------------------------------------------------------
 * Load-time repack  [ARCH Memory and caching; ENG Reading weights]
 *
 * Rewrites GGUF blocks into two streams the kernels read as contiguous
 * 1 KiB stripes: a weight stream `qs` and an f16 scale stream `d`.  It is a
 * layout change only (a bijection; the bytes are the same weights).
 *
 * Tiled layout (n_mat matrices of rows x cols, each padded independently):
 *   tile = 16 rows x 4 blocks (128 columns); NT = ceil(rows/16),
 *   KT = ceil(cols/128); tile (rt, kt) has index t = rt*KT + kt and matrix m
 *   starts at m*NT*KT tiles.  Positions beyond rows / cols hold zero weights
 *   and a zero scale.
 *   Q4_0 qs: 1024 B per tile.  16-byte chunk c = 16*s + r (s = 8-column slice
 *     0..3, r = row 0..15 in the tile) holds 4 little-endian u32 words; word
 *     j covers block 4*kt + j, row 16*rt + r, columns 8*s + i (i = 0..7) of
 *     that block.  The unsigned nibble (weight + 8) of column i = 2u is at
 *     bits 4u..4u+3, that of column i = 2u + 1 at bits 16+4u..19+4u.
 *   Q8_0 qs: 2048 B per tile, two 1024-B halves h = 0, 1.  In half h, chunk
 *     c = 16*s + r holds 8 bytes of block 4*kt + 2h, then 8 bytes of block
 *     4*kt + 2h + 1; byte i is (weight of column 8*s + i) + 128.
 *   d: 128 B per tile; the f16 scale of row 16*rt + r, block 4*kt + j is at
 *     byte 8*r + 2*j.
 * ------------------------------------------------------------------------ */

/* Sizes of the two packed streams (host only, no HIP call). */
int qg_packed_bytes(int qtype, int64_t n_mat, int64_t rows, int64_t cols,
                    size_t *qs_bytes, size_t *d_bytes);

/* blocks: n_mat*rows*(cols/32) GGUF blocks (18 B or 34 B each), 2-byte
 * aligned.  qs 16-byte aligned, d 8-byte aligned, sized by qg_packed_bytes.
 * Outputs must not overlap the input. */
int qg_repack(int qtype, int64_t n_mat, int64_t rows, int64_t cols,
              const void *blocks, void *qs, void *d, void *stream);

/* ------------------------------------------------------------------------
 * GEMV / batched GEMV  [ENG Kernel families: cooperative GEMV (decode),
 * batched GEMV twins (speculative verify); Fewer passes: y += W.x]
 *
 *   Y[:, j] = (accumulate ? Y[:, j] : 0) + W X[:, j],  j < ncols, ncols 1..8.
 * With accumulate the product is summed first and added to Y once.  Column j
 * of an ncols-wide call is bitwise equal to a 1-column call on X[:, j] (the
 * per-row reduction order depends only on rows and cols).
 * qs / d: the packed streams of one matrix (qg_repack with n_mat = 1).
 * Y must not overlap X.
 * ------------------------------------------------------------------------ */
size_t qg_gemv_ws_bytes(int64_t rows, int64_t cols);

int qgemv_q4_0(const void *qs, const void *d, int64_t rows, int64_t cols,
               const float *X, int64_t ldx, int32_t ncols, float *Y, int64_t ldy,
               int32_t accumulate, void *ws, size_t ws_bytes, void *stream);

int qgemv_q8_0(const void *qs, const void *d, int64_t rows, int64_t cols,
               const float *X, int64_t ldx, int32_t ncols, float *Y, int64_t ldy,
               int32_t accumulate, void *ws, size_t ws_bytes, void *stream);

/* ------------------------------------------------------------------------
 * 16-column prefill GEMM  [ENG Kernel families: prefill GEMM; Batching and
 * prefill: row-stationary GEMM at 16 columns, split-K pinned per shape;
 * ARCH Prefill: each weight block read once for all 16 columns]
 *
 *   Y = (accumulate ? Y : 0) + W X,  X cols x 16, Y rows x 16.
 * Runs on the matrix cores (f16 operands after exact dequantisation, f32
 * accumulate; the block scale is applied in f32 to each block's product).
 * ------------------------------------------------------------------------ */
size_t qg_gemm16_ws_bytes(int qtype, int64_t rows, int64_t cols);

int qgemm16(int qtype, const void *qs, const void *d, int64_t rows, int64_t cols,
            const float *X, int64_t ldx, float *Y, int64_t ldy, int32_t accumulate,
            void *ws, size_t ws_bytes, void *stream);

/* ------------------------------------------------------------------------
 * A prefill pass over several matrices in one launch  [ARCH Prefill: the
 * prompt runs 16 columns per pass through every weight matrix; ENG Batching
 * and prefill: the 16-column GEMM; ENG Fewer passes: fewer launches]
 *
 *   for each problem i < n:  Y_i = (accumulate_i ? Y_i : 0) + W_i X_i,
 *   X_i cols_i x 16, Y_i rows_i x 16, each as qgemm16 (same checks).
 * The launch picks each problem's K split for the pass as a whole: K cut
 * into segments about as long as the shortest K among the problems (at
 * least one), all counts then multiplied by the smallest factor that gives
 * at least two work units per CU of the current device; segments at least
 * 4 tile columns long, at most 255 of them.  qg_gemm16_batch_splits reports
 * these counts (host only); Y_i is bitwise equal to qgemm16 on problem i
 * with that split pinned (qg_plan_set(QG_OP_GEMV, qtype, rows, cols, 16,
 * QG_PLAN_SPLIT(splits[i]))), and the same on every call.  The problems run
 * concurrently in one launch, so no Y_i may overlap any X_j or any other
 * Y_j (QG_EINVAL).  1 <= n <= QG_BATCH_MAX (else QG_ESHAPE); Q4_0 and Q8_0
 * problems may be mixed.  `p` is a HOST array of n descriptors; the library
 * copies it into the launch.  Errors of the split query: those of the
 * descriptors (as qgemm16_batch), QG_EINVAL for a null `splits`.
 * ------------------------------------------------------------------------ */
#define QG_BATCH_MAX 8

typedef struct {
  int32_t qtype;       /* QG_Q4_0 or QG_Q8_0 */
  int32_t accumulate;  /* 0: Y = W X;  1: Y += W X */
  const void *qs;      /* packed weights of one matrix (qg_repack, n_mat = 1) */
  const void *d;
  int64_t rows, cols;
  const float *X;      /* cols x 16, column-major, leading dimension ldx */
  int64_t ldx;
  float *Y;            /* rows x 16, column-major, leading dimension ldy */
  int64_t ldy;
} qg_gemm16_problem;

size_t qg_gemm16_batch_ws_bytes(const qg_gemm16_problem *p, int32_t n);

int qg_gemm16_batch_splits(const qg_gemm16_problem *p, int32_t n, int32_t *splits);

int qgemm16_batch(const qg_gemm16_problem *p, int32_t n, void *ws, size_t ws_bytes,
                  void *stream);

/* ------------------------------------------------------------------------
 * Fused gate/up + SiLU  [ENG Kernel families: fused gate/up, both FFN
 * projections in one sweep, SiLU applied before writing]
 *
 *   H[:, j] = silu(Wg X[:, j]) * (Wu X[:, j]),  silu(g) = g / (1 + e^-g),
 *   ncols 1..8.  Wg and Wu have the same rows x cols.  H rows x ncols.
 * ------------------------------------------------------------------------ */
size_t qg_gateup_ws_bytes(int64_t rows, int64_t cols);

int gateup_silu(int qtype, const void *g_qs, const void *g_d, const void *u_qs,
                const void *u_d, int64_t rows, int64_t cols, const float *X,
                int64_t ldx, int32_t ncols, float *H, int64_t ldh,
                void *ws, size_t ws_bytes, void *stream);

/* ------------------------------------------------------------------------
 * Requantisation to Q8_0 at load  [ENG What it runs: the Q4_1 / Q5_0 /
 * K-quant tensors of the public MoE file are requantized to Q8_0 on the way
 * to the GPU; ARCH where the weights live: converted once and kept]
 *
 *   Each run of 32 values of src (in order) becomes one Q8_0 block of dst:
 *   with v the run's float32 values, d = max|v| / 127 rounded to float32,
 *   r = 1 / d rounded to float32 (0 when d is 0), q_j = v_j * r rounded to
 *   float32 and then to the nearest integer, halves away from zero; d is
 *   stored as binary16 (nearest even).
 *   Source layouts, the public GGUF ones (values as float32, one rounding):
 *     Q4_1  20 B / 32 values: f16 d, f16 m, 16 nibble bytes; v = w d + m.
 *     Q5_0  22 B / 32: f16 d, 32 high bits, nibbles; v = (w - 16) d.
 *     Q5_1  24 B / 32: d, m, high bits, nibbles; v = w d + m.
 *     Q4_K 144 B / 256: f16 d, f16 dmin, 12 bytes of 6-bit scales and mins
 *           of 8 sub-blocks, 128 nibble bytes; v = (d sc) w - dmin m.
 *     Q5_K 176 B / 256: Q4_K plus 32 bytes of fifth bits.
 *     Q6_K 210 B / 256: 128 bytes low nibbles, 64 bytes 2-bit tops, 16 int8
 *           scales, f16 d; v = (d sc) (w - 32).
 *   n_blocks counts source blocks; dst receives n_blocks * 34 bytes (Q4_1,
 *   Q5_0, Q5_1) or n_blocks * 8 * 34 bytes (K-quants) of canonical Q8_0
 *   blocks, ready for qg_repack(QG_Q8_0, ...).  src and dst: device memory,
 *   2-byte aligned, not overlapping.  Errors: QG_EINVAL (source type, null
 *   pointer, overlap), QG_ESHAPE (n_blocks < 1 or more than 2^36 output
 *   blocks), QG_EALIGN, QG_EHIP.  Asynchronous on `stream`; the bytes are a
 *   function of the source bytes alone.
 * ------------------------------------------------------------------------ */
int qg_requant_q8_0(int src_type, int64_t n_blocks, const void *src, void *dst, void *stream);

/* ------------------------------------------------------------------------
 * RMSNorm prologue  [TJS Llama-style differences: RMSNorm takes the root
 * mean square, no mean subtracted; ENG: the norm fused ahead of the router
 * (kept, +4-5% decode) and into the GEMV (0.91x on Metal: to be measured)]
 *
 *   n(X)[k, j] = X[k, j] * gamma[k] / sqrt(mean_k X[k, j]^2 + eps)
 *
 * gateup_silu_rmsnorm: H = gateup_silu of n(X), with the norm folded into
 * the call: each workgroup stages X * gamma and multiplies both products of
 * a column by that column's 1 / rms (the products are linear in X).  gamma:
 * cols floats, device, 16-byte aligned; eps >= 0 and finite, else QG_EINVAL.
 * Shapes whose K segments do not each stage all of K (cols > 5120 with more
 * than one segment) return QG_EUNSUPPORTED.  Workspace: qg_gateup_ws_bytes.
 * Column j is bitwise equal to a 1-column call on column j.
 *
 * qg_rmsnorm: Y = n(X) on its own (a workgroup per column); Y may be X itself
 * (same ld), not a shifted overlap.  Its 1 / rms has the same bits as the
 * fused form's (the squares are summed in the same order).
 * ------------------------------------------------------------------------ */
int gateup_silu_rmsnorm(int qtype, const void *g_qs, const void *g_d, const void *u_qs,
                        const void *u_d, int64_t rows, int64_t cols, const float *X,
                        int64_t ldx, int32_t ncols, const float *gamma, float eps, float *H,
                        int64_t ldh, void *ws, size_t ws_bytes, void *stream);

int qg_rmsnorm(const float *X, int64_t ldx, int64_t cols, int32_t ncols, const float *gamma,
               float eps, float *Y, int64_t ldy, void *stream);

/* ------------------------------------------------------------------------
 * LM head + greedy argmax  [ARCH One token, end to end: head over the whole
 * vocabulary, greedy sampling on the GPU; ENG Fewer passes: GPU argmax,
 * lowest-index tie-breaking; ENG Speculation: drafts over a row prefix]
 *
 *   *out_idx = the lowest r < n_rows maximising (W x)[r];  *out_val = that
 *   maximum (out_val may be NULL).  Only rows < n_rows are read (up to the
 *   16-row tile holding row n_rows - 1).  -0 equals +0; inputs are finite
 *   (a NaN logit ranks below every number).  The logits never reach memory.
 * ------------------------------------------------------------------------ */
size_t qg_lmhead_ws_bytes(int64_t rows, int64_t cols);

int lmhead_argmax(int qtype, const void *qs, const void *d, int64_t rows, int64_t cols,
                  int64_t n_rows, const float *x, int32_t *out_idx, float *out_val,
                  void *ws, size_t ws_bytes, void *stream);

/* lmhead_argmax for callers that cannot allocate device memory (code under
 * HIP graph capture, serving loops or harnesses that forbid hipMalloc): the
 * same computation and the same result bits, with the workspace replaced
 * by a library-owned device array of QG_NOALLOC_SCRATCH_BYTES (2 MiB) per
 * GPU, held until the process ends.  No allocation happens in the call.
 * Each call first clears the array's counter words with a small kernel on
 * `stream` (graph-safe), then runs the head.  Every call on one GPU uses
 * that GPU's array: calls that may overlap in time on one GPU (different
 * streams, or threads) race and must not be issued.  Shapes whose built-in
 * launch needs more scratch than QG_NOALLOC_SCRATCH_BYTES (none up to
 * about three million rows) return QG_EUNSUPPORTED before anything is
 * launched; other errors as lmhead_argmax (QG_EHIP also if the array's
 * address cannot be obtained). */
int lmhead_argmax_noalloc(int qtype, const void *qs, const void *d, int64_t rows,
                          int64_t cols, int64_t n_rows, const float *x, int32_t *out_idx,
                          float *out_val, void *stream);

/* ------------------------------------------------------------------------
 * LM head + top-k candidates  [ARCH One token, end to end: greedy and top-k
 * sampling on the GPU, a few bytes read back instead of the 1 MB logits;
 * ENG Sampling, Fewer passes: GPU top-k, lowest-index ties; TJS Reduce
 * sampling on the GPU: a small top-k on the GPU, the host finishes the
 * draw from the candidates]
 *
 *   out_idx[j], out_val[j] (j < k): the k largest logits (W x)[r] over
 *   r < n_rows, ordered by value descending, then row ascending.  Rows are
 *   read as for lmhead_argmax; the logits never reach memory (each row
 *   group keeps its k best, the last workgroup to finish merges them).
 *   1 <= k <= min(QG_TOPK_MAX, n_rows), else QG_ESHAPE.  out_idx: k int32,
 *   out_val: k floats or NULL, both device memory, 4-byte aligned.
 * ------------------------------------------------------------------------ */
size_t qg_lmhead_topk_ws_bytes(int64_t rows, int64_t cols, int32_t k);

int lmhead_topk(int qtype, const void *qs, const void *d, int64_t rows, int64_t cols,
                int64_t n_rows, const float *x, int32_t k, int32_t *out_idx, float *out_val,
                void *ws, size_t ws_bytes, void *stream);

/* ------------------------------------------------------------------------
 * MoE FFN  [ENG What it runs: 256 experts, 8 active per token, plus a shared
 * expert; Kernel families: router, top-k, expert gate/up and down, weighted
 * combine, all on the GPU, no readback; MOE: experts stacked by role]
 *
 * Per token t (column t of X, hidden rows):
 *   l = R x_t (f32 router, n_expert x hidden, row-major, 16-byte aligned);
 *   sel = the top_k experts by (l descending, index ascending);
 *   p = softmax(l[sel]) if normalize_topk, else softmax(l)[sel];
 *   Y[:, t] += sum_k p_k Down_e(silu(Gate_e x_t) * Up_e x_t)     (e = sel_k)
 *            + SharedDown(silu(SharedGate x_t) * SharedUp x_t)   (if sh_ffn > 0)
 * The expert sum is formed in f32 in k order, the shared expert added last,
 * then the total is added to Y once.  Gate and up stacks: qg_repack with
 * n_mat = n_expert, rows = ffn, cols = hidden; down stack: n_mat = n_expert,
 * rows = hidden, cols = ffn; the shared matrices: n_mat = 1, ffn -> sh_ffn.
 * The gate and up matrices of each selected expert are read once for all
 * tokens routed to it (up to 4 tokens per pass); the down matrices once per
 * (token, rank) when ffn is at most a few thousand (the combine then runs
 * in on-chip memory), else once for all tokens routed to the expert.
 * topk_idx / topk_w (ntok x top_k, row-major, may be NULL) receive sel and p.
 * Limits: ntok 1..16 per call, top_k 1..8, n_expert 1..1024,
 * hidden and ffn multiples of 128 and at most 16384.
 * ------------------------------------------------------------------------ */
typedef struct {
  int64_t hidden, ffn;
  int32_t n_expert, top_k, normalize_topk;
  int32_t qtype;
  const float *router;
  const void *gate_qs, *up_qs, *down_qs;
  const void *gate_d, *up_d, *down_d;
  int64_t sh_ffn; /* 0 = no shared expert */
  const void *sh_gate_qs, *sh_up_qs, *sh_down_qs;
  const void *sh_gate_d, *sh_up_d, *sh_down_d;
  /* RMSNorm ahead of router and experts (ENG: norm fused with the router);
   * NULL = none.  hidden floats, 16-byte aligned; the router and every
   * expert read X * norm_weight / sqrt(mean(X^2) + norm_eps), the residual
   * Y is not normalised.  hidden <= 5120 (every expert unit stages all of
   * the hidden range), else QG_EUNSUPPORTED; norm_eps >= 0 and finite. */
  const float *norm_weight;
  float norm_eps;
} qg_moe;

size_t qg_moe_ws_bytes(const qg_moe *m, int32_t ntok);

int moe_ffn(const qg_moe *m, const float *X, int64_t ldx, int32_t ntok, float *Y,
            int64_t ldy, int32_t *topk_idx, float *topk_w, void *ws, size_t ws_bytes,
            void *stream);

/* ------------------------------------------------------------------------
 * Launch plans and their tuning  [ENG What each trick bought, the reading-
 * weights table: a device autotune of workgroup size and rows per
 * workgroup, about a second at load, with a 3% noise margin; ARCH Engine,
 * its file table: an autotune module beside the kernels]
 *
 * A plan fixes how a product call is laid out on the GPU: 0 = the built-in
 * choice; 1..16 = that many waves (row tiles) per workgroup, K segments
 * reduced across workgroups; QG_PLAN_SW = the K segments as waves of one
 * workgroup.  These never change what is summed: the K segments and their
 * order are a function of the shape, so every such plan gives the same
 * bits.  A plan may add QG_PLAN_SPLIT(s), s = 1..255 K segments instead of
 * the shape's own (the split-K of the pages' autotune): a different
 * summation order, so results that differ by rounding (within the products'
 * float tolerance), the same bits on every call while the entry stands
 * (pin it with qg_plan_set for runs that must repeat); a split needing
 * more workspace than the call brings is not usable by that call (the
 * *_ws_bytes queries leave room for twice the shape's own split).  Plans
 * live in a per-process table keyed by (current device, op,
 * qtype, rows, cols, ncols); every later call of that op on that shape and
 * column count uses the entry, or the built-in choice where the entry does
 * not fit the call (checked before anything is launched).  Ops:
 *   QG_OP_GEMV    qgemv_q4_0 / qgemv_q8_0 (ncols 1..8; store and
 *                 accumulate share the entry) and qgemm16 (ncols 16:
 *                 plans 8..16 only)
 *   QG_OP_GATEUP  gateup_silu and gateup_silu_rmsnorm
 *   QG_OP_LMHEAD  lmhead_argmax and lmhead_topk (ncols 1)
 * The MoE layer and the grouped prefill pass keep their own launch shapes.
 *
 * qg_tune_*: the arguments of the call they tune (same checks, same errors)
 * and flags; each candidate plan (built-in, 4, 8, 12, 16 waves, QG_PLAN_SW;
 * 8, 12, 16 for 16 columns; with flags & QG_TUNE_SPLIT each of these also at
 * half, one less, one more and twice the shape's own K segments) runs 1 + 10 times on the
 * caller's stream in three rounds, timed with HIP events (blocks the host
 * until done); the fastest stays only if more than 3% faster than the
 * built-in choice, else the entry is 0. Without QG_TUNE_SPLIT the tuned calls
 * keep their bits. The outputs are overwritten (qg_tune_gemv stores W X, it
 * never accumulates) and end equal to the tuned call's. *plan (may be NULL)
 * receives the entry. Calls racing with a tuning call on another thread see
 * the old or the new entry.
 * qg_plan_set pins an entry (QG_EINVAL for an op or plan outside the
 * above); a plan | QG_PLAN_STRICT makes the calls that cannot use it fail
 * (QG_EUNSUPPORTED; QG_EWORKSPACE for a split their workspace cannot hold)
 * instead of taking the built-in choice.  qg_plan_get
 * reads an entry (0 when none), qg_plan_reset empties the table.
 * ------------------------------------------------------------------------ */
#define QG_OP_GEMV 0
#define QG_OP_GATEUP 1
#define QG_OP_LMHEAD 2
#define QG_PLAN_SW 0x100
#define QG_PLAN_STRICT 0x200
#define QG_PLAN_SPLIT(s) ((int32_t)(s) << 12)
#define QG_TUNE_SPLIT 1

int qg_tune_gemv(int qtype, const void *qs, const void *d, int64_t rows, int64_t cols,
                 const float *X, int64_t ldx, int32_t ncols, float *Y, int64_t ldy,
                 void *ws, size_t ws_bytes, void *stream, int32_t flags, int32_t *plan);

int qg_tune_gateup(int qtype, const void *g_qs, const void *g_d, const void *u_qs,
                   const void *u_d, int64_t rows, int64_t cols, const float *X, int64_t ldx,
                   int32_t ncols, float *H, int64_t ldh, void *ws, size_t ws_bytes,
                   void *stream, int32_t flags, int32_t *plan);

int qg_tune_lmhead(int qtype, const void *qs, const void *d, int64_t rows, int64_t cols,
                   int64_t n_rows, const float *x, int32_t *out_idx, float *out_val,
                   void *ws, size_t ws_bytes, void *stream, int32_t flags, int32_t *plan);

int qg_plan_set(int op, int qtype, int64_t rows, int64_t cols, int32_t ncols, int32_t plan);

int qg_plan_get(int op, int qtype, int64_t rows, int64_t cols, int32_t ncols, int32_t *plan);

void qg_plan_reset(void);

#ifdef __cplusplus
}
#endif
#endif /* QGEMM_H */
