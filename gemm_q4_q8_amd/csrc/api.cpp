// C-ABI entry points of libqgemm: argument checks (host only, before any HIP
// call) and dispatch to the kernel launchers.  What each call computes is
// stated, with its sources, in include/qgemm.h.
#include <stdio.h>
#include <string.h>

#include "internal.h"
#include "qgemm.h"

using namespace qg;

namespace qg {
static thread_local char g_last_hip[256] = "no HIP error recorded";
void record_hip_error(hipError_t e) {
  snprintf(g_last_hip, sizeof(g_last_hip), "%s: %s", hipGetErrorName(e), hipGetErrorString(e));
}
}  // namespace qg

namespace {

bool aligned(const void *p, size_t a) { return ((uintptr_t)p % a) == 0; }
bool qtype_ok(int q) { return q == QG_Q4_0 || q == QG_Q8_0; }

// Byte range [lo, hi) of a column-major f32 matrix.
struct Range {
  uintptr_t lo, hi;
};
Range span(const float *p, int64_t ld, int64_t len, int64_t ncols) {
  Range r;
  r.lo = (uintptr_t)p;
  r.hi = (uintptr_t)(p + (ncols - 1) * ld + len);
  return r;
}
bool overlap(Range a, Range b) { return a.lo < b.hi && b.lo < a.hi; }

int check_matrix(const void *qs, const void *d, int64_t rows, int64_t cols) {
  if (!qs || !d) return QG_EINVAL;
  if (rows <= 0 || cols <= 0 || cols % 32) return QG_ESHAPE;
  if (rows > (int64_t)1 << 31 || cols > (int64_t)1 << 24) return QG_EUNSUPPORTED;
  if (!aligned(qs, 16) || !aligned(d, 8)) return QG_EALIGN;
  return QG_OK;
}

int check_act(const float *X, int64_t ldx, int64_t len, int ncols) {
  if (!X) return QG_EINVAL;
  if (ldx < len) return QG_ESHAPE;
  if (!aligned(X, 16) || ldx % 4) return QG_EALIGN;
  (void)ncols;
  return QG_OK;
}

int check_out(const float *Y, int64_t ldy, int64_t len) {
  if (!Y) return QG_EINVAL;
  if (ldy < len) return QG_ESHAPE;
  if (!aligned(Y, 4)) return QG_EALIGN;
  return QG_OK;
}

int qmv_common(int qtype, const void *qs, const void *d, int64_t rows, int64_t cols, const float *X,
               int64_t ldx, int ncols, float *Y, int64_t ldy, int accumulate, void *ws, size_t ws_bytes,
               void *stream, bool gemm16, bool tune = false, int32_t flags = 0, int32_t *plan = nullptr) {
  if (!qtype_ok(qtype)) return QG_EINVAL;
  int st = check_matrix(qs, d, rows, cols);
  if (st) return st;
  if (!gemm16 && (ncols < 1 || ncols > 8)) return QG_ESHAPE;
  if ((st = check_act(X, ldx, cols, ncols))) return st;
  if ((st = check_out(Y, ldy, rows))) return st;
  if (overlap(span(X, ldx, cols, ncols), span(Y, ldy, rows, ncols))) return QG_EINVAL;
  const int slots = gemm16 ? gemm16_splits(rows, cols) : gemv_segments(rows, cols, 1, 8);
  if (!ws) return QG_EWORKSPACE;
  if (ws_bytes < qmv_ws_bytes(rows, cols, slots, 1, gemm16 ? 16 : 8, false)) return QG_EWORKSPACE;
  if (!aligned(ws, 256)) return QG_EALIGN;
  QmvCall c;
  memset(&c, 0, sizeof(c));
  c.qtype = qtype;
  c.nmat = 1;
  c.qs[0] = c.qs[1] = qs;
  c.d[0] = c.d[1] = d;
  c.rows = rows;
  c.cols = cols;
  c.n_rows = rows;
  c.X = X;
  c.ldx = ldx;
  c.ncols = ncols;
  c.Y = Y;
  c.ldy = ldy;
  c.epi = accumulate ? EPI_ACC : EPI_STORE;
  c.ws = ws;
  c.ws_bytes = ws_bytes;
  c.stream = (hipStream_t)stream;
  return tune ? tune_call(c, flags, plan) : launch_qmv(c);
}

}  // namespace

extern "C" {

const char *qg_strerror(int status) {
  switch (status) {
    case QG_OK: return "ok";
    case QG_EINVAL: return "invalid argument (null pointer, bad type id, or output overlapping input)";
    case QG_ESHAPE: return "invalid shape (cols % 32, non-positive size, ncols, n_rows or top_k out of range)";
    case QG_EALIGN: return "misaligned pointer or leading dimension";
    case QG_EUNSUPPORTED: return "request outside what this build supports";
    case QG_EWORKSPACE: return "workspace missing or too small";
    case QG_EHIP: return "HIP launch error";
  }
  return "unknown status";
}

const char *qg_last_hip_error(void) { return qg::g_last_hip; }

int qg_packed_bytes(int qtype, int64_t n_mat, int64_t rows, int64_t cols, size_t *qs_bytes,
                    size_t *d_bytes) {
  if (!qtype_ok(qtype) || !qs_bytes || !d_bytes) return QG_EINVAL;
  if (n_mat <= 0 || rows <= 0 || cols <= 0 || cols % 32) return QG_ESHAPE;
  const int64_t NT = (rows + 15) / 16, KT = (cols / 32 + 3) / 4;
  const int64_t tiles = n_mat * NT * KT;
  *qs_bytes = (size_t)tiles * (qtype == QG_Q4_0 ? 1024 : 2048);
  *d_bytes = (size_t)tiles * 128;
  return QG_OK;
}

int qg_repack(int qtype, int64_t n_mat, int64_t rows, int64_t cols, const void *blocks, void *qs,
              void *d, void *stream) {
  size_t qb, db;
  int st = qg_packed_bytes(qtype, n_mat, rows, cols, &qb, &db);
  if (st) return st;
  if (!blocks || !qs || !d) return QG_EINVAL;
  if (!aligned(blocks, 2) || !aligned(qs, 16) || !aligned(d, 8)) return QG_EALIGN;
  const size_t in_bytes = (size_t)n_mat * rows * (cols / 32) * (qtype == QG_Q4_0 ? 18 : 34);
  const Range in{(uintptr_t)blocks, (uintptr_t)blocks + in_bytes};
  const Range oq{(uintptr_t)qs, (uintptr_t)qs + qb};
  const Range od{(uintptr_t)d, (uintptr_t)d + db};
  if (overlap(in, oq) || overlap(in, od) || overlap(oq, od)) return QG_EINVAL;
  return launch_repack(qtype, n_mat, rows, cols, blocks, qs, d, (hipStream_t)stream);
}

int qg_requant_q8_0(int src_type, int64_t n_blocks, const void *src, void *dst, void *stream) {
  int bs, runs = 1;
  switch (src_type) {
    case QG_Q4_1: bs = 20; break;
    case QG_Q5_0: bs = 22; break;
    case QG_Q5_1: bs = 24; break;
    case QG_Q4_K: bs = 144; runs = 8; break;
    case QG_Q5_K: bs = 176; runs = 8; break;
    case QG_Q6_K: bs = 210; runs = 8; break;
    default: return QG_EINVAL;
  }
  if (n_blocks < 1 || n_blocks > ((int64_t)1 << 36) / runs) return QG_ESHAPE;
  if (!src || !dst) return QG_EINVAL;
  if (!aligned(src, 2) || !aligned(dst, 2)) return QG_EALIGN;
  const Range in{(uintptr_t)src, (uintptr_t)src + (uintptr_t)(n_blocks * bs)};
  const Range out{(uintptr_t)dst, (uintptr_t)dst + (uintptr_t)(n_blocks * runs * 34)};
  if (overlap(in, out)) return QG_EINVAL;
  return launch_requant_q8_0(src_type, n_blocks, src, dst, stream);
}

// Workspace queries leave room for a plan's K split of up to twice the
// shape's own (the calls themselves need only the shape's own).
static int split_room(int S, int64_t cols) {
  const int64_t KT = (cols / 32 + 3) / 4;
  const int64_t r = 2 * (int64_t)S;
  return (int)(r < KT ? r : (KT > S ? KT : S));
}

// The least workspace each call takes (its shape's own split).
static size_t gateup_ws_min(int64_t rows, int64_t cols) {
  return qmv_ws_bytes(rows, cols, gemv_segments(rows, cols, 2, 8), 2, 8, false);
}
static size_t lmhead_ws_min(int64_t rows, int64_t cols, int32_t k) {
  return qmv_ws_bytes(rows, cols, gemv_segments(rows, cols, 1, 1), 1, 1, k == 0, k);
}

size_t qg_gemv_ws_bytes(int64_t rows, int64_t cols) {
  if (rows <= 0 || cols <= 0 || cols % 32) return 0;
  return qmv_ws_bytes(rows, cols, split_room(gemv_segments(rows, cols, 1, 8), cols), 1, 8, false);
}

size_t qg_gateup_ws_bytes(int64_t rows, int64_t cols) {
  if (rows <= 0 || cols <= 0 || cols % 32) return 0;
  return qmv_ws_bytes(rows, cols, split_room(gemv_segments(rows, cols, 2, 8), cols), 2, 8, false);
}

size_t qg_gemm16_ws_bytes(int qtype, int64_t rows, int64_t cols) {
  if (!qtype_ok(qtype) || rows <= 0 || cols <= 0 || cols % 32) return 0;
  return qmv_ws_bytes(rows, cols, split_room(gemm16_splits(rows, cols), cols), 1, 16, false);
}

size_t qg_lmhead_ws_bytes(int64_t rows, int64_t cols) {
  if (rows <= 0 || cols <= 0 || cols % 32) return 0;
  return qmv_ws_bytes(rows, cols, split_room(gemv_segments(rows, cols, 1, 1), cols), 1, 1, true);
}

size_t qg_lmhead_topk_ws_bytes(int64_t rows, int64_t cols, int32_t k) {
  if (rows <= 0 || cols <= 0 || cols % 32 || k < 1 || k > QG_TOPK_MAX) return 0;
  return qmv_ws_bytes(rows, cols, split_room(gemv_segments(rows, cols, 1, 1), cols), 1, 1, false, k);
}

int qgemv_q4_0(const void *qs, const void *d, int64_t rows, int64_t cols, const float *X, int64_t ldx,
               int32_t ncols, float *Y, int64_t ldy, int32_t accumulate, void *ws, size_t ws_bytes,
               void *stream) {
  return qmv_common(QG_Q4_0, qs, d, rows, cols, X, ldx, ncols, Y, ldy, accumulate, ws, ws_bytes, stream,
                    false);
}

int qgemv_q8_0(const void *qs, const void *d, int64_t rows, int64_t cols, const float *X, int64_t ldx,
               int32_t ncols, float *Y, int64_t ldy, int32_t accumulate, void *ws, size_t ws_bytes,
               void *stream) {
  return qmv_common(QG_Q8_0, qs, d, rows, cols, X, ldx, ncols, Y, ldy, accumulate, ws, ws_bytes, stream,
                    false);
}

int qgemm16(int qtype, const void *qs, const void *d, int64_t rows, int64_t cols, const float *X,
            int64_t ldx, float *Y, int64_t ldy, int32_t accumulate, void *ws, size_t ws_bytes,
            void *stream) {
  return qmv_common(qtype, qs, d, rows, cols, X, ldx, 16, Y, ldy, accumulate, ws, ws_bytes, stream, true);
}

static int check_batch(const qg_gemm16_problem *p, int32_t n) {
  if (!p) return QG_EINVAL;
  if (n < 1 || n > QG_BATCH_MAX) return QG_ESHAPE;
  for (int i = 0; i < n; ++i) {
    if (!qtype_ok(p[i].qtype)) return QG_EINVAL;
    int st = check_matrix(p[i].qs, p[i].d, p[i].rows, p[i].cols);
    if (st) return st;
    if ((st = check_act(p[i].X, p[i].ldx, p[i].cols, 16))) return st;
    if ((st = check_out(p[i].Y, p[i].ldy, p[i].rows))) return st;
  }
  // the problems run concurrently: no output may overlap any input or
  // another output
  for (int i = 0; i < n; ++i) {
    const Range yi = span(p[i].Y, p[i].ldy, p[i].rows, 16);
    for (int j = 0; j < n; ++j) {
      if (overlap(yi, span(p[j].X, p[j].ldx, p[j].cols, 16))) return QG_EINVAL;
      if (j != i && overlap(yi, span(p[j].Y, p[j].ldy, p[j].rows, 16))) return QG_EINVAL;
    }
  }
  return QG_OK;
}

size_t qg_gemm16_batch_ws_bytes(const qg_gemm16_problem *p, int32_t n) {
  if (check_batch(p, n)) return 0;
  return gemm16_batch_ws_bytes(p, n);
}

int qg_gemm16_batch_splits(const qg_gemm16_problem *p, int32_t n, int32_t *splits) {
  if (!splits) return QG_EINVAL;
  int st = check_batch(p, n);
  if (st) return st;
  int S[QG_BATCH_MAX];
  gemm16_batch_splits(p, n, S);
  for (int i = 0; i < n; ++i) splits[i] = S[i];
  return QG_OK;
}

int qgemm16_batch(const qg_gemm16_problem *p, int32_t n, void *ws, size_t ws_bytes, void *stream) {
  int st = check_batch(p, n);
  if (st) return st;
  const size_t need = gemm16_batch_ws_bytes(p, n);
  if (need == 0) return QG_EUNSUPPORTED;
  if (!ws || ws_bytes < need) return QG_EWORKSPACE;
  if (!aligned(ws, 256)) return QG_EALIGN;
  return launch_gemm16_batch(p, n, ws, ws_bytes, (hipStream_t)stream);
}

static int gateup_common(int qtype, const void *g_qs, const void *g_d, const void *u_qs, const void *u_d,
                         int64_t rows, int64_t cols, const float *X, int64_t ldx, int32_t ncols,
                         const float *gamma, float eps, float *H, int64_t ldh, void *ws, size_t ws_bytes,
                         void *stream, bool tune = false, int32_t flags = 0, int32_t *plan = nullptr);

int gateup_silu(int qtype, const void *g_qs, const void *g_d, const void *u_qs, const void *u_d,
                int64_t rows, int64_t cols, const float *X, int64_t ldx, int32_t ncols, float *H,
                int64_t ldh, void *ws, size_t ws_bytes, void *stream) {
  return gateup_common(qtype, g_qs, g_d, u_qs, u_d, rows, cols, X, ldx, ncols, nullptr, 0.0f, H, ldh, ws,
                       ws_bytes, stream);
}

int gateup_silu_rmsnorm(int qtype, const void *g_qs, const void *g_d, const void *u_qs, const void *u_d,
                        int64_t rows, int64_t cols, const float *X, int64_t ldx, int32_t ncols,
                        const float *gamma, float eps, float *H, int64_t ldh, void *ws, size_t ws_bytes,
                        void *stream) {
  if (!gamma) return QG_EINVAL;
  if (!aligned(gamma, 16)) return QG_EALIGN;
  if (!(eps >= 0.0f) || eps > 3.0e38f) return QG_EINVAL;  // also rejects NaN
  return gateup_common(qtype, g_qs, g_d, u_qs, u_d, rows, cols, X, ldx, ncols, gamma, eps, H, ldh, ws,
                       ws_bytes, stream);
}

int qg_rmsnorm(const float *X, int64_t ldx, int64_t cols, int32_t ncols, const float *gamma, float eps, float *Y,
               int64_t ldy, void *stream) {
  if (!X || !Y || !gamma) return QG_EINVAL;
  if (cols < 1 || ncols < 1 || ldx < cols || ldy < cols) return QG_ESHAPE;
  if (!aligned(X, 4) || !aligned(Y, 4) || !aligned(gamma, 4)) return QG_EALIGN;
  if (!(eps >= 0.0f) || eps > 3.0e38f) return QG_EINVAL;
  // y may be x itself (same columns), not a shifted copy of it
  if (Y != X && overlap(span(X, ldx, cols, ncols), span(Y, ldy, cols, ncols))) return QG_EINVAL;
  if (Y == X && ldy != ldx) return QG_EINVAL;
  return launch_rmsnorm(X, ldx, cols, ncols, gamma, eps, Y, ldy, stream);
}

static int gateup_common(int qtype, const void *g_qs, const void *g_d, const void *u_qs, const void *u_d,
                         int64_t rows, int64_t cols, const float *X, int64_t ldx, int32_t ncols,
                         const float *gamma, float eps, float *H, int64_t ldh, void *ws, size_t ws_bytes,
                         void *stream, bool tune, int32_t flags, int32_t *plan) {
  if (!qtype_ok(qtype)) return QG_EINVAL;
  int st = check_matrix(g_qs, g_d, rows, cols);
  if (st) return st;
  if ((st = check_matrix(u_qs, u_d, rows, cols))) return st;
  if (ncols < 1 || ncols > 8) return QG_ESHAPE;
  if ((st = check_act(X, ldx, cols, ncols))) return st;
  if ((st = check_out(H, ldh, rows))) return st;
  if (overlap(span(X, ldx, cols, ncols), span(H, ldh, rows, ncols))) return QG_EINVAL;
  if (!ws || ws_bytes < gateup_ws_min(rows, cols)) return QG_EWORKSPACE;
  if (!aligned(ws, 256)) return QG_EALIGN;
  QmvCall c;
  memset(&c, 0, sizeof(c));
  c.qtype = qtype;
  c.nmat = 2;
  c.qs[0] = g_qs;
  c.qs[1] = u_qs;
  c.d[0] = g_d;
  c.d[1] = u_d;
  c.rows = rows;
  c.cols = cols;
  c.n_rows = rows;
  c.X = X;
  c.ldx = ldx;
  c.ncols = ncols;
  c.Y = H;
  c.ldy = ldh;
  c.epi = EPI_SILU;
  c.gamma = gamma;
  c.norm_eps = eps;
  c.ws = ws;
  c.ws_bytes = ws_bytes;
  c.stream = (hipStream_t)stream;
  return tune ? tune_call(c, flags, plan) : launch_qmv(c);
}

static int lmhead_argmax_common(int qtype, const void *qs, const void *d, int64_t rows, int64_t cols,
                                int64_t n_rows, const float *x, int32_t *out_idx, float *out_val, void *ws,
                                size_t ws_bytes, void *stream, bool tune, int32_t flags, int32_t *plan) {
  if (!qtype_ok(qtype)) return QG_EINVAL;
  int st = check_matrix(qs, d, rows, cols);
  if (st) return st;
  if (n_rows < 1 || n_rows > rows) return QG_ESHAPE;
  if ((st = check_act(x, cols, cols, 1))) return st;
  if (!out_idx) return QG_EINVAL;
  if (!aligned(out_idx, 4) || (out_val && !aligned(out_val, 4))) return QG_EALIGN;
  if (!ws || ws_bytes < lmhead_ws_min(rows, cols, 0)) return QG_EWORKSPACE;
  if (!aligned(ws, 256)) return QG_EALIGN;
  QmvCall c;
  memset(&c, 0, sizeof(c));
  c.qtype = qtype;
  c.nmat = 1;
  c.qs[0] = c.qs[1] = qs;
  c.d[0] = c.d[1] = d;
  c.rows = rows;
  c.cols = cols;
  c.n_rows = n_rows;
  c.X = x;
  c.ldx = cols;
  c.ncols = 1;
  c.Y = nullptr;
  c.ldy = 0;
  c.epi = EPI_ARGMAX;
  c.out_idx = out_idx;
  c.out_val = out_val;
  c.ws = ws;
  c.ws_bytes = ws_bytes;
  c.stream = (hipStream_t)stream;
  return tune ? tune_call(c, flags, plan) : launch_qmv(c);
}

int lmhead_argmax(int qtype, const void *qs, const void *d, int64_t rows, int64_t cols, int64_t n_rows,
                  const float *x, int32_t *out_idx, float *out_val, void *ws, size_t ws_bytes,
                  void *stream) {
  return lmhead_argmax_common(qtype, qs, d, rows, cols, n_rows, x, out_idx, out_val, ws, ws_bytes, stream,
                              false, 0, nullptr);
}

int lmhead_argmax_noalloc(int qtype, const void *qs, const void *d, int64_t rows, int64_t cols, int64_t n_rows,
                          const float *x, int32_t *out_idx, float *out_val, void *stream) {
  // the checks lmhead_argmax makes before its workspace, so that a bad call
  // touches nothing
  if (!qtype_ok(qtype)) return QG_EINVAL;
  int st = check_matrix(qs, d, rows, cols);
  if (st) return st;
  if (n_rows < 1 || n_rows > rows) return QG_ESHAPE;
  if ((st = check_act(x, cols, cols, 1))) return st;
  if (!out_idx) return QG_EINVAL;
  if (!aligned(out_idx, 4) || (out_val && !aligned(out_val, 4))) return QG_EALIGN;
  if (lmhead_ws_min(rows, cols, 0) > QG_NOALLOC_SCRATCH_BYTES) return QG_EUNSUPPORTED;
  void *ws = nullptr;
  if ((st = noalloc_scratch(&ws))) return st;
  // the counters the head uses (word 0 and one per row group) start at zero
  const int64_t words = (n_rows + 15) / 16 + 1;
  if ((st = launch_clear_words(ws, (int)(words < (int64_t)WS_SYNC_WORDS ? words : (int64_t)WS_SYNC_WORDS),
                               (hipStream_t)stream)))
    return st;
  return lmhead_argmax_common(qtype, qs, d, rows, cols, n_rows, x, out_idx, out_val, ws, QG_NOALLOC_SCRATCH_BYTES,
                              stream, false, 0, nullptr);
}

int qg_tune_lmhead(int qtype, const void *qs, const void *d, int64_t rows, int64_t cols, int64_t n_rows,
                   const float *x, int32_t *out_idx, float *out_val, void *ws, size_t ws_bytes, void *stream,
                   int32_t flags, int32_t *plan) {
  return lmhead_argmax_common(qtype, qs, d, rows, cols, n_rows, x, out_idx, out_val, ws, ws_bytes, stream,
                              true, flags, plan);
}

int qg_tune_gemv(int qtype, const void *qs, const void *d, int64_t rows, int64_t cols, const float *X,
                 int64_t ldx, int32_t ncols, float *Y, int64_t ldy, void *ws, size_t ws_bytes, void *stream,
                 int32_t flags, int32_t *plan) {
  return qmv_common(qtype, qs, d, rows, cols, X, ldx, ncols, Y, ldy, 0, ws, ws_bytes, stream, ncols == 16,
                    true, flags, plan);
}

int qg_tune_gateup(int qtype, const void *g_qs, const void *g_d, const void *u_qs, const void *u_d,
                   int64_t rows, int64_t cols, const float *X, int64_t ldx, int32_t ncols, float *H,
                   int64_t ldh, void *ws, size_t ws_bytes, void *stream, int32_t flags, int32_t *plan) {
  return gateup_common(qtype, g_qs, g_d, u_qs, u_d, rows, cols, X, ldx, ncols, nullptr, 0.0f, H, ldh, ws,
                       ws_bytes, stream, true, flags, plan);
}

int lmhead_topk(int qtype, const void *qs, const void *d, int64_t rows, int64_t cols, int64_t n_rows,
                const float *x, int32_t k, int32_t *out_idx, float *out_val, void *ws, size_t ws_bytes,
                void *stream) {
  if (!qtype_ok(qtype)) return QG_EINVAL;
  int st = check_matrix(qs, d, rows, cols);
  if (st) return st;
  if (n_rows < 1 || n_rows > rows) return QG_ESHAPE;
  if (k < 1 || k > QG_TOPK_MAX || k > n_rows) return QG_ESHAPE;
  if ((st = check_act(x, cols, cols, 1))) return st;
  if (!out_idx) return QG_EINVAL;
  if (!aligned(out_idx, 4) || (out_val && !aligned(out_val, 4))) return QG_EALIGN;
  if (!ws || ws_bytes < lmhead_ws_min(rows, cols, k)) return QG_EWORKSPACE;
  if (!aligned(ws, 256)) return QG_EALIGN;
  QmvCall c;
  memset(&c, 0, sizeof(c));
  c.qtype = qtype;
  c.nmat = 1;
  c.qs[0] = c.qs[1] = qs;
  c.d[0] = c.d[1] = d;
  c.rows = rows;
  c.cols = cols;
  c.n_rows = n_rows;
  c.X = x;
  c.ldx = cols;
  c.ncols = 1;
  c.Y = nullptr;
  c.ldy = 0;
  c.epi = EPI_TOPK;
  c.out_idx = out_idx;
  c.out_val = out_val;
  c.topk = k;
  c.ws = ws;
  c.ws_bytes = ws_bytes;
  c.stream = (hipStream_t)stream;
  return launch_qmv(c);
}

static int check_moe(const qg_moe *m, int32_t ntok) {
  if (!m) return QG_EINVAL;
  if (!qtype_ok(m->qtype)) return QG_EINVAL;
  if (ntok < 1 || ntok > 16) return QG_ESHAPE;
  if (m->n_expert < 1 || m->n_expert > 1024) return QG_ESHAPE;
  if (m->top_k < 1 || m->top_k > 8 || m->top_k > m->n_expert) return QG_ESHAPE;
  if (m->hidden <= 0 || m->hidden % 128 || m->hidden > 16384) return QG_ESHAPE;
  if (m->ffn <= 0 || m->ffn % 128 || m->ffn > 16384) return QG_ESHAPE;
  if (m->sh_ffn < 0 || m->sh_ffn % 128 || m->sh_ffn > 16384) return QG_ESHAPE;
  if (!m->router || !m->gate_qs || !m->up_qs || !m->down_qs || !m->gate_d || !m->up_d || !m->down_d)
    return QG_EINVAL;
  if (!aligned(m->router, 16)) return QG_EALIGN;
  const void *q[3] = {m->gate_qs, m->up_qs, m->down_qs};
  const void *d[3] = {m->gate_d, m->up_d, m->down_d};
  for (int i = 0; i < 3; ++i)
    if (!aligned(q[i], 16) || !aligned(d[i], 8)) return QG_EALIGN;
  if (m->norm_weight) {
    if (!aligned(m->norm_weight, 16)) return QG_EALIGN;
    if (!(m->norm_eps >= 0.0f) || m->norm_eps > 3.0e38f) return QG_EINVAL;
    if (!dot_interleaved(m->hidden)) return QG_EUNSUPPORTED;
  }
  if (m->sh_ffn > 0) {
    const void *sq[3] = {m->sh_gate_qs, m->sh_up_qs, m->sh_down_qs};
    const void *sd[3] = {m->sh_gate_d, m->sh_up_d, m->sh_down_d};
    for (int i = 0; i < 3; ++i) {
      if (!sq[i] || !sd[i]) return QG_EINVAL;
      if (!aligned(sq[i], 16) || !aligned(sd[i], 8)) return QG_EALIGN;
    }
  }
  return QG_OK;
}

size_t qg_moe_ws_bytes(const qg_moe *m, int32_t ntok) {
  if (check_moe(m, ntok) != QG_OK) return 0;
  return moe_ws_bytes(m, ntok);
}

int qg_device_memory(int32_t device, int32_t *clock_khz, int32_t *bus_bits) {
  if (!clock_khz || !bus_bits) return QG_EINVAL;
  int c = 0, w = 0;
  hipError_t e = hipDeviceGetAttribute(&c, hipDeviceAttributeMemoryClockRate, device);
  if (e == hipSuccess) e = hipDeviceGetAttribute(&w, hipDeviceAttributeMemoryBusWidth, device);
  if (e != hipSuccess) {
    record_hip_error(e);
    return QG_EHIP;
  }
  *clock_khz = c;
  *bus_bits = w;
  return QG_OK;
}

int qg_read_probe(const void *p, size_t bytes, uint32_t *sink, void *stream) {
  if (!p || !sink) return QG_EINVAL;
  if (bytes == 0 || bytes % 16) return QG_ESHAPE;
  if (!aligned(p, 16) || !aligned(sink, 4)) return QG_EALIGN;
  return launch_read_probe(p, bytes, sink, stream);
}

int moe_ffn(const qg_moe *m, const float *X, int64_t ldx, int32_t ntok, float *Y, int64_t ldy,
            int32_t *topk_idx, float *topk_w, void *ws, size_t ws_bytes, void *stream) {
  int st = check_moe(m, ntok);
  if (st) return st;
  if ((st = check_act(X, ldx, m->hidden, ntok))) return st;
  if ((st = check_out(Y, ldy, m->hidden))) return st;
  if (overlap(span(X, ldx, m->hidden, ntok), span(Y, ldy, m->hidden, ntok))) return QG_EINVAL;
  if ((topk_idx && !aligned(topk_idx, 4)) || (topk_w && !aligned(topk_w, 4))) return QG_EALIGN;
  if (!ws || ws_bytes < moe_ws_bytes(m, ntok)) return QG_EWORKSPACE;
  if (!aligned(ws, 256)) return QG_EALIGN;
  MoeCall c;
  c.m = m;
  c.X = X;
  c.ldx = ldx;
  c.ntok = ntok;
  c.Y = Y;
  c.ldy = ldy;
  c.topk_idx = topk_idx;
  c.topk_w = topk_w;
  c.ws = ws;
  c.ws_bytes = ws_bytes;
  c.stream = (hipStream_t)stream;
  return launch_moe(c);
}

}  // extern "C"
