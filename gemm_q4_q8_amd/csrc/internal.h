// Host-side interfaces between the C-ABI layer (api.cpp) and the kernel
// launchers (*.hip).  Not installed; not part of the ABI.
#pragma once
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "qgemm.h"

namespace qg {

enum Epi { EPI_STORE = 0, EPI_ACC = 1, EPI_SILU = 2, EPI_ARGMAX = 3, EPI_TOPK = 4 };

// One launch of the tiled product kernel.
struct QmvCall {
  int qtype;
  int nmat;                 // 1, or 2 for gate/up
  const void *qs[2];
  const void *d[2];
  int64_t rows, cols;       // logical matrix size
  int64_t n_rows;           // rows actually produced (argmax: prefix), else rows
  const float *X;
  int64_t ldx;
  int ncols;                // 1..8 (dot path) or 16 (matrix-core path)
  float *Y;
  int64_t ldy;
  int epi;
  int32_t *out_idx;         // argmax (1), top-k (topk)
  float *out_val;
  int topk;                 // top-k: candidates wanted, 1..QG_TOPK_MAX
  const float *gamma;       // gate/up with an RMSNorm prologue: weights (cols), eps
  float norm_eps;
  void *ws;
  size_t ws_bytes;
  hipStream_t stream;
  int plan;                 // 0: the plan table's entry (else the built-in choice)
};

// Launch plans of the product calls: 0 = the built-in choice; 1..16 = that
// many waves per workgroup (segments across workgroups); QG_PLAN_SW = the
// K segments inside one workgroup.  No plan changes a result bit (the
// segments and their order are a function of the shape).  PLAN_FORCED
// marks a plan fixed by the caller (the tuner), bypassing the table.
constexpr int PLAN_W_MASK = 0x1F, PLAN_FORCED = 1 << 30;
constexpr int PLAN_S_SHIFT = 12, PLAN_S_MASK = 0xFF << PLAN_S_SHIFT;  // K segments (0: the shape's own)
int plan_lookup(const QmvCall &c);                // tune.cpp
int builtin_split(const QmvCall &c);              // the shape's own K segments for this call
int tune_call(QmvCall c, int32_t flags, int32_t *plan_out);  // times the plans, stores the winner

// K segments of the dot path: a function of the matrix shape (and of the
// widest batch the entry point takes) only, so that every column count gives
// the same per-row reduction order.
int gemv_segments(int64_t rows, int64_t cols, int nmat, int ncols_max);
// Compute units of the current device (queried once per device).
int device_cus();
// Interleaved K segments for a matrix of `cols` inputs (1..8 columns).
bool dot_interleaved(int64_t cols);
// K splits of the 16-column matrix-core path.
int gemm16_splits(int64_t rows, int64_t cols);

// Workspace: counters, argmax candidates, and `slots` partial sums per output.
// Every workspace starts with WS_SYNC_WORDS counters shared by all entry
// points.  They are zero between calls (each call's last workgroup resets
// what it used), and no call ever writes anything else there, so one
// workspace can serve calls of any shape in stream order.
constexpr size_t WS_SYNC_WORDS = QG_WS_SYNC_BYTES / 4;

size_t qmv_ws_bytes(int64_t rows, int64_t cols, int slots, int nmat, int ncols_max, bool argmax, int topk = 0);

int launch_qmv(const QmvCall &c);  // returns 0 or a QG_ status
// Several 16-column problems in one launch (0 from the size query: too many
// row groups for the counter words).
void gemm16_batch_splits(const qg_gemm16_problem *p, int n, int *S);
size_t gemm16_batch_ws_bytes(const qg_gemm16_problem *p, int n);
int launch_gemm16_batch(const qg_gemm16_problem *p, int n, void *ws, size_t ws_bytes, hipStream_t stream);
int launch_repack(int qtype, int64_t n_mat, int64_t rows, int64_t cols, const void *blocks,
                  void *qs, void *d, hipStream_t stream);

// Requantisation to Q8_0, the stand-alone RMSNorm, and the streaming-read
// probe (the bench's measured read ceiling).
int launch_requant_q8_0(int src_type, int64_t nb, const void *src, void *dst, void *stream);
int launch_rmsnorm(const float *X, int64_t ldx, int64_t cols, int ncols, const float *gamma, float eps, float *Y,
                   int64_t ldy, void *stream);
int launch_read_probe(const void *p, size_t bytes, uint32_t *sink, void *stream);

// The current device's library-owned scratch (its address, looked up once
// per device), and a graph-safe zero fill of n words.
int noalloc_scratch(void **out);
int launch_clear_words(void *p, int n, hipStream_t stream);

struct MoeCall {
  const qg_moe *m;
  const float *X;
  int64_t ldx;
  int ntok;
  float *Y;
  int64_t ldy;
  int32_t *topk_idx;
  float *topk_w;
  void *ws;
  size_t ws_bytes;
  hipStream_t stream;
};
size_t moe_ws_bytes(const qg_moe *m, int ntok);
int launch_moe(const MoeCall &c);

// Launch bookkeeping: clear errors left by earlier calls of other code on
// this thread, then turn the launch result into a status and remember the
// HIP error text for qg_last_hip_error().
void record_hip_error(hipError_t e);
inline void clear_hip_error() { (void)hipGetLastError(); }
inline int launch_status() {
  const hipError_t e = hipGetLastError();
  if (e == hipSuccess) return 0;
  record_hip_error(e);
  return -6;  // QG_EHIP
}

}  // namespace qg
