// Launch plans per shape and their tuning ("Engine and kernels", What each
// trick bought, the reading-weights table: workgroup size and rows per
// workgroup timed on the device at load, about a second, a candidate kept
// only past a 3% noise margin).  Here the choice is between workgroup sizes
// and where the K segments are summed; the segments themselves, and so the
// result bits, are fixed by the shape, which the GPU tests check plan by
// plan.
#include <hip/hip_runtime.h>

#include <atomic>
#include <map>
#include <mutex>
#include <tuple>
#include <vector>

#include "internal.h"
#include "qgemm.h"

namespace qg {
namespace {

// (device, op, qtype, rows, cols, ncols)
using PlanKey = std::tuple<int, int, int, int64_t, int64_t, int>;

std::mutex g_mu;
std::map<PlanKey, int> g_plans;
std::atomic<int> g_n_plans{0};

int op_of(int epi) {
  if (epi == EPI_SILU) return QG_OP_GATEUP;
  if (epi == EPI_ARGMAX || epi == EPI_TOPK) return QG_OP_LMHEAD;
  return QG_OP_GEMV;
}

int current_device() {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) dev = 0;
  return dev;
}

bool shape_ok(int op, int qtype, int64_t rows, int64_t cols, int ncols) {
  if (qtype != QG_Q4_0 && qtype != QG_Q8_0) return false;
  if (rows <= 0 || cols <= 0 || cols % 32) return false;
  if (op == QG_OP_GEMV) return (ncols >= 1 && ncols <= 8) || ncols == 16;
  if (op == QG_OP_GATEUP) return ncols >= 1 && ncols <= 8;
  if (op == QG_OP_LMHEAD) return ncols == 1;
  return false;
}

bool plan_ok(int op, int ncols, int plan) {
  if (plan == 0) return true;
  if (plan & QG_PLAN_STRICT) {
    plan &= ~QG_PLAN_STRICT;
    if (plan == 0) return false;
  }
  const int layout = plan & ~PLAN_S_MASK;  // what remains besides the K segments
  if (layout == 0) return true;
  if (op == QG_OP_GEMV && ncols == 16) return layout >= 8 && layout <= 16;
  return (layout >= 1 && layout <= 16) || layout == QG_PLAN_SW;
}

void store_plan(const PlanKey &k, int plan) {
  std::lock_guard<std::mutex> l(g_mu);
  g_plans[k] = plan;
  g_n_plans.store((int)g_plans.size(), std::memory_order_release);
}

}  // namespace

int plan_lookup(const QmvCall &c) {
  if (g_n_plans.load(std::memory_order_acquire) == 0) return 0;
  const PlanKey k{current_device(), op_of(c.epi), c.qtype, c.rows, c.cols, c.ncols};
  std::lock_guard<std::mutex> l(g_mu);
  const auto it = g_plans.find(k);
  return it == g_plans.end() ? 0 : it->second;
}

// Times every candidate plan on the call's own buffers and keeps the
// winner.  The call must not accumulate into its output (the launches
// repeat).  Every candidate is a layout the built-in choice itself takes
// for some shape; one the call cannot use is refused before launching and
// dropped.  With QG_TUNE_SPLIT the K segments are candidates too: half,
// one less, one more and twice the shape's own (within the K range and the
// workspace the size queries give).
int tune_call(QmvCall c, int32_t flags, int32_t *plan_out) {
  static const int kGemv[] = {0, 4, 8, 12, 16, QG_PLAN_SW};
  static const int kGemm16[] = {0, 8, 12, 16};
  const bool g16 = c.ncols == 16;
  const int *lay = g16 ? kGemm16 : kGemv;
  const int nlay = g16 ? 4 : 6;
  std::vector<int> splits{0};
  if (flags & QG_TUNE_SPLIT) {
    const int S = builtin_split(c);
    const int64_t KT = (c.cols / 32 + 3) / 4;
    for (int sp : {S / 2, S - 1, S + 1, 2 * S}) {
      bool seen = sp == S;
      for (int q : splits) seen = seen || q == sp;
      if (!seen && sp >= 1 && sp <= KT && sp <= 255) splits.push_back(sp);
    }
  }
  std::vector<int> cand;
  for (int sp : splits)
    for (int i = 0; i < nlay; ++i) cand.push_back(lay[i] | (sp << PLAN_S_SHIFT));
  const int n = (int)cand.size();
  constexpr int ROUNDS = 3, REPS = 10;
  std::vector<float> best(n, 3.0e38f);
  std::vector<char> usable(n, 1);
  hipEvent_t e0 = nullptr, e1 = nullptr;
  hipError_t he = hipEventCreate(&e0);
  if (he == hipSuccess) he = hipEventCreate(&e1);
  int st = QG_OK;
  if (he != hipSuccess) {
    record_hip_error(he);
    st = QG_EHIP;
  }
  for (int r = 0; r < ROUNDS && st == QG_OK; ++r) {
    for (int i = 0; i < n && st == QG_OK; ++i) {
      if (!usable[i]) continue;
      c.plan = cand[i] | PLAN_FORCED;
      int s = launch_qmv(c);  // warm-up, and whether the plan fits
      if ((s == QG_EUNSUPPORTED || s == QG_EWORKSPACE) && i > 0) {
        usable[i] = false;
        continue;
      }
      if (s == QG_OK && (he = hipEventRecord(e0, c.stream)) != hipSuccess) s = QG_EHIP;
      for (int k = 0; k < REPS && s == QG_OK; ++k) s = launch_qmv(c);
      if (s == QG_OK && (he = hipEventRecord(e1, c.stream)) != hipSuccess) s = QG_EHIP;
      if (s == QG_OK && (he = hipEventSynchronize(e1)) != hipSuccess) s = QG_EHIP;
      float ms = 0.0f;
      if (s == QG_OK && (he = hipEventElapsedTime(&ms, e0, e1)) != hipSuccess) s = QG_EHIP;
      if (s == QG_EHIP && he != hipSuccess) record_hip_error(he);
      if (s) {
        st = s;
        break;
      }
      if (ms / REPS < best[i]) best[i] = ms / REPS;
    }
  }
  int chosen = 0;
  if (st == QG_OK) {
    int bi = 0;
    for (int i = 1; i < n; ++i)
      if (usable[i] && best[i] < best[bi]) bi = i;
    if (bi != 0 && best[bi] < 0.97f * best[0]) chosen = cand[bi];
    store_plan(PlanKey{current_device(), op_of(c.epi), c.qtype, c.rows, c.cols, c.ncols}, chosen);
    if (plan_out) *plan_out = chosen;
    // the outputs as the tuned call leaves them (the same bits as any plan)
    c.plan = chosen | PLAN_FORCED;
    st = launch_qmv(c);
    if (st == QG_OK && (he = hipStreamSynchronize(c.stream)) != hipSuccess) {
      record_hip_error(he);
      st = QG_EHIP;
    }
  }
  if (e0) (void)hipEventDestroy(e0);
  if (e1) (void)hipEventDestroy(e1);
  return st;
}

}  // namespace qg

extern "C" {

int qg_plan_set(int op, int qtype, int64_t rows, int64_t cols, int32_t ncols, int32_t plan) {
  if (!qg::shape_ok(op, qtype, rows, cols, ncols)) return QG_EINVAL;
  if (!qg::plan_ok(op, ncols, plan)) return QG_EINVAL;
  qg::store_plan(qg::PlanKey{qg::current_device(), op, qtype, rows, cols, ncols}, plan);
  return QG_OK;
}

int qg_plan_get(int op, int qtype, int64_t rows, int64_t cols, int32_t ncols, int32_t *plan) {
  if (!plan || !qg::shape_ok(op, qtype, rows, cols, ncols)) return QG_EINVAL;
  const qg::PlanKey k{qg::current_device(), op, qtype, rows, cols, ncols};
  std::lock_guard<std::mutex> l(qg::g_mu);
  const auto it = qg::g_plans.find(k);
  *plan = it == qg::g_plans.end() ? 0 : it->second;
  return QG_OK;
}

void qg_plan_reset(void) {
  std::lock_guard<std::mutex> l(qg::g_mu);
  qg::g_plans.clear();
  qg::g_n_plans.store(0, std::memory_order_release);
}

}  // extern "C"
