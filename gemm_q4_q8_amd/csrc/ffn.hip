// Fused decode FFN of one layer, one token: h = SiLU(Wg x) * (Wu x), then
// y += Wd h, in one persistent launch.
//
// What is computed ("Engine and kernels", Kernel families: the fused gate/up
// with SiLU applied before writing, and the down projection with the
// residual epilogue y += W x): exactly what gateup_silu followed by a
// 1-column qgemv with accumulate compute, with the same K segments and the
// same reduction order, so h and y are bitwise equal to that pair of calls.
//
// Why one launch: the down projection's weights do not depend on h.  A
// workgroup (16 waves, one per CU) takes work units in order, all gate/up
// units first, then the down units; a down unit issues its first weight
// loads, then waits for the h row tiles its K segment reads (a ready flag
// per row tile, raised by the gate/up unit that wrote it).  So the down
// stream's first loads overlap the last gate/up units, and the second
// launch with its start-up is gone.  Each phase uses the work split that
// suits it (the row tiles a unit holds do not change any sum, only which
// workgroup computes it): gate/up as the separate call runs it (with
// interleaved segments, R row tiles x S segments summed inside the
// workgroup), down with as many row tiles per unit as make its units fit
// one round of the grid (units of fewer waves leave the others idle).
//
// Progress: the first gridDim.x units are taken by blockIdx, the rest from
// an atomic queue in unit order, and the grid is no larger than the gate/up
// unit count nor than what the device holds at once.  So a down unit is
// handed out only after every gate/up unit has been handed out to a running
// workgroup, and gate/up units never wait, so every wait ends.  (A bounded
// wait still guards the kernel: should one ever time out, it sets the error
// word and the kernel ends.)
#include <string.h>

#include <algorithm>

#include "common.h"
#include "dot_unit.h"
#include "internal.h"
#include "qgemm.h"

namespace qg {

struct FfnArgs {
  DotArgs A, B;       // gate/up (producer) and down (consumer)
  int NA, NB;         // work units of each phase
  uint32_t *queue;    // units beyond the first gridDim.x
  uint32_t *done;     // workgroups finished
};

// Waves per workgroup: 16 (Q4_0), 12 (Q8_0, whose units need more than the
// 128 registers a wave of a 16-wave workgroup may hold).
#ifndef FFN_WQ4
#define FFN_WQ4 16
#endif
template <int QT>
constexpr int ffn_waves() { return QT == Q4 ? FFN_WQ4 : 12; }

template <int QT, int PFA, int PFB>
__global__ void __launch_bounds__(ffn_waves<QT>() * 64) ffn_kernel(FfnArgs f) {
  constexpr int FFN_W = ffn_waves<QT>();
  extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
  __shared__ uint32_t flag;
  __shared__ int s_next;
  const int tid = threadIdx.x;
  float bv = 0.0f;
  int32_t bi = 0;
  const int total = f.NA + f.NB;
  int unit = blockIdx.x;
  while (unit < total) {
    uint32_t nxt = 0;
    auto take_next = [&]() {
      if (tid == 0) nxt = gridDim.x + __hip_atomic_fetch_add(f.queue, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    };
    if (unit < f.NA) {
      dot_unit<QT, 1, 2, EPI_SILU, 1, PFA, FFN_W, PH_PRODUCE, DOT_MF>(f.A, unit / f.A.S, unit % f.A.S, smem, &flag,
                                                               bv, bi, take_next);
    } else {
      // segment-major, so the first down units read the first h rows
      const int ub = unit - f.NA;
      dot_unit<QT, 1, 1, EPI_ACC, 1, PFB, FFN_W, PH_CONSUME, DOT_MF>(f.B, ub % f.B.G, ub / f.B.G, smem, &flag, bv,
                                                              bi, take_next);
    }
    if (tid == 0) s_next = (int)nxt;
    __syncthreads();
    unit = s_next;
    __syncthreads();  // s_next and the LDS tiles are reused
  }
  // the last workgroup out lowers the ready flags and resets the queue
  if (arrive_last(f.done, gridDim.x, &flag)) {
    for (int i = tid; i < f.A.NT; i += FFN_W * 64) st_agent_u32(f.A.ready + i, 0u);
    if (tid == 0) st_agent_u32(f.queue, 0u);
  }
}

static int64_t cdiv(int64_t a, int64_t b) { return (a + b - 1) / b; }

// Workspace: counters (done, queue, error word, the split-K counters of both
// phases, one ready flag per h row tile), then the segment partials of both
// phases.  Its size depends on the shape only.
struct FfnLayout {
  size_t part_a, part_b, total;
  int SA, SB;
};

static FfnLayout ffn_layout(int64_t hidden, int64_t ffn) {
  FfnLayout L;
  L.SA = gemv_segments(ffn, hidden, 2, 8);  // as gateup_silu
  L.SB = gemv_segments(hidden, ffn, 1, 8);  // as qgemv
  size_t o = QG_WS_SYNC_BYTES;
  L.part_a = o;
  if (L.SA > 1) o += (size_t)L.SA * 2 * cdiv(ffn, 16) * dot_part_floats(1) * 4;
  o = (o + 255) & ~size_t(255);
  L.part_b = o;
  if (L.SB > 1) o += (size_t)L.SB * cdiv(hidden, 16) * dot_part_floats(1) * 4;
  L.total = (o + 255) & ~size_t(255);
  return L;
}

size_t ffn_ws_bytes(int64_t hidden, int64_t ffn) { return ffn_layout(hidden, ffn).total; }

// One phase's arguments: S segments across workgroups or (SW > 1) inside
// the workgroup, R row tiles per unit, NWU = R * SW waves of the 16.
static DotArgs phase_args(const void *qs0, const void *d0, const void *qs1, const void *d1, int64_t rows,
                          int64_t cols, int S, int SW, int R, const float *X, float *Y, float *part,
                          uint32_t *cnt, uint32_t *ready, uint32_t *err) {
  DotArgs a;
  memset(&a, 0, sizeof(a));
  a.qs0 = (const uint8_t *)qs0;
  a.d0 = (const uint8_t *)d0;
  a.qs1 = (const uint8_t *)qs1;
  a.d1 = (const uint8_t *)d1;
  a.rows = rows;
  a.cols = cols;
  a.NT = (int)cdiv(rows, 16);
  a.KT = (int)cdiv(cols / 32, 4);
  a.S = S;
  a.SW = SW;
  a.IL = dot_interleaved(cols) ? 1 : 0;  // as the separate calls
  a.NWU = R * SW;
  a.G = (int)cdiv(a.NT, R);
  a.units = (int64_t)a.G * S;
  a.X = X;
  a.ldx = cols;
  a.ncols = 1;
  a.Y = Y;
  a.ldy = rows;
  a.part = part;
  a.cnt = cnt;
  a.ready = ready;
  a.err = err;
  return a;
}

template <int QT>
static int launch_ffn_t(const FfnCall &c) {
  constexpr int QW = QT == Q4 ? 1 : 2;
  constexpr int PFA = 4 / (2 * QW) < 2 ? 2 : 4 / (2 * QW);
  constexpr int PFB = 4 / QW < 2 ? 2 : 4 / QW;
  const FfnLayout L = ffn_layout(c.hidden, c.ffn);
  if (c.ws_bytes < L.total) return QG_EWORKSPACE;
  const int64_t KTA = cdiv(c.hidden / 32, 4), KTB = cdiv(c.ffn / 32, 4);
  const int64_t NTA = cdiv(c.ffn, 16), NTB = cdiv(c.hidden, 16);
  if (KTA * QTraits<QT>::tile_bytes >= ((int64_t)1 << 31) || KTB * QTraits<QT>::tile_bytes >= ((int64_t)1 << 31))
    return QG_EUNSUPPORTED;
  auto kern = ffn_kernel<QT, PFA, PFB>;
  constexpr int FFN_W = ffn_waves<QT>();

  // the device: CUs and workgroups it holds at once (per device)
  static int resident[64], ncus[64];
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess || dev < 0 || dev >= 64) {
    record_hip_error(e == hipSuccess ? hipErrorInvalidDevice : e);
    return QG_EHIP;
  }
  if (resident[dev] == 0) {
    int per_cu = 0, ncu = 0;
    e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, (const void *)kern, FFN_W * 64, 65536);
    if (e == hipSuccess) e = hipDeviceGetAttribute(&ncu, hipDeviceAttributeMultiprocessorCount, dev);
    if (e != hipSuccess) {
      record_hip_error(e);
      return QG_EHIP;
    }
    if (per_cu < 1 || ncu < 1) return QG_EUNSUPPORTED;
    resident[dev] = per_cu * ncu;
    ncus[dev] = ncu;
  }
  const int64_t ncu = ncus[dev];

  // gate/up: interleaved segments inside the workgroup when R row tiles x
  // S segments fit its waves (R = row tiles per CU), else S across
  // workgroups with as many row tiles per unit as spread the units over the
  // CUs
  int SA = L.SA, SWA = 1, RA;
  const int64_t Rin = cdiv(NTA, ncu);
  if (dot_interleaved(c.hidden) && L.SA > 1 && Rin * L.SA <= FFN_W) {
    SWA = L.SA;
    SA = 1;
    RA = (int)Rin;
  } else {
    RA = (int)std::min<int64_t>(FFN_W, std::max<int64_t>(1, cdiv(NTA * L.SA, ncu)));
  }
  const int64_t NA = cdiv(NTA, RA) * SA;
  const int grid = (int)std::min<int64_t>(NA, resident[dev]);
  // down: S across workgroups, row tiles per unit so that its units fit
  // one round of the grid
  const int SB = L.SB;
  const int RB = (int)std::min<int64_t>(FFN_W, cdiv(NTB, std::max(1, grid / SB)));

  uint8_t *ws = (uint8_t *)c.ws;
  uint32_t *w32 = (uint32_t *)ws;
  FfnArgs f;
  f.done = w32 + 0;
  f.queue = w32 + 1;
  uint32_t *err = w32 + 2;
  uint32_t *cnt_a = w32 + 4;
  uint32_t *cnt_b = cnt_a + cdiv(NTA, RA);
  uint32_t *ready = cnt_b + cdiv(NTB, RB);
  if ((size_t)(ready + NTA - w32) > WS_SYNC_WORDS) return QG_EUNSUPPORTED;
  f.A = phase_args(c.g_qs, c.g_d, c.u_qs, c.u_d, c.ffn, c.hidden, SA, SWA, RA, c.x, c.h, (float *)(ws + L.part_a),
                   cnt_a, ready, err);
  f.B = phase_args(c.d_qs, c.d_d, c.d_qs, c.d_d, c.hidden, c.ffn, SB, 1, RB, c.h, c.y, (float *)(ws + L.part_b),
                   cnt_b, ready, err);
  f.B.ready_n = (int)NTA;
  f.NA = (int)f.A.units;
  f.NB = (int)f.B.units;

  // staged activations (+ the in-workgroup segment sums of gate/up)
  const size_t lds_a = (size_t)(f.A.IL ? KTA : cdiv(KTA, SA)) * TILE_BLOCKS * 64 +
                       (size_t)(SWA - 1) * RA * 2 * dot_part_floats(1) * 4;
  const size_t lds_b = (size_t)(f.B.IL ? KTB : cdiv(KTB, SB)) * TILE_BLOCKS * 64;
  const size_t lds = lds_a > lds_b ? lds_a : lds_b;
  if (lds > 65536) return QG_EUNSUPPORTED;
  clear_hip_error();
  hipLaunchKernelGGL(kern, dim3((unsigned)grid), dim3(FFN_W * 64), lds, c.stream, f);
  return launch_status();
}

int launch_ffn(const FfnCall &c) {
  if (c.qtype == QG_Q4_0) return launch_ffn_t<Q4>(c);
  if (c.qtype == QG_Q8_0) return launch_ffn_t<Q8>(c);
  return QG_EINVAL;
}

}  // namespace qg
