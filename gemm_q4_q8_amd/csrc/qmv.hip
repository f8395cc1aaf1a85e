// Tiled quantised products on gfx950: the decode GEMV and its batched twins,
// the fused gate/up with SiLU, the LM head with argmax (dot path, 1..8
// columns), and the 16-column prefill GEMM on the matrix cores.
//
// What is computed ("Engine and kernels", Kernel families and What each
// trick bought): y = W x over Q4_0 / Q8_0 blocks dequantised in registers,
// f32 sums, optional y += W x into the residual, gate/up fused with SiLU
// before writing, greedy argmax with lowest-index ties, and a 16-column GEMM
// with split-K pinned per shape.
//
// Dot path (1..8 columns): one workgroup per (row group, K segment); the
// unit's work (activation staging, weight streaming, reduction, epilogue)
// is dot_unit.h.  K segments per shape: gemv_segments() below.
//
// Matrix-core path (16 columns): WKT waves take WKT consecutive K segments
// of RT row tiles; per block and row tile one v_mfma_f32_16x16x32_f16 with
// A = activations (16 columns x 32), B = the block's weights, the block
// scale applied to the 4 outputs each lane holds; waves of a workgroup, then
// splits, summed in index order.
#include "common.h"
#include "dot_unit.h"
#include "internal.h"
#include "qgemm.h"

namespace qg {

static size_t align256(size_t v) { return (v + 255) & ~size_t(255); }
static int64_t cdiv(int64_t a, int64_t b) { return (a + b - 1) / b; }

// --------------------------------------------------------------- dot path
template <int QT, int NC, int NMAT, int EPI, int RT, int PF, int WKT, bool MF>
__global__ void __launch_bounds__(WKT * 64) dot_kernel(DotArgs a) {
  constexpr int NTHR = WKT * 64;
  extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
  __shared__ uint32_t flag;
  __shared__ float wave_v[WKT];
  __shared__ int32_t wave_i[WKT];

  const int tid = threadIdx.x, lane = tid & 63;
  const int wk = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int64_t u = xcd_unit(a.per_xcd);
  if (u >= a.units) return;
  const int g = (int)(u / a.S), s = (int)(u % a.S);
  float bv = __builtin_nanf("");  // argmax: this lane's best (value, row)
  int32_t bi = 0x7fffffff;
  const bool emitted = dot_unit<QT, NC, NMAT, EPI, RT, PF, WKT, PH_PLAIN, MF>(a, g, s, smem, &flag, bv, bi);

  if constexpr (EPI == EPI_ARGMAX) {
    if (!emitted) return;
    // ---- argmax of this row group, then of all row groups
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) {
      const float ov = __shfl_xor(bv, off);
      const int32_t oi = __shfl_xor(bi, off);
      if (ranks_before(ov, oi, bv, bi)) { bv = ov; bi = oi; }
    }
    if (lane == 0) { wave_v[wk] = bv; wave_i[wk] = bi; }
    __syncthreads();
    if (tid == 0) {
      for (int w = 1; w < WKT; ++w)
        if (ranks_before(wave_v[w], wave_i[w], bv, bi)) { bv = wave_v[w]; bi = wave_i[w]; }
      st_agent(a.cand_v + g, bv);
      st_agent_u32((uint32_t *)a.cand_i + g, (uint32_t)bi);
    }
    if (!arrive_last(a.gcnt, (uint32_t)a.G, &flag)) return;
    bv = __builtin_nanf("");
    bi = 0x7fffffff;
    for (int qq = tid; qq < a.G; qq += NTHR) {
      const float v = ld_agent(a.cand_v + qq);
      const int32_t i = (int32_t)ld_agent_u32((const uint32_t *)a.cand_i + qq);
      if (ranks_before(v, i, bv, bi)) { bv = v; bi = i; }
    }
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) {
      const float ov = __shfl_xor(bv, off);
      const int32_t oi = __shfl_xor(bi, off);
      if (ranks_before(ov, oi, bv, bi)) { bv = ov; bi = oi; }
    }
    __syncthreads();  // wave_v / wave_i are reused
    if (lane == 0) { wave_v[wk] = bv; wave_i[wk] = bi; }
    __syncthreads();
    if (tid == 0) {
      for (int w = 1; w < WKT; ++w)
        if (ranks_before(wave_v[w], wave_i[w], bv, bi)) { bv = wave_v[w]; bi = wave_i[w]; }
      *a.out_idx = bi;
      if (a.out_val) *a.out_val = bv;
    }
  }
}

// ------------------------------------------------------- matrix-core path
struct MmaArgs {
  const uint8_t *qs, *d;
  int64_t rows, cols;
  int NT, KT;
  int Q;              // K segments: WKT per workgroup, S workgroups per row group
  int S;
  int G;              // row groups of RT row tiles
  int64_t units;
  int64_t per_xcd;
  int nkt_max;
  const float *X;
  int64_t ldx;
  float *Y;
  int64_t ldy;
  float *part;        // [S][NT*16][16]
  uint32_t *cnt;
};

template <int QT, int EPI, int RT, int PF, int WKT>
__global__ void __launch_bounds__(WKT * 64) mma_kernel(MmaArgs a) {
  constexpr int NC = 16;
  constexpr int NTHR = WKT * 64;
  constexpr int TB = QTraits<QT>::tile_bytes;
  constexpr int QW = (QT == Q4) ? 1 : 2;
  extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
  __shared__ uint32_t flag;

  const int tid = threadIdx.x, lane = tid & 63;
  const int wk = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int64_t u = xcd_unit(a.per_xcd);
  if (u >= a.units) return;
  const int g = (int)(u / a.S), s = (int)(u % a.S);
  const int q0 = s * WKT;
  const int q1 = (q0 + WKT < a.Q) ? q0 + WKT : a.Q;
  const int kt0 = seg_begin(q0, a.KT, a.Q);
  const int kt1 = seg_begin(q1, a.KT, a.Q);
  const int nkt = kt1 - kt0;
  const int q = q0 + wk;
  const int wb = q < q1 ? seg_begin(q, a.KT, a.Q) : kt1;
  const int we = q < q1 ? seg_begin(q + 1, a.KT, a.Q) : kt1;

  _Float16 *xs = (_Float16 *)smem;
  float *red = (float *)smem;
  const int r = lane & 15, sl = lane >> 4;
  const int64_t rt_base = (int64_t)g * RT;

  u4 wq[PF][RT][QW];
  u2 wd[PF][RT];
  const uint32_t lane_off = (uint32_t)lane * 16u, d_off = (uint32_t)r * 8u;
  auto load = [&](int slot, int kt) {
#pragma unroll
    for (int t = 0; t < RT; ++t) {
      const int64_t trow = (rt_base + t < a.NT) ? rt_base + t : (int64_t)a.NT - 1;
      const int64_t tile = trow * a.KT + kt;
      const uint8_t *tq = a.qs + tile * TB;
      const uint8_t *td = a.d + tile * TILE_D_BYTES;
      wq[slot][t][0] = ld_stream(tq + lane_off);
      if constexpr (QW == 2) wq[slot][t][QW - 1] = ld_stream(tq + 1024 + lane_off);
      wd[slot][t] = ld_stream2(td + d_off);
    }
  };
  const int nseg = we - wb;
  if (nseg > 0) {
#pragma unroll
    for (int p = 0; p < PF; ++p) load(p, wb + (p < nseg ? p : nseg - 1));
  }

  {
    constexpr int XB = 4;
    const int nvec = nkt * TILE_BLOCKS * NC * 4;
    for (int v0 = tid; v0 < nvec; v0 += XB * NTHR) {
      float4 lo[XB], hi[XB];
      bool ok[XB];
#pragma unroll
      for (int b = 0; b < XB; ++b) {
        const int v = v0 + b * NTHR;
        const int qq = v & 3, c = (v >> 2) % NC, bl = (v >> 2) / NC;
        const int64_t k = ((int64_t)kt0 * TILE_BLOCKS + bl) * 32 + qq * 8;
        ok[b] = v < nvec && k < a.cols;
        const float4 *p = (const float4 *)(a.X + (ok[b] ? (int64_t)c * a.ldx + k : 0));
        lo[b] = p[0];
        hi[b] = p[1];
      }
#pragma unroll
      for (int b = 0; b < XB; ++b) {
        const int v = v0 + b * NTHR;
        if (v < nvec) {
          h8 hv = {0, 0, 0, 0, 0, 0, 0, 0};
          if (ok[b]) hv = cvt8(lo[b], hi[b]);
          *(h8 *)(xs + (size_t)v * 8) = hv;
        }
      }
    }
  }
  __syncthreads();

  float acc[RT][4];
#pragma unroll
  for (int t = 0; t < RT; ++t)
#pragma unroll
    for (int i = 0; i < 4; ++i) acc[t][i] = 0.0f;

  const Q4Magic mg = q4_magic();
  auto compute = [&](int slot, int kt) {
    const int bl0 = (kt - kt0) * TILE_BLOCKS;
#pragma unroll
    for (int j = 0; j < TILE_BLOCKS; ++j) {
      const h8 A = *(const h8 *)(xs + ((size_t)(bl0 + j) * 16 + r) * 32 + sl * 8);
#pragma unroll
      for (int t = 0; t < RT; ++t) {
        h2 w[4];
        if constexpr (QT == Q4) unpack_q4(wq[slot][t][0][j], w, mg);
        else unpack_q8(wq[slot][t][j >> 1][(j & 1) * 2], wq[slot][t][j >> 1][(j & 1) * 2 + 1], w);
        h8 B = {w[0][0], w[0][1], w[1][0], w[1][1], w[2][0], w[2][1], w[3][0], w[3][1]};
        const f4 D = __builtin_amdgcn_mfma_f32_16x16x32_f16(A, B, f4{0.f, 0.f, 0.f, 0.f}, 0, 0, 0);
        const float dj = scale_of(wd[slot][t], j);
#pragma unroll
        for (int i = 0; i < 4; ++i) acc[t][i] = __builtin_fmaf(dj, D[i], acc[t][i]);
      }
    }
  };

  int k = 0;
  for (; k + 2 * PF <= nseg; k += PF) {
#pragma unroll
    for (int p = 0; p < PF; ++p) {
      compute(p, wb + k + p);
      load(p, wb + k + p + PF);
    }
  }
#pragma unroll
  for (int p = 0; p < PF; ++p) {
    if (k + p < nseg) {
      compute(p, wb + k + p);
      if (k + p + PF < nseg) load(p, wb + k + p + PF);
    }
  }
#pragma unroll
  for (int p = 0; p < PF; ++p)
    if (k + PF + p < nseg) compute(p, wb + k + PF + p);

  // per-wave partials -> LDS: lane holds D[4 sl + i][r] = (column 4 sl + i, row r)
  __syncthreads();
#pragma unroll
  for (int t = 0; t < RT; ++t)
#pragma unroll
    for (int i = 0; i < 4; ++i) red[((wk * RT + t) * 16 + r) * 16 + sl * 4 + i] = acc[t][i];
  __syncthreads();

  const int64_t rows_pad = (int64_t)a.NT * 16;
  constexpr int NOUT = RT * 16 * NC;
  const int nw = q1 - q0;
  auto red_at = [&](int w, int t, int rr, int c) -> float { return red[((w * RT + t) * 16 + rr) * NC + c]; };
  auto emit = [&](int t, int rr, int c, float v) {
    const int64_t row = (rt_base + t) * 16 + rr;
    if (row >= a.rows) return;
    float *yp = a.Y + (int64_t)c * a.ldy + row;
    if constexpr (EPI == EPI_STORE) *yp = v;
    else *yp = *yp + v;
  };

  if (a.S == 1) {
    for (int o = tid; o < NOUT; o += NTHR) {
      const int c = o % NC, rr = (o / NC) % 16, t = o / (16 * NC);
      float x = red_at(0, t, rr, c);
      for (int w = 1; w < nw; ++w) x += red_at(w, t, rr, c);
      emit(t, rr, c, x);
    }
  } else {
    for (int o = tid; o < NOUT; o += NTHR) {
      const int c = o % NC, rr = (o / NC) % 16, t = o / (16 * NC);
      if (rt_base + t >= a.NT) continue;
      const int64_t row = (rt_base + t) * 16 + rr;
      float x = red_at(0, t, rr, c);
      for (int w = 1; w < nw; ++w) x += red_at(w, t, rr, c);
      st_agent(a.part + ((int64_t)s * rows_pad + row) * NC + c, x);
    }
    if (!arrive_last(a.cnt + g, (uint32_t)a.S, &flag)) return;
    for (int o = tid; o < NOUT; o += NTHR) {
      const int c = o % NC, rr = (o / NC) % 16, t = o / (16 * NC);
      if (rt_base + t >= a.NT) continue;
      const int64_t row = (rt_base + t) * 16 + rr;
      float x = ld_agent(a.part + row * NC + c);
      for (int ss = 1; ss < a.S; ++ss) x += ld_agent(a.part + ((int64_t)ss * rows_pad + row) * NC + c);
      emit(t, rr, c, x);
    }
  }
}

// ---------------------------------------------------------------- host side
constexpr int DOT_STREAMS = 2048;     // (row tile, segment, matrix) weight streams
constexpr size_t DOT_X_LDS = 65536;   // staged activations per workgroup
constexpr size_t LDS_HARD = 163840;   // gfx950 LDS per workgroup

// K segments of the dot path: about DOT_STREAMS weight streams of one row
// tile and one segment each (measured on the decode shapes: more streams,
// or more bytes in flight per stream, only lengthen the queues and the
// tail), at least 4 tile columns per segment, and few enough tile columns
// per segment that `ncols_max` columns of f16 activations fit in DOT_X_LDS.
int gemv_segments(int64_t rows, int64_t cols, int nmat, int ncols_max) {
  const int64_t NT = cdiv(rows, 16), KT = cdiv(cols / 32, 4);
  // rounded down (the fused FFN needs the gate/up units in one round of
  // resident workgroups), except that 1.5 or more becomes 2
  const int64_t want = (int64_t)DOT_STREAMS * nmat;
  int64_t s = want / NT;
  if (s < 2 && 2 * want >= 3 * NT) s = 2;
  if (s > KT / 4) s = KT / 4;
  const int64_t lds_min = cdiv(KT * TILE_BLOCKS * ncols_max * 64, (int64_t)DOT_X_LDS);
  if (s < lds_min) s = lds_min;
  if (s < 1) s = 1;
  if (s > KT) s = KT;
  return (int)s;
}

// Splits of K for the matrix-core path (16 columns of f16 activations per
// workgroup in at most 64 KiB of LDS, two tile columns per wave at least).
int gemm16_splits(int64_t rows, int64_t cols) {
  const int64_t NT = cdiv(rows, 16), KT = cdiv(cols / 32, 4);
  int64_t s = cdiv(2048, NT);
  const int64_t cap = KT / 8;
  if (s > cap) s = cap;
  const int64_t lds_min = cdiv(KT, 16);
  if (s < lds_min) s = lds_min;
  if (s < 1) s = 1;
  if (s > KT) s = KT;
  return (int)s;
}

size_t qmv_ws_bytes(int64_t rows, int64_t cols, int slots, int nmat, int ncols_max, bool argmax) {
  const int64_t NT = cdiv(rows, 16);
  (void)cols;
  size_t b = QG_WS_SYNC_BYTES;                      // counters
  if (argmax) b += 2 * align256((size_t)NT * 4);    // candidates
  if (slots > 1) b += (size_t)slots * nmat * NT * 16 * ncols_max * 4;
  return b;
}

// Buffer ranges carry 32-bit sizes: the activation columns and one row
// tile's weights must each span less than 2^31 bytes.
static bool ranges_fit(const QmvCall &c, int64_t NT, int64_t KT, int64_t tile_bytes) {
  (void)NT;
  const int64_t xb = ((int64_t)(c.ncols - 1) * c.ldx + c.cols) * 4;
  return xb < ((int64_t)1 << 31) && KT * tile_bytes < ((int64_t)1 << 31);
}

static int grant_lds(const void *kern, size_t lds, size_t &granted) {
  if (lds > 65536 && lds > granted) {
    const hipError_t e = hipFuncSetAttribute(kern, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    if (e != hipSuccess) {
      record_hip_error(e);
      return QG_EHIP;
    }
    granted = lds;
  }
  return QG_OK;
}

template <int QT, int NC, int NMAT, int EPI, int RT, int PF, int WKT, bool MF>
static int launch_dot_t(const QmvCall &c, int S) {
  const int64_t NT = cdiv(c.rows, 16), KT = cdiv(c.cols / 32, 4);
  const int64_t NTu = cdiv(c.n_rows, 16);  // row tiles actually produced
  DotArgs a;
  a.qs0 = (const uint8_t *)c.qs[0];
  a.d0 = (const uint8_t *)c.d[0];
  a.qs1 = (const uint8_t *)c.qs[NMAT - 1];
  a.d1 = (const uint8_t *)c.d[NMAT - 1];
  a.rows = c.n_rows;
  a.cols = c.cols;
  a.NT = (int)NTu;
  a.KT = (int)KT;
  a.S = S;
  a.G = (int)cdiv(NTu, (int64_t)WKT * RT);
  a.units = (int64_t)a.G * S;
  a.per_xcd = cdiv(a.units, 8);
  a.X = c.X;
  a.ldx = c.ldx;
  a.ncols = c.ncols;
  a.Y = c.Y;
  a.ldy = c.ldy;
  // counters: word 0 for the argmax, words 1..G for the row groups
  if (S > 1 && (size_t)a.G + 1 > WS_SYNC_WORDS) return QG_EUNSUPPORTED;
  uint8_t *ws = (uint8_t *)c.ws;
  a.gcnt = (uint32_t *)ws;
  a.cnt = (uint32_t *)ws + 1;
  size_t off = QG_WS_SYNC_BYTES;
  a.cand_v = nullptr;
  a.cand_i = nullptr;
  if (EPI == EPI_ARGMAX) {
    a.cand_v = (float *)(ws + off);
    off += align256((size_t)NT * 4);
    a.cand_i = (int32_t *)(ws + off);
    off += align256((size_t)NT * 4);
  }
  a.part = (float *)(ws + off);
  a.out_idx = c.out_idx;
  a.out_val = c.out_val;
  a.ready = nullptr;
  a.err = nullptr;
  if (!ranges_fit(c, NT, KT, QTraits<QT>::tile_bytes)) return QG_EUNSUPPORTED;
  const size_t need = off + (S > 1 ? (size_t)S * NMAT * NTu * 16 * NC * 4 : 0);
  if (need > c.ws_bytes) return QG_EWORKSPACE;

  const size_t lds = (size_t)cdiv(KT, S) * TILE_BLOCKS * NC * 64;
  if (lds > LDS_HARD - 1024) return QG_EUNSUPPORTED;
  auto kern = dot_kernel<QT, NC, NMAT, EPI, RT, PF, WKT, MF>;
  static size_t granted = 65536;  // per instantiation; only ever raised
  int st = grant_lds((const void *)kern, lds, granted);
  if (st) return st;
  clear_hip_error();
  hipLaunchKernelGGL(kern, dim3((unsigned)(a.per_xcd * 8)), dim3(WKT * 64), lds, c.stream, a);
  return launch_status();
}

// One row tile per wave, about 4 KiB of weights in flight per wave (PF tile
// columns).  Workgroups of 8 waves unless that leaves CUs idle.
template <int QT, int NC, int NMAT, int EPI>
static int launch_dot(const QmvCall &c, int S) {
  constexpr int QW = QT == Q4 ? 1 : 2;
  constexpr int PF0 = 4 / (NMAT * QW);
  constexpr int PF = PF0 < 2 ? 2 : PF0;
  const int64_t NTu = cdiv(c.n_rows, 16);
  constexpr bool MF = DOT_MF;
  if (cdiv(NTu, 8) * S >= 256) return launch_dot_t<QT, NC, NMAT, EPI, 1, PF, 8, MF>(c, S);
  return launch_dot_t<QT, NC, NMAT, EPI, 1, PF, 4, MF>(c, S);
}

template <int QT, int EPI>
static int dispatch_dot(const QmvCall &c, int S) {
  switch (c.ncols) {
    case 1: return launch_dot<QT, 1, 1, EPI>(c, S);
    case 2: return launch_dot<QT, 2, 1, EPI>(c, S);
    case 3: return launch_dot<QT, 3, 1, EPI>(c, S);
    case 4: return launch_dot<QT, 4, 1, EPI>(c, S);
    case 5: return launch_dot<QT, 5, 1, EPI>(c, S);
    case 6: return launch_dot<QT, 6, 1, EPI>(c, S);
    case 7: return launch_dot<QT, 7, 1, EPI>(c, S);
    case 8: return launch_dot<QT, 8, 1, EPI>(c, S);
  }
  return QG_ESHAPE;
}

template <int QT>
static int dispatch_silu(const QmvCall &c, int S) {
  switch (c.ncols) {
    case 1: return launch_dot<QT, 1, 2, EPI_SILU>(c, S);
    case 2: return launch_dot<QT, 2, 2, EPI_SILU>(c, S);
    case 3: return launch_dot<QT, 3, 2, EPI_SILU>(c, S);
    case 4: return launch_dot<QT, 4, 2, EPI_SILU>(c, S);
    case 5: return launch_dot<QT, 5, 2, EPI_SILU>(c, S);
    case 6: return launch_dot<QT, 6, 2, EPI_SILU>(c, S);
    case 7: return launch_dot<QT, 7, 2, EPI_SILU>(c, S);
    case 8: return launch_dot<QT, 8, 2, EPI_SILU>(c, S);
  }
  return QG_ESHAPE;
}

template <int QT, int EPI, int RT, int PF, int WKT>
static int launch_mma_t(const QmvCall &c) {
  const int S = gemm16_splits(c.rows, c.cols);
  const int Q = WKT * S;
  const int64_t NT = cdiv(c.rows, 16), KT = cdiv(c.cols / 32, 4);
  MmaArgs a;
  a.qs = (const uint8_t *)c.qs[0];
  a.d = (const uint8_t *)c.d[0];
  a.rows = c.rows;
  a.cols = c.cols;
  a.NT = (int)NT;
  a.KT = (int)KT;
  a.Q = Q;
  a.S = S;
  a.G = (int)cdiv(NT, RT);
  a.units = (int64_t)a.G * S;
  a.per_xcd = cdiv(a.units, 8);
  int nkt_max = 0;
  for (int s = 0; s < S; ++s) {
    const int q0 = s * WKT, q1 = q0 + WKT < Q ? q0 + WKT : Q;
    const int n = seg_begin(q1, (int)KT, Q) - seg_begin(q0, (int)KT, Q);
    if (n > nkt_max) nkt_max = n;
  }
  a.nkt_max = nkt_max;
  a.X = c.X;
  a.ldx = c.ldx;
  a.Y = c.Y;
  a.ldy = c.ldy;
  if (S > 1 && (size_t)a.G + 1 > WS_SYNC_WORDS) return QG_EUNSUPPORTED;
  uint8_t *ws = (uint8_t *)c.ws;
  a.cnt = (uint32_t *)ws + 1;
  a.part = (float *)(ws + QG_WS_SYNC_BYTES);
  const size_t need = QG_WS_SYNC_BYTES + (S > 1 ? (size_t)S * NT * 16 * 16 * 4 : 0);
  if (need > c.ws_bytes) return QG_EWORKSPACE;
  const size_t x_bytes = (size_t)nkt_max * TILE_BLOCKS * 16 * 64;
  const size_t r_bytes = (size_t)WKT * RT * 16 * 16 * 4;
  const size_t lds = x_bytes > r_bytes ? x_bytes : r_bytes;
  if (lds > LDS_HARD - 1024) return QG_EUNSUPPORTED;
  auto kern = mma_kernel<QT, EPI, RT, PF, WKT>;
  static size_t granted = 65536;
  int st = grant_lds((const void *)kern, lds, granted);
  if (st) return st;
  clear_hip_error();
  hipLaunchKernelGGL(kern, dim3((unsigned)(a.per_xcd * 8)), dim3(WKT * 64), lds, c.stream, a);
  return launch_status();
}

template <int QT>
static int dispatch_qt(const QmvCall &c) {
  if (c.ncols == 16) {
    if (c.epi == EPI_STORE) return launch_mma_t<QT, EPI_STORE, 4, 2, 4>(c);
    if (c.epi == EPI_ACC) return launch_mma_t<QT, EPI_ACC, 4, 2, 4>(c);
    return QG_EUNSUPPORTED;
  }
  switch (c.epi) {
    case EPI_STORE: return dispatch_dot<QT, EPI_STORE>(c, gemv_segments(c.rows, c.cols, 1, 8));
    case EPI_ACC: return dispatch_dot<QT, EPI_ACC>(c, gemv_segments(c.rows, c.cols, 1, 8));
    case EPI_SILU: return dispatch_silu<QT>(c, gemv_segments(c.rows, c.cols, 2, 8));
    case EPI_ARGMAX:
      if (c.ncols != 1) return QG_ESHAPE;
      return launch_dot<QT, 1, 1, EPI_ARGMAX>(c, gemv_segments(c.rows, c.cols, 1, 1));
  }
  return QG_EINVAL;
}

int launch_qmv(const QmvCall &c) {
  if (c.qtype == QG_Q4_0) return dispatch_qt<Q4>(c);
  if (c.qtype == QG_Q8_0) return dispatch_qt<Q8>(c);
  return QG_EINVAL;
}

}  // namespace qg
