// Tiled quantised products on gfx950: the decode GEMV and its batched twins,
// the fused gate/up with SiLU, the LM head with argmax, and the 16-column
// prefill GEMM on the matrix cores.  One kernel template serves them all.
//
// What is computed ("Engine and kernels", Kernel families and What each
// trick bought): y = W x over Q4_0 / Q8_0 blocks dequantised in registers,
// f32 sums, optional y += W x into the residual, gate/up fused with SiLU
// before writing, greedy argmax with lowest-index ties, and a 16-column GEMM
// with split-K pinned per shape.
//
// How it maps to MI355X:
//  * A workgroup of 4 waves owns RT row tiles (16 rows each) and a K range;
//    each wave streams a contiguous quarter of that range, PF tile columns
//    ahead, with nontemporal loads.  Each lane reads one 16-byte chunk per
//    tile (a whole wave reads a contiguous 1 KiB stripe), so every HBM read
//    is fully coalesced.
//  * The K range of the activations is staged once in LDS as f16, laid out
//    [block][column][32]; lanes of a row group read it with broadcast.
//  * Dot path (1..8 columns): weights become exact f16 pairs (two ALU ops per
//    pair) and meet the activations in v_dot2_f32_f16; each block's partial
//    is scaled by its f16 scale in f32.
//  * Matrix-core path (16 columns): one v_mfma_f32_16x16x32_f16 per block
//    and row tile, A = activations (16 columns x 32), B = the block's
//    weights; the block scale multiplies the 4 outputs each lane holds.
//  * Reduction order is fixed: tile columns in order within a wave, a 2-step
//    lane butterfly,
//    waves in index order, then K splits in index order (the last-arriving
//    workgroup sums all splits).  It depends on the shape only.
#include "common.h"
#include "internal.h"
#include "qgemm.h"

namespace qg {

constexpr int WK = 4;            // waves per workgroup (split of the K range)
constexpr int NTHR = WK * 64;
constexpr int PF = 2;            // tile columns in flight per wave

struct QmvArgs {
  const uint8_t *qs0, *qs1, *d0, *d1;
  int64_t rows;       // outputs produced (n_rows for the LM head)
  int64_t cols;
  int NT, KT;         // tiles of the packed matrix
  int S;              // K splits
  int G;              // row groups of RT tiles
  int64_t units;      // G * S
  int64_t per_xcd;
  int nkt_max;        // tile columns of the largest split (LDS sizing)
  const float *X;
  int64_t ldx;
  int ncols;
  float *Y;
  int64_t ldy;
  float *part;        // [S][NMAT][NT*16][NC]
  uint32_t *cnt;      // [G]
  uint32_t *gcnt;     // argmax: one counter
  float *cand_v;      // argmax: [G]
  int32_t *cand_i;
  int32_t *out_idx;
  float *out_val;
};

// Row tiles per wave on the dot path: at most 16 accumulators per lane
// ("Engine and kernels", verify twins keep 16 accumulators per thread), and
// at most 4 tiles of weights in flight per tile column.
template <int NC, int NMAT>
constexpr int rt_dot() {
  return (16 / (NC * NMAT)) < 1 ? 1 : ((16 / (NC * NMAT)) > 4 / NMAT ? 4 / NMAT : 16 / (NC * NMAT));
}
constexpr int RT_MFMA = 4;

static size_t align256(size_t v) { return (v + 255) & ~size_t(255); }

// Bytes of LDS before the argmax values: max(staged activations, partials).
template <int NC, int NMAT, int RT>
__host__ __device__ constexpr size_t red_offset_impl(size_t x_bytes) {
  return x_bytes > (size_t)WK * NMAT * RT * 16 * NC * 4 ? x_bytes : (size_t)WK * NMAT * RT * 16 * NC * 4;
}
template <int NC, int NMAT, int RT>
__host__ __device__ inline size_t red_offset(int nkt_max) {
  return red_offset_impl<NC, NMAT, RT>((size_t)nkt_max * TILE_BLOCKS * NC * 64);
}

template <int QT, int NC, int NMAT, int EPI, bool MFMA, int RT>
__global__ void __launch_bounds__(NTHR) qmv_kernel(QmvArgs a) {
  extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
  __shared__ uint32_t flag;
  __shared__ float wave_v[WK];
  __shared__ int32_t wave_i[WK];

  constexpr int TB = QTraits<QT>::tile_bytes;
  constexpr int QW = (QT == Q4) ? 1 : 2;   // 16-byte loads per lane per tile
  constexpr int NACC = MFMA ? 4 : NC;

  const int tid = threadIdx.x, lane = tid & 63, wk = tid >> 6;
  const int64_t u = xcd_unit(a.per_xcd);
  if (u >= a.units) return;
  const int g = (int)(u / a.S), s = (int)(u % a.S);
  const int kt0 = (int)((int64_t)s * a.KT / a.S);
  const int kt1 = (int)((int64_t)(s + 1) * a.KT / a.S);
  const int nkt = kt1 - kt0;

  // LDS: the staged activations, later reused for the cross-wave partials
  _Float16 *xs = (_Float16 *)smem;
  float *red = (float *)smem;
  float *vals = (float *)(smem + red_offset<NC, NMAT, RT>(a.nkt_max));

  const int r = lane & 15, sl = lane >> 4;
  const int64_t rt_base = (int64_t)g * RT;

  // ---- 1. start the weight stream: PF tile columns in flight per wave.
  // Row tiles past the matrix (last row group) re-read the last row tile;
  // their results are never written.
  u4 wq[PF][NMAT][RT][QW];
  u2 wd[PF][NMAT][RT];
  auto load = [&](int slot, int kt) {
#pragma unroll
    for (int m = 0; m < NMAT; ++m) {
      const uint8_t *qsm = m ? a.qs1 : a.qs0;
      const uint8_t *dsm = m ? a.d1 : a.d0;
#pragma unroll
      for (int t = 0; t < RT; ++t) {
        const int64_t trow = (rt_base + t < a.NT) ? rt_base + t : (int64_t)a.NT - 1;
        const int64_t tile = trow * a.KT + kt;
        const uint8_t *tp = qsm + tile * TB + lane * 16;
        wq[slot][m][t][0] = ld_stream(tp);
        if constexpr (QW == 2) wq[slot][m][t][QW - 1] = ld_stream(tp + 1024);
        wd[slot][m][t] = ld_stream2(dsm + tile * TILE_D_BYTES + r * 8);
      }
    }
  };
  // wave wk streams the contiguous tile columns [wb, we) of the range
  const int wb = kt0 + (int)((int64_t)nkt * wk / WK);
  const int we = kt0 + (int)((int64_t)nkt * (wk + 1) / WK);
#pragma unroll
  for (int p = 0; p < PF; ++p)
    if (wb + p < we) load(p, wb + p);

  // ---- 2. activations of this K range -> LDS, f16, [block][column][32]
  {
    const int nvec = nkt * TILE_BLOCKS * NC * 4;
    for (int v = tid; v < nvec; v += NTHR) {
      const int q = v & 3, c = (v >> 2) % NC, bl = (v >> 2) / NC;
      const int64_t k = ((int64_t)kt0 * TILE_BLOCKS + bl) * 32 + q * 8;
      h8 hv = {0, 0, 0, 0, 0, 0, 0, 0};
      if (k < a.cols && c < a.ncols) {
        const float4 *p = (const float4 *)(a.X + (int64_t)c * a.ldx + k);
        hv = cvt8(p[0], p[1]);
      }
      *(h8 *)(xs + (size_t)v * 8) = hv;
    }
  }
  __syncthreads();

  // ---- 3. stream the weight tiles
  float acc[NMAT][RT][NACC];
#pragma unroll
  for (int m = 0; m < NMAT; ++m)
#pragma unroll
    for (int t = 0; t < RT; ++t)
#pragma unroll
      for (int c = 0; c < NACC; ++c) acc[m][t][c] = 0.0f;

  auto compute = [&](int slot, int kt) {
    const int bl0 = (kt - kt0) * TILE_BLOCKS;
#pragma unroll
    for (int j = 0; j < TILE_BLOCKS; ++j) {
      if constexpr (MFMA) {
        const h8 A = *(const h8 *)(xs + ((size_t)(bl0 + j) * 16 + r) * 32 + sl * 8);
#pragma unroll
        for (int t = 0; t < RT; ++t) {
          h2 w[4];
          if constexpr (QT == Q4) unpack_q4(wq[slot][0][t][0][j], w);
          else unpack_q8(wq[slot][0][t][j >> 1][(j & 1) * 2], wq[slot][0][t][j >> 1][(j & 1) * 2 + 1], w);
          h8 B = {w[0][0], w[0][1], w[1][0], w[1][1], w[2][0], w[2][1], w[3][0], w[3][1]};
          const f4 D = __builtin_amdgcn_mfma_f32_16x16x32_f16(A, B, f4{0.f, 0.f, 0.f, 0.f}, 0, 0, 0);
          const float dj = scale_of(wd[slot][0][t], j);
#pragma unroll
          for (int i = 0; i < 4; ++i) acc[0][t][i] = __builtin_fmaf(dj, D[i], acc[0][t][i]);
        }
      } else {
        h2 xv[NC][4];
#pragma unroll
        for (int c = 0; c < NC; ++c) {
          const h8 xx = *(const h8 *)(xs + ((size_t)(bl0 + j) * NC + c) * 32 + sl * 8);
#pragma unroll
          for (int p = 0; p < 4; ++p) xv[c][p] = lo_pair(xx, p);
        }
#pragma unroll
        for (int m = 0; m < NMAT; ++m)
#pragma unroll
          for (int t = 0; t < RT; ++t) {
            h2 w[4];
            if constexpr (QT == Q4) unpack_q4(wq[slot][m][t][0][j], w);
            else unpack_q8(wq[slot][m][t][j >> 1][(j & 1) * 2], wq[slot][m][t][j >> 1][(j & 1) * 2 + 1], w);
            const float dj = scale_of(wd[slot][m][t], j);
#pragma unroll
            for (int c = 0; c < NC; ++c) {
              float p = __builtin_amdgcn_fdot2(w[0], xv[c][0], 0.0f, false);
              p = __builtin_amdgcn_fdot2(w[1], xv[c][1], p, false);
              p = __builtin_amdgcn_fdot2(w[2], xv[c][2], p, false);
              p = __builtin_amdgcn_fdot2(w[3], xv[c][3], p, false);
              acc[m][t][c] = __builtin_fmaf(dj, p, acc[m][t][c]);
            }
          }
      }
    }
  };

  for (int kt = wb; kt < we; kt += PF) {
#pragma unroll
    for (int p = 0; p < PF; ++p) {
      const int ktc = kt + p;
      if (ktc < we) {
        compute(p, ktc);
        if (ktc + PF < we) load(p, ktc + PF);
      }
    }
  }

  // ---- 4. reduce inside the workgroup (fixed order)
  __syncthreads();  // every wave is done with the staged activations
  if constexpr (MFMA) {
#pragma unroll
    for (int t = 0; t < RT; ++t)
#pragma unroll
      for (int i = 0; i < 4; ++i)
        red[((wk * RT + t) * 16 + r) * 16 + sl * 4 + i] = acc[0][t][i];
  } else {
#pragma unroll
    for (int m = 0; m < NMAT; ++m)
#pragma unroll
      for (int t = 0; t < RT; ++t)
#pragma unroll
        for (int c = 0; c < NC; ++c) {
          float v = acc[m][t][c];
          v += __shfl_xor(v, 16);
          v += __shfl_xor(v, 32);
          if (sl == 0) red[(((wk * NMAT + m) * RT + t) * 16 + r) * NC + c] = v;
        }
  }
  __syncthreads();

  const int64_t rows_pad = (int64_t)a.NT * 16;
  constexpr int NOUT = RT * 16 * NC;

  auto emit = [&](int t, int rr, int c, const float (&v)[NMAT]) {
    const int64_t row = (rt_base + t) * 16 + rr;
    if (row >= a.rows) {
      if (EPI == EPI_ARGMAX) vals[t * 16 + rr] = 0.0f;
      return;
    }
    float *yp = a.Y + (int64_t)c * a.ldy + row;
    if constexpr (EPI == EPI_STORE) {
      *yp = v[0];
    } else if constexpr (EPI == EPI_ACC) {
      *yp = *yp + v[0];
    } else if constexpr (EPI == EPI_SILU) {
      const float gg = v[0];
      const float sg = gg / (1.0f + expf(-gg));
      *yp = sg * v[NMAT - 1];
    } else {
      vals[t * 16 + rr] = v[0];
    }
  };

  if (a.S == 1) {
    for (int o = tid; o < NOUT; o += NTHR) {
      const int c = o % NC, rr = (o / NC) % 16, t = o / (16 * NC);
      float v[NMAT];
#pragma unroll
      for (int m = 0; m < NMAT; ++m) {
        float x = red[((m * RT + t) * 16 + rr) * NC + c];
#pragma unroll
        for (int w = 1; w < WK; ++w) x += red[(((w * NMAT + m) * RT + t) * 16 + rr) * NC + c];
        v[m] = x;
      }
      emit(t, rr, c, v);
    }
  } else {
    for (int o = tid; o < NOUT; o += NTHR) {
      const int c = o % NC, rr = (o / NC) % 16, t = o / (16 * NC);
      if (rt_base + t >= a.NT) continue;
      const int64_t row = (rt_base + t) * 16 + rr;
#pragma unroll
      for (int m = 0; m < NMAT; ++m) {
        float x = red[((m * RT + t) * 16 + rr) * NC + c];
#pragma unroll
        for (int w = 1; w < WK; ++w) x += red[(((w * NMAT + m) * RT + t) * 16 + rr) * NC + c];
        st_agent(a.part + (((int64_t)s * NMAT + m) * rows_pad + row) * NC + c, x);
      }
    }
    if (!arrive_last(a.cnt + g, (uint32_t)a.S, &flag)) return;
    for (int o = tid; o < NOUT; o += NTHR) {
      const int c = o % NC, rr = (o / NC) % 16, t = o / (16 * NC);
      float v[NMAT];
      if (rt_base + t < a.NT) {
        const int64_t row = (rt_base + t) * 16 + rr;
#pragma unroll
        for (int m = 0; m < NMAT; ++m) {
          float x = ld_agent(a.part + ((int64_t)m * rows_pad + row) * NC + c);
          for (int q = 1; q < a.S; ++q)
            x += ld_agent(a.part + (((int64_t)q * NMAT + m) * rows_pad + row) * NC + c);
          v[m] = x;
        }
      } else {
#pragma unroll
        for (int m = 0; m < NMAT; ++m) v[m] = 0.0f;
      }
      emit(t, rr, c, v);
    }
  }

  if constexpr (EPI == EPI_ARGMAX) {
    // ---- 5. argmax of this row group, then of all row groups
    __syncthreads();
    if (wk == 0) {
      float bv = __builtin_nanf("");
      int32_t bi = 0x7fffffff;
      const int64_t row = rt_base * 16 + lane;
      if (lane < RT * 16 && row < a.rows) { bv = vals[lane]; bi = (int32_t)row; }
#pragma unroll
      for (int off = 32; off >= 1; off >>= 1) {
        const float ov = __shfl_xor(bv, off);
        const int32_t oi = __shfl_xor(bi, off);
        if (ranks_before(ov, oi, bv, bi)) { bv = ov; bi = oi; }
      }
      if (lane == 0) { st_agent(a.cand_v + g, bv); st_agent_u32((uint32_t *)a.cand_i + g, (uint32_t)bi); }
    }
    if (!arrive_last(a.gcnt, (uint32_t)a.G, &flag)) return;
    float bv = __builtin_nanf("");
    int32_t bi = 0x7fffffff;
    for (int q = tid; q < a.G; q += NTHR) {
      const float v = ld_agent(a.cand_v + q);
      const int32_t i = (int32_t)ld_agent_u32((const uint32_t *)a.cand_i + q);
      if (ranks_before(v, i, bv, bi)) { bv = v; bi = i; }
    }
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) {
      const float ov = __shfl_xor(bv, off);
      const int32_t oi = __shfl_xor(bi, off);
      if (ranks_before(ov, oi, bv, bi)) { bv = ov; bi = oi; }
    }
    if (lane == 0) { wave_v[wk] = bv; wave_i[wk] = bi; }
    __syncthreads();
    if (tid == 0) {
      for (int w = 1; w < WK; ++w)
        if (ranks_before(wave_v[w], wave_i[w], bv, bi)) { bv = wave_v[w]; bi = wave_i[w]; }
      *a.out_idx = bi;
      if (a.out_val) *a.out_val = bv;
    }
  }
}

// ---------------------------------------------------------------- host side
static int64_t cdiv(int64_t a, int64_t b) { return (a + b - 1) / b; }

int gemv_splits(int64_t rows, int64_t cols) {
  const int64_t NT = cdiv(rows, 16), KT = cdiv(cols / 32, 4);
  int64_t s = cdiv(2048, NT);                       // >= ~512 workgroups at 1 column
  const int64_t cap = KT / (2 * WK);                // >= 2 tile columns per wave
  if (s > cap) s = cap;
  const int64_t lds_min = cdiv(KT, 32);             // 8 columns of f16 x in <= 64 KiB
  if (s < lds_min) s = lds_min;
  if (s < 1) s = 1;
  if (s > KT) s = KT;
  return (int)s;
}

int gemm16_splits(int64_t rows, int64_t cols) {
  const int64_t NT = cdiv(rows, 16), KT = cdiv(cols / 32, 4);
  int64_t s = cdiv(2048, NT);
  const int64_t cap = KT / (2 * WK);
  if (s > cap) s = cap;
  const int64_t lds_min = cdiv(KT, 16);             // 16 columns of f16 x in <= 64 KiB
  if (s < lds_min) s = lds_min;
  if (s < 1) s = 1;
  if (s > KT) s = KT;
  return (int)s;
}

size_t qmv_ws_bytes(int64_t rows, int64_t cols, int splits, int nmat, int ncols_max, bool argmax) {
  const int64_t NT = cdiv(rows, 16);
  (void)cols;
  size_t b = align256((size_t)NT * 4);              // split counters
  b += 256;                                         // argmax counter
  if (argmax) b += 2 * align256((size_t)NT * 4);    // candidates
  if (splits > 1) b += (size_t)splits * nmat * NT * 16 * ncols_max * 4;
  return b;
}

template <int QT, int NC, int NMAT, int EPI, bool MFMA, int RT>
static int launch_t(const QmvCall &c) {
  const int64_t NT = cdiv(c.rows, 16), KT = cdiv(c.cols / 32, 4);
  const int64_t NTu = cdiv(c.n_rows, 16);           // tiles actually produced
  QmvArgs a;
  a.qs0 = (const uint8_t *)c.qs[0];
  a.d0 = (const uint8_t *)c.d[0];
  a.qs1 = (const uint8_t *)c.qs[NMAT - 1];
  a.d1 = (const uint8_t *)c.d[NMAT - 1];
  a.rows = c.n_rows;
  a.cols = c.cols;
  a.NT = (int)NTu;
  a.KT = (int)KT;
  a.S = MFMA ? gemm16_splits(c.rows, c.cols) : gemv_splits(c.rows, c.cols);
  a.G = (int)cdiv(NTu, RT);
  a.units = (int64_t)a.G * a.S;
  a.per_xcd = cdiv(a.units, 8);
  a.nkt_max = (int)cdiv(KT, a.S);
  a.X = c.X;
  a.ldx = c.ldx;
  a.ncols = c.ncols;
  a.Y = c.Y;
  a.ldy = c.ldy;
  uint8_t *ws = (uint8_t *)c.ws;
  a.cnt = (uint32_t *)ws;
  size_t off = align256((size_t)NT * 4);
  a.gcnt = (uint32_t *)(ws + off);
  off += 256;
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
  // partial sums are indexed with the padded row count of the produced tiles
  const size_t need = off + (a.S > 1 ? (size_t)a.S * NMAT * NTu * 16 * NC * 4 : 0);
  if (need > c.ws_bytes) return QG_EWORKSPACE;

  const size_t lds = red_offset<NC, NMAT, RT>(a.nkt_max) + (EPI == EPI_ARGMAX ? (size_t)RT * 16 * 4 : 0);
  auto kern = qmv_kernel<QT, NC, NMAT, EPI, MFMA, RT>;
  if (lds > 65536) {
    static size_t granted = 0;  // per instantiation; raised once, never lowered
    if (lds > granted) {
      if (hipFuncSetAttribute((const void *)kern, hipFuncAttributeMaxDynamicSharedMemorySize, 163840) !=
          hipSuccess)
        return QG_EHIP;
      granted = 163840;
    }
    if (lds > 163840) return QG_EUNSUPPORTED;
  }
  const int64_t grid = a.per_xcd * 8;
  clear_hip_error();
  hipLaunchKernelGGL(kern, dim3((unsigned)grid), dim3(NTHR), lds, c.stream, a);
  return launch_status();
}

template <int QT, int EPI>
static int dispatch_dot(const QmvCall &c) {
  switch (c.ncols) {
    case 1: return launch_t<QT, 1, 1, EPI, false, rt_dot<1, 1>()>(c);
    case 2: return launch_t<QT, 2, 1, EPI, false, rt_dot<2, 1>()>(c);
    case 3: return launch_t<QT, 3, 1, EPI, false, rt_dot<3, 1>()>(c);
    case 4: return launch_t<QT, 4, 1, EPI, false, rt_dot<4, 1>()>(c);
    case 5: return launch_t<QT, 5, 1, EPI, false, rt_dot<5, 1>()>(c);
    case 6: return launch_t<QT, 6, 1, EPI, false, rt_dot<6, 1>()>(c);
    case 7: return launch_t<QT, 7, 1, EPI, false, rt_dot<7, 1>()>(c);
    case 8: return launch_t<QT, 8, 1, EPI, false, rt_dot<8, 1>()>(c);
  }
  return QG_ESHAPE;
}

template <int QT>
static int dispatch_silu(const QmvCall &c) {
  switch (c.ncols) {
    case 1: return launch_t<QT, 1, 2, EPI_SILU, false, rt_dot<1, 2>()>(c);
    case 2: return launch_t<QT, 2, 2, EPI_SILU, false, rt_dot<2, 2>()>(c);
    case 3: return launch_t<QT, 3, 2, EPI_SILU, false, rt_dot<3, 2>()>(c);
    case 4: return launch_t<QT, 4, 2, EPI_SILU, false, rt_dot<4, 2>()>(c);
    case 5: return launch_t<QT, 5, 2, EPI_SILU, false, rt_dot<5, 2>()>(c);
    case 6: return launch_t<QT, 6, 2, EPI_SILU, false, rt_dot<6, 2>()>(c);
    case 7: return launch_t<QT, 7, 2, EPI_SILU, false, rt_dot<7, 2>()>(c);
    case 8: return launch_t<QT, 8, 2, EPI_SILU, false, rt_dot<8, 2>()>(c);
  }
  return QG_ESHAPE;
}

template <int QT>
static int dispatch_qt(const QmvCall &c) {
  if (c.ncols == 16) {
    if (c.epi == EPI_STORE) return launch_t<QT, 16, 1, EPI_STORE, true, RT_MFMA>(c);
    if (c.epi == EPI_ACC) return launch_t<QT, 16, 1, EPI_ACC, true, RT_MFMA>(c);
    return QG_EUNSUPPORTED;
  }
  switch (c.epi) {
    case EPI_STORE: return dispatch_dot<QT, EPI_STORE>(c);
    case EPI_ACC: return dispatch_dot<QT, EPI_ACC>(c);
    case EPI_SILU: return dispatch_silu<QT>(c);
    case EPI_ARGMAX:
      if (c.ncols != 1) return QG_ESHAPE;
      return launch_t<QT, 1, 1, EPI_ARGMAX, false, rt_dot<1, 1>()>(c);
  }
  return QG_EINVAL;
}

int launch_qmv(const QmvCall &c) {
  if (c.qtype == QG_Q4_0) return dispatch_qt<Q4>(c);
  if (c.qtype == QG_Q8_0) return dispatch_qt<Q8>(c);
  return QG_EINVAL;
}

}  // namespace qg
