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
//  * K is cut into Q contiguous segments, Q a function of the matrix shape
//    only.  One wave streams one segment for RT row tiles (16 rows each),
//    PF tile columns ahead, with nontemporal 16-byte loads: a wave reads a
//    contiguous 1 KiB stripe per load, so every HBM read is fully coalesced.
//  * A workgroup of WKT waves takes WKT consecutive segments of the same row
//    tiles; their activations are staged once in LDS as f16, laid out
//    [block][column][32], and read with broadcast.  When the segments of a
//    row group need more than one workgroup (wide batches with long K), the
//    last workgroup to finish combines them.
//  * Dot path (1..8 columns): weights become exact f16 pairs and meet the
//    activations in v_dot2_f32_f16; each block's partial is scaled by its
//    f16 scale in f32.
//  * Matrix-core path (16 columns): one v_mfma_f32_16x16x32_f16 per block
//    and row tile, A = activations (16 columns x 32), B = the block's
//    weights; the block scale multiplies the 4 outputs each lane holds.
//  * Reduction order, dot path: tile columns in order within a wave, a
//    2-step lane butterfly, then the Q segment partials summed in segment
//    order.  It depends on the shape only, so column j of a batched call is
//    bitwise equal to a 1-column call on that column ("Architecture",
//    Speculative decoding: each checked column gives bit-identical logits).
//    Matrix-core path: waves of a workgroup, then splits, in index order.
#include "common.h"
#include "internal.h"
#include "qgemm.h"

namespace qg {

struct QmvArgs {
  const uint8_t *qs0, *qs1, *d0, *d1;
  int64_t rows;       // outputs produced (n_rows for the LM head)
  int64_t cols;
  int NT, KT;         // row tiles produced, tile columns of the matrix
  int Q;              // K segments (dot path) or waves x splits (matrix cores)
  int S;              // workgroups per row group
  int G;              // row groups of RT tiles
  int64_t units;      // G * S
  int64_t per_xcd;
  int nkt_max;        // tile columns staged by the widest workgroup
  const float *X;
  int64_t ldx;
  int ncols;
  float *Y;
  int64_t ldy;
  float *part;        // partial sums exchanged between workgroups
  uint32_t *cnt;      // [G]
  uint32_t *gcnt;     // argmax: one counter
  float *cand_v;      // argmax: [G]
  int32_t *cand_i;
  int32_t *out_idx;
  float *out_val;
};

static size_t align256(size_t v) { return (v + 255) & ~size_t(255); }
static int64_t cdiv(int64_t a, int64_t b) { return (a + b - 1) / b; }

// Segment q of a K range of kt tile columns cut into n pieces.
__host__ __device__ inline int seg_begin(int q, int kt, int n) { return (int)((int64_t)kt * q / n); }

template <int QT, int NC, int NMAT, int EPI, bool MFMA, int RT, int PF, int WKT>
__global__ void __launch_bounds__(WKT * 64) qmv_kernel(QmvArgs a) {
  constexpr int NTHR = WKT * 64;
  extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
  __shared__ uint32_t flag;
  __shared__ float wave_v[WKT];
  __shared__ int32_t wave_i[WKT];

  constexpr int TB = QTraits<QT>::tile_bytes;
  constexpr int QW = (QT == Q4) ? 1 : 2;   // 16-byte loads per lane per tile
  constexpr int NACC = MFMA ? 4 : NC;

  // the wave index is uniform across the wave; readfirstlane tells the
  // compiler, so segment bounds and tile addresses live in scalar registers
  const int tid = threadIdx.x, lane = tid & 63;
  const int wk = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int64_t u = xcd_unit(a.per_xcd);
  if (u >= a.units) return;
  const int g = (int)(u / a.S), s = (int)(u % a.S);
  // segments of this workgroup: [q0, q1); its tile columns [kt0, kt1)
  const int q0 = s * WKT;
  const int q1 = (q0 + WKT < a.Q) ? q0 + WKT : a.Q;
  const int kt0 = seg_begin(q0, a.KT, a.Q);
  const int kt1 = seg_begin(q1, a.KT, a.Q);
  const int nkt = kt1 - kt0;
  // this wave's segment
  const int q = q0 + wk;
  const int wb = q < q1 ? seg_begin(q, a.KT, a.Q) : kt1;
  const int we = q < q1 ? seg_begin(q + 1, a.KT, a.Q) : kt1;

  // LDS: the staged activations, later reused for the per-wave partials
  _Float16 *xs = (_Float16 *)smem;
  float *red = (float *)smem;
  const size_t x_bytes = (size_t)a.nkt_max * TILE_BLOCKS * NC * 64;
  const size_t r_bytes = (size_t)WKT * NMAT * RT * 16 * NC * 4;
  float *vals = (float *)(smem + (x_bytes > r_bytes ? x_bytes : r_bytes));

  const int r = lane & 15, sl = lane >> 4;
  const int64_t rt_base = (int64_t)g * RT;

  // ---- 1. start the weight stream: PF tile columns in flight per wave.
  // Row tiles past the matrix (last row group) re-read the last row tile;
  // their results are never written.
  u4 wq[PF][NMAT][RT][QW];
  u2 wd[PF][NMAT][RT];
  // 32-bit lane offsets: uniform base + zero-extended offset addressing
  const uint32_t lane_off = (uint32_t)lane * 16u, d_off = (uint32_t)r * 8u;
  auto load = [&](int slot, int kt) {
#pragma unroll
    for (int m = 0; m < NMAT; ++m) {
      const uint8_t *qsm = m ? a.qs1 : a.qs0;
      const uint8_t *dsm = m ? a.d1 : a.d0;
#pragma unroll
      for (int t = 0; t < RT; ++t) {
        const int64_t trow = (rt_base + t < a.NT) ? rt_base + t : (int64_t)a.NT - 1;
        const int64_t tile = trow * a.KT + kt;
        const uint8_t *tq = qsm + tile * TB;            // uniform
        const uint8_t *td = dsm + tile * TILE_D_BYTES;  // uniform
        wq[slot][m][t][0] = ld_stream(tq + lane_off);
        if constexpr (QW == 2) wq[slot][m][t][QW - 1] = ld_stream(tq + 1024 + lane_off);
        wd[slot][m][t] = ld_stream2(td + d_off);
      }
    }
  };
  // prologue: tile columns wb .. wb+PF-1 (clamped to the segment, so that
  // no branch separates these loads from their uses)
  const int nseg = we - wb;  // 0 for a wave without a segment
  if (nseg > 0) {
#pragma unroll
    for (int p = 0; p < PF; ++p) load(p, wb + (p < nseg ? p : nseg - 1));
  }

  // ---- 2. activations of this K range -> LDS, f16, [block][column][32]
  // Each thread converts 8 consecutive k of one column per chunk.  Chunks go
  // in batches of XB whose loads are all issued before any is used (an
  // out-of-range chunk re-reads column 0, k 0 and stores zeros), so staging
  // costs about one L2 round trip per batch instead of one per chunk.
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
        ok[b] = v < nvec && k < a.cols && c < a.ncols;
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

  // ---- 3. stream the weight tiles
  float acc[NMAT][RT][NACC];
#pragma unroll
  for (int m = 0; m < NMAT; ++m)
#pragma unroll
    for (int t = 0; t < RT; ++t)
#pragma unroll
      for (int c = 0; c < NACC; ++c) acc[m][t][c] = 0.0f;

  const Q4Magic mg = q4_magic();
  auto compute = [&](int slot, int kt) {
    const int bl0 = (kt - kt0) * TILE_BLOCKS;
#pragma unroll
    for (int j = 0; j < TILE_BLOCKS; ++j) {
      if constexpr (MFMA) {
        const h8 A = *(const h8 *)(xs + ((size_t)(bl0 + j) * 16 + r) * 32 + sl * 8);
#pragma unroll
        for (int t = 0; t < RT; ++t) {
          h2 w[4];
          if constexpr (QT == Q4) unpack_q4(wq[slot][0][t][0][j], w, mg);
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
            if constexpr (QT == Q4) unpack_q4(wq[slot][m][t][0][j], w, mg);
            else unpack_q8(wq[slot][m][t][j >> 1][(j & 1) * 2], wq[slot][m][t][j >> 1][(j & 1) * 2 + 1], w);
            const float dj = scale_of(wd[slot][m][t], j);
#pragma unroll
            for (int c = 0; c < NC; ++c) {
              float p = dot2_first(w[0], xv[c][0]);
              p = __builtin_amdgcn_fdot2(w[1], xv[c][1], p, false);
              p = __builtin_amdgcn_fdot2(w[2], xv[c][2], p, false);
              p = __builtin_amdgcn_fdot2(w[3], xv[c][3], p, false);
              acc[m][t][c] = __builtin_fmaf(dj, p, acc[m][t][c]);
            }
          }
      }
    }
  };

  // steady state: branch-free, PF tile columns always in flight (the loop
  // condition guarantees every load below is inside the segment)
  int k = 0;
  for (; k + 2 * PF <= nseg; k += PF) {
#pragma unroll
    for (int p = 0; p < PF; ++p) {
      compute(p, wb + k + p);
      load(p, wb + k + p + PF);
    }
  }
  // drain: fewer than 2*PF tile columns left
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

  // ---- 4. per-wave partials -> LDS
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
  const int nw = q1 - q0;  // waves of this workgroup that own a segment
  auto red_at = [&](int w, int m, int t, int rr, int c) -> float {
    return red[(((w * NMAT + m) * RT + t) * 16 + rr) * NC + c];
  };

  auto emit = [&](int t, int rr, int c, const float (&v)[NMAT]) {
    const int64_t row = (rt_base + t) * 16 + rr;
    if (row >= a.rows) {
      if (EPI == EPI_ARGMAX) vals[t * 16 + rr] = 0.0f;
      return;
    }
    if constexpr (EPI == EPI_ARGMAX) {
      vals[t * 16 + rr] = v[0];
    } else {
      float *yp = a.Y + (int64_t)c * a.ldy + row;
      if constexpr (EPI == EPI_STORE) {
        *yp = v[0];
      } else if constexpr (EPI == EPI_ACC) {
        *yp = *yp + v[0];
      } else {
        const float gg = v[0];
        const float sg = gg / (1.0f + expf(-gg));
        *yp = sg * v[NMAT - 1];
      }
    }
  };

  if (a.S == 1) {
    for (int o = tid; o < NOUT; o += NTHR) {
      const int c = o % NC, rr = (o / NC) % 16, t = o / (16 * NC);
      float v[NMAT];
#pragma unroll
      for (int m = 0; m < NMAT; ++m) {
        float x = red_at(0, m, t, rr, c);
        for (int w = 1; w < nw; ++w) x += red_at(w, m, t, rr, c);
        v[m] = x;
      }
      emit(t, rr, c, v);
    }
  } else {
    // Dot path: publish every segment partial (partial q at slot q).
    // Matrix cores: publish the workgroup sum (slot s).
    for (int o = tid; o < NOUT; o += NTHR) {
      const int c = o % NC, rr = (o / NC) % 16, t = o / (16 * NC);
      if (rt_base + t >= a.NT) continue;
      const int64_t row = (rt_base + t) * 16 + rr;
#pragma unroll
      for (int m = 0; m < NMAT; ++m) {
        if constexpr (MFMA) {
          float x = red_at(0, m, t, rr, c);
          for (int w = 1; w < nw; ++w) x += red_at(w, m, t, rr, c);
          st_agent(a.part + (((int64_t)s * NMAT + m) * rows_pad + row) * NC + c, x);
        } else {
          for (int w = 0; w < nw; ++w)
            st_agent(a.part + (((int64_t)(q0 + w) * NMAT + m) * rows_pad + row) * NC + c, red_at(w, m, t, rr, c));
        }
      }
    }
    if (!arrive_last(a.cnt + g, (uint32_t)a.S, &flag)) return;
    const int nslots = MFMA ? a.S : a.Q;
    for (int o = tid; o < NOUT; o += NTHR) {
      const int c = o % NC, rr = (o / NC) % 16, t = o / (16 * NC);
      float v[NMAT];
      if (rt_base + t < a.NT) {
        const int64_t row = (rt_base + t) * 16 + rr;
#pragma unroll
        for (int m = 0; m < NMAT; ++m) {
          float x = ld_agent(a.part + ((int64_t)m * rows_pad + row) * NC + c);
          for (int qq = 1; qq < nslots; ++qq)
            x += ld_agent(a.part + (((int64_t)qq * NMAT + m) * rows_pad + row) * NC + c);
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

// ---------------------------------------------------------------- host side
static int64_t pow2ceil(int64_t v) {
  int64_t p = 1;
  while (p < v) p <<= 1;
  return p;
}
static int64_t pow2floor(int64_t v) {
  int64_t p = 1;
  while (p * 2 <= v) p <<= 1;
  return p;
}

constexpr size_t LDS_SOFT = 81920;    // keeps two or more workgroups per CU
constexpr size_t LDS_HARD = 163840;   // gfx950 LDS per workgroup

// Segments of K for the dot path: enough waves to fill the GPU at one
// column (about 2048 waves for two row tiles per wave), at least two tile
// columns per segment, and few enough tile columns per workgroup that eight
// columns of f16 activations of four segments fit in LDS.
int gemv_segments(int64_t rows, int64_t cols) {
  const int64_t NT = cdiv(rows, 16), KT = cdiv(cols / 32, 4);
  int64_t q = pow2ceil(cdiv(2048, cdiv(NT, 2)));
  if (q < 4) q = 4;
  if (q > 16) q = 16;
  const int64_t qmax = pow2floor(KT / 2 > 1 ? KT / 2 : 1);
  if (q > qmax) q = qmax;
  const int64_t lds_q = pow2ceil(cdiv(KT * TILE_BLOCKS * 8 * 64 * 4, (int64_t)LDS_HARD - 8192));
  if (q < lds_q) q = lds_q;
  if (q > KT) q = KT;
  return (int)q;
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

template <int QT, int NC, int NMAT, int EPI, bool MFMA, int RT, int PF, int WKT>
static int launch_t(const QmvCall &c, int Q, int S) {
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
  a.Q = Q;
  a.S = S;
  a.G = (int)cdiv(NTu, RT);
  a.units = (int64_t)a.G * a.S;
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
  const int slots = MFMA ? S : Q;
  const size_t need = off + (S > 1 ? (size_t)slots * NMAT * NTu * 16 * NC * 4 : 0);
  if (need > c.ws_bytes) return QG_EWORKSPACE;

  const size_t x_bytes = (size_t)nkt_max * TILE_BLOCKS * NC * 64;
  const size_t r_bytes = (size_t)WKT * NMAT * RT * 16 * NC * 4;
  const size_t lds = (x_bytes > r_bytes ? x_bytes : r_bytes) + (EPI == EPI_ARGMAX ? (size_t)RT * 16 * 4 : 0);
  if (lds > LDS_HARD - 1024) return QG_EUNSUPPORTED;  // static LDS needs the rest
  auto kern = qmv_kernel<QT, NC, NMAT, EPI, MFMA, RT, PF, WKT>;
  if (lds > 65536) {
    static size_t granted = 65536;  // per instantiation; only ever raised
    if (lds > granted) {
      const hipError_t e = hipFuncSetAttribute((const void *)kern, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
      if (e != hipSuccess) {
        record_hip_error(e);
        return QG_EHIP;
      }
      granted = lds;
    }
  }
  const int64_t grid = a.per_xcd * 8;
  clear_hip_error();
  hipLaunchKernelGGL(kern, dim3((unsigned)grid), dim3(WKT * 64), lds, c.stream, a);
  return launch_status();
}

// Staged activation bytes of the widest workgroup when WKT waves take
// consecutive segments
static size_t x_lds(int64_t KT, int Q, int wkt, int nc) {
  int nmax = 0;
  for (int s = 0; s * wkt < Q; ++s) {
    const int q0 = s * wkt, q1 = q0 + wkt < Q ? q0 + wkt : Q;
    const int n = seg_begin(q1, (int)KT, Q) - seg_begin(q0, (int)KT, Q);
    if (n > nmax) nmax = n;
  }
  return (size_t)nmax * TILE_BLOCKS * nc * 64;
}

// Dot path: RT row tiles per wave keeps at most 16 accumulators per lane
// ("Engine and kernels", verify twins keep 16 accumulators per thread);
// PF keeps about eight 16-byte loads in flight per lane.
template <int QT, int NC, int NMAT, int EPI>
static int launch_dot(const QmvCall &c) {
  constexpr int QW = QT == Q4 ? 1 : 2;
  constexpr int RT = NC == 1 ? (NMAT == 1 ? 2 : 1)
                             : (NC * NMAT * QW > 4 ? 1
                                                   : ((16 / (NC * NMAT)) < 1 ? 1 : ((16 / (NC * NMAT)) > 2 ? 2 : 16 / (NC * NMAT))));
  constexpr int PF0 = 8 / (RT * NMAT * QW);
  constexpr int PF = PF0 < 2 ? 2 : (PF0 > 4 ? 4 : PF0);
  const int Q = gemv_segments(c.rows, c.cols);
  const int64_t KT = cdiv(c.cols / 32, 4);
  // the widest workgroup (fewest workgroups per row group) whose staged
  // activations fit; 16-wave workgroups (128 VGPRs) only where they do not
  // spill: one column of one matrix
  if constexpr (NC == 1 && NMAT == 1) {
    if (Q >= 16 && x_lds(KT, Q, 16, NC) <= LDS_SOFT)
      return launch_t<QT, NC, NMAT, EPI, false, RT, PF, 16>(c, Q, 1);
  }
  if (Q >= 8 && x_lds(KT, Q, 8, NC) <= (NC == 1 ? LDS_SOFT : LDS_HARD))
    return launch_t<QT, NC, NMAT, EPI, false, RT, PF, 8>(c, Q, (int)cdiv(Q, 8));
  return launch_t<QT, NC, NMAT, EPI, false, RT, PF, 4>(c, Q, (int)cdiv(Q, 4));
}

template <int QT, int EPI>
static int dispatch_dot(const QmvCall &c) {
  switch (c.ncols) {
    case 1: return launch_dot<QT, 1, 1, EPI>(c);
    case 2: return launch_dot<QT, 2, 1, EPI>(c);
    case 3: return launch_dot<QT, 3, 1, EPI>(c);
    case 4: return launch_dot<QT, 4, 1, EPI>(c);
    case 5: return launch_dot<QT, 5, 1, EPI>(c);
    case 6: return launch_dot<QT, 6, 1, EPI>(c);
    case 7: return launch_dot<QT, 7, 1, EPI>(c);
    case 8: return launch_dot<QT, 8, 1, EPI>(c);
  }
  return QG_ESHAPE;
}

template <int QT>
static int dispatch_silu(const QmvCall &c) {
  switch (c.ncols) {
    case 1: return launch_dot<QT, 1, 2, EPI_SILU>(c);
    case 2: return launch_dot<QT, 2, 2, EPI_SILU>(c);
    case 3: return launch_dot<QT, 3, 2, EPI_SILU>(c);
    case 4: return launch_dot<QT, 4, 2, EPI_SILU>(c);
    case 5: return launch_dot<QT, 5, 2, EPI_SILU>(c);
    case 6: return launch_dot<QT, 6, 2, EPI_SILU>(c);
    case 7: return launch_dot<QT, 7, 2, EPI_SILU>(c);
    case 8: return launch_dot<QT, 8, 2, EPI_SILU>(c);
  }
  return QG_ESHAPE;
}

template <int QT, int EPI>
static int launch_mfma(const QmvCall &c) {
  const int S = gemm16_splits(c.rows, c.cols);
  return launch_t<QT, 16, 1, EPI, true, 4, 2, 4>(c, 4 * S, S);
}

template <int QT>
static int dispatch_qt(const QmvCall &c) {
  if (c.ncols == 16) {
    if (c.epi == EPI_STORE) return launch_mfma<QT, EPI_STORE>(c);
    if (c.epi == EPI_ACC) return launch_mfma<QT, EPI_ACC>(c);
    return QG_EUNSUPPORTED;
  }
  switch (c.epi) {
    case EPI_STORE: return dispatch_dot<QT, EPI_STORE>(c);
    case EPI_ACC: return dispatch_dot<QT, EPI_ACC>(c);
    case EPI_SILU: return dispatch_silu<QT>(c);
    case EPI_ARGMAX:
      if (c.ncols != 1) return QG_ESHAPE;
      return launch_dot<QT, 1, 1, EPI_ARGMAX>(c);
  }
  return QG_EINVAL;
}

int launch_qmv(const QmvCall &c) {
  if (c.qtype == QG_Q4_0) return dispatch_qt<Q4>(c);
  if (c.qtype == QG_Q8_0) return dispatch_qt<Q8>(c);
  return QG_EINVAL;
}

}  // namespace qg
