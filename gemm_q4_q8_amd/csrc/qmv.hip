// Tiled quantised products on gfx950: the decode GEMV and its batched twins
// (1..8 columns), the fused gate/up with SiLU, the LM head with argmax, and
// the 16-column prefill GEMM.
//
// What is computed ("Engine and kernels", Kernel families and What each
// trick bought): y = W x over Q4_0 / Q8_0 blocks dequantised in registers,
// f32 sums, optional y += W x into the residual, gate/up fused with SiLU
// before writing, greedy argmax with lowest-index ties, and a 16-column GEMM
// with split-K pinned per shape.
//
// One kernel, dot_kernel: a workgroup per (row group, K segment) runs the
// work unit of dot_unit.h (activation staging, weight streaming, block
// products on the matrix cores, segment reduction, epilogue); the argmax
// across row groups is added here.  K segments per shape: gemv_segments()
// (1..8 columns, the same for every column count) and gemm16_splits().
#include <string.h>

#include <algorithm>

#include "common.h"
#include "dot_unit.h"
#include "internal.h"
#include "qgemm.h"

namespace qg {

static size_t align256(size_t v) { return (v + 255) & ~size_t(255); }
static int64_t cdiv(int64_t a, int64_t b) { return (a + b - 1) / b; }

// --------------------------------------------------------------- dot path
// WKT > 0: workgroups of WKT waves; WKT == 0: as many waves as launched, at
// most WMAX (the launch planner picks the size per shape).
template <int QT, int NC, int NMAT, int EPI, int RT, int PF, int WKT, int WMAX, bool RMSN = false>
__global__ void __launch_bounds__(WMAX * 64) dot_kernel(DotArgs a) {
  static_assert(WKT <= WMAX, "workgroup size");
  const int NTHR = WKT > 0 ? WKT * 64 : (int)blockDim.x;
  const int NW = NTHR >> 6;
  extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
  __shared__ uint32_t flag;
  __shared__ float wave_v[WMAX];
  __shared__ int32_t wave_i[WMAX];

  const int tid = threadIdx.x, lane = tid & 63;
  const int wk = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int64_t u = xcd_unit(a.per_xcd);
  if (u >= a.units) return;
  const int g = (int)(u / a.S), s = (int)(u % a.S);
  float bv = __builtin_nanf("");  // argmax: this lane's best (value, row)
  int32_t bi = 0x7fffffff;
  const bool emitted =
      dot_unit<QT, NC, NMAT, EPI, RT, PF, WKT, PH_PLAIN, RMSN>(a, g, s, smem, &flag, bv, bi);

  if constexpr (EPI == EPI_TOPK) {
    if (!emitted) return;
    // ---- the k best rows of this row group: each emitting lane holds one
    // row (bv, bi), the others none; rank keys (value descending, index
    // ascending; 0 = none), k rounds of a wave maximum in wave 0
    __shared__ uint64_t s_key[WMAX * 64];
    const int k = a.topk;
    s_key[tid] = bi != 0x7fffffff ? rank_key(bv, bi) : 0;
    __syncthreads();
    if (wk == 0) {
      uint64_t key[WMAX];
      uint64_t loc = 0;
#pragma unroll
      for (int j = 0; j < WMAX; ++j) {
        key[j] = j < NW ? s_key[lane + 64 * j] : 0;
        loc = key[j] > loc ? key[j] : loc;
      }
      uint64_t mine = 0;  // lane kk: the key of rank kk
      for (int kk = 0; kk < k; ++kk) {
        const uint64_t w = wave_max_key(loc);
        if (lane == kk) mine = w;
        if (w != 0 && loc == w) {  // the owner drops the winner
          loc = 0;
#pragma unroll
          for (int j = 0; j < WMAX; ++j) {
            if (key[j] == w) key[j] = 0;
            loc = key[j] > loc ? key[j] : loc;
          }
        }
      }
      if (lane < k) st_agent_u64(a.cand_k + (int64_t)g * k + lane, mine);
    }
    if (!arrive_last(a.gcnt, (uint32_t)a.G, &flag)) return;
    // ---- merge of the G * k candidates.  Each thread keeps the best
    // QG_TOPK_MAX of its share, sorted (an exchange chain per candidate;
    // candidates loaded TKB at a time with coherent loads over a bounded
    // range, slots past the end read 0 = none) ...
    const int64_t nc = (int64_t)a.G * k;
    uint64_t top[QG_TOPK_MAX];
#pragma unroll
    for (int j = 0; j < QG_TOPK_MAX; ++j) top[j] = 0;
    const __amdgpu_buffer_rsrc_t rk = buf_range(a.cand_k, (uint32_t)(nc * 8));
    constexpr int TKB = 16;
    for (int64_t q0 = tid; q0 < nc; q0 += TKB * NTHR) {
      uint64_t v[TKB];
#pragma unroll
      for (int b = 0; b < TKB; ++b) {
        const int64_t q = q0 + (int64_t)b * NTHR;
        const u2 p = __builtin_amdgcn_raw_buffer_load_b64(rk, q < nc ? (uint32_t)(q * 8) : 0xFFFFFFC0u, 0, 16);
        v[b] = ((uint64_t)p[1] << 32) | p[0];
      }
#pragma unroll
      for (int b = 0; b < TKB; ++b) {
        uint64_t c = v[b];
#pragma unroll
        for (int j = 0; j < QG_TOPK_MAX; ++j) {
          const uint64_t hi = c > top[j] ? c : top[j];
          c = c > top[j] ? top[j] : c;
          top[j] = hi;
        }
      }
    }
    // ... each wave takes its k best heads (the owner of a head pops it) ...
    __syncthreads();  // s_key is reused
    for (int kk = 0; kk < k; ++kk) {
      const uint64_t w = wave_max_key(top[0]);
      if (lane == 0) s_key[wk * QG_TOPK_MAX + kk] = w;
      if (w != 0 && top[0] == w) {
#pragma unroll
        for (int j = 0; j < QG_TOPK_MAX - 1; ++j) top[j] = top[j + 1];
        top[QG_TOPK_MAX - 1] = 0;
      }
    }
    __syncthreads();
    // ... and wave 0 merges the waves' lists
    if (wk == 0) {
      constexpr int NJ = (WMAX * QG_TOPK_MAX + 63) / 64;
      uint64_t key[NJ];
      uint64_t loc = 0;
#pragma unroll
      for (int j = 0; j < NJ; ++j) {
        const int e = lane + 64 * j;
        key[j] = (e / QG_TOPK_MAX < NW && e % QG_TOPK_MAX < k) ? s_key[e] : 0;
        loc = key[j] > loc ? key[j] : loc;
      }
      uint64_t mine = 0;
      for (int kk = 0; kk < k; ++kk) {
        const uint64_t w = wave_max_key(loc);
        if (lane == kk) mine = w;
        if (w != 0 && loc == w) {
          loc = 0;
#pragma unroll
          for (int j = 0; j < NJ; ++j) {
            if (key[j] == w) key[j] = 0;
            loc = key[j] > loc ? key[j] : loc;
          }
        }
      }
      if (lane < k) {
        a.out_idx[lane] = rank_key_index(mine);
        if (a.out_val) a.out_val[lane] = rank_key_value(mine);
      }
    }
  }

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
      for (int w = 1; w < NW; ++w)
        if (ranks_before(wave_v[w], wave_i[w], bv, bi)) { bv = wave_v[w]; bi = wave_i[w]; }
      st_agent(a.cand_v + g, bv);
      st_agent_u32((uint32_t *)a.cand_i + g, (uint32_t)bi);
    }
    if (!arrive_last(a.gcnt, (uint32_t)a.G, &flag)) return;
    bv = __builtin_nanf("");
    bi = 0x7fffffff;
    // candidates in batches of 4 per thread, all loaded before any is used
    // (coherent loads over bounded ranges; slots past G are skipped)
    const __amdgpu_buffer_rsrc_t rv = buf_range(a.cand_v, (uint32_t)a.G * 4u);
    const __amdgpu_buffer_rsrc_t ri = buf_range(a.cand_i, (uint32_t)a.G * 4u);
    for (int q0 = tid; q0 < a.G; q0 += 4 * NTHR) {
      float v[4];
      int32_t id[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int q = q0 + j * NTHR;
        const uint32_t o = q < a.G ? (uint32_t)q * 4u : 0xFFFFFFC0u;
        v[j] = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(rv, o, 0, 16));
        id[j] = (int32_t)__builtin_amdgcn_raw_buffer_load_b32(ri, o, 0, 16);
      }
#pragma unroll
      for (int j = 0; j < 4; ++j)
        if (q0 + j * NTHR < a.G && ranks_before(v[j], id[j], bv, bi)) { bv = v[j]; bi = id[j]; }
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
      for (int w = 1; w < NW; ++w)
        if (ranks_before(wave_v[w], wave_i[w], bv, bi)) { bv = wave_v[w]; bi = wave_i[w]; }
      *a.out_idx = bi;
      if (a.out_val) *a.out_val = bv;
    }
  }
}

// ----------------------------------------------- grouped 16-column problems
// One launch over several 16-column problems (a prefill pass through several
// matrices).  Each workgroup takes one work unit (row group of G16_W row
// tiles, K segment) of one problem, with the problem's own K segments and
// order, so every output is bitwise equal to the single-problem call.  The
// workgroups are small, so several reside on each CU: while one stages its
// activations, publishes its partial sums or waits for its first weights,
// the others stream, and the units of the next problem start as soon as
// CUs free up, without a launch boundary between problems.  The units are
// those of the single-problem call with 8 waves (its activations stream in
// chunks of G16_PF tile columns).  Measured alternatives at the prefill
// pass (Q4_0 and Q8_0, 5120 -> 17408 and back, 75-77 us as built): the
// whole K segment staged first and 4 tile columns in flight, the same;
// 4-wave workgroups, 84 us; reducer workgroups at the end of the launch
// summing the segments (no unit waiting for a counter), 93 us: every
// workgroup of a launch holds the same LDS, so reducers waiting at the tail
// took the slots of units still to run.
constexpr int G16_W = 8;   // waves per workgroup
constexpr int G16_RT = 1;  // row tiles per wave
constexpr int G16_PF = 2;  // tile columns in flight per wave

struct G16Prob {
  const uint8_t *qs, *d;
  const float *X;
  float *Y;
  int64_t rows, cols, ldx, ldy;
  float *part;
  uint32_t *cnt;
  int NT, KT, S, G;
  int qt, acc;
};
// Ranges of consecutive units of one problem, in launch order (a problem
// holds at most two: one in each round of the launch).
constexpr int G16_RANGES = 2 * QG_BATCH_MAX;
struct G16Args {
  // range j covers launch units rstart[j] .. rstart[j + 1] - 1, which are
  // units rlu0[j] .. of problem rprob[j]; past the last range: INT64_MAX
  int64_t rstart[G16_RANGES];
  int64_t rlu0[G16_RANGES];
  int32_t rprob[G16_RANGES];
  G16Prob p[QG_BATCH_MAX];
  int n;
  int64_t units;
};

template <int W>
__global__ void __launch_bounds__(W * 64) gemm16_batch_kernel(G16Args b) {
  extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
  __shared__ uint32_t flag;
  // units in launch order, dealt round-robin to the XCDs (workgroup b runs
  // on XCD b % 8): every XCD gets the same mix of problems, so the XCDs
  // finish together (a contiguous range per XCD gave some XCDs twice the
  // bytes of others)
  const int64_t u = blockIdx.x;
  if (u >= b.units) return;
  // the range holding unit u from the first-unit numbers (one scalar
  // load), then its problem's one descriptor, read in place through a
  // uniform index (a select over every descriptor made a chain of dependent
  // scalar loads ahead of the first weight load)
  int ri = 0;
#pragma unroll
  for (int j = 1; j < G16_RANGES; ++j) ri += u >= b.rstart[j] ? 1 : 0;
  ri = __builtin_amdgcn_readfirstlane(ri);
  const int pi = __builtin_amdgcn_readfirstlane(b.rprob[ri]);
  const G16Prob &P = b.p[pi];
  DotArgs a = {};
  a.qs0 = a.qs1 = P.qs;
  a.d0 = a.d1 = P.d;
  a.rows = P.rows;
  a.cols = P.cols;
  a.NT = P.NT;
  a.KT = P.KT;
  a.S = P.S;
  a.SW = 1;
  a.IL = 0;
  a.G = P.G;
  a.X = P.X;
  a.ldx = P.ldx;
  a.ncols = 16;
  a.Y = P.Y;
  a.ldy = P.ldy;
  a.part = P.part;
  a.cnt = P.cnt;
  const int64_t lu = u - b.rstart[ri] + b.rlu0[ri];
  const int g = (int)(lu / P.S), s = (int)(lu % P.S);
  float bv = 0.0f;
  int32_t bi = 0;
  if (P.qt == Q4) {
    if (P.acc) dot_unit<Q4, 16, 1, EPI_ACC, G16_RT, G16_PF, W, PH_PLAIN>(a, g, s, smem, &flag, bv, bi);
    else dot_unit<Q4, 16, 1, EPI_STORE, G16_RT, G16_PF, W, PH_PLAIN>(a, g, s, smem, &flag, bv, bi);
  } else {
    if (P.acc) dot_unit<Q8, 16, 1, EPI_ACC, G16_RT, G16_PF, W, PH_PLAIN>(a, g, s, smem, &flag, bv, bi);
    else dot_unit<Q8, 16, 1, EPI_STORE, G16_RT, G16_PF, W, PH_PLAIN>(a, g, s, smem, &flag, bv, bi);
  }
}

// ---------------------------------------------------------------- host side
int device_cus() {
  static int cus[64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
  if (cus[dev] == 0) {
    int n = 0;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n < 1) n = 256;
    cus[dev] = n;
  }
  return cus[dev];
}

constexpr int DOT_STREAMS = 2048;     // (row tile, segment, matrix) weight streams
constexpr size_t DOT_X_LDS = 131072;  // staged activations of a contiguous segment, 8 columns
constexpr size_t LDS_HARD = 163840;   // gfx950 LDS per workgroup
constexpr size_t DOT_SW_LDS = 131072;  // in-workgroup segments: activations + sums
constexpr int64_t DOT_IL_TILES = 40;   // interleaved segments up to K = 5120

// Interleaved K segments (segment q of n: tile columns q, q + n, ...) up to
// K = 5120 (both model widths of the pages); a function of the shape only,
// so every column count of a shape sums in the same order.  Measured
// (K = 5120 and 2048): the waves of a workgroup then stream neighbouring
// tiles and finish together (gate/up 21.7 -> 20.3 us, verify Q4_0 4
// columns 15.5 -> 15.1 us).
bool dot_interleaved(int64_t cols) { return cdiv(cols / 32, 4) <= DOT_IL_TILES; }

// K segments of the dot path: about DOT_STREAMS weight streams of one row
// tile and one segment each (measured on the decode shapes: more streams,
// or more bytes in flight per stream, only lengthen the queues and the
// tail), at least 4 tile columns per segment, and few enough tile columns
// per segment that `ncols_max` columns of staged activations fit in DOT_X_LDS.
int gemv_segments(int64_t rows, int64_t cols, int nmat, int ncols_max) {
  const int64_t NT = cdiv(rows, 16), KT = cdiv(cols / 32, 4);
  int64_t s;
  if (dot_interleaved(cols)) {
    // interleaved segments run inside one workgroup of R row tiles x S
    // segments, one per CU of a 256-CU part (a constant: the order must not
    // depend on the device): the most segments that keep it within 15
    // waves (measured: 12 to 15 waves per CU beat 10 and 16 on the verify
    // and gate/up shapes)
    const int64_t R = cdiv(NT, 256);
    s = 15 / R;
  } else {
    // about DOT_STREAMS weight streams per matrix, rounded down (the fused
    // FFN needs its gate/up units in one round of resident workgroups),
    // except that 1.5 or more becomes 2
    const int64_t want = (int64_t)DOT_STREAMS * nmat;
    s = want / NT;
    if (s < 2 && 2 * want >= 3 * NT) s = 2;
  }
  if (s > KT / 4) s = KT / 4;
  const int64_t lds_min = cdiv((int64_t)dot_stage_bytes(KT, ncols_max), (int64_t)DOT_X_LDS);
  if (s < lds_min) s = lds_min;
  if (s < 1) s = 1;
  if (s > KT) s = KT;
  return (int)s;
}

// K segments of the 16-column GEMM (its activations stream through LDS in
// chunks, so the segment length is free): about GEMM16_STREAMS (row tile,
// segment) weight streams, at least 4 tile columns per segment, and few
// enough that workgroups of at most 16 waves fit one per CU of a 256-CU
// part (a constant, so the reduction order stays a function of the shape).
constexpr int GEMM16_STREAMS = 3000;
int gemm16_splits(int64_t rows, int64_t cols) {
  const int64_t NT = cdiv(rows, 16), KT = cdiv(cols / 32, 4);
  int64_t s = (GEMM16_STREAMS + NT / 2) / NT;  // nearest
  if (s > 256 / cdiv(NT, 16)) s = 256 / cdiv(NT, 16);
  if (s > KT / 4) s = KT / 4;
  if (s < 1) s = 1;
  return (int)s;
}

size_t qmv_ws_bytes(int64_t rows, int64_t cols, int slots, int nmat, int ncols_max, bool argmax, int topk) {
  const int64_t NT = cdiv(rows, 16);
  (void)cols;
  size_t b = QG_WS_SYNC_BYTES;                      // counters
  if (argmax) b += 2 * align256((size_t)NT * 4);    // candidates
  if (topk > 0) b += align256((size_t)NT * topk * 8);  // top-k candidates (row groups <= row tiles)
  if (slots > 1) b += (size_t)slots * nmat * NT * dot_part_floats(ncols_max) * 4;
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

// S segments across workgroups; SW > 1: segments inside each workgroup
// instead (S must then be 1), W = R * SW waves for R row tiles.
template <int QT, int NC, int NMAT, int EPI, int RT, int PF, int WKT, int WMAX = WKT, bool RMSN = false>
static int launch_dot_t(const QmvCall &c, int S, int W = WKT, int SW = 1) {
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
  a.SW = SW;
  a.IL = NC < 16 && dot_interleaved(c.cols) ? 1 : 0;
  if (W < 1 || W > WMAX || (WKT > 0 && W != WKT)) return QG_EUNSUPPORTED;
  if (NC >= 16 && WKT == 0 && W < DOT_XS_WMIN) return QG_EUNSUPPORTED;
  if (SW < 1 || (SW > 1 && (S != 1 || NC >= 16 || W % SW != 0))) return QG_EUNSUPPORTED;
  a.G = (int)cdiv(NTu, (int64_t)(W / SW) * RT);
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
  a.cand_k = nullptr;
  a.topk = c.topk;
  if (EPI == EPI_TOPK) {
    if (c.topk < 1 || c.topk > QG_TOPK_MAX) return QG_ESHAPE;
    a.cand_k = (uint64_t *)(ws + off);
    off += align256((size_t)NT * c.topk * 8);
  }
  if (EPI == EPI_ARGMAX) {
    a.cand_v = (float *)(ws + off);
    off += align256((size_t)NT * 4);
    a.cand_i = (int32_t *)(ws + off);
    off += align256((size_t)NT * 4);
  }
  a.part = (float *)(ws + off);
  a.out_idx = c.out_idx;
  a.out_val = c.out_val;
  a.gamma = RMSN ? c.gamma : nullptr;
  a.norm_eps = c.norm_eps;
  // the RMSNorm prologue needs every unit to stage all of K
  if (RMSN && !(a.IL || S == 1)) return QG_EUNSUPPORTED;
  a.xmap = a.ymap = nullptr;
  a.xspan = 0;
  if (!ranges_fit(c, NT, KT, QTraits<QT>::tile_bytes)) return QG_EUNSUPPORTED;
  const size_t pbytes = S > 1 ? (size_t)S * NMAT * NTu * dot_part_floats(NC) * 4 : 0;
  if (pbytes >= ((size_t)1 << 31)) return QG_EUNSUPPORTED;  // one bounded range
  const size_t need = off + pbytes;
  if (need > c.ws_bytes) return QG_EWORKSPACE;

  // staged activations: the unit's tile columns (all of K with in-workgroup
  // segments; at most ceil(KT / S) otherwise), or (16 columns) two chunks
  // of PF tile columns; then the in-workgroup segment sums
  size_t lds = NC >= 16 ? dot_stage_bytes(2 * X16_CHUNK, NC) : dot_stage_bytes(SW > 1 ? KT : cdiv(KT, S), NC);
  lds += (size_t)(SW - 1) * (W / SW) * NMAT * RT * (NC < 4 ? NC : 4) * 64 * 4;
  if (RMSN) lds += (size_t)NC * KT * TILE_BLOCKS * 4 * 4 + (size_t)NC * 4;  // squares per piece, 1/rms
  if (lds > LDS_HARD - 1024) return QG_EUNSUPPORTED;
  auto kern = dot_kernel<QT, NC, NMAT, EPI, RT, PF, WKT, WMAX, RMSN>;
  static size_t granted = 65536;  // per instantiation; only ever raised
  int st = grant_lds((const void *)kern, lds, granted);
  if (st) return st;
  clear_hip_error();
  hipLaunchKernelGGL(kern, dim3((unsigned)(a.per_xcd * 8)), dim3(W * 64), lds, c.stream, a);
  return launch_status();
}

// Workgroup size, one row tile per wave.  A CU that holds two of the
// launch's workgroups streams twice the bytes and finishes last (measured:
// a launch of a few more workgroups than CUs takes about 1.4x as long), so
// when the workgroups can be made few enough to take one CU each, they are:
// 4 waves where that already holds (small matrices: more CUs busy), else the
// smallest size from 8 to 16 waves that does.  Launches that take several
// rounds anyway use 8 waves.
static int dot_waves(int64_t NTu, int S) {
  const int64_t ncu = device_cus();
  if (cdiv(NTu, 4) * S <= ncu) return 4;
  for (int w = 8; w <= 16; ++w)
    if (cdiv(NTu, w) * S <= ncu) return w;
  return 8;
}

// One row tile per wave, about 4 KiB of weights in flight per wave (PF tile
// columns).
template <int QT, int NC, int NMAT, int EPI, bool RMSN = false>
static int launch_dot(const QmvCall &c, int S) {
  constexpr int QW = QT == Q4 ? 1 : 2;
  // the LM head (a gigabyte-scale stream) keeps about 12 KiB of weights in
  // flight per wave (at most 8 tile columns): a streaming read at this size
  // gains from deeper queues (Q8_0 248,320 x 5120: 219.5 us with 4 tile
  // columns, 215.5 with 6, 228.5 with 8, where the registers leave 3 waves
  // per SIMD)
  constexpr bool HEAD = EPI == EPI_ARGMAX || EPI == EPI_TOPK;
  constexpr int PF0 = HEAD ? (12 / (NMAT * QW) < 8 ? 12 / (NMAT * QW) : 8) : 4 / (NMAT * QW);
  constexpr int PF = PF0 < 2 ? 2 : PF0;
  const int64_t NTu = cdiv(c.n_rows, 16);
  const int W = dot_waves(NTu, S);
  const int plan = c.plan & ~(PLAN_FORCED | PLAN_S_MASK);
  bool sw_ok = false, sw = false;
  int64_t R = 1;
  if (S > 1) {
    // The segments as waves of one workgroup, summed through LDS: no
    // partials in memory and no second round trip at the end (about 2-3 us
    // on the decode shapes), same segments and order, so the same bits as
    // across workgroups.  Possible when a workgroup of R row tiles x S
    // segments (at most 16 waves) leaves one workgroup per CU and the whole
    // K range of activations fits in LDS; chosen with interleaved segments
    // (measured faster on every such shape), or with contiguous ones when
    // it keeps at least 90% of the CUs the split across workgroups would
    // use or each CU's share of the weights is small (<= 192 KiB: the tail
    // is then a large part of the time); the decode down projection stays
    // across workgroups (its waves would finish far apart).
    const int64_t ncu = device_cus();
    R = cdiv(NTu, ncu);
    const int64_t KT = cdiv(c.cols / 32, 4);
    constexpr int NI = NC < 4 ? NC : 4;
    const size_t lds = dot_stage_bytes(KT, NC) + (size_t)(S - 1) * R * NMAT * NI * 64 * 4;
    const int64_t u_sw = cdiv(NTu, R), u_cross = cdiv(NTu, (int64_t)W) * S;
    const int64_t cu_bytes = (int64_t)NMAT * R * KT * (QTraits<QT>::tile_bytes + TILE_D_BYTES);
    sw_ok = R * S <= 16 && lds <= DOT_SW_LDS;
    sw = sw_ok && (dot_interleaved(c.cols) || 10 * u_sw >= 9 * u_cross || cu_bytes <= 196608);
  }
  // A plan from the plan table (or the tuner) replaces the choice above; it
  // changes no sum (same segments, same order).
  if (plan) {
    if (plan & ~(PLAN_W_MASK | QG_PLAN_SW)) return QG_EUNSUPPORTED;
    if (plan & QG_PLAN_SW) {
      if (!sw_ok || (plan & PLAN_W_MASK)) return QG_EUNSUPPORTED;
      sw = true;
    } else {
      const int Wp = plan & PLAN_W_MASK;
      if (Wp > 16) return QG_EUNSUPPORTED;
      if (Wp <= 8) return launch_dot_t<QT, NC, NMAT, EPI, 1, PF, 0, 8, RMSN>(c, S, Wp);
      return launch_dot_t<QT, NC, NMAT, EPI, 1, PF, 0, 16, RMSN>(c, S, Wp);
    }
  }
  if (sw) return launch_dot_t<QT, NC, NMAT, EPI, 1, PF, 0, 16, RMSN>(c, 1, (int)(R * S), S);
  if (W <= 8) return launch_dot_t<QT, NC, NMAT, EPI, 1, PF, 0, 8, RMSN>(c, S, W);
  return launch_dot_t<QT, NC, NMAT, EPI, 1, PF, 0, 16, RMSN>(c, S, W);
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

template <int QT, bool RMSN>
static int dispatch_silu_t(const QmvCall &c, int S) {
  switch (c.ncols) {
    case 1: return launch_dot<QT, 1, 2, EPI_SILU, RMSN>(c, S);
    case 2: return launch_dot<QT, 2, 2, EPI_SILU, RMSN>(c, S);
    case 3: return launch_dot<QT, 3, 2, EPI_SILU, RMSN>(c, S);
    case 4: return launch_dot<QT, 4, 2, EPI_SILU, RMSN>(c, S);
    case 5: return launch_dot<QT, 5, 2, EPI_SILU, RMSN>(c, S);
    case 6: return launch_dot<QT, 6, 2, EPI_SILU, RMSN>(c, S);
    case 7: return launch_dot<QT, 7, 2, EPI_SILU, RMSN>(c, S);
    case 8: return launch_dot<QT, 8, 2, EPI_SILU, RMSN>(c, S);
  }
  return QG_ESHAPE;
}

template <int QT>
static int dispatch_silu(const QmvCall &c, int S) {
  return c.gamma ? dispatch_silu_t<QT, true>(c, S) : dispatch_silu_t<QT, false>(c, S);
}

// 16 columns: the shared dot unit on the matrix cores (one row tile per
// wave, PF = 2 tile columns in flight; measured best on the prefill shapes,
// as was the workgroup size below: a smaller workgroup waits less at the
// per-chunk barrier, so the smallest size that keeps one per CU).
template <int QT, int EPI>
static int launch_gemm16(const QmvCall &c) {
  const int Sp = (c.plan & PLAN_S_MASK) >> PLAN_S_SHIFT;
  const int S = Sp ? Sp : gemm16_splits(c.rows, c.cols);
  // at least 8 waves (the activation chunks are sized for them), else as
  // for the GEMV: one workgroup per CU when 8 to 16 waves allow it
  const int64_t NTu = cdiv(c.n_rows, 16), ncu = device_cus();
  int W = 8;
  for (int w = 8; w <= 16; ++w)
    if (cdiv(NTu, w) * S <= ncu) {
      W = w;
      break;
    }
  const int plan = c.plan & ~(PLAN_FORCED | PLAN_S_MASK);
  if (plan) {
    if (plan < 8 || plan > 16) return QG_EUNSUPPORTED;  // 8 to 16 waves, no in-workgroup segments
    W = plan;
  }
  if (W == 8) return launch_dot_t<QT, 16, 1, EPI, 1, 2, 8>(c, S);
  return launch_dot_t<QT, 16, 1, EPI, 1, 2, 0, 16>(c, S, W);
}

template <int QT>
static int dispatch_qt(const QmvCall &c) {
  // a plan's K segments replace the shape's own (a different summation
  // order: the sums change by rounding only)
  const int Sp = (c.plan & PLAN_S_MASK) >> PLAN_S_SHIFT;
  if (Sp > cdiv(c.cols / 32, 4)) return QG_EUNSUPPORTED;
  auto seg = [Sp](int S) { return Sp ? Sp : S; };
  if (c.ncols == 16) {
    if (c.epi == EPI_STORE) return launch_gemm16<QT, EPI_STORE>(c);
    if (c.epi == EPI_ACC) return launch_gemm16<QT, EPI_ACC>(c);
    return QG_EUNSUPPORTED;
  }
  switch (c.epi) {
    case EPI_STORE: return dispatch_dot<QT, EPI_STORE>(c, seg(gemv_segments(c.rows, c.cols, 1, 8)));
    case EPI_ACC: return dispatch_dot<QT, EPI_ACC>(c, seg(gemv_segments(c.rows, c.cols, 1, 8)));
    case EPI_SILU: return dispatch_silu<QT>(c, seg(gemv_segments(c.rows, c.cols, 2, 8)));
    case EPI_ARGMAX:
      if (c.ncols != 1) return QG_ESHAPE;
      return launch_dot<QT, 1, 1, EPI_ARGMAX>(c, seg(gemv_segments(c.rows, c.cols, 1, 1)));
    case EPI_TOPK:
      if (c.ncols != 1) return QG_ESHAPE;
      return launch_dot<QT, 1, 1, EPI_TOPK>(c, seg(gemv_segments(c.rows, c.cols, 1, 1)));
  }
  return QG_EINVAL;
}

// K segments of each problem of a grouped launch.  Each problem's K is cut
// into segments about as long as the shortest K of the launch (at least
// one), so that the units of all problems stream about equally many tile
// columns and only the longer problems pay a hand-off; these counts are
// then multiplied by the smallest factor that gives at least two units per
// CU (a launch whose units are all resident at once).  Segments stay at
// least 4 tile columns long and at most 255.  Measured at the prefill pass
// (5120 -> 17408 and back, Q4_0 and Q8_0, largest units first): the counts
// this gives (1 and 3) took 56.9 us against 60.1-62.0 us for (2, 6), (1,
// 4) and the single-problem splits (3, 9).
void gemm16_batch_splits(const qg_gemm16_problem *p, int n, int *S) {
  int64_t ktmin = INT64_MAX;
  for (int i = 0; i < n; ++i) ktmin = std::min<int64_t>(ktmin, cdiv(p[i].cols / 32, 4));
  int64_t base[QG_BATCH_MAX], cap[QG_BATCH_MAX], G[QG_BATCH_MAX];
  for (int i = 0; i < n; ++i) {
    const int64_t KT = cdiv(p[i].cols / 32, 4);
    base[i] = std::max<int64_t>(1, (KT + ktmin / 2) / ktmin);
    cap[i] = std::min<int64_t>(255, std::max<int64_t>(1, KT / 4));
    G[i] = cdiv(cdiv(p[i].rows, 16), G16_W * G16_RT);
  }
  const int64_t want = 2 * (int64_t)device_cus();
  for (int64_t m = 1;; ++m) {
    int64_t units = 0;
    bool grows = false;
    for (int i = 0; i < n; ++i) {
      S[i] = (int)std::min(base[i] * m, cap[i]);
      units += G[i] * S[i];
      grows |= base[i] * m < cap[i];
    }
    if (units >= want || !grows) break;
  }
}

// Workspace of a grouped launch: the counters of every problem's row groups
// in the shared counter words, then each problem's segment partials.  Fills
// `b` when given (the pointers inside `ws`, the launch order of the units).
//
// Launch order.  The hardware hands out workgroups in launch order, so the
// problems take their units in order of decreasing weight bytes per unit
// (ties: the caller's order): long units start first, short ones fill in at
// the end (measured at the prefill pass with the single-problem splits:
// 71.6 us with the caller's order Q4_0 before Q8_0, 66.1 us largest units
// first).  When the units make more than one and at most two rounds of one
// unit per CU, the first round takes the largest units and the second the
// rest in increasing size: the units CU c receives, c and c + CUs, then pair
// a long unit with a short one (measured at the prefill pass, 512 units on
// 256 CUs: 55.4-58.0 us largest first throughout, 53.2-54.0 us paired).
// The order changes no sum.
static size_t gemm16_batch_layout(const qg_gemm16_problem *p, int n, G16Args *b, uint8_t *ws) {
  size_t off = QG_WS_SYNC_BYTES, words = 0;
  int ord[QG_BATCH_MAX], Sp[QG_BATCH_MAX];
  int64_t ubytes[QG_BATCH_MAX], nunits[QG_BATCH_MAX];
  gemm16_batch_splits(p, n, Sp);
  int64_t U = 0;
  for (int i = 0; i < n; ++i) {
    const int64_t NT = cdiv(p[i].rows, 16), KT = cdiv(p[i].cols / 32, 4);
    const int S = Sp[i];
    const int64_t G = cdiv(NT, G16_W * G16_RT);
    const int64_t tb = p[i].qtype == QG_Q4_0 ? QTraits<Q4>::tile_bytes : QTraits<Q8>::tile_bytes;
    ubytes[i] = (int64_t)G16_W * G16_RT * cdiv(KT, S) * tb;
    nunits[i] = G * S;
    U += G * S;
    ord[i] = i;
    if (b) {
      G16Prob &q = b->p[i];
      q.qs = (const uint8_t *)p[i].qs;
      q.d = (const uint8_t *)p[i].d;
      q.X = p[i].X;
      q.Y = p[i].Y;
      q.rows = p[i].rows;
      q.cols = p[i].cols;
      q.ldx = p[i].ldx;
      q.ldy = p[i].ldy;
      q.part = (float *)(ws + off);
      q.cnt = (uint32_t *)ws + words;
      q.NT = (int)NT;
      q.KT = (int)KT;
      q.S = S;
      q.G = (int)G;
      q.qt = p[i].qtype == QG_Q4_0 ? Q4 : Q8;
      q.acc = p[i].accumulate ? 1 : 0;
    }
    words += (size_t)G;
    if (S > 1) off += align256((size_t)S * NT * dot_part_floats(16) * 4);
  }
  for (int i = 1; i < n; ++i)  // stable insertion sort, decreasing unit bytes
    for (int j = i; j > 0 && ubytes[ord[j]] > ubytes[ord[j - 1]]; --j) {
      const int t = ord[j];
      ord[j] = ord[j - 1];
      ord[j - 1] = t;
    }
  if (b) {
    int nr = 0;
    int64_t next = 0;
    auto add = [&](int prob, int64_t lu0, int64_t cnt) {
      if (cnt <= 0) return;
      b->rstart[nr] = next;
      b->rlu0[nr] = lu0;
      b->rprob[nr] = prob;
      ++nr;
      next += cnt;
    };
    const int64_t R = device_cus();
    if (U > R && U <= 2 * R) {
      int64_t first[QG_BATCH_MAX], left = R;
      for (int k = 0; k < n; ++k) {
        const int i = ord[k];
        first[i] = nunits[i] < left ? nunits[i] : left;
        left -= first[i];
        add(i, 0, first[i]);
      }
      for (int k = n - 1; k >= 0; --k) add(ord[k], first[ord[k]], nunits[ord[k]] - first[ord[k]]);
    } else {
      for (int k = 0; k < n; ++k) add(ord[k], 0, nunits[ord[k]]);
    }
    for (int j = nr; j < G16_RANGES; ++j) {
      b->rstart[j] = INT64_MAX;
      b->rlu0[j] = 0;
      b->rprob[j] = 0;
    }
    b->n = n;
    b->units = U;
  }
  return words > WS_SYNC_WORDS ? 0 : off;
}

size_t gemm16_batch_ws_bytes(const qg_gemm16_problem *p, int n) { return gemm16_batch_layout(p, n, nullptr, nullptr); }

int launch_gemm16_batch(const qg_gemm16_problem *p, int n, void *ws, size_t ws_bytes, hipStream_t stream) {
  G16Args b;
  memset(&b, 0, sizeof(b));
  const size_t need = gemm16_batch_layout(p, n, &b, (uint8_t *)ws);
  if (need == 0) return QG_EUNSUPPORTED;
  if (need > ws_bytes) return QG_EWORKSPACE;
  for (int i = 0; i < n; ++i) {
    const G16Prob &q = b.p[i];
    const int64_t xb = (15 * q.ldx + q.cols) * 4, tb = q.qt == Q4 ? 1024 : 2048;
    if (xb >= ((int64_t)1 << 31) || (int64_t)q.KT * tb >= ((int64_t)1 << 31)) return QG_EUNSUPPORTED;
    if ((size_t)q.S * q.NT * dot_part_floats(16) * 4 >= ((size_t)1 << 31)) return QG_EUNSUPPORTED;
  }
  const size_t lds = dot_stage_bytes(2 * X16_CHUNK, 16);  // two chunks
  clear_hip_error();
  hipLaunchKernelGGL(gemm16_batch_kernel<G16_W>, dim3((unsigned)b.units), dim3(G16_W * 64), lds, stream, b);
  return launch_status();
}

int builtin_split(const QmvCall &c) {
  if (c.ncols == 16) return gemm16_splits(c.rows, c.cols);
  if (c.epi == EPI_SILU) return gemv_segments(c.rows, c.cols, 2, 8);
  if (c.epi == EPI_ARGMAX || c.epi == EPI_TOPK) return gemv_segments(c.rows, c.cols, 1, 1);
  return gemv_segments(c.rows, c.cols, 1, 8);
}

static int dispatch_qmv(const QmvCall &c) {
  if (c.qtype == QG_Q4_0) return dispatch_qt<Q4>(c);
  if (c.qtype == QG_Q8_0) return dispatch_qt<Q8>(c);
  return QG_EINVAL;
}

// The plan table's entry for this call, unless the caller fixed the plan;
// an entry the call cannot use (refused before anything is launched) gives
// way to the built-in choice, unless it is marked strict (a split needing
// more workspace than the call brings counts as unusable).
int launch_qmv(const QmvCall &c0) {
  QmvCall c = c0;
  const bool forced = (c.plan & PLAN_FORCED) != 0;
  if (!forced) c.plan = plan_lookup(c);
  const bool strict = (c.plan & QG_PLAN_STRICT) != 0;
  c.plan &= ~QG_PLAN_STRICT;
  int st = dispatch_qmv(c);
  if ((st == QG_EUNSUPPORTED || st == QG_EWORKSPACE) && !forced && !strict && c.plan) {
    c.plan = 0;
    st = dispatch_qmv(c);
  }
  return st;
}

}  // namespace qg
