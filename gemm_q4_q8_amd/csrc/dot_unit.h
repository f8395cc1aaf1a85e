// One work unit of the product kernels: W row tiles (one per wave, of one
// matrix or of gate and up together) over one K segment, used by the GEMV
// (1..8 columns), gate/up, LM head and 16-column GEMM kernels and the MoE
// expert kernels.
//
// What is computed ("Engine and kernels", Kernel families): y = W x over
// Q4_0 / Q8_0 blocks dequantised in registers with f32 sums, with the
// epilogues of the kernel families (store, y += W x, SiLU(gate) * up, and
// the per-row values an argmax needs).  Activations are f32 ("Correctness
// and portability": f16 only for block scales, the KV cache and the wire),
// so products of 1..8 columns carry each activation at f32 range and
// 22-bit precision into the matrix cores (below); only the 16-column
// prefill tiles take plain f16 activation operands.
//
// How (MI355X):
//  * The workgroup stages its activations once in LDS.  1..8 columns: each
//    value x of (tile column t, column c) as x = 2^e_tc (hi + lo), hi =
//    f16(x 2^-e_tc), lo = f16(x 2^-e_tc - hi), the power of two chosen per
//    128 values of a column so that their largest |x| lands in [2^14,
//    2^15): hi + lo holds x to 22 significant bits at any f32 magnitude.
//    16 columns: f16 in double-buffered chunks.
//  * One wave streams one row tile across its segment, PF tile columns
//    ahead; each 16-byte load of a wave reads a contiguous 1 KiB stripe.
//    The stream is a bounded buffer range, so loads past it return zeros
//    without touching memory and the loop has no branch around its loads.
//  * Weights become exact f16 values; per block, one matrix-core product
//    (activation rows x the block's 16 weight rows).  With 1..8 columns the
//    hi parts sit in product rows 0..NC-1 and the lo parts in rows LO..,
//    rows a narrow batch leaves idle, so the split costs no extra product;
//    each lane sums its results over the tile's four blocks, each times the
//    block's f16 scale, then adds that tile sum times 2^e_tc into its f32
//    accumulators; hi and lo sums meet once, after the stream.
//  * Segments: S of them, contiguous K ranges or interleaved tile columns
//    (segment q takes q, q + S, ...), chosen by the shape; summed in
//    segment order, either by the last workgroup of the row group (from
//    partials in memory) or, with the segments as waves of one workgroup,
//    through LDS.  The order depends on the shape only, so each activation
//    column of a batched call is bitwise equal to a 1-column call
//    ("Architecture", Speculative decoding).
#pragma once
#include "common.h"
#include "internal.h"

namespace qg {

// Segment q of a K range of kt tile columns cut into n pieces.
__host__ __device__ inline int seg_begin(int q, int kt, int n) { return (int)((int64_t)kt * q / n); }

// PH_PRODUCE: outputs are written with coherent (agent-scope) stores, for a
// consumer in another workgroup of the same launch.
enum Phase { PH_PLAIN = 0, PH_PRODUCE = 1 };

struct DotArgs {
  const uint8_t *qs0, *qs1, *d0, *d1;
  int64_t rows;       // outputs produced (n_rows for the LM head)
  int64_t cols;
  int NT, KT;         // row tiles produced, tile columns of the matrix
  int S;              // K segments across workgroups
  int SW;             // K segments inside one workgroup (<= 1: none): wave wk
                      // streams segment wk / R of row tile wk % R, R = waves / SW
  int IL;             // interleaved segments: segment q of n holds tile columns
                      // q, q + n, q + 2n, ...; otherwise contiguous ranges
  int G;              // row groups of R * RT row tiles
  int64_t units;      // G * S workgroups
  int64_t per_xcd;
  const float *X;
  int64_t ldx;
  int ncols;
  float *Y;
  int64_t ldy;
  float *part;        // segment partials [S][NMAT][NT][NI][64 lanes]
  uint32_t *cnt;      // [G]
  uint32_t *gcnt;     // argmax: one counter
  float *cand_v;      // argmax: [G]
  int32_t *cand_i;
  uint64_t *cand_k;   // top-k: [G][topk] rank keys of each row group's best rows
  int topk;
  int32_t *out_idx;
  float *out_val;
  const float *gamma; // RMSNorm prologue: the weights (cols), and eps
  float norm_eps;
  const int32_t *xmap, *ymap;  // MoE: column c reads X column xmap[c], writes Y column ymap[c]
  int64_t xspan;      // bytes of X the columns may read (0: the ncols columns)
};

// Floats of one row tile's segment partial: NI values per lane, 64 lanes
// (NI: columns per lane, at most 4).
__host__ __device__ constexpr int dot_part_floats(int nc) { return (nc < 4 ? nc : 4) * 64; }

// Columns of the per-tile powers of two in LDS (a multiple of 4, so a lane
// reads its four columns as one 16-byte vector).
__host__ __device__ constexpr int dot_scale_cols(int nc) { return (nc + 3) & ~3; }

// LDS bytes of `ntiles` staged tile columns (4 blocks each) of `nc`
// activation columns: 16 columns, f16 values; 1..8 columns, the hi and lo
// halves of every value plus one f32 power of two per (tile, column).
__host__ __device__ constexpr size_t dot_stage_bytes(int64_t ntiles, int nc) {
  return nc >= 16 ? (size_t)ntiles * TILE_BLOCKS * nc * 64
                  : (size_t)ntiles * (TILE_BLOCKS * nc * 2 * 64 + dot_scale_cols(nc) * 4);
}

// Smallest workgroup (waves) a streamed-staging unit of launch-time size
// runs with: its per-thread chunk pieces are sized for it.
constexpr int DOT_XS_WMIN = 8;
// Tile columns of 16-column activations per LDS chunk (double-buffered).
constexpr int X16_CHUNK = 2;

// Register fence after a matrix-core product and the FMAs that read its
// result.  The matrix core reads A and B and writes all four result
// registers over several passes after the instruction issues; a register it
// still reads or writes must not be handed to another value meanwhile.  The
// statement takes A, B and the whole result and rewrites the accumulators
// the FMAs produced, so it is ordered after those FMAs (which wait for the
// product to complete) and all of A, B and D stay allocated until then, also
// the result values no FMA reads (fewer than four columns).
template <int NI>
__device__ __forceinline__ void mfma_fence(float (&acc)[NI], const h8 &A, const h8 &B, const f4 &D) {
  static_assert(NI >= 1 && NI <= 4, "columns per lane");
  if constexpr (NI == 1) __asm__ volatile("" : "+v"(acc[0]) : "v"(A), "v"(B), "v"(D));
  else if constexpr (NI == 2) __asm__ volatile("" : "+v"(acc[0]), "+v"(acc[1]) : "v"(A), "v"(B), "v"(D));
  else if constexpr (NI == 3)
    __asm__ volatile("" : "+v"(acc[0]), "+v"(acc[1]), "+v"(acc[2]) : "v"(A), "v"(B), "v"(D));
  else
    __asm__ volatile("" : "+v"(acc[0]), "+v"(acc[1]), "+v"(acc[2]), "+v"(acc[3]) : "v"(A), "v"(B), "v"(D));
}

// The same, one fence over the four block products of a tile.
#define QG_FENCE_IN "v"(A[0]), "v"(A[1]), "v"(A[2]), "v"(A[3]), "v"(B[0]), "v"(B[1]), "v"(B[2]), "v"(B[3]), \
                    "v"(D[0]), "v"(D[1]), "v"(D[2]), "v"(D[3])
template <int NI>
__device__ __forceinline__ void mfma_fence(float (&acc)[NI], const h8 (&A)[4], const h8 (&B)[4], const f4 (&D)[4]) {
  static_assert(NI >= 1 && NI <= 4, "columns per lane");
  if constexpr (NI == 1) __asm__ volatile("" : "+v"(acc[0]) : QG_FENCE_IN);
  else if constexpr (NI == 2) __asm__ volatile("" : "+v"(acc[0]), "+v"(acc[1]) : QG_FENCE_IN);
  else if constexpr (NI == 3) __asm__ volatile("" : "+v"(acc[0]), "+v"(acc[1]), "+v"(acc[2]) : QG_FENCE_IN);
  else __asm__ volatile("" : "+v"(acc[0]), "+v"(acc[1]), "+v"(acc[2]), "+v"(acc[3]) : QG_FENCE_IN);
}
#undef QG_FENCE_IN

// Half offset of 16-byte chunk q (0..3) of activation row g in LDS.  A row
// is 32 halves (64 bytes); its chunks are stored in the order q ^ ((g >> 1)
// & 3), so that the rows g .. g + 7 a group of 8 lanes reads at once (one
// chunk each) cover all 128 bytes of banks instead of two 16-byte columns
// of them (measured: 3.5 bank-conflict cycles per LDS instruction without).
__device__ __forceinline__ size_t xrow(size_t g, int q) { return g * 32 + (size_t)((q ^ ((int)(g >> 1) & 3)) * 8); }

// The largest of a value over the 16 lanes of a DPP row (all active): the
// quad permutes [1,0,3,2] and [2,3,0,1], then the half-row mirror and the
// row mirror (each step pairs lanes holding maxima of disjoint groups).
__device__ __forceinline__ float row16_max(float m) {
#pragma unroll
  for (int step = 0; step < 4; ++step)
    m = fmaxf(m, __builtin_bit_cast(float, dpp_partner(__builtin_bit_cast(int, m), step)));
  return m;
}

// The power of two of a tile column whose largest magnitude is m: `up` =
// 2^(14 - E) for m in [2^E, 2^(E+1)), so m * up lies in [2^14, 2^15) (below
// the f16 maximum 65504 after rounding), and `down` = 1 / up.  Magnitudes
// below 2^-112 (zero included) share the largest factor 2^126.
__device__ __forceinline__ void tile_pow2(float m, float &up, float &down) {
  const uint32_t be = (__builtin_bit_cast(uint32_t, m) >> 23) & 0xFFu;
  const uint32_t bc = be < 15u ? 15u : be;
  up = __builtin_bit_cast(float, (268u - bc) << 23);
  down = __builtin_bit_cast(float, (bc - 14u) << 23);
}

// x * up split into hi + lo, both f16 (round to nearest even): hi the
// rounded value, lo the rounded remainder (the remainder itself is exact in
// f32), so hi + lo agrees with x * up to 22 significant bits.
__device__ __forceinline__ void split_hl(const float (&x)[8], float up, h8 &H, h8 &L) {
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    const float t = x[e] * up;
    const _Float16 h = (_Float16)t;
    H[e] = h;
    L[e] = (_Float16)(t - (float)h);
  }
}

// The unit (row group g, segment s) of the launch `a`.  RMSN (gate/up): the
// activations are RMS-normalised first, as x * gamma staged, times
// 1 / sqrt(mean(x^2) + eps) per column applied to the two products (the
// same value, since the products are linear in x); every such unit reads
// all of K for the column's squares.  Returns true when this workgroup
// emitted the outputs of row group g (its only segment, or the last of its
// segments to finish).  For the argmax epilogue, (bv, bi) then hold each
// lane's best (value, row).
template <int QT, int NC, int NMAT, int EPI, int RT, int PF, int WKT, int PH, bool RMSN = false>
__device__ __forceinline__ bool dot_unit(const DotArgs &a, int g, int s, uint8_t *smem, uint32_t *flag,
                                          float &bv, int32_t &bi) {
  // WKT == 0: one row tile per wave of the workgroup as launched (at least
  // XWMIN waves when the activations stream in chunks)
  const int NTHR = WKT > 0 ? WKT * 64 : (int)blockDim.x;
  // Wide batches stream their activations in chunks of X16_CHUNK tile
  // columns, double-buffered in LDS and staged one chunk ahead of the
  // products (the
  // whole segment would take several L2 round trips before the first
  // product); narrow ones stage the whole segment up front, as hi / lo
  // pairs.
  constexpr bool F16 = NC >= 16;  // f16 operands (16 columns), else hi / lo pairs
  constexpr bool XS = F16;         // activations streamed in chunks
  static_assert(F16 ? NC == 16 : (NC >= 1 && NC <= 8), "column count");
  constexpr int XC = F16 ? NC : 2 * NC;  // activation rows of a block in LDS: hi, then lo
  constexpr int LO = NC <= 4 ? 4 : 8;   // matrix-core row of the lo part of column 0
  // accumulators per lane: the 4 D values of lane (r, sl) are product rows
  // 4 sl + i
  constexpr int NI = NC < 4 ? NC : 4;
  constexpr int TB = QTraits<QT>::tile_bytes;
  constexpr int QW = (QT == Q4) ? 1 : 2;  // 16-byte loads per lane per tile
  // tile columns per activation chunk (16 columns): the weight stream runs
  // PF tile columns ahead, a whole number of chunks
  constexpr int CT = XS ? X16_CHUNK : PF;
  static_assert(PF % CT == 0, "weight prefetch: whole chunks");
  constexpr int CHH = CT * TILE_BLOCKS * NC * 32;  // halves per chunk buffer
  constexpr int XWMIN = WKT > 0 ? WKT : DOT_XS_WMIN;

  const int tid = threadIdx.x, lane = tid & 63;
  const int wk = __builtin_amdgcn_readfirstlane(tid >> 6);
  // the workgroup's K range, and inside it this wave's stream: all of it,
  // or (SW > 1) in-workgroup segment wsg of SW.  Interleaved segments: the
  // wave's segment q of nq takes tile columns q, q + nq, ... (wst = nq);
  // contiguous ones: its range [wkt0, wkt0 + wnkt) of the unit's columns.
  const int SW = (!F16 && a.SW > 1) ? a.SW : 1;
  const int R = (NTHR >> 6) / SW;
  const int wrt = wk % R, wsg = wk / R;
  const bool IL = !F16 && a.IL;
  const int kt0 = IL ? 0 : seg_begin(s, a.KT, a.S);
  const int nkt = IL ? a.KT : seg_begin(s + 1, a.KT, a.S) - kt0;
  const int wq_i = SW > 1 ? wsg : s, wq_n = SW > 1 ? SW : a.S;  // this wave's segment of how many
  const int wkt0 = IL ? wq_i : seg_begin(wsg, nkt, SW);        // first tile column, relative to kt0
  const int wst = IL ? wq_n : 1;                               // step between its tile columns
  const int wnkt = IL ? (nkt - wq_i + wq_n - 1) / wq_n : seg_begin(wsg + 1, nkt, SW) - wkt0;
  const int64_t rt_base = ((int64_t)g * R + wrt) * RT;
  const int r = lane & 15, sl = lane >> 4;

  // Which activations the unit stages.  Interleaved segments across
  // workgroups: only the unit's own tile columns (wq_i, wq_i + wq_n, ...),
  // compacted; with the norm it still reads all of K (for the squares) and
  // keeps its own columns.  Otherwise the unit's K range [kt0, kt0 + nkt).
  const bool own = IL && SW == 1;
  const int nlt = (own && !RMSN) ? wnkt : nkt;  // tile columns read
  const int nst = own ? wnkt : nkt;             // tile columns staged
  auto ld_tile = [&](int lt) -> int { return (own && !RMSN) ? wq_i + lt * wq_n : kt0 + lt; };
  auto st_tile = [&](int lt) -> int {
    if (own && RMSN) return lt % wq_n == wq_i ? lt / wq_n : -1;
    return lt;
  };
  _Float16 *xs = (_Float16 *)smem;
  constexpr int SCC = dot_scale_cols(NC);
  float *scl = (float *)(smem + (size_t)nst * TILE_BLOCKS * XC * 64);  // [staged tile][SCC columns]

  // activations: a bounded range over the columns; a piece outside the
  // staged range or the matrix reads zeros
  const int nvec = nlt * TILE_BLOCKS * NC * 4;  // 8-value pieces read by the unit (whole staging)
  const __amdgpu_buffer_rsrc_t rx =
      buf_range(a.X, (uint32_t)(a.xspan ? a.xspan : ((int64_t)(a.ncols - 1) * a.ldx + a.cols) * 4));
  // the X column piece v reads (through the column map, if any); a piece's
  // column does not change from chunk to chunk, so streamed staging looks
  // it up once, not inside the weight stream (a map load there would make
  // every chunk wait for all weight loads in flight)
  // Pieces (8 values) are numbered (block, column, quarter) for 16 columns,
  // and (tile column, column, block, quarter) for 1..8 columns: the 16
  // pieces of one tile column of one column are then the 16 lanes of one
  // DPP row (the span is a multiple of 16).
  auto p_col = [&](int v) -> int { return F16 ? (v >> 2) % NC : (v >> 4) % NC; };
  auto x_col = [&](int v) -> int64_t {
    const int c = p_col(v);
    return c < a.ncols && a.xmap ? a.xmap[c] : c;
  };
  // piece v = (block, column, 8 k) of the `span` pieces from tile column
  // rel0 on (streamed chunks) or of the unit's read range (whole staging):
  // its k, or -1 when it lies outside the span, the segment or the matrix
  auto x_k = [&](int v, int rel0, int span) -> int64_t {
    const int qq = v & 3, c = p_col(v);
    const int bl = F16 ? (v >> 2) / NC : ((v >> 4) / NC) * TILE_BLOCKS + ((v >> 2) & 3);  // block read
    const int64_t gb = F16 ? (int64_t)(kt0 + rel0) * TILE_BLOCKS + bl
                           : (int64_t)ld_tile(bl >> 2) * TILE_BLOCKS + (bl & 3);
    const int64_t k = gb * 32 + qq * 8;
    const bool ok = v < span && (!XS || rel0 * TILE_BLOCKS + bl < nkt * TILE_BLOCKS) && k < a.cols && c < a.ncols;
    return ok ? k : -1;
  };
  // RMSNorm: gamma over the same 8 k of a piece (its range: cols floats;
  // a piece outside reads zeros), and per piece read the sum of its 8
  // squares, [column][piece along K], past the staged activations and the
  // in-workgroup sums; then 1 / rms per column
  static_assert(!RMSN || (!F16 && EPI == EPI_SILU), "RMSNorm prologue: gate/up, 1..8 columns");
  const __amdgpu_buffer_rsrc_t rg = buf_range(a.gamma, RMSN ? (uint32_t)(a.cols * 4) : 0u);
  const int npc = nlt * TILE_BLOCKS * 4;  // pieces of one column
  float *ssq = (float *)(smem + dot_stage_bytes(nst, NC) +
                         (SW > 1 ? (size_t)(SW - 1) * R * NMAT * RT * NI * 64 * 4 : 0));
  float *inv_rms = ssq + (size_t)NC * npc;
  struct XPiece {
    u4 lo, hi, glo, ghi;
  };
  auto x_ld = [&](int v, int rel0, int span, int64_t xc, XPiece &pc) {
    const int64_t k = x_k(v, rel0, span);
    const uint32_t o = k >= 0 ? (uint32_t)((xc * a.ldx + k) * 4) : 0xFFFFFFC0u;
    pc.lo = __builtin_amdgcn_raw_buffer_load_b128(rx, o, 0, 0);
    pc.hi = __builtin_amdgcn_raw_buffer_load_b128(rx, o + 16u, 0, 0);
    if constexpr (RMSN) {
      const uint32_t og = k >= 0 ? (uint32_t)(k * 4) : 0xFFFFFFC0u;
      pc.glo = __builtin_amdgcn_raw_buffer_load_b128(rg, og, 0, 0);
      pc.ghi = __builtin_amdgcn_raw_buffer_load_b128(rg, og + 16u, 0, 0);
    }
  };
  // Every lane of a DPP row runs x_put together, so the row maximum below
  // sees the whole tile column of its column.
  auto x_put = [&](int v, int span, _Float16 *dst, const XPiece &pc) {
    const int qq = v & 3, c = p_col(v);
    const int bl = F16 ? (v >> 2) / NC : ((v >> 4) / NC) * TILE_BLOCKS + ((v >> 2) & 3);
    float x[8];
    {
      const float4 lo = __builtin_bit_cast(float4, pc.lo), hi = __builtin_bit_cast(float4, pc.hi);
      x[0] = lo[0]; x[1] = lo[1]; x[2] = lo[2]; x[3] = lo[3];
      x[4] = hi[0]; x[5] = hi[1]; x[6] = hi[2]; x[7] = hi[3];
    }
    if constexpr (RMSN) {
      // the piece's squares in k order, then x * gamma
      float q = x[0] * x[0];
#pragma unroll
      for (int e = 1; e < 8; ++e) q = __builtin_fmaf(x[e], x[e], q);
      if (v < span) ssq[(size_t)c * npc + bl * 4 + qq] = q;
      const float4 glo = __builtin_bit_cast(float4, pc.glo), ghi = __builtin_bit_cast(float4, pc.ghi);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        x[e] *= glo[e];
        x[4 + e] *= ghi[e];
      }
    }
    if constexpr (F16) {
      if (v < span) {
        h8 hv;
#pragma unroll
        for (int e = 0; e < 8; ++e) hv[e] = (_Float16)x[e];
        *(h8 *)(dst + xrow((size_t)bl * XC + c, qq)) = hv;
      }
    } else {
      float m = 0.0f;
#pragma unroll
      for (int e = 0; e < 8; ++e) m = fmaxf(m, __builtin_fabsf(x[e]));
      m = row16_max(m);
      float up, down;
      tile_pow2(m, up, down);
      h8 H, L;
      split_hl(x, up, H, L);
      const int st = st_tile(bl >> 2);
      if (v < span && st >= 0) {
        const int sb = st * TILE_BLOCKS + (bl & 3);
        *(h8 *)(xs + xrow((size_t)sb * XC + c, qq)) = H;
        *(h8 *)(xs + xrow((size_t)sb * XC + NC + c, qq)) = L;
        if ((v & 15) == 0) scl[(size_t)st * SCC + c] = down;
      }
    }
  };

  // 16 columns: wave w stages columns w, w + waves, ... of each chunk, lane
  // l the 4 values at k 4 l .. 4 l + 3 of the chunk's 256, so that each load
  // instruction reads one column's contiguous KiB (two 16-byte loads of 8
  // consecutive values per lane touched every cache line twice).
  static_assert(!XS || (CT * 128 == 256 && !RMSN), "16-column chunks: 256 values per column");
  constexpr int XCW = XS ? (NC + XWMIN - 1) / XWMIN : 1;  // columns per wave at most
  auto f16_ld = [&](int j, int rel0, u4 &pc) {
    const int c = wk + j * (NTHR >> 6);
    const int kr = 4 * lane, t = kr >> 7;
    const int64_t k = (int64_t)(kt0 + rel0 + t) * 128 + (kr & 127);
    const bool ok = c < NC && c < a.ncols && rel0 + t < nkt && k < a.cols;
    const uint32_t o = ok ? (uint32_t)(((int64_t)c * a.ldx + k) * 4) : 0xFFFFFFC0u;
    pc = __builtin_amdgcn_raw_buffer_load_b128(rx, o, 0, 0);
  };
  auto f16_put = [&](int j, _Float16 *dst, const u4 &pc) {
    const int c = wk + j * (NTHR >> 6);
    if (c >= NC) return;
    const int kr = 4 * lane;
    const int blk = kr >> 5, qq = (kr >> 3) & 3, h = (kr >> 2) & 1;  // block of the chunk, 16-byte piece, half
    const float4 f = __builtin_bit_cast(float4, pc);
    const h4 hv = {(_Float16)f[0], (_Float16)f[1], (_Float16)f[2], (_Float16)f[3]};
    *(h4 *)(dst + xrow((size_t)blk * XC + c, qq) + 4 * h) = hv;
  };

  // one bounded range per (matrix, row tile) over this segment; row tiles
  // past the matrix get an empty range
  __amdgpu_buffer_rsrc_t rq[NMAT][RT], rd[NMAT][RT];
#pragma unroll
  for (int m = 0; m < NMAT; ++m)
#pragma unroll
    for (int t = 0; t < RT; ++t) {
      const bool in = rt_base + t < a.NT;
      // the range starts at the wave's first tile column and spans its
      // last one (interleaved: the tiles between belong to other waves)
      const int64_t tile = (in ? rt_base + t : 0) * a.KT + kt0 + wkt0;
      const uint32_t span = wnkt > 0 ? (uint32_t)((wnkt - 1) * wst + 1) : 0u;
      rq[m][t] = buf_range((m ? a.qs1 : a.qs0) + tile * TB, in ? span * TB : 0u);
      rd[m][t] = buf_range((m ? a.d1 : a.d0) + tile * TILE_D_BYTES, in ? span * TILE_D_BYTES : 0u);
    }
  u4 wq[PF][NMAT][RT][QW];
  u2 wd[PF][NMAT][RT];
  const uint32_t lane_off = (uint32_t)lane * 16u, d_off = (uint32_t)r * 8u;
  auto load = [&](int slot, int rel_) {  // rel_: the wave's rel_-th tile column
    // past the wave's last tile column: an offset beyond every range
    const int rel = rel_ < wnkt ? rel_ * wst : 0x7FFF;
#pragma unroll
    for (int m = 0; m < NMAT; ++m)
#pragma unroll
      for (int t = 0; t < RT; ++t) {
        const uint32_t qo = (uint32_t)rel * TB + lane_off;
        wq[slot][m][t][0] = buf_ld16(rq[m][t], qo);
        if constexpr (QW == 2) wq[slot][m][t][1] = buf_ld16(rq[m][t], qo + 1024u);
        wd[slot][m][t] = buf_ld8(rd[m][t], (uint32_t)rel * TILE_D_BYTES + d_off);
      }
  };

  // ---- 1. start the activations (first round) and the weight stream.
  // Batches of 4 to 7 columns stage several pieces per thread: the first
  // round then takes a whole batch, so that staging costs one memory round
  // trip less (measured, verify at 4 columns: Q8_0 5120 x 5120 11.15 ->
  // 10.4 us, Q4_0 5120 -> 17408 17.7 -> 17.2 us; the 16-token MoE layer,
  // whose expert entries are 4-column units, 67.0 -> 66.4 us; at 8 columns,
  // whose segments run across workgroups with few pieces per thread, no
  // gain).  The norm forms keep one piece (theirs carry gamma too).
  constexpr int XB = RMSN && QT == Q8 && NMAT == 2 ? 2 : 4;  // pieces per later batch
  constexpr int X0 = (!XS && NC >= 4 && NC < 8 && !RMSN) ? XB : 1;
  const int span0 = nvec;
  XPiece xp[X0];
  u4 fp[XCW];
  if constexpr (XS) {
#pragma unroll
    for (int j = 0; j < XCW; ++j) f16_ld(j, 0, fp[j]);
  } else {
#pragma unroll
    for (int i = 0; i < X0; ++i) x_ld(tid + i * NTHR, 0, span0, x_col(tid + i * NTHR), xp[i]);
  }
#pragma unroll
  for (int p = 0; p < PF; ++p) load(p, p);

  // ---- 2. staging (XS: chunk 0 into buffer 0).  Otherwise further pieces
  // of the read range go in batches of XB whose loads are all issued before
  // any is used.
  //
  // A piece past the range is loaded (it reads zeros) but not stored, so no
  // store waits for its load; left pending, that load would be waited for
  // wherever its register is next written, which can be inside the weight
  // stream, at every tile.  So each staging step ends with a wait of its
  // own: after each batch, for everything (the weight tiles were issued
  // earlier and return first); after the first pieces, for everything with
  // one matrix, else for everything but the first weight tiles.  The wait
  // at the loop's entry also shapes the waits the compiler places inside
  // it: measured, one matrix streams best after the full wait (6-7 loads
  // kept in flight per wave: decode down 14.0 -> 13.1 us), gate and up
  // together after the partial one (the full wait keeps more in flight
  // there and was 0.6 us slower).
  constexpr int NWL = PF * NMAT * RT * (QW + 1);  // loads of the first PF tile columns
  static_assert(NWL <= 63, "wait count");
  constexpr int WAIT_ALL = 0x0F70;                // vmcnt(0), other counters untouched
  constexpr int WAIT_X0 = NMAT == 1 ? WAIT_ALL : (WAIT_ALL | (NWL & 15) | ((NWL >> 4) << 14));
  if constexpr (XS) {
#pragma unroll
    for (int j = 0; j < XCW; ++j) f16_put(j, xs, fp[j]);
  } else {
#pragma unroll
    for (int i = 0; i < X0; ++i) x_put(tid + i * NTHR, span0, xs, xp[i]);
  }
  if constexpr (!XS) {
    __builtin_amdgcn_s_waitcnt(WAIT_X0);
    for (int v0 = tid + X0 * NTHR; v0 < nvec; v0 += XB * NTHR) {
      XPiece pc[XB];
#pragma unroll
      for (int b = 0; b < XB; ++b) x_ld(v0 + b * NTHR, 0, nvec, x_col(v0 + b * NTHR), pc[b]);
#pragma unroll
      for (int b = 0; b < XB; ++b) x_put(v0 + b * NTHR, nvec, xs, pc[b]);
      __builtin_amdgcn_s_waitcnt(WAIT_ALL);
    }
  }
  __syncthreads();
  if constexpr (RMSN) {
    // 1 / rms per column: lane l adds the column's pieces l, l + 64, ... in
    // order, then a fixed wave tree, so every workgroup (and every column
    // count) gets the same bits
    for (int c = wk; c < NC; c += NTHR >> 6) {
      float t = 0.0f;
      for (int p = lane; p < npc; p += 64) t += ssq[(size_t)c * npc + p];
      t = wave_sum(t);
      if (lane == 0) inv_rms[c] = 1.0f / __builtin_sqrtf(t / (float)a.cols + a.norm_eps);
    }
    __syncthreads();
  }

  // ---- 3. stream the weight tiles of the segment
  float acc[NMAT][RT][NI];
#pragma unroll
  for (int m = 0; m < NMAT; ++m)
#pragma unroll
    for (int t = 0; t < RT; ++t)
#pragma unroll
      for (int c = 0; c < NI; ++c) acc[m][t][c] = 0.0f;

  const Q4Magic mg = q4_magic();
  // matrix-core A operands: lane (r, sl) holds product row r, k 8 sl ..
  // 8 sl + 7.  16 columns: row r is column r.  1..8 columns: row c < NC is
  // column c's hi part, row LO + c its lo part.  Row r of A reaches only
  // row r of the product, so the lanes of the other rows load any staged
  // row (that of column 0): their results sit in accumulators nothing reads,
  // and every lane loads without a branch.  16 columns issue the four
  // blocks' reads and products together (the products of a tile overlap
  // the LDS reads); narrower batches, whose streams are bound by memory,
  // keep one block at a time.
  h8 A[TILE_BLOCKS];
  const int arow = F16 ? r : (r < NC ? r : (r >= LO && r < LO + NC ? NC + r - LO : 0));
  // 1..8 columns: the column of this lane's result i is cb + i (its hi or
  // its lo part); past NC it is unused, and reads a valid scale
  const int cb = (4 * sl) & (LO - 1);
  auto compute = [&](int slot, int rel) {
    if constexpr (F16) {
      // the slot of tile column rel in its chunk's buffer
      const int bl0 = ((((rel / CT) & 1) * CT) + rel % CT) * TILE_BLOCKS;
#pragma unroll
      for (int j = 0; j < TILE_BLOCKS; ++j) A[j] = *(const h8 *)(xs + xrow((size_t)(bl0 + j) * XC + r, sl));
#pragma unroll
      for (int m = 0; m < NMAT; ++m)
#pragma unroll
        for (int t = 0; t < RT; ++t) {
          h8 B[TILE_BLOCKS];
          f4 D[TILE_BLOCKS];
#pragma unroll
          for (int j = 0; j < TILE_BLOCKS; ++j) {
            h2 w[4];
            if constexpr (QT == Q4) unpack_q4(wq[slot][m][t][0][j], w, mg);
            else unpack_q8(wq[slot][m][t][j >> 1][(j & 1) * 2], wq[slot][m][t][j >> 1][(j & 1) * 2 + 1], w);
            B[j] = h8{w[0][0], w[0][1], w[1][0], w[1][1], w[2][0], w[2][1], w[3][0], w[3][1]};
            D[j] = __builtin_amdgcn_mfma_f32_16x16x32_f16(A[j], B[j], f4{0.f, 0.f, 0.f, 0.f}, 0, 0, 0);
          }
#pragma unroll
          for (int j = 0; j < TILE_BLOCKS; ++j) {
            const float dj = scale_of(wd[slot][m][t], j);
#pragma unroll
            for (int i = 0; i < NI; ++i) acc[m][t][i] = __builtin_fmaf(dj, D[j][i], acc[m][t][i]);
          }
          mfma_fence(acc[m][t], A, B, D);
        }
    } else {
      // staged tile of this tile column: compacted (own columns), else its
      // place in the unit's range
      const int st = own ? rel : wkt0 + rel * wst;
      // the powers of two of this lane's columns cb .. cb + 3 in this tile
      const float4 sv = *(const float4 *)(scl + (size_t)st * SCC + cb);
      float ts[NMAT][RT][NI];  // the tile's sums, block by block
#pragma unroll
      for (int j = 0; j < TILE_BLOCKS; ++j) {
        A[0] = *(const h8 *)(xs + xrow((size_t)(st * TILE_BLOCKS + j) * XC + arow, sl));
#pragma unroll
        for (int m = 0; m < NMAT; ++m)
#pragma unroll
          for (int t = 0; t < RT; ++t) {
            h2 w[4];
            if constexpr (QT == Q4) unpack_q4(wq[slot][m][t][0][j], w, mg);
            else unpack_q8(wq[slot][m][t][j >> 1][(j & 1) * 2], wq[slot][m][t][j >> 1][(j & 1) * 2 + 1], w);
            const h8 B = {w[0][0], w[0][1], w[1][0], w[1][1], w[2][0], w[2][1], w[3][0], w[3][1]};
            const f4 D = __builtin_amdgcn_mfma_f32_16x16x32_f16(A[0], B, f4{0.f, 0.f, 0.f, 0.f}, 0, 0, 0);
            const float dj = scale_of(wd[slot][m][t], j);
#pragma unroll
            for (int i = 0; i < NI; ++i) ts[m][t][i] = j == 0 ? dj * D[i] : __builtin_fmaf(dj, D[i], ts[m][t][i]);
            mfma_fence(ts[m][t], A[0], B, D);
          }
      }
#pragma unroll
      for (int m = 0; m < NMAT; ++m)
#pragma unroll
        for (int t = 0; t < RT; ++t)
#pragma unroll
          for (int i = 0; i < NI; ++i) acc[m][t][i] = __builtin_fmaf(sv[i], ts[m][t][i], acc[m][t][i]);
    }
  };

  // PF tile columns in flight; loads past the segment read nothing
  if constexpr (XS) {
    // every wave runs the same trip count: the chunk hand-over is a barrier
    // Chunk q (tile columns q CT ..) sits in buffer q % 2; the next chunk
    // is loaded as chunk q starts and stored into the other buffer as it
    // ends, where the barrier of chunk q - 1 has retired every read of it.
    const bool live = rt_base < a.NT;
    for (int k = 0; k < nkt; k += PF) {
#pragma unroll
      for (int c0 = 0; c0 < PF; c0 += CT) {
        u4 np[XCW];
#pragma unroll
        for (int j = 0; j < XCW; ++j) f16_ld(j, k + c0 + CT, np[j]);
#pragma unroll
        for (int p = c0; p < c0 + CT; ++p) {
          if (live && k + p < nkt) compute(p, k + p);
          load(p, k + p + PF);
        }
        _Float16 *nb = xs + ((((k + c0) / CT) + 1) & 1) * CHH;
#pragma unroll
        for (int j = 0; j < XCW; ++j) f16_put(j, nb, np[j]);
        __syncthreads();
      }
    }
  } else {
    const int nseg = rt_base < a.NT ? wnkt : 0;
    for (int k = 0; k < nseg; k += PF) {
#pragma unroll
      for (int p = 0; p < PF; ++p) {
        if (k + p < nseg) compute(p, k + p);
        load(p, k + p + PF);
      }
    }
    // hi and lo sums of each column meet: lane (r, sl) of a hi row adds
    // lane (r, sl + LO / 4)
    if constexpr (!F16) {
#pragma unroll
      for (int m = 0; m < NMAT; ++m)
#pragma unroll
        for (int t = 0; t < RT; ++t)
#pragma unroll
          for (int i = 0; i < NI; ++i) acc[m][t][i] += __shfl_down(acc[m][t][i], LO * 4);
    }
  }

  // ---- 4. per-row sums: lane (r, sl) holds column 4 sl + i of row r (1..8
  // columns: in its hi lanes, which now hold hi + lo)
  // (t, i) -> the column this lane handles, or -1
  auto col_of = [&](int t, int i) -> int {
    (void)t;
    const int c = 4 * sl + i;
    return c < NC ? c : -1;
  };

  auto emit = [&](int t, int c, const float (&v)[NMAT]) {
    const int64_t row = (rt_base + t) * 16 + r;
    if (rt_base + t >= a.NT || row >= a.rows || c >= a.ncols) return;
    if constexpr (EPI == EPI_ARGMAX || EPI == EPI_TOPK) {
      if (ranks_before(v[0], (int32_t)row, bv, bi)) { bv = v[0]; bi = (int32_t)row; }
    } else {
      float *yp = a.Y + (int64_t)(a.ymap ? a.ymap[c] : c) * a.ldy + row;
      float out;
      if constexpr (EPI == EPI_STORE) {
        out = v[0];
      } else if constexpr (EPI == EPI_ACC) {
        out = *yp + v[0];
      } else {
        float gg = v[0], uu = v[NMAT - 1];
        if constexpr (RMSN) {
          gg *= inv_rms[c];
          uu *= inv_rms[c];
        }
        const float sg = gg / (1.0f + expf(-gg));
        out = sg * uu;
      }
      if constexpr (PH == PH_PRODUCE) st_agent(yp, out);
      else *yp = out;
    }
  };

  // in-workgroup segments: the waves of segments 1.. leave their sums in
  // LDS (past the staged activations, which slower waves may still read);
  // the segment-0 wave of each row tile adds them in segment order, the
  // same order as the partials of segments across workgroups
  if (SW > 1) {
    constexpr int NV = NMAT * RT * NI;
    float *red = (float *)(smem + dot_stage_bytes(nst, NC));
    if (wsg > 0) {
#pragma unroll
      for (int m = 0; m < NMAT; ++m)
#pragma unroll
        for (int t = 0; t < RT; ++t)
#pragma unroll
          for (int i = 0; i < NI; ++i)
            red[((((wsg - 1) * R + wrt) * NV) + (m * RT + t) * NI + i) * 64 + lane] = acc[m][t][i];
    }
    __syncthreads();
    if (wsg == 0) {
      for (int q = 1; q < SW; ++q)
#pragma unroll
        for (int m = 0; m < NMAT; ++m)
#pragma unroll
          for (int t = 0; t < RT; ++t)
#pragma unroll
            for (int i = 0; i < NI; ++i)
              acc[m][t][i] += red[((((q - 1) * R + wrt) * NV) + (m * RT + t) * NI + i) * 64 + lane];
    }
  }

  bool emitted;
  if (a.S == 1) {
#pragma unroll
    for (int t = 0; t < RT; ++t)
#pragma unroll
      for (int i = 0; i < NI; ++i) {
        const int c = col_of(t, i);
        if (c >= 0 && wsg == 0) {
          float v[NMAT];
#pragma unroll
          for (int m = 0; m < NMAT; ++m) v[m] = acc[m][t][i];
          emit(t, c, v);
        }
      }
    emitted = true;
  } else {
    // publish the segment partials; the last workgroup of the row group
    // adds them in segment order
    // layout [segment][matrix][row tile][value i][lane]: each store and
    // load instruction of a wave covers one contiguous run
    auto pidx = [&](int ss, int m, int t, int i) -> int64_t {
      return ((((int64_t)ss * NMAT + m) * a.NT + (rt_base + t)) * NI + i) * 64 + lane;
    };
#pragma unroll
    for (int t = 0; t < RT; ++t)
#pragma unroll
      for (int i = 0; i < NI; ++i) {
        const int c = col_of(t, i);
        if (c >= 0 && rt_base + t < a.NT) {
#pragma unroll
          for (int m = 0; m < NMAT; ++m) st_agent(a.part + pidx(s, m, t, i), acc[m][t][i]);
        }
      }
    emitted = arrive_last(a.cnt + g, (uint32_t)a.S, flag);
    if (emitted) {
      // every segment's partial of every value this lane emits is loaded
      // before any is added (one round trip per RB segments, not one per
      // segment and value), then they are added in segment order; coherent
      // loads (sc1) over a bounded range of this launch's partials
      constexpr int RB = RT * NI * NMAT >= 8 ? 4 : 8;
      const int64_t pbytes = (int64_t)a.S * NMAT * a.NT * NI * 64 * 4;
      const __amdgpu_buffer_rsrc_t rp = buf_range(a.part, (uint32_t)(pbytes < 0x7FFFFFFF ? pbytes : 0x7FFFFFFF));
      auto poff = [&](int ss, int m, int t, int i) -> uint32_t {
        return (ss < a.S && col_of(t, i) >= 0 && rt_base + t < a.NT) ? (uint32_t)(pidx(ss, m, t, i) * 4)
                                                                      : 0xFFFFFFC0u;
      };
      float v[RT][NI][NMAT];
      for (int s0 = 0; s0 < a.S; s0 += RB) {
        float p[RT][NI][NMAT][RB];
#pragma unroll
        for (int t = 0; t < RT; ++t)
#pragma unroll
          for (int i = 0; i < NI; ++i)
#pragma unroll
            for (int m = 0; m < NMAT; ++m)
#pragma unroll
              for (int j = 0; j < RB; ++j)
                p[t][i][m][j] = __builtin_bit_cast(
                    float, __builtin_amdgcn_raw_buffer_load_b32(rp, poff(s0 + j, m, t, i), 0, 16));
#pragma unroll
        for (int t = 0; t < RT; ++t)
#pragma unroll
          for (int i = 0; i < NI; ++i)
#pragma unroll
            for (int m = 0; m < NMAT; ++m)
#pragma unroll
              for (int j = 0; j < RB; ++j)
                if (s0 + j < a.S) v[t][i][m] = s0 + j == 0 ? p[t][i][m][j] : v[t][i][m] + p[t][i][m][j];
      }
#pragma unroll
      for (int t = 0; t < RT; ++t)
#pragma unroll
        for (int i = 0; i < NI; ++i) {
          const int c = col_of(t, i);
          if (c >= 0 && rt_base + t < a.NT) emit(t, c, v[t][i]);
        }
    }
  }
  return emitted;
}

}  // namespace qg
