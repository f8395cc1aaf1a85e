// One work unit of the product kernels: W row tiles (one per wave, of one
// matrix or of gate and up together) over one K segment, used by the GEMV
// (1..8 columns), gate/up, LM head and 16-column GEMM kernels, the fused
// FFN and the MoE expert kernels.
//
// What is computed ("Engine and kernels", Kernel families): y = W x over
// Q4_0 / Q8_0 blocks dequantised in registers with f32 sums, with the
// epilogues of the kernel families (store, y += W x, SiLU(gate) * up, and
// the per-row values an argmax needs).
//
// How (MI355X):
//  * The workgroup stages its activations once in LDS as f16,
//    [block][column][32] (16 columns: in double-buffered chunks).
//  * One wave streams one row tile across its segment, PF tile columns
//    ahead; each 16-byte load of a wave reads a contiguous 1 KiB stripe.
//    The stream is a bounded buffer range, so loads past it return zeros
//    without touching memory and the loop has no branch around its loads.
//  * Weights become exact f16 values; per block, one matrix-core product
//    (activation columns x the block's 16 rows) gives each lane its columns,
//    scaled by the block's f16 scale into f32 accumulators.
//  * Segments: S of them, contiguous K ranges or interleaved tile columns
//    (segment q takes q, q + S, ...), chosen by the shape; summed in
//    segment order, either by the last workgroup of the row group (from
//    partials in memory) or, with the segments as waves of one workgroup,
//    through LDS.  The order depends on the shape only, so each activation
//    column of a batched call is bitwise equal to a 1-column call
//    ("Architecture", Speculative decoding).
//
// Phases, for the fused FFN: a producer unit (gate/up) publishes the h rows
// of its row group with coherent stores and then raises the ready flag of
// each of its row tiles; a consumer unit (down) issues its first weight
// loads, waits until the flags of the h row tiles its K segment reads are
// raised, and reads h with coherent loads.
#pragma once
#include "common.h"
#include "internal.h"

namespace qg {

// Segment q of a K range of kt tile columns cut into n pieces.
__host__ __device__ inline int seg_begin(int q, int kt, int n) { return (int)((int64_t)kt * q / n); }

enum Phase { PH_PLAIN = 0, PH_PRODUCE = 1, PH_CONSUME = 2 };

// Multiply form of the dot path: the matrix cores (true) or v_dot2 (false).
#ifndef DOT_MF
#define DOT_MF true
#endif

// Polls before a consumer gives up waiting (about 0.1 s); a correct launch
// never gets near it, it only guarantees the kernel ends.
constexpr int WAIT_POLLS = 1 << 20;

struct DotArgs {
  const uint8_t *qs0, *qs1, *d0, *d1;
  int64_t rows;       // outputs produced (n_rows for the LM head)
  int64_t cols;
  int NT, KT;         // row tiles produced, tile columns of the matrix
  int S;              // K segments across workgroups
  int SW;             // K segments inside one workgroup (<= 1: none): wave wk
                      // streams segment wk / R of row tile wk % R, R = waves / SW
  int IL;             // interleaved segments: segment q of n holds tile columns
                      // q, q + n, q + 2n, ... (every unit stages all of K);
                      // otherwise contiguous ranges
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
  uint32_t *ready;    // fused FFN: one flag per h row tile, raised by its producer unit
  int ready_n;        // fused FFN, consumer: h row tiles (flags) in all
  uint32_t *err;      // fused FFN: set when a wait gave up
  int NWU;            // waves of the unit (<= 0: every wave of the workgroup); the
                      // other waves only take part in its barriers
  const float *gamma; // RMSNorm prologue: the weights (cols), and eps
  float norm_eps;
  const int32_t *xmap, *ymap;  // MoE: column c reads X column xmap[c], writes Y column ymap[c]
  int64_t xspan;      // bytes of X the columns may read (0: the ncols columns)
};

// The default `staged` hook of dot_unit: nothing.
struct NoHook {
  __device__ void operator()() const {}
};

// Register fence after a matrix-core product and the FMAs that read its
// result.  The matrix core reads A and B and writes all four result
// registers over several passes after the instruction issues; a register it
// still reads or writes must not be handed to another value meanwhile.  The
// statement takes A, B and the whole result and rewrites the accumulators
// the FMAs produced, so it is ordered after those FMAs (which wait for the
// product to complete) and all of A, B and D stay allocated until then, also
// the result values no FMA reads (fewer than four columns).
// Floats of one row tile's segment partial: NI values per lane, 64 lanes
// (NI: columns per lane, at most 4 in the matrix-core form).
__host__ __device__ constexpr int dot_part_floats(int nc) { return (DOT_MF ? (nc < 4 ? nc : 4) : nc) * 64; }

// Smallest workgroup (waves) a streamed-staging unit of launch-time size
// runs with: its per-thread chunk pieces are sized for it.
constexpr int DOT_XS_WMIN = 8;

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

// The unit (row group g, segment s) of the launch `a`.  RMSN (gate/up,
// units that stage all of K): the activations are RMS-normalised first, as
// x * gamma staged, times 1 / sqrt(mean(x^2) + eps) per column applied to
// the two products (the same value, since the products are linear in x).
// Returns true when
// this workgroup emitted the outputs of row group g (its only segment, or
// the last of its segments to finish).  For the argmax epilogue, (bv, bi)
// then hold each lane's best (value, row).  `staged` runs once the
// activations are in LDS and the first weight loads are in flight (the
// fused FFN takes its next work unit there, so that round trip overlaps the
// stream).
template <int QT, int NC, int NMAT, int EPI, int RT, int PF, int WKT, int PH, bool MF = false,
          class Hook = NoHook, bool RMSN = false>
__device__ __forceinline__ bool dot_unit(const DotArgs &a, int g, int s, uint8_t *smem, uint32_t *flag,
                                          float &bv, int32_t &bi, Hook staged = Hook()) {
  // WKT == 0: one row tile per wave of the workgroup as launched (at least
  // XWMIN waves when the activations stream in chunks)
  const int NTHR = WKT > 0 ? WKT * 64 : (int)blockDim.x;
  constexpr int XC = NC;  // activation columns in the LDS layout
  // accumulators per lane: dot form, one per column; matrix-core form, the
  // 4 D values of lane (r, sl) are columns 4 sl + i
  constexpr int NI = MF ? (NC < 4 ? NC : 4) : NC;
  constexpr int TB = QTraits<QT>::tile_bytes;
  constexpr int QW = (QT == Q4) ? 1 : 2;  // 16-byte loads per lane per tile
  constexpr int XAUX = PH == PH_CONSUME ? 16 : 0;  // sc1: h comes from other XCDs
  // Wide batches stream their activations in chunks of PF tile columns,
  // double-buffered in LDS and staged one chunk ahead of the products (the
  // whole segment would take several L2 round trips before the first
  // product); narrow ones stage the whole segment up front.
  constexpr bool XS = NC >= 16;
  constexpr int CHV = PF * TILE_BLOCKS * NC * 4;   // 8-value pieces per chunk
  constexpr int CHH = PF * TILE_BLOCKS * NC * 32;  // halves per chunk buffer
  constexpr int XWMIN = WKT > 0 ? WKT : DOT_XS_WMIN;
  constexpr int XR = (CHV + XWMIN * 64 - 1) / (XWMIN * 64);  // pieces per thread per chunk (at most)

  const int tid = threadIdx.x, lane = tid & 63;
  const int wk = __builtin_amdgcn_readfirstlane(tid >> 6);
  // the workgroup's K range (staged in LDS), and inside it this wave's
  // stream: all of it, or (SW > 1) in-workgroup segment wsg of SW.
  // Interleaved segments: the workgroup stages all of K and the wave's
  // segment q of nq takes tile columns q, q + nq, ... (wst = nq);
  // contiguous ones: its range [wkt0, wkt0 + wnkt) of the staged columns.
  const int SW = (!XS && a.SW > 1) ? a.SW : 1;
  const int NWA = a.NWU > 0 ? a.NWU : (NTHR >> 6);  // waves of the unit
  const bool idle = wk >= NWA;                      // stages, waits at barriers, streams nothing
  const int R = NWA / SW;
  const int wrt = idle ? 0 : wk % R, wsg = idle ? 0 : wk / R;
  const bool IL = !XS && a.IL;
  const int kt0 = IL ? 0 : seg_begin(s, a.KT, a.S);
  const int nkt = IL ? a.KT : seg_begin(s + 1, a.KT, a.S) - kt0;
  const int wq_i = SW > 1 ? wsg : s, wq_n = SW > 1 ? SW : a.S;  // this wave's segment of how many
  const int wkt0 = IL ? wq_i : seg_begin(wsg, nkt, SW);        // first tile column, relative to kt0
  const int wst = IL ? wq_n : 1;                               // step between its tile columns
  const int wnkt = IL ? (nkt - wq_i + wq_n - 1) / wq_n : seg_begin(wsg + 1, nkt, SW) - wkt0;
  const int64_t rt_base = idle ? (int64_t)a.NT : ((int64_t)g * R + wrt) * RT;
  const int r = lane & 15, sl = lane >> 4;
  _Float16 *xs = (_Float16 *)smem;

  // activations: a bounded range over the columns; a chunk outside the
  // segment or the matrix reads zeros
  const int nvec = nkt * TILE_BLOCKS * NC * 4;  // 8-value pieces of the segment
  const __amdgpu_buffer_rsrc_t rx =
      buf_range(a.X, (uint32_t)(a.xspan ? a.xspan : ((int64_t)(a.ncols - 1) * a.ldx + a.cols) * 4));
  // the X column piece v reads (through the column map, if any); a piece's
  // column does not change from chunk to chunk, so streamed staging looks
  // it up once, not inside the weight stream (a map load there would make
  // every chunk wait for all weight loads in flight)
  auto x_col = [&](int v) -> int64_t {
    const int c = (v >> 2) % NC;
    return c < a.ncols && a.xmap ? a.xmap[c] : c;
  };
  // piece v of the `span` pieces from tile column rel0 on: (block, column,
  // 8 k) -> byte offset in X column xc, or past any range (reads zeros) when
  // it lies outside the span, the segment or the matrix
  auto x_off = [&](int v, int rel0, int span, int64_t xc) -> uint32_t {
    const int qq = v & 3, c = (v >> 2) % NC, bl = (v >> 2) / NC;
    const int64_t k = ((int64_t)(kt0 + rel0) * TILE_BLOCKS + bl) * 32 + qq * 8;
    const bool ok = v < span && rel0 * TILE_BLOCKS + bl < nkt * TILE_BLOCKS && k < a.cols && c < a.ncols;
    return ok ? (uint32_t)((xc * a.ldx + k) * 4) : 0xFFFFFFC0u;
  };
  // RMSNorm: gamma over the same 8 k of a piece (its range: cols floats;
  // a piece outside reads zeros), and per staged piece the sum of its 8
  // squares, [column][piece along K], past the staged activations and the
  // in-workgroup sums; then 1 / rms per column
  static_assert(!RMSN || (!XS && EPI == EPI_SILU), "RMSNorm prologue: gate/up, staged whole");
  const __amdgpu_buffer_rsrc_t rg = buf_range(a.gamma, RMSN ? (uint32_t)(a.cols * 4) : 0u);
  const int npc = nkt * TILE_BLOCKS * 4;  // pieces of one column
  float *ssq = (float *)(smem + (size_t)nkt * TILE_BLOCKS * NC * 64 +
                         (SW > 1 ? (size_t)(SW - 1) * R * NMAT * RT * NI * 64 * 4 : 0));
  float *inv_rms = ssq + (size_t)NC * npc;
  struct XPiece {
    u4 lo, hi, glo, ghi;
  };
  auto x_ld = [&](int v, int rel0, int span, int64_t xc, XPiece &pc) {
    const uint32_t o = x_off(v, rel0, span, xc);
    pc.lo = __builtin_amdgcn_raw_buffer_load_b128(rx, o, 0, XAUX);
    pc.hi = __builtin_amdgcn_raw_buffer_load_b128(rx, o + 16u, 0, XAUX);
    if constexpr (RMSN) {
      const int qq = v & 3, bl = (v >> 2) / NC;
      const int64_t k = ((int64_t)(kt0 + rel0) * TILE_BLOCKS + bl) * 32 + qq * 8;
      const uint32_t og = o != 0xFFFFFFC0u ? (uint32_t)(k * 4) : 0xFFFFFFC0u;
      pc.glo = __builtin_amdgcn_raw_buffer_load_b128(rg, og, 0, 0);
      pc.ghi = __builtin_amdgcn_raw_buffer_load_b128(rg, og + 16u, 0, 0);
    }
  };
  auto x_put = [&](int v, int span, _Float16 *dst, const XPiece &pc) {
    if (v < span) {
      const int qq = v & 3, c = (v >> 2) % NC, bl = (v >> 2) / NC;
      float4 lo = __builtin_bit_cast(float4, pc.lo), hi = __builtin_bit_cast(float4, pc.hi);
      if constexpr (RMSN) {
        // the piece's squares in k order, then x * gamma
        float q = lo[0] * lo[0];
        q = __builtin_fmaf(lo[1], lo[1], q);
        q = __builtin_fmaf(lo[2], lo[2], q);
        q = __builtin_fmaf(lo[3], lo[3], q);
        q = __builtin_fmaf(hi[0], hi[0], q);
        q = __builtin_fmaf(hi[1], hi[1], q);
        q = __builtin_fmaf(hi[2], hi[2], q);
        q = __builtin_fmaf(hi[3], hi[3], q);
        ssq[(size_t)c * npc + bl * 4 + qq] = q;
        const float4 glo = __builtin_bit_cast(float4, pc.glo), ghi = __builtin_bit_cast(float4, pc.ghi);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          lo[e] *= glo[e];
          hi[e] *= ghi[e];
        }
      }
      *(h8 *)(dst + ((size_t)bl * XC + c) * 32 + qq * 8) = cvt8(lo, hi);
    }
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

  // ---- 1. start the weight stream, and (first round) the activations
  constexpr int X0 = XS ? XR : 1;
  const int span0 = XS ? CHV : nvec;
  XPiece xp[X0];
  int64_t xcs[X0];
#pragma unroll
  for (int i = 0; i < X0; ++i) xcs[i] = x_col(tid + i * NTHR);
  if constexpr (PH != PH_CONSUME) {
#pragma unroll
    for (int i = 0; i < X0; ++i) x_ld(tid + i * NTHR, 0, span0, xcs[i], xp[i]);
  }
#pragma unroll
  for (int p = 0; p < PF; ++p) load(p, p);

  if constexpr (PH == PH_CONSUME) {
    // the activations are h rows other workgroups produce: wait until the
    // ready flags of the h row tiles of this segment's tile columns (8 row
    // tiles of 16 to a column of 128) are raised
    if (wk == 0) {
      const int f0 = kt0 * 8, nf = (nkt * 8 < a.ready_n - f0) ? nkt * 8 : a.ready_n - f0;
      for (int it = 0;; ++it) {
        bool ok = true;
        for (int j = lane; j < nf; j += 64) ok = ok && ld_agent_u32(a.ready + f0 + j) != 0u;
        if (__all(ok)) break;
        if (it >= WAIT_POLLS) {
          if (lane == 0) st_agent_u32(a.err, 1u);
          break;
        }
        __builtin_amdgcn_s_sleep(2);
      }
    }
    __syncthreads();
#pragma unroll
    for (int i = 0; i < X0; ++i) x_ld(tid + i * NTHR, 0, span0, xcs[i], xp[i]);
  }

  // ---- 2. staging: f16 in LDS, [block][column][32] (XS: chunk 0 into
  // buffer 0).  Otherwise further pieces of the segment go in batches of XB
  // whose loads are all issued before any is used.
  //
  // A piece past the segment is loaded (it reads zeros) but not stored, so
  // no store waits for its load; left pending, that load would be waited
  // for wherever its register is next written, which can be inside the
  // weight stream, at every tile.  So each staging step ends with a wait of
  // its own: after each batch, for everything (the weight tiles were issued
  // earlier and return first); after the first pieces, for everything with
  // one matrix or when the activations came last, else for everything but
  // the first weight tiles.  The wait at the loop's entry also shapes the
  // waits the compiler places inside it: measured, one matrix streams best
  // after the full wait (6-7 loads kept in flight per wave: decode down
  // 14.0 -> 13.1 us), gate and up together after the partial one (the full
  // wait keeps more in flight there and was 0.6 us slower).
  constexpr int NWL = PF * NMAT * RT * (QW + 1);  // loads of the first PF tile columns
  static_assert(NWL <= 63, "wait count");
  constexpr int WAIT_ALL = 0x0F70;                // vmcnt(0), other counters untouched
  constexpr int WAIT_X0 =
      (PH == PH_CONSUME || NMAT == 1) ? WAIT_ALL : (WAIT_ALL | (NWL & 15) | ((NWL >> 4) << 14));
#pragma unroll
  for (int i = 0; i < X0; ++i) x_put(tid + i * NTHR, span0, xs, xp[i]);
  if constexpr (!XS) {
    __builtin_amdgcn_s_waitcnt(WAIT_X0);
    constexpr int XB = 4;
    for (int v0 = tid + NTHR; v0 < nvec; v0 += XB * NTHR) {
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
  staged();

  // ---- 3. stream the weight tiles of the segment
  float acc[NMAT][RT][NI];
#pragma unroll
  for (int m = 0; m < NMAT; ++m)
#pragma unroll
    for (int t = 0; t < RT; ++t)
#pragma unroll
      for (int c = 0; c < NI; ++c) acc[m][t][c] = 0.0f;

  const Q4Magic mg = q4_magic();
  // matrix-core A operands of a tile's four blocks: lane (r, sl) holds
  // column r, k 8 sl .. 8 sl + 7.  Lanes of columns past NC keep zeros: they
  // never load (exec-masked), so the registers set to zero here stay zero.
  // 16 columns issue the four blocks' reads and products together (the
  // products of a tile overlap the LDS reads); narrower batches, whose
  // streams are bound by memory, keep one block at a time (fewer registers:
  // the fused FFN keeps two workgroups per CU).
#ifndef DOT_GA_MIN
#define DOT_GA_MIN 16
#endif
  constexpr bool GA = NC >= DOT_GA_MIN;
  h8 A[TILE_BLOCKS];
#pragma unroll
  for (int j = 0; j < TILE_BLOCKS; ++j) A[j] = h8{0, 0, 0, 0, 0, 0, 0, 0};
  auto compute = [&](int slot, int rel) {
    // block index in LDS: the staged range's own (this wave's stream starts
    // wkt0 tile columns in), or, streaming, the slot of tile column rel in
    // its chunk's buffer
    const int bl0 = XS ? ((((rel / PF) & 1) * PF) + rel % PF) * TILE_BLOCKS : (wkt0 + rel * wst) * TILE_BLOCKS;
    if constexpr (MF) {
      // per block: D (16 columns x 16 rows) = X_blk^T W_blk^T on the matrix
      // cores from the exact f16 weights, then each lane's 4 D values get
      // the block scale of its row, blocks in order
      if constexpr (!GA) {
#pragma unroll
        for (int j = 0; j < TILE_BLOCKS; ++j) {
          if (NC == 16 || r < NC) A[0] = *(const h8 *)(xs + ((size_t)(bl0 + j) * XC + r) * 32 + sl * 8);
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
              for (int i = 0; i < NI; ++i) acc[m][t][i] = __builtin_fmaf(dj, D[i], acc[m][t][i]);
              mfma_fence(acc[m][t], A[0], B, D);
            }
        }
        return;
      }
#pragma unroll
      for (int j = 0; j < TILE_BLOCKS; ++j)
        if (NC == 16 || r < NC) A[j] = *(const h8 *)(xs + ((size_t)(bl0 + j) * XC + r) * 32 + sl * 8);
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
      return;
    }
#pragma unroll
    for (int j = 0; j < TILE_BLOCKS; ++j) {
      h2 xv[NC][4];
#pragma unroll
      for (int c = 0; c < NC; ++c) {
        const h8 xx = *(const h8 *)(xs + ((size_t)(bl0 + j) * XC + c) * 32 + sl * 8);
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
  };

  // PF tile columns in flight; loads past the segment read nothing
  if constexpr (XS) {
    // every wave runs the same trip count: the chunk hand-over is a barrier
    const bool live = rt_base < a.NT;
    for (int k = 0; k < nkt; k += PF) {
      XPiece np[XR];
#pragma unroll
      for (int i = 0; i < XR; ++i) x_ld(tid + i * NTHR, k + PF, CHV, xcs[i], np[i]);
#pragma unroll
      for (int p = 0; p < PF; ++p) {
        if (live && k + p < nkt) compute(p, k + p);
        load(p, k + p + PF);
      }
      _Float16 *nb = xs + (((k / PF) + 1) & 1) * CHH;
#pragma unroll
      for (int i = 0; i < XR; ++i) x_put(tid + i * NTHR, CHV, nb, np[i]);
      __syncthreads();
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
  }

  // ---- 4. per-row sums.  Dot form: after the butterfly every lane of row r
  // holds the same (bitwise) sum of the wave's segment, and lane (r, sl)
  // handles the outputs o = t * NC + c with o % 4 == sl.  Matrix-core form:
  // lane (r, sl) holds column 4 sl + i of row r.
  if constexpr (!MF) {
#pragma unroll
    for (int m = 0; m < NMAT; ++m)
#pragma unroll
      for (int t = 0; t < RT; ++t)
#pragma unroll
        for (int c = 0; c < NC; ++c) {
          float v = acc[m][t][c];
          v += __shfl_xor(v, 16);
          v += __shfl_xor(v, 32);
          acc[m][t][c] = v;
        }
  }
  // (t, i) -> the column this lane handles, or -1
  auto col_of = [&](int t, int i) -> int {
    if constexpr (MF) {
      const int c = 4 * sl + i;
      return c < NC ? c : -1;
    } else {
      return ((t * NC + i) & 3) == sl ? i : -1;
    }
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
    float *red = (float *)(smem + (size_t)((a.KT + a.S - 1) / a.S) * TILE_BLOCKS * NC * 64);
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

  if constexpr (PH == PH_PRODUCE) {
    // h rows of row group g are out: raise the flags of its row tiles once
    // every wave's stores are acknowledged
    if (emitted && a.ready) {
      __asm__ volatile("s_waitcnt vmcnt(0)" ::: "memory");
      __syncthreads();
      const int64_t f = (int64_t)g * R * RT + tid;
      if (tid < R * RT && f < a.NT) st_agent_u32(a.ready + f, 1u);
    }
  }
  return emitted;
}

}  // namespace qg
