// MoE FFN on gfx950: router, top-k, grouped expert gate/up + SiLU, grouped
// expert down and the weighted combine, in three stream-ordered launches
// with no host readback ("Engine and kernels", Kernel families: router,
// top-k, expert gate/up and down and the weighted combine all on the GPU;
// the MoE model has 256 experts, 8 active per token, plus a shared expert).
// Experts are stacked by role ("A 235B model in a browser window": all gate
// matrices in one tensor, all up in a second, all down in a third).
//
//  1. router: a few waves per (token, expert) form that f32 logit (f32
//     operands, f32 FMA); the last workgroup to store a token's logits picks
//     its top k (value descending, index ascending) and softmax weights, and
//     the last of those builds a work list in expert index order of entries
//     of at most 4 routed slots of one expert (slot = token * k + rank).
//  2. gate/up: the work unit of dot_unit.h over (listed expert, row group, K
//     segment): each expert's gate and up tiles are read once for all of its
//     slots (the unit's activation columns are the routed tokens' x, through
//     a column map) and h = silu(g) * u is written per slot.
//  3. down, token-major (3'): one workgroup per (token, output row group),
//     one wave per rank and one for the shared expert, each a 1-column
//     product of its expert's rows with its slot's h; the waves meet in LDS,
//     sum_k p_k z_k in rank order plus the shared expert, added to Y once.
//     For wide experts (h columns too large for LDS) the entry-grouped form:
//     the dot unit over (listed expert, row group) writes z = D h per slot
//     and the last workgroup to finish a row group forms the same sum.
// Workgroups beyond the listed experts exit at once (the grid is the worst
// case, the list is on the device).
#include <string.h>

#include "common.h"
#include "dot_unit.h"
#include "internal.h"
#include "qgemm.h"

namespace qg {

constexpr int RW = 16;      // router: experts (waves) per workgroup, = TMAX
constexpr int TMAX = 16;    // tokens per call
constexpr int MOE_WMAX = 16;  // expert units: at most 16 waves (row tiles) per workgroup

struct MoeArgs {
  int64_t H, F, SF, Fmax;
  int E, k, norm, T, Umax;
  int rparts;             // router: waves per logit (parts of the hidden range)
  const float *R;
  const uint8_t *gq, *uq, *dq, *gd, *ud, *dd;
  const uint8_t *sgq, *suq, *sdq, *sgd, *sud, *sdd;
  int64_t gu_qs_stride, gu_d_stride, dn_qs_stride, dn_d_stride;
  const float *X;
  int64_t ldx;
  float *Y;
  int64_t ldy;
  int32_t *topk_idx;
  float *topk_w;
  uint32_t *rcnt, *tcnt, *dcnt, *gcnt, *nused;
  float *logits, *pw, *hbuf, *zbuf, *gpart, *dpart;
  int32_t *sel, *used_e, *used_cnt, *used_slot;
  int S_gu, G_gu, G_dn;   // gate/up K segments and row groups (at Fmax rows); down row groups
  int W_gu, W_dn;         // row tiles per gate/up and per down workgroup
  int sw_gu;              // gate/up K segments as waves of one workgroup (summed in LDS)
  int dn_tok, R_dt, G_dt; // token-major down: on/off, row tiles per wave, row groups
  int sel_local;          // one token: each gate/up workgroup selects the experts itself
  int il_gu;              // gate/up: interleaved K segments
  int nsh;                // shared-expert entries (tokens in groups of the unit width)
  const float *rms_w;     // RMSNorm ahead of router and experts (NULL: none), and eps
  float rms_eps;
  int64_t gpart_per;      // gate/up partial floats per listed expert
  int S_dn;               // entry-grouped down: K segments across workgroups
  uint32_t *dscnt;        // ... their counters, per (listed expert, row group)
  int64_t dpart_per;      // ... and partial floats per listed expert
};

static size_t a256(size_t v) { return (v + 255) & ~size_t(255); }
// LDS of one wave of the token-major down projection: its h column as hi
// and lo halves (f16 each) and one f32 power of two per tile column of 128
__host__ __device__ constexpr size_t dn_tok_stage_bytes(int64_t fmax) { return (size_t)fmax * 4 + (size_t)fmax / 32; }
__host__ __device__ static inline int64_t cdiv(int64_t a, int64_t b) { return (a + b - 1) / b; }

// Column capacity of the expert units: a work-list entry holds at most this
// many routed slots of one expert (an expert with more gets several
// entries, each reading its weights once for its slots).
static int moe_nc(int T) { return T <= 1 ? 1 : T <= 2 ? 2 : 4; }
// gate/up K segments: short streams at one or two tokens (latency-bound),
// one segment when more columns share each weight tile
static int moe_s_gu(int64_t H, int T) {
  const int64_t KT = H / 128;
  int64_t s = T <= 2 ? KT / 4 : 1;
  return (int)(s < 1 ? 1 : s);
}

// Waves (row tiles) per expert workgroup: gate/up, down.
static void moe_waves(int T, int &w_gu, int &w_dn) {
  // measured on the 256-expert layer: small gate/up workgroups at one or
  // two tokens (many short streams), 8 row tiles once several tokens share
  // the experts (fewer, longer units)
  w_gu = T <= 2 ? 2 : 8;
  w_dn = 8;
}

struct MoeLayout {
  size_t nused, logits, sel, pw, used_e, used_cnt, used_slot, hbuf, zbuf, gpart, dpart, total;
  int64_t umax;  // work-list entries at most
  size_t rcnt_w, dcnt_w, gcnt_w, dscnt_w, sync_words;  // counter word offsets
  int S_gu, G_gu, G_dn, nsh, S_dn;
  int64_t dpart_per;
  int W_gu, W_dn, sw_gu, dn_tok, R_dt;
  int64_t gpart_per;
};

static MoeLayout moe_layout(const qg_moe *m, int T) {
  MoeLayout L;
  const int64_t Fmax = m->sh_ffn > m->ffn ? m->sh_ffn : m->ffn;
  const int nc = moe_nc(T);
  // work-list entries: each holds at least one slot and at most nc of one expert
  const int64_t by_e = (int64_t)m->n_expert * ((T + nc - 1) / nc);
  const int64_t umax = (int64_t)T * m->top_k < by_e ? (int64_t)T * m->top_k : by_e;
  const int64_t slots = (int64_t)T * m->top_k + T;
  L.umax = umax;
  L.S_gu = moe_s_gu(m->hidden, T);
  moe_waves(T, L.W_gu, L.W_dn);
  // gate/up segments as waves of one workgroup (no partials in memory)
  // when the workgroup stays within 16 waves and its activations (all of
  // K, nc columns) plus the segment sums fit comfortably in LDS
  L.sw_gu = L.S_gu > 1 && L.W_gu * L.S_gu <= MOE_WMAX &&
            dot_stage_bytes(m->hidden / 128, nc) + (size_t)L.S_gu * L.W_gu * 2 * 4 * 64 * 4 <= 65536;
  // the token-major down projection (see moe_down_tok_kernel; measured
  // faster than the entry-grouped one at 1 to 16 tokens) while each wave's
  // h column fits in LDS; more row tiles per wave as tokens add workgroups
  L.R_dt = T <= 2 ? 1 : T <= 8 ? 2 : 4;
  L.dn_tok = (size_t)(m->top_k + 1) * (dn_tok_stage_bytes(Fmax) + (size_t)L.R_dt * 64) <= 131072;
  L.G_gu = (int)cdiv(Fmax / 16, L.W_gu);
  L.G_dn = (int)cdiv(m->hidden / 16, L.W_dn);
  L.gpart_per = L.S_gu > 1 ? (int64_t)L.S_gu * 2 * (Fmax / 16) * dot_part_floats(nc) : 0;
  // entry-grouped down (wide experts): contiguous K segments across
  // workgroups so that each unit's h columns fit in 64 KiB of LDS
  L.S_dn = L.dn_tok ? 1 : (int)cdiv((int64_t)dot_stage_bytes(Fmax / 128, nc), 65536);
  if (L.S_dn > Fmax / 128) L.S_dn = (int)(Fmax / 128);
  L.dpart_per = L.S_dn > 1 ? (int64_t)L.S_dn * (m->hidden / 16) * dot_part_floats(nc) : 0;
  // counters (in the shared counter words): the router's, one per down row
  // group, one per (listed expert, gate/up row group)
  L.rcnt_w = 0;  // then one word per token
  L.dcnt_w = 4 + TMAX;
  L.gcnt_w = L.dcnt_w + (size_t)L.G_dn;
  L.nsh = m->sh_ffn > 0 ? (T + nc - 1) / nc : 0;  // shared-expert entries
  L.dscnt_w = L.gcnt_w + (size_t)(umax + L.nsh) * L.G_gu;
  L.sync_words = L.dscnt_w + (L.S_dn > 1 ? (size_t)(umax + L.nsh) * L.G_dn : 0);
  size_t o = QG_WS_SYNC_BYTES;
  L.nused = o; o += 256;
  L.logits = o; o += a256((size_t)T * m->n_expert * 4);
  L.sel = o; o += a256((size_t)T * m->top_k * 4);
  L.pw = o; o += a256((size_t)T * m->top_k * 4);
  L.used_e = o; o += a256((size_t)umax * 4);
  L.used_cnt = o; o += a256((size_t)umax * 4);
  L.used_slot = o; o += a256((size_t)umax * TMAX * 4);
  L.hbuf = o; o += a256((size_t)slots * Fmax * 4);
  L.zbuf = o; o += a256((size_t)slots * m->hidden * 4);
  L.gpart = o; o += a256((size_t)(umax + L.nsh) * L.gpart_per * 4);
  L.dpart = o; o += a256((size_t)(umax + L.nsh) * L.dpart_per * 4);
  L.total = o;
  return L;
}

size_t moe_ws_bytes(const qg_moe *m, int ntok) { return moe_layout(m, ntok).total; }

// One token's selection, by one wave: the token's logits in registers (NJ
// per lane, n_expert <= 64 NJ), k rounds of a wave maximum over each lane's
// best remaining key (after which only the lane that owned the winner looks
// at its keys again), then the softmax weights.  Lane kk < k receives the
// expert of rank kk and its weight.
template <int NJ>
__device__ __forceinline__ void select_token(const MoeArgs &a, int t, int lane, int32_t &out_e, float &out_p) {
  float lv[NJ];
  uint64_t key[NJ];
#pragma unroll
  for (int j = 0; j < NJ; ++j) {
    const int ee = lane + 64 * j;
    lv[j] = ee < a.E ? ld_agent(a.logits + (int64_t)t * a.E + ee) : 0.0f;
    key[j] = ee < a.E ? rank_key(lv[j], ee) : 0;
  }
  uint64_t loc = 0;  // this lane's best remaining key
#pragma unroll
  for (int j = 0; j < NJ; ++j) loc = key[j] > loc ? key[j] : loc;
  float mx = 0.0f, sumsel = 0.0f, my_ex = 0.0f;
  int32_t my_e = 0;  // lane kk: the expert of rank kk
  for (int kk = 0; kk < a.k; ++kk) {
    const uint64_t w = wave_max_key(loc);
    const int32_t bi = rank_key_index(w);
    const float bv = rank_key_value(w);
    if (kk == 0) mx = bv;  // the largest logit
    const float ex = expf(bv - mx);
    sumsel += ex;
    if (lane == kk) {
      my_e = bi;
      my_ex = ex;
    }
    if (loc == w) {  // the owner: drop the winner, find its next best
      loc = 0;
#pragma unroll
      for (int j = 0; j < NJ; ++j) {
        if (key[j] == w) key[j] = 0;
        loc = key[j] > loc ? key[j] : loc;
      }
    }
  }
  float sum = sumsel;
  if (!a.norm) {
    float part = 0.0f;
#pragma unroll
    for (int j = 0; j < NJ; ++j)
      if (lane + 64 * j < a.E) part += expf(lv[j] - mx);
    sum = wave_sum(part);
  }
  out_e = my_e;
  out_p = my_ex / sum;
}

// ------------------------------------------------------------ 1. router
// P waves per (token, expert) pair (P parts of the hidden range, P larger
// when there are few pairs, so that the router matrix is read by many CUs);
// the parts meet in LDS in part order.  The pairs are token-major, so the
// logits of one token come from a run of consecutive workgroups.  With
// several tokens, the last workgroup to store a token's logits selects that
// token with one wave (the token's logits in registers, NJ per lane,
// n_expert <= 64 NJ: k rounds of a wave maximum over each lane's best
// remaining key), so the tokens are selected on different CUs at once
// (measured at 16 tokens, 256 experts: the router 17.0 -> 14.5 us against
// one workgroup selecting every token with one wave each).  The last
// selector builds the work list.
template <int NCAP, int NJ>
__global__ void __launch_bounds__(RW * 64) moe_router_kernel(MoeArgs a) {
  constexpr int NTHR = RW * 64;
  constexpr int NSLOT = TMAX * 8;       // routed slots at most (top_k <= 8)
  constexpr int MW = NSLOT / 32;        // mask words per expert
  __shared__ uint32_t flag;
  __shared__ int32_t s_sel[NSLOT];
  __shared__ uint32_t s_mask[1024 * MW];  // per expert: bit s = slot s chose it (n_expert <= 1024)
  __shared__ int32_t s_cnt[1024], s_off[1024];
  __shared__ int32_t s_wtot[RW];
  __shared__ float s_part[RW], s_sq[RW];
  __shared__ uint32_t s_mine[RW];
  const int tid = threadIdx.x, lane = tid & 63, wk = tid >> 6;
  const int P = a.rparts, LG = RW / P;  // LG logits per workgroup
  const int64_t npair = (int64_t)a.E * a.T;
  {
    // wave -> (token, expert, part of the hidden range); the P parts of a
    // logit are adjacent waves of one workgroup
    const int hp = (int)cdiv(cdiv(a.H, P), 4) * 4;
    const int64_t item = ((int64_t)blockIdx.x * RW + wk) / P;
    const int p = wk % P;
    const int t = (int)(item / a.E), e = (int)(item % a.E);
    // with the RMSNorm: R (x * w) here, the same pass summing x^2; every
    // logit of token t is then scaled by its 1 / rms (one positive factor
    // per token, so it changes no ranking, only the softmax weights)
    float v = 0.0f, sq = 0.0f;
    if (item < npair) {
      const int64_t hb = (int64_t)p * hp, he = hb + hp < a.H ? hb + hp : a.H;
      for (int64_t h0 = hb; h0 < he; h0 += 2048) {
        float4 rv[8], xv[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          const int64_t h = h0 + ((int64_t)j * 64 + lane) * 4;
          rv[j] = h < he ? *(const float4 *)(a.R + (int64_t)e * a.H + h) : float4{0, 0, 0, 0};
          xv[j] = h < he ? *(const float4 *)(a.X + (int64_t)t * a.ldx + h) : float4{0, 0, 0, 0};
        }
        if (a.rms_w) {
#pragma unroll
          for (int j = 0; j < 8; ++j) {
            const int64_t h = h0 + ((int64_t)j * 64 + lane) * 4;
            const float4 w = h < he ? *(const float4 *)(a.rms_w + h) : float4{0, 0, 0, 0};
            sq = __builtin_fmaf(xv[j].x, xv[j].x, sq);
            sq = __builtin_fmaf(xv[j].y, xv[j].y, sq);
            sq = __builtin_fmaf(xv[j].z, xv[j].z, sq);
            sq = __builtin_fmaf(xv[j].w, xv[j].w, sq);
            xv[j].x *= w.x;
            xv[j].y *= w.y;
            xv[j].z *= w.z;
            xv[j].w *= w.w;
          }
        }
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          v = __builtin_fmaf(rv[j].x, xv[j].x, v);
          v = __builtin_fmaf(rv[j].y, xv[j].y, v);
          v = __builtin_fmaf(rv[j].z, xv[j].z, v);
          v = __builtin_fmaf(rv[j].w, xv[j].w, v);
        }
      }
      v = wave_sum(v);
      if (a.rms_w) sq = wave_sum(sq);
    }
    if (lane == 0) {
      s_part[wk] = v;
      s_sq[wk] = sq;
    }
    __syncthreads();
    if (tid < LG) {
      const int64_t it = (int64_t)blockIdx.x * LG + tid;
      if (it < npair) {
        float l = s_part[tid * P];
        for (int q = 1; q < P; ++q) l += s_part[tid * P + q];
        if (a.rms_w) {
          float ss = s_sq[tid * P];
          for (int q = 1; q < P; ++q) ss += s_sq[tid * P + q];
          l *= 1.0f / __builtin_sqrtf(ss / (float)a.H + a.rms_eps);
        }
        st_agent(a.logits + it, l);  // [token][expert]
      }
    }
  }
  // one token: the gate/up workgroups select (no work list needed)
  if (a.sel_local) return;

  // ---- per-token arrival.  This workgroup's logits belong to tokens ta..tb;
  // token t's come from workgroups t E / LG .. ((t + 1) E - 1) / LG, and the
  // last of them to arrive (after its stores are acknowledged) selects it.
  const int64_t i0 = (int64_t)blockIdx.x * LG;
  const int64_t i1 = (i0 + LG < npair ? i0 + LG : npair) - 1;
  const int ta = (int)(i0 / a.E), tb = (int)(i1 / a.E);  // tb - ta < LG <= RW
  __asm__ volatile("s_waitcnt vmcnt(0)" ::: "memory");
  __syncthreads();
  if (tid <= tb - ta) {
    const int t = ta + tid;
    const uint32_t nwg = (uint32_t)(((int64_t)(t + 1) * a.E - 1) / LG - ((int64_t)t * a.E) / LG + 1);
    const uint32_t old = __hip_atomic_fetch_add(a.tcnt + t, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    const bool last = old == nwg - 1;
    if (last) __hip_atomic_store(a.tcnt + t, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    s_mine[tid] = last ? 1u : 0u;
  }
  __syncthreads();
  int nsel = 0;
  for (int j = 0; j <= tb - ta; ++j) nsel += (int)s_mine[j];
  if (nsel == 0) return;

  // ---- top-k and softmax weights of the tokens this workgroup completed,
  // one wave each; published with coherent stores for the work list
  if (wk <= tb - ta && s_mine[wk]) {
    const int t = ta + wk;
    int32_t my_e;
    float my_p;
    select_token<NJ>(a, t, lane, my_e, my_p);
    if (lane < a.k) {
      const int kk = lane;
      st_agent_u32((uint32_t *)a.sel + t * a.k + kk, (uint32_t)my_e);
      a.pw[t * a.k + kk] = my_p;
      if (a.topk_idx) a.topk_idx[t * a.k + kk] = my_e;
      if (a.topk_w) a.topk_w[t * a.k + kk] = my_p;
    }
  }
  // ---- the last selector builds the work list
  __asm__ volatile("s_waitcnt vmcnt(0)" ::: "memory");
  __syncthreads();
  if (tid == 0) {
    const uint32_t old = __hip_atomic_fetch_add(a.rcnt, (uint32_t)nsel, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    const uint32_t last = old + (uint32_t)nsel == (uint32_t)a.T ? 1u : 0u;
    if (last) __hip_atomic_store(a.rcnt, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    flag = last;
  }
  __syncthreads();
  if (!flag) return;

  // Work list: entries of at most NCAP slots of one expert, experts in
  // index order, an expert's slots in slot order.  Each expert's slots as a
  // bit mask (LDS atomic or, the same bits in any order), its count and each
  // slot's position among them by population counts, entry offsets by a scan
  // over the experts.
  const int nslot = a.T * a.k;
  for (int i = tid; i < nslot; i += NTHR) s_sel[i] = (int32_t)ld_agent_u32((const uint32_t *)a.sel + i);
  for (int i = tid; i < a.E * MW; i += NTHR) s_mask[i] = 0u;
  __syncthreads();
  if (tid < nslot) atomicOr(&s_mask[s_sel[tid] * MW + (tid >> 5)], 1u << (tid & 31));
  __syncthreads();
  for (int ee = tid; ee < a.E; ee += NTHR) {
    int c = 0;
#pragma unroll
    for (int w = 0; w < MW; ++w) c += __builtin_popcount(s_mask[ee * MW + w]);
    s_cnt[ee] = c;
  }
  __syncthreads();
  int run = 0;  // entries of the experts before this pass
  for (int base = 0; base < a.E; base += NTHR) {
    const int ee = base + tid;
    const int ne = ee < a.E ? (s_cnt[ee] + NCAP - 1) / NCAP : 0;
    int incl = ne;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
      const int o = __shfl_up(incl, off);
      if (lane >= off) incl += o;
    }
    if (lane == 63) s_wtot[wk] = incl;
    __syncthreads();
    int before = run;
    for (int w = 0; w < wk; ++w) before += s_wtot[w];
    int total = run;
    for (int w = 0; w < RW; ++w) total += s_wtot[w];
    if (ee < a.E) s_off[ee] = before + incl - ne;
    __syncthreads();
    run = total;
  }
  if (tid == 0) *a.nused = (uint32_t)run;
  // each slot: its position among its expert's slots -> (entry, column)
  if (tid < nslot) {
    const int ee = s_sel[tid];
    int pos = 0;
#pragma unroll
    for (int w = 0; w < MW; ++w) {
      const uint32_t m = s_mask[ee * MW + w];
      const int lo = (tid >> 5) > w ? 32 : (tid >> 5) == w ? (tid & 31) : 0;
      pos += __builtin_popcount(lo == 32 ? m : (m & ((1u << lo) - 1u)));
    }
    const int u = s_off[ee] + pos / NCAP, col = pos % NCAP;
    a.used_slot[u * TMAX + col] = tid;
    if (col == 0) {
      const int left = s_cnt[ee] - pos;
      a.used_e[u] = ee;
      a.used_cnt[u] = left < NCAP ? left : NCAP;
    }
  }
}

// --------------------------------------------- 2./3. grouped expert units
// The work-list entry u (or, for u >= nused, the shared expert's entry of
// tokens (u - nused) * NC ...) of a unit: its matrices, rows, and column
// maps (activation column -> token or slot, output column -> slot).
// Returns the column count, 0 when the unit has no entry.
template <bool GATEUP, int NC>
__device__ __forceinline__ int moe_expert(const MoeArgs &a, int u, DotArgs &d, int32_t *s_x, int32_t *s_y,
                                          const int32_t *loc_e = nullptr, const int32_t *loc_slot = nullptr) {
  const int tid = threadIdx.x;
  // every value below is the same in all lanes (read from one address);
  // readfirstlane lets the compiler see that, so the expert's weight
  // ranges are scalar and its loads need no per-lane loop
  const int nused = loc_e ? a.k : __builtin_amdgcn_readfirstlane((int)*a.nused);
  const int nsh = a.SF > 0 ? (a.T + NC - 1) / NC : 0;
  if (u >= nused + nsh) return 0;
  const bool shared = u >= nused;
  int nc;
  if (shared) {
    const int t0 = (u - nused) * NC;
    nc = a.T - t0 < NC ? a.T - t0 : NC;
    if (tid < nc) {
      s_x[tid] = GATEUP ? t0 + tid : a.T * a.k + t0 + tid;
      s_y[tid] = a.T * a.k + t0 + tid;
    }
    if (GATEUP) {
      d.qs0 = a.sgq; d.qs1 = a.suq; d.d0 = a.sgd; d.d1 = a.sud;
    } else {
      d.qs0 = d.qs1 = a.sdq; d.d0 = d.d1 = a.sdd;
    }
  } else {
    // the work-list entry, or (one token, selected locally) the expert of
    // index-order position u and its slot
    const int e = __builtin_amdgcn_readfirstlane(loc_e ? loc_e[u] : a.used_e[u]);
    nc = loc_e ? 1 : __builtin_amdgcn_readfirstlane(a.used_cnt[u]);
    if (tid < nc) {
      const int q = loc_e ? loc_slot[u] : a.used_slot[u * TMAX + tid];
      s_x[tid] = GATEUP ? q / a.k : q;
      s_y[tid] = q;
    }
    if (GATEUP) {
      d.qs0 = a.gq + (int64_t)e * a.gu_qs_stride; d.qs1 = a.uq + (int64_t)e * a.gu_qs_stride;
      d.d0 = a.gd + (int64_t)e * a.gu_d_stride; d.d1 = a.ud + (int64_t)e * a.gu_d_stride;
    } else {
      d.qs0 = d.qs1 = a.dq + (int64_t)e * a.dn_qs_stride;
      d.d0 = d.d1 = a.dd + (int64_t)e * a.dn_d_stride;
    }
  }
  const int64_t f = shared ? a.SF : a.F;  // this expert's ffn width
  d.rows = GATEUP ? f : a.H;
  d.cols = GATEUP ? a.H : f;
  d.NT = (int)(d.rows / 16);
  d.KT = (int)(d.cols / 128);
  d.ncols = nc;
  d.xmap = s_x;
  d.ymap = s_y;
  return nc;
}

template <int QT, int NC, int PF, bool RMSN>
__global__ void __launch_bounds__(MOE_WMAX * 64) moe_gateup_kernel(MoeArgs a) {
  extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
  __shared__ uint32_t flag;
  __shared__ int32_t s_x[TMAX], s_y[TMAX];
  __shared__ int32_t s_le[8], s_ls[8];
  const int sx = a.sw_gu ? 1 : a.S_gu;  // segments across workgroups
  const int per = a.G_gu * sx;
  const int u = blockIdx.x / per, g = (blockIdx.x % per) / sx, s = blockIdx.x % sx;
  if (a.sel_local) {
    // one token: wave 0 selects the experts (the same bits in every
    // workgroup) and lists them in expert index order; workgroup 0 also
    // publishes the selection and the weights
    const int tid = threadIdx.x;
    if (tid < 64) {
      int32_t my_e;
      float my_p;
      if (a.E <= 256) select_token<4>(a, 0, tid, my_e, my_p);
      else select_token<16>(a, 0, tid, my_e, my_p);
      int pos = 0;
      for (int j = 0; j < a.k; ++j) pos += __shfl(my_e, j) < my_e ? 1 : 0;
      if (tid < a.k) {
        s_le[pos] = my_e;
        s_ls[pos] = tid;
        if (blockIdx.x == 0) {
          a.sel[tid] = my_e;
          a.pw[tid] = my_p;
          if (a.topk_idx) a.topk_idx[tid] = my_e;
          if (a.topk_w) a.topk_w[tid] = my_p;
        }
      }
    }
    __syncthreads();
  }
  DotArgs d = {};
  if (!moe_expert<true, NC>(a, u, d, s_x, s_y, a.sel_local ? s_le : nullptr, s_ls)) return;
  d.S = sx;
  d.SW = a.sw_gu ? a.S_gu : 1;
  d.IL = a.il_gu;
  d.G = (int)cdiv(d.NT, a.W_gu);
  if (g >= d.G) return;
  d.X = a.X;
  d.ldx = a.ldx;
  d.xspan = ((int64_t)(a.T - 1) * a.ldx + a.H) * 4;  // every token's column
  d.Y = a.hbuf;
  d.ldy = a.Fmax;
  d.part = a.gpart + (int64_t)u * a.gpart_per;
  d.cnt = a.gcnt + (int64_t)u * a.G_gu;
  d.gamma = a.rms_w;
  d.norm_eps = a.rms_eps;
  __syncthreads();  // the column maps
  float bv = 0.0f;
  int32_t bi = 0;
  dot_unit<QT, NC, 2, EPI_SILU, 1, PF, 0, PH_PLAIN, RMSN>(d, g, s, smem, &flag, bv, bi);
}

template <int QT, int NC, int PF>
__global__ void __launch_bounds__(MOE_WMAX * 64) moe_down_kernel(MoeArgs a) {
  const int NTHR = a.W_dn * 64;
  extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
  __shared__ uint32_t flag;
  __shared__ int32_t s_x[TMAX], s_y[TMAX];
  const int tid = threadIdx.x;
  const int per = a.G_dn * a.S_dn;
  const int u = blockIdx.x / per, g = (blockIdx.x % per) / a.S_dn, s = blockIdx.x % a.S_dn;
  DotArgs d = {};
  if (!moe_expert<false, NC>(a, u, d, s_x, s_y)) return;
  d.S = a.S_dn;
  d.G = a.G_dn;
  d.part = a.dpart + (int64_t)u * a.dpart_per;
  d.cnt = a.dscnt + (int64_t)u * a.G_dn;
  d.X = a.hbuf;
  d.ldx = a.Fmax;
  d.xspan = (int64_t)(a.T * a.k + a.T) * a.Fmax * 4;  // every slot's h
  d.Y = a.zbuf;
  d.ldy = a.H;
  __syncthreads();  // the column maps
  float bv = 0.0f;
  int32_t bi = 0;
  // coherent stores of z (the combine below may run on another XCD); with
  // K segments, only the workgroup that adds them up goes on
  if (!dot_unit<QT, NC, 1, EPI_STORE, 1, PF, 0, PH_PRODUCE>(d, g, s, smem, &flag, bv, bi)) return;

  // ---- weighted combine of this row group, by the last expert to finish
  const uint32_t target = *a.nused + (a.SF > 0 ? (uint32_t)((a.T + NC - 1) / NC) : 0u);
  if (!arrive_last(a.dcnt + g, target, &flag)) return;
  const int64_t r0 = (int64_t)g * a.W_dn * 16;
  const int nr = (int)((a.H - r0) < a.W_dn * 16 ? (a.H - r0) : a.W_dn * 16);
  const __amdgpu_buffer_rsrc_t rz = buf_range(a.zbuf, (uint32_t)((int64_t)(a.T * a.k + a.T) * a.H * 4));
  const __amdgpu_buffer_rsrc_t rpw = buf_range(a.pw, (uint32_t)(a.T * a.k * 4));
  for (int o = tid; o < nr * a.T; o += NTHR) {
    const int t = o / nr, rr = o % nr;
    const int64_t row = r0 + rr;
    // all k (<= 8) slot outputs and weights, and the shared expert's, are
    // loaded before the sum: bounded ranges, offsets past them read zeros
    float z[8], p[8];
#pragma unroll
    for (int kk = 0; kk < 8; ++kk) {
      const uint32_t zo = kk < a.k ? (uint32_t)(((int64_t)(t * a.k + kk) * a.H + row) * 4) : 0xFFFFFFC0u;
      const uint32_t po = kk < a.k ? (uint32_t)((t * a.k + kk) * 4) : 0xFFFFFFC0u;
      z[kk] = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(rz, zo, 0, 16));
      p[kk] = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(rpw, po, 0, 0));
    }
    const uint32_t so = a.SF > 0 ? (uint32_t)(((int64_t)(a.T * a.k + t) * a.H + row) * 4) : 0xFFFFFFC0u;
    const float zs = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(rz, so, 0, 16));
    float *yp = a.Y + (int64_t)t * a.ldy + row;
    const float y0 = *yp;
    float sum = 0.0f;
#pragma unroll
    for (int kk = 0; kk < 8; ++kk)
      if (kk < a.k) sum = __builtin_fmaf(p[kk], z[kk], sum);
    if (a.SF > 0) sum += zs;
    *yp = y0 + sum;
  }
}

// ------------------------------------- 3'. down, token-major (few tokens)
// One workgroup per (token, group of R row tiles of the output), one wave
// per routed slot of the token plus one for the shared expert.  Each wave
// stages its slot's h column in LDS (as the dot unit stages activations:
// hi and lo f16 halves under one power of two per 128 values, so h keeps
// f32 range and 22 significant bits) and streams its expert's R row
// tiles over all of K; the waves' row sums meet in LDS and are combined in
// rank order, sum_k p_k z_k + shared, then added to Y once.  An expert is
// read once per token that routed to it (not once for all of them, as in
// the entry-grouped form), in exchange for no per-slot outputs in memory,
// no cross-workgroup counters and one launch-wide round trip less.
template <int QT, int PF>
__global__ void __launch_bounds__(576) moe_down_tok_kernel(MoeArgs a) {
  constexpr int TB = QTraits<QT>::tile_bytes;
  constexpr int QW = QT == Q4 ? 1 : 2;
  constexpr int RMAX = 4;
  extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
  const int tid = threadIdx.x, lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int nw = a.k + (a.SF > 0 ? 1 : 0);
  const int t = blockIdx.x / a.G_dt, g = blockIdx.x % a.G_dt;
  const int R = a.R_dt;
  const int r = lane & 15, sl = lane >> 4;
  const bool shared = w == a.k;
  const int slot = shared ? a.T * a.k + t : t * a.k + w;
  const int e = shared ? 0 : a.sel[t * a.k + w];
  const int64_t K = shared ? a.SF : a.F;
  const int KT = (int)(K / 128);
  const uint8_t *qs = shared ? a.sdq : a.dq + (int64_t)e * a.dn_qs_stride;
  const uint8_t *ds = shared ? a.sdd : a.dd + (int64_t)e * a.dn_d_stride;

  // this wave's R row tiles, all of K: one bounded range each for the
  // weights and the scales (rows past the matrix: an empty range)
  const int NT = (int)(a.H / 16);
  const int rt0 = g * R;
  const int nrt = NT - rt0 < R ? NT - rt0 : R;
  const __amdgpu_buffer_rsrc_t rq = buf_range(qs + (int64_t)rt0 * KT * TB, (uint32_t)(nrt * KT * TB));
  const __amdgpu_buffer_rsrc_t rd = buf_range(ds + (int64_t)rt0 * KT * TILE_D_BYTES, (uint32_t)(nrt * KT * TILE_D_BYTES));
  const int ntile = R * KT;  // tile n: row tile n / KT, tile column n % KT
  u4 wq[PF][QW];
  u2 wd[PF];
  auto load = [&](int slotp, int n) {
    const uint32_t qo = (uint32_t)n * TB + (uint32_t)lane * 16u;
    wq[slotp][0] = buf_ld16(rq, qo);
    if constexpr (QW == 2) wq[slotp][1] = buf_ld16(rq, qo + 1024u);
    wd[slotp] = buf_ld8(rd, (uint32_t)n * TILE_D_BYTES + (uint32_t)r * 8u);
  };
#pragma unroll
  for (int p = 0; p < PF; ++p) load(p, p);

  // h column of this slot in LDS: hi halves [K], lo halves [K], then the
  // power of two of each tile column of 128.  A tile column is 16 pieces of
  // 8 values, the 16 lanes of one DPP row (K / 8 is a multiple of 16, so
  // every row runs the loop together).
  uint8_t *wbase = smem + (size_t)w * dn_tok_stage_bytes(a.Fmax);
  _Float16 *xh = (_Float16 *)wbase, *xl = xh + a.Fmax;
  float *xsc = (float *)(wbase + (size_t)a.Fmax * 4);
  const float *hcol = a.hbuf + (int64_t)slot * a.Fmax;
  for (int v = lane; v < (int)(K / 8); v += 64) {
    const float4 lo = *(const float4 *)(hcol + v * 8), hi = *(const float4 *)(hcol + v * 8 + 4);
    const float x[8] = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
    float m = 0.0f;
#pragma unroll
    for (int e = 0; e < 8; ++e) m = fmaxf(m, __builtin_fabsf(x[e]));
    m = row16_max(m);
    float up, down;
    tile_pow2(m, up, down);
    h8 H, L;
    split_hl(x, up, H, L);
    *(h8 *)(xh + v * 8) = H;
    *(h8 *)(xl + v * 8) = L;
    if ((v & 15) == 0) xsc[v >> 4] = down;
  }
  __syncthreads();

  const Q4Magic mg = q4_magic();
  float acc[RMAX];
#pragma unroll
  for (int i = 0; i < RMAX; ++i) acc[i] = 0.0f;
  for (int n0 = 0; n0 < ntile; n0 += PF) {
#pragma unroll
    for (int p = 0; p < PF; ++p) {
      const int n = n0 + p;
      if (n < ntile) {
        const int i = n / KT, kt = n % KT;
        float part = 0.0f;
#pragma unroll
        for (int j = 0; j < TILE_BLOCKS; ++j) {
          h2 wv[4];
          if constexpr (QT == Q4) unpack_q4(wq[p][0][j], wv, mg);
          else unpack_q8(wq[p][j >> 1][(j & 1) * 2], wq[p][j >> 1][(j & 1) * 2 + 1], wv);
          const h8 hh = *(const h8 *)(xh + (kt * TILE_BLOCKS + j) * 32 + sl * 8);
          const h8 hl = *(const h8 *)(xl + (kt * TILE_BLOCKS + j) * 32 + sl * 8);
          // w . hi, then w . lo into the same f32 sum (exact f16 products)
          float q = dot2_first(wv[0], lo_pair(hh, 0));
#pragma unroll
          for (int u = 1; u < 4; ++u) q = __builtin_amdgcn_fdot2(wv[u], lo_pair(hh, u), q, false);
#pragma unroll
          for (int u = 0; u < 4; ++u) q = __builtin_amdgcn_fdot2(wv[u], lo_pair(hl, u), q, false);
          part = __builtin_fmaf(scale_of(wd[p], j), q, part);
        }
        const float sc = xsc[kt];
#pragma unroll
        for (int ii = 0; ii < RMAX; ++ii)
          if (ii == i) acc[ii] = __builtin_fmaf(sc, part, acc[ii]);
      }
      load(p, n + PF);
    }
  }

  // row sums (the 4 slices of each row), then the combine through LDS
  float *zs = (float *)(smem + (size_t)nw * dn_tok_stage_bytes(a.Fmax));  // [wave][R * 16]
#pragma unroll
  for (int i = 0; i < RMAX; ++i) {
    float v = acc[i];
    v += __shfl_xor(v, 16);
    v += __shfl_xor(v, 32);
    if (i < R && sl == 0) zs[w * R * 16 + i * 16 + r] = v;
  }
  __syncthreads();
  if (tid < nrt * 16) {
    const int64_t row = (int64_t)rt0 * 16 + tid;
    float sum = 0.0f;
    for (int kk = 0; kk < a.k; ++kk) sum = __builtin_fmaf(a.pw[t * a.k + kk], zs[kk * R * 16 + tid], sum);
    if (a.SF > 0) sum += zs[a.k * R * 16 + tid];
    float *yp = a.Y + (int64_t)t * a.ldy + row;
    *yp = *yp + sum;
  }
}

// ------------------------------------------------------------ host side
static int grant(const void *kern, size_t lds, size_t &granted) {
  if (lds > 163840 - 1024) return QG_EUNSUPPORTED;
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

// LDS of a unit's staged activations: at most ceil(KT / S) tile columns
template <int NC>
static size_t unit_lds(int64_t KT, int S) {
  return dot_stage_bytes(cdiv(KT, S), NC);
}

template <int QT, int NC>
static int launch_moe_t(const MoeCall &c, MoeArgs &a) {
  constexpr int QW = QT == Q4 ? 1 : 2;
  constexpr int PFG = 4 / (2 * QW) < 2 ? 2 : 4 / (2 * QW);
  constexpr int PFD = 4 / QW < 2 ? 2 : 4 / QW;
  clear_hip_error();
  int st = QG_OK;
  const dim3 rgrid((unsigned)cdiv((int64_t)a.E * a.T * a.rparts, RW));
  if (a.E <= 256)
    hipLaunchKernelGGL((moe_router_kernel<NC, 4>), rgrid, dim3(RW * 64), 0, c.stream, a);
  else
    hipLaunchKernelGGL((moe_router_kernel<NC, 16>), rgrid, dim3(RW * 64), 0, c.stream, a);
  if (launch_status() != QG_OK) return QG_EHIP;

  // with the RMSNorm, every unit stages all of K (interleaved segments)
  if (a.rms_w && !(a.il_gu || a.sw_gu)) return QG_EUNSUPPORTED;
  auto kg = a.rms_w ? moe_gateup_kernel<QT, NC, PFG, true> : moe_gateup_kernel<QT, NC, PFG, false>;
  // in-workgroup segments: all of K staged, plus the segment sums; across
  // workgroups, the unit's tile columns (with the norm, also the squares
  // per piece and 1 / rms per column)
  size_t lds_g = a.sw_gu ? unit_lds<NC>(a.H / 128, 1) + (size_t)(a.S_gu - 1) * a.W_gu * 2 * (NC < 4 ? NC : 4) * 64 * 4
                         : unit_lds<NC>(a.H / 128, a.S_gu);
  if (a.rms_w) lds_g += (size_t)NC * (a.H / 128) * TILE_BLOCKS * 4 * 4 + (size_t)NC * 4;
  const int sx = a.sw_gu ? 1 : a.S_gu;
  const int wg_threads = a.W_gu * (a.sw_gu ? a.S_gu : 1) * 64;
  static size_t granted_g[2] = {65536, 65536};  // per kernel: without, with the norm
  st = grant((const void *)kg, lds_g, granted_g[a.rms_w ? 1 : 0]);
  if (st) return st;
  clear_hip_error();
  hipLaunchKernelGGL(kg, dim3((unsigned)((int64_t)(a.Umax + a.nsh) * a.G_gu * sx)), dim3(wg_threads), lds_g,
                     c.stream, a);
  if (launch_status() != QG_OK) return QG_EHIP;

  if (a.dn_tok) {
    auto kt = moe_down_tok_kernel<QT, PFD>;
    const int nw = a.k + (a.SF > 0 ? 1 : 0);
    const size_t lds_t = (size_t)nw * dn_tok_stage_bytes(a.Fmax) + (size_t)nw * a.R_dt * 16 * 4;
    static size_t granted_t = 65536;
    if ((st = grant((const void *)kt, lds_t, granted_t))) return st;
    clear_hip_error();
    hipLaunchKernelGGL(kt, dim3((unsigned)(a.T * a.G_dt)), dim3(nw * 64), lds_t, c.stream, a);
    return launch_status();
  }
  auto kd = moe_down_kernel<QT, NC, PFD>;
  const size_t lds_d = unit_lds<NC>(a.Fmax / 128, a.S_dn);
  static size_t granted_d = 65536;
  if ((st = grant((const void *)kd, lds_d, granted_d))) return st;
  clear_hip_error();
  hipLaunchKernelGGL(kd, dim3((unsigned)((int64_t)(a.Umax + a.nsh) * a.G_dn * a.S_dn)), dim3(a.W_dn * 64), lds_d,
                     c.stream, a);
  return launch_status();
}

template <int QT>
static int launch_moe_q(const MoeCall &c, MoeArgs &a) {
  if (a.T <= 1) return launch_moe_t<QT, 1>(c, a);
  if (a.T <= 2) return launch_moe_t<QT, 2>(c, a);
  return launch_moe_t<QT, 4>(c, a);
}

int launch_moe(const MoeCall &c) {
  const qg_moe *m = c.m;
  const MoeLayout L = moe_layout(m, c.ntok);
  if (c.ws_bytes < L.total) return QG_EWORKSPACE;
  if (L.sync_words > WS_SYNC_WORDS) return QG_EUNSUPPORTED;
  MoeArgs a;
  a.H = m->hidden;
  a.F = m->ffn;
  a.SF = m->sh_ffn;
  a.Fmax = m->sh_ffn > m->ffn ? m->sh_ffn : m->ffn;
  a.E = m->n_expert;
  a.k = m->top_k;
  a.norm = m->normalize_topk ? 1 : 0;
  a.rms_w = m->norm_weight;
  a.rms_eps = m->norm_eps;
  a.T = c.ntok;
  a.Umax = (int)L.umax;
  // enough router waves to spread the router matrix over the device, each
  // part at least one float4 per lane
  a.rparts = 1;
  while (a.rparts < RW && (int64_t)a.E * a.T * a.rparts < 2048 && a.H / (2 * a.rparts) >= 256) a.rparts *= 2;
  a.R = m->router;
  a.gq = (const uint8_t *)m->gate_qs; a.uq = (const uint8_t *)m->up_qs; a.dq = (const uint8_t *)m->down_qs;
  a.gd = (const uint8_t *)m->gate_d; a.ud = (const uint8_t *)m->up_d; a.dd = (const uint8_t *)m->down_d;
  a.sgq = (const uint8_t *)m->sh_gate_qs; a.suq = (const uint8_t *)m->sh_up_qs; a.sdq = (const uint8_t *)m->sh_down_qs;
  a.sgd = (const uint8_t *)m->sh_gate_d; a.sud = (const uint8_t *)m->sh_up_d; a.sdd = (const uint8_t *)m->sh_down_d;
  const int64_t tb = m->qtype == QG_Q4_0 ? 1024 : 2048;
  const int64_t gu_tiles = (a.F / 16) * (a.H / 128);
  const int64_t dn_tiles = (a.H / 16) * (a.F / 128);
  a.gu_qs_stride = gu_tiles * tb;
  a.gu_d_stride = gu_tiles * 128;
  a.dn_qs_stride = dn_tiles * tb;
  a.dn_d_stride = dn_tiles * 128;
  a.X = c.X;
  a.ldx = c.ldx;
  a.Y = c.Y;
  a.ldy = c.ldy;
  a.topk_idx = c.topk_idx;
  a.topk_w = c.topk_w;
  uint8_t *ws = (uint8_t *)c.ws;
  uint32_t *w32 = (uint32_t *)ws;
  a.rcnt = w32 + L.rcnt_w;
  a.tcnt = a.rcnt + 1;
  a.dcnt = w32 + L.dcnt_w;
  a.gcnt = w32 + L.gcnt_w;
  a.nused = (uint32_t *)(ws + L.nused);
  a.logits = (float *)(ws + L.logits);
  a.sel = (int32_t *)(ws + L.sel);
  a.pw = (float *)(ws + L.pw);
  a.used_e = (int32_t *)(ws + L.used_e);
  a.used_cnt = (int32_t *)(ws + L.used_cnt);
  a.used_slot = (int32_t *)(ws + L.used_slot);
  a.hbuf = (float *)(ws + L.hbuf);
  a.zbuf = (float *)(ws + L.zbuf);
  a.gpart = (float *)(ws + L.gpart);
  a.S_gu = L.S_gu;
  a.G_gu = L.G_gu;
  a.G_dn = L.G_dn;
  a.gpart_per = L.gpart_per;
  a.S_dn = L.S_dn;
  a.dpart = (float *)(ws + L.dpart);
  a.dpart_per = L.dpart_per;
  a.dscnt = w32 + L.dscnt_w;
  a.W_gu = L.W_gu;
  a.W_dn = L.W_dn;
  a.sw_gu = L.sw_gu;
  a.dn_tok = L.dn_tok;
  a.sel_local = c.ntok == 1 && L.dn_tok;
  a.il_gu = dot_interleaved(a.H) ? 1 : 0;
  a.R_dt = L.R_dt;
  a.G_dt = (int)cdiv(a.H / 16, L.R_dt);
  if (a.R_dt < 1 || a.R_dt > 4) return QG_EUNSUPPORTED;
  if (a.W_gu < 1 || a.W_dn < 1 || a.W_dn > MOE_WMAX || a.W_gu * (a.sw_gu ? a.S_gu : 1) > MOE_WMAX)
    return QG_EUNSUPPORTED;
  a.nsh = L.nsh;
  if (m->qtype == QG_Q4_0) return launch_moe_q<Q4>(c, a);
  return launch_moe_q<Q8>(c, a);
}

}  // namespace qg
