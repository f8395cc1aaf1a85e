// MoE FFN on gfx950: router, top-k, grouped expert gate/up + SiLU, grouped
// expert down and the weighted combine, in three stream-ordered launches
// with no host readback ("Engine and kernels", Kernel families: router,
// top-k, expert gate/up and down and the weighted combine all on the GPU;
// the MoE model has 256 experts, 8 active per token, plus a shared expert).
// Experts are stacked by role ("A 235B model in a browser window": all gate
// matrices in one tensor, all up in a second, all down in a third).
//
//  1. router: f32 logits (f32 operands, f32 FMA), then the last workgroup
//     picks the top k per token (value descending, index ascending), the
//     softmax weights, and a work list of the distinct experts in index
//     order, each with its routed slots (slot = token * k + rank).
//  2. gate/up: one workgroup per (listed expert, row group) reads that
//     expert's gate and up tiles once for all of its slots and writes
//     h = silu(g) * u per slot.
//  3. down: one workgroup per (listed expert, row group) writes z = D h per
//     slot; the last workgroup to finish a row group forms, per token,
//     sum_k p_k z_k in rank order, adds the shared expert, and adds the
//     total to Y once.
// Workgroups beyond the listed experts exit at once (the grid is the worst
// case, the list is on the device).
#include "common.h"
#include "internal.h"
#include "qgemm.h"

namespace qg {

constexpr int MW = 4;              // waves per workgroup
constexpr int MTHR = MW * 64;
constexpr int EPW = 4;             // router experts per wave
constexpr int TMAX = 16;           // tokens per call
constexpr int RT_GU = 1;           // row tiles per gate/up workgroup
constexpr int RT_DN = 2;           // row tiles per down workgroup

struct MoeArgs {
  int64_t H, F, SF, Fmax;
  int E, k, norm, T, Umax;
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
  uint32_t *rcnt, *dcnt, *nused;
  float *logits, *pw, *hbuf, *zbuf;
  int32_t *sel, *used_e, *used_cnt, *used_slot;
  int gu_groups, sh_gu_units, dn_groups, sh_dn_units;
};

static size_t a256(size_t v) { return (v + 255) & ~size_t(255); }

struct MoeLayout {
  size_t rcnt, dcnt, nused, logits, sel, pw, used_e, used_cnt, used_slot, hbuf, zbuf, total;
};

static MoeLayout moe_layout(const qg_moe *m, int T) {
  MoeLayout L;
  const int64_t Fmax = m->sh_ffn > m->ffn ? m->sh_ffn : m->ffn;
  const int64_t umax = (int64_t)m->n_expert < (int64_t)T * m->top_k ? m->n_expert : (int64_t)T * m->top_k;
  const int64_t slots = (int64_t)T * m->top_k + T;
  // counters (in the shared counter words): the router's, then one per
  // down-projection row group; data after them
  L.rcnt = 0;
  L.dcnt = 4;
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
  L.total = o;
  return L;
}

size_t moe_ws_bytes(const qg_moe *m, int ntok) { return moe_layout(m, ntok).total; }

// ------------------------------------------------------------ 1. router
template <int NTC>
__global__ void __launch_bounds__(MTHR) moe_router_kernel(MoeArgs a) {
  __shared__ uint32_t flag;
  __shared__ int32_t s_sel[TMAX * 8];
  __shared__ int32_t s_cnt[MTHR];
  const int tid = threadIdx.x, lane = tid & 63, wk = tid >> 6;
  const int e0 = (blockIdx.x * MW + wk) * EPW;
  float acc[EPW][NTC];
#pragma unroll
  for (int i = 0; i < EPW; ++i)
#pragma unroll
    for (int t = 0; t < NTC; ++t) acc[i][t] = 0.0f;

  for (int64_t h = lane * 4; h < a.H; h += 256) {
    float4 rv[EPW];
#pragma unroll
    for (int i = 0; i < EPW; ++i)
      rv[i] = (e0 + i < a.E) ? *(const float4 *)(a.R + (int64_t)(e0 + i) * a.H + h) : float4{0, 0, 0, 0};
#pragma unroll
    for (int t = 0; t < NTC; ++t) {
      if (t < a.T) {
        const float4 xv = *(const float4 *)(a.X + (int64_t)t * a.ldx + h);
#pragma unroll
        for (int i = 0; i < EPW; ++i) {
          float v = acc[i][t];
          v = __builtin_fmaf(rv[i].x, xv.x, v);
          v = __builtin_fmaf(rv[i].y, xv.y, v);
          v = __builtin_fmaf(rv[i].z, xv.z, v);
          v = __builtin_fmaf(rv[i].w, xv.w, v);
          acc[i][t] = v;
        }
      }
    }
  }
#pragma unroll
  for (int i = 0; i < EPW; ++i)
#pragma unroll
    for (int t = 0; t < NTC; ++t) {
      if (t < a.T) {
        float v = acc[i][t];
#pragma unroll
        for (int off = 32; off >= 1; off >>= 1) v += __shfl_xor(v, off);
        if (lane == 0 && e0 + i < a.E) st_agent(a.logits + (int64_t)t * a.E + e0 + i, v);
      }
    }
  if (!arrive_last(a.rcnt, gridDim.x, &flag)) return;

  // ---- top-k and softmax weights, one wave per token
  for (int t = wk; t < a.T; t += MW) {
    float lv[16];
#pragma unroll
    for (int j = 0; j < 16; ++j) {
      const int e = lane + 64 * j;
      lv[j] = e < a.E ? ld_agent(a.logits + (int64_t)t * a.E + e) : 0.0f;
    }
    uint32_t taken = 0;
    float selv[8];
    int32_t seli[8];
    for (int kk = 0; kk < a.k; ++kk) {
      float bv = __builtin_nanf("");
      int32_t bi = 0x7fffffff;
#pragma unroll
      for (int j = 0; j < 16; ++j) {
        const int e = lane + 64 * j;
        if (e < a.E && !((taken >> j) & 1u) && ranks_before(lv[j], e, bv, bi)) { bv = lv[j]; bi = e; }
      }
#pragma unroll
      for (int off = 32; off >= 1; off >>= 1) {
        const float ov = __shfl_xor(bv, off);
        const int32_t oi = __shfl_xor(bi, off);
        if (ranks_before(ov, oi, bv, bi)) { bv = ov; bi = oi; }
      }
      if ((bi & 63) == lane) taken |= 1u << (bi >> 6);
      selv[kk] = bv;
      seli[kk] = bi;
    }
    const float mx = selv[0];
    float sum = 0.0f;
    if (a.norm) {
      for (int kk = 0; kk < a.k; ++kk) sum += expf(selv[kk] - mx);
    } else {
      float part = 0.0f;
#pragma unroll
      for (int j = 0; j < 16; ++j)
        if (lane + 64 * j < a.E) part += expf(lv[j] - mx);
#pragma unroll
      for (int off = 32; off >= 1; off >>= 1) part += __shfl_xor(part, off);
      sum = part;
    }
    if (lane == 0) {
      for (int kk = 0; kk < a.k; ++kk) {
        const float p = expf(selv[kk] - mx) / sum;
        a.sel[t * a.k + kk] = seli[kk];
        a.pw[t * a.k + kk] = p;
        s_sel[t * a.k + kk] = seli[kk];
        if (a.topk_idx) a.topk_idx[t * a.k + kk] = seli[kk];
        if (a.topk_w) a.topk_w[t * a.k + kk] = p;
      }
    }
  }
  __syncthreads();

  // ---- work list: used experts in index order, each with its slots in order
  const int nslot = a.T * a.k;
  const int ept = (a.E + MTHR - 1) / MTHR;
  const int e_lo = tid * ept;
  const int e_hi = (e_lo + ept < a.E) ? e_lo + ept : a.E;
  int mine = 0;
  for (int e = e_lo; e < e_hi; ++e) {
    bool used = false;
    for (int q = 0; q < nslot; ++q) used |= (s_sel[q] == e);
    mine += used ? 1 : 0;
  }
  s_cnt[tid] = mine;
  __syncthreads();
  if (tid == 0) {
    int run = 0;
    for (int i = 0; i < MTHR; ++i) { const int c = s_cnt[i]; s_cnt[i] = run; run += c; }
    *a.nused = (uint32_t)run;
  }
  __syncthreads();
  int u = s_cnt[tid];
  for (int e = e_lo; e < e_hi; ++e) {
    int c = 0;
    for (int q = 0; q < nslot; ++q)
      if (s_sel[q] == e) a.used_slot[u * TMAX + c++] = q;
    if (c) { a.used_e[u] = e; a.used_cnt[u] = c; ++u; }
  }
}

// ------------------------------------------------- 2./3. grouped experts
// NMAT = 2: gate/up + SiLU into hbuf.  NMAT = 1: down into zbuf + combine.
template <int QT, int NCM, int NMAT, int RT>
__global__ void __launch_bounds__(MTHR) moe_expert_kernel(MoeArgs a) {
  extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
  __shared__ uint32_t flag;
  __shared__ int32_t s_slot[TMAX];
  constexpr int TB = QTraits<QT>::tile_bytes;
  constexpr int QW = (QT == Q4) ? 1 : 2;
  const int tid = threadIdx.x, lane = tid & 63, wk = tid >> 6;

  const int unit = blockIdx.x;
  const int sh_units = NMAT == 2 ? a.sh_gu_units : a.sh_dn_units;
  const int groups = NMAT == 2 ? a.gu_groups : a.dn_groups;
  const bool shared = unit < sh_units;
  int nc, rg;
  const uint8_t *q0, *q1, *d0, *d1;
  int64_t K;
  if (shared) {
    rg = unit;
    nc = a.T;
    if (NMAT == 2) { q0 = a.sgq; q1 = a.suq; d0 = a.sgd; d1 = a.sud; K = a.H; }
    else { q0 = q1 = a.sdq; d0 = d1 = a.sdd; K = a.SF; }
    if (tid < nc) s_slot[tid] = a.T * a.k + tid;
  } else {
    const int uu = (unit - sh_units) / groups;
    rg = (unit - sh_units) % groups;
    if (uu >= (int)*a.nused) return;
    const int e = a.used_e[uu];
    nc = a.used_cnt[uu];
    if (NMAT == 2) {
      q0 = a.gq + (int64_t)e * a.gu_qs_stride; q1 = a.uq + (int64_t)e * a.gu_qs_stride;
      d0 = a.gd + (int64_t)e * a.gu_d_stride; d1 = a.ud + (int64_t)e * a.gu_d_stride;
      K = a.H;
    } else {
      q0 = q1 = a.dq + (int64_t)e * a.dn_qs_stride;
      d0 = d1 = a.dd + (int64_t)e * a.dn_d_stride;
      K = a.F;
    }
    if (tid < nc) s_slot[tid] = a.used_slot[uu * TMAX + tid];
  }
  const int64_t rows = NMAT == 2 ? (shared ? a.SF : a.F) : a.H;
  const int NTr = (int)(rows / 16);
  const int KT = (int)(K / 128);
  const int64_t rt_base = (int64_t)rg * RT;
  if (rt_base >= NTr) return;
  __syncthreads();

  // ---- stage the input columns (x of each routed token, or h of each slot)
  _Float16 *xs = (_Float16 *)smem;
  float *red = (float *)smem;
  {
    const int nvec = KT * 4 * nc * 4;
    for (int v = tid; v < nvec; v += MTHR) {
      const int q = v & 3, c = (v >> 2) % nc, bl = (v >> 2) / nc;
      const int64_t kk = (int64_t)bl * 32 + q * 8;
      const int slot = s_slot[c];
      const float *src = NMAT == 2 ? a.X + (int64_t)(shared ? c : slot / a.k) * a.ldx
                                   : a.hbuf + (int64_t)slot * a.Fmax;
      const float4 *p = (const float4 *)(src + kk);
      *(h8 *)(xs + (size_t)v * 8) = cvt8(p[0], p[1]);
    }
  }
  __syncthreads();

  const int r = lane & 15, sl = lane >> 4;
  float acc[NMAT][RT][NCM];
#pragma unroll
  for (int m = 0; m < NMAT; ++m)
#pragma unroll
    for (int t = 0; t < RT; ++t)
#pragma unroll
      for (int c = 0; c < NCM; ++c) acc[m][t][c] = 0.0f;

  const Q4Magic mg = q4_magic();
  for (int kt = wk; kt < KT; kt += MW) {
    u4 wq[NMAT][RT][QW];
    u2 wdd[NMAT][RT];
#pragma unroll
    for (int m = 0; m < NMAT; ++m)
#pragma unroll
      for (int t = 0; t < RT; ++t) {
        const int64_t tile = (rt_base + t) * KT + kt;
        const uint8_t *tp = (m ? q1 : q0) + tile * TB + lane * 16;
        wq[m][t][0] = ld_stream(tp);
        if constexpr (QW == 2) wq[m][t][QW - 1] = ld_stream(tp + 1024);
        wdd[m][t] = ld_stream2((m ? d1 : d0) + tile * TILE_D_BYTES + r * 8);
      }
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      h2 xv[NCM][4];
#pragma unroll
      for (int c = 0; c < NCM; ++c) {
        if (c < nc) {
          const h8 xx = *(const h8 *)(xs + ((size_t)(kt * 4 + j) * nc + c) * 32 + sl * 8);
#pragma unroll
          for (int p = 0; p < 4; ++p) xv[c][p] = lo_pair(xx, p);
        }
      }
#pragma unroll
      for (int m = 0; m < NMAT; ++m)
#pragma unroll
        for (int t = 0; t < RT; ++t) {
          h2 w[4];
          if constexpr (QT == Q4) unpack_q4(wq[m][t][0][j], w, mg);
          else unpack_q8(wq[m][t][j >> 1][(j & 1) * 2], wq[m][t][j >> 1][(j & 1) * 2 + 1], w);
          const float dj = scale_of(wdd[m][t], j);
#pragma unroll
          for (int c = 0; c < NCM; ++c) {
            if (c < nc) {
              float p = dot2_first(w[0], xv[c][0]);
              p = __builtin_amdgcn_fdot2(w[1], xv[c][1], p, false);
              p = __builtin_amdgcn_fdot2(w[2], xv[c][2], p, false);
              p = __builtin_amdgcn_fdot2(w[3], xv[c][3], p, false);
              acc[m][t][c] = __builtin_fmaf(dj, p, acc[m][t][c]);
            }
          }
        }
    }
  }

  __syncthreads();
#pragma unroll
  for (int m = 0; m < NMAT; ++m)
#pragma unroll
    for (int t = 0; t < RT; ++t)
#pragma unroll
      for (int c = 0; c < NCM; ++c) {
        if (c < nc) {
          float v = acc[m][t][c];
          v += __shfl_xor(v, 16);
          v += __shfl_xor(v, 32);
          if (sl == 0) red[(((wk * NMAT + m) * RT + t) * 16 + r) * nc + c] = v;
        }
      }
  __syncthreads();

  const int nout = RT * 16 * nc;
  for (int o = tid; o < nout; o += MTHR) {
    const int c = o % nc, rr = (o / nc) % 16, t = o / (16 * nc);
    float v[NMAT];
#pragma unroll
    for (int m = 0; m < NMAT; ++m) {
      float x = red[((m * RT + t) * 16 + rr) * nc + c];
#pragma unroll
      for (int w = 1; w < MW; ++w) x += red[(((w * NMAT + m) * RT + t) * 16 + rr) * nc + c];
      v[m] = x;
    }
    const int64_t row = (rt_base + t) * 16 + rr;
    const int slot = s_slot[c];
    if constexpr (NMAT == 2) {
      const float gg = v[0];
      a.hbuf[(int64_t)slot * a.Fmax + row] = gg / (1.0f + expf(-gg)) * v[1];
    } else {
      st_agent(a.zbuf + (int64_t)slot * a.H + row, v[0]);
    }
  }

  if constexpr (NMAT == 1) {
    // ---- weighted combine of this row group, by the last expert to finish
    const uint32_t target = *a.nused + (a.SF > 0 ? 1u : 0u);
    if (!arrive_last(a.dcnt + rg, target, &flag)) return;
    const int n = RT * 16 * a.T;
    for (int o = tid; o < n; o += MTHR) {
      const int t = o / (RT * 16), rr = o % (RT * 16);
      const int64_t row = rt_base * 16 + rr;
      float sum = 0.0f;
      for (int kk = 0; kk < a.k; ++kk)
        sum = __builtin_fmaf(a.pw[t * a.k + kk], ld_agent(a.zbuf + (int64_t)(t * a.k + kk) * a.H + row), sum);
      if (a.SF > 0) sum += ld_agent(a.zbuf + (int64_t)(a.T * a.k + t) * a.H + row);
      float *yp = a.Y + (int64_t)t * a.ldy + row;
      *yp = *yp + sum;
    }
  }
}

// ------------------------------------------------------------ host side
template <int QT, int NCM>
static int launch_moe_t(const MoeCall &c, MoeArgs &a) {
  const int ntc = NCM;
  const unsigned rgrid = (unsigned)((a.E + MW * EPW - 1) / (MW * EPW));
  clear_hip_error();
  hipLaunchKernelGGL(moe_router_kernel<ntc>, dim3(rgrid), dim3(MTHR), 0, c.stream, a);
  if (launch_status() != QG_OK) return QG_EHIP;

  const int T = a.T;
  size_t x_gu = (size_t)(a.H / 128) * 4 * T * 64;
  size_t r_gu = (size_t)MW * 2 * RT_GU * 16 * T * 4;
  size_t lds_gu = x_gu > r_gu ? x_gu : r_gu;
  const unsigned ggrid = (unsigned)(a.sh_gu_units + (int64_t)a.Umax * a.gu_groups);
  auto kg = moe_expert_kernel<QT, NCM, 2, RT_GU>;
  if (lds_gu > 163840 - 1024) return QG_EUNSUPPORTED;
  if (lds_gu > 65536) {
    static size_t granted = 65536;
    if (lds_gu > granted) {
      const hipError_t e = hipFuncSetAttribute((const void *)kg, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds_gu);
      if (e != hipSuccess) {
        record_hip_error(e);
        return QG_EHIP;
      }
      granted = lds_gu;
    }
  }
  clear_hip_error();
  hipLaunchKernelGGL(kg, dim3(ggrid), dim3(MTHR), lds_gu, c.stream, a);
  if (launch_status() != QG_OK) return QG_EHIP;

  size_t x_dn = (size_t)(a.Fmax / 128) * 4 * T * 64;
  size_t r_dn = (size_t)MW * 1 * RT_DN * 16 * T * 4;
  size_t lds_dn = x_dn > r_dn ? x_dn : r_dn;
  const unsigned dgrid = (unsigned)(a.sh_dn_units + (int64_t)a.Umax * a.dn_groups);
  auto kd = moe_expert_kernel<QT, NCM, 1, RT_DN>;
  if (lds_dn > 163840 - 1024) return QG_EUNSUPPORTED;
  if (lds_dn > 65536) {
    static size_t granted = 65536;
    if (lds_dn > granted) {
      const hipError_t e = hipFuncSetAttribute((const void *)kd, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds_dn);
      if (e != hipSuccess) {
        record_hip_error(e);
        return QG_EHIP;
      }
      granted = lds_dn;
    }
  }
  clear_hip_error();
  hipLaunchKernelGGL(kd, dim3(dgrid), dim3(MTHR), lds_dn, c.stream, a);
  return launch_status();
}

template <int QT>
static int launch_moe_q(const MoeCall &c, MoeArgs &a) {
  if (a.T <= 1) return launch_moe_t<QT, 1>(c, a);
  if (a.T <= 2) return launch_moe_t<QT, 2>(c, a);
  if (a.T <= 4) return launch_moe_t<QT, 4>(c, a);
  if (a.T <= 8) return launch_moe_t<QT, 8>(c, a);
  return launch_moe_t<QT, 16>(c, a);
}

int launch_moe(const MoeCall &c) {
  const qg_moe *m = c.m;
  const MoeLayout L = moe_layout(m, c.ntok);
  if (c.ws_bytes < L.total) return QG_EWORKSPACE;
  MoeArgs a;
  a.H = m->hidden;
  a.F = m->ffn;
  a.SF = m->sh_ffn;
  a.Fmax = m->sh_ffn > m->ffn ? m->sh_ffn : m->ffn;
  a.E = m->n_expert;
  a.k = m->top_k;
  a.norm = m->normalize_topk ? 1 : 0;
  a.T = c.ntok;
  a.Umax = (int)((int64_t)a.E < (int64_t)a.T * a.k ? a.E : a.T * a.k);
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
  a.rcnt = (uint32_t *)(ws + L.rcnt);
  a.dcnt = (uint32_t *)(ws + L.dcnt);
  a.nused = (uint32_t *)(ws + L.nused);
  a.logits = (float *)(ws + L.logits);
  a.sel = (int32_t *)(ws + L.sel);
  a.pw = (float *)(ws + L.pw);
  a.used_e = (int32_t *)(ws + L.used_e);
  a.used_cnt = (int32_t *)(ws + L.used_cnt);
  a.used_slot = (int32_t *)(ws + L.used_slot);
  a.hbuf = (float *)(ws + L.hbuf);
  a.zbuf = (float *)(ws + L.zbuf);
  a.gu_groups = (int)((a.F / 16 + RT_GU - 1) / RT_GU);
  a.sh_gu_units = a.SF > 0 ? (int)((a.SF / 16 + RT_GU - 1) / RT_GU) : 0;
  a.dn_groups = (int)((a.H / 16 + RT_DN - 1) / RT_DN);
  a.sh_dn_units = a.SF > 0 ? a.dn_groups : 0;
  if (m->qtype == QG_Q4_0) return launch_moe_q<Q4>(c, a);
  return launch_moe_q<Q8>(c, a);
}

}  // namespace qg
