// Load-time requantisation of Q4_1 / Q5_0 / Q5_1 and Q4_K / Q5_K / Q6_K
// blocks to Q8_0.
//
// What is computed ("Engine and kernels", What it runs: the few Q4_1 / Q5_0
// / K-quant tensors of the public MoE file are requantized to Q8_0 on the
// way to the GPU; "Architecture", where the weights live: converted once,
// the result kept).  The source layouts are the public GGUF ones:
//   Q4_1 = f16 d, f16 m, 16 nibble bytes, value w * d + m;
//   Q5_0 = f16 d, 32 high bits, 16 nibble bytes, value (w - 16) * d;
//   Q5_1 = f16 d, f16 m, high bits, nibbles, value w * d + m (weight j: low
//   nibble of byte j plus high bit j; weight j + 16: high nibble plus bit
//   j + 16);
//   Q4_K (144 B per 256 values) = f16 d, f16 dmin, 12 bytes of 6-bit scales
//   and mins for eight sub-blocks of 32, 128 nibble bytes (bytes 32 c ..
//   32 c + 31 hold sub-block 2 c in low and 2 c + 1 in high nibbles), value
//   (d * sc) * w - dmin * m;
//   Q5_K (176 B) = Q4_K plus 32 bytes whose bit j is the fifth bit of the
//   weights of sub-block j;
//   Q6_K (210 B) = 128 bytes of low nibbles, 64 bytes of 2-bit tops, 16
//   int8 scales (one per 16 values), f16 d; value (d * sc) * (w - 32).
// Every run of 32 values is requantised to one Q8_0 block by the usual
// rule, in float32 steps each rounded once: d = max|v| / 127, q = v * (1 /
// d) rounded half away from zero, d stored as binary16.  The output is
// canonical Q8_0 blocks, which qg_repack then tiles; the conversion runs on
// the GPU, so the source bytes are uploaded once, smaller than the Q8_0
// result.
#include "common.h"
#include "internal.h"
#include "qgemm.h"

namespace qg {

constexpr int SRC_Q4_1 = 3, SRC_Q5_0 = 6, SRC_Q5_1 = 7, SRC_Q4_K = 12, SRC_Q5_K = 13, SRC_Q6_K = 14;

// 16-bit words per source block and 32-value runs (output blocks) per source
// block.  Every field of every format starts at an even byte, so one reader
// of 16-bit words serves LDS and global memory at any 2-byte alignment.
template <int SRC>
struct Src {
  static constexpr int WORDS = SRC == SRC_Q4_1   ? 10
                               : SRC == SRC_Q5_0 ? 11
                               : SRC == SRC_Q5_1 ? 12
                               : SRC == SRC_Q4_K ? 72
                               : SRC == SRC_Q5_K ? 88
                                                 : 105;
  static constexpr int RUNS = SRC >= SRC_Q4_K ? 8 : 1;
};

__device__ __forceinline__ float f16_bits(uint32_t b) {
  return (float)__builtin_bit_cast(_Float16, (uint16_t)b);
}

// Rounds half away from zero for |x| < 2^23: x plus the largest float below
// one half, carrying x's sign, truncated toward zero.  The sum reaches the
// next integer away from zero exactly when |x - trunc(x)| >= 1/2 (a sum that
// is a tie rounds to the even neighbour, which is then that integer), so
// this equals roundf(x) there; the host tests check it for every float of
// magnitude up to 128, the range of the quotients here.  Three instructions
// instead of roundf's six before the conversion.
// x must be a rounded float: contraction stays off here and where x is
// formed, or a product feeding x would be fused into the sum.
__device__ __forceinline__ int round_half_away(float x) {
#pragma clang fp contract(off)
  return (int)(x + __builtin_copysignf(0x1.fffffep-2f, x));
}

// The Q8_0 block of 32 float32 values, written as 17 16-bit words.
template <class Out>
__device__ __forceinline__ void store_q8_0(const float (&v)[32], Out *out) {
  float amax = 0.0f;
#pragma unroll
  for (int j = 0; j < 32; ++j) amax = __builtin_fmaxf(amax, __builtin_fabsf(v[j]));
  const float dq = amax / 127.0f;
  const float id = dq != 0.0f ? 1.0f / dq : 0.0f;
  out[0] = __builtin_bit_cast(uint16_t, (_Float16)dq);
  {
#pragma clang fp contract(off)
#pragma unroll
    for (int j = 0; j < 32; j += 2) {
      const int q0 = round_half_away(v[j] * id), q1 = round_half_away(v[j + 1] * id);
      out[1 + j / 2] = (uint16_t)((uint32_t)(q0 & 0xFF) | ((uint32_t)(q1 & 0xFF) << 8));
    }
  }
}

// Values of one Q4_1 / Q5_0 / Q5_1 block held as 16-bit words at `in`.
template <int SRC, class In>
__device__ __forceinline__ void legacy_values(const In *in, float (&v)[32]) {
  constexpr int SW = Src<SRC>::WORDS;
  uint16_t wsrc[SW];
#pragma unroll
  for (int i = 0; i < SW; ++i) wsrc[i] = in[i];
  const float d = f16_bits(wsrc[0]);
  const float m = SRC == SRC_Q5_0 ? 0.0f : f16_bits(wsrc[1]);
  const uint32_t qh = SRC == SRC_Q4_1 ? 0u
                      : SRC == SRC_Q5_0 ? ((uint32_t)wsrc[1] | ((uint32_t)wsrc[2] << 16))
                                        : ((uint32_t)wsrc[2] | ((uint32_t)wsrc[3] << 16));
  constexpr int QS = SRC == SRC_Q4_1 ? 2 : SRC == SRC_Q5_0 ? 3 : 4;  // first nibble word
  // Q5_0's offset folded into the product: (w - 16) d = w d - 16 d, both
  // terms exact in float32.
  const float m0 = SRC == SRC_Q5_0 ? -16.0f * d : m;
#pragma unroll
  for (int g = 0; g < 4; ++g) {  // weights 4g .. 4g + 3 and 16 + 4g .. 16 + 4g + 3
    const uint32_t qs = (uint32_t)wsrc[QS + 2 * g] | ((uint32_t)wsrc[QS + 2 * g + 1] << 16);
    uint32_t lo = qs & 0x0F0F0F0Fu, hi = (qs >> 4) & 0x0F0F0F0Fu;
    if (SRC != SRC_Q4_1) {
      // Four high bits to bit 4 of four bytes: b * 0x00204081 = b | b << 7 |
      // b << 14 | b << 21 holds bit i of the nibble b at bit 8 i (the copies
      // do not overlap).  Both factors fit 24 bits; the compiler would use a
      // quarter-rate 32-bit multiply, so the full-rate 24-bit one is named.
      auto spread = [](uint32_t b) {
        uint32_t r;
        __asm__("v_mul_u32_u24 %0, %1, %2" : "=v"(r) : "v"(b), "v"(0x00204081u));
        return (r & 0x01010101u) << 4;
      };
      lo |= spread((qh >> (4 * g)) & 15u);
      hi |= spread((qh >> (16 + 4 * g)) & 15u);
    }
    {
      // w d is exact in float32 (at most 5 by 11 significant bits), so a
      // fused w d + m rounds the same single sum.
#pragma clang fp contract(fast)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        v[4 * g + i] = (float)((lo >> (8 * i)) & 0xFFu) * d + m0;
        v[16 + 4 * g + i] = (float)((hi >> (8 * i)) & 0xFFu) * d + m0;
      }
    }
  }
}

// Values of run r (0..7, values 32 r .. 32 r + 31) of a K-quant super-block
// held as 16-bit words at `w`.
template <int SRC, class In>
__device__ __forceinline__ void kquant_values(const In *w, int r, float (&v)[32]) {
  if constexpr (SRC == SRC_Q6_K) {
    // Run r lies in half n = r / 4 as its quarter k = r % 4: low nibbles
    // (k < 2) or high nibbles (k >= 2) of bytes 64 n + 32 (k % 2) + l, top
    // bits 2k, 2k + 1 of bytes 128 + 32 n + l, scales 2 r (values 0..15)
    // and 2 r + 1 (16..31).
    const int n = r >> 2, k = r & 3;
    const float d = f16_bits(w[104]);
    const uint32_t scw = w[96 + r];
    // d * sc is exact (11 by 8 significant bits); its product with w - 32
    // is the one rounding of each value.
    const float ds0 = d * (float)(int8_t)(scw & 0xFFu), ds1 = d * (float)(int8_t)(scw >> 8);
    const In *ql = w + 32 * n + 16 * (k & 1);
    const In *qh = w + 64 + 16 * n;
    const int lsh = k >= 2 ? 4 : 0, hsh = 2 * k;
    // four values per 32-bit word, one byte each (low 4 bits from ql, the
    // top 2 from qh), then byte conversions; ds * (w - 32) as the fused ds *
    // w - 32 ds (32 ds is exact), one rounding of the same exact value
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const uint32_t a = (uint32_t)ql[2 * i] | ((uint32_t)ql[2 * i + 1] << 16);
      const uint32_t b = (uint32_t)qh[2 * i] | ((uint32_t)qh[2 * i + 1] << 16);
      const uint32_t q4 = ((a >> lsh) & 0x0F0F0F0Fu) | (((b >> hsh) & 0x03030303u) << 4);
      const float ds = i < 4 ? ds0 : ds1, m32 = -32.0f * ds;
#pragma unroll
      for (int e = 0; e < 4; ++e) v[4 * i + e] = __builtin_fmaf(ds, (float)((q4 >> (8 * e)) & 0xFFu), m32);
    }
  } else {
    // 6-bit scale and min of sub-block r from the 12 bytes at words 2..7:
    // r < 4 takes the low 6 bits of bytes r and r + 4; r >= 4 takes the
    // nibbles of byte r + 4 and, as bits 4-5, the top bits of bytes r - 4
    // (scale) and r (min).
    auto sbyte = [&](int i) { return ((uint32_t)w[2 + (i >> 1)] >> (8 * (i & 1))) & 0xFFu; };
    uint32_t sc, mn;
    if (r < 4) {
      sc = sbyte(r) & 63u;
      mn = sbyte(r + 4) & 63u;
    } else {
      const uint32_t b = sbyte(r + 4);
      sc = (b & 15u) | ((sbyte(r - 4) >> 6) << 4);
      mn = (b >> 4) | ((sbyte(r) >> 6) << 4);
    }
    // d * sc and dmin * m are exact (11 by 6 bits), and so is d1 * w (17 by
    // 5 bits): the fused d1 * w - m1 is the one rounding of each value.
    const float d1 = f16_bits(w[0]) * (float)sc, m1 = f16_bits(w[1]) * (float)mn;
    constexpr int QS = SRC == SRC_Q4_K ? 8 : 24;  // first word of the nibbles
    const In *qs = w + QS + 16 * (r >> 1);
    const int sh = 4 * (r & 1);
    // four values per 32-bit word, one byte each, then byte conversions
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const uint32_t a = (uint32_t)qs[2 * i] | ((uint32_t)qs[2 * i + 1] << 16);
      uint32_t q4 = (a >> sh) & 0x0F0F0F0Fu;
      if (SRC == SRC_Q5_K) {
        const uint32_t hb = (uint32_t)w[8 + 2 * i] | ((uint32_t)w[8 + 2 * i + 1] << 16);
        q4 |= ((hb >> r) & 0x01010101u) << 4;
      }
#pragma unroll
      for (int e = 0; e < 4; ++e) v[4 * i + e] = __builtin_fmaf(d1, (float)((q4 >> (8 * e)) & 0xFFu), -m1);
    }
  }
}

// Requantises run r of the source block held as 16-bit words at `in` into
// the 17 words of its Q8_0 block at `out`.
template <int SRC, class In, class Out>
__device__ __forceinline__ void requant_run(const In *in, int r, Out *out) {
  float v[32];
  if constexpr (Src<SRC>::RUNS == 1) legacy_values<SRC>(in, v);
  else kquant_values<SRC>(in, r, v);
  store_q8_0(v, out);
}

constexpr int RQ_RUNS = 256;  // output blocks per workgroup, one per thread

// Any 2-byte alignment: each thread reads its source block and writes its
// output block as 16-bit words.  nout = output blocks.
template <int SRC>
__global__ void __launch_bounds__(RQ_RUNS) requant_kernel(int64_t nout, const uint16_t *src, uint16_t *dst) {
  constexpr int SW = Src<SRC>::WORDS, R = Src<SRC>::RUNS;
  const int64_t b = (int64_t)blockIdx.x * RQ_RUNS + threadIdx.x;
  if (b >= nout) return;
  requant_run<SRC>(src + (b / R) * SW, (int)(b % R), dst + b * 17);
}

// 16-byte aligned source and destination: a workgroup's NSB = 256 / RUNS
// source blocks are one contiguous run of NSB * 2 * SW bytes and its 256
// output blocks one of 256 * 34 bytes, both multiples of 16, so full runs
// move as coalesced 16-byte loads and stores through LDS and each thread
// converts one output block there.  The last, partial run moves as 16-bit
// words.  nsrc = source blocks.
template <int SRC>
__global__ void __launch_bounds__(RQ_RUNS) requant_lds_kernel(int64_t nsrc, const uint16_t *src, uint16_t *dst) {
  constexpr int SW = Src<SRC>::WORDS, R = Src<SRC>::RUNS, NSB = RQ_RUNS / R;
  constexpr int IN16 = NSB * SW * 2 / 16, OUT16 = RQ_RUNS * 34 / 16;
  static_assert(NSB * SW * 2 % 16 == 0 && RQ_RUNS * 34 % 16 == 0, "runs of whole 16-byte pieces");
  __shared__ uint4 lin[IN16];
  __shared__ uint4 lout[OUT16];
  const int tid = threadIdx.x;
  const int64_t s0 = (int64_t)blockIdx.x * NSB;
  const int ns = (int)min<int64_t>(NSB, nsrc - s0);
  const uint16_t *s = src + s0 * SW;
  uint16_t *o = dst + s0 * R * 17;
  auto *lin16 = (uint16_t *)lin;
  auto *lout16 = (uint16_t *)lout;
  if (ns == NSB) {
#pragma unroll
    for (int i = tid; i < IN16; i += RQ_RUNS) lin[i] = ((const uint4 *)s)[i];
  } else {
    for (int i = tid; i < ns * SW; i += RQ_RUNS) lin16[i] = s[i];
  }
  __syncthreads();
  if (tid < ns * R) requant_run<SRC>(lin16 + (tid / R) * SW, tid % R, lout16 + tid * 17);
  __syncthreads();
  if (ns == NSB) {
#pragma unroll
    for (int i = tid; i < OUT16; i += RQ_RUNS) ((uint4 *)o)[i] = lout[i];
  } else {
    for (int i = tid; i < ns * R * 17; i += RQ_RUNS) o[i] = lout16[i];
  }
}

template <int SRC>
static void launch_rq(int64_t nb, const uint16_t *s, uint16_t *o, bool vec, hipStream_t st) {
  constexpr int R = Src<SRC>::RUNS;
  if (vec) {
    const dim3 grid((unsigned)((nb + RQ_RUNS / R - 1) / (RQ_RUNS / R)));
    hipLaunchKernelGGL(requant_lds_kernel<SRC>, grid, dim3(RQ_RUNS), 0, st, nb, s, o);
  } else {
    const dim3 grid((unsigned)((nb * R + RQ_RUNS - 1) / RQ_RUNS));
    hipLaunchKernelGGL(requant_kernel<SRC>, grid, dim3(RQ_RUNS), 0, st, nb * R, s, o);
  }
}

// nb source blocks; the caller has checked the type, nb * runs <= 2^36 and
// 2-byte alignment.
int launch_requant_q8_0(int src_type, int64_t nb, const void *src, void *dst, void *stream) {
  clear_hip_error();
  const auto *s = (const uint16_t *)src;
  auto *o = (uint16_t *)dst;
  hipStream_t st = (hipStream_t)stream;
  const bool vec = ((uintptr_t)src % 16 == 0) && ((uintptr_t)dst % 16 == 0);
  switch (src_type) {
    case SRC_Q4_1: launch_rq<SRC_Q4_1>(nb, s, o, vec, st); break;
    case SRC_Q5_0: launch_rq<SRC_Q5_0>(nb, s, o, vec, st); break;
    case SRC_Q5_1: launch_rq<SRC_Q5_1>(nb, s, o, vec, st); break;
    case SRC_Q4_K: launch_rq<SRC_Q4_K>(nb, s, o, vec, st); break;
    case SRC_Q5_K: launch_rq<SRC_Q5_K>(nb, s, o, vec, st); break;
    case SRC_Q6_K: launch_rq<SRC_Q6_K>(nb, s, o, vec, st); break;
    default: return QG_EINVAL;
  }
  return launch_status();
}

}  // namespace qg
