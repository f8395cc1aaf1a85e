// Load-time requantisation of Q4_1 / Q5_0 / Q5_1 blocks to Q8_0.
//
// What is computed ("Engine and kernels", What it runs: the few Q4_1 / Q5_0
// / K-quant tensors of the public MoE file are requantized to Q8_0 on the
// way to the GPU; "Architecture", where the weights live: converted once,
// the result kept).  The source layouts are the public GGUF ones (K-quants
// are not covered): Q4_1 = f16 d, f16 m, 16 nibble bytes, value w * d + m;
// Q5_0 = f16 d, 32 high bits, 16 nibble bytes, value (w - 16) * d; Q5_1 =
// f16 d, f16 m, high bits, nibbles, value w * d + m (weight j: low nibble of
// byte j plus high bit j; weight j + 16: high nibble plus bit j + 16).  Each
// block is requantised to Q8_0 by the usual rule, in float32 steps each
// rounded once: d = max|v| / 127, q = v * (1 / d) rounded half away from
// zero, d stored as binary16.  The output is canonical Q8_0 blocks, which
// qg_repack then tiles; the conversion runs on the GPU, so the source bytes
// are uploaded once, smaller than the Q8_0 result.
#include "common.h"
#include "internal.h"
#include "qgemm.h"

namespace qg {

constexpr int SRC_Q4_1 = 3, SRC_Q5_0 = 6, SRC_Q5_1 = 7;

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

// Requantises one block held as 16-bit words at `in` (SW words) into the 17
// words of its Q8_0 block at `out`.
template <int SRC, class In, class Out>
__device__ __forceinline__ void requant_block(const In *in, Out *out) {
  constexpr int SW = SRC == SRC_Q4_1 ? 10 : SRC == SRC_Q5_0 ? 11 : 12;  // source words per block
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
  float v[32];
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

constexpr int RQ_BLOCKS = 256;  // blocks per workgroup, one per thread

// Any 2-byte alignment: each thread reads and writes its own block as
// 16-bit words.
template <int SRC>
__global__ void __launch_bounds__(RQ_BLOCKS) requant_kernel(int64_t nb, const uint16_t *src, uint16_t *dst) {
  constexpr int SW = SRC == SRC_Q4_1 ? 10 : SRC == SRC_Q5_0 ? 11 : 12;
  const int64_t b = (int64_t)blockIdx.x * RQ_BLOCKS + threadIdx.x;
  if (b >= nb) return;
  requant_block<SRC>(src + b * SW, dst + b * 17);
}

// 16-byte aligned source and destination: a workgroup's 256 blocks are one
// contiguous run of 256 * 2 * SW source bytes and 256 * 34 output bytes,
// both multiples of 16, so full runs move as coalesced 16-byte loads and
// stores through LDS and each thread converts one block there.  The last,
// partial run moves as 16-bit words.
template <int SRC>
__global__ void __launch_bounds__(RQ_BLOCKS) requant_lds_kernel(int64_t nb, const uint16_t *src, uint16_t *dst) {
  constexpr int SW = SRC == SRC_Q4_1 ? 10 : SRC == SRC_Q5_0 ? 11 : 12;
  constexpr int IN16 = RQ_BLOCKS * SW * 2 / 16, OUT16 = RQ_BLOCKS * 34 / 16;
  static_assert(RQ_BLOCKS * SW * 2 % 16 == 0 && RQ_BLOCKS * 34 % 16 == 0, "runs of whole 16-byte pieces");
  __shared__ uint4 lin[IN16];
  __shared__ uint4 lout[OUT16];
  const int tid = threadIdx.x;
  const int64_t b0 = (int64_t)blockIdx.x * RQ_BLOCKS;
  const int nblk = (int)min<int64_t>(RQ_BLOCKS, nb - b0);
  const uint16_t *s = src + b0 * SW;
  uint16_t *o = dst + b0 * 17;
  auto *lin16 = (uint16_t *)lin;
  auto *lout16 = (uint16_t *)lout;
  if (nblk == RQ_BLOCKS) {
#pragma unroll
    for (int i = tid; i < IN16; i += RQ_BLOCKS) lin[i] = ((const uint4 *)s)[i];
  } else {
    for (int i = tid; i < nblk * SW; i += RQ_BLOCKS) lin16[i] = s[i];
  }
  __syncthreads();
  if (tid < nblk) requant_block<SRC>(lin16 + tid * SW, lout16 + tid * 17);
  __syncthreads();
  if (nblk == RQ_BLOCKS) {
#pragma unroll
    for (int i = tid; i < OUT16; i += RQ_BLOCKS) ((uint4 *)o)[i] = lout[i];
  } else {
    for (int i = tid; i < nblk * 17; i += RQ_BLOCKS) o[i] = lout16[i];
  }
}

int launch_requant_q8_0(int src_type, int64_t nb, const void *src, void *dst, void *stream) {
  const dim3 grid((unsigned)((nb + RQ_BLOCKS - 1) / RQ_BLOCKS));
  clear_hip_error();
  const auto *s = (const uint16_t *)src;
  auto *o = (uint16_t *)dst;
  hipStream_t st = (hipStream_t)stream;
  const bool vec = ((uintptr_t)src % 16 == 0) && ((uintptr_t)dst % 16 == 0);
  if (src_type == SRC_Q4_1) {
    if (vec) hipLaunchKernelGGL(requant_lds_kernel<SRC_Q4_1>, grid, dim3(RQ_BLOCKS), 0, st, nb, s, o);
    else hipLaunchKernelGGL(requant_kernel<SRC_Q4_1>, grid, dim3(RQ_BLOCKS), 0, st, nb, s, o);
  } else if (src_type == SRC_Q5_0) {
    if (vec) hipLaunchKernelGGL(requant_lds_kernel<SRC_Q5_0>, grid, dim3(RQ_BLOCKS), 0, st, nb, s, o);
    else hipLaunchKernelGGL(requant_kernel<SRC_Q5_0>, grid, dim3(RQ_BLOCKS), 0, st, nb, s, o);
  } else {
    if (vec) hipLaunchKernelGGL(requant_lds_kernel<SRC_Q5_1>, grid, dim3(RQ_BLOCKS), 0, st, nb, s, o);
    else hipLaunchKernelGGL(requant_kernel<SRC_Q5_1>, grid, dim3(RQ_BLOCKS), 0, st, nb, s, o);
  }
  return launch_status();
}

}  // namespace qg
