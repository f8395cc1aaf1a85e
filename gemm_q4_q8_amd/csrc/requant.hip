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

// One thread per block.  Every block size is even, so each block is read
// and written as 16-bit words.
template <int SRC>
__global__ void __launch_bounds__(256) requant_kernel(int64_t nb, const uint16_t *src, uint16_t *dst) {
  constexpr int SW = SRC == SRC_Q4_1 ? 10 : SRC == SRC_Q5_0 ? 11 : 12;  // source words per block
  const int64_t b = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (b >= nb) return;
  uint16_t wsrc[SW];
#pragma unroll
  for (int i = 0; i < SW; ++i) wsrc[i] = src[b * SW + i];
  const float d = f16_bits(wsrc[0]);
  const float m = SRC == SRC_Q5_0 ? 0.0f : f16_bits(wsrc[1]);
  const uint32_t qh = SRC == SRC_Q4_1 ? 0u
                      : SRC == SRC_Q5_0 ? ((uint32_t)wsrc[1] | ((uint32_t)wsrc[2] << 16))
                                        : ((uint32_t)wsrc[2] | ((uint32_t)wsrc[3] << 16));
  constexpr int QS = SRC == SRC_Q4_1 ? 2 : SRC == SRC_Q5_0 ? 3 : 4;  // first nibble word
  float v[32];
#pragma unroll
  for (int j = 0; j < 16; ++j) {
    const uint32_t byte = (wsrc[QS + j / 2] >> (8 * (j & 1))) & 0xFFu;
    int lo = (int)(byte & 15u), hi = (int)(byte >> 4);
    if (SRC != SRC_Q4_1) {
      lo |= (int)((qh >> j) & 1u) << 4;
      hi |= (int)((qh >> (j + 16)) & 1u) << 4;
    }
    if (SRC == SRC_Q5_0) {
      v[j] = (float)(lo - 16) * d;
      v[j + 16] = (float)(hi - 16) * d;
    } else {
      v[j] = (float)lo * d + m;
      v[j + 16] = (float)hi * d + m;
    }
  }
  float amax = 0.0f;
#pragma unroll
  for (int j = 0; j < 32; ++j) amax = __builtin_fmaxf(amax, __builtin_fabsf(v[j]));
  const float dq = amax / 127.0f;
  const float id = dq != 0.0f ? 1.0f / dq : 0.0f;
  uint16_t out[17];
  out[0] = __builtin_bit_cast(uint16_t, (_Float16)dq);
#pragma unroll
  for (int j = 0; j < 32; j += 2) {
    const int q0 = (int)__builtin_roundf(v[j] * id), q1 = (int)__builtin_roundf(v[j + 1] * id);
    out[1 + j / 2] = (uint16_t)((uint32_t)(q0 & 0xFF) | ((uint32_t)(q1 & 0xFF) << 8));
  }
#pragma unroll
  for (int i = 0; i < 17; ++i) dst[b * 17 + i] = out[i];
}

int launch_requant_q8_0(int src_type, int64_t nb, const void *src, void *dst, void *stream) {
  const dim3 grid((unsigned)((nb + 255) / 256));
  clear_hip_error();
  const auto *s = (const uint16_t *)src;
  auto *o = (uint16_t *)dst;
  hipStream_t st = (hipStream_t)stream;
  if (src_type == SRC_Q4_1) hipLaunchKernelGGL(requant_kernel<SRC_Q4_1>, grid, dim3(256), 0, st, nb, s, o);
  else if (src_type == SRC_Q5_0) hipLaunchKernelGGL(requant_kernel<SRC_Q5_0>, grid, dim3(256), 0, st, nb, s, o);
  else hipLaunchKernelGGL(requant_kernel<SRC_Q5_1>, grid, dim3(256), 0, st, nb, s, o);
  return launch_status();
}

}  // namespace qg
