// RMSNorm of activation columns: y = x * gamma / sqrt(mean(x^2) + eps).
//
// What is computed ("Running LLMs in the browser with Three.js", the
// Llama-style differences: the root mean square, no mean subtracted;
// "Engine and kernels": the norm ahead of the router and the gate/up
// products).  The stand-alone form of the prologue that gateup_silu_rmsnorm
// fuses into its staging; it sums the squares in the same order (pieces of
// 8 consecutive k, lane l of one wave taking pieces l, l + 64, ... in order,
// then a fixed wave tree), so 1 / rms has the same bits in both.
#include "common.h"
#include "internal.h"
#include "qgemm.h"

namespace qg {

// One workgroup of 4 waves per column: wave 0 sums the squares (the order
// above), then all four write the scaled column.  Every element is read
// before any is written, so y may be x.  Loads are issued RMS_NB pieces (or
// 8 elements) per lane at a time before any is used.
constexpr int RMS_NB = 8;
constexpr int RMS_W = 4;

__global__ void __launch_bounds__(RMS_W * 64) rmsnorm_kernel(const float *X, int64_t ldx, int64_t cols,
                                                              const float *gamma, float eps, float *Y,
                                                              int64_t ldy) {
  __shared__ float s_inv;
  const int tid = threadIdx.x, lane = tid & 63;
  const float *x = X + (int64_t)blockIdx.x * ldx;
  float *y = Y + (int64_t)blockIdx.x * ldy;
  if (tid < 64) {
    const int64_t np = (cols + 7) / 8;
    float t = 0.0f;
    for (int64_t p0 = lane; p0 < np; p0 += 64 * RMS_NB) {
      float v[RMS_NB][8];
#pragma unroll
      for (int b = 0; b < RMS_NB; ++b)
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const int64_t k = (p0 + 64 * b) * 8 + e;
          v[b][e] = k < cols ? x[k] : 0.0f;
        }
#pragma unroll
      for (int b = 0; b < RMS_NB; ++b) {
        if (p0 + 64 * b >= np) break;
        float q = v[b][0] * v[b][0];
#pragma unroll
        for (int e = 1; e < 8; ++e) q = __builtin_fmaf(v[b][e], v[b][e], q);
        t += q;
      }
    }
    t = wave_sum(t);
    if (lane == 0) s_inv = 1.0f / __builtin_sqrtf(t / (float)cols + eps);
  }
  __syncthreads();
  const float inv = s_inv;
  for (int64_t k0 = tid; k0 < cols; k0 += RMS_W * 64 * 8) {
    float xv[8], gv[8];
#pragma unroll
    for (int b = 0; b < 8; ++b) {
      const int64_t k = k0 + RMS_W * 64 * b;
      xv[b] = k < cols ? x[k] : 0.0f;
      gv[b] = k < cols ? gamma[k] : 0.0f;
    }
#pragma unroll
    for (int b = 0; b < 8; ++b) {
      const int64_t k = k0 + RMS_W * 64 * b;
      if (k < cols) y[k] = xv[b] * gv[b] * inv;
    }
  }
}

int launch_rmsnorm(const float *X, int64_t ldx, int64_t cols, int ncols, const float *gamma, float eps, float *Y,
                   int64_t ldy, void *stream) {
  clear_hip_error();
  hipLaunchKernelGGL(rmsnorm_kernel, dim3((unsigned)ncols), dim3(RMS_W * 64), 0, (hipStream_t)stream, X, ldx, cols, gamma,
                     eps, Y, ldy);
  return launch_status();
}

}  // namespace qg
