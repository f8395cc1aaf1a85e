// Load-time repack of GGUF Q4_0 / Q8_0 blocks into the tiled weight and
// scale streams ("Architecture", Memory and caching: matrices are repacked on
// the way into separate nibble and scale arrays so kernels read contiguous
// stripes; "Engine and kernels", Reading weights: layout, not compression).
//
// One thread writes one 16-byte chunk of a tile; it gathers the 8-column
// slices of that chunk's blocks straight from the GGUF bytes.  Writes are
// fully coalesced; reads are 2-byte loads at the 18 / 34-byte block stride.
// Padding positions (beyond rows or cols) receive zero weights and zero
// scales, so the product kernels never test for ragged tiles.
#include "common.h"
#include "internal.h"
#include "qgemm.h"

namespace qg {

struct RepackArgs {
  const uint8_t *src;
  uint8_t *qs;
  uint8_t *d;
  int64_t rows, nb;   // GGUF rows and blocks per row (per matrix)
  int64_t NT, KT;     // tiles per matrix
  int64_t chunks;     // total 16-byte weight chunks over all matrices
  int64_t dslots;     // total 8-byte scale words over all matrices
};

__device__ __forceinline__ uint16_t ld16(const uint8_t *p) { return *(const uint16_t *)p; }

template <int QT>
__global__ void __launch_bounds__(256) repack_kernel(RepackArgs a) {
  constexpr int BB = QTraits<QT>::block_bytes;
  constexpr int CPT = QTraits<QT>::tile_bytes / 16;  // chunks per tile (64 or 128)
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const int64_t tiles_per_mat = a.NT * a.KT;
  if (i < a.chunks) {
    const int64_t tile = i / CPT;
    const int chunk = (int)(i % CPT);
    const int64_t m = tile / tiles_per_mat;
    const int64_t tm = tile % tiles_per_mat;
    const int64_t rt = tm / a.KT, kt = tm % a.KT;
    const int h = chunk / 64, c = chunk % 64;          // h: Q8_0 half
    const int s = c / 16, r = c % 16;
    const int64_t row = rt * 16 + r;
    const uint8_t *rowp = a.src + (m * a.rows + row) * a.nb * BB;
    u4 out;
    if constexpr (QT == Q4) {
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int64_t b = kt * 4 + j;
        uint32_t word = 0x88888888u;                   // zero weights
        if (row < a.rows && b < a.nb) {
          // columns 8s..8s+7: low nibbles (s < 2) or high nibbles (s >= 2)
          // of GGUF bytes qs[8*(s&1) .. 8*(s&1)+7]
          const uint8_t *q = rowp + b * BB + 2 + 8 * (s & 1);
          const int shift = (s >> 1) * 4;
          uint32_t nib[8];
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const uint16_t v = ld16(q + 2 * e);
            nib[2 * e] = ((v & 0xFFu) >> shift) & 0xFu;
            nib[2 * e + 1] = ((v >> 8) >> shift) & 0xFu;
          }
          word = 0;
#pragma unroll
          for (int uu = 0; uu < 4; ++uu) word |= (nib[2 * uu] << (4 * uu)) | (nib[2 * uu + 1] << (16 + 4 * uu));
        }
        out[j] = word;
      }
    } else {
#pragma unroll
      for (int jj = 0; jj < 2; ++jj) {
        const int64_t b = kt * 4 + 2 * h + jj;
        uint32_t w0 = 0x80808080u, w1 = 0x80808080u;   // zero weights (biased)
        if (row < a.rows && b < a.nb) {
          const uint8_t *q = rowp + b * BB + 2 + 8 * s;
          w0 = ((uint32_t)ld16(q) | ((uint32_t)ld16(q + 2) << 16)) ^ 0x80808080u;
          w1 = ((uint32_t)ld16(q + 4) | ((uint32_t)ld16(q + 6) << 16)) ^ 0x80808080u;
        }
        out[2 * jj] = w0;
        out[2 * jj + 1] = w1;
      }
    }
    *(u4 *)(a.qs + i * 16) = out;
  }
  if (i < a.dslots) {
    // scale word: tile, row r -> f16 scales of blocks 4kt .. 4kt+3
    const int64_t tile = i / 16;
    const int r = (int)(i % 16);
    const int64_t m = tile / tiles_per_mat;
    const int64_t tm = tile % tiles_per_mat;
    const int64_t rt = tm / a.KT, kt = tm % a.KT;
    const int64_t row = rt * 16 + r;
    const uint8_t *rowp = a.src + (m * a.rows + row) * a.nb * BB;
    uint32_t dw[2] = {0, 0};
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int64_t b = kt * 4 + j;
      uint32_t v = 0;
      if (row < a.rows && b < a.nb) v = ld16(rowp + b * BB);
      dw[j >> 1] |= v << (16 * (j & 1));
    }
    *(u2 *)(a.d + i * 8) = u2{dw[0], dw[1]};
  }
}

int launch_repack(int qtype, int64_t n_mat, int64_t rows, int64_t cols, const void *blocks, void *qs,
                  void *d, hipStream_t stream) {
  RepackArgs a;
  a.src = (const uint8_t *)blocks;
  a.qs = (uint8_t *)qs;
  a.d = (uint8_t *)d;
  a.rows = rows;
  a.nb = cols / 32;
  a.NT = (rows + 15) / 16;
  a.KT = (a.nb + 3) / 4;
  const int64_t tiles = n_mat * a.NT * a.KT;
  const int cpt = qtype == QG_Q4_0 ? 64 : 128;
  a.chunks = tiles * cpt;
  a.dslots = tiles * 16;
  const int64_t n = a.chunks > a.dslots ? a.chunks : a.dslots;
  const int64_t grid = (n + 255) / 256;
  if (grid > 0x7fffffff) return QG_EUNSUPPORTED;
  clear_hip_error();
  if (qtype == QG_Q4_0)
    hipLaunchKernelGGL(repack_kernel<Q4>, dim3((unsigned)grid), dim3(256), 0, stream, a);
  else
    hipLaunchKernelGGL(repack_kernel<Q8>, dim3((unsigned)grid), dim3(256), 0, stream, a);
  return launch_status();
}

}  // namespace qg
