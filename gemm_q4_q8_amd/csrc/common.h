// Device helpers shared by the gfx950 kernels of libqgemm.
//
// Weight decoding follows the GGUF block definition ("Engine and kernels",
// What it runs: 32 weights plus one f16 scale per block) in the tiled layout
// declared in include/qgemm.h.  Weights become exact f16 values in registers
// ("Reading weights": dequantise in registers, full-precision weights never
// exist in memory); activations enter as f16; every sum is f32 ("Correctness
// and portability": no f16 accumulation).
#pragma once
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace qg {

typedef _Float16 h2 __attribute__((ext_vector_type(2)));
typedef _Float16 h4 __attribute__((ext_vector_type(4)));
typedef _Float16 h8 __attribute__((ext_vector_type(8)));
typedef float f4 __attribute__((ext_vector_type(4)));
typedef uint32_t u4 __attribute__((ext_vector_type(4)));
typedef uint32_t u2 __attribute__((ext_vector_type(2)));

constexpr int Q4 = 2;
constexpr int Q8 = 8;
constexpr int TILE_ROWS = 16;
constexpr int TILE_BLOCKS = 4;
constexpr int TILE_COLS = 128;
constexpr int TILE_D_BYTES = 128;
template <int QT> struct QTraits;
template <> struct QTraits<Q4> { static constexpr int tile_bytes = 1024; static constexpr int block_bytes = 18; };
template <> struct QTraits<Q8> { static constexpr int tile_bytes = 2048; static constexpr int block_bytes = 34; };

__device__ __forceinline__ h2 as_h2(uint32_t v) { return __builtin_bit_cast(h2, v); }

// (w & mask) | bits in one VALU op.  gfx950 VOP3 encodings take no literal
// constants and one scalar operand, so the mask rides in an SGPR and the OR
// pattern in a VGPR (the compiler would otherwise split the op in two).
__device__ __forceinline__ uint32_t and_or(uint32_t w, uint32_t mask, uint32_t bits) {
  uint32_t r;
  __asm__("v_and_or_b32 %0, %1, %2, %3" : "=v"(r) : "v"(w), "s"(mask), "v"(bits));
  return r;
}

// Q4_0: one u32 word of the tiled layout = 8 nibbles of one block slice;
// pair u holds columns (2u, 2u + 1) at bits (4u, 16 + 4u).  A nibble n at
// bits 0..3 of a 16-bit half, under the f16 pattern 0x6400 (1024.0, ulp 1),
// reads as 1024 + n; a nibble at bits 4..7 under 0x5400 (64.0, ulp 1/16)
// reads as 64 + n.  Both are exact, and subtracting 1032 or 72 leaves the
// weight n - 8 exactly.  One shift by 8 brings pairs 2 and 3 into place.
// The two OR patterns live in VGPRs for the whole kernel: `Q4Magic` is made
// once by an opaque move, so the compiler keeps it instead of re-creating
// the constants before every use.
struct Q4Magic {
  uint32_t lo, hi;  // 0x64006400, 0x54005400
};
__device__ __forceinline__ Q4Magic q4_magic() {
  Q4Magic m;
  __asm__ volatile("v_mov_b32 %0, 0x64006400" : "=v"(m.lo));
  __asm__ volatile("v_mov_b32 %0, 0x54005400" : "=v"(m.hi));
  return m;
}

__device__ __forceinline__ void unpack_q4(uint32_t w, h2 out[4], Q4Magic mg) {
  const h2 b_lo = {(_Float16)1032.0f, (_Float16)1032.0f};
  const h2 b_hi = {(_Float16)72.0f, (_Float16)72.0f};
  const uint32_t w8 = w >> 8;
  out[0] = as_h2(and_or(w, 0x000F000Fu, mg.lo)) - b_lo;
  out[1] = as_h2(and_or(w, 0x00F000F0u, mg.hi)) - b_hi;
  out[2] = as_h2(and_or(w8, 0x000F000Fu, mg.lo)) - b_lo;
  out[3] = as_h2(and_or(w8, 0x00F000F0u, mg.hi)) - b_hi;
}

// The dot product of a weight pair and an activation pair, starting a new
// sum (v_dot2_f32_f16 with an inline zero accumulator; the accumulating
// v_dot2c form would need a register cleared first).
__device__ __forceinline__ float dot2_first(h2 a, h2 b) {
  float r;
  __asm__("v_dot2_f32_f16 %0, %1, %2, 0" : "=v"(r) : "v"(a), "v"(b));
  return r;
}

// Streaming loads of weights and scales: each byte is read once per call,
// so they bypass cache allocation (nontemporal) and leave L2 to the
// activations and partial sums.
__device__ __forceinline__ u4 ld_stream(const uint8_t *p) { return __builtin_nontemporal_load((const u4 *)p); }
__device__ __forceinline__ u2 ld_stream2(const uint8_t *p) { return __builtin_nontemporal_load((const u2 *)p); }

// Bounded streams: a raw buffer resource over [base, base + bytes).  A load
// at an offset at or beyond `bytes` returns zeros and reads no memory (the
// buffer range check of gfx9), so a prefetch loop can run past the end of
// its range without a branch around its loads.  Offsets go in the VGPR
// offset, which is what the range check covers.
// A range belongs to the wave: every lane passes the same base and size.
// The descriptor lives in scalar registers; taking both from the first lane
// says so to the compiler, which otherwise, where it cannot prove the values
// uniform (e.g. an expert chosen at run time), wraps each load in a loop
// over the distinct per-lane descriptors.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t buf_range(const void *base, uint32_t bytes) {
  const uint64_t b = (uint64_t)base;
  const uint64_t ub = ((uint64_t)__builtin_amdgcn_readfirstlane((uint32_t)(b >> 32)) << 32) |
                      (uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)b);
  return __builtin_amdgcn_make_buffer_rsrc((void *)ub, (short)0, (int)__builtin_amdgcn_readfirstlane(bytes),
                                           0x00020000);
}
// nontemporal (aux bit 1): streamed once, no cache allocation
__device__ __forceinline__ u4 buf_ld16(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  return __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 2);
}
__device__ __forceinline__ u2 buf_ld8(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  return __builtin_amdgcn_raw_buffer_load_b64(r, off, 0, 2);
}

// Q8_0: two u32 words = 8 biased bytes (q + 128) of one block slice.  A byte
// permute puts each byte under a 0x64 high byte (1024 + b, exact), then
// subtracting 1152 = 1024 + 128 leaves q exactly.
__device__ __forceinline__ void unpack_q8(uint32_t w0, uint32_t w1, h2 out[4]) {
  const h2 bias = {(_Float16)1152.0f, (_Float16)1152.0f};
  out[0] = as_h2(__builtin_amdgcn_perm(0x64646464u, w0, 0x05010400u)) - bias;
  out[1] = as_h2(__builtin_amdgcn_perm(0x64646464u, w0, 0x05030402u)) - bias;
  out[2] = as_h2(__builtin_amdgcn_perm(0x64646464u, w1, 0x05010400u)) - bias;
  out[3] = as_h2(__builtin_amdgcn_perm(0x64646464u, w1, 0x05030402u)) - bias;
}

// The f16 scale number j (0..3) of a lane's 8-byte scale word.
__device__ __forceinline__ float scale_of(u2 dw, int j) {
  uint32_t w = (j < 2) ? dw[0] : dw[1];
  uint16_t b = (j & 1) ? (uint16_t)(w >> 16) : (uint16_t)(w & 0xFFFF);
  return (float)__builtin_bit_cast(_Float16, b);
}

__device__ __forceinline__ h8 cvt8(const float4 lo, const float4 hi) {
  h8 r;
  r[0] = (_Float16)lo.x; r[1] = (_Float16)lo.y; r[2] = (_Float16)lo.z; r[3] = (_Float16)lo.w;
  r[4] = (_Float16)hi.x; r[5] = (_Float16)hi.y; r[6] = (_Float16)hi.z; r[7] = (_Float16)hi.w;
  return r;
}

__device__ __forceinline__ h2 lo_pair(h8 v, int u) {
  h2 r;
  r[0] = v[2 * u];
  r[1] = v[2 * u + 1];
  return r;
}

// Agent-scope relaxed accesses for data exchanged between workgroups (the
// L2 caches of the eight XCDs are not coherent with each other).
__device__ __forceinline__ void st_agent(float *p, float v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ float ld_agent(const float *p) {
  return __hip_atomic_load(const_cast<float *>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void st_agent_u32(uint32_t *p, uint32_t v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void st_agent_u64(uint64_t *p, uint64_t v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ uint32_t ld_agent_u32(const uint32_t *p) {
  return __hip_atomic_load(const_cast<uint32_t *>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// "Last one in" for a group of `target` workgroups sharing a counter.
// Everything workgroups exchange goes through agent-scope atomic stores and
// loads (st_agent / ld_agent above), which are coherent across the XCDs'
// L2 caches by themselves.  So no cache-wide fence is needed (on gfx950 a
// device-scope fence writes back and invalidates a whole L2): each thread
// waits until its own stores are acknowledged, the workgroup increments the
// counter with a relaxed agent-scope atomic, and the workgroup that sees
// target - 1 is last.  It resets the counter to zero for the next call.  Its
// later ld_agent loads are issued only after the counter returned.
// `flag` is an LDS word.
__device__ __forceinline__ bool arrive_last(uint32_t *cnt, uint32_t target, uint32_t *flag) {
  __asm__ volatile("s_waitcnt vmcnt(0)" ::: "memory");
  __syncthreads();
  if (threadIdx.x == 0) {
    const uint32_t old = __hip_atomic_fetch_add(cnt, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    const uint32_t last = (old == target - 1) ? 1u : 0u;
    if (last) __hip_atomic_store(cnt, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    *flag = last;
  }
  __syncthreads();
  const bool last = *flag != 0;
  __asm__ volatile("" ::: "memory");
  return last;
}

// Order for argmax / top-k: larger value first, then lower index; a NaN
// ranks below every number.
__device__ __forceinline__ bool ranks_before(float va, int32_t ia, float vb, int32_t ib) {
  bool na = va != va, nb = vb != vb;
  if (na || nb) return nb && (!na || ia < ib);
  return va > vb || (va == vb && ia < ib);
}

// Wave-wide reductions without LDS round trips.  Lane exchanges by DPP: the
// quad permutes [1,0,3,2] and [2,3,0,1] pair lanes at distance 1 and 2; once
// values agree within groups of 4 (then 8), the half-row mirror (then the
// row mirror) pairs each group with its neighbour; a swizzle (xor 16 within
// 32 lanes) joins the two rows of each half, and the halves meet through
// readlane.  The combine is symmetric, so every lane ends with the same bits.
__device__ __forceinline__ int dpp_partner(int v, int step) {
  switch (step) {
    case 0: return __builtin_amdgcn_mov_dpp(v, 0xB1, 0xF, 0xF, false);   // quad_perm [1,0,3,2]
    case 1: return __builtin_amdgcn_mov_dpp(v, 0x4E, 0xF, 0xF, false);   // quad_perm [2,3,0,1]
    case 2: return __builtin_amdgcn_mov_dpp(v, 0x141, 0xF, 0xF, false);  // row_half_mirror
    case 3: return __builtin_amdgcn_mov_dpp(v, 0x140, 0xF, 0xF, false);  // row_mirror
  }
  return __builtin_amdgcn_ds_swizzle(v, 0x401F);                          // xor 16
}

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int step = 0; step < 5; ++step)
    v += __builtin_bit_cast(float, dpp_partner(__builtin_bit_cast(int, v), step));
  const int b = __builtin_bit_cast(int, v);
  return __builtin_bit_cast(float, __builtin_amdgcn_readlane(b, 0)) +
         __builtin_bit_cast(float, __builtin_amdgcn_readlane(b, 32));
}

// The wave's largest 64-bit value, in every lane.  Four DPP steps leave each
// row of 16 lanes holding its row's maximum; the four rows then meet
// through readlane (the swizzle step of wave_sum, an LDS round trip for
// each 32-bit half, made a selection round about three times slower).
__device__ __forceinline__ uint64_t wave_max_u64(uint64_t v) {
#pragma unroll
  for (int step = 0; step < 4; ++step) {
    const uint32_t lo = (uint32_t)dpp_partner((int)(uint32_t)v, step);
    const uint32_t hi = (uint32_t)dpp_partner((int)(uint32_t)(v >> 32), step);
    const uint64_t o = ((uint64_t)hi << 32) | lo;
    v = o > v ? o : v;
  }
  uint64_t m = 0;
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const uint64_t o = ((uint64_t)(uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)(v >> 32), 16 * r) << 32) |
                       (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)v, 16 * r);
    m = o > m ? o : m;
  }
  return m;
}

// The order of ranks_before as one unsigned key: the value's bits mapped to
// an order-preserving code (negatives complemented, positives with the sign
// bit set, -0 as +0, every NaN as 0), above the complemented index.  Larger
// key = ranks first; every key of a real index is above 0.
__device__ __forceinline__ uint64_t rank_key(float v, int32_t i) {
  const uint32_t b = __builtin_bit_cast(uint32_t, v);
  uint32_t c = (b & 0x80000000u) ? ~b : (b | 0x80000000u);
  if (v == 0.0f) c = 0x80000000u;
  if (v != v) c = 0u;
  return ((uint64_t)c << 32) | (0xFFFFFFFFu - (uint32_t)i);
}
__device__ __forceinline__ int32_t rank_key_index(uint64_t k) { return (int32_t)(0xFFFFFFFFu - (uint32_t)k); }
// the value back (a NaN for code 0)
__device__ __forceinline__ float rank_key_value(uint64_t k) {
  const uint32_t c = (uint32_t)(k >> 32);
  return __builtin_bit_cast(float, (c & 0x80000000u) ? (c & 0x7FFFFFFFu) : ~c);
}

// The wave's largest rank key (as wave_max_u64) in fewer dependent steps: a
// 32-bit maximum over the value codes (the upper halves), then the lanes
// holding that code by ballot; when one lane holds it, its key is the
// answer (one readlane), and when several do (equal values), the full
// 64-bit maximum decides by index.  Measured on the MoE token selection
// (8 rounds over 256 keys): 2.6 us with the 64-bit maximum every round.
__device__ __forceinline__ uint64_t wave_max_key(uint64_t v) {
  const uint32_t hi = (uint32_t)(v >> 32);
  uint32_t m = hi;
#pragma unroll
  for (int step = 0; step < 4; ++step) {
    const uint32_t o = (uint32_t)dpp_partner((int)m, step);
    m = o > m ? o : m;
  }
  uint32_t mh = 0;
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const uint32_t o = (uint32_t)__builtin_amdgcn_readlane((int)m, 16 * r);
    mh = o > mh ? o : mh;
  }
  const uint64_t who = __ballot(hi == mh);
  if (__popcll(who) == 1) {
    const int l = __builtin_ctzll(who);
    return ((uint64_t)mh << 32) | (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)v, l);
  }
  return wave_max_u64(v);
}

// blockIdx -> work unit, so that each XCD (workgroups are dealt to the eight
// XCDs round-robin) takes a contiguous range of units.
__device__ __forceinline__ int64_t xcd_unit(int64_t per_xcd) {
  int64_t b = blockIdx.x;
  return (b & 7) * per_xcd + (b >> 3);
}

}  // namespace qg
