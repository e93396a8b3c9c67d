// Counter-based random numbers for sampled drafting and verification.
//
// Philox4x64-10 (Salmon, Moraes, Dror and Shaw, "Parallel random numbers: as easy
// as 1, 2, 3", SC 2011): a block maps a 4-word counter and a 2-word key to four
// 64-bit words through 10 rounds of two 64 x 64 -> 128-bit multiplications, the key
// advancing by two Weyl constants between rounds.  The four words are read as
// eight 32-bit values, low half of word 0 first.  A 32-bit value h gives the
// uniform u = (h + 1/2) 2^-32 on (0, 1) and the Gumbel variate -ln(-ln u).
//
// Key (seed, stream); counters per draw family:
//   kStreamDraft  drafter noise of flattened block row m and token v:
//                 (16 (v >> 5) + (v & 15), m >> 2, step, 0), value 2 (m & 3) + ((v >> 4) & 1)
//                 -- one block covers rows 4g..4g+3 times tokens v and v + 16, the
//                 elements one lane holds of two adjacent 16 x 16 MFMA output blocks;
//   kStreamAccept acceptance uniform of row i of sequence b: (i, b, step, 0), value 0;
//   kStreamEmit   noise of the residual / bonus draw of sequence b, token v:
//                 (v >> 3, b, step, 0), value v & 7.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace dflash {

constexpr uint64_t kPhiloxM0 = 0xD2E7470EE14C6C93ull, kPhiloxM1 = 0xCA5A826395121157ull;
constexpr uint64_t kPhiloxW0 = 0x9E3779B97F4A7C15ull, kPhiloxW1 = 0xBB67AE8584CAA73Bull;
constexpr uint64_t kStreamDraft = 1, kStreamAccept = 2, kStreamEmit = 3;

// Eight 32-bit values of the block at counter (c0, c1, c2, c3), key (k0, k1).
// ROLLED keeps the 10 rounds a loop: callers that unroll a large epilogue around it
// (the tiled GEMM) stay small enough for their accumulator arrays to be unrolled
// into registers.
template <bool ROLLED = false>
__device__ __forceinline__ void philox_u32x8(uint64_t c0, uint64_t c1, uint64_t c2, uint64_t c3,
                                             uint64_t k0, uint64_t k1, uint32_t out[8]) {
#pragma unroll(ROLLED ? 1 : 10)
  for (int r = 0; r < 10; ++r) {
    const uint64_t lo0 = c0 * kPhiloxM0, hi0 = __umul64hi(c0, kPhiloxM0);
    const uint64_t lo1 = c2 * kPhiloxM1, hi1 = __umul64hi(c2, kPhiloxM1);
    c0 = hi1 ^ c1 ^ k0;
    c1 = lo1;
    c2 = hi0 ^ c3 ^ k1;
    c3 = lo0;
    k0 += kPhiloxW0;
    k1 += kPhiloxW1;
  }
  out[0] = static_cast<uint32_t>(c0);
  out[1] = static_cast<uint32_t>(c0 >> 32);
  out[2] = static_cast<uint32_t>(c1);
  out[3] = static_cast<uint32_t>(c1 >> 32);
  out[4] = static_cast<uint32_t>(c2);
  out[5] = static_cast<uint32_t>(c2 >> 32);
  out[6] = static_cast<uint32_t>(c3);
  out[7] = static_cast<uint32_t>(c3 >> 32);
}

constexpr float kLn2 = 0.693147180559945309f;
constexpr float kLog2e = 1.442695040888963407f;

__device__ __forceinline__ float ln_f32(float x) { return __builtin_amdgcn_logf(x) * kLn2; }

// ln of the uniform (h + 1/2) 2^-32, in float.  Below 1/2 u itself is formed (one
// rounding).  Above, w = 1 - u = (~h + 1/2) 2^-32 is formed instead, and ln(1 - w)
// comes from a short series when w < 2^-7 (truncation below 2^-30 relative) and
// from the logarithm of the rounded 1 - w otherwise (error below 2^-18 relative).
__device__ __forceinline__ float ln_uniform(uint32_t h) {
  const bool low = h < 0x80000000u;
  const float x = (static_cast<float>(low ? h : ~h) + 0.5f) * 0x1p-32f;
  float l = ln_f32(low ? x : 1.f - x);
  if (!low && x < 0x1p-7f) l = -x * (1.f + x * (0.5f + x * (0.33333333f + x * 0.25f)));
  return l;
}

__device__ __forceinline__ float uniform_f32(uint32_t h) { return (static_cast<float>(h) + 0.5f) * 0x1p-32f; }

__device__ __forceinline__ float gumbel_f32(uint32_t h) { return -ln_f32(-ln_uniform(h)); }

// Online log-sum-exp pair (max, sum of exp(s - max)); merging keeps empty pairs
// (max = -inf, sum = 0) neutral.
__device__ __forceinline__ void lse_merge(float& m, float& s, float m2, float s2) {
  const float M = fmaxf(m, m2);
  if (M == -INFINITY) return;
  s = s * __builtin_amdgcn_exp2f((m - M) * kLog2e) + s2 * __builtin_amdgcn_exp2f((m2 - M) * kLog2e);
  m = M;
}

}  // namespace dflash
