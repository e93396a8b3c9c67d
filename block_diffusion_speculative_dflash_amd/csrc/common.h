// Shared device helpers for the gfx950 kernels: element types, 8-element MFMA
// fragments, conversions, wavefront reductions, the RoPE rotation.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace dflash {

typedef __bf16 bf16;
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16;
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int kWave = 64;
constexpr int kThreads = 256;  // 4 wavefronts per workgroup everywhere

__device__ __forceinline__ float to_f32(float x) { return x; }
__device__ __forceinline__ float to_f32(bf16 x) { return static_cast<float>(x); }
__device__ __forceinline__ float to_f32(f16 x) { return static_cast<float>(x); }

// round to nearest even
template <typename T> __device__ __forceinline__ T from_f32(float x);
template <> __device__ __forceinline__ float from_f32<float>(float x) { return x; }
template <> __device__ __forceinline__ bf16 from_f32<bf16>(float x) { return static_cast<bf16>(x); }
template <> __device__ __forceinline__ f16 from_f32<f16>(float x) { return static_cast<f16>(x); }

// Device-detected error bits (the DFLASH_DEVERR_* values of the C header).
constexpr uint32_t kErrToken = 1u, kErrRows = 2u, kErrCtxLen = 4u, kErrRange = 8u, kErrBlock = 16u,
                   kErrOverflow = 32u, kErrTimeout = 64u;

// Bound of every spin-wait on other workgroups (polls with a ~100-cycle sleep, about
// a quarter of a second in all): a wait that runs out sets kErrTimeout and the kernel
// exits rather than hang.
constexpr long long kSpinLimit = 1ll << 22;

// Conversion of an activation, q/k/v or K/V value to the compute type.  For fp16 a
// finite value beyond the largest finite fp16 (65504) saturates to +-65504 instead
// of becoming an infinity, and a value that is not finite passes through; both set
// `bad`, which the caller reports as kErrOverflow.  fp32 values pass unchanged.
// Selects, not branches: an epilogue converts dozens of values per lane.
template <typename T> __device__ __forceinline__ T to_act(float x, bool& bad);
template <> __device__ __forceinline__ float to_act<float>(float x, bool&) { return x; }
template <> __device__ __forceinline__ f16 to_act<f16>(float x, bool& bad) {
  const float a = fabsf(x);
  bad = bad || !(a <= 65504.f);
  return static_cast<f16>(a > 65504.f ? copysignf(65504.f, x) : x);  // NaN stays NaN
}
__device__ __forceinline__ void report_overflow(bool bad, uint32_t* dev_error) {
  if (bad && dev_error != nullptr) atomicOr(dev_error, kErrOverflow);
}

// Sum over each aligned group of 8 lanes (every lane of the group gets it): DPP
// quad permutations for the pairs and quads, then the half-row mirror for the other
// quad of the 8.  The same additions, in the same pairing, as an xor 1, 2, 4
// butterfly.
__device__ __forceinline__ float dpp_sum8(float x) {
  x += __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), 0xB1, 0xF, 0xF, true));   // quad_perm [1,0,3,2]
  x += __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), 0x4E, 0xF, 0xF, true));   // quad_perm [2,3,0,1]
  x += __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), 0x141, 0xF, 0xF, true));  // row_half_mirror
  return x;
}

// Activation / compute type of a drafter whose weights arrive as T: bf16 drafters
// compute in fp16, fp32 drafters in fp32.
template <typename T> struct ActOf;
template <> struct ActOf<bf16> { typedef f16 type; };
template <> struct ActOf<float> { typedef float type; };

// Element offset of (row m, reduction index k) in a fragment-packed operand:
// [m / 16][k / 32][lane][8] with lane = 16 * ((k % 32) / 8) + m % 16, i.e. one
// 32-wide K step of 16 rows is 64 lanes x 8 contiguous elements, exactly the
// MFMA operand a wavefront loads with one 16-byte load per lane.
__host__ __device__ __forceinline__ size_t pa_index(int m, int k, int ksteps) {
  return ((static_cast<size_t>(m >> 4) * ksteps + (k >> 5)) * 64 + (((k & 31) >> 3) * 16 + (m & 15))) * 8 +
         (k & 7);
}

// ---------------------------------------------------------------------------
// 8-element fragments.  One K-step of the GEMMs is 32 reduction elements: lane l
// of a wavefront holds 8 consecutive elements, rows/columns indexed by l % 16,
// reduction offset 8 * (l / 16).  A and B use the same lane -> k mapping, so
// any permutation of k inside one step still yields the full dot product.
// ---------------------------------------------------------------------------
template <typename T> struct Frag;

template <> struct Frag<bf16> {
  bf16x8 v;
  __device__ __forceinline__ void zero() {
    for (int i = 0; i < 8; ++i) v[i] = static_cast<bf16>(0.0f);
  }
  // 16-byte aligned vector load of 8 elements
  __device__ __forceinline__ void load(const bf16* p) { v = *reinterpret_cast<const bf16x8*>(p); }
  // element-wise load of the first `valid` elements, zeros after (any alignment)
  __device__ __forceinline__ void load_masked(const bf16* p, int valid) {
    for (int i = 0; i < 8; ++i) v[i] = (i < valid) ? p[i] : static_cast<bf16>(0.0f);
  }
  // acc[16x16] += A[16x32] * B[32x16]; lane holds A row (l%16) and B column (l%16)
  static __device__ __forceinline__ void mma(f32x4& acc, const Frag& a, const Frag& b) {
    acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a.v, b.v, acc, 0, 0, 0);
  }
};

template <> struct Frag<f16> {
  f16x8 v;
  __device__ __forceinline__ void zero() {
    for (int i = 0; i < 8; ++i) v[i] = static_cast<f16>(0.0f);
  }
  __device__ __forceinline__ void load(const f16* p) { v = *reinterpret_cast<const f16x8*>(p); }
  __device__ __forceinline__ void load_masked(const f16* p, int valid) {
    for (int i = 0; i < 8; ++i) v[i] = (i < valid) ? p[i] : static_cast<f16>(0.0f);
  }
  static __device__ __forceinline__ void mma(f32x4& acc, const Frag& a, const Frag& b) {
    acc = __builtin_amdgcn_mfma_f32_16x16x32_f16(a.v, b.v, acc, 0, 0, 0);
  }
};

template <> struct Frag<float> {
  float v[8];
  __device__ __forceinline__ void zero() {
    for (int i = 0; i < 8; ++i) v[i] = 0.0f;
  }
  __device__ __forceinline__ void load(const float* p) {
    const float4 a = reinterpret_cast<const float4*>(p)[0];
    const float4 b = reinterpret_cast<const float4*>(p)[1];
    v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w;
    v[4] = b.x; v[5] = b.y; v[6] = b.z; v[7] = b.w;
  }
  __device__ __forceinline__ void load_masked(const float* p, int valid) {
    for (int i = 0; i < 8; ++i) v[i] = (i < valid) ? p[i] : 0.0f;
  }
  // fp32 MFMA takes one reduction element per lane: eight 16x16x4 steps, step j
  // using element j of every lane, cover the lane's 8 elements.
  static __device__ __forceinline__ void mma(f32x4& acc, const Frag& a, const Frag& b) {
#pragma unroll
    for (int j = 0; j < 8; ++j) acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a.v[j], b.v[j], acc, 0, 0, 0);
  }
};

// ---------------------------------------------------------------------------
// wavefront reductions (64 lanes)
// ---------------------------------------------------------------------------
__device__ __forceinline__ float wave_sum(float x) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) x += __shfl_xor(x, o, kWave);
  return x;
}

// The value of the lane the DPP control CTRL selects (a permutation inside each row of
// 16 lanes).
template <int CTRL>
__device__ __forceinline__ float dpp_f32(float x) {
  return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), CTRL, 0xF, 0xF, true));
}
template <int CTRL>
__device__ __forceinline__ uint32_t dpp_u32(uint32_t x) {
  return static_cast<uint32_t>(__builtin_amdgcn_mov_dpp(static_cast<int>(x), CTRL, 0xF, 0xF, true));
}
// Max (min, sum) over the four lanes l, l^16, l^32, l^48 (gfx950 lane-group swaps:
// called with the same value as both operands, a swap leaves each lane its own value
// and its partner's).
__device__ __forceinline__ float lane_group_max(float x) {
  const unsigned u = __float_as_uint(x);
  const auto a = __builtin_amdgcn_permlane16_swap(u, u, false, false);
  const float y = fmaxf(__uint_as_float(a[0]), __uint_as_float(a[1]));
  const unsigned w = __float_as_uint(y);
  const auto b = __builtin_amdgcn_permlane32_swap(w, w, false, false);
  return fmaxf(__uint_as_float(b[0]), __uint_as_float(b[1]));
}
__device__ __forceinline__ float lane_group_sum(float x) {
  const unsigned u = __float_as_uint(x);
  const auto a = __builtin_amdgcn_permlane16_swap(u, u, false, false);
  const float y = __uint_as_float(a[0]) + __uint_as_float(a[1]);
  const unsigned w = __float_as_uint(y);
  const auto b = __builtin_amdgcn_permlane32_swap(w, w, false, false);
  return __uint_as_float(b[0]) + __uint_as_float(b[1]);
}
__device__ __forceinline__ uint32_t lane_group_min(uint32_t x) {
  const auto a = __builtin_amdgcn_permlane16_swap(x, x, false, false);
  const uint32_t y = min(static_cast<uint32_t>(a[0]), static_cast<uint32_t>(a[1]));
  const auto b = __builtin_amdgcn_permlane32_swap(y, y, false, false);
  return min(static_cast<uint32_t>(b[0]), static_cast<uint32_t>(b[1]));
}

// (value, index) max over the wavefront, ties to the smaller index; every lane gets
// it.  The max by DPP inside each row of 16 lanes (quad permutations xor 1 and xor 2,
// half-row mirror, row mirror) and the lane-group swaps across the four rows, then the
// smallest index among the lanes holding it the same way: no LDS round trips.  A NaN
// value is never picked (it counts as -inf).  Indices are non-negative.
__device__ __forceinline__ void wave_argmax(float& v, int& i) {
  const float x = v != v ? -INFINITY : v;
  float m = x;
  m = fmaxf(m, dpp_f32<0xB1>(m));
  m = fmaxf(m, dpp_f32<0x4E>(m));
  m = fmaxf(m, dpp_f32<0x141>(m));
  m = fmaxf(m, dpp_f32<0x140>(m));
  m = lane_group_max(m);
  uint32_t c = x == m ? static_cast<uint32_t>(i) : 0xFFFFFFFFu;
  c = min(c, dpp_u32<0xB1>(c));
  c = min(c, dpp_u32<0x4E>(c));
  c = min(c, dpp_u32<0x141>(c));
  c = min(c, dpp_u32<0x140>(c));
  c = lane_group_min(c);
  v = m;
  i = static_cast<int>(c);
}

// Order-preserving map of a float onto uint32 (larger float -> larger integer).
__device__ __forceinline__ uint32_t ordered_bits(float f) {
  const uint32_t u = __float_as_uint(f);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// 64-bit argmax key: value in the high word, (~index) in the low word, so the
// maximum key is the largest value and, among equal values, the smallest index.
__device__ __forceinline__ unsigned long long argmax_key(float v, int idx) {
  return (static_cast<unsigned long long>(ordered_bits(v)) << 32) |
         static_cast<unsigned long long>(0xFFFFFFFFu - static_cast<uint32_t>(idx));
}

__device__ __forceinline__ int argmax_key_index(unsigned long long key) {
  return static_cast<int>(0xFFFFFFFFu - static_cast<uint32_t>(key & 0xFFFFFFFFull));
}

// ---------------------------------------------------------------------------
// Cross-workgroup hand-off without cache maintenance.  Data another workgroup
// will read inside the same kernel is written with device-coherent (agent-scope)
// stores and read with device-coherent loads; the writer waits for its stores to
// complete before it bumps the arrival counter (an atomic), so the workgroup that
// sees the last arrival also sees every store.  Agent-scope fences, which write
// back and invalidate the L2 of the CU's XCD, are never used: at one per
// workgroup they cost more than the work itself.
// ---------------------------------------------------------------------------
__device__ __forceinline__ void coherent_store(float* p, float v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ float coherent_load(const float* p) {
  return __hip_atomic_load(const_cast<float*>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
// Two consecutive floats (8-byte aligned) in one device-coherent load.
__device__ __forceinline__ float2 coherent_load2(const float* p) {
  const unsigned long long u = __hip_atomic_load(reinterpret_cast<unsigned long long*>(const_cast<float*>(p)),
                                                 __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  return make_float2(__uint_as_float(static_cast<uint32_t>(u)), __uint_as_float(static_cast<uint32_t>(u >> 32)));
}
// 16 bytes as two device-coherent 8-byte loads / stores (the destination type V is
// any 16-byte vector), and a device-coherent 2-byte store.
template <typename V>
__device__ __forceinline__ V coherent_load16(const void* p) {
  static_assert(sizeof(V) == 16, "16-byte value");
  unsigned long long* q = reinterpret_cast<unsigned long long*>(const_cast<void*>(p));
  union {
    unsigned long long u[2];
    V v;
  } x;
  x.u[0] = __hip_atomic_load(q, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  x.u[1] = __hip_atomic_load(q + 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  return x.v;
}
template <typename V>
__device__ __forceinline__ void coherent_store16(void* p, const V& v) {
  static_assert(sizeof(V) == 16, "16-byte value");
  unsigned long long* q = reinterpret_cast<unsigned long long*>(p);
  union {
    unsigned long long u[2];
    V v;
  } x;
  x.v = v;
  __hip_atomic_store(q, x.u[0], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  __hip_atomic_store(q + 1, x.u[1], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void coherent_store(f16* p, f16 v) {
  __hip_atomic_store(reinterpret_cast<unsigned short*>(p), __builtin_bit_cast(unsigned short, v), __ATOMIC_RELAXED,
                     __HIP_MEMORY_SCOPE_AGENT);
}

// Stores and loads of data that another workgroup reads (or wrote) inside the same
// kernel launch: device-coherent when COH, plain otherwise.
template <bool COH, typename T>
__device__ __forceinline__ void put(T* p, T v) {
  if constexpr (COH) coherent_store(p, v);
  else *p = v;
}
template <bool COH>
__device__ __forceinline__ float get(const float* p) {
  if constexpr (COH) return coherent_load(p);
  else return *p;
}
template <bool COH, typename V>
__device__ __forceinline__ V get16(const void* p) {
  if constexpr (COH) return coherent_load16<V>(p);
  else return *reinterpret_cast<const V*>(p);
}
template <bool COH, typename V>
__device__ __forceinline__ void put16(void* p, const V& v) {
  if constexpr (COH) coherent_store16(p, v);
  else *reinterpret_cast<V*>(p) = v;
}

// All of this thread's memory operations have completed.
__device__ __forceinline__ void wait_memory() { __builtin_amdgcn_s_waitcnt(0); }
// Arrival counter: returns true in exactly one thread block, the last of `expected`.
__device__ __forceinline__ bool arrive_last(unsigned* counter, unsigned expected, int* flag_lds) {
  wait_memory();
  __syncthreads();
  if (threadIdx.x == 0) {
    const unsigned prev = __hip_atomic_fetch_add(counter, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    *flag_lds = prev == expected - 1;
  }
  __syncthreads();
  return *flag_lds != 0;
}
__device__ __forceinline__ void reset_counter(unsigned* counter) {
  __hip_atomic_store(counter, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// ---------------------------------------------------------------------------
// RoPE, rotate-half pairing (i, i + dh/2), angle pos * theta^(-2i/dh).  The angle
// is formed and reduced modulo 2*pi in double precision, because positions reach
// 2.6e5 where one float ulp of the angle is already 0.03 rad; sin/cos of the
// reduced angle are then taken in float.
// ---------------------------------------------------------------------------
__device__ __forceinline__ double rope_inv_freq(int i, int head_dim, float theta) {
  return pow(static_cast<double>(theta), -2.0 * static_cast<double>(i) / static_cast<double>(head_dim));
}

__device__ __forceinline__ void rope_sincos(int pos, double inv_freq, float* s, float* c) {
  const double two_pi = 6.283185307179586476925286766559;
  double a = static_cast<double>(pos) * inv_freq;
  a -= two_pi * floor(a / two_pi);
  sincosf(static_cast<float>(a), s, c);
}

}  // namespace dflash
