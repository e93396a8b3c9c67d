// Small kernels of the step: block construction, greedy verify + commit, and the
// committed-length update of a prefill injection.
#include <algorithm>

#include "common.h"
#include "internal.h"

namespace dflash {

// Block construction (hotdry blog, block-level masked parallel prediction): row 0
// of sequence b is the anchor's embedding at position P_b, rows 1..k-1 the mask
// embedding.  Writes the fp32 residual h, the first layer's RMSNorm input h*g and
// the row's sum of squares (one partial per row).
template <typename T>
__global__ __launch_bounds__(kThreads) void embed_kernel(EmbedArgs a) {
  typedef typename ActOf<T>::type TA;
  __shared__ float red[kThreads / kWave];
  const int m = blockIdx.x;
  int b = m / a.block_k, i = m % a.block_k;
  if (a.row_map != nullptr) {  // compacted block rows: row m is (b, i) of the map, if live
    if (m >= *a.m_live) return;
    const int e = a.row_map[m];
    b = e / a.block_k;
    i = e % a.block_k;
  }
  const int d = a.hidden;
  int tok = a.anchor[b];
  if (tok < 0 || tok >= a.vocab) {
    if (threadIdx.x == 0 && i == 0) atomicOr(a.dev_error, kErrToken);
    tok = min(max(tok, 0), a.vocab - 1);
  }
  if (threadIdx.x == 0 && i == 0 && a.ctx_len[b] < 0) atomicOr(a.dev_error, kErrCtxLen);
  const T* src = i == 0 ? static_cast<const T*>(a.embed) + static_cast<size_t>(tok) * d
                        : static_cast<const T*>(a.mask_embed);
  const T* gain = static_cast<const T*>(a.gain);
  TA* xa = static_cast<TA*>(a.xa);
  float* h = a.h + static_cast<size_t>(m) * d;
  const int steps = (d + kKStep - 1) / kKStep;
  // 8 consecutive features per thread and pass: one 16- (bf16) or 32-byte (fp32) load
  // of the row and of the gain, two 16-byte stores of h, and one store of the packed
  // operand (8 consecutive k of one row are contiguous in the fragment layout)
  typedef T T8 __attribute__((ext_vector_type(8)));
  typedef TA TA8 __attribute__((ext_vector_type(8)));
  float ss = 0.f;
  bool bad = false;
  for (int n0 = threadIdx.x * 8; n0 < d; n0 += kThreads * 8) {  // d is a multiple of 64
    const T8 sv = *reinterpret_cast<const T8*>(src + n0);
    const T8 gv = *reinterpret_cast<const T8*>(gain + n0);
    float v[8];
    TA8 out;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      v[j] = to_f32(static_cast<T>(sv[j]));
      out[j] = to_act<TA>(v[j] * to_f32(static_cast<T>(gv[j])), bad);
      ss += v[j] * v[j];
    }
    reinterpret_cast<float4*>(h + n0)[0] = make_float4(v[0], v[1], v[2], v[3]);
    reinterpret_cast<float4*>(h + n0)[1] = make_float4(v[4], v[5], v[6], v[7]);
    *reinterpret_cast<TA8*>(xa + pa_index(m, n0, steps)) = out;
  }
  report_overflow(bad, a.dev_error);
  ss = wave_sum(ss);
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = ss;
  __syncthreads();
  if (threadIdx.x == 0) {
    float t = 0.f;
    for (int w = 0; w < kThreads / kWave; ++w) t += red[w];
    a.ssq[m] = t;
  }
}

// Compaction of the block rows: an exclusive scan of the clamped block lengths in
// chunks of kCompactThreads sequences (wavefront scans, then one across the
// wavefronts), then each sequence's (b, i) entries of the row map.
constexpr int kCompactThreads = 1024;
__global__ __launch_bounds__(kCompactThreads) void compact_rows_kernel(CompactArgs a) {
  __shared__ int wave_tot[kCompactThreads / kWave];
  __shared__ int carry_s;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  if (tid == 0) carry_s = 0;
  __syncthreads();
  for (int base = 0; base < a.batch; base += kCompactThreads) {
    const int b = base + tid;
    const int raw = b < a.batch ? a.counts[b] : 0;
    if (raw < 0 || raw > a.rows_per_seq) atomicOr(a.dev_error, a.err_bit);
    const int kb = min(max(raw, 0), a.rows_per_seq);
    int incl = kb;  // inclusive scan within the wavefront
#pragma unroll
    for (int o = 1; o < kWave; o <<= 1) {
      const int v = __shfl_up(incl, o, kWave);
      if (lane >= o) incl += v;
    }
    if (lane == kWave - 1) wave_tot[w] = incl;
    __syncthreads();
    int before = carry_s;
    for (int j = 0; j < w; ++j) before += wave_tot[j];
    const int row0 = before + incl - kb;
    if (b < a.batch) {
      a.seq_row0[b] = row0;
      for (int i = 0; i < kb; ++i) a.row_map[row0 + i] = b * a.rows_per_seq + i;
    }
    __syncthreads();  // every thread has read carry_s and wave_tot
    if (tid == kCompactThreads - 1) carry_s = row0 + kb;
    __syncthreads();
  }
  if (tid == 0) a.seq_row0[a.batch] = carry_s;
}

hipError_t launch_compact_rows(const CompactArgs& a, hipStream_t stream) {
  if (a.batch <= 0 || a.rows_per_seq <= 0) return hipErrorInvalidValue;
  hipLaunchKernelGGL(compact_rows_kernel, dim3(1), dim3(kCompactThreads), 0, stream, a);
  return hipGetLastError();
}

// One thread per 16 bytes of the packed output, in output order: a wavefront writes one
// contiguous 1 KB fragment (16 rows x 32 k) and reads 16 row pieces of 64 bytes.
__global__ __launch_bounds__(kThreads) void pack_taps_kernel(PackTapsArgs a) {
  const long long idx = static_cast<long long>(blockIdx.x) * kThreads + threadIdx.x;
  const int lane = static_cast<int>(idx & 63);
  const long long frag = idx >> 6;  // (row block, k step)
  const int mb = static_cast<int>(frag / a.steps), st = static_cast<int>(frag % a.steps);
  const int m = mb * 16 + (lane & 15);
  if (m >= a.rows || (a.m_live != nullptr && m >= *a.m_live)) return;
  const int row = a.row_map != nullptr ? a.row_map[m] : m;
  const int k = st * kKStep + 8 * (lane >> 4);
  const uint4 v = *reinterpret_cast<const uint4*>(static_cast<const bf16*>(a.taps) + static_cast<size_t>(row) * a.lda + k);
  *reinterpret_cast<uint4*>(static_cast<bf16*>(a.out) + pa_index(m, k, a.steps)) = v;
}

hipError_t launch_pack_taps(const PackTapsArgs& a, hipStream_t stream) {
  if (a.rows <= 0 || a.steps <= 0 || a.lda < a.steps * kKStep || a.lda % 8 != 0) return hipErrorInvalidValue;
  const long long n = static_cast<long long>((a.rows + 15) / 16) * a.steps * kWave;
  const long long blocks = (n + kThreads - 1) / kThreads;
  if (blocks > (1ll << 31) - 1) return hipErrorInvalidValue;
  hipLaunchKernelGGL(pack_taps_kernel, dim3(static_cast<unsigned>(blocks)), dim3(kThreads), 0, stream, a);
  return hipGetLastError();
}

__global__ __launch_bounds__(kThreads) void rope_table_kernel(RopeTabArgs a) {
  const int half = a.head_dim / 2;
  const long long n = static_cast<long long>(a.batch) * a.rows_per_seq * half;
  const long long idx = static_cast<long long>(blockIdx.x) * kThreads + threadIdx.x;
  if (idx >= n) return;
  const int d = static_cast<int>(idx % half);
  const long long row = idx / half;
  const int b = static_cast<int>(row / a.rows_per_seq), i = static_cast<int>(row % a.rows_per_seq);
  float sn, cs;
  rope_sincos(max(a.ctx_len[b], 0) + i, rope_inv_freq(d, a.head_dim, a.theta), &sn, &cs);
  a.tab[idx] = make_float2(sn, cs);
}

hipError_t launch_rope_table(const RopeTabArgs& a, hipStream_t stream) {
  if (a.batch <= 0 || a.rows_per_seq <= 0 || a.head_dim < 2) return hipErrorInvalidValue;
  const long long n = static_cast<long long>(a.batch) * a.rows_per_seq * (a.head_dim / 2);
  const long long blocks = (n + kThreads - 1) / kThreads;
  if (blocks > (1ll << 31) - 1) return hipErrorInvalidValue;
  hipLaunchKernelGGL(rope_table_kernel, dim3(static_cast<unsigned>(blocks)), dim3(kThreads), 0, stream, a);
  return hipGetLastError();
}

hipError_t launch_embed(bool f32, const EmbedArgs& a, hipStream_t stream) {
  const dim3 grid(a.batch * a.block_k);
  if (!f32) hipLaunchKernelGGL(embed_kernel<bf16>, grid, dim3(kThreads), 0, stream, a);
  else hipLaunchKernelGGL(embed_kernel<float>, grid, dim3(kThreads), 0, stream, a);
  return hipGetLastError();
}

// Greedy verification (zhihu answer §2: accept until the first error; the target
// takes over there).  One wavefront per sequence: lane i tests draft[i] ==
// target[i]; the accepted length is the length of the all-true prefix, i.e. the
// index of the first zero of the ballot mask (an AND prefix scan over the block).
// The bonus token target[a] becomes the next anchor and the committed length moves
// past it; the ring rows of rejected positions stay behind as dead rows.
__global__ __launch_bounds__(kThreads) void verify_kernel(VerifyArgs a) {
  const int lane = threadIdx.x & 63;
  const int b = blockIdx.x * (kThreads / kWave) + (threadIdx.x >> 6);
  if (b >= a.batch) return;
  const int k = a.block_k;
  const int32_t* dr = a.draft + static_cast<size_t>(b) * k;
  const int32_t* tg = a.target + static_cast<size_t>(b) * (k + 1);
  int kb = k;  // drafts of this sequence's block
  if (a.block_len != nullptr) {
    kb = a.block_len[b];
    if ((kb < 0 || kb > k) && lane == 0) atomicOr(a.dev_error, kErrBlock);
    kb = min(max(kb, 0), k);
  }
  bool bad = false;
  int t = 0;
  if (lane <= k) {
    t = tg[lane];
    if (t < 0 || t >= a.vocab) { bad = true; t = min(max(t, 0), a.vocab - 1); }
  }
  bool match = false;
  if (lane < kb) {
    int dv = dr[lane];
    if (dv < 0 || dv >= a.vocab) { bad = true; dv = min(max(dv, 0), a.vocab - 1); }
    match = (dv == t);
  }
  const unsigned long long ones = __ballot(match);
  // lanes >= kb never match, so the first zero bit is at most kb
  const int acc = __ffsll(static_cast<long long>(~ones)) - 1;
  const int bonus = __shfl(t, acc, kWave);
  if (lane <= k) a.out_tokens[static_cast<size_t>(b) * (k + 1) + lane] = lane <= acc ? t : -1;
  if (__ballot(bad) != 0ull && lane == 0) atomicOr(a.dev_error, kErrToken);
  if (lane == 0) {
    const int P = a.ctx_len[b];
    if (P < 0) atomicOr(a.dev_error, kErrCtxLen);
    a.accept_len[b] = acc;
    a.anchor[b] = bonus;
    a.ctx_len[b] = max(P, 0) + acc + 1;
  }
}

hipError_t launch_verify(const VerifyArgs& a, hipStream_t stream) {
  const dim3 grid((a.batch + 3) / 4);
  hipLaunchKernelGGL(verify_kernel, grid, dim3(kThreads), 0, stream, a);
  return hipGetLastError();
}

// Runtime block-size controller, one thread per sequence (the hotdry blog's dynamic
// fallback; rungs full k, half k/2, off).  The moving average is float32 with every
// operation rounded separately (no contraction into fused multiply-adds), so the
// rung decisions taken from it are reproducible operation by operation.
__global__ void adapt_kernel(AdaptArgs a) {
#pragma clang fp contract(off)
  const int b = blockIdx.x * blockDim.x + threadIdx.x;
  if (b >= a.batch) return;
  const int full = a.block_k, h = a.block_k / 2;
  const int half = (h > 0 && h < full) ? h : 0;  // 0: no middle rung
  int kb = a.block_len[b];
  if (kb < 0 || kb > full) {
    atomicOr(a.dev_error, kErrBlock);
    kb = min(max(kb, 0), full);
  }
  float m = a.ema[b];
  int off = a.off_left[b];
  if (kb == 0) {
    off -= 1;
    if (off <= 0) {
      kb = half > 0 ? half : full;
      m = a.theta_down;
      off = 0;
    }
  } else {
    const int acc = min(max(a.accept_len[b], 0), kb);
    // correctly rounded division (hipcc's default), then products and sums kept
    // apart by the contract(off) pragma of this function
    const float scale = static_cast<float>(full) / static_cast<float>(kb);
    const float tau = 1.f + static_cast<float>(acc) * scale;
    const float step = a.alpha * (tau - m);
    m = m + step;
    if (kb == full) {
      if (m < a.theta_down) {
        if (half > 0) {
          kb = half;
        } else {
          kb = 0;
          off = a.cooldown;
        }
      }
    } else if (m < a.theta_off) {
      kb = 0;
      off = a.cooldown;
    } else if (m >= a.theta_up) {
      kb = full;
    }
  }
  a.block_len[b] = kb;
  a.ema[b] = m;
  a.off_left[b] = off;
}

hipError_t launch_adapt(const AdaptArgs& a, hipStream_t stream) {
  hipLaunchKernelGGL(adapt_kernel, dim3((a.batch + 255) / 256), dim3(256), 0, stream, a);
  return hipGetLastError();
}

__global__ void commit_rows_kernel(int32_t* ctx_len, const int32_t* n_rows, int batch, int n_max,
                                   uint32_t* dev_error) {
  const int b = blockIdx.x * blockDim.x + threadIdx.x;
  if (b >= batch) return;
  int n = n_rows[b];
  if (n < 0 || n > n_max) { atomicOr(dev_error, kErrRows); n = min(max(n, 0), n_max); }
  const int P = ctx_len[b];
  if (P < 0) atomicOr(dev_error, kErrCtxLen);
  ctx_len[b] = max(P, 0) + n;
}

hipError_t launch_commit_rows(int32_t* ctx_len, const int32_t* n_rows, int batch, int n_max,
                              uint32_t* dev_error, hipStream_t stream) {
  hipLaunchKernelGGL(commit_rows_kernel, dim3((batch + 255) / 256), dim3(256), 0, stream, ctx_len,
                     n_rows, batch, n_max, dev_error);
  return hipGetLastError();
}

// Debug poisoning of the ring slots no window reaches: one workgroup per (layer,
// sequence, kv head) fills the rows of positions ctx_len .. ctx_len + n_dead - 1.
__global__ __launch_bounds__(kThreads) void poison_ring_kernel(PoisonRingArgs a) {
  const int item = blockIdx.x;  // (layer * B + b) * Hkv + head
  const int b = (item / a.n_kv_heads) % a.batch;
  const int P = max(a.ctx_len[b], 0);
  const int per_row = a.row_bytes / 16;
  const size_t base = static_cast<size_t>(item) * a.cache_slots * a.row_bytes;
  const uint4 ones = make_uint4(~0u, ~0u, ~0u, ~0u);
  for (int t = threadIdx.x; t < a.n_dead * per_row; t += blockDim.x) {
    const int p = P + t / per_row;
    const int slot = p < a.sink ? p : a.sink + (p - a.sink) % (a.cache_slots - a.sink);
    const size_t off = base + static_cast<size_t>(slot) * a.row_bytes + (t % per_row) * 16;
    *reinterpret_cast<uint4*>(static_cast<char*>(a.cache_k) + off) = ones;
    *reinterpret_cast<uint4*>(static_cast<char*>(a.cache_v) + off) = ones;
  }
}

hipError_t launch_poison_ring(const PoisonRingArgs& a, hipStream_t stream) {
  const long long items = static_cast<long long>(a.n_layers) * a.batch * a.n_kv_heads;
  if (a.n_dead <= 0 || items <= 0) return hipSuccess;
  hipLaunchKernelGGL(poison_ring_kernel, dim3(static_cast<unsigned>(items)), dim3(kThreads), 0, stream, a);
  return hipGetLastError();
}

// Fill of 16-byte words with one value (a kernel, not hipMemsetAsync, so callers may
// capture it into a graph).
__global__ __launch_bounds__(kThreads) void fill_kernel(uint4* p, size_t n, unsigned v) {
  const uint4 w = make_uint4(v, v, v, v);
  for (size_t i = static_cast<size_t>(blockIdx.x) * blockDim.x + threadIdx.x; i < n;
       i += static_cast<size_t>(gridDim.x) * blockDim.x)
    p[i] = w;
}

static hipError_t launch_fill(void* p, size_t bytes, unsigned v, hipStream_t stream) {
  const size_t n = bytes / 16;
  if (n == 0) return hipSuccess;
  const size_t blocks = std::min<size_t>((n + kThreads - 1) / kThreads, 4096);
  hipLaunchKernelGGL(fill_kernel, dim3(static_cast<unsigned>(blocks)), dim3(kThreads), 0, stream,
                     static_cast<uint4*>(p), n, v);
  return hipGetLastError();
}

hipError_t launch_fill_ones(void* p, size_t bytes, hipStream_t stream) { return launch_fill(p, bytes, ~0u, stream); }
hipError_t launch_fill_zero(void* p, size_t bytes, hipStream_t stream) { return launch_fill(p, bytes, 0u, stream); }

}  // namespace dflash
