// Sampled (temperature > 0) verification and the drafter's per-row log-sum-exp.
//
// Rejection sampling as the aufer article's data-flow section names the target's
// check (the zhihu answer's §2 gives the draft / verify / accept loop, §6 the
// guarantee that the target's distribution is kept).  With q_i = softmax(z_i / T)
// the drafter's distribution at block row i, p_i = softmax(t_i / T) the target's:
// draft x_i is accepted while u_i q_i(x_i) <= p_i(x_i); at the first rejection a
// the emitted token is a draw from max(0, p_a - q_a) (from p_a if rounding left no
// positive entry); after k acceptances it is a draw from p_k.  Draws are Gumbel-max
// over Philox4x64-10 noise (philox.h).
//
// Two kernels, both reading the caller's fp32 logits once in chunks of 2048 G
// entries (G = 4, 2 or 1 groups of 8 per thread, each kernel taking the largest
// that still gives it >= 256 workgroups):
//  1. (chunk, row i <= k, sequence b): log-sum-exp partial of t_i / T; the last
//     workgroup of a row to arrive merges that row's partials, and the last row of
//     a sequence to finish runs the k acceptance tests in one wavefront (lane i,
//     ballot, first zero = a) -- two arrival levels, so no counter sees more than
//     max(n_chunks, k + 1) atomics;
//  2. (chunk, sequence b): the residual (or bonus) row a, scores + noise, split-vocab
//     argmax through keys; the last arriving workgroup commits: accepted length,
//     emitted tokens, anchor, committed length.
#include "common.h"
#include "internal.h"
#include "philox.h"

namespace dflash {

// LM-head finalisation, one workgroup per draft row: the draft is the largest of the
// column tiles' best keys (order-preserving value bits over the inverted index, so a
// tie goes to the lower index; -1 past the sequence's block length), and, when the
// tiles left (max, sum) pairs (sampling), the row's log-sum-exp merged in a fixed
// order.  The tiles store their keys with plain stores: no same-address atomics and no
// arrival counter in the LM head itself.
__global__ __launch_bounds__(kThreads) void head_finalize_kernel(HeadFinalizeArgs a) {
  __shared__ float red_m[kThreads / kWave], red_s[kThreads / kWave];
  __shared__ unsigned long long red_k[kThreads / kWave];
  const int tid = threadIdx.x, row = blockIdx.x;
  const int n_parts = a.n_parts;
  const bool in_block = a.block_len == nullptr || row % a.rows_per_seq < a.block_len[row / a.rows_per_seq];
  int krow = row;  // the row of the keys
  if (a.seq_row0 != nullptr) {  // compacted: only rows inside the block have keys
    if (!in_block) {
      if (tid == 0) a.draft[row] = -1;
      return;  // uniform per workgroup
    }
    krow = a.seq_row0[row / a.rows_per_seq] + row % a.rows_per_seq;
  }
  const unsigned long long* kp = a.keys + static_cast<size_t>(krow) * n_parts;
  unsigned long long best = 0ull;
  for (int t0 = tid; t0 < n_parts; t0 += 4 * kThreads) {
    unsigned long long v[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int t = t0 + u * kThreads;
      v[u] = t < n_parts ? kp[t] : 0ull;
    }
#pragma unroll
    for (int u = 0; u < 4; ++u) best = v[u] > best ? v[u] : best;
  }
  float m = -INFINITY, s = 0.f;
  if (a.part != nullptr) {
    const float2* p = a.part + static_cast<size_t>(krow) * n_parts;
    for (int t0 = tid; t0 < n_parts; t0 += 4 * kThreads) {
      float2 v[4];
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const int t = t0 + u * kThreads;
        v[u] = t < n_parts ? p[t] : make_float2(-INFINITY, 0.f);
      }
#pragma unroll
      for (int u = 0; u < 4; ++u) lse_merge(m, s, v[u].x, v[u].y);
    }
  }
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) {
    const unsigned long long ok = __shfl_xor(best, o, kWave);
    best = ok > best ? ok : best;
    const float om = __shfl_xor(m, o, kWave), os = __shfl_xor(s, o, kWave);
    lse_merge(m, s, om, os);
  }
  if ((tid & 63) == 0) {
    red_k[tid >> 6] = best;
    red_m[tid >> 6] = m;
    red_s[tid >> 6] = s;
  }
  __syncthreads();
  if (tid == 0) {
    for (int w = 1; w < kThreads / kWave; ++w) {
      best = red_k[w] > best ? red_k[w] : best;
      lse_merge(m, s, red_m[w], red_s[w]);
    }
    a.draft[row] = in_block ? argmax_key_index(best) : -1;
    if (a.part != nullptr) a.lse[row] = m + ln_f32(s);
  }
}

hipError_t launch_head_finalize(const HeadFinalizeArgs& a, hipStream_t stream) {
  if (a.rows <= 0 || a.n_parts <= 0 || (a.part != nullptr) != (a.lse != nullptr)) return hipErrorInvalidValue;
  hipLaunchKernelGGL(head_finalize_kernel, dim3(a.rows), dim3(kThreads), 0, stream, a);
  return hipGetLastError();
}

// Loads the n <= 8 logits row[v0 .. v0 + n) (v0 a multiple of 8); float4 pairs when
// rows are 16-byte aligned (vocab % 4 == 0), scalar loads otherwise.
__device__ __forceinline__ void load8(const float* row, int v0, int n, bool vec, float out[8]) {
  if (vec && n == 8) {
    const float4 a = *reinterpret_cast<const float4*>(row + v0);
    const float4 c = *reinterpret_cast<const float4*>(row + v0 + 4);
    out[0] = a.x; out[1] = a.y; out[2] = a.z; out[3] = a.w;
    out[4] = c.x; out[5] = c.y; out[6] = c.z; out[7] = c.w;
  } else {
#pragma unroll
    for (int e = 0; e < 8; ++e) out[e] = e < n ? row[v0 + e] : -INFINITY;
  }
}

// log-sum-exp of the partials pr[0 .. n) (device-coherent loads, four in flight per
// lane), reduced over one wavefront; every lane returns the result
__device__ __forceinline__ float wave_lse_of_partials(const float* pr, int n) {
  const int lane = threadIdx.x & 63;
  float m = -INFINITY, s = 0.f;
  for (int c0 = lane; c0 < n; c0 += 4 * kWave) {
    float2 v[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int c = c0 + u * kWave;
      v[u] = c < n ? coherent_load2(pr + 2 * c) : make_float2(-INFINITY, 0.f);
    }
#pragma unroll
    for (int u = 0; u < 4; ++u) lse_merge(m, s, v[u].x, v[u].y);
  }
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) {
    const float om = __shfl_xor(m, o, kWave), os = __shfl_xor(s, o, kWave);
    lse_merge(m, s, om, os);
  }
  return m + ln_f32(s);
}

template <int G>
__global__ __launch_bounds__(kThreads) void verify_lse_kernel(VerifySampledArgs a) {
  constexpr int kGroups = G, kChunk = 8 * kThreads * G;
  __shared__ float red_m[kThreads / kWave], red_s[kThreads / kWave];
  __shared__ int last_s;
  const int chunk = blockIdx.x, i = blockIdx.y, b = blockIdx.z, tid = threadIdx.x;
  const int k = a.block_k, V = a.vocab;
  const int kb = a.block_len != nullptr ? min(max(a.block_len[b], 0), k) : k;
  if (i > kb) return;  // target rows past the bonus row of this sequence's block: unused
  const bool vec = (V & 3) == 0;
  const float* trow_b = a.target_logits + static_cast<size_t>(b) * (k + 1) * V;
  const float* row = trow_b + static_cast<size_t>(i) * V;
  const int v0 = chunk * kChunk, v1 = min(V, v0 + kChunk);

  float vals[kGroups][8];
#pragma unroll
  for (int j = 0; j < kGroups; ++j) {
    const int vb = v0 + 8 * (tid + kThreads * j);
    load8(row, vb, max(0, min(8, v1 - vb)), vec, vals[j]);
  }
  float m = -INFINITY;
#pragma unroll
  for (int j = 0; j < kGroups; ++j)
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      vals[j][e] *= a.inv_temp;
      m = fmaxf(m, vals[j][e]);
    }
  float s = 0.f;
  if (m != -INFINITY) {
#pragma unroll
    for (int j = 0; j < kGroups; ++j)
#pragma unroll
      for (int e = 0; e < 8; ++e) s += __builtin_amdgcn_exp2f((vals[j][e] - m) * kLog2e);
  }
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) {
    const float om = __shfl_xor(m, o, kWave), os = __shfl_xor(s, o, kWave);
    lse_merge(m, s, om, os);
  }
  if ((tid & 63) == 0) {
    red_m[tid >> 6] = m;
    red_s[tid >> 6] = s;
  }
  __syncthreads();
  if (tid == 0) {
    for (int w = 1; w < kThreads / kWave; ++w) lse_merge(m, s, red_m[w], red_s[w]);
    float* dst = reinterpret_cast<float*>(a.part + (static_cast<size_t>(b) * (k + 1) + i) * a.n_chunks + chunk);
    coherent_store(dst, m);
    coherent_store(dst + 1, s);
  }
  unsigned* row_cnt = &a.counters[2 * a.batch + static_cast<size_t>(b) * (k + 1) + i];
  if (!arrive_last(row_cnt, static_cast<unsigned>(a.n_chunks), &last_s)) return;

  // last workgroup of row (b, i): the row's log-sum-exp
  if (tid < kWave) {
    const float* pr = reinterpret_cast<const float*>(a.part + (static_cast<size_t>(b) * (k + 1) + i) * a.n_chunks);
    const float l = wave_lse_of_partials(pr, a.n_chunks);
    if (tid == 0) {
      coherent_store(&a.row_lse[static_cast<size_t>(b) * (k + 1) + i], l);
      reset_counter(row_cnt);
    }
  }
  if (!arrive_last(&a.counters[b], static_cast<unsigned>(kb + 1), &last_s)) return;

  // last row of sequence b: the acceptance tests
  if (tid < kWave) {
    const int lane = tid;
    const float lse_t = lane <= kb ? coherent_load(&a.row_lse[static_cast<size_t>(b) * (k + 1) + lane]) : 0.f;
    bool ok = false, bad = false;
    if (lane < kb) {
      int x = a.draft[static_cast<size_t>(b) * k + lane];
      if (x < 0 || x >= V) { bad = true; x = min(max(x, 0), V - 1); }
      const float lp = trow_b[static_cast<size_t>(lane) * V + x] * a.inv_temp - lse_t;
      const float lq = a.draft_logits[(static_cast<size_t>(b) * k + lane) * V + x] * a.inv_temp -
                       a.draft_lse[static_cast<size_t>(b) * k + lane];
      uint32_t h[8];
      const unsigned long long step = a.step_dev != nullptr ? *a.step_dev : a.step;
      philox_u32x8(static_cast<unsigned>(lane), static_cast<unsigned>(b), step, 0ull, a.seed, kStreamAccept, h);
      ok = lp - lq - ln_uniform(h[0]) >= 0.f;  // u q(x) <= p(x)
    }
    const unsigned long long ones = __ballot(ok);
    const int acc = __ffsll(static_cast<long long>(~ones)) - 1;  // lanes >= kb never accept: acc <= kb
    const float lse_a = __shfl(lse_t, acc, kWave);
    if (__ballot(bad) != 0ull && lane == 0) atomicOr(a.dev_error, kErrToken);
    if (lane == 0) {
      if (a.block_len != nullptr && (a.block_len[b] < 0 || a.block_len[b] > k)) atomicOr(a.dev_error, kErrBlock);
      const float lq_a = acc < kb ? a.draft_lse[static_cast<size_t>(b) * k + acc] : 0.f;
      a.decision[b] = make_float4(static_cast<float>(acc), lse_a, lq_a, 0.f);
      reset_counter(&a.counters[b]);
    }
  }
}

template <int G>
__global__ __launch_bounds__(kThreads) void verify_emit_kernel(VerifySampledArgs a) {
  constexpr int kGroups = G, kChunk = 8 * kThreads * G;
  __shared__ unsigned long long red[2][kThreads / kWave];
  __shared__ int last_s, tok_s;
  const int chunk = blockIdx.x, b = blockIdx.y, tid = threadIdx.x, lane = tid & 63;
  const int k = a.block_k, V = a.vocab;
  const bool vec = (V & 3) == 0;
  const float4 dec = a.decision[b];
  const int kb = a.block_len != nullptr ? min(max(a.block_len[b], 0), k) : k;
  const int acc = min(max(static_cast<int>(dec.x), 0), kb);
  const bool resid = acc < kb;  // otherwise the bonus draw from target row kb
  const float lse_p = dec.y, lse_q = dec.z;
  const float* trow = a.target_logits + (static_cast<size_t>(b) * (k + 1) + acc) * V;
  const float* zrow = a.draft_logits + (static_cast<size_t>(b) * k + min(acc, k - 1)) * V;
  const int v0 = chunk * kChunk, v1 = min(V, v0 + kChunk);

  const unsigned long long step = a.step_dev != nullptr ? *a.step_dev : a.step;
  unsigned long long kr = 0ull, kp = 0ull;  // residual draw, draw from p itself
#pragma unroll
  for (int j = 0; j < kGroups; ++j) {
    const int vb = v0 + 8 * (tid + kThreads * j);
    const int n = max(0, min(8, v1 - vb));
    if (n == 0) continue;
    float tv[8], zv[8];
    load8(trow, vb, n, vec, tv);
    if (resid) load8(zrow, vb, n, vec, zv);
    uint32_t h[8];
    philox_u32x8(static_cast<unsigned>(vb >> 3), static_cast<unsigned>(b), step, 0ull, a.seed, kStreamEmit, h);
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      if (e >= n) continue;
      const int v = vb + e;
      const float g = gumbel_f32(h[e]);
      const float lp = tv[e] * a.inv_temp - lse_p;
      const unsigned long long kpe = argmax_key(lp + g, v);
      kp = kpe > kp ? kpe : kp;
      if (resid) {
        const float lq = zv[e] * a.inv_temp - lse_q;
        if (lp > lq) {  // log(p - q) = log p + log(1 - q / p)
          const float lr = lp + ln_f32(-expm1f(lq - lp));
          const unsigned long long kre = argmax_key(lr + g, v);
          kr = kre > kr ? kre : kr;
        }
      }
    }
  }
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) {
    const unsigned long long orr = __shfl_xor(kr, o, kWave), op = __shfl_xor(kp, o, kWave);
    kr = orr > kr ? orr : kr;
    kp = op > kp ? op : kp;
  }
  if (lane == 0) {
    red[0][tid >> 6] = kr;
    red[1][tid >> 6] = kp;
  }
  __syncthreads();
  unsigned long long* keys = a.keys + static_cast<size_t>(b) * 2 * kKeyStride;
  if (tid == 0) {
    for (int w = 1; w < kThreads / kWave; ++w) {
      kr = red[0][w] > kr ? red[0][w] : kr;
      kp = red[1][w] > kp ? red[1][w] : kp;
    }
    if (kr != 0ull) atomicMax(&keys[0], kr);
    if (kp != 0ull) atomicMax(&keys[kKeyStride], kp);
  }
  if (!arrive_last(&a.counters[a.batch + b], static_cast<unsigned>(a.n_chunks_emit), &last_s)) return;

  if (tid == 0) {
    const unsigned long long fr = __hip_atomic_exchange(&keys[0], 0ull, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    const unsigned long long fp =
        __hip_atomic_exchange(&keys[kKeyStride], 0ull, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    tok_s = argmax_key_index(resid && fr != 0ull ? fr : fp);
  }
  __syncthreads();
  const int y = tok_s;
  for (int t = tid; t <= k; t += kThreads) {
    int tok = -1;
    if (t < acc) tok = min(max(a.draft[static_cast<size_t>(b) * k + t], 0), V - 1);
    else if (t == acc) tok = y;
    a.out_tokens[static_cast<size_t>(b) * (k + 1) + t] = tok;
  }
  if (tid == 0) {
    const int P = a.ctx_len[b];
    if (P < 0) atomicOr(a.dev_error, kErrCtxLen);
    a.accept_len[b] = acc;
    a.anchor[b] = y;
    a.ctx_len[b] = max(P, 0) + acc + 1;
    reset_counter(&a.counters[a.batch + b]);
  }
}

hipError_t launch_verify_sampled(const VerifySampledArgs& a, hipStream_t stream) {
  if (a.batch <= 0 || a.block_k <= 0 || a.block_k >= kWave) return hipErrorInvalidValue;
  const long long rows_lse = static_cast<long long>(a.batch) * (a.block_k + 1);
  const int g1 = verify_groups(rows_lse, a.vocab), g2 = verify_groups(a.batch, a.vocab);
  if (a.n_chunks != verify_chunks(rows_lse, a.vocab) || a.n_chunks_emit != verify_chunks(a.batch, a.vocab))
    return hipErrorInvalidValue;
  const dim3 grid1(a.n_chunks, a.block_k + 1, a.batch), grid2(a.n_chunks_emit, a.batch);
  switch (g1) {
    case 1: hipLaunchKernelGGL(verify_lse_kernel<1>, grid1, dim3(kThreads), 0, stream, a); break;
    case 2: hipLaunchKernelGGL(verify_lse_kernel<2>, grid1, dim3(kThreads), 0, stream, a); break;
    default: hipLaunchKernelGGL(verify_lse_kernel<4>, grid1, dim3(kThreads), 0, stream, a); break;
  }
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  switch (g2) {
    case 1: hipLaunchKernelGGL(verify_emit_kernel<1>, grid2, dim3(kThreads), 0, stream, a); break;
    case 2: hipLaunchKernelGGL(verify_emit_kernel<2>, grid2, dim3(kThreads), 0, stream, a); break;
    default: hipLaunchKernelGGL(verify_emit_kernel<4>, grid2, dim3(kThreads), 0, stream, a); break;
  }
  return hipGetLastError();
}

}  // namespace dflash
