// Block attention: every query row of the block attends to the last min(P, W)
// committed positions (read from the layer's K/V ring) and to all k block rows,
// with no causal mask inside the block (hotdry blog: one forward fills the whole
// masked block; zhihu answer §4: parallel decoding inside a block; the drafter is
// all sliding-window attention with window W).
//
// Workgroup = (key split, kv head g, sequence b, row block).  Query rows are the
// G = Hq/Hkv query heads of group g times the k block rows (<= 64 per row block),
// pre-scaled by 1/sqrt(dh) and held in LDS.  Keys stream through LDS in chunks of
// 32 with an online softmax; each thread owns a quarter of one query row's output.
// Long contexts are split over workgroups (flash-decoding); the last workgroup to
// finish a (b, g, row block) merges the partial (max, sum, output) triples in split
// order, so the result does not depend on arrival order.
#include "common.h"
#include "internal.h"

namespace dflash {

constexpr int kRows = 64;  // query rows per workgroup
constexpr int kKC = 32;    // keys per LDS chunk

template <typename T, int DH>
__global__ __launch_bounds__(kThreads) void attention_kernel(AttnArgs a) {
  constexpr int DQ = DH / 4;  // output dims per thread
  __shared__ float qs[kRows][DH + 1];
  __shared__ float ks[kKC][DH + 1];
  __shared__ float vs[kKC][DH];
  __shared__ float ps[kRows][kKC + 1];
  __shared__ int last_s;

  const int tid = threadIdx.x;
  const int split = blockIdx.x, g = blockIdx.y;
  const int b = blockIdx.z / a.n_rb, rb = blockIdx.z % a.n_rb;
  const int k = a.block_k, G = a.n_q_heads / a.n_kv_heads;
  const int P = max(a.ctx_len[b], 0);
  const int n_ctx = min(P, a.window);
  const int n_keys = n_ctx + k;
  const int n_split_b = (n_keys + a.keys_per_split - 1) / a.keys_per_split;
  if (split >= n_split_b) return;
  const int j0 = split * a.keys_per_split;
  const int j1 = min(n_keys, j0 + a.keys_per_split);
  const int R = G * k;
  const int r0 = rb * kRows;
  const int nr = min(kRows, R - r0);

  const T* qg = static_cast<const T*>(a.q);
  const T* kbg = static_cast<const T*>(a.kb);
  const T* vbg = static_cast<const T*>(a.vb);
  const size_t seq_base = (static_cast<size_t>(b) * a.n_kv_heads + g) * a.cache_slots;
  const T* ck = static_cast<const T*>(a.cache_k) + seq_base * DH;
  const T* cv = static_cast<const T*>(a.cache_v) + seq_base * DH;

  // query rows: row r -> head g*G + r / k, block row r % k
  const float scale = 1.f / sqrtf(static_cast<float>(DH));
  for (int idx = tid; idx < kRows * DH; idx += kThreads) {
    const int rr = idx / DH, d = idx % DH;
    float v = 0.f;
    if (rr < nr) {
      const int r = r0 + rr, hl = r / k, i = r % k;
      v = to_f32(qg[((static_cast<size_t>(b) * k + i) * a.n_q_heads + g * G + hl) * DH + d]) * scale;
    }
    qs[rr][d] = v;
  }

  const int rr = tid >> 2, qd = tid & 3;  // this thread: query row rr, dims qd*DQ ..
  float o[DQ];
#pragma unroll
  for (int d = 0; d < DQ; ++d) o[d] = 0.f;
  float m_run = -INFINITY, l_run = 0.f;

  for (int c0 = j0; c0 < j1; c0 += kKC) {
    const int nc = min(kKC, j1 - c0);
    __syncthreads();  // previous chunk fully consumed (and qs written on entry)
    for (int idx = tid; idx < kKC * DH; idx += kThreads) {
      const int jj = idx / DH, d = idx % DH;
      float kv = 0.f, vv = 0.f;
      if (jj < nc) {
        const int j = c0 + jj;
        if (j < n_ctx) {
          const int slot = (P - n_ctx + j) % a.cache_slots;
          kv = to_f32(ck[static_cast<size_t>(slot) * DH + d]);
          vv = to_f32(cv[static_cast<size_t>(slot) * DH + d]);
        } else {
          const size_t row = (static_cast<size_t>(b) * k + (j - n_ctx)) * a.n_kv_heads + g;
          kv = to_f32(kbg[row * DH + d]);
          vv = to_f32(vbg[row * DH + d]);
        }
      }
      ks[jj][d] = kv;
      vs[jj][d] = vv;
    }
    __syncthreads();

    // scores of row rr against keys qd, qd+4, ..
    float sc[kKC / 4];
    float cmax = -INFINITY;
#pragma unroll
    for (int t = 0; t < kKC / 4; ++t) {
      const int jj = qd + 4 * t;
      float s = -INFINITY;
      if (jj < nc) {
        s = 0.f;
        for (int d = 0; d < DH; ++d) s += qs[rr][d] * ks[jj][d];
      }
      sc[t] = s;
      cmax = fmaxf(cmax, s);
    }
    cmax = fmaxf(cmax, __shfl_xor(cmax, 1, kWave));
    cmax = fmaxf(cmax, __shfl_xor(cmax, 2, kWave));
    const float m_new = fmaxf(m_run, cmax);
    const float corr = expf(m_run - m_new);  // m_run = -inf on the first chunk -> 0
    float psum = 0.f;
#pragma unroll
    for (int t = 0; t < kKC / 4; ++t) {
      const float pj = (qd + 4 * t < nc) ? expf(sc[t] - m_new) : 0.f;
      ps[rr][qd + 4 * t] = pj;
      psum += pj;
    }
    psum += __shfl_xor(psum, 1, kWave);
    psum += __shfl_xor(psum, 2, kWave);
    l_run = l_run * corr + psum;
    m_run = m_new;
#pragma unroll
    for (int d = 0; d < DQ; ++d) o[d] *= corr;
    __syncthreads();
    for (int jj = 0; jj < nc; ++jj) {
      const float pj = ps[rr][jj];
#pragma unroll
      for (int d = 0; d < DQ; ++d) o[d] += pj * vs[jj][qd * DQ + d];
    }
  }

  T* out = static_cast<T*>(a.out);
  const int Hq = a.n_q_heads;
  if (n_split_b == 1) {
    if (rr < nr) {
      const int r = r0 + rr, hl = r / k, i = r % k;
      T* dst = out + ((static_cast<size_t>(b) * k + i) * Hq + g * G + hl) * DH + qd * DQ;
      const float inv = 1.f / l_run;
#pragma unroll
      for (int d = 0; d < DQ; ++d) dst[d] = from_f32<T>(o[d] * inv);
    }
    return;
  }

  // split: write the partial triple, the last workgroup merges
  const size_t grp = (static_cast<size_t>(b) * a.n_kv_heads + g) * a.n_rb + rb;
  {
    float* po = a.part_o + ((grp * a.max_splits + split) * kRows + rr) * DH + qd * DQ;
#pragma unroll
    for (int d = 0; d < DQ; ++d) po[d] = o[d];
    if (qd == 0) {
      float* pml = a.part_ml + ((grp * a.max_splits + split) * kRows + rr) * 2;
      pml[0] = m_run;
      pml[1] = l_run;
    }
  }
  __threadfence();
  __syncthreads();
  if (tid == 0) {
    const unsigned prev = atomicAdd(&a.counters[grp], 1u);
    last_s = (prev == static_cast<unsigned>(n_split_b - 1));
  }
  __syncthreads();
  if (!last_s) return;
  __threadfence();
  if (rr < nr) {
    float mx = -INFINITY;
    for (int s = 0; s < n_split_b; ++s)
      mx = fmaxf(mx, a.part_ml[((grp * a.max_splits + s) * kRows + rr) * 2]);
    float acc[DQ];
#pragma unroll
    for (int d = 0; d < DQ; ++d) acc[d] = 0.f;
    float lsum = 0.f;
    for (int s = 0; s < n_split_b; ++s) {
      const float* pml = a.part_ml + ((grp * a.max_splits + s) * kRows + rr) * 2;
      const float w = expf(pml[0] - mx);
      lsum += pml[1] * w;
      const float* po = a.part_o + ((grp * a.max_splits + s) * kRows + rr) * DH + qd * DQ;
#pragma unroll
      for (int d = 0; d < DQ; ++d) acc[d] += po[d] * w;
    }
    const int r = r0 + rr, hl = r / k, i = r % k;
    T* dst = out + ((static_cast<size_t>(b) * k + i) * Hq + g * G + hl) * DH + qd * DQ;
    const float inv = 1.f / lsum;
#pragma unroll
    for (int d = 0; d < DQ; ++d) dst[d] = from_f32<T>(acc[d] * inv);
  }
  if (tid == 0) atomicExch(&a.counters[grp], 0u);
}

template <typename T>
static hipError_t launch_dh(const AttnArgs& a, hipStream_t s) {
  const dim3 grid(a.max_splits, a.n_kv_heads, a.batch * a.n_rb);
  if (a.head_dim == 128) hipLaunchKernelGGL((attention_kernel<T, 128>), grid, dim3(kThreads), 0, s, a);
  else if (a.head_dim == 64) hipLaunchKernelGGL((attention_kernel<T, 64>), grid, dim3(kThreads), 0, s, a);
  else return hipErrorInvalidValue;
  return hipGetLastError();
}

hipError_t launch_attention(int elem_bytes, const AttnArgs& a, hipStream_t stream) {
  return elem_bytes == 2 ? launch_dh<bf16>(a, stream) : launch_dh<float>(a, stream);
}

}  // namespace dflash
