// Target stand-in for benchmarks (not part of libdflash): plants the target's
// tokens from the device drafts so that exactly a* drafts of each sequence are
// accepted, with a* taken from a precomputed per-step table (clipped to the
// sequence's block length when per-sequence block lengths are in use; the kernel
// then also writes each sequence's injection row count k_b + 1, as a serving
// runtime would).  This replaces the
// target model's verify forward, which needs trained weights.
//   T[i] = draft[i] for i < a*;  T[a*] = a token different from draft[a*] when
//   a* < k;  every other entry (and the bonus T[k] when a* = k) is filler.
// It also accumulates the accepted lengths of the previous step into a 64-bit
// running total, so a timed run can report accepted tokens without host syncs.
#include <hip/hip_runtime.h>
#include <stdint.h>

extern "C" {

constexpr int kPlantThreads = 1024;

// sum of accept_len[0 .. batch) over the workgroup (kPlantThreads threads)
__device__ long long block_sum(const int32_t* accept_len, int batch) {
  __shared__ long long part[kPlantThreads / 64];
  long long v = 0;
  for (int b = threadIdx.x; b < batch; b += blockDim.x) v += accept_len[b];
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
  if ((threadIdx.x & 63) == 0) part[threadIdx.x >> 6] = v;
  __syncthreads();
  long long t = 0;
  for (int w = 0; w < kPlantThreads / 64; ++w) t += part[w];
  return t;
}

__global__ __launch_bounds__(kPlantThreads) void plant_kernel(const int32_t* draft, int32_t* target, const int32_t* a_star_tab,
                             const int32_t* fill_tab, int32_t* step_counter, int n_tab_steps,
                             const int32_t* accept_len, long long* accept_total, const int32_t* block_len,
                             int32_t* n_rows_out, long long* kb_total, int batch, int k, int vocab) {
  __shared__ int step_s;
  if (threadIdx.x == 0) step_s = step_counter[0];
  __syncthreads();
  const int s = step_s % n_tab_steps;
  for (int idx = threadIdx.x; idx < batch * (k + 1); idx += blockDim.x) {
    const int b = idx / (k + 1), i = idx % (k + 1);
    const int kb = block_len != nullptr ? min(max(block_len[b], 0), k) : k;
    const int a = min(min(max(a_star_tab[s * batch + b], 0), k), kb);
    const int f = fill_tab[(static_cast<long long>(s) * batch + b) * (k + 1) + i];
    int t;
    if (i < a) t = draft[b * k + i];
    else if (i == a && a < kb) t = (draft[b * k + i] + 1 + f % (vocab - 1)) % vocab;
    else t = f % vocab;
    target[idx] = t;
    if (i == 0 && n_rows_out != nullptr) n_rows_out[b] = kb + 1;
  }
  const long long add = block_sum(accept_len, batch);
  __syncthreads();
  const long long kbs = block_len != nullptr ? block_sum(block_len, batch) : 0;
  if (threadIdx.x == 0) {
    accept_total[0] += add;
    step_counter[0] = step_s + 1;
    if (kb_total != nullptr) kb_total[0] += kbs;
  }
}

// Stand-in for sampled verification: target [B, k+1, V] holds filler logits.  Each
// step first restores the entries the previous step planted, then, per sequence,
// sets t[i, draft[i]] = +1e4 for i < a* (the draft gets probability ~1: accepted)
// and t[a*, draft[a*]] = -1e4 when a* < k (probability 0: rejected), so exactly a*
// drafts are accepted at any temperature up to 100.  Advances *rng_step (the device
// step word the sampled calls read) and accumulates accepted lengths like
// plant_kernel.
__global__ __launch_bounds__(kPlantThreads) void plant_logits_kernel(const int32_t* draft, float* target, const int32_t* a_star_tab,
                                    int32_t* step_counter, int n_tab_steps, int32_t* saved_idx,
                                    float* saved_val, const int32_t* accept_len, long long* accept_total,
                                    unsigned long long* rng_step, const int32_t* block_len, int32_t* n_rows_out,
                                    long long* kb_total, int batch, int k, int vocab) {
  __shared__ int step_s;
  if (threadIdx.x == 0) step_s = step_counter[0];
  __syncthreads();
  const int s = step_s % n_tab_steps;
  for (int idx = threadIdx.x; idx < batch * (k + 1); idx += blockDim.x) {
    const int b = idx / (k + 1), i = idx % (k + 1);
    float* row = target + static_cast<size_t>(idx) * vocab;
    const int old = saved_idx[idx];
    if (old >= 0 && old < vocab) row[old] = saved_val[idx];
    const int kb = block_len != nullptr ? min(max(block_len[b], 0), k) : k;
    const int a = min(min(max(a_star_tab[s * batch + b], 0), k), kb);
    if (i == 0 && n_rows_out != nullptr) n_rows_out[b] = kb + 1;
    int x = -1;
    if (i < kb && i <= a) {
      x = min(max(draft[b * k + i], 0), vocab - 1);
      saved_val[idx] = row[x];
      row[x] = i < a ? 1.0e4f : -1.0e4f;
    }
    saved_idx[idx] = x;
  }
  const long long add = block_sum(accept_len, batch);
  __syncthreads();
  const long long kbs = block_len != nullptr ? block_sum(block_len, batch) : 0;
  if (threadIdx.x == 0) {
    accept_total[0] += add;
    step_counter[0] = step_s + 1;
    if (rng_step != nullptr) rng_step[0] += 1ull;
    if (kb_total != nullptr) kb_total[0] += kbs;
  }
}

int dflash_harness_plant_logits(const int32_t* draft, float* target, const int32_t* a_star_tab,
                                int32_t* step_counter, int n_tab_steps, int32_t* saved_idx, float* saved_val,
                                const int32_t* accept_len, long long* accept_total,
                                unsigned long long* rng_step, const int32_t* block_len, int32_t* n_rows_out,
                                long long* kb_total, int batch, int k, int vocab, hipStream_t stream) {
  if (batch < 1 || k < 1 || vocab < 2 || n_tab_steps < 1) return -1;
  hipLaunchKernelGGL(plant_logits_kernel, dim3(1), dim3(kPlantThreads), 0, stream, draft, target, a_star_tab,
                     step_counter, n_tab_steps, saved_idx, saved_val, accept_len, accept_total, rng_step,
                     block_len, n_rows_out, kb_total, batch, k, vocab);
  return hipGetLastError() == hipSuccess ? 0 : -4;
}

int dflash_harness_plant(const int32_t* draft, int32_t* target, const int32_t* a_star_tab,
                         const int32_t* fill_tab, int32_t* step_counter, int n_tab_steps,
                         const int32_t* accept_len, long long* accept_total, const int32_t* block_len,
                         int32_t* n_rows_out, long long* kb_total, int batch, int k, int vocab,
                         hipStream_t stream) {
  if (batch < 1 || k < 1 || vocab < 2 || n_tab_steps < 1) return -1;
  hipLaunchKernelGGL(plant_kernel, dim3(1), dim3(kPlantThreads), 0, stream, draft, target, a_star_tab,
                     fill_tab, step_counter, n_tab_steps, accept_len, accept_total, block_len, n_rows_out,
                     kb_total, batch, k, vocab);
  return hipGetLastError() == hipSuccess ? 0 : -4;
}

}  // extern "C"
