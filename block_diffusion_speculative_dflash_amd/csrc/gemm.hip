// Weight-streaming GEMM with fused epilogues: out[m, n] = sum_k A[m, k] * W[n, k].
//
// Every projection of the drafter is y = x W^T with W in nn.Linear layout.  At
// draft batch sizes the rows of x are few (B*k = 8 .. 72 at B <= 8), so the cost
// is reading W once from HBM.  One workgroup (4 wavefronts) owns a 64-column tile
// of the output and a K range; the four wavefronts take interleaved pairs of
// 32-element K steps, load W rows and x rows straight into MFMA fragments
// (16 x 16 x 32 bf16, or 16 x 16 x 4 fp32 eight times for fp32 drafters), and
// reduce their accumulators through LDS in a fixed order.  When the tile count
// alone cannot fill the 256 CUs, K is split across workgroups: each writes an
// fp32 partial tile, and the last to arrive (device-scope counter) sums the
// partials in split order, so results are bitwise reproducible.
//
// The epilogue then runs on the reduced 64-column tile in LDS and fuses what the
// method does next (RMSNorm scale of the input rows, RoPE, KV-ring scatter,
// residual add, SwiGLU, split-vocab argmax), so none of those becomes a separate
// launch.  RMSNorm is folded as out = (x*g) W^T * rsqrt(mean(x^2) + eps): the
// producer of x writes x*g and per-tile sums of x^2, the consumer applies the
// per-row factor to its accumulators, which is exact in real arithmetic because
// the projection is linear.
#include "common.h"
#include "internal.h"

namespace dflash {

// Weight row feeding local column c (0..63) of tile tile_n, or nullptr past N.
// QKV / INJECT tiles hold 32 RoPE pairs: column c < 32 is head dim sub*32 + c and
// column c + 32 is its rotate-half partner (dim + dh/2).  SWIGLU tiles hold 32
// gate rows then the 32 matching up rows.
template <typename T, int EPI>
__device__ __forceinline__ const T* b_row(const GemmArgs& g, int tile_n, int c) {
  const T* W = static_cast<const T*>(g.W);
  if constexpr (EPI == EPI_FUSE || EPI == EPI_RESID || EPI == EPI_ARGMAX) {
    const int n = tile_n * kBN + c;
    return n < g.N ? W + static_cast<size_t>(n) * g.ldw : nullptr;
  } else if constexpr (EPI == EPI_SWIGLU) {
    const int j = tile_n * (kBN / 2) + (c & 31);
    if (j >= g.ffn) return nullptr;
    return W + static_cast<size_t>(c < 32 ? j : g.ffn + j) * g.ldw;
  } else {
    const int tph = g.head_dim / kBN;  // tiles per head
    const int sub = tile_n % tph;
    const int dim = sub * 32 + (c & 31) + (c >> 5) * (g.head_dim / 2);
    if constexpr (EPI == EPI_QKV) {
      const int hd = tile_n / tph;
      return W + static_cast<size_t>(hd * g.head_dim + dim) * g.ldw;
    } else {
      const int hpl = 2 * g.n_kv_heads;  // K heads then V heads of one layer
      const int l = tile_n / (tph * hpl);
      const int hd = (tile_n / tph) % hpl;
      const size_t row = static_cast<size_t>(l) * (g.n_q_heads + 2 * g.n_kv_heads) * g.head_dim +
                         static_cast<size_t>(g.n_q_heads + hd) * g.head_dim + dim;
      return W + row * g.ldw;
    }
  }
}

template <typename T, int BM, int EPI, bool VEC>
__global__ __launch_bounds__(kThreads) void gemm_kernel(GemmArgs g) {
  constexpr int MT = BM / 16;
  constexpr int NT = kBN / 16;
  constexpr int U = 2;  // K steps per wavefront per iteration
  __shared__ float tile[BM][kBN + 4];
  __shared__ float rs_s[BM];
  __shared__ int last_s;

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int tile_n = blockIdx.x, tile_m = blockIdx.y, split = blockIdx.z;
  const int m0 = tile_m * BM;
  const T* A = static_cast<const T*>(g.A);

  const T* brow[NT];
#pragma unroll
  for (int ni = 0; ni < NT; ++ni) brow[ni] = b_row<T, EPI>(g, tile_n, ni * 16 + (lane & 15));
  const T* arow[MT];
#pragma unroll
  for (int mi = 0; mi < MT; ++mi) {
    const int m = m0 + mi * 16 + (lane & 15);
    arow[mi] = m < g.M ? A + static_cast<size_t>(m) * g.lda : nullptr;
  }

  const int kq = 8 * (lane >> 4);
  const int kb = split * g.k_split;
  const int ke = min(g.K, kb + g.k_split);
  const int nsteps = ke > kb ? (ke - kb + kKStep - 1) / kKStep : 0;

  f32x4 acc[MT][NT];
#pragma unroll
  for (int mi = 0; mi < MT; ++mi)
#pragma unroll
    for (int ni = 0; ni < NT; ++ni) acc[mi][ni] = f32x4{0.f, 0.f, 0.f, 0.f};

  for (int s0 = wave * U; s0 < nsteps; s0 += 4 * U) {
    Frag<T> fa[U][MT], fb[U][NT];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int s = s0 + u;
      const int k = kb + s * kKStep + kq;
      const int valid = ke - k;
      const bool full = VEC && (kb + (s + 1) * kKStep <= ke);
#pragma unroll
      for (int ni = 0; ni < NT; ++ni) {
        if (brow[ni] != nullptr && valid > 0) {
          if (full) fb[u][ni].load(brow[ni] + k);
          else fb[u][ni].load_masked(brow[ni] + k, min(valid, 8));
        } else {
          fb[u][ni].zero();
        }
      }
#pragma unroll
      for (int mi = 0; mi < MT; ++mi) {
        if (arow[mi] != nullptr && valid > 0) {
          if (full) fa[u][mi].load(arow[mi] + k);
          else fa[u][mi].load_masked(arow[mi] + k, min(valid, 8));
        } else {
          fa[u][mi].zero();
        }
      }
    }
#pragma unroll
    for (int u = 0; u < U; ++u)
#pragma unroll
      for (int mi = 0; mi < MT; ++mi)
#pragma unroll
        for (int ni = 0; ni < NT; ++ni) Frag<T>::mma(acc[mi][ni], fa[u][mi], fb[u][ni]);
  }

  // Cross-wavefront reduction in fixed order 0, 1, 2, 3.  MFMA output layout:
  // lane l, register r holds row 4*(l/16) + r, column l%16 of each 16x16 block.
  for (int w = 0; w < 4; ++w) {
    if (wave == w) {
#pragma unroll
      for (int mi = 0; mi < MT; ++mi)
#pragma unroll
        for (int ni = 0; ni < NT; ++ni)
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const int row = mi * 16 + 4 * (lane >> 4) + r;
            const int col = ni * 16 + (lane & 15);
            tile[row][col] = (w == 0 ? 0.f : tile[row][col]) + acc[mi][ni][r];
          }
    }
    __syncthreads();
  }

  if (g.splits > 1) {
    const size_t np = static_cast<size_t>(g.n_tiles) * kBN;
    for (int idx = tid; idx < BM * kBN; idx += kThreads) {
      const int r = idx / kBN, c = idx % kBN, m = m0 + r;
      if (m < g.M) g.partials[(static_cast<size_t>(split) * g.M + m) * np + tile_n * kBN + c] = tile[r][c];
    }
    __threadfence();
    __syncthreads();
    if (tid == 0) {
      const unsigned prev = atomicAdd(&g.counters[tile_m * g.n_tiles + tile_n], 1u);
      last_s = (prev == static_cast<unsigned>(g.splits - 1));
    }
    __syncthreads();
    if (!last_s) return;
    __threadfence();
    for (int idx = tid; idx < BM * kBN; idx += kThreads) {
      const int r = idx / kBN, c = idx % kBN, m = m0 + r;
      if (m >= g.M) continue;
      float s = 0.f;
      for (int sp = 0; sp < g.splits; ++sp)
        s += g.partials[(static_cast<size_t>(sp) * g.M + m) * np + tile_n * kBN + c];
      tile[r][c] = s;
    }
    if (tid == 0) atomicExch(&g.counters[tile_m * g.n_tiles + tile_n], 0u);
  }

  // per-row RMSNorm factor of the A rows
  if (tid < BM) {
    const int m = m0 + tid;
    float f = 1.f;
    if (g.ssq_in != nullptr && m < g.M) {
      float s = 0.f;
      for (int p = 0; p < g.np_in; ++p) s += g.ssq_in[static_cast<size_t>(m) * g.np_in + p];
      f = 1.f / sqrtf(s / static_cast<float>(g.norm_dim) + g.eps);
    }
    rs_s[tid] = f;
  }
  __syncthreads();

  if constexpr (EPI == EPI_FUSE || EPI == EPI_RESID) {
    T* out = static_cast<T*>(g.out);
    const T* gain = static_cast<const T*>(g.gain);
    for (int r = wave; r < BM; r += 4) {
      const int m = m0 + r;
      if (m >= g.M) continue;
      const int n = tile_n * kBN + lane;
      float v = 0.f;
      if (n < g.N) {
        v = tile[r][lane] * rs_s[r];
        if constexpr (EPI == EPI_RESID) {
          float* hp = g.h + static_cast<size_t>(m) * g.N + n;
          v += *hp;
          *hp = v;
        }
        out[static_cast<size_t>(m) * g.ldo + n] = from_f32<T>(v * to_f32(gain[n]));
      }
      const float ss = wave_sum(v * v);
      if (lane == 0) g.ssq_out[static_cast<size_t>(m) * g.np_out + tile_n] = ss;
    }
  } else if constexpr (EPI == EPI_SWIGLU) {
    T* act = static_cast<T*>(g.out);
    for (int idx = tid; idx < BM * 32; idx += kThreads) {
      const int r = idx >> 5, p = idx & 31, m = m0 + r;
      const int j = tile_n * 32 + p;
      if (m >= g.M || j >= g.ffn) continue;
      const float gv = tile[r][p] * rs_s[r];
      const float uv = tile[r][p + 32] * rs_s[r];
      act[static_cast<size_t>(m) * g.ldo + j] = from_f32<T>(gv / (1.f + expf(-gv)) * uv);
    }
  } else if constexpr (EPI == EPI_QKV || EPI == EPI_INJECT) {
    const int dh = g.head_dim, half = dh / 2;
    const int tph = dh / kBN;
    const int sub = tile_n % tph;
    const int p = tid & 31;  // constant per thread: kThreads is a multiple of 32
    const int d1 = sub * 32 + p;
    const double inv_freq = rope_inv_freq(d1, dh, g.theta);
    int kind, head, layer = 0;  // kind 0 = q, 1 = k, 2 = v
    if constexpr (EPI == EPI_QKV) {
      const int hd = tile_n / tph;
      kind = hd < g.n_q_heads ? 0 : (hd < g.n_q_heads + g.n_kv_heads ? 1 : 2);
      head = kind == 0 ? hd : (kind == 1 ? hd - g.n_q_heads : hd - g.n_q_heads - g.n_kv_heads);
    } else {
      const int hpl = 2 * g.n_kv_heads;
      layer = tile_n / (tph * hpl);
      const int hd = (tile_n / tph) % hpl;
      kind = hd < g.n_kv_heads ? 1 : 2;
      head = kind == 1 ? hd : hd - g.n_kv_heads;
    }
    for (int idx = tid; idx < BM * 32; idx += kThreads) {
      const int r = idx >> 5, m = m0 + r;
      if (m >= g.M) continue;
      const int b = m / g.rows_per_seq, i = m % g.rows_per_seq;
      int n_valid = g.rows_per_seq;
      if constexpr (EPI == EPI_INJECT) {
        const int nr = g.n_rows[b];
        if (nr < 0 || nr > g.rows_per_seq) {
          if (i == 0 && p == 0) atomicOr(g.dev_error, 2u);
        }
        n_valid = min(max(nr, 0), g.rows_per_seq);
      }
      if (i >= n_valid) continue;
      const int pos = max(g.ctx_len[b], 0) + i;
      const float x1 = tile[r][p] * rs_s[r], x2 = tile[r][p + 32] * rs_s[r];
      float y1 = x1, y2 = x2;
      if (kind != 2) {
        float sn, cs;
        rope_sincos(pos, inv_freq, &sn, &cs);
        y1 = x1 * cs - x2 * sn;
        y2 = x2 * cs + x1 * sn;
      }
      T* dst;
      if constexpr (EPI == EPI_QKV) {
        if (kind == 0) dst = static_cast<T*>(g.out) + (static_cast<size_t>(m) * g.n_q_heads + head) * dh;
        else dst = static_cast<T*>(kind == 1 ? g.out2 : g.out3) + (static_cast<size_t>(m) * g.n_kv_heads + head) * dh;
      } else {
        const int slot = pos % g.cache_slots;
        dst = static_cast<T*>(kind == 1 ? g.cache_k : g.cache_v) +
              (((static_cast<size_t>(layer) * g.batch + b) * g.n_kv_heads + head) * g.cache_slots + slot) * dh;
      }
      dst[d1] = from_f32<T>(y1);
      dst[d1 + half] = from_f32<T>(y2);
    }
  } else {  // EPI_ARGMAX
    for (int r = wave; r < BM; r += 4) {
      const int m = m0 + r;
      if (m >= g.M) continue;
      const int n = tile_n * kBN + lane;
      float v = -INFINITY;
      int idx = 0x7FFFFFFF;
      if (n < g.N) {
        v = tile[r][lane] * rs_s[r];
        idx = n;
        if (g.logits != nullptr) g.logits[static_cast<size_t>(m) * g.N + n] = v;
      }
      wave_argmax(v, idx);
      if (lane == 0) atomicMax(&g.keys[m], argmax_key(v, idx));
    }
    __threadfence();
    __syncthreads();
    if (tid == 0) {
      const unsigned prev = atomicAdd(&g.counters[tile_m], 1u);
      last_s = (prev == static_cast<unsigned>(g.n_tiles - 1));
    }
    __syncthreads();
    if (!last_s) return;
    __threadfence();
    for (int r = tid; r < BM; r += kThreads) {
      const int m = m0 + r;
      if (m >= g.M) continue;
      const unsigned long long key =
          __hip_atomic_exchange(&g.keys[m], 0ull, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      g.draft[m] = argmax_key_index(key);
    }
    if (tid == 0) atomicExch(&g.counters[tile_m], 0u);
  }
}

template <typename T, int BM, int EPI>
static hipError_t launch_t(const GemmPlan& p, const GemmArgs& a, hipStream_t s) {
  const dim3 grid(p.n_tiles, p.m_tiles, p.splits);
  if (p.vec) hipLaunchKernelGGL((gemm_kernel<T, BM, EPI, true>), grid, dim3(kThreads), 0, s, a);
  else hipLaunchKernelGGL((gemm_kernel<T, BM, EPI, false>), grid, dim3(kThreads), 0, s, a);
  return hipGetLastError();
}

template <typename T, int EPI>
static hipError_t launch_bm(const GemmPlan& p, const GemmArgs& a, hipStream_t s) {
  switch (p.bm) {
    case 16: return launch_t<T, 16, EPI>(p, a, s);
    case 32: return launch_t<T, 32, EPI>(p, a, s);
    case 64: return launch_t<T, 64, EPI>(p, a, s);
    default: return hipErrorInvalidValue;
  }
}

template <typename T>
static hipError_t launch_epi(int epi, const GemmPlan& p, const GemmArgs& a, hipStream_t s) {
  switch (epi) {
    case EPI_FUSE: return launch_bm<T, EPI_FUSE>(p, a, s);
    case EPI_INJECT: return launch_bm<T, EPI_INJECT>(p, a, s);
    case EPI_QKV: return launch_bm<T, EPI_QKV>(p, a, s);
    case EPI_RESID: return launch_bm<T, EPI_RESID>(p, a, s);
    case EPI_SWIGLU: return launch_bm<T, EPI_SWIGLU>(p, a, s);
    case EPI_ARGMAX: return launch_bm<T, EPI_ARGMAX>(p, a, s);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_gemm(int epi, int elem_bytes, const GemmPlan& plan, const GemmArgs& args,
                       hipStream_t stream) {
  if (plan.n_tiles <= 0 || plan.m_tiles <= 0 || plan.splits <= 0) return hipErrorInvalidValue;
  return elem_bytes == 2 ? launch_epi<bf16>(epi, plan, args, stream)
                         : launch_epi<float>(epi, plan, args, stream);
}

}  // namespace dflash
