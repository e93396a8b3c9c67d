// Device body of the weight-streaming GEMM (one workgroup's work item), shared by
// the standalone GEMM kernel (gemm.hip) and the persistent layer kernel
// (persist.hip).  The algorithm is described in gemm.hip.
#pragma once

#include <type_traits>

#include "common.h"
#include "epilogue.h"
#include "gemm.h"
#include "philox.h"

namespace dflash {

// Sampled drafts from the reduced tile in LDS (EPI_SAMPLE).  A work unit is a group
// of 4 rows times the column pair (c, c + 16) of one 32-column half of the tile:
// one Philox block holds the Gumbel noise of its 8 logits.  Per row the unit keeps
// the best key of s + noise (s = logits / T) and the log-sum-exp pair of s; the 32
// units of a row group are 32 consecutive lanes and reduce with xor shuffles.
template <int BM>
__device__ __forceinline__ void sample_tile(const GemmArgs& g, const float (*tile)[kBN + 4], const float* rs,
                                            int tile_n, int m0) {
  static_assert((BM * 8) % kWave == 0, "units fill whole wavefronts");
  const unsigned long long step = g.step_dev != nullptr ? *g.step_dev : g.step;
  for (int u = threadIdx.x; u < BM * 8; u += kThreads) {
    const int rg = u >> 5, cp = u & 31;
    const int col0 = (cp >> 4) * 32 + (cp & 15);
    const int v0 = tile_n * kBN + col0;
    uint32_t h[8];
    philox_u32x8(16ull * static_cast<unsigned>(v0 >> 5) + static_cast<unsigned>(v0 & 15),
                 static_cast<unsigned>((m0 >> 2) + rg), step, 0ull, g.seed, kStreamDraft, h);
    unsigned long long key[4];
    float mx[4], sm[4];
#pragma unroll
    for (int rr = 0; rr < 4; ++rr) {
      const int r = 4 * rg + rr, m = m0 + r;
      float sv[2];
      key[rr] = 0ull;
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        const int col = col0 + 16 * j, v = tile_n * kBN + col;
        sv[j] = -INFINITY;
        if (v < g.N && m < g.M) {
          const float z = tile[r][col] * rs[r];
          if (g.logits != nullptr) g.logits[static_cast<size_t>(m) * g.N + v] = z;
          sv[j] = z * g.inv_temp;
          const unsigned long long kj = argmax_key(sv[j] + gumbel_f32(h[2 * rr + j]), v);
          key[rr] = kj > key[rr] ? kj : key[rr];
        }
      }
      mx[rr] = fmaxf(sv[0], sv[1]);
      sm[rr] = mx[rr] == -INFINITY ? 0.f
                                   : __builtin_amdgcn_exp2f((sv[0] - mx[rr]) * kLog2e) +
                                         __builtin_amdgcn_exp2f((sv[1] - mx[rr]) * kLog2e);
    }
#pragma unroll
    for (int o = 1; o < 32; o <<= 1)
#pragma unroll
      for (int rr = 0; rr < 4; ++rr) {
        const unsigned long long ok = __shfl_xor(key[rr], o, kWave);
        key[rr] = ok > key[rr] ? ok : key[rr];
        const float om = __shfl_xor(mx[rr], o, kWave), os = __shfl_xor(sm[rr], o, kWave);
        lse_merge(mx[rr], sm[rr], om, os);
      }
    if (cp == 0) {
#pragma unroll
      for (int rr = 0; rr < 4; ++rr) {
        const int m = m0 + 4 * rg + rr;
        if (m < g.M) {
          g.keys[static_cast<size_t>(m) * g.n_parts + tile_n] = key[rr];
          g.lse_part[static_cast<size_t>(m) * g.n_parts + tile_n] = make_float2(mx[rr], sm[rr]);
        }
      }
    }
  }
}

// LDS of one streaming-GEMM workgroup.
template <int MT>
struct StreamLds {
  static constexpr int BM = MT * 16;
  float tile[BM][kBN + 4];
  float xpart[3][BM][kBN + 4];  // partial tiles of wavefronts 1..3
  float rs[BM];
  int last;
};

// One workgroup's work item (bx, by, bz) of the weight-streaming GEMM (the kernel's
// blockIdx).  `hook(tile_n, s_lo, s_hi)` runs after the weight loads of the first
// pipeline stages are issued and before anything that depends on the A operand is
// read: the persistent layer kernel waits there for the producers of the A columns
// of K steps [s_lo, s_hi), so the weight stream is already in flight during the wait.
// `done(tile_n)` runs in the workgroup that finished output tile tile_n, after its
// epilogue (all threads).  COH: the A operand, the RMSNorm
// partials and the residual are read, and the outputs written, device-coherently
// (producer and consumer inside one launch).
template <typename TIN, int MT, int EPI, int D, bool COH, typename Hook, typename Done>
__device__ __forceinline__ void gemm_body(const GemmArgs& g, int bx, int by, int bz, StreamLds<MT>& lds,
                                          Hook hook, Done done) {
  typedef typename ActOf<TIN>::type TA;
  typedef typename std::conditional<EPI == EPI_FUSE, TIN, TA>::type E;
  constexpr bool APK = EPI != EPI_FUSE;  // only the fusion GEMM reads a row-major A
  constexpr int BM = MT * 16;
  auto& tile = lds.tile;
  float* rs_s = lds.rs;

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // uniform per wavefront
  const int tile_m = by;
  const int m0 = tile_m * BM;
  // this workgroup's output tile, its piece of the tile's K steps, and the tile's
  // piece count (all uniform per workgroup)
  int tile_n, split, n_split, s_lo, s_hi;
  if (g.piece_base > 0) {
    const int w = bx, wide = g.piece_base + 1, n_wide = g.piece_extra * wide;
    if (w < n_wide) {
      tile_n = w / wide;
      split = w % wide;
      n_split = wide;
    } else {
      tile_n = g.piece_extra + (w - n_wide) / g.piece_base;
      split = (w - n_wide) % g.piece_base;
      n_split = g.piece_base;
    }
    s_lo = split * g.S / n_split;
    s_hi = (split + 1) * g.S / n_split;
  } else {
    tile_n = bx;
    split = bz;
    n_split = g.splits;
    s_lo = split * g.steps_per_split;
    s_hi = min(g.S, s_lo + g.steps_per_split);
  }

  size_t wtile = tile_n;
  if constexpr (EPI == EPI_INJECT) {
    const int l = tile_n / g.inj_tiles;
    wtile = static_cast<size_t>(l) * g.layer_tiles + g.inj_tile0 + tile_n % g.inj_tiles;
  }
  const E* Wt = static_cast<const E*>(g.W) + wtile * g.S * kTileStepElems + lane * 8;
  const int n_w = (s_hi - s_lo + 3) >> 2;  // steps per wavefront, rounded up
  const int NI = (n_w + D - 1) / D * D;

  const E* At = static_cast<const E*>(g.A);
  const E* arow[MT];
  if constexpr (APK) {
    At += static_cast<size_t>(tile_m) * MT * g.S * 512 + lane * 8;
  } else {
#pragma unroll
    for (int mi = 0; mi < MT; ++mi) {
      const int m = m0 + mi * 16 + (lane & 15);
      arow[mi] = m < g.M ? At + static_cast<size_t>(m) * g.lda : nullptr;
    }
  }
  const int kq = 8 * (lane >> 4);
  const bool a_vec = (g.lda % 8) == 0;

  f32x4 acc[MT][4];
#pragma unroll
  for (int mi = 0; mi < MT; ++mi)
#pragma unroll
    for (int ni = 0; ni < 4; ++ni) acc[mi][ni] = f32x4{0.f, 0.f, 0.f, 0.f};
  Frag<E> fa[D][MT], fb[D][4];

  // Step i of this wavefront.  Past the split's last step the loads repeat the last
  // step (a valid address) and the multiply is skipped by a wavefront-uniform
  // branch; the loaded values are never selected on, so the compiler can keep the
  // loads of D steps in flight and wait only where each fragment is consumed.
#define DFLASH_LOAD_W(u, i)                                                                \
  {                                                                                        \
    const int s_ = s_lo + wave + 4 * (i);                                                  \
    const int sc_ = s_ < s_hi ? s_ : s_hi - 1;                                             \
    _Pragma("unroll") for (int ni = 0; ni < 4; ++ni)                                       \
        fb[u][ni].load(Wt + (static_cast<size_t>(sc_) * 4 + ni) * 512);                    \
  }
#define DFLASH_LOAD_A(u, i)                                                                \
  {                                                                                        \
    const int s_ = s_lo + wave + 4 * (i);                                                  \
    const bool ok_ = s_ < s_hi;                                                            \
    const int sc_ = ok_ ? s_ : s_hi - 1;                                                   \
    _Pragma("unroll") for (int mi = 0; mi < MT; ++mi) {                                    \
      if constexpr (APK) {                                                                 \
        if constexpr (COH)                                                                 \
          fa[u][mi].v = coherent_load16<decltype(fa[u][mi].v)>(At + (static_cast<size_t>(mi) * g.S + sc_) * 512); \
        else                                                                               \
          fa[u][mi].load(At + (static_cast<size_t>(mi) * g.S + sc_) * 512);                \
      } else {                                                                             \
        const int k_ = sc_ * kKStep + kq;                                                  \
        const int valid_ = ok_ ? g.K - k_ : 0;                                             \
        if (arow[mi] != nullptr && valid_ >= 8 && a_vec) fa[u][mi].load(arow[mi] + k_);    \
        else if (arow[mi] != nullptr && valid_ > 0) fa[u][mi].load_masked(arow[mi] + k_, min(valid_, 8)); \
        else fa[u][mi].zero();                                                             \
      }                                                                                    \
    }                                                                                      \
  }
#define DFLASH_LOAD(u, i) \
  DFLASH_LOAD_W(u, i)     \
  DFLASH_LOAD_A(u, i)
#define DFLASH_MMA(u, i)                                                \
  if (s_lo + wave + 4 * (i) < s_hi) {                                   \
    _Pragma("unroll") for (int mi = 0; mi < MT; ++mi)                   \
        _Pragma("unroll") for (int ni = 0; ni < 4; ++ni)                \
            Frag<E>::mma(acc[mi][ni], fa[u][mi], fb[u][ni]);            \
  }

  // prologue: the weights of the first D steps, then (after the hook) the
  // A operand of those steps and the epilogue's own inputs
#pragma unroll
  for (int u = 0; u < D; ++u) DFLASH_LOAD_W(u, u);
  hook(tile_n, s_lo, s_hi);
#pragma unroll
  for (int u = 0; u < D; ++u) DFLASH_LOAD_A(u, u);
  // Loads the epilogue needs but the product does not (RMSNorm partial sums, the
  // residual tile) are issued before the main loop so their latency overlaps it.
  float ssq_part = 0.f;
  {
    const int r = tid >> 2, q = tid & 3, m = m0 + r;
    if (g.ssq_in != nullptr && r < BM && m < g.M) {
      const float* src = g.ssq_in + static_cast<size_t>(m) * g.np_in;
      float v[16];
#pragma unroll
      for (int t = 0; t < 16; ++t) v[t] = q + 4 * t < g.np_in ? get<COH>(src + q + 4 * t) : 0.f;
      for (int p = q + 64; p < g.np_in; p += 4) ssq_part += get<COH>(src + p);
#pragma unroll
      for (int t = 0; t < 16; ++t) ssq_part += v[t];
    }
  }
  float hres[(EPI == EPI_RESID) ? (BM + 31) / 32 : 1][8];
  if constexpr (EPI == EPI_RESID) {
    const int c8 = tid & 7;
#pragma unroll
    for (int it = 0; it < (BM + 31) / 32; ++it) {
      const int r = (tid >> 3) + 32 * it, m = m0 + r;
      const int n0 = tile_n * kBN + c8 * 8;
      if (r < BM && m < g.M && n0 < g.N) {
        const float4* hp = reinterpret_cast<const float4*>(g.h + static_cast<size_t>(m) * g.N + n0);
        const float4 h0 = get16<COH, float4>(hp), h1 = get16<COH, float4>(hp + 1);
        hres[it][0] = h0.x; hres[it][1] = h0.y; hres[it][2] = h0.z; hres[it][3] = h0.w;
        hres[it][4] = h1.x; hres[it][5] = h1.y; hres[it][6] = h1.z; hres[it][7] = h1.w;
      }
    }
  }

  int i0 = 0;
  for (; i0 < NI - D; i0 += D) {
#pragma unroll
    for (int u = 0; u < D; ++u) {
      DFLASH_MMA(u, i0 + u);
      DFLASH_LOAD(u, i0 + D + u);
    }
  }
#pragma unroll
  for (int u = 0; u < D; ++u) DFLASH_MMA(u, i0 + u);
#undef DFLASH_LOAD
#undef DFLASH_LOAD_W
#undef DFLASH_LOAD_A
#undef DFLASH_MMA

  // Cross-wavefront reduction in fixed order 0, 1, 2, 3.  MFMA output layout:
  // lane l, register r holds row 4*(l/16) + r, column l%16 of each 16x16 block.
  {
    // every wavefront stores its partial tile (wavefront 0's into the output tile
    // itself), then all threads sum them in order: one barrier between, instead of
    // one per wavefront
    auto& xpart = lds.xpart;
#pragma unroll
    for (int mi = 0; mi < MT; ++mi)
#pragma unroll
      for (int ni = 0; ni < 4; ++ni)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int row = mi * 16 + 4 * (lane >> 4) + r, col = ni * 16 + (lane & 15);
          (wave == 0 ? tile[row] : xpart[wave - 1][row])[col] = acc[mi][ni][r];
        }
    __syncthreads();
#pragma unroll
    for (int e = 0; e < BM * kBN / kThreads; ++e) {
      const int idx = tid + e * kThreads, row = idx / kBN, col = idx % kBN;
      tile[row][col] = (((0.f + tile[row][col]) + xpart[0][row][col]) + xpart[1][row][col]) + xpart[2][row][col];
    }
    __syncthreads();
  }

  if (n_split > 1) {
    const size_t np = static_cast<size_t>(g.n_tiles) * kBN;
    for (int idx = tid; idx < BM * kBN; idx += kThreads) {
      const int r = idx / kBN, c = idx % kBN, m = m0 + r;
      if (m < g.M)
        coherent_store(&g.partials[(static_cast<size_t>(split) * g.M + m) * np + tile_n * kBN + c], tile[r][c]);
    }
    unsigned* counter = &g.counters[tile_m * g.n_tiles + tile_n];
    if (!arrive_last(counter, n_split, &lds.last)) return;
    // every partial of this thread's elements is requested before any is summed
    constexpr int PER = BM * kBN / kThreads;  // elements per thread
    constexpr int kMaxSplits = 16 / MT;  // the plan never splits further
    float pv[PER][kMaxSplits];
#pragma unroll
    for (int e = 0; e < PER; ++e) {
      const int idx = tid + e * kThreads, r = idx / kBN, c = idx % kBN, m = min(m0 + r, g.M - 1);
#pragma unroll
      for (int sp = 0; sp < kMaxSplits; ++sp)
        if (sp < n_split)
          pv[e][sp] = coherent_load(&g.partials[(static_cast<size_t>(sp) * g.M + m) * np + tile_n * kBN + c]);
    }
#pragma unroll
    for (int e = 0; e < PER; ++e) {
      const int idx = tid + e * kThreads, r = idx / kBN, c = idx % kBN;
      float s = 0.f;
#pragma unroll
      for (int sp = 0; sp < kMaxSplits; ++sp)
        if (sp < n_split) s += pv[e][sp];
      tile[r][c] = s;
    }
    if (tid == 0) reset_counter(counter);
  }

  // per-row RMSNorm factor of the A rows: 4 threads per row combine the partials
  {
    const int r = tid >> 2, q = tid & 3;
    float s = ssq_part;
    const int m = m0 + r;
    const bool have = g.ssq_in != nullptr && r < BM && m < g.M;
    (void)q;
    s += __shfl_xor(s, 1, kWave);
    s += __shfl_xor(s, 2, kWave);
    if (q == 0 && r < BM) rs_s[r] = have ? 1.f / sqrtf(s / static_cast<float>(g.norm_dim) + g.eps) : 1.f;
  }
  __syncthreads();

  if constexpr (EPI != EPI_ARGMAX && EPI != EPI_SAMPLE) {
    epilogue_tile<TIN, EPI, BM, kThreads, COH>(g, tile, rs_s, tile_n, m0, g.M, hres);
    done(tile_n);
  } else {  // EPI_ARGMAX, EPI_SAMPLE
    if constexpr (EPI == EPI_SAMPLE) sample_tile<BM>(g, tile, rs_s, tile_n, m0);
    else for (int r = wave; r < BM; r += 4) {
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
      if (lane == 0) g.keys[static_cast<size_t>(m) * g.n_parts + tile_n] = argmax_key(v, idx);
    }
    // the row's draft is the largest tile key: launch_head_finalize, after this kernel
  }
}

}  // namespace dflash
