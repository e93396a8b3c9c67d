// Tiled MFMA GEMM for many rows (batch x block >= 128): out[m, n] = sum_k A[m, k] W[n, k].
//
// Once the draft batch has hundreds of rows the projections are compute-bound, and a
// kernel that streams W once per 64-row block (the weight-streaming GEMM) would read
// every weight matrix M/64 times.  Here one workgroup owns a BM x BN output tile
// (256 x 256, 128 x 384 or 256 x 128 with 8 wavefronts, 128 x 128 with 4) and walks K
// in 32-wide steps:
//
//  * Both operands are fragment-packed (weights by dflash_pack_weights, activations
//    by the producing epilogue), so one K step of a 16-row (or 16-column) block is
//    one contiguous 1 KB chunk, exactly one wavefront MFMA operand.  Chunks go from
//    HBM/L2 straight into LDS with the gfx950 16-byte LDS-DMA load (64 lanes x 16 B
//    = 1 KB per instruction, no staging registers), into four stage buffers: the
//    loads of steps s+2..s+4 are in flight while step s is multiplied.  The fusion GEMM's A operand
//    is the caller's row-major taps; there each lane supplies its own row address and
//    the DMA gathers the same fragment layout.
//  * Wavefront (wm, wn) owns WM x WN blocks of 16 x 16; its fragments for step s+1
//    are read from LDS while the MFMAs of step s issue (two register sets, reads
//    interleaved one per WM*WN/(WM+WN) MFMAs).
//  * One barrier per step.  The DMA is issued from inline assembly so the compiler's
//    wait-count pass does not drain it before every LDS read; the kernel waits with
//    explicit vmcnt counts instead (every wavefront issues the same number of DMA
//    loads per stage; rows/columns past the end re-load a valid chunk).
//  * The output tile goes through LDS 64 columns at a time into the same fused
//    epilogues as the weight-streaming GEMM, or (greedy LM head, SwiGLU on 256 x 256
//    tiles, residual on 256 x 128) the product is computed transposed and the
//    epilogue works from the accumulators: a lane holds 4 consecutive columns of one
//    row.  K may be split over workgroups: fp32 partial tiles in the accumulators'
//    layout, summed in split order by gemm_tiled_reduce_kernel, which runs the epilogue.
//  * Workgroup x runs on XCD x mod 8; tiles are renumbered so each XCD works on a
//    contiguous run of tiles, m fastest, so the workgroups that share a weight tile
//    share that XCD's L2.  The LM head and those SwiGLU launches may be persistent:
//    one workgroup per CU walks a stride of its XCD's tiles and issues the next
//    tile's first loads before the current tile's epilogue.
#include <type_traits>

#include "common.h"
#include "epilogue.h"
#include "gemm.h"
#include "philox.h"

namespace dflash {

template <int NWM, int NWN, int WM, int WN>
struct TileCfg {
  static constexpr int NW = NWM * NWN, NT = 64 * NW, WM_ = WM, WN_ = WN;
  static constexpr int AFR = NWM * WM, BFR = NWN * WN, FR = AFR + BFR;
  static constexpr int BM = 16 * AFR, BN = 16 * BFR, SUB = BFR / 4;
  static constexpr int LPW = FR / NW;      // DMA loads per wavefront per stage
  static constexpr int STAGE = FR * 1024;  // bytes per stage
  static constexpr int NST = 4;
  static constexpr int MAIN = NST * STAGE;
  static constexpr int TILE = BM * (kBN + 4) * 4;
  // epilogue subtiles per round: two when the LDS has room for both (with the rest of
  // the kernel's LDS under 150 KB), else one
  static constexpr int PAIR = (SUB % 2 == 0 && 2 * TILE <= 150 * 1024 - 3 * 1024) ? 2 : 1;
  static constexpr int BYTES = MAIN > PAIR * TILE ? MAIN : PAIR * TILE;
  static_assert(FR % NW == 0, "chunks split evenly over the wavefronts");
  static_assert(WN % 2 == 0, "pairs of 16-column blocks (the sampled noise layout)");
  static_assert(BFR % 4 == 0, "whole 64-column subtiles");
};

// The larger of a 64-bit key and the key of the lane CTRL selects.
template <int CTRL>
__device__ __forceinline__ unsigned long long dpp_max_key(unsigned long long k) {
  const uint32_t lo =
      static_cast<uint32_t>(__builtin_amdgcn_mov_dpp(static_cast<int>(static_cast<uint32_t>(k)), CTRL, 0xF, 0xF, true));
  const uint32_t hi = static_cast<uint32_t>(
      __builtin_amdgcn_mov_dpp(static_cast<int>(static_cast<uint32_t>(k >> 32)), CTRL, 0xF, 0xF, true));
  const unsigned long long o = (static_cast<unsigned long long>(hi) << 32) | lo;
  return o > k ? o : k;
}
// One butterfly round of the sampled epilogue's row reduction: the best key and the
// merged log-sum-exp pair of this lane and the lane CTRL selects.
template <int CTRL>
__device__ __forceinline__ void dpp_sample_round(unsigned long long& key, float& mx, float& sm) {
  key = dpp_max_key<CTRL>(key);
  const float om = dpp_f32<CTRL>(mx), os = dpp_f32<CTRL>(sm);
  lse_merge(mx, sm, om, os);
}

// Element (16-byte unit) of split sp's partial of tile (tm, tn), wavefront w, 16 x 16
// block (i, j), lane l: [split][tile, m fastest][wavefront][i][j][lane].
template <typename C>
__device__ __forceinline__ size_t tiled_part_index(int sp, int m_tiles, int n_big, int tm, int tn, int w, int i, int j,
                                                   int l) {
  const size_t tiles_all = static_cast<size_t>(m_tiles) * n_big;
  const size_t tile = static_cast<size_t>(tn) * m_tiles + tm;
  return ((((static_cast<size_t>(sp) * tiles_all + tile) * C::NW + w) * C::WM_ + i) * C::WN_ + j) * kWave + l;
}

// Whether a tiled GEMM computes its tile transposed (see gemm_tiled_kernel): the greedy
// LM head, SwiGLU when every wavefront covers whole 64-column subtiles, and the
// residual GEMM on 256 x 128 tiles.
template <int EPI, int NWM, int NWN, int WM, int WN>
constexpr bool tiled_trans() {
  return EPI == EPI_ARGMAX || (EPI == EPI_SWIGLU && WN % 4 == 0) ||
         (EPI == EPI_RESID && NWM == 4 && NWN == 2 && WM == 4 && WN == 4);
}

constexpr int vmcnt_wait(int n) { return (n & 0xF) | ((n >> 4) << 14) | (0x7 << 4) | (0xF << 8); }
// vmcnt <= n and every LDS read of this wavefront complete (lgkmcnt 0)
constexpr int vm_lgkm_wait(int n) { return (n & 0xF) | ((n >> 4) << 14) | (0x7 << 4); }

// 1 KB DMA: lane l's 16 bytes at gp land at LDS byte lds + 16 * l.  m0 (the LDS
// base of the DMA) is declared clobbered; no other code in these kernels uses m0.
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"
__device__ __forceinline__ void dma_1k(const void* gp, uint32_t lds) {
  asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, off" ::"v"(gp), "s"(lds) : "m0");
}
#pragma clang diagnostic pop

template <int EPI, int NWM, int NWN, int WM, int WN>
__global__ __launch_bounds__(64 * NWM * NWN) __attribute__((amdgpu_waves_per_eu(NWM * NWN == 4 ? 2 : 1, 2))) void gemm_tiled_kernel(GemmArgs g) {
  using C = TileCfg<NWM, NWN, WM, WN>;
  constexpr int AFR = C::AFR, BFR = C::BFR, BM = C::BM, SUB = C::SUB, LPW = C::LPW, NW = C::NW, NT = C::NT;
  // TRANS: the product is computed transposed (W A^T, each MFMA's operands swapped), so
  // a lane holds 4 consecutive output columns of one row, and the epilogue runs from
  // the accumulators (see tiled_trans).  PERS: such launches may be persistent (not
  // the residual GEMM: its grids are one tile per CU).
  constexpr bool TRANS = tiled_trans<EPI, NWM, NWN, WM, WN>();
  constexpr bool PERS = TRANS && EPI != EPI_RESID;
  // packed activations; the fusion GEMM reads row-major taps unless they were packed
  const bool APK = EPI != EPI_FUSE || g.a_packed != 0;
  typedef typename std::conditional<EPI == EPI_FUSE, bf16, f16>::type E;
  typedef typename std::conditional<EPI == EPI_FUSE, bf16x8, f16x8>::type E8;

  __shared__ __attribute__((aligned(1024))) char smem[C::BYTES];
  __shared__ __attribute__((aligned(16))) float rs_s[BM];
  __shared__ unsigned long long best_s[BM];

  const int tid = threadIdx.x, lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave % NWM, wn = wave / NWM;
  const int n_big = (g.n_tiles + SUB - 1) / SUB;
  // compacted block rows: tiles past the live rows have nothing to do
  int M = g.M;
  if (g.m_live != nullptr) M = min(M, max(*g.m_live, 0));
  // Tiles (split, n tile, m tile), m fastest, renumbered XCD-contiguous.  One tile per
  // workgroup, or (persistent LM head, one workgroup per CU) a stride through the
  // XCD's run of tiles: tile L, L + nwg/8, ..., so the XCD's workgroups still work
  // on neighbouring tiles at any time.
  const int nwg = gridDim.x, x = blockIdx.x, xcd = x & 7;
  int L, L_end, L_step;
  if (PERS && g.persist != 0) {
    const int T = g.m_tiles * n_big, q = T >> 3, r8 = T & 7;
    L = xcd * q + min(xcd, r8) + (x >> 3);
    L_end = xcd * q + min(xcd, r8) + q + (xcd < r8 ? 1 : 0);
    L_step = nwg >> 3;
  } else {
    const int q = nwg >> 3, r8 = nwg & 7;
    L = xcd * q + min(xcd, r8) + (x >> 3);
    L_end = L + 1;
    L_step = 1;
  }
  while (L < L_end && (L % g.m_tiles) * BM >= M) L += L_step;
  if (L >= L_end) return;  // uniform per workgroup
  const int m_blocks = (g.M + 15) >> 4;

  // per-chunk source addresses (at step s_lo) and per-step strides, LDS offsets
  const uint32_t lds0 = static_cast<uint32_t>(reinterpret_cast<uintptr_t>((__attribute__((address_space(3))) char*)smem));
  const char* src[LPW];
  uint32_t stride[LPW], ldsoff[LPW];
#pragma unroll
  for (int j = 0; j < LPW; ++j) {
    const int c = wave + NW * j;
    stride[j] = c < AFR ? (APK ? 1024u : static_cast<uint32_t>(kKStep * 2)) : 4096u;
    ldsoff[j] = __builtin_amdgcn_readfirstlane(lds0 + c * 1024);
  }
  auto set_src = [&](int tm, int tn, int s_lo) {
#pragma unroll
    for (int j = 0; j < LPW; ++j) {
      const int c = wave + NW * j;
      if (c < AFR) {
        if (APK) {
          const int mb = min(tm * AFR + c, m_blocks - 1);
          src[j] = static_cast<const char*>(g.A) + ((static_cast<size_t>(mb) * g.S + s_lo) * 512 + lane * 8) * 2;
        } else {
          int row = min(tm * BM + c * 16 + (lane & 15), M - 1);
          if (g.row_map != nullptr) row = g.row_map[row];  // compacted rows: gather the tap row
          src[j] = static_cast<const char*>(g.A) +
                   (static_cast<size_t>(row) * g.lda + static_cast<size_t>(s_lo) * kKStep + (lane >> 4) * 8) * 2;
        }
      } else {
        const int cb = c - AFR;
        const int t = min(tn * SUB + cb / 4, g.n_tiles - 1);
        size_t wt = t;
        if constexpr (EPI == EPI_INJECT) wt = static_cast<size_t>(t / g.inj_tiles) * g.layer_tiles + g.inj_tile0 + t % g.inj_tiles;
        src[j] = static_cast<const char*>(g.W) + (((wt * g.S + s_lo) * 4 + (cb & 3)) * 512 + lane * 8) * 2;
      }
    }
  };
  auto issue = [&](int s, int buf) {
#pragma unroll
    for (int j = 0; j < LPW; ++j) dma_1k(src[j] + static_cast<size_t>(s) * stride[j], ldsoff[j] + buf * C::STAGE);
  };

  f32x4 acc[WM][WN];
  E8 fa0[WM], fb0[WN], fa1[WM], fb1[WN];
  auto read = [&](int buf, E8* fa, E8* fb) {
    const E* st = reinterpret_cast<const E*>(smem + buf * C::STAGE);
#pragma unroll
    for (int j = 0; j < WN; ++j) fb[j] = *reinterpret_cast<const E8*>(st + (AFR + wn * WN + j) * 512 + lane * 8);
#pragma unroll
    for (int i = 0; i < WM; ++i) fa[i] = *reinterpret_cast<const E8*>(st + (wm * WM + i) * 512 + lane * 8);
  };
  // One step's work in LPW chunks: chunk c issues its share of the next step's
  // fragment reads and of this step's MFMAs (interleaved), then, when `dma`, the c-th
  // of this wavefront's DMA loads of stage ds into buffer db.  Spreading the DMA
  // issue over the step keeps it from holding back the MFMA stream after a barrier.
  auto step_work = [&](int buf_next, const E8* fa, const E8* fb, E8* fan, E8* fbn, bool dma, int ds, int db) {
    const E* st = reinterpret_cast<const E*>(smem + buf_next * C::STAGE);
    auto chunk = [&](auto cc) {
      constexpr int c = decltype(cc)::value;
      constexpr int MM = WM * WN, NR = WM + WN;
      // MFMAs spread evenly.  Eight wavefronts (one workgroup per CU): the reads in
      // all chunks but the last (so they have landed when the step ends) and the DMA
      // loads at the ends of chunks 0 .. LPW-2, the last two together, so none is
      // issued right before the step's wait.  Four wavefronts (two workgroups per CU,
      // whose steps interleave): reads and DMA loads spread over all chunks.
      constexpr bool LATE_FREE = NW == 8 && LPW > 1;
      constexpr int RC = LATE_FREE ? LPW - 1 : LPW;
      constexpr int q0 = c * MM / LPW, q1 = (c + 1) * MM / LPW;
      constexpr int r0 = c < RC ? c * NR / RC : NR, r1 = c < RC ? (c + 1) * NR / RC : NR;
#pragma unroll
      for (int r = r0; r < r1; ++r) {
        if (r < WN) fbn[r] = *reinterpret_cast<const E8*>(st + (AFR + wn * WN + r) * 512 + lane * 8);
        else fan[r - WN] = *reinterpret_cast<const E8*>(st + (wm * WM + r - WN) * 512 + lane * 8);
      }
#pragma unroll
      for (int q = q0; q < q1; ++q) {
        const int i = q / WN, j = q % WN;
        if constexpr (EPI == EPI_FUSE) acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(fa[i], fb[j], acc[i][j], 0, 0, 0);
        else if constexpr (TRANS)  // columns x rows
          acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_f16(fb[j], fa[i], acc[i][j], 0, 0, 0);
        else acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_f16(fa[i], fb[j], acc[i][j], 0, 0, 0);
      }
      constexpr int nm = q1 - q0, nr = r1 - r0, per = nm / (nr + 1);
#pragma unroll
      for (int k = 0; k < nr; ++k) {
        if constexpr (per > 0) __builtin_amdgcn_sched_group_barrier(0x008, per, 0);  // MFMA
        __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);                            // LDS read
      }
      if constexpr (nm - per * nr > 0) __builtin_amdgcn_sched_group_barrier(0x008, nm - per * nr, 0);
      if constexpr (!LATE_FREE) {
        if (dma) dma_1k(src[c] + static_cast<size_t>(ds) * stride[c], ldsoff[c] + db * C::STAGE);
      } else if constexpr (c < LPW - 1) {
        if (dma) dma_1k(src[c] + static_cast<size_t>(ds) * stride[c], ldsoff[c] + db * C::STAGE);
        if constexpr (c == LPW - 2)
          if (dma) dma_1k(src[c + 1] + static_cast<size_t>(ds) * stride[c + 1], ldsoff[c + 1] + db * C::STAGE);
      }
    };
    static_assert(LPW >= 1 && LPW <= 4, "one to four DMA loads per wavefront and stage");
    chunk(std::integral_constant<int, 0>{});
    if constexpr (LPW > 1) chunk(std::integral_constant<int, 1>{});
    if constexpr (LPW > 2) chunk(std::integral_constant<int, 2>{});
    if constexpr (LPW > 3) chunk(std::integral_constant<int, 3>{});
  };

  auto issue_prologue = [&](int S) {  // stages 0..3 in flight
    issue(0, 0);
    if (1 < S) issue(1, 1);
    if (2 < S) issue(2, 2);
    if (3 < S) issue(3, 3);
  };

  int prev_tm = -1;
  for (bool first = true;; first = false) {
  // lane and thread ids, opaque to the compiler on every tile: it would otherwise
  // hoist the epilogue's per-lane row addresses out of a persistent workgroup's tile
  // loop and keep them (spilled) across the main loop
  int lane_t = lane, tid_t = tid;
  if constexpr (PERS) asm volatile("" : "+v"(lane_t), "+v"(tid_t));
  const int tm = L % g.m_tiles, rest = L / g.m_tiles;
  const int tn = rest % n_big, split = rest / n_big;
  const int m0 = tm * BM;
  const int s_lo = split * g.steps_per_split;
  const int S = min(g.S, s_lo + g.steps_per_split) - s_lo;  // steps of this split (>= 1)
  // a persistent workgroup's later tiles had their prologue issued during the
  // previous tile's epilogue
  if (first) set_src(tm, tn, s_lo);

  // RMSNorm factor of this tile's A rows (thread r < BM: row m0 + r), kept while the
  // m tile stays the same.  The row's partial sums are loaded all 16 back to back
  // (clamped index, no branch: a branch per load made each wait for the previous) and
  // summed before the DMA issue.  Summed after it, they would wait for every stage:
  // the compiler counts only its own loads, not the DMA loads issued after them.
  const bool new_rows = tm != prev_tm;
  prev_tm = tm;
  const int r_own = tid_t < BM ? tid_t : BM - 1;
  const bool rs_vec = g.ssq_in != nullptr && (g.np_in & 3) == 0 && g.np_in >= 4 && g.np_in <= 64;
  const float* ssq_row =
      g.ssq_in != nullptr ? g.ssq_in + static_cast<size_t>(min(m0 + r_own, g.M - 1)) * g.np_in : nullptr;
  float ssq_sum = 0.f;
  if (rs_vec && new_rows) {
    const float4* row4 = reinterpret_cast<const float4*>(ssq_row);
    const int n4 = g.np_in >> 2;
    float4 v[16];
#pragma unroll
    for (int t = 0; t < 16; ++t) v[t] = row4[min(t, n4 - 1)];
#pragma unroll
    for (int t = 0; t < 16; ++t) ssq_sum += t < n4 ? (v[t].x + v[t].y) + (v[t].z + v[t].w) : 0.f;
    asm volatile("" ::"v"(ssq_sum));  // taken here, not sunk into the branch that uses it
  }

  // prologue: stages 0..3 in flight, wait for 0 and 1.  (On a persistent workgroup's
  // later tiles the key stores of the previous tile are younger than the DMA loads;
  // vector memory loads complete in order, so the count still covers stages 0 and 1.)
  if (first) issue_prologue(S);
  if (3 < S) __builtin_amdgcn_s_waitcnt(vmcnt_wait(2 * LPW));
  else if (2 < S) __builtin_amdgcn_s_waitcnt(vmcnt_wait(LPW));
  else __builtin_amdgcn_s_waitcnt(vmcnt_wait(0));
  if (tid_t < BM) {
    if (new_rows) {
      float f = 1.f;
      if (g.ssq_in != nullptr && m0 + tid_t < g.M) {
        float sum = 0.f;
        if (rs_vec) {
          sum = ssq_sum;
        } else {
          for (int t = 0; t < g.np_in; ++t) sum += ssq_row[t];
        }
        f = 1.f / sqrtf(sum / static_cast<float>(g.norm_dim) + g.eps);
      }
      rs_s[tid_t] = f;  // the previous tile's epilogue read rs_s before its key barrier
    }
    // the same thread stored row tid_t's key of the previous tile
    if constexpr (EPI == EPI_ARGMAX || EPI == EPI_SAMPLE) best_s[tid_t] = 0ull;
  }
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
  read(0, fa0, fb0);
  if (4 < S) {  // stage 4 goes into buffer 0 at step 0: every wavefront has its stage-0 fragments
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_waitcnt(vm_lgkm_wait(63));
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
  }
  // Step t multiplies the fragments read during step t-1 and reads those of step
  // t+1 (stage t+1 landed at the end of step t-1).  The DMA of stage t+4 goes into
  // the buffer of stage t: every wavefront's reads of stage t completed (lgkmcnt 0)
  // before the barrier that ended step t-1, so four stages are in flight and a DMA
  // has three steps to land.  Groups of four steps with every condition true (t + 4
  // < S) run without branches; the last steps check theirs.
#pragma unroll
  for (int i = 0; i < WM; ++i)
#pragma unroll
    for (int j = 0; j < WN; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};
  // persistent launch: the workgroup's next tile, and whether its first three stages
  // are issued during this tile's last K steps (XT: whole groups of four steps, at
  // least two of them, so the tail is exactly the last four steps and issues no stage
  // of this tile)
  int L_next = L_end;
  if constexpr (PERS) {
    if (g.persist != 0) {
      L_next = L + L_step;
      while (L_next < L_end && (L_next % g.m_tiles) * BM >= M) L_next += L_step;
    }
  }
  const bool XT = PERS && L_next < L_end && (S & 3) == 0 && S >= 8;
  int s = 0;
  for (; s + 8 <= S; s += 4) {
#define DFLASH_FULL(u, fac, fbc, fan, fbn)                                    \
  step_work((u + 1) & 3, fac, fbc, fan, fbn, true, s + u + 4, u);             \
  asm volatile("" ::: "memory");                                              \
  __builtin_amdgcn_s_waitcnt(vm_lgkm_wait(2 * LPW));                          \
  __builtin_amdgcn_s_barrier();                                               \
  asm volatile("" ::: "memory");
    DFLASH_FULL(0, fa0, fb0, fa1, fb1)
    DFLASH_FULL(1, fa1, fb1, fa0, fb0)
    DFLASH_FULL(2, fa0, fb0, fa1, fb1)
    DFLASH_FULL(3, fa1, fb1, fa0, fb0)
#undef DFLASH_FULL
  }
  // Residual GEMM on 256 x 128 tiles (computed transposed): the epilogue's residual
  // values (a 16-byte piece per 16 x 16 block: the lane's row and 4 columns) and the
  // next RMSNorm's gains of the lane's columns are loaded before the last four to seven
  // steps, so their latency hides behind them instead of following the loop.  They are
  // younger than the DMA loads of the stages the first two remaining steps wait for, so
  // those two waits allow NH more loads in flight.
  constexpr bool HV_PRE = EPI == EPI_RESID && TRANS;
  constexpr int NH = HV_PRE ? WM * WN + WN : 0;
  static_assert(2 * LPW + NH <= 63, "vmcnt range");
  float4 hv_pre[HV_PRE ? WM : 1][HV_PRE ? WN : 1];
  uint2 gn_pre[HV_PRE ? WN : 1];  // 4 gains (bf16) of block j's columns
  if constexpr (HV_PRE) {
#pragma unroll
    for (int j = 0; j < WN; ++j) {
      const int n0 = (tn * BFR + wn * WN + j) * 16 + 4 * (lane_t >> 4);
      const int nc = n0 < g.N ? n0 : 0;  // columns past N: a valid piece, unused
      gn_pre[j] = *reinterpret_cast<const uint2*>(static_cast<const bf16*>(g.gain) + nc);
#pragma unroll
      for (int i = 0; i < WM; ++i) {
        const int m = min(m0 + (wm * WM + i) * 16 + (lane_t & 15), M - 1);  // rows past M: a valid row, unused
        hv_pre[i][j] = *reinterpret_cast<const float4*>(g.h + static_cast<size_t>(m) * g.N + nc);
      }
    }
  }
  // XT: from here on the DMA sources are the next tile's; its stage v (v < 3) goes into
  // buffer v at step S - 4 + v, whose stage was read during the previous step, before
  // that step's barrier (stage 3 waits for the barrier after the loop: the step before
  // S - 1 ends without one).  The waits of steps S - 4 and S - 3 then have two stages'
  // loads younger than the one they wait for, as in the main loop.
  if (XT) set_src(L_next % g.m_tiles, L_next / g.m_tiles, 0);
#define DFLASH_STEP(u, fac, fbc, fan, fbn, X)                                                       \
  if (s + u < S) {                                                                                  \
    const bool cur_ = s + u + 4 < S;                                                                \
    step_work((u + 1) & 3, fac, fbc, fan, fbn, cur_ || (XT && s + u + 4 - S < 3),                   \
              cur_ ? s + u + 4 : s + u + 4 - S, u);                                                 \
    if (s + u + 2 < S) {                                                                            \
      asm volatile("" ::: "memory");                                                                \
      if (cur_ || XT) __builtin_amdgcn_s_waitcnt(vm_lgkm_wait(2 * LPW + (X)));                      \
      else if (s + u + 3 < S) __builtin_amdgcn_s_waitcnt(vm_lgkm_wait(LPW + (X)));                  \
      else __builtin_amdgcn_s_waitcnt(vm_lgkm_wait(X));                                             \
      __builtin_amdgcn_s_barrier();                                                                 \
      asm volatile("" ::: "memory");                                                                \
    }                                                                                               \
  }
  if (s < S) {
    DFLASH_STEP(0, fa0, fb0, fa1, fb1, NH)
    DFLASH_STEP(1, fa1, fb1, fa0, fb0, NH)
    DFLASH_STEP(2, fa0, fb0, fa1, fb1, 0)
    DFLASH_STEP(3, fa1, fb1, fa0, fb0, 0)
    s += 4;
  }
  for (; s < S; s += 4) {
    DFLASH_STEP(0, fa0, fb0, fa1, fb1, 0)
    DFLASH_STEP(1, fa1, fb1, fa0, fb0, 0)
    DFLASH_STEP(2, fa0, fb0, fa1, fb1, 0)
    DFLASH_STEP(3, fa1, fb1, fa0, fb0, 0)
  }
#undef DFLASH_STEP
  __syncthreads();  // every wavefront is done with the stage buffers

  // persistent launch: the next tile's first four stages are in flight from here on,
  // so their loads overlap this tile's epilogue (which works from the accumulators, not
  // the LDS)
  if constexpr (PERS) {
    if (L_next < L_end) {
      if (XT) {
        issue(3, 3);
      } else {
        set_src(L_next % g.m_tiles, L_next / g.m_tiles, 0);
        issue_prologue(g.S);
      }
    }
  }

  float(*tile)[kBN + 4] = reinterpret_cast<float(*)[kBN + 4]>(smem);

  if constexpr (EPI != EPI_ARGMAX && EPI != EPI_SAMPLE) {  // the LM head never splits K
    if (g.splits > 1) {
      // Split K: the partial tile goes out in the accumulators' own layout (one
      // 16-byte value per lane and 16 x 16 block, a whole 1 KB per wavefront store);
      // gemm_tiled_reduce_kernel, launched next, sums the splits and runs the epilogue
      f32x4* part = reinterpret_cast<f32x4*>(g.partials);
#pragma unroll
      for (int i = 0; i < WM; ++i)
#pragma unroll
        for (int j = 0; j < WN; ++j) part[tiled_part_index<C>(split, g.m_tiles, n_big, tm, tn, wave, i, j, lane_t)] = acc[i][j];
      return;
    }
  }

  if constexpr (EPI == EPI_ARGMAX) {
    // The greedy LM head multiplies W A^T (the operands swapped): lane l, register r of
    // block (i, j) holds row (wm WM + i) 16 + l % 16 and vocabulary column
    // (tn BFR + wn WN + j) 16 + 4 (l / 16) + r, so a lane holds 4 WN columns of one row.
    const int nbase = (tn * BFR + wn * WN) * 16 + 4 * (lane_t >> 4);
    if (g.logits != nullptr) {  // logits out (uniform branch; tests only)
#pragma unroll
      for (int i = 0; i < WM; ++i) {
        const int r = (wm * WM + i) * 16 + (lane_t & 15), m = m0 + r;
        if (m >= M) continue;
        const size_t mo = g.row_map != nullptr ? g.row_map[m] : m;
#pragma unroll
        for (int j = 0; j < WN; ++j)
#pragma unroll
          for (int rr = 0; rr < 4; ++rr) {
            const int n = nbase + j * 16 + rr;
            if (n < g.N) g.logits[mo * g.N + n] = acc[i][j][rr] * rs_s[r];
          }
      }
    }
    // split-vocab argmax straight from the accumulators: per row the largest scaled
    // logit of the wavefront's columns (columns past N excluded) in-lane, then across
    // the four lanes l, l^16, l^32, l^48 that share the row (lane-group swaps), then the
    // smallest column holding it the same way, then the row's 64-bit key (order-
    // preserving value bits, ~column) across the NWN column wavefronts through an LDS
    // max.  Equal values go to the smallest column; NaN logits are never picked.
    // FULL: every column of the tile is below N (all tiles but the last), no masks
    auto argmax_rows = [&](auto full) {
      constexpr bool FULL = decltype(full)::value;
#pragma unroll
      for (int i = 0; i < WM; ++i) {
        const int r = (wm * WM + i) * 16 + (lane_t & 15);
        const float f = rs_s[r];
        float v[WN][4], mx = -INFINITY;
#pragma unroll
        for (int j = 0; j < WN; ++j)
#pragma unroll
          for (int rr = 0; rr < 4; ++rr) {
            v[j][rr] = acc[i][j][rr] * f;
            mx = fmaxf(mx, FULL || nbase + j * 16 + rr < g.N ? v[j][rr] : -INFINITY);
          }
        mx = lane_group_max(mx);
        uint32_t col = 0xFFFFFFFFu;
#pragma unroll
        for (int j = WN - 1; j >= 0; --j)
#pragma unroll
          for (int rr = 3; rr >= 0; --rr) {
            const int n = nbase + j * 16 + rr;
            col = (FULL || n < g.N) && v[j][rr] == mx ? static_cast<uint32_t>(n) : col;
          }
        col = lane_group_min(col);
        if ((lane_t >> 4) == 0 && col != 0xFFFFFFFFu) atomicMax(&best_s[r], argmax_key(mx, static_cast<int>(col)));
      }
    };
    if ((tn + 1) * C::BN <= g.N) argmax_rows(std::true_type{});
    else argmax_rows(std::false_type{});
  } else if constexpr (EPI == EPI_SAMPLE) {
    // sampled drafts straight from the accumulators: for each pair of adjacent 16 x 16
    // column blocks (2p, 2p + 1) one Philox block gives the noise of the lane's 4 rows
    // x 2 columns; per row the best key of s + noise (s = logits / T) and the
    // log-sum-exp pair of s go across the 16 lanes sharing the row (DPP), then across
    // the NWN column wavefronts through LDS (the stage buffers are dead)
    float2* lse_s = reinterpret_cast<float2*>(smem);  // [BM][NWN]
    const unsigned long long step = g.step_dev != nullptr ? *g.step_dev : g.step;
#pragma unroll
    for (int i = 0; i < WM; ++i) {
      const int rb = (wm * WM + i) * 16 + 4 * (lane_t >> 4);
      uint32_t h[WN / 2][8];
#pragma unroll
      for (int p = 0; p < WN / 2; ++p) {
        const int cb = tn * BFR + wn * WN + 2 * p;  // even: BFR and WN are
        philox_u32x8<true>(16ull * static_cast<unsigned>(cb >> 1) + static_cast<unsigned>(lane_t & 15),
                     static_cast<unsigned>((m0 + rb) >> 2), step, 0ull, g.seed, kStreamDraft, h[p]);
      }
#pragma unroll
      for (int rr = 0; rr < 4; ++rr) {
        const int r = rb + rr, m = m0 + r;
        const float f = rs_s[r];
        unsigned long long key = 0ull;
        float sv[WN], mx = -INFINITY;
#pragma unroll
        for (int j = 0; j < WN; ++j) {
          const int n = (tn * BFR + wn * WN + j) * 16 + (lane_t & 15);
          sv[j] = -INFINITY;
          if (n < g.N && m < M) {
            const float z = acc[i][j][rr] * f;
            if (g.logits != nullptr) g.logits[static_cast<size_t>(m) * g.N + n] = z;
            sv[j] = z * g.inv_temp;
            const unsigned long long kj = argmax_key(sv[j] + gumbel_f32(h[j >> 1][2 * rr + (j & 1)]), n);
            key = kj > key ? kj : key;
          }
          mx = fmaxf(mx, sv[j]);
        }
        float sm = 0.f;
        if (mx != -INFINITY) {
#pragma unroll
          for (int j = 0; j < WN; ++j) sm += __builtin_amdgcn_exp2f((sv[j] - mx) * kLog2e);
        }
        // across the 16 lanes of the row: DPP quad permutations, half-row and row mirrors
        dpp_sample_round<0xB1>(key, mx, sm);
        dpp_sample_round<0x4E>(key, mx, sm);
        dpp_sample_round<0x141>(key, mx, sm);
        dpp_sample_round<0x140>(key, mx, sm);
        if ((lane_t & 15) == 0) {
          if (key != 0ull) atomicMax(&best_s[r], key);
          lse_s[r * NWN + wn] = make_float2(mx, sm);
        }
      }
    }
  } else if constexpr (EPI == EPI_RESID && TRANS) {
    // Residual add from the accumulators: a lane holds 4 consecutive columns of one row
    // per 16 x 16 block; x = acc * rs + h goes back to the residual stream (16 bytes) and,
    // times the next RMSNorm's gain, into the packed next operand (8 bytes); the row's
    // sum of x^2 over each 64-column subtile (its 4 blocks, then the four lanes l, l^16,
    // l^32, l^48) is that subtile's RMSNorm partial.
    typedef typename ActOf<bf16>::type TA;
    typedef TA TA4 __attribute__((ext_vector_type(4)));
    TA* out = static_cast<TA*>(g.out);
    bool bad = false;
#pragma unroll
    for (int i = 0; i < WM; ++i) {
      const int r = (wm * WM + i) * 16 + (lane_t & 15), m = m0 + r;
      const float f = rs_s[r];
      const bool row_ok = m < M;
#pragma unroll
      for (int sj = 0; sj < WN / 4; ++sj) {
        const int tile_n = tn * SUB + (wn * WN) / 4 + sj;  // 64-column subtile
        float ss = 0.f;
#pragma unroll
        for (int jj = 0; jj < 4; ++jj) {
          const int j = 4 * sj + jj;
          const int n0 = (tn * BFR + wn * WN + j) * 16 + 4 * (lane_t >> 4);
          const float4 hv = hv_pre[i][j];
          const float x[4] = {acc[i][j][0] * f + hv.x, acc[i][j][1] * f + hv.y, acc[i][j][2] * f + hv.z,
                              acc[i][j][3] * f + hv.w};
          const bf16* gq = reinterpret_cast<const bf16*>(&gn_pre[j]);
          TA4 y;
          bool sat = false;
#pragma unroll
          for (int k = 0; k < 4; ++k) y[k] = to_act<TA>(x[k] * to_f32(gq[k]), sat);
          if (row_ok && n0 < g.N) {
            *reinterpret_cast<TA4*>(out + pa_index(m, n0, g.out_steps)) = y;
            *reinterpret_cast<float4*>(g.h + static_cast<size_t>(m) * g.N + n0) = make_float4(x[0], x[1], x[2], x[3]);
            ss += (x[0] * x[0] + x[1] * x[1]) + (x[2] * x[2] + x[3] * x[3]);
            bad = bad || sat;
          }
        }
        ss = lane_group_sum(ss);
        if ((lane_t >> 4) == 0 && row_ok && tile_n < g.n_tiles) g.ssq_out[static_cast<size_t>(m) * g.np_out + tile_n] = ss;
      }
    }
    report_overflow(bad, g.dev_error);
  } else if constexpr (EPI == EPI_SWIGLU && TRANS) {
    // SwiGLU from the accumulators: wavefront column blocks 4s, 4s + 1 are the gate
    // columns and 4s + 2, 4s + 3 the up columns of 64-column subtile s (32 FFN
    // columns); a lane holds 4 consecutive FFN columns of one row and writes them as
    // one 8-byte piece of the packed down-projection operand.  Columns past ffn are
    // the down projection's K padding and get zeros.
    typedef typename ActOf<bf16>::type TA;
    typedef TA TA4 __attribute__((ext_vector_type(4)));
    TA* act = static_cast<TA*>(g.out);
    bool bad = false;
#pragma unroll
    for (int i = 0; i < WM; ++i) {
      const int r = (wm * WM + i) * 16 + (lane_t & 15), m = m0 + r;
      const float f = rs_s[r];
#pragma unroll
      for (int sj = 0; sj < WN / 4; ++sj)
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          const int tile_n = tn * SUB + (wn * WN) / 4 + sj;  // 64-column subtile
          const int c0 = tile_n * 32 + h * 16 + 4 * (lane_t >> 4);
          TA4 y;
          bool sat = false;
#pragma unroll
          for (int rr = 0; rr < 4; ++rr) {
            const float gq = acc[i][4 * sj + h][rr] * f, uq = acc[i][4 * sj + 2 + h][rr] * f;
            const float v = gq * __builtin_amdgcn_rcpf(1.f + __builtin_amdgcn_exp2f(-gq * kLog2e)) * uq;
            y[rr] = to_act<TA>(c0 + rr < g.ffn ? v : 0.f, sat);
          }
          // rows past M (compacted away) and subtiles past n_tiles (the last tile of a
          // ragged N) do not exist: nothing stored, nothing reported
          if (m < M && tile_n < g.n_tiles) {
            *reinterpret_cast<TA4*>(act + pa_index(m, c0, g.out_steps)) = y;
            bad = bad || sat;
          }
        }
    }
    report_overflow(bad, g.dev_error);
    // a later tile of a persistent workgroup rewrites rs_s for new rows
    if (L_next < L_end) __syncthreads();
  } else {
    // The tile goes through the fused epilogue 64 columns at a time, C::PAIR subtiles
    // per round (each in its own LDS tile), the rows' QKV / INJECT targets found once.
    constexpr bool ROWS = EPI == EPI_QKV || EPI == EPI_INJECT;  // with the angle table
    EpiRows<BM, NT> er{};
    if constexpr (ROWS)
      if (g.rope_tab != nullptr) epilogue_rows<EPI, BM, NT>(g, m0, M, er);
    constexpr int PAIR = C::PAIR;
    float(*tiles)[BM][kBN + 4] = reinterpret_cast<float(*)[BM][kBN + 4]>(smem);
#pragma unroll
    for (int s0 = 0; s0 < SUB; s0 += PAIR) {
      __syncthreads();
#pragma unroll
      for (int j = 0; j < WN; ++j) {
        const int cb = wn * WN + j;  // column block of the workgroup tile
        if (cb / 4 < s0 || cb / 4 >= s0 + PAIR) continue;
#pragma unroll
        for (int i = 0; i < WM; ++i)
#pragma unroll
          for (int rr = 0; rr < 4; ++rr)
            tiles[cb / 4 - s0][(wm * WM + i) * 16 + 4 * (lane_t >> 4) + rr][(cb & 3) * 16 + (lane_t & 15)] = acc[i][j][rr];
      }
      __syncthreads();
#pragma unroll
      for (int q = 0; q < PAIR; ++q) {
        const int tile_n = tn * SUB + s0 + q;
        if (s0 + q < SUB && tile_n < g.n_tiles) {
          if (ROWS && g.rope_tab != nullptr) epilogue_tile<bf16, EPI, BM, NT, false, ROWS>(g, tiles[q], rs_s, tile_n, m0, M, nullptr, er);
          else epilogue_tile<bf16, EPI, BM, NT>(g, tiles[q], rs_s, tile_n, m0, M, nullptr);
        }
      }
    }
  }

  if constexpr (EPI == EPI_ARGMAX || EPI == EPI_SAMPLE) {
    __syncthreads();
    for (int r = tid_t; r < BM; r += NT)
      if (m0 + r < M) g.keys[static_cast<size_t>(m0 + r) * g.n_parts + tn] = best_s[r];
    if constexpr (EPI == EPI_SAMPLE) {
      const float2* lse_s = reinterpret_cast<const float2*>(smem);
      for (int r = tid_t; r < BM; r += NT) {
        if (m0 + r >= M) continue;
        float mx = -INFINITY, sm = 0.f;
#pragma unroll
        for (int w = 0; w < NWN; ++w) lse_merge(mx, sm, lse_s[r * NWN + w].x, lse_s[r * NWN + w].y);
        g.lse_part[static_cast<size_t>(m0 + r) * g.n_parts + tn] = make_float2(mx, sm);
      }
    }
    // the row's draft is the largest tile key: launch_head_finalize, after this kernel
  }
  if (L_next >= L_end) return;
  L = L_next;
  }
}

// Split-K reduction and epilogue of the tiled GEMM: one workgroup (4 wavefronts) per
// (tile, 64-column subtile).  The subtile's 16 x 16 blocks are summed over the splits
// in split order (plain loads: the partials were written by the previous kernel),
// placed in the LDS tile, and the subtile goes through the same fused epilogue as an
// unsplit tile.
template <int EPI, int NWM, int NWN, int WM, int WN>
__global__ __launch_bounds__(kThreads) void gemm_tiled_reduce_kernel(GemmArgs g) {
  using C = TileCfg<NWM, NWN, WM, WN>;
  constexpr int BM = C::BM, SUB = C::SUB, AFR = C::AFR;
  constexpr int NF = AFR * 4;                       // 16 x 16 blocks of one subtile
  constexpr int FPW = NF / (kThreads / kWave);      // blocks per wavefront
  static_assert(NF % (kThreads / kWave) == 0, "blocks split evenly over the wavefronts");
  __shared__ __attribute__((aligned(16))) float tile[BM][kBN + 4];
  __shared__ float rs_s[BM];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int n_big = (g.n_tiles + SUB - 1) / SUB;
  const int sub = blockIdx.x % SUB, t = blockIdx.x / SUB;
  const int tm = t % g.m_tiles, tn = t / g.m_tiles;
  const int m0 = tm * BM, tile_n = tn * SUB + sub;
  int M = g.M;
  if (g.m_live != nullptr) M = min(M, max(*g.m_live, 0));
  if (m0 >= M || tile_n >= g.n_tiles) return;  // uniform per workgroup
  const f32x4* part = reinterpret_cast<const f32x4*>(g.partials);
  // block f of the subtile: row block rb = f / 4, column block cb = SUB-relative f % 4
  auto src = [&](int sp, int f) -> size_t {
    const int rb = f >> 2, cb = sub * 4 + (f & 3);
    const int wm = rb / WM, i = rb % WM, wn = cb / WN, j = cb % WN;
    return tiled_part_index<C>(sp, g.m_tiles, n_big, tm, tn, wm + NWM * wn, i, j, lane);
  };
  f32x4 sum[FPW];
#pragma unroll
  for (int q = 0; q < FPW; ++q) sum[q] = part[src(0, wave * FPW + q)];
  for (int sp = 1; sp < g.splits; ++sp) {
    f32x4 v[FPW];
#pragma unroll
    for (int q = 0; q < FPW; ++q) v[q] = part[src(sp, wave * FPW + q)];
#pragma unroll
    for (int q = 0; q < FPW; ++q) sum[q] += v[q];
  }
  // MFMA layout: lane l, register r holds row 4 * (l / 16) + r, column l % 16 (a
  // transposed product: row l % 16, column 4 * (l / 16) + r)
#pragma unroll
  for (int q = 0; q < FPW; ++q) {
    const int f = wave * FPW + q, rb = f >> 2, cb = f & 3;
#pragma unroll
    for (int rr = 0; rr < 4; ++rr) {
      if constexpr (tiled_trans<EPI, NWM, NWN, WM, WN>()) tile[rb * 16 + (lane & 15)][cb * 16 + 4 * (lane >> 4) + rr] = sum[q][rr];
      else tile[rb * 16 + 4 * (lane >> 4) + rr][cb * 16 + (lane & 15)] = sum[q][rr];
    }
  }
  for (int r = tid; r < BM; r += kThreads) {
    float f = 1.f;
    if (g.ssq_in != nullptr && m0 + r < g.M) {
      const float* row = g.ssq_in + static_cast<size_t>(m0 + r) * g.np_in;
      float ssum = 0.f;
      for (int k = 0; k < g.np_in; ++k) ssum += row[k];
      f = 1.f / sqrtf(ssum / static_cast<float>(g.norm_dim) + g.eps);
    }
    rs_s[r] = f;
  }
  __syncthreads();
  epilogue_tile<bf16, EPI, BM, kThreads>(g, tile, rs_s, tile_n, m0, M, nullptr);
}

template <int EPI, int NWM, int NWN, int WM, int WN>
static hipError_t launch_cfg(const GemmPlan& p, const GemmArgs& a, hipStream_t s) {
  using C = TileCfg<NWM, NWN, WM, WN>;
  const int n_big = (p.n_tiles + C::SUB - 1) / C::SUB;
  long long grid = static_cast<long long>(p.m_tiles) * n_big * p.splits;
  if (p.m_tiles != (a.M + C::BM - 1) / C::BM || grid <= 0 || grid > (1ll << 31) - 1) return hipErrorInvalidValue;
  if (a.persist != 0) {
    // persistent launch: one workgroup per CU (the 8-wavefront tiles hold one), the
    // same number on every XCD, each with at least two tiles
    if (!tiled_trans<EPI, NWM, NWN, WM, WN>() || EPI == EPI_RESID || p.splits != 1 || C::NW != 8 ||
        a.persist % 8 != 0 || grid < 2ll * a.persist)
      return hipErrorInvalidValue;
    grid = a.persist;
  }
  hipLaunchKernelGGL((gemm_tiled_kernel<EPI, NWM, NWN, WM, WN>), dim3(static_cast<unsigned>(grid)), dim3(C::NT), 0, s, a);
  if (p.splits > 1) {
    if constexpr (EPI == EPI_ARGMAX || EPI == EPI_SAMPLE) {
      return hipErrorInvalidValue;
    } else {
      if (hipGetLastError() != hipSuccess) return hipErrorLaunchFailure;
      const long long rgrid = static_cast<long long>(p.m_tiles) * n_big * C::SUB;
      hipLaunchKernelGGL((gemm_tiled_reduce_kernel<EPI, NWM, NWN, WM, WN>), dim3(static_cast<unsigned>(rgrid)),
                         dim3(kThreads), 0, s, a);
    }
  }
  return hipGetLastError();
}

template <int EPI>
static hipError_t launch_tile(const GemmPlan& p, const GemmArgs& a, hipStream_t s) {
  switch (p.mt) {
    case kTile256: return launch_cfg<EPI, 2, 4, 8, 4>(p, a, s);
    case kTile128: return launch_cfg<EPI, 2, 2, 4, 4>(p, a, s);
    case kTile128x384: return launch_cfg<EPI, 2, 4, 4, 6>(p, a, s);
    case kTile256x128: return launch_cfg<EPI, 4, 2, 4, 4>(p, a, s);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_gemm_tiled(int epi, const GemmPlan& plan, const GemmArgs& a, hipStream_t stream) {
  if (plan.n_tiles <= 0 || plan.m_tiles <= 0 || plan.splits <= 0 || a.S <= 0) return hipErrorInvalidValue;
  if (a.steps_per_split * (plan.splits - 1) >= a.S) return hipErrorInvalidValue;  // every split has a step
  switch (epi) {
    case EPI_FUSE: return launch_tile<EPI_FUSE>(plan, a, stream);
    case EPI_INJECT: return launch_tile<EPI_INJECT>(plan, a, stream);
    case EPI_QKV: return launch_tile<EPI_QKV>(plan, a, stream);
    case EPI_RESID: return launch_tile<EPI_RESID>(plan, a, stream);
    case EPI_SWIGLU: return launch_tile<EPI_SWIGLU>(plan, a, stream);
    case EPI_ARGMAX: return plan.splits == 1 ? launch_tile<EPI_ARGMAX>(plan, a, stream) : hipErrorInvalidValue;
    case EPI_SAMPLE: return plan.splits == 1 ? launch_tile<EPI_SAMPLE>(plan, a, stream) : hipErrorInvalidValue;
    default: return hipErrorInvalidValue;
  }
}

}  // namespace dflash
