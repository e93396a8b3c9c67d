// Persistent layer kernel for the weight-streaming draft step (bf16 drafters whose
// block rows fit the streaming GEMM, head_dim 128).
//
// The pages' system removes the microsecond-scale gaps between operators by running
// the model as one persistent engine (the hotdry blog's TileRT section: one
// long-lived kernel walks tile-level tasks; the aufer article's micro-op section: the
// gaps between small operators dominate at batch 1).  Here one launch runs a whole
// draft layer: QKV projection -> block attention -> key-split merge -> O projection
// -> gate/up + SwiGLU -> down projection.  The grid is co-resident (at most the
// occupancy limit times the CUs); each phase's work items (the same items, with the
// same split-K plans, as the separate kernels' workgroups, so the results are
// bitwise those of the separate kernels) go round-robin over the workgroups, and an
// item waits only for the items whose results it reads (below), so the phases
// overlap where the dependencies allow.
//
// What the single launch buys: a projection's weights do not depend on the previous
// phase, so a workgroup issues the weight loads of its next item's first pipeline
// stages before it waits, and the weight stream continues through the phase
// boundary instead of draining and ramping up again around a kernel launch.
//
// Coherence: the eight XCD L2 caches are not coherent with each other inside one
// launch, so everything that crosses a phase boundary (q/k/v, attention partials and
// output, the residual stream, RMSNorm inputs and partial sums, the SwiGLU
// activations) is written and read with device-coherent accesses (the COH bodies).
// The MLP's normalised input and its RMSNorm partials have buffers of their own, so
// the O projection never overwrites what a late QKV item may still read.
#include "attention_body.h"
#include "common.h"
#include "epilogue.h"
#include "gemm.h"
#include "gemm_body.h"
#include "internal.h"

namespace dflash {

constexpr int kPersistDH = 128;
constexpr int kPersistKG = 2;

template <int MT, int NW>
struct PersistLds {
  union {
    StreamLds<MT> gemm;
    AttnLds<f16, kPersistDH, NW, kPersistKG> attn;
    MergeLds<kPersistDH, 8> merge;
  };
  int flag;
};

// Dependencies between work items instead of barriers between phases: a workgroup
// that finishes an output tile (or an attention item) adds one to the signal word of
// what it produced once its stores have completed; a work item waits, before it
// reads anything produced in this launch, until the words of exactly the tiles it
// consumes are complete:
//   attention of kv group g   all QKV tiles of g's q heads and of its k and v heads
//   merge of row group r      every key split of r
//   O piece, K steps s..e     the attention output of the heads covering s..e
//   gate/up                   every O tile (RMSNorm needs whole rows)
//   down piece, K steps s..e  the gate/up tiles s..e (tile t produces act step t)
// Every wait is on items of an earlier phase and every workgroup walks the phases in
// order, so on a co-resident grid every wait ends; it is bounded anyway (kSpinLimit
// polls, then the time-out error bit and a uniform false) so nothing can hang.

// One thread polls until *c >= need (uniform result).
__device__ __forceinline__ bool poll_ge(const unsigned* c, unsigned need, uint32_t* dev_error) {
  for (long long it = 0; __hip_atomic_load(const_cast<unsigned*>(c), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) < need;
       ++it) {
    if (it > kSpinLimit) {
      atomicOr(dev_error, kErrTimeout);
      return false;
    }
    __builtin_amdgcn_s_sleep(1);
  }
  return true;
}

// Thread 0 waits for words c[0], c[stride], .. c[(n-1) stride] >= need; uniform result.
__device__ __forceinline__ bool wait_words(const unsigned* c, int n, int stride, unsigned need, uint32_t* dev_error,
                                           int* flag_lds) {
  if (threadIdx.x == 0) {
    int ok = 1;
    for (int i = 0; i < n && ok; ++i) ok = poll_ge(c + static_cast<size_t>(i) * stride, need, dev_error) ? 1 : 0;
    *flag_lds = ok;
  }
  __syncthreads();
  return *flag_lds != 0;
}

// This workgroup's stores have completed; then one thread adds one to *c, and the
// producer whose add completes the count (need) sets c's ready flag, the word waiters
// poll: polling the counter itself while producers still add to it is much slower.
__device__ __forceinline__ void signal_add(unsigned* c, unsigned need) {
  wait_memory();
  __syncthreads();
  if (threadIdx.x == 0 && __hip_atomic_fetch_add(c, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) + 1 == need)
    __hip_atomic_store(c + kSigReady, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Thread 0 waits for the ready flags of counter words c[0], c[stride], ..; uniform.
__device__ __forceinline__ bool wait_ready(const unsigned* c, int n, int stride, uint32_t* dev_error, int* flag_lds) {
  return wait_words(c + kSigReady, n, stride, 1u, dev_error, flag_lds);
}

template <int MT, int NW>
__global__ __launch_bounds__(kThreads, 2) void layer_kernel(LayerArgs a) {
  // pipeline depth: as the separate kernels, but 6 at one row block (8 would spill at
  // the two waves per SIMD the co-resident grid needs)
  constexpr int D = MT == 4 ? 2 : (MT == 1 ? 6 : 4);
  __shared__ PersistLds<MT, NW> lds;
  const int n_wg = gridDim.x;
  bool ok = true;  // uniform: false once a wait timed out
  unsigned* sig = a.sig;
  const int Hq = a.gemm[0].n_q_heads, Hkv = a.gemm[0].n_kv_heads, G = a.group, tph = a.tiles_per_head;

  // GEMM phase i: items round-robin; `wait(tile_n, s_lo, s_hi)` runs once the item's
  // first weight loads are in flight, `done(tile_n)` after the epilogue of a tile
  auto gemm_phase = [&](auto epi_tag, int i, auto wait, auto done) {
    constexpr int EPI = decltype(epi_tag)::value;
    const GemmArgs& g = a.gemm[i];
    const PhaseGrid pg = a.grid[i];
    const int n = pg.x * pg.y * pg.z;
    for (int item = blockIdx.x; item < n && ok; item += n_wg) {
      __syncthreads();  // the previous item is done with LDS
      gemm_body<bf16, MT, EPI, D, true>(
          g, item % pg.x, (item / pg.x) % pg.y, item / (pg.x * pg.y), lds.gemm,
          [&](int tile_n, int s_lo, int s_hi) {
            if (ok) ok = wait(tile_n, s_lo, s_hi);
          },
          done);
    }
  };
  auto no_wait = [](int, int, int) { return true; };

  // QKV projection: a finished tile counts towards its kv group
  const unsigned qkv_need = static_cast<unsigned>((G + 2) * tph);
  gemm_phase(std::integral_constant<int, EPI_QKV>{}, 0, no_wait, [&](int tile_n) {
    const int hd = tile_n / tph;
    const int g = hd < Hq ? hd / G : (hd < Hq + Hkv ? hd - Hq : hd - Hq - Hkv);
    signal_add(&sig[kSigQkv + g], qkv_need);
  });

  // attention items ((b, g, rb) row group, key split)
  const AttnArgs& at = a.attn;
  const unsigned att_need = static_cast<unsigned>(at.max_splits), fin_need = static_cast<unsigned>(a.fin_need);
  for (int item = blockIdx.x; item < a.attn_items && ok; item += n_wg) {
    const int grp = item / at.max_splits, g = (grp / at.n_rb) % Hkv;
    __syncthreads();
    if (!(ok = wait_ready(&sig[kSigQkv + g], 1, 1, a.dev_error, &lds.flag))) break;
    attention_body<f16, kPersistDH, NW, kPersistKG, true>(at, item, lds.attn);
    if (a.merge_items == 0) signal_add(&sig[kSigFin + g], fin_need);
    else signal_add(&sig[kSigAtt + grp], att_need);
  }
  // merge items (one row of a row group each)
  for (int item = blockIdx.x; item < a.merge_items && ok; item += n_wg) {
    const int grp = item / at.rows_per_block, g = (grp / at.n_rb) % Hkv;
    __syncthreads();
    if (!(ok = wait_ready(&sig[kSigAtt + grp], 1, 1, a.dev_error, &lds.flag))) break;
    merge_body<f16, kPersistDH, 8, true>(at, item, lds.merge);
    signal_add(&sig[kSigFin + g], fin_need);
  }

  // O projection + residual: a piece reads the attention output of its K steps' heads
  const int dh = a.gemm[0].head_dim;
  gemm_phase(
      std::integral_constant<int, EPI_RESID>{}, 1,
      [&](int, int s_lo, int s_hi) {
        const int g0 = (s_lo * kKStep / dh) / G, g1 = ((s_hi * kKStep - 1) / dh) / G;
        return wait_ready(&sig[kSigFin + g0], g1 - g0 + 1, 1, a.dev_error, &lds.flag);
      },
      [&](int) { signal_add(&sig[kSigO], static_cast<unsigned>(a.o_tiles)); });

  // gate/up + SwiGLU: every O tile (RMSNorm of whole rows)
  gemm_phase(
      std::integral_constant<int, EPI_SWIGLU>{}, 2,
      [&](int, int, int) {
        return wait_ready(&sig[kSigO], 1, 1, a.dev_error, &lds.flag);
      },
      [&](int tile_n) { signal_add(&sig[kSigGu + tile_n], 1u); });

  // down + residual: a piece reads act steps s_lo .. s_hi-1, produced by gate/up tiles
  // with the same indices
  gemm_phase(
      std::integral_constant<int, EPI_RESID>{}, 3,
      [&](int, int s_lo, int s_hi) {
        return wait_ready(&sig[kSigGu + s_lo], s_hi - s_lo, 1, a.dev_error, &lds.flag);
      },
      [](int) {});
}

template <int MT, int NW>
static hipError_t launch_mt_nw(const LayerArgs& a, int grid, hipStream_t s) {
  hipLaunchKernelGGL((layer_kernel<MT, NW>), dim3(grid), dim3(kThreads), 0, s, a);
  return hipGetLastError();
}

template <int MT, int NW>
static int capacity_mt_nw(int cus) {
  int per_cu = 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, layer_kernel<MT, NW>, kThreads, 0) != hipSuccess)
    return 0;
  return per_cu * cus;
}

static bool persist_shape_ok(int mt, int nw) { return (mt == 1 || mt == 2 || mt == 4) && (nw == 1 || nw == 2); }

int persistent_capacity(int mt, int nw, int cus) {
  if (!persist_shape_ok(mt, nw)) return 0;
  switch (mt * 10 + nw) {
    case 11: return capacity_mt_nw<1, 1>(cus);
    case 12: return capacity_mt_nw<1, 2>(cus);
    case 21: return capacity_mt_nw<2, 1>(cus);
    case 22: return capacity_mt_nw<2, 2>(cus);
    case 41: return capacity_mt_nw<4, 1>(cus);
    default: return capacity_mt_nw<4, 2>(cus);
  }
}

hipError_t launch_layer_persistent(const LayerArgs& a, int mt, int nw, int grid, hipStream_t stream) {
  if (!persist_shape_ok(mt, nw) || grid <= 0) return hipErrorInvalidValue;
  switch (mt * 10 + nw) {
    case 11: return launch_mt_nw<1, 1>(a, grid, stream);
    case 12: return launch_mt_nw<1, 2>(a, grid, stream);
    case 21: return launch_mt_nw<2, 1>(a, grid, stream);
    case 22: return launch_mt_nw<2, 2>(a, grid, stream);
    case 41: return launch_mt_nw<4, 1>(a, grid, stream);
    default: return launch_mt_nw<4, 2>(a, grid, stream);
  }
}

}  // namespace dflash
