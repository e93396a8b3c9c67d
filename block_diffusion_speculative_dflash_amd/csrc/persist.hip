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
// bitwise those of the separate kernels) go round-robin over the workgroups, and a
// grid barrier separates dependent phases.
//
// What the single launch buys: a projection's weights do not depend on the previous
// phase, so a workgroup issues the weight loads of its next item's first pipeline
// stages before it waits at the barrier, and the weight stream continues through the
// phase boundary instead of draining and ramping up again around a kernel launch.
//
// Coherence: the eight XCD L2 caches are not coherent with each other inside one
// launch, so everything that crosses a phase boundary (q/k/v, attention partials and
// output, the residual stream, RMSNorm inputs and partial sums, the SwiGLU
// activations) is written and read with device-coherent accesses (the COH bodies).
// A barrier is an arrival counter per phase: a workgroup waits for its own stores to
// complete, then adds one; waiting workgroups poll with a sleep and give up after a
// bounded number of polls, setting the time-out error bit instead of hanging.
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

// Grid barrier p: an arrival counter and a release flag on separate 128-byte lines
// (kBarrierWords words per barrier).  A workgroup done with a phase waits for its own
// stores to complete and adds one to the counter; the one that brings it to n_wg sets
// the flag.  Waiting workgroups poll only the flag, one thread each, with a sleep
// between polls, and give up after kSpinLimit polls (time-out error bit, uniform
// false) instead of hanging.
constexpr int kBarrierWords = 64;  // 256 bytes: counter at word 0, flag at word 32

__device__ __forceinline__ void grid_arrive(unsigned* bar, unsigned n_wg) {
  wait_memory();
  __syncthreads();
  if (threadIdx.x == 0) {
    const unsigned prev = __hip_atomic_fetch_add(bar, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    if (prev == n_wg - 1) __hip_atomic_store(bar + 32, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
}

__device__ __forceinline__ bool grid_wait(unsigned* bar, uint32_t* dev_error, int* flag_lds) {
  if (threadIdx.x == 0) {
    int ok = 1;
    for (long long it = 0; __hip_atomic_load(bar + 32, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) == 0u; ++it) {
      if (it > kSpinLimit) {
        ok = 0;
        atomicOr(dev_error, kErrTimeout);
        break;
      }
      __builtin_amdgcn_s_sleep(2);
    }
    *flag_lds = ok;
  }
  __syncthreads();
  return *flag_lds != 0;
}

template <int MT, int NW>
__global__ __launch_bounds__(kThreads, 2) void layer_kernel(LayerArgs a) {
  constexpr int D = MT == 4 ? 2 : (MT == 1 ? 8 : 4);
  __shared__ PersistLds<MT, NW> lds;
  const unsigned n_wg = gridDim.x;
  bool ok = true;  // uniform: false once a barrier timed out
  auto bar = [&](int p) { return a.barrier + p * kBarrierWords; };

  // GEMM phase: items round-robin; the first item's weight loads go out before the
  // wait for the previous phase (wait_bar < 0: nothing to wait for)
  auto gemm_phase = [&](auto epi_tag, int i, int wait_bar) {
    constexpr int EPI = decltype(epi_tag)::value;
    const GemmArgs& g = a.gemm[i];
    const PhaseGrid pg = a.grid[i];
    const int n = pg.x * pg.y * pg.z;
    bool waited = wait_bar < 0;
    for (int item = blockIdx.x; item < n && ok; item += n_wg) {
      __syncthreads();  // the previous item is done with LDS
      gemm_body<bf16, MT, EPI, D, true>(g, item % pg.x, (item / pg.x) % pg.y, item / (pg.x * pg.y), lds.gemm, [&] {
        if (!waited) {
          ok = grid_wait(bar(wait_bar), a.dev_error, &lds.flag);
          waited = true;
        }
      });
    }
    if (!waited && ok) ok = grid_wait(bar(wait_bar), a.dev_error, &lds.flag);
  };

  gemm_phase(std::integral_constant<int, EPI_QKV>{}, 0, -1);
  grid_arrive(bar(0), n_wg);
  if (ok) ok = grid_wait(bar(0), a.dev_error, &lds.flag);
  for (int item = blockIdx.x; item < a.attn_items && ok; item += n_wg) {
    __syncthreads();
    attention_body<f16, kPersistDH, NW, kPersistKG, true>(a.attn, item, lds.attn);
  }
  grid_arrive(bar(1), n_wg);
  int last = 1;
  if (a.merge_items > 0) {
    if (ok) ok = grid_wait(bar(1), a.dev_error, &lds.flag);
    for (int item = blockIdx.x; item < a.merge_items && ok; item += n_wg) {
      __syncthreads();
      merge_body<f16, kPersistDH, 8, true>(a.attn, item, lds.merge);
    }
    grid_arrive(bar(2), n_wg);
    last = 2;
  }
  gemm_phase(std::integral_constant<int, EPI_RESID>{}, 1, last);  // O projection + residual
  grid_arrive(bar(3), n_wg);
  gemm_phase(std::integral_constant<int, EPI_SWIGLU>{}, 2, 3);  // gate/up + SwiGLU
  grid_arrive(bar(4), n_wg);
  gemm_phase(std::integral_constant<int, EPI_RESID>{}, 3, 4);  // down + residual
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
