// Weight-streaming GEMM with fused epilogues: out[m, n] = sum_k A[m, k] * W[n, k].
//
// Every projection of the drafter is y = x W^T (nn.Linear layout).  At draft batch
// sizes x has few rows (B*k = 8 .. 72 at B <= 8), so the cost is reading W once from
// HBM.  Both operands are fragment-packed (see pa_index): every wavefront load is a
// 16-byte load per lane covering 1 KB of contiguous memory, the layout a 64-lane
// MFMA operand wants.  One workgroup (4 wavefronts) owns a 64-column output tile and
// a range of 32-wide K steps; wavefront w takes steps w, w+4, w+8, .. through a
// D-stage register pipeline (the loads of step i+D are in flight while step i is
// multiplied), with 16x16x32 fp16/bf16 MFMA (fp32 drafters: 16x16x4 fp32, eight per
// step).  The four wavefronts reduce through LDS in a fixed order.  When the tiles
// alone cannot fill the 256 CUs, K is split across workgroups: each writes an fp32
// partial tile and the last to arrive (device-scope counter) sums them in split
// order, so results are bitwise reproducible.
//
// The epilogue runs on the reduced tile in LDS and fuses what the method does next
// (RMSNorm factor of the input rows, RoPE, KV-ring scatter, residual add, SwiGLU,
// split-vocab argmax) and writes the next GEMM's operand already packed.  RMSNorm is
// folded as RMSNorm(x) W^T = ((x*g) W^T) * rsqrt(mean(x^2) + eps): the producer of x
// stores x*g and per-tile sums of x^2; the consumer applies the per-row factor to
// its accumulators (exact in real arithmetic, the projection being linear).
#include "gemm_body.h"

namespace dflash {

template <typename TIN, int MT, int EPI, int D>
__global__ __launch_bounds__(kThreads) void gemm_kernel(GemmArgs g) {
  __shared__ StreamLds<MT> lds;
  gemm_body<TIN, MT, EPI, D, false>(g, blockIdx.x, blockIdx.y, blockIdx.z, lds, [](int, int, int) {}, [](int) {});
}

template <typename TIN, int MT, int EPI>
static hipError_t launch_t(const GemmPlan& p, const GemmArgs& a, hipStream_t s) {
  const dim3 grid = p.piece_base > 0 ? dim3(p.n_tiles * p.piece_base + p.piece_extra, p.m_tiles, 1)
                                     : dim3(p.n_tiles, p.m_tiles, p.splits);
  constexpr int D = MT == 4 ? 2 : (MT == 1 ? 8 : 4);
  if (p.depth != D) return hipErrorInvalidValue;
  if (p.piece_base > 0 && (p.piece_extra >= p.n_tiles || p.splits != p.piece_base + (p.piece_extra > 0) ||
                           p.splits > 16 / MT || a.piece_base != p.piece_base || a.piece_extra != p.piece_extra))
    return hipErrorInvalidValue;
  hipLaunchKernelGGL((gemm_kernel<TIN, MT, EPI, D>), grid, dim3(kThreads), 0, s, a);
  return hipGetLastError();
}

template <typename TIN, int EPI>
static hipError_t launch_mt(const GemmPlan& p, const GemmArgs& a, hipStream_t s) {
  switch (p.mt) {
    case 1: return launch_t<TIN, 1, EPI>(p, a, s);
    case 2: return launch_t<TIN, 2, EPI>(p, a, s);
    case 4: return launch_t<TIN, 4, EPI>(p, a, s);
    default: return hipErrorInvalidValue;
  }
}

template <typename TIN>
static hipError_t launch_epi(int epi, const GemmPlan& p, const GemmArgs& a, hipStream_t s) {
  switch (epi) {
    case EPI_FUSE: return launch_mt<TIN, EPI_FUSE>(p, a, s);
    case EPI_INJECT: return launch_mt<TIN, EPI_INJECT>(p, a, s);
    case EPI_QKV: return launch_mt<TIN, EPI_QKV>(p, a, s);
    case EPI_RESID: return launch_mt<TIN, EPI_RESID>(p, a, s);
    case EPI_SWIGLU: return launch_mt<TIN, EPI_SWIGLU>(p, a, s);
    case EPI_ARGMAX: return launch_mt<TIN, EPI_ARGMAX>(p, a, s);
    case EPI_SAMPLE: return launch_mt<TIN, EPI_SAMPLE>(p, a, s);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_gemm(int epi, bool f32, const GemmPlan& plan, const GemmArgs& args,
                       hipStream_t stream) {
  if (plan.n_tiles <= 0 || plan.m_tiles <= 0 || plan.splits <= 0 || args.S <= 0) return hipErrorInvalidValue;
  return f32 ? launch_epi<float>(epi, plan, args, stream) : launch_epi<bf16>(epi, plan, args, stream);
}

}  // namespace dflash
