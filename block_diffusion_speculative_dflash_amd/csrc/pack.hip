// One-time repacking of the drafter's nn.Linear weights into the fragment-major
// layout the GEMMs stream: [tile][K step][4 column blocks][64 lanes][8], so each
// wavefront load reads 1 KB of contiguous memory.  Tile columns follow the fused
// epilogue that consumes them (plain rows; SwiGLU gate/up pairs; RoPE pairs of a
// head), rows past N and K past the end are zero.  bf16 weights of a bf16 drafter
// become fp16 (exact inside fp16's normal range; a value beyond +-65504 saturates
// and sets DFLASH_DEVERR_RANGE) except fuse_w, which stays bf16.
#include <algorithm>
#include <type_traits>

#include "common.h"
#include "internal.h"

namespace dflash {

__device__ __forceinline__ int pack_row(const PackArgs& a, int t, int c) {
  if (a.kind == PACK_PLAIN) {
    const int n = t * kBN + c;
    return n < a.N ? n : -1;
  }
  if (a.kind == PACK_SWIGLU) {
    const int j = t * (kBN / 2) + (c & 31);
    if (j >= a.ffn) return -1;
    return c < 32 ? j : a.ffn + j;
  }
  const int tph = a.head_dim / kBN;
  const int hd = t / tph, sub = t % tph;
  return hd * a.head_dim + sub * 32 + (c & 31) + (c >> 5) * (a.head_dim / 2);
}

template <typename TS, typename TD>
__global__ __launch_bounds__(kThreads) void pack_kernel(PackArgs a) {
  const size_t chunks = static_cast<size_t>(a.n_tiles) * a.S * 4 * 64;
  const TS* src = static_cast<const TS*>(a.src);
  TD* dst = static_cast<TD*>(a.dst);
  bool range_err = false;
  for (size_t idx = blockIdx.x * static_cast<size_t>(blockDim.x) + threadIdx.x; idx < chunks;
       idx += static_cast<size_t>(gridDim.x) * blockDim.x) {
    const int lane = static_cast<int>(idx % 64);
    const int ni = static_cast<int>((idx / 64) % 4);
    const int s = static_cast<int>((idx / 256) % a.S);
    const int t = static_cast<int>(idx / (256 * static_cast<size_t>(a.S)));
    const int row = pack_row(a, t, ni * 16 + (lane & 15));
    const int k0 = s * kKStep + 8 * (lane >> 4);
    for (int j = 0; j < 8; ++j) {
      float v = 0.f;
      if (row >= 0 && k0 + j < a.K) v = to_f32(src[static_cast<size_t>(row) * a.K + k0 + j]);
      if (fabsf(v) > 65504.f && sizeof(TD) == 2 && !std::is_same<TD, bf16>::value) {
        range_err = true;
        v = copysignf(65504.f, v);
      }
      dst[idx * 8 + j] = from_f32<TD>(v);
    }
  }
  if (range_err) atomicOr(a.dev_error, kErrRange);
}

hipError_t launch_pack(bool f32, const PackArgs& a, hipStream_t stream) {
  const size_t chunks = static_cast<size_t>(a.n_tiles) * a.S * 256;
  const int blocks = static_cast<int>(std::min<size_t>((chunks + kThreads - 1) / kThreads, 65536));
  if (f32) hipLaunchKernelGGL((pack_kernel<float, float>), dim3(blocks), dim3(kThreads), 0, stream, a);
  else if (a.dst_f16) hipLaunchKernelGGL((pack_kernel<bf16, f16>), dim3(blocks), dim3(kThreads), 0, stream, a);
  else hipLaunchKernelGGL((pack_kernel<bf16, bf16>), dim3(blocks), dim3(kThreads), 0, stream, a);
  return hipGetLastError();
}

}  // namespace dflash
