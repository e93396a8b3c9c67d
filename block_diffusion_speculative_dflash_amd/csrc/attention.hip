// Block attention on MFMA: every query row of the block attends to the sink
// positions 0..min(s, P)-1, the last W committed positions that are not sink
// positions (the layer's K/V ring), and all k block rows,
// with no causal mask inside the block (hotdry blog: one forward fills the whole
// masked block, all-SWA drafter with window W; zhihu answer §4: parallel decoding
// inside a block).
//
// Workgroup = (sequence b, kv head g, row block, key split).  The rows of kv head g
// are its G = Hq/Hkv query heads times the k block rows; a row block is up to four
// tiles of 16 of them.  The workgroup's wavefronts are row tile x key group: it
// streams its keys in rounds of two 32-key chunks, every chunk's K and V rows loaded
// from HBM once, cooperatively, into LDS (the next round's loads in flight in
// registers meanwhile); key group g computes on chunk g of each round, and the two
// groups' (max, sum, O) states of a row tile merge in LDS at the end.
//
// Everything is computed transposed so that one query row lives in one lane:
//   S^T = K Q^T     A = 16 keys x 32 head dims (straight from the key rows),
//                   B = Q^T; lane l gets the scores of row l%16 for keys 4*(l/16)+r
//   softmax         running max / sum per lane in log2 units (native exp2); across
//                   keys: in-lane, then the four lanes of a row (lane swaps 16, 32);
//                   the reference maximum moves lazily, and the output rescale is
//                   skipped when no row's reference moved
//   O^T += V^T P^T  B = P^T straight from the score registers: its 32 reduction
//                   slots are keys {4q..4q+3, 16+4q..16+4q+3} for lane group q, and
//                   A = V^T uses the same key order, read from the chunk's V rows
//                   in LDS with the gfx950 transposing LDS read (two 8-byte reads
//                   per 16 x 32 operand)
// so the row statistics scale the output accumulators without any data exchange.
// When one sequence's keys are split over several items (long full-attention
// contexts at small batch), each writes its unnormalised partial and a second kernel
// merges them in split order; either way the result does not depend on scheduling.
#include "attention_body.h"

namespace dflash {

template <typename T, int DH, int NW, int KG>
__global__ __launch_bounds__(64 * NW * KG) void attention_kernel(AttnArgs a) {
  __shared__ AttnLds<T, DH, NW, KG> lds;
  attention_body<T, DH, NW, KG, false>(a, blockIdx.x, lds);
}

template <typename T, int DH, int NSUB>
__global__ __launch_bounds__(kThreads) void attention_merge_kernel(AttnArgs a) {
  __shared__ MergeLds<DH, NSUB> lds;
  merge_body<T, DH, NSUB, false>(a, blockIdx.x, lds);
}

// Key groups per workgroup.  Two measured best at every shape tried (batch 1 to 256,
// windows 128 to 4232): four issue all of a round's loads at once and pay a second
// LDS merge step.
template <typename T, int NW> constexpr int key_groups() { return 2; }

template <typename T, int DH, int NW>
static void launch_nw(const AttnArgs& a, hipStream_t s) {
  constexpr int KG = key_groups<T, NW>();
  const long long wgs = static_cast<long long>(a.batch) * a.n_kv_heads * a.n_rb * a.max_splits;
  hipLaunchKernelGGL((attention_kernel<T, DH, NW, KG>), dim3(static_cast<unsigned>(wgs)), dim3(64 * NW * KG), 0, s,
                     a);
}

template <typename T, int DH, int NSUB>
static void launch_merge(const AttnArgs& a, hipStream_t s) {
  constexpr int RPW = kThreads / (DH / 4 * NSUB);
  const long long wgs = static_cast<long long>(a.batch) * a.n_kv_heads * a.n_rb * ((a.rows_per_block + RPW - 1) / RPW);
  hipLaunchKernelGGL((attention_merge_kernel<T, DH, NSUB>), dim3(static_cast<unsigned>(wgs)), dim3(kThreads), 0, s, a);
}

template <typename T, int DH>
static hipError_t launch_dh(const AttnArgs& a, hipStream_t s) {
  switch (a.rows_per_block / 16) {
    case 1: launch_nw<T, DH, 1>(a, s); break;
    case 2: launch_nw<T, DH, 2>(a, s); break;
    case 3: launch_nw<T, DH, 3>(a, s); break;
    case 4: launch_nw<T, DH, 4>(a, s); break;
    default: return hipErrorInvalidValue;
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || a.max_splits == 1) return e;
  // split subsets per row: about as many as there are splits (DH = 128: 8 rows per
  // workgroup with 1 subset, down to 1 row with 8)
  if (a.max_splits >= 8) launch_merge<T, DH, 8>(a, s);
  else if (a.max_splits >= 4) launch_merge<T, DH, 4>(a, s);
  else if (a.max_splits >= 2) launch_merge<T, DH, 2>(a, s);
  return hipGetLastError();
}

hipError_t launch_attention(bool f32, const AttnArgs& a, hipStream_t stream) {
  if (a.head_dim == 128) return f32 ? launch_dh<float, 128>(a, stream) : launch_dh<f16, 128>(a, stream);
  if (a.head_dim == 64) return f32 ? launch_dh<float, 64>(a, stream) : launch_dh<f16, 64>(a, stream);
  return hipErrorInvalidValue;
}

}  // namespace dflash
