// Internal launch interface between the C-ABI layer (api.hip) and the kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace dflash {

// Epilogues of the weight-streaming GEMM; each fuses the step that follows the
// projection so no intermediate makes an extra HBM round trip.
enum Epi : int {
  EPI_FUSE = 0,    // fused feature: cu = u * fuse_norm (bf16/f32) + per-tile sum of u^2
  EPI_INJECT = 1,  // K/V injection: scale by RMSNorm factor, RoPE on K, write ring slots
  EPI_QKV = 2,     // block q/k/v: scale by RMSNorm factor, RoPE on q and k
  EPI_RESID = 3,   // residual add into h, next RMSNorm input h*g + per-tile sum of h^2
  EPI_SWIGLU = 4,  // silu(gate) * up with the RMSNorm factor applied to both
  EPI_ARGMAX = 5,  // logits = scale * acc, split-vocab argmax, optional logits out
};

constexpr int kBN = 64;      // output columns per workgroup tile
constexpr int kKStep = 32;   // reduction elements per MFMA step

// Everything any epilogue needs; unused fields stay zero.
struct GemmArgs {
  // A operand: activations [M, K], row stride lda elements
  const void* A;
  int lda, M, K;
  // B operand: weight rows; how a tile column maps to a row depends on the epilogue
  const void* W;
  int ldw;        // row stride of W (elements)
  int N;          // real output columns (F for SWIGLU, V for ARGMAX)
  int n_tiles;    // workgroup tiles along N
  int m_tiles;
  // split-K
  int splits, k_split;
  float* partials;     // [splits, M, n_tiles * kBN] fp32
  unsigned* counters;  // zero-initialised; one per (m tile, n tile), or per m tile (ARGMAX)
  // RMSNorm of the A rows, folded into the epilogue as a per-row factor
  const float* ssq_in;  // [M, np_in] partial sums of squares, or nullptr (factor 1)
  int np_in, norm_dim;
  float eps;
  // next RMSNorm input produced by FUSE / RESID
  float* ssq_out;    // [M, np_out]
  int np_out;
  const void* gain;  // [N] gain of the next RMSNorm (fuse_norm, mlp_norm, ...)
  // outputs
  void* out;   // FUSE: cu [M, N]; RESID: x = h*g [M, N]; SWIGLU: act [M, ldo]; QKV: q
  int ldo;
  void* out2;  // QKV: block k  [M, Hkv, dh]
  void* out3;  // QKV: block v  [M, Hkv, dh]
  float* h;    // RESID: residual stream [M, N] fp32
  // geometry of QKV / INJECT
  int rows_per_seq;         // k (QKV) or n_max (INJECT)
  const int32_t* ctx_len;   // [B]
  const int32_t* n_rows;    // [B] (INJECT)
  int n_q_heads, n_kv_heads, head_dim, n_layers, batch, cache_slots, ffn;
  float theta;
  void* cache_k;  // [L, B, Hkv, C, dh]
  void* cache_v;
  // ARGMAX
  unsigned long long* keys;  // [M] zero-initialised argmax keys
  int32_t* draft;            // [M]
  float* logits;             // [M, N] or nullptr
  uint32_t* dev_error;
};

struct GemmPlan {
  int bm, m_tiles, n_tiles, splits, k_split;
  bool vec;  // rows 16-byte aligned and K multiple of 8: vector loads
};

// elem_bytes: 2 (bf16) or 4 (f32)
hipError_t launch_gemm(int epi, int elem_bytes, const GemmPlan& plan, const GemmArgs& args,
                       hipStream_t stream);

struct EmbedArgs {
  const int32_t* anchor;   // [B]
  const int32_t* ctx_len;  // [B] (checked only)
  const void* embed;       // [V, d]
  const void* mask_embed;  // [d]
  const void* gain;        // attn_norm of layer 0 [d]
  float* h;                // [M, d]
  void* xa;                // [M, d]
  float* ssq;              // [M, 1]
  int batch, block_k, hidden, vocab;
  uint32_t* dev_error;
};
hipError_t launch_embed(int elem_bytes, const EmbedArgs& a, hipStream_t stream);

struct AttnArgs {
  const void* q;   // [B*k, Hq, dh]
  const void* kb;  // [B*k, Hkv, dh]
  const void* vb;
  const void* cache_k;  // layer base: [B, Hkv, C, dh]
  const void* cache_v;
  const int32_t* ctx_len;
  void* out;  // [B*k, Hq*dh]
  float* part_o;   // [B, Hkv, n_rb, max_splits, 64, dh]
  float* part_ml;  // [B, Hkv, n_rb, max_splits, 64, 2]
  unsigned* counters;  // [B, Hkv, n_rb]
  int batch, block_k, n_q_heads, n_kv_heads, head_dim, cache_slots, window;
  int keys_per_split, max_splits, n_rb;
};
hipError_t launch_attention(int elem_bytes, const AttnArgs& a, hipStream_t stream);

struct VerifyArgs {
  const int32_t* draft;   // [B, k]
  const int32_t* target;  // [B, k+1]
  int32_t* ctx_len;
  int32_t* anchor;
  int32_t* accept_len;
  int32_t* out_tokens;
  uint32_t* dev_error;
  int batch, block_k, vocab;
};
hipError_t launch_verify(const VerifyArgs& a, hipStream_t stream);

hipError_t launch_commit_rows(int32_t* ctx_len, const int32_t* n_rows, int batch, int n_max,
                              uint32_t* dev_error, hipStream_t stream);

}  // namespace dflash
