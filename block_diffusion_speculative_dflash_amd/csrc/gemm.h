// GEMM interface: epilogue kinds, tile constants, the argument block and launchers
// of the weight-streaming (gemm.hip) and tiled (gemm_tiled.hip) GEMMs.
//
// Element types.  A drafter whose caller-facing dtype is bf16 keeps weights and
// taps in bf16 but computes in fp16: the packed weight copy, the activations that
// feed MFMA, q/k/v and the K/V cache are fp16 (bf16 values in fp16's normal range
// convert exactly; fp16 rounds 8x finer than bf16 at the same bytes and MFMA
// rate), accumulation and the residual stream are fp32.  The fusion GEMM multiplies
// the caller's bf16 taps by a bf16 packed copy of fuse_w, both exact.  An fp32
// drafter is fp32 throughout.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace dflash {

enum Epi : int {
  EPI_FUSE = 0,    // fused feature: cu = u * fuse_norm (packed) + per-tile sum of u^2
  EPI_INJECT = 1,  // K/V injection: RMSNorm factor, RoPE on K, write ring slots
  EPI_QKV = 2,     // block q/k/v: RMSNorm factor, RoPE on q and k
  EPI_RESID = 3,   // residual add into h, next RMSNorm input h*g (packed) + per-tile sum of h^2
  EPI_SWIGLU = 4,  // silu(gate) * up with the RMSNorm factor applied to both (packed)
  EPI_ARGMAX = 5,  // logits = factor * acc, split-vocab argmax, optional logits out
  EPI_SAMPLE = 6,  // logits out, Gumbel-max draw over logits / T, per-tile log-sum-exp partials
};

constexpr int kBN = 64;           // output columns per workgroup tile (4 MFMA column blocks)
constexpr int kKeyStride = 16;    // argmax keys one 128-byte line apart (u64 elements)
constexpr int kKStep = 32;        // reduction elements per MFMA step
constexpr int kTileStepElems = 4 * 512;  // one packed weight tile step: 4 fragments x 64 lanes x 8

inline int ksteps(int K) { return (K + kKStep - 1) / kKStep; }

struct GemmArgs {
  // A operand: fragment-packed [M/16][S][64][8] activations, or (fusion GEMM only)
  // the caller's row-major taps with row stride lda
  const void* A;
  int lda, M, K, S;
  // B operand: packed weight region; tile t starts at W + wtile(t) * S * kTileStepElems
  const void* W;
  int N, n_tiles, m_tiles;
  int layer_tiles, inj_tile0, inj_tiles;  // INJECT: K/V head tiles inside per-layer QKV regions
  // split-K: split z of a tile covers steps [z * steps_per_split, ..).  Balanced
  // pieces (streaming GEMM, piece_base > 0): grid x enumerates (tile, piece) pairs,
  // tiles 0 .. piece_extra-1 having piece_base + 1 pieces and the rest piece_base;
  // piece p of P covers steps [p*S/P, (p+1)*S/P), and splits is the largest P.
  int splits, steps_per_split;
  int piece_base, piece_extra;
  // split-K partials, fp32: streaming GEMM [splits, M, n_tiles * kBN]; tiled GEMM
  // [splits, m_tiles * n_big tiles, wavefront, WM, WN, lane] 16-byte accumulator blocks
  float* partials;
  unsigned* counters;  // zero-initialised; one per (m tile, n tile), or per m tile (ARGMAX)
  // RMSNorm of the A rows, folded into the epilogue as a per-row factor
  const float* ssq_in;  // [M, np_in] partial sums of squares, or nullptr (factor 1)
  int np_in, norm_dim;
  float eps;
  // next RMSNorm input produced by FUSE / RESID
  float* ssq_out;  // [M, np_out]
  int np_out;
  const void* gain;  // [N] gain of the next RMSNorm, caller's weight type
  // outputs
  void* out;      // FUSE cu, RESID x, SWIGLU act: packed with out_steps K steps; QKV: q rows
  int out_steps;
  void* out2;     // QKV: block k  [M, Hkv, dh]
  void* out3;     // QKV: block v  [M, Hkv, dh]
  float* h;       // RESID: residual stream [M, N] fp32
  int rows_per_seq;        // k (QKV) or n_max (INJECT)
  const int32_t* ctx_len;  // [B]
  const int32_t* n_rows;   // [B] (INJECT)
  int n_q_heads, n_kv_heads, head_dim, n_layers, batch, cache_slots, ffn;
  int sink;  // INJECT: positions < sink keep slot = position; the rest ring over cache_slots - sink
  float theta;
  // QKV / INJECT: when set, the (sin, cos) of row (b, i)'s position for rotation pair
  // d, at rope_tab[(b * rows_per_seq + i) * head_dim / 2 + d], instead of computing it
  const float2* rope_tab;
  void* cache_k;  // [L, B, Hkv, C, dh]
  void* cache_v;
  unsigned long long* keys;  // ARGMAX / SAMPLE: [M, n_parts] best key of each column tile
  int32_t* draft;            // [M]
  const int32_t* block_len;  // ARGMAX / SAMPLE: [B] or nullptr; rows i >= block_len[b] draft -1
  float* logits;             // [M, N] or nullptr
  uint32_t* dev_error;
  // EPI_SAMPLE: s = logits / T; draft = argmax(s + Gumbel noise of row m);
  // lse_part[m * n_parts + t] = (max, sum exp(s - max)) over column tile t
  float inv_temp;
  unsigned long long seed, step;
  const unsigned long long* step_dev;  // when set, the step is read from here at run time
  float2* lse_part;
  int n_parts;
  // tiled greedy LM head or SwiGLU on tiles whose epilogue works from the accumulators:
  // the grid is one workgroup per CU (a multiple of 8), each walking a stride of its
  // XCD's tiles; 0: one workgroup per tile
  int persist;
  // compacted rows (tiled GEMMs of a draft step with per-sequence block lengths or
  // of an injection with per-sequence row counts): rows at or beyond *m_live do not
  // exist (their tiles exit, the epilogues skip them), and live row m stands for
  // uncompacted row row_map[m] (sequence row_map[m] / rows_per_seq, position
  // row_map[m] % rows_per_seq; the fusion GEMM gathers that tap row); nullptr: all M
  // rows, uncompacted
  const int32_t* m_live;
  const int32_t* row_map;
  // tiled fusion GEMM: A is the taps already fragment-packed (compacted rows), not
  // the caller's row-major taps
  int a_packed;
};

struct GemmPlan {
  int tiled;    // 0: weight-streaming GEMM, 1: tiled MFMA GEMM
  int mt;       // streaming: 16-row MFMA blocks per workgroup (1, 2 or 4); tiled: a kTile* shape
  int m_tiles, n_tiles, splits, steps_per_split, depth;
  int piece_base, piece_extra;  // streaming: balanced K pieces (0: uniform splits)
};

// tiled GEMM tile shapes (GemmPlan::mt)
constexpr int kTile128 = 128;        // 128 x 128, 4 wavefronts of 64 x 64, two workgroups per CU
constexpr int kTile256 = 256;        // 256 x 256, 8 wavefronts of 128 x 64
constexpr int kTile128x384 = 1384;   // 128 x 384, 8 wavefronts of 64 x 96
constexpr int kTile256x128 = 2128;   // 256 x 128, 8 wavefronts of 64 x 64
inline int tile_rows(int cfg) { return cfg == kTile128x384 ? 128 : (cfg == kTile256x128 ? 256 : cfg); }
inline int tile_cols(int cfg) { return cfg == kTile128x384 ? 384 : (cfg == kTile256x128 ? 128 : cfg); }

// f32: true for an fp32 drafter, false for a bf16 drafter (fp16 compute)
hipError_t launch_gemm(int epi, bool f32, const GemmPlan& plan, const GemmArgs& args,
                       hipStream_t stream);
// bf16 drafters only; m_tiles counts plan.mt-row tiles, n_tiles 64-column tiles.
// The fusion GEMM needs K % 32 == 0 and a row stride that is a multiple of 8.
hipError_t launch_gemm_tiled(int epi, const GemmPlan& plan, const GemmArgs& args, hipStream_t stream);

}  // namespace dflash
