// Internal launch interface between the C-ABI layer (api.hip) and the kernels other
// than the GEMMs (gemm.h): packing, block construction, attention, verification.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "gemm.h"

namespace dflash {

// ---------------------------------------------------------------------------
// weight packing
// ---------------------------------------------------------------------------
enum PackKind : int {
  PACK_PLAIN = 0,   // tile column c -> row tile*64 + c
  PACK_SWIGLU = 1,  // 32 gate rows then the 32 matching up rows
  PACK_HEADS = 2,   // per head: 32 RoPE pairs (dim, dim + dh/2) per tile
};

struct PackArgs {
  const void* src;  // [rows, K] row-major, caller's type
  int K, N, n_tiles, S, kind, head_dim, ffn;
  void* dst;        // packed [n_tiles][S][4][64][8]
  int dst_f16;      // bf16 source -> 1: fp16 copy, 0: bf16 copy (float source: float copy)
  uint32_t* dev_error;
};
hipError_t launch_pack(bool f32, const PackArgs& a, hipStream_t stream);

// ---------------------------------------------------------------------------
struct EmbedArgs {
  const int32_t* anchor;   // [B]
  const int32_t* ctx_len;  // [B] (checked only)
  const void* embed;       // [V, d]
  const void* mask_embed;  // [d]
  const void* gain;        // attn_norm of layer 0 [d]
  float* h;                // [M, d]
  void* xa;                // packed [M/16][d/32][64][8]
  float* ssq;              // [M, 1]
  int batch, block_k, hidden, vocab;
  uint32_t* dev_error;
  // compacted block rows (see CompactArgs), or nullptr: row m is (m / k, m % k)
  const int32_t* row_map;
  const int32_t* m_live;
};
hipError_t launch_embed(bool f32, const EmbedArgs& a, hipStream_t stream);

struct AttnArgs {
  const void* q;   // [B*k, Hq, dh]
  const void* kb;  // [B*k, Hkv, dh]
  const void* vb;
  const void* cache_k;  // layer base: [B, Hkv, C, dh]
  const void* cache_v;
  const int32_t* ctx_len;
  void* out;       // packed [B*k / 16][Hq*dh / 32][64][8]
  int out_steps;
  float* part_o;   // [B, Hkv, n_rb, max_splits, 64, dh]
  float* part_ml;  // [B, Hkv, n_rb, max_splits, 64, 2]
  unsigned* counters;  // [B, Hkv, n_rb]
  int batch, block_k, n_q_heads, n_kv_heads, head_dim, cache_slots, window, sink;
  int keys_per_split, max_splits, n_rb, rows_per_block;  // rows_per_block: 16, 32, 48 or 64
  const int32_t* block_len;  // [B] or nullptr: block keys of sequence b are rows 0 .. block_len[b]-1
  int balance;  // 1: pair long and short contexts on a CU (see balanced_sequence); batch <= kMaxBalanceBatch
  // compacted block rows: sequence b's rows start at seq_row0[b] in q, kb, vb and out,
  // and rows i >= block_len[b] are neither read as keys nor written; nullptr: b * k
  const int32_t* seq_row0;
};
constexpr int kMaxBalanceBatch = 256;
hipError_t launch_attention(bool f32, const AttnArgs& a, hipStream_t stream);

struct VerifyArgs {
  const int32_t* draft;   // [B, k]
  const int32_t* target;  // [B, k+1]
  int32_t* ctx_len;
  int32_t* anchor;
  int32_t* accept_len;
  int32_t* out_tokens;
  uint32_t* dev_error;
  const int32_t* block_len;  // [B] or nullptr (k drafts each)
  int batch, block_k, vocab;
};
hipError_t launch_verify(const VerifyArgs& a, hipStream_t stream);

// Runtime block-size controller (one thread per sequence).
struct AdaptArgs {
  const int32_t* accept_len;
  int32_t* block_len;
  float* ema;
  int32_t* off_left;
  uint32_t* dev_error;
  int batch, block_k, cooldown;
  float alpha, theta_down, theta_off, theta_up;
};
hipError_t launch_adapt(const AdaptArgs& a, hipStream_t stream);

// LM-head finalisation: per row the largest of the column tiles' argmax keys -> draft
// (-1 past the block length), and with part != nullptr the log-sum-exp of the tiles'
// (max, sum) partials -> lse.
struct HeadFinalizeArgs {
  const unsigned long long* keys;  // [rows, n_parts]
  const float2* part;              // [rows, n_parts] or nullptr
  int n_parts, rows, rows_per_seq;
  int32_t* draft;                  // [rows]
  float* lse;                      // [rows], with part
  const int32_t* block_len;        // [rows / rows_per_seq] or nullptr
  const int32_t* seq_row0;         // compacted rows: the keys of (b, i) are at row seq_row0[b] + i
};
hipError_t launch_head_finalize(const HeadFinalizeArgs& a, hipStream_t stream);

// Sampled verification: per-row log-sum-exp of the target logits and the
// acceptance scan (first kernel), then the residual / bonus draw and the commit.
struct VerifySampledArgs {
  const int32_t* draft;         // [B, k]
  const float* draft_logits;    // [B, k, V]
  const float* draft_lse;       // [B, k]  log-sum-exp of draft_logits / T
  const float* target_logits;   // [B, k+1, V]
  const int32_t* block_len;     // [B] or nullptr (k drafts each)
  int32_t* ctx_len;
  int32_t* anchor;
  int32_t* accept_len;
  int32_t* out_tokens;
  uint32_t* dev_error;
  float2* part;                 // [B, k+1, n_chunks] target row partials
  float* row_lse;               // [B, k+1] log-sum-exp of each target row / T
  unsigned* counters;           // [B (k+3)] zero-initialised arrival counters: per sequence
                                // (rows done), per sequence (emit chunks), per row (chunks)
  float4* decision;             // [B] (accepted length, target lse, draft lse, -)
  unsigned long long* keys;     // [2 B * kKeyStride] zero-initialised argmax keys
  int batch, block_k, vocab;
  int n_chunks;       // chunks per row of the log-sum-exp kernel
  int n_chunks_emit;  // chunks per sequence of the emit kernel
  float inv_temp;
  unsigned long long seed, step;
  const unsigned long long* step_dev;  // when set, the step is read from here at run time
};
// Vocabulary entries per verify workgroup: kVerifyGroupChunk * G, with G = 4, 2 or 1
// the largest that still gives a kernel over `rows` rows >= 256 workgroups (the
// log-sum-exp kernel covers B (k+1) rows, the emit kernel B).
constexpr int kVerifyGroupChunk = 2048;
inline int verify_groups(long long rows, int vocab) {
  for (int G = 4; G > 1; G >>= 1) {
    const long long chunks = (vocab + kVerifyGroupChunk * G - 1) / (kVerifyGroupChunk * G);
    if (rows * chunks >= 256) return G;
  }
  return 1;
}
inline int verify_chunks(long long rows, int vocab) {
  const int G = verify_groups(rows, vocab);
  return (vocab + kVerifyGroupChunk * G - 1) / (kVerifyGroupChunk * G);
}
hipError_t launch_verify_sampled(const VerifySampledArgs& a, hipStream_t stream);

hipError_t launch_commit_rows(int32_t* ctx_len, const int32_t* n_rows, int batch, int n_max,
                              uint32_t* dev_error, hipStream_t stream);

// Compaction of per-sequence row blocks (the draft step's blocks of block_len[b]
// rows, an injection's n_rows[b] rows): sequence b keeps counts[b] rows (clamped to
// [0, rows_per_seq]; out-of-range counts set err_bit), numbered consecutively in
// sequence order.  seq_row0[b] = first row of b, seq_row0[B] = number of live rows;
// row_map[m] = b * rows_per_seq + i, the uncompacted row of live row m.  One workgroup.
// (sin, cos) of every rotation pair at every row's position: tab[(b * rows_per_seq +
// i) * head_dim / 2 + d] for the position max(ctx_len[b], 0) + i, computed as the
// GEMM epilogues compute it (angle reduced in double precision).
struct RopeTabArgs {
  const int32_t* ctx_len;  // [B]
  float2* tab;
  int batch, rows_per_seq, head_dim;
  float theta;
};
hipError_t launch_rope_table(const RopeTabArgs& a, hipStream_t stream);

// Fragment packing of the fusion GEMM's A operand (the taps, bf16): live row m (row
// row_map[m] of the caller's row-major taps when compacted, else row m) goes to
// out[pa_index(m, k, steps)].
struct PackTapsArgs {
  const void* taps;  // [rows, lda] bf16
  void* out;         // packed [ceil(rows / 16), steps, 64, 8] bf16
  int lda, rows, steps;
  const int32_t* row_map;  // or nullptr
  const int32_t* m_live;   // or nullptr: all rows
};
hipError_t launch_pack_taps(const PackTapsArgs& a, hipStream_t stream);

struct CompactArgs {
  const int32_t* counts;  // [B]
  int32_t* seq_row0;      // [B + 1]
  int32_t* row_map;       // [B * rows_per_seq]
  int batch, rows_per_seq;
  uint32_t* dev_error;
  uint32_t err_bit;
};
hipError_t launch_compact_rows(const CompactArgs& a, hipStream_t stream);

// Persistent layer kernel (persist.hip): one launch per draft layer, phases QKV ->
// attention -> merge -> O -> gate/up -> down with tile-level dependencies.
struct PhaseGrid {
  int x, y, z;  // the separate kernel's grid: work item i = (i % x, i / x % y, i / (x y))
};
// Signal words of one layer (zero at launch), word offsets:
constexpr int kSigQkv = 0;      // [Hkv] finished QKV tiles of each kv group's heads
constexpr int kSigFin = 256;    // [Hkv] finished attention output row groups of each kv group
constexpr int kSigO = 512;      // finished O projection tiles
constexpr int kSigAtt = 1024;   // [B Hkv n_rb] finished attention items (key splits) per row group
constexpr int kSigGu = 8192;    // [gate/up tiles] flags: tile done
constexpr int kSigReady = 16384;  // + w: ready flag of counter word w (set once by the producer that completes it)
constexpr int kSigWords = 32768;
constexpr int kSigMaxHkv = 256, kSigMaxGroups = kSigGu - kSigAtt, kSigMaxGu = kSigReady - kSigGu;
struct LayerArgs {
  GemmArgs gemm[4];    // QKV, O, gate/up, down (bf16 drafter, streaming plans, own partials and counters)
  PhaseGrid grid[4];
  AttnArgs attn;       // rows_per_block 16 or 32, two key groups, no balancing
  int attn_items;      // B * Hkv * n_rb * max_splits
  int merge_items;     // 0 when no sequence's keys are split
  unsigned* sig;       // kSigWords signal words
  uint32_t* dev_error;
  int group;           // q heads per kv head
  int tiles_per_head;  // 64-column tiles per head (head_dim / 64)
  int o_tiles;         // output tiles of the O projection
  int fin_need;        // finished row groups of a kv group before its heads' attention output is complete
};
// Co-resident workgroups of the layer kernel for streaming row blocks mt (1, 2, 4) and
// attention row tiles nw (1, 2): 0 when unsupported.
int persistent_capacity(int mt, int nw, int cus);
hipError_t launch_layer_persistent(const LayerArgs& a, int mt, int nw, int grid, hipStream_t stream);

// Debug poisoning: all-ones bytes (NaN in fp16 and fp32) into memory no later call
// may depend on.
struct PoisonRingArgs {
  void* cache_k;  // [L, B, Hkv, C, dh]
  void* cache_v;
  const int32_t* ctx_len;
  int n_layers, batch, n_kv_heads, cache_slots, sink, n_dead;  // positions ctx_len .. ctx_len + n_dead - 1
  int row_bytes;                                               // dh * element size (a multiple of 16)
};
hipError_t launch_poison_ring(const PoisonRingArgs& a, hipStream_t stream);
hipError_t launch_fill_ones(void* p, size_t bytes, hipStream_t stream);  // p, bytes: multiples of 16
hipError_t launch_fill_zero(void* p, size_t bytes, hipStream_t stream);  // p, bytes: multiples of 16

}  // namespace dflash
