/*
 * dflash.h — C ABI of the MI355X (gfx950) DFlash block draft-and-verify step.
 *
 * The method (DFlash, "Block Diffusion for Flash Speculative Decoding", as the
 * zhihu answer on MiMo-V2.5-Pro-UltraSpeed explains it in §5.1-§5.4, and as the
 * hotdry blog on MiMo-V2.5 speculative-decoding draft scheduling deploys it):
 *   1. fuse the hidden states of 5 target layers with one linear projection and
 *      RMSNorm into a context feature, and inject that feature into every draft
 *      layer's K/V, kept in a KV cache (zhihu §5.1, §5.2);
 *   2. fill a whole block of k positions — the visible anchor token plus k-1 mask
 *      positions — with one forward pass of a small transformer whose attention is
 *      a 128-token sliding window over the committed context (hotdry blog: block
 *      level masked parallel prediction, SWA drafter; zhihu §5.3, §5.4);
 *   3. verify the block greedily: accept drafts up to the first one that differs
 *      from the target's token, take the target's token there as a bonus, and
 *      commit or roll back (zhihu §2, draft / verify / accept steps).
 *
 * Conventions shared by every call
 *   - All pointers are DEVICE pointers unless marked (host).  The caller owns every
 *     buffer: weights, taps, the decode state, the workspace and the outputs.  The
 *     library allocates nothing, keeps no pointer after a call returns, and holds
 *     no global state apart from read-only kernel code.
 *   - Every call only enqueues work on `stream` and returns; results are valid once
 *     the stream reaches that point.  Calls on one workspace must not overlap.
 *   - Synchronous errors: argument validation happens on the host before anything
 *     is enqueued, and a failure returns a negative dflash_status with nothing
 *     enqueued.  A failed kernel launch returns DFLASH_E_HIP.
 *   - Asynchronous errors: contract violations only the device can see (a token id
 *     outside [0, vocab), a row count outside [0, n_max], a negative committed
 *     length) are clamped into range and OR-ed into *cache->dev_error as the
 *     DFLASH_DEVERR_* bits.  The caller reads that word after synchronising.
 *   - Matrices use the nn.Linear layout [out, in], row-major, rows contiguous.
 *   - dims->dtype is the element type of the caller's weights and taps:
 *     DFLASH_BF16 (bfloat16) or DFLASH_F32 (float).  A bf16 drafter computes in
 *     fp16 with fp32 accumulation: its K/V cache, q/k/v and the activations that
 *     feed the matrix cores are fp16 (bf16 weights convert to fp16 exactly inside
 *     fp16's normal range, and fp16 rounds 8x finer than bf16 at the same bytes);
 *     the residual stream is fp32.  A value headed for fp16 storage that lies beyond
 *     fp16's finite range is stored as +-65504 and sets DFLASH_DEVERR_OVERFLOW (so
 *     weights or inputs far outside the trained range are reported, not silently
 *     turned into infinities); the attention output, a convex combination of fp16
 *     values, and the softmax weights (at most 2^8 before normalisation) cannot
 *     exceed the range.  An fp32 drafter is fp32 throughout.  Token ids are int32.
 *   - The GEMM weights are read from a packed copy (dflash_pack_weights), laid out
 *     so every wavefront load is 1 KB of contiguous memory.
 *   - Order of one decode round: dflash_draft_step -> (target model verifies) ->
 *     dflash_fuse_inject(commit = 0) -> dflash_verify_commit.  The K/V rows for the
 *     k+1 positions the target just processed are written as tentative rows, and
 *     verify_commit moves the committed length past the accepted ones; rows past it
 *     are rolled back simply by not being committed (nothing is copied).
 */
#ifndef DFLASH_H
#define DFLASH_H

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  DFLASH_OK = 0,
  DFLASH_E_INVALID = -1,     /* bad dims, NULL or misaligned pointer, bad argument */
  DFLASH_E_UNSUPPORTED = -2, /* valid but not handled by this library (e.g. head_dim) */
  DFLASH_E_WORKSPACE = -3,   /* workspace NULL or smaller than dflash_workspace_bytes */
  DFLASH_E_HIP = -4,         /* a HIP runtime call or kernel launch failed */
  DFLASH_E_TOO_LARGE = -5    /* dflash_draft_step_noalloc: the dims need more than its scratch */
} dflash_status;

typedef enum { DFLASH_F32 = 0, DFLASH_BF16 = 1 } dflash_dtype;

/* Bits OR-ed into cache->dev_error by the device. */
#define DFLASH_DEVERR_TOKEN 1u   /* anchor, draft or target token outside [0, vocab): clamped */
#define DFLASH_DEVERR_ROWS 2u    /* n_rows[b] outside [0, n_max]: clamped */
#define DFLASH_DEVERR_CTXLEN 4u  /* ctx_len[b] negative: treated as 0 */
#define DFLASH_DEVERR_RANGE 8u   /* a bf16 weight beyond the fp16 range: saturated when packed */
#define DFLASH_DEVERR_BLOCK 16u  /* block_len[b] outside [0, k]: clamped */
#define DFLASH_DEVERR_OVERFLOW 32u /* bf16 drafter: an fp16 activation, q/k/v or K/V value beyond
                                      +-65504 (saturated there) or not finite */
#define DFLASH_DEVERR_TIMEOUT 64u  /* dflash_draft_step_persistent: a bounded wait for another
                                      workgroup's results ran out (the kernel exited; that call's
                                      results are invalid).  Only if other work on the GPU keeps
                                      part of the grid from running for about a quarter of a
                                      second */

/* (host) Static shapes of one drafter; read during a call only.
 *   batch B, block_k k (1..63), n_layers L, hidden d, n_q_heads Hq, n_kv_heads Hkv
 *   (Hq % Hkv == 0), head_dim dh (64 or 128), ffn F (SwiGLU width), vocab V,
 *   n_taps (the pages fix 5), tap_dim d_t, window W (committed positions each block
 *   query sees), cache_slots C (slots per layer/sequence/kv head, C >= s + W + k),
 *   dtype (dflash_dtype), max_inject_rows (largest n_max a fuse_inject call may
 *   use, >= k + 1; sizes the workspace), rms_eps, rope_theta (RoPE base), sink s
 *   (attention sink: positions 0..s-1 stay visible to every block query after they
 *   leave the window, as the aufer article's micro-op section names it for this
 *   drafter; 0 = plain sliding window).
 * Accepted ranges (any field outside: DFLASH_E_INVALID, size queries return 0):
 *   batch <= 65536, n_layers <= 64, hidden a multiple of 64 up to 65536,
 *   n_q_heads <= 1024, ffn <= 2^20, 2 <= vocab <= 2^24, n_taps <= 64,
 *   tap_dim <= 65536, window <= 2^24, sink <= 2^20, cache_slots <= 2^26,
 *   max_inject_rows <= 65536, rms_eps >= 0, rope_theta > 0, and batch * max_inject_rows
 *   * hidden <= 2e9, batch * block_k * vocab <= 4e9. */
typedef struct {
  int32_t batch, block_k, n_layers, hidden, n_q_heads, n_kv_heads, head_dim, ffn,
      vocab, n_taps, tap_dim, window, cache_slots, dtype, max_inject_rows;
  float rms_eps, rope_theta;
  int32_t sink;
} dflash_dims;

/* (host) Device pointers to the drafter weights, all in dims->dtype, all
 * 16-byte aligned, no biases (hidden must be a multiple of 64):
 *   fuse_w [d, n_taps*d_t]   projection of the concatenated taps (ascending depth)
 *   fuse_norm [d]            RMSNorm gain of the fused feature
 *   embed [V, d]             token embedding (the anchor row)
 *   mask_embed [d]           embedding of every mask position of the block
 *   attn_norm [L, d]         pre-attention RMSNorm gains
 *   w_qkv [L, (Hq+2Hkv)*dh, d]  q rows, then k rows, then v rows; the k and v rows
 *                            also project the fused feature into the cache
 *   w_o [L, d, Hq*dh]        attention output projection
 *   mlp_norm [L, d]          pre-MLP RMSNorm gains
 *   w_gate_up [L, 2F, d]     SwiGLU gate rows (first F) then up rows
 *   w_down [L, d, F]         SwiGLU down projection
 *   final_norm [d]           RMSNorm gain before the LM head
 *   lm_head [V, d]           LM head (independent of embed)
 *   packed                   dflash_packed_bytes(dims) bytes written by
 *                            dflash_pack_weights from the six matrices above
 *                            (fuse_w, w_qkv, w_o, w_gate_up, w_down, lm_head).
 * dflash_fuse_inject and dflash_draft_step read those six matrices only through
 * `packed`; after packing they may be freed (set to NULL).  embed, mask_embed and
 * the norm gains are always read directly. */
typedef struct {
  const void *fuse_w, *fuse_norm, *embed, *mask_embed, *attn_norm, *w_qkv, *w_o,
      *mlp_norm, *w_gate_up, *w_down, *final_norm, *lm_head, *packed;
} dflash_weights;

/* (host) The whole decode state, caller-owned device memory:
 *   k, v       [L, B, Hkv, C, dh], fp16 for a bf16 drafter and float for an fp32
 *              drafter (16-byte aligned); logical position p of sequence b lives
 *              in slot p if p < s (the sink), else in slot s + (p - s) % (C - s);
 *              k rows carry RoPE at position p
 *   ctx_len    [B] int32 committed length P_b (a logical position, may exceed C)
 *   anchor     [B] int32 token at position P_b (the visible first row of the block)
 *   dev_error  [1] uint32 sticky DFLASH_DEVERR_* bits
 *   block_len  [B] int32 or NULL: the number of draft rows k_b in [0, k] of sequence b
 *              this round (NULL: k for every sequence).  A block of k_b rows is the
 *              anchor plus k_b - 1 mask rows and its keys; rows past k_b are not part
 *              of it (their drafts read -1, their logits are unspecified); k_b = 0
 *              turns speculation off for the sequence (the round commits the target's
 *              own next token).  The verify calls test k_b drafts and take the bonus
 *              from target row k_b; the fuse_inject of the round writes k_b + 1 rows
 *              (n_rows[b] = k_b + 1).  dflash_adapt_block_len updates it. */
typedef struct {
  void *k, *v;
  int32_t *ctx_len, *anchor;
  uint32_t *dev_error;
  int32_t *block_len;
} dflash_cache;

/* Bytes of device workspace the three calls need for these dims.  The workspace
 * must be zero-filled once before its first use; every call leaves the counters it
 * uses at zero again.  Returns 0 for invalid dims. */
size_t dflash_workspace_bytes(const dflash_dims *dims);

/* Static string naming a dflash_status value. */
const char *dflash_status_string(int status);

/* Bytes of the packed weight copy for these dims (0 for invalid dims). */
size_t dflash_packed_bytes(const dflash_dims *dims);

/* Repack the GEMM weights (w->fuse_w, w_qkv, w_o, w_gate_up, w_down, lm_head, in
 * nn.Linear layout) into `packed` (packed_bytes >= dflash_packed_bytes(dims),
 * 16-byte aligned), once, before the first fuse_inject / draft_step.  Enqueued on
 * `stream`; dev_error (device, may be NULL) receives DFLASH_DEVERR_RANGE if a bf16
 * weight exceeds the fp16 range (it is saturated). */
int dflash_pack_weights(const dflash_dims *dims, const dflash_weights *w, void *packed,
                        size_t packed_bytes, uint32_t *dev_error, hipStream_t stream);

/* Feature fusion + KV injection (zhihu answer §5.1 feature fusion, §5.2 KV
 * injection; hotdry blog: all-SWA drafter with a 128-token window).
 *   taps     [B, n_max, n_taps, d_t] in dims->dtype: for sequence b, rows
 *            0..n_rows[b]-1 are the tapped target hidden states of logical positions
 *            ctx_len[b] .. ctx_len[b]+n_rows[b]-1, taps in ascending target depth;
 *            rows past n_rows[b] are ignored
 *   n_rows   [B] int32 device array, each in [0, n_max]
 *   n_max    (host) 1 .. dims->max_inject_rows
 *   commit   (host) 0: rows are tentative (the per-round path, n_rows = k+1);
 *            1: also advance ctx_len[b] by n_rows[b] (prefill)
 * A call may carry more rows for a sequence than its ring holds (C - s slots after
 * the sink): the cache then ends as if the rows were written in position order,
 * every ring slot holding the last of the rows that map to it.
 * For every row and layer l: c = RMSNorm(fuse_w . concat(taps)) * fuse_norm, then
 * K = RoPE(W_k^l c, position) and V = W_v^l c are written to the position's slot
 * (see dflash_cache). */
int dflash_fuse_inject(const dflash_dims *dims, const dflash_weights *w,
                       const void *taps, const int32_t *n_rows, int32_t n_max,
                       int32_t commit, const dflash_cache *cache, void *workspace,
                       size_t workspace_bytes, hipStream_t stream);

/* One block draft (hotdry blog: block-level masked parallel prediction, one
 * forward fills the whole block; zhihu §5.3, §5.4).  Row 0 of sequence b's block is
 * embed[anchor[b]] at position P_b = ctx_len[b]; rows 1..k-1 are mask_embed at
 * P_b+1 .. P_b+k-1.  Each of the L pre-norm layers applies RMSNorm, the fused QKV
 * projection with RoPE, attention of every block row over the sink positions
 * 0..min(s, P_b)-1, the last W committed positions that are not sink positions,
 * and all k block rows (bidirectional inside the block, GQA),
 * the output projection with residual, and a SwiGLU MLP with residual.  A final
 * RMSNorm and the LM head give logits; row i's argmax (lowest id on ties) is the
 * draft for position P_b+i+1.
 *   draft       [B, k] int32 output
 *   logits_out  NULL, or [B, k, V] float output of the logits (for tests); with
 *               cache->block_len, rows i >= block_len[b] are unspecified
 * With cache->block_len and at least 128 block rows (bf16), the rows of shrunken
 * blocks are compacted away before the first GEMM: the projections, the attention
 * and the LM head compute only the sum of the block lengths in rows (the hotdry
 * blog's fallback section: a shorter block should cost less).
 * Reads the cache, writes only draft, logits_out and the workspace. */
int dflash_draft_step(const dflash_dims *dims, const dflash_weights *w,
                      const dflash_cache *cache, int32_t *draft, float *logits_out,
                      void *workspace, size_t workspace_bytes, hipStream_t stream);

/* Greedy verification, bonus token, commit / rollback, in place (zhihu answer §2:
 * accept drafts up to the first error, the target takes over there; §6: the
 * accepted output equals what the target would emit by itself).
 *   draft       [B, k] int32 drafts of dflash_draft_step
 *   target      [B, k+1] int32: target[b, i] is the target's greedy token for
 *               position P_b+i+1 given the anchor and draft[b, 0..i-1]
 *   accept_len  [B] int32 output a_b in [0, k]: leading drafts equal to target
 *   out_tokens  [B, k+1] int32 output: target[b, 0..a_b], then -1
 * Updates ctx_len[b] += a_b + 1 and anchor[b] = target[b, a_b].  The K/V rows the
 * preceding fuse_inject wrote for positions P_b .. P_b+a_b become committed; those
 * for P_b+a_b+1 .. P_b+k are rolled back (never read again before being
 * rewritten). */
int dflash_verify_commit(const dflash_dims *dims, const int32_t *draft,
                         const int32_t *target, const dflash_cache *cache,
                         int32_t *accept_len, int32_t *out_tokens, hipStream_t stream);

/* (host) Parameters of sampled drafting and verification.
 *   temperature  T > 0 and finite: the drafter's and the target's distributions are
 *                softmax(logits / T) (one temperature for both)
 *   reserved     must be 0
 *   seed, step   key word and counter word of the random draws; give every decode
 *                round a new step (draws of different rounds are then independent)
 *   step_dev     optional device pointer: when non-NULL the kernels read the step
 *                from *step_dev when they run and `step` is ignored, so a captured
 *                HIP graph draws new numbers on every replay once the caller
 *                advances that word between rounds
 * Every draw comes from Philox4x64-10 (Salmon, Moraes, Dror, Shaw, "Parallel random
 * numbers: as easy as 1, 2, 3", SC 2011), key (seed, stream), its four output
 * words read as eight 32-bit values h (low half of word 0 first); a uniform is
 * (h + 1/2) 2^-32 and a Gumbel variate -ln(-ln u); a sample of softmax(s) is
 * argmax_v (s_v + Gumbel_v), smallest v on ties.  Streams and counters:
 *   1  draft noise of block row m = b*k + i, token v: counter
 *      (16 (v >> 5) + (v & 15), m >> 2, step, 0), value 2 (m & 3) + ((v >> 4) & 1)
 *   2  acceptance uniform of row i of sequence b: counter (i, b, step, 0), value 0
 *   3  noise of the emitted token of sequence b, token v: counter (v >> 3, b, step, 0),
 *      value v & 7 */
typedef struct {
  float temperature;
  uint32_t reserved;
  uint64_t seed, step;
  const uint64_t *step_dev;
} dflash_sampling;

/* Sampled drafting: the forward of dflash_draft_step, with draft[b, i] a sample of
 * q_i = softmax(z[b, i] / T) instead of its argmax (stream 1 above).
 *   sampling    (host) temperature, seed, step
 *   draft       [B, k] int32 output
 *   logits_out  [B, k, V] float output, required: the raw logits z (the verify
 *               reads the draft's residual row from here)
 *   lse_out     [B, k] float output, required: natural log-sum-exp of z[b, i] / T
 * Reads the cache, writes only draft, logits_out, lse_out and the workspace. */
int dflash_draft_step_sampled(const dflash_dims *dims, const dflash_weights *w,
                              const dflash_cache *cache, const dflash_sampling *sampling,
                              int32_t *draft, float *logits_out, float *lse_out,
                              void *workspace, size_t workspace_bytes, hipStream_t stream);

/* Sampled verification by rejection sampling, commit / rollback, in place (the
 * aufer article's data-flow section names the target's check rejection sampling;
 * zhihu answer §2 gives the accept loop, §6 the guarantee that the output follows
 * the target's distribution).  With p_i = softmax(target_logits[b, i] / T) and
 * q_i = softmax(draft_logits[b, i] / T): draft[b, i] is accepted while
 * u_i q_i(x_i) <= p_i(x_i) (u_i from stream 2); at the first rejection a_b the
 * emitted token is a sample of max(0, p_a - q_a) (of p_a if rounding left no
 * positive entry); after k acceptances, a sample of p_k (stream 3).
 *   sampling       (host) the same temperature, seed and step as the draft call
 *   draft          [B, k] int32 drafts of dflash_draft_step_sampled
 *   draft_logits   [B, k, V] float (its logits_out), 16-byte aligned
 *   draft_lse      [B, k] float (its lse_out)
 *   target_logits  [B, k+1, V] float, 16-byte aligned: row i is the target's logits
 *                  for position P_b+i+1 given the anchor and draft[b, 0..i-1]
 *   accept_len     [B] int32 output a_b in [0, k]
 *   out_tokens     [B, k+1] int32 output: draft[b, 0..a_b-1], the emitted token, -1
 * Updates ctx_len[b] += a_b + 1 and anchor[b] = emitted token, with the same
 * commit / rollback of K/V rows as dflash_verify_commit.  Uses the workspace of the
 * other calls (they must not overlap on it). */
int dflash_verify_sampled(const dflash_dims *dims, const dflash_sampling *sampling,
                          const int32_t *draft, const float *draft_logits,
                          const float *draft_lse, const float *target_logits,
                          const dflash_cache *cache, int32_t *accept_len,
                          int32_t *out_tokens, void *workspace, size_t workspace_bytes,
                          hipStream_t stream);

/* (host) Parameters of the runtime block-size controller (the hotdry blog's dynamic
 * fallback: while measured acceptance stays below the scenario's threshold the
 * block is shrunk step by step, 8 -> 4, or speculation is turned off for a while;
 * its reference thresholds on the mean accepted length at block 8 are code >= 6.0,
 * math >= 5.0, agent >= 4.0, open chat < 4.0).  Rungs: full k, half k/2 (absent when
 * 0), off.  Per sequence a float32 moving average m of the accepted length at the
 * full block: after a round of k_b > 0 drafts with a accepted,
 * tau = 1 + a * (k / k_b), m = m + alpha * (tau - m) (each operation rounded).
 *   full: m < theta_down -> one rung down;  half: m < theta_off -> off,
 *   m >= theta_up -> full;  off: `cooldown` rounds, then half (full if there is no
 *   half rung) with m = theta_down.
 * Suggested: alpha 0.25, theta_down 4.0, theta_off 2.0, theta_up 6.0, cooldown 16. */
typedef struct {
  float alpha, theta_down, theta_off, theta_up;
  int32_t cooldown;
} dflash_adapt_params;

/* One controller round after a verify call, in place:
 *   params      (host) the controller parameters (0 < alpha <= 1, cooldown >= 1)
 *   accept_len  [B] int32 accepted lengths of the round just verified
 *   cache       its block_len (required here) is read and updated
 *   ema         [B] float moving averages m (initialise to theta_up)
 *   off_left    [B] int32 rounds left with speculation off (initialise to 0)
 * Sequences whose block_len is 0 count their cool-down down and ignore accept_len. */
int dflash_adapt_block_len(const dflash_dims *dims, const dflash_adapt_params *params,
                           const int32_t *accept_len, const dflash_cache *cache, float *ema,
                           int32_t *off_left, hipStream_t stream);

/* dflash_draft_step with every draft layer run as ONE launch of a persistent layer
 * kernel instead of one kernel per operator (the pages' execution-model point: the
 * hotdry blog's TileRT section and the aufer article's micro-op section locate the
 * batch-1 cost in the gaps between many small operators).  Inside a launch the
 * phases QKV -> attention -> key-split merge -> O -> gate/up -> down overlap: each
 * work item (the separate kernels' workgroups, with the same plans) waits only for
 * the items that produce what it reads (every wait bounded: DFLASH_DEVERR_TIMEOUT,
 * never a hang), and a projection's first weight loads are issued before its wait.
 * Covers bf16 drafters with batch * block_k <= 64 block rows and head_dim 128;
 * returns DFLASH_E_UNSUPPORTED (nothing enqueued) otherwise.  Same arguments, same
 * results as dflash_draft_step (bitwise, when a sequence's keys are split into 1 or
 * at least 8 pieces; otherwise the split merge sums in another order). */
int dflash_draft_step_persistent(const dflash_dims *dims, const dflash_weights *w,
                                 const dflash_cache *cache, int32_t *draft, float *logits_out,
                                 void *workspace, size_t workspace_bytes, hipStream_t stream);

/* For callers that cannot allocate device memory (code under HIP graph capture,
 * tight serving loops, harnesses that forbid hipMalloc): dflash_draft_step without
 * a workspace argument.  Its workspace is a static device array of the library,
 * DFLASH_NOALLOC_SCRATCH_BYTES bytes on every GPU the library runs on, held until
 * the process ends; the call allocates nothing.  Dims whose workspace
 * (dflash_workspace_bytes) exceeds that size return DFLASH_E_TOO_LARGE with nothing
 * enqueued (96 MiB covers the batch-1 and batch-8 drafters of hidden 4096).  Every
 * call on one GPU uses the same array and clears its counters first: calls that
 * overlap on one GPU (two streams, two threads) race and must be serialised by the
 * caller.  Results are those of dflash_draft_step. */
#define DFLASH_NOALLOC_SCRATCH_BYTES ((size_t)96 << 20)
int dflash_draft_step_noalloc(const dflash_dims *dims, const dflash_weights *w,
                              const dflash_cache *cache, int32_t *draft, float *logits_out,
                              hipStream_t stream);

/* Same as dflash_draft_step, and records head_begin / head_end on `stream` right
 * before and after the fused final-norm + LM-head + argmax kernel, so a caller can
 * time that kernel alone with hipEventElapsedTime.  Either event may be NULL. */
int dflash_draft_step_timed(const dflash_dims *dims, const dflash_weights *w,
                            const dflash_cache *cache, int32_t *draft,
                            float *logits_out, void *workspace, size_t workspace_bytes,
                            hipStream_t stream, hipEvent_t head_begin,
                            hipEvent_t head_end);

/* Same as dflash_draft_step_sampled, with the LM-head events of
 * dflash_draft_step_timed around the fused LM-head + sampling kernel. */
int dflash_draft_step_sampled_timed(const dflash_dims *dims, const dflash_weights *w,
                                    const dflash_cache *cache, const dflash_sampling *sampling,
                                    int32_t *draft, float *logits_out, float *lse_out,
                                    void *workspace, size_t workspace_bytes,
                                    hipStream_t stream, hipEvent_t head_begin,
                                    hipEvent_t head_end);

/* Debug aid: fill memory whose content no later call may depend on with all-ones
 * bytes (NaN as fp16 and fp32), so that a kernel reading it would show up as
 * non-finite or changed results.  `what` is an OR of
 *   DFLASH_POISON_RING       the ring slots of positions ctx_len[b] ..
 *                            ctx_len[b] + (C - s - W) - 1 of every layer, sequence and
 *                            kv head: after dflash_verify_commit they hold the
 *                            rolled-back rows, and no block's window reaches them before
 *                            the next dflash_fuse_inject rewrites them
 *   DFLASH_POISON_WORKSPACE  every workspace byte except the arrival counters and
 *                            zero-initialised keys, which each call leaves at zero
 * Enqueued on `stream`; the other calls' results must not change (the tests check
 * this bitwise).  workspace may be NULL without DFLASH_POISON_WORKSPACE, cache may be
 * NULL without DFLASH_POISON_RING. */
#define DFLASH_POISON_RING 1
#define DFLASH_POISON_WORKSPACE 2
int dflash_debug_poison(const dflash_dims *dims, const dflash_cache *cache, void *workspace,
                        size_t workspace_bytes, int32_t what, hipStream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* DFLASH_H */
