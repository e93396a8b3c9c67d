// C ABI of libdflash: host-side validation, packed-weight and workspace layouts,
// launch plans and the kernel sequence of each call.  See include/dflash.h.
#include <algorithm>
#include <cmath>
#include <cstring>
#include <mutex>

#include "../../include/dflash.h"
#include "internal.h"

using namespace dflash;

namespace {

constexpr size_t kAlign = 256;
constexpr size_t kPartialCap = size_t(32) << 20;   // split-K partial tiles of the streaming GEMM
constexpr size_t kPartialMax = size_t(512) << 20;  // upper bound with the tiled GEMM
constexpr int kGemmCounters = 1 << 16;
constexpr int kSplitBelow = 256;                   // streaming GEMM: split K only below this many tiles (one per CU)
constexpr int kCUs = 256;
constexpr int kTiledMinRows = 128;                 // bf16 GEMMs with at least this many rows go tiled

size_t align_up(size_t x) { return (x + kAlign - 1) / kAlign * kAlign; }
int cdiv(int a, int b) { return (a + b - 1) / b; }
int round_up(int a, int b) { return cdiv(a, b) * b; }

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }
bool aligned4(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 3u) == 0; }
bool aligned8(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 7u) == 0; }

bool is_f32(const dflash_dims& d) { return d.dtype == DFLASH_F32; }
size_t elem(const dflash_dims& d) { return is_f32(d) ? 4 : 2; }  // weights, activations, cache

bool dims_ok(const dflash_dims* d) {
  if (d == nullptr) return false;
  // field ranges that keep every size and index computed from them far inside int32
  // (per field) and size_t (products)
  if (d->batch < 1 || d->batch > (1 << 16) || d->block_k < 1 || d->block_k > 63) return false;
  if (d->n_layers < 1 || d->n_layers > 64) return false;
  if (d->hidden < 64 || d->hidden > (1 << 16) || d->hidden % 64 != 0) return false;
  if (d->n_q_heads < 1 || d->n_q_heads > 1024 || d->n_kv_heads < 1 || d->n_q_heads % d->n_kv_heads != 0)
    return false;
  if (d->head_dim != 64 && d->head_dim != 128) return false;
  if (d->ffn < 1 || d->ffn > (1 << 20) || d->vocab < 2 || d->vocab > (1 << 24)) return false;
  if (d->n_taps < 1 || d->n_taps > 64 || d->tap_dim < 1 || d->tap_dim > (1 << 16)) return false;
  if (d->window < 1 || d->window > (1 << 24) || d->sink < 0 || d->sink > (1 << 20)) return false;
  if (d->cache_slots > (1 << 26) || d->cache_slots < d->sink + d->window + d->block_k) return false;
  if (d->max_inject_rows > (1 << 16)) return false;
  if (d->dtype != DFLASH_F32 && d->dtype != DFLASH_BF16) return false;
  if (d->max_inject_rows < d->block_k + 1) return false;
  if (!(d->rms_eps >= 0.f) || !(d->rope_theta > 0.f)) return false;
  // 32-bit row indices inside the kernels
  const double mi = double(d->batch) * d->max_inject_rows;
  if (mi * d->hidden > 2.0e9 || double(d->batch) * d->block_k * d->vocab > 4.0e9) return false;
  return true;
}

// ---------------------------------------------------------------------------
// packed weights: one region per matrix, [tiles][K steps][4][64][8]
// ---------------------------------------------------------------------------
struct Region {
  size_t off;  // bytes
  int tiles, S;
};

struct PackLayout {
  Region fuse, lm;
  Region qkv[64], o[64], gu[64], down[64];  // per layer (n_layers <= 64 checked)
  size_t total;
};

bool pack_layout(const dflash_dims& d, PackLayout& P) {
  if (d.n_layers > 64) return false;
  const size_t e = elem(d);
  size_t off = 0;
  auto region = [&](int tiles, int K) {
    Region r{off, tiles, ksteps(K)};
    off = align_up(off + size_t(tiles) * r.S * kTileStepElems * e);
    return r;
  };
  const int qkv_tiles = (d.n_q_heads + 2 * d.n_kv_heads) * (d.head_dim / kBN);
  // Region sizes are multiples of one tile step (4 KB), so the QKV regions of all
  // layers are contiguous: layer l's tiles follow layer l-1's (the injection GEMM
  // walks the K/V head tiles of every layer with one stride).
  P.fuse = region(cdiv(d.hidden, kBN), d.n_taps * d.tap_dim);
  for (int l = 0; l < d.n_layers; ++l) P.qkv[l] = region(qkv_tiles, d.hidden);
  for (int l = 0; l < d.n_layers; ++l) P.o[l] = region(cdiv(d.hidden, kBN), d.n_q_heads * d.head_dim);
  for (int l = 0; l < d.n_layers; ++l) P.gu[l] = region(cdiv(d.ffn, kBN / 2), d.hidden);
  for (int l = 0; l < d.n_layers; ++l) P.down[l] = region(cdiv(d.hidden, kBN), d.ffn);
  P.lm = region(cdiv(d.vocab, kBN), d.hidden);
  P.total = off;
  return true;
}

// ---------------------------------------------------------------------------
// workspace
// ---------------------------------------------------------------------------
struct AttnPlan {
  int n_rb, rows, kps, max_splits;
};

AttnPlan attn_plan(const dflash_dims& d) {
  AttnPlan p;
  const int G = d.n_q_heads / d.n_kv_heads;
  const int row_tiles = cdiv(G * d.block_k, 16);
  // one workgroup per (sequence, kv head, row block of <= 4 tiles, key split); its
  // wavefronts are the row tiles and share every K/V chunk through LDS
  const int nw = std::min(4, row_tiles);
  p.n_rb = cdiv(row_tiles, nw);
  p.rows = 16 * nw;
  // Split keys only for long key lists over few workgroups: a split costs a merge
  // kernel (a fixed few microseconds) plus writing and reading fp32 partials, which
  // measured slower than one workgroup walking up to ~1000 keys, or than leaving the
  // keys whole once there are >= 256 workgroups.  When splitting, fill about 256
  // workgroups with >= 256 keys each.
  const int max_keys = d.sink + d.window + d.block_k;
  const long long base = static_cast<long long>(d.batch) * d.n_kv_heads * p.n_rb;
  p.kps = round_up(max_keys, 32);
  if (max_keys > 1024 && base < 256) {
    const int want = static_cast<int>((256 + base - 1) / base);
    p.kps = std::min(p.kps, std::max(256, round_up(cdiv(max_keys, want), 32)));
  }
  p.max_splits = cdiv(max_keys, p.kps);
  return p;
}

size_t partial_bytes(const dflash_dims& d);

struct Layout {
  size_t h, xa, ssq, q, kb, vb, o, act, cu, ssq_c, partials, counters, keys, attn_cnt, attn_o,
      attn_ml, lse_part, v_part, v_cnt, v_rowlse, v_dec, v_keys, xa2, ssq2, sig, row_map, seq_row0, rope, taps_pk,
      total;
  int v_chunks;
  int np_d, S_d, S_o, S_f;
  AttnPlan ap;
};

Layout layout(const dflash_dims& d) {
  Layout L{};
  const size_t e = elem(d);
  const size_t Mb = size_t(d.batch) * d.block_k;
  const size_t Mi = size_t(d.batch) * d.max_inject_rows;
  const size_t Mb64 = round_up(int(Mb), 64), Mi64 = round_up(int(Mi), 64);  // packed A row padding
  L.np_d = cdiv(d.hidden, kBN);
  L.S_d = ksteps(d.hidden);
  L.S_o = ksteps(d.n_q_heads * d.head_dim);
  L.S_f = ksteps(d.ffn);
  L.ap = attn_plan(d);
  size_t off = 0;
  auto take = [&](size_t bytes) { const size_t o = off; off = align_up(off + bytes); return o; };
  L.h = take(Mb * d.hidden * 4);
  L.xa = take(Mb64 * L.S_d * 32 * e);
  L.ssq = take(Mb * L.np_d * 4);
  L.q = take(Mb * d.n_q_heads * d.head_dim * e);
  L.kb = take(Mb * d.n_kv_heads * d.head_dim * e);
  L.vb = take(Mb * d.n_kv_heads * d.head_dim * e);
  L.o = take(Mb64 * L.S_o * 32 * e);
  L.act = take(Mb64 * L.S_f * 32 * e);
  L.cu = take(Mi64 * L.S_d * 32 * e);
  L.ssq_c = take(Mi * L.np_d * 4);
  L.partials = take(partial_bytes(d));
  L.counters = take(size_t(kGemmCounters) * 4);
  L.keys = take(Mb * size_t(cdiv(d.vocab, kBN)) * 8);  // LM head: best key per row and column tile
  // attention split partials per (sequence, kv head, row block): row blocks of the
  // separate kernel (up to 4 row tiles) or of the persistent layer kernel (up to 2)
  const int row_tiles = cdiv(d.n_q_heads / d.n_kv_heads * d.block_k, 16);
  const int n_rb_alloc = std::max(L.ap.n_rb, cdiv(row_tiles, std::min(2, row_tiles)));
  const size_t groups = size_t(d.batch) * d.n_kv_heads * n_rb_alloc;
  L.attn_cnt = take(groups * 4);
  L.attn_o = take(groups * L.ap.max_splits * 64 * d.head_dim * 4);
  L.attn_ml = take(groups * L.ap.max_splits * 64 * 2 * 4);
  // sampled drafting / verification
  L.lse_part = take(Mb * size_t(cdiv(d.vocab, kBN)) * 8);
  L.v_chunks = verify_chunks(static_cast<long long>(d.batch) * (d.block_k + 1), d.vocab);
  L.v_part = take(size_t(d.batch) * (d.block_k + 1) * L.v_chunks * 8);
  L.v_cnt = take(size_t(d.batch) * (d.block_k + 3) * 4);
  L.v_rowlse = take(size_t(d.batch) * (d.block_k + 1) * 4);
  L.v_dec = take(size_t(d.batch) * 16);
  L.v_keys = take(size_t(d.batch) * 2 * kKeyStride * 8);
  // persistent layer kernel: the MLP input and its RMSNorm partials in their own
  // buffers (the QKV projection may still read xa / ssq while O writes them), and the
  // signal words of every layer
  L.xa2 = take(Mb64 * L.S_d * 32 * e);
  L.ssq2 = take(Mb * L.np_d * 4);
  L.sig = take(size_t(d.n_layers) * kSigWords * 4);
  // compacted rows: blocks of the runtime block size / injection rows, large batches
  L.row_map = take(std::max(Mb, Mi) * 4);
  L.seq_row0 = take((size_t(d.batch) + 1) * 4);
  // (sin, cos) of the rows' rotation angles for the tiled QKV / injection epilogues
  L.rope = take(std::max(Mb, Mi) * (d.head_dim / 2) * 8);
  // the verify round's taps (B(k + 1) rows) fragment-packed for the tiled fusion GEMM
  L.taps_pk = take(e == 2 ? size_t(round_up(d.batch * (d.block_k + 1), 64)) * d.n_taps * d.tap_dim * 2 : 0);
  L.total = off;
  return L;
}

// Tile plan of one weight-streaming GEMM.  Split K while the grid has fewer than
// kSplitBelow tiles (measured on the batch-1 projections with weights cold in HBM:
// fewer splits leave loads idle, more add reduction cost), every split keeps >= 8
// steps, the partial tiles fit their region, and their traffic stays below a quarter
// of the weight bytes.
GemmPlan stream_plan(int M, int n_tiles, int S, bool allow_split, size_t partial_cap) {
  GemmPlan p{};
  p.mt = M <= 16 ? 1 : (M <= 32 ? 2 : 4);
  p.depth = p.mt == 4 ? 2 : (p.mt == 1 ? 8 : 4);
  p.m_tiles = cdiv(M, 16 * p.mt);
  p.n_tiles = n_tiles;
  int splits = 1;
  if (allow_split) {
    const int m_pad = p.m_tiles * 16 * p.mt;
    const int K = S * kKStep;
    while (true) {
      const int s2 = splits * 2;
      if (n_tiles * p.m_tiles * splits >= kSplitBelow) break;
      if (cdiv(S, s2) < 8) break;
      if (double(s2) * M * n_tiles * kBN * 4 > double(std::min(partial_cap, kPartialCap))) break;
      if (s2 > std::max(1, K / (16 * m_pad))) break;
      if (s2 > 16 / p.mt) break;  // partial sums of one thread stay in registers
      if (size_t(p.m_tiles) * n_tiles > size_t(kGemmCounters)) break;
      splits = s2;
    }
  }
  p.steps_per_split = cdiv(S, splits);
  p.splits = cdiv(S, p.steps_per_split);
  // Balanced pieces.  A grid of uniform splits that does not divide evenly over the
  // CUs leaves some CUs with one workgroup and others with two, and the kernel ends
  // with the doubly loaded ones (measured on the batch-1 QKV projection: 384
  // workgroups, main loop 6.7 us on singly and 9.3 us on doubly loaded CUs).  Then
  // aim at two workgroups per CU with near-equal K pieces (P or P + 1 per tile).
  if (allow_split && (size_t(n_tiles) * p.m_tiles * p.splits) % kCUs != 0) {
    const int per_row = 2 * kCUs / p.m_tiles;
    const int base = per_row / n_tiles, extra = per_row % n_tiles;
    const int maxp = base + (extra > 0 ? 1 : 0);
    if (base >= 2 && maxp <= 16 / p.mt && S / maxp >= 8 &&
        double(maxp) * M * n_tiles * kBN * 4 <= double(std::min(partial_cap, kPartialCap)) &&
        size_t(p.m_tiles) * n_tiles <= size_t(kGemmCounters)) {
      p.piece_base = base;
      p.piece_extra = extra;
      p.splits = maxp;
      p.steps_per_split = cdiv(S, base);  // the longest piece
    }
  }
  return p;
}

// Tile plan of one tiled GEMM: 256 x 256 tiles (one workgroup per CU) or 128 x 128
// (two per CU), K split 1..8 ways.  Cost model with per-CU rates measured on MI355X
// (batch-64 and batch-256 drafter shapes, every tile shape and split count timed):
// a 256 x 256 workgroup multiplies at ~4.3 TFLOP/s; 128 x 128 workgroups reach
// ~3.5 TFLOP/s per CU two at a time but only ~2.0 alone (one wavefront per SIMD).
// The dispatcher fills CUs as workgroups finish, so the grid runs in rounds of one
// workgroup per CU slot; a last round of at most one 128 x 128 workgroup per CU
// runs at the single-workgroup rate.  Split K costs its fp32 partial-tile traffic
// plus ~20 us for the last arriver's reduction.  partial_cap = 0 disables splitting.
GemmPlan tiled_plan(int M, int n_tiles, int S, bool allow_split, size_t partial_cap) {
  constexpr double r256 = 4.3e12, r128_pair = 3.5e12, r128_alone = 2.0e12, hbm = 5.0e12, split_fixed = 20e-6;
  constexpr double r128x384 = 4.0e12, r256x128 = 3.7e12;
  GemmPlan best{};
  double best_t = 1e30;
  for (int cfg : {kTile256, kTile128, kTile128x384, kTile256x128}) {
    const int bm = tile_rows(cfg), bn = tile_cols(cfg);
    const int m_tiles = cdiv(M, bm), n_big = cdiv(n_tiles, bn / kBN);
    for (int want = 1; want <= (allow_split ? 8 : 1); ++want) {
      const int sps = cdiv(S, want);
      const int splits = cdiv(S, sps);
      if (splits != want) continue;
      if (splits > 1) {
        if (sps < 16) continue;
        // partials of whole tiles, padding included
        if (double(splits) * m_tiles * bm * n_big * bn * 4 > double(partial_cap)) continue;
        if (size_t(m_tiles) * n_big > size_t(kGemmCounters)) continue;
      }
      const long long n = static_cast<long long>(m_tiles) * n_big * splits;
      const double work = 2.0 * bm * bn * kKStep * sps;  // flops of one workgroup
      double t;
      if (cfg != kTile128) {  // one workgroup per CU
        const double rate = cfg == kTile256 ? r256 : (cfg == kTile128x384 ? r128x384 : r256x128);
        t = static_cast<double>((n + kCUs - 1) / kCUs) * work / rate;
      } else {
        const long long full = n / (2 * kCUs), rem = n - full * 2 * kCUs;
        t = static_cast<double>(full) * work / (r128_pair / 2);
        if (rem > kCUs) t += work / (r128_pair / 2);
        else if (rem > 0) t += work / r128_alone;
      }
      if (splits > 1) t += 2.0 * splits * M * n_tiles * kBN * 4 / hbm + split_fixed;
      if (t < best_t * 0.999) {
        best_t = t;
        best.tiled = 1;
        best.mt = cfg;
        best.m_tiles = m_tiles;
        best.n_tiles = n_tiles;
        best.splits = splits;
        best.steps_per_split = sps;
        best.depth = 0;
      }
    }
  }
  return best;
}

bool use_tiled(const dflash_dims& d, int M) { return !is_f32(d) && M >= kTiledMinRows; }

GemmPlan gemm_plan(const dflash_dims& d, int epi, int M, int n_tiles, int S, bool allow_split,
                   size_t partial_cap) {
  // The fusion GEMM (K = 5 taps x tap width) goes tiled from 65 rows: one 128-row tile
  // streams fuse_w once where two 64-row streaming tiles read it twice, and its long K
  // amortises the tiled kernel's fixed costs (batch 8's 72 rows: 61 against 66-72 us).
  if (use_tiled(d, M) || (epi == EPI_FUSE && !is_f32(d) && M > 64))
    return tiled_plan(M, n_tiles, S, allow_split && epi != EPI_ARGMAX, partial_cap);
  return stream_plan(M, n_tiles, S, allow_split, partial_cap);
}

// Bytes of split-K partial tiles the GEMMs of this drafter may use: the streaming
// GEMM's fixed cap, or what the tiled plans at the largest row counts ask for.
size_t partial_bytes(const dflash_dims& d) {
  size_t need = kPartialCap;
  const int tph = d.head_dim / kBN;
  const int qkv_tiles = (d.n_q_heads + 2 * d.n_kv_heads) * tph;
  const int D = d.hidden, Sd = ksteps(D);
  struct G { int M, n_tiles, S; };
  // injection row counts: the verify round's k + 1 per sequence and the largest call
  const int Mb = d.batch * d.block_k, Mi = d.batch * d.max_inject_rows;
  const int Mv = d.batch * std::min(d.block_k + 1, d.max_inject_rows);
  const G gs[] = {{Mi, cdiv(D, kBN), ksteps(d.n_taps * d.tap_dim)},
                  {Mi, d.n_layers * 2 * d.n_kv_heads * tph, Sd},
                  {Mv, cdiv(D, kBN), ksteps(d.n_taps * d.tap_dim)},
                  {Mv, d.n_layers * 2 * d.n_kv_heads * tph, Sd},
                  {Mb, qkv_tiles, Sd},
                  {Mb, cdiv(D, kBN), ksteps(d.n_q_heads * d.head_dim)},
                  {Mb, cdiv(d.ffn, kBN / 2), Sd},
                  {Mb, cdiv(D, kBN), ksteps(d.ffn)}};
  for (const G& g : gs) {
    if (!use_tiled(d, g.M)) continue;
    const GemmPlan p = tiled_plan(g.M, g.n_tiles, g.S, true, kPartialMax);
    if (p.splits > 1)
      need = std::max(need, size_t(p.splits) * p.m_tiles * tile_rows(p.mt) *
                                cdiv(g.n_tiles, tile_cols(p.mt) / kBN) * tile_cols(p.mt) * 4);
  }
  return need;
}

struct Ctx {
  const dflash_dims& d;
  const Layout& L;
  const PackLayout& P;
  char* ws;
  const char* packed;
  uint32_t* dev_error;
  const int32_t* m_live = nullptr;   // compacted block rows (draft step), else nullptr
  const int32_t* row_map = nullptr;
  template <typename X> X* at(size_t off) const { return reinterpret_cast<X*>(ws + off); }
  const void* reg(const Region& r) const { return packed + r.off; }
};

GemmArgs base_args(const Ctx& c) {
  GemmArgs a;
  std::memset(&a, 0, sizeof(a));
  a.partials = c.at<float>(c.L.partials);
  a.counters = c.at<unsigned>(c.L.counters);
  a.eps = c.d.rms_eps;
  a.norm_dim = c.d.hidden;
  a.n_q_heads = c.d.n_q_heads;
  a.n_kv_heads = c.d.n_kv_heads;
  a.head_dim = c.d.head_dim;
  a.n_layers = c.d.n_layers;
  a.batch = c.d.batch;
  a.cache_slots = c.d.cache_slots;
  a.sink = c.d.sink;
  a.ffn = c.d.ffn;
  a.theta = c.d.rope_theta;
  a.dev_error = c.dev_error;
  a.m_live = c.m_live;
  a.row_map = c.row_map;
  return a;
}

#define DF_CHECK(call)                             \
  do {                                             \
    if ((call) != hipSuccess) return DFLASH_E_HIP; \
  } while (0)

// The plan of one GEMM, with its split fields copied into the arguments.
GemmPlan plan_gemm(int epi, const Ctx& c, GemmArgs& a, bool allow_split) {
  const size_t cap = partial_bytes(c.d);
  // the tiled fusion GEMM gathers whole 16-byte pieces of tap rows
  const bool fuse_ok = epi != EPI_FUSE || (a.K == a.S * kKStep && a.lda % 8 == 0);
  const GemmPlan p = fuse_ok ? gemm_plan(c.d, epi, a.M, a.n_tiles, a.S, allow_split, cap)
                             : stream_plan(a.M, a.n_tiles, a.S, allow_split, cap);
  a.splits = p.splits;
  a.steps_per_split = p.steps_per_split;
  a.piece_base = p.tiled ? 0 : p.piece_base;
  a.piece_extra = p.tiled ? 0 : p.piece_extra;
  a.m_tiles = p.m_tiles;
  return p;
}

int device_cus(int* cus);

int run_gemm(int epi, const Ctx& c, GemmArgs a, bool allow_split, hipStream_t s) {
  const GemmPlan p = plan_gemm(epi, c, a, allow_split);
  a.persist = 0;
  // the tiled greedy LM head, and SwiGLU on 256-row tiles (whose epilogues work from the
  // accumulators), walk their tiles with one workgroup per CU once there are at least
  // two tiles per CU: each tile's first loads overlap the previous epilogue
  if (p.tiled && p.splits == 1 &&
      (epi == EPI_ARGMAX ? p.mt != kTile128 : (epi == EPI_SWIGLU && (p.mt == kTile256 || p.mt == kTile256x128)))) {
    int cus = 0;
    const long long tiles = static_cast<long long>(p.m_tiles) * ((p.n_tiles * kBN + tile_cols(p.mt) - 1) / tile_cols(p.mt));
    if (device_cus(&cus) == DFLASH_OK && cus % 8 == 0 && tiles >= 2ll * cus) a.persist = cus;
  }
  if (p.tiled) DF_CHECK(launch_gemm_tiled(epi, p, a, s));
  else DF_CHECK(launch_gemm(epi, is_f32(c.d), p, a, s));
  return DFLASH_OK;
}

// The separate streaming kernel's grid, as the persistent kernel's work items.
PhaseGrid stream_grid(const GemmPlan& p) {
  if (p.piece_base > 0) return PhaseGrid{p.n_tiles * p.piece_base + p.piece_extra, p.m_tiles, 1};
  return PhaseGrid{p.n_tiles, p.m_tiles, p.splits};
}

// Compute units of the current device, looked up once per device.
int device_cus(int* cus) {
  static std::mutex mu;
  static int n[64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return DFLASH_E_HIP;
  std::lock_guard<std::mutex> lock(mu);
  if (n[dev] == 0 && (hipDeviceGetAttribute(&n[dev], hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
                      n[dev] <= 0)) {
    n[dev] = 0;
    return DFLASH_E_HIP;
  }
  *cus = n[dev];
  return DFLASH_OK;
}

bool sampling_ok(const dflash_sampling* smp) {
  return smp != nullptr && smp->temperature > 0.f && std::isfinite(smp->temperature) && smp->reserved == 0 &&
         (smp->step_dev == nullptr || aligned8(smp->step_dev));
}

// smp == nullptr: greedy drafts (argmax); otherwise Gumbel-max draws at temperature
// smp->temperature, raw logits to logits_out and row log-sum-exps of logits / T to lse_out.
// zero_counters: clear the workspace's arrival counters before the first kernel (the
// shared scratch of the no-allocation entry point, whose previous contents are not
// the caller's to vouch for).
// persistent: every draft layer as one launch of the persistent layer kernel
// (DFLASH_E_UNSUPPORTED, before anything is enqueued, for drafters it does not cover).
int draft_impl(const dflash_dims* dims, const dflash_weights* w, const dflash_cache* cache,
               const dflash_sampling* smp, int32_t* draft, float* logits_out, float* lse_out,
               void* workspace, size_t workspace_bytes, hipStream_t stream, hipEvent_t ev0,
               hipEvent_t ev1, bool zero_counters = false, bool persistent = false) {
  if (!dims_ok(dims) || w == nullptr || cache == nullptr || draft == nullptr) return DFLASH_E_INVALID;
  if (smp != nullptr && (!sampling_ok(smp) || logits_out == nullptr || lse_out == nullptr || !aligned4(lse_out)))
    return DFLASH_E_INVALID;
  const dflash_dims& d = *dims;
  const void* wp[] = {w->embed, w->mask_embed, w->attn_norm, w->mlp_norm, w->final_norm, w->packed};
  for (const void* p : wp)
    if (p == nullptr || !aligned16(p)) return DFLASH_E_INVALID;
  if (!cache->k || !cache->v || !aligned16(cache->k) || !aligned16(cache->v)) return DFLASH_E_INVALID;
  if (!cache->ctx_len || !cache->anchor || !cache->dev_error || !aligned4(draft)) return DFLASH_E_INVALID;
  if (!aligned4(cache->block_len)) return DFLASH_E_INVALID;
  if (logits_out != nullptr && !aligned4(logits_out)) return DFLASH_E_INVALID;
  PackLayout P;
  if (!pack_layout(d, P)) return DFLASH_E_UNSUPPORTED;
  const Layout L = layout(d);
  if (workspace == nullptr || !aligned16(workspace) || workspace_bytes < L.total) return DFLASH_E_WORKSPACE;

  Ctx c{d, L, P, static_cast<char*>(workspace), static_cast<const char*>(w->packed), cache->dev_error};
  const bool f32 = is_f32(d);
  const size_t e = elem(d);
  const int D = d.hidden, k = d.block_k, B = d.batch, F = d.ffn;
  const int Mb = B * k;
  // Runtime block size on the tiled GEMMs (greedy drafts): the rows of shrunken blocks
  // are compacted away, so the GEMMs multiply only the live rows
  const bool compact = cache->block_len != nullptr && smp == nullptr && !persistent && use_tiled(d, Mb);
  if (compact) {
    CompactArgs ca;
    ca.counts = cache->block_len;
    ca.seq_row0 = c.at<int32_t>(L.seq_row0);
    ca.row_map = c.at<int32_t>(L.row_map);
    ca.batch = B;
    ca.rows_per_seq = k;
    ca.dev_error = cache->dev_error;
    ca.err_bit = DFLASH_DEVERR_BLOCK;
    DF_CHECK(launch_compact_rows(ca, stream));
    c.m_live = ca.seq_row0 + B;
    c.row_map = ca.row_map;
  }

  // Persistent layer kernel: bf16 drafters whose block rows stay on the streaming GEMM,
  // head_dim 128; attention with at most two 16-row tiles per workgroup (the same
  // per-row arithmetic as the separate kernel, so the same results bitwise)
  const int G = d.n_q_heads / d.n_kv_heads;
  const int p_nw = std::min(2, cdiv(G * k, 16));
  const int p_mt = Mb <= 16 ? 1 : (Mb <= 32 ? 2 : 4);
  int p_capacity = 0;
  if (persistent) {
    if (f32 || use_tiled(d, Mb) || Mb > 64 || d.head_dim != 128) return DFLASH_E_UNSUPPORTED;
    int cus = 0;
    if (int st = device_cus(&cus)) return st;
    p_capacity = persistent_capacity(p_mt, p_nw, cus);
    if (p_capacity <= 0) return DFLASH_E_UNSUPPORTED;
    const int row_tiles = cdiv(G * k, 16);
    if (d.n_kv_heads > kSigMaxHkv || B * d.n_kv_heads * cdiv(row_tiles, p_nw) > kSigMaxGroups ||
        cdiv(F, kBN / 2) > kSigMaxGu)
      return DFLASH_E_UNSUPPORTED;
    DF_CHECK(launch_fill_zero(c.at<void>(L.sig), size_t(d.n_layers) * kSigWords * 4, stream));
  }
  // the tiled QKV epilogue reads the rows' rotation angles from a table built once
  // per step (every layer rotates the same positions)
  const float2* rope_tab = nullptr;
  if (use_tiled(d, Mb) && !persistent) {
    RopeTabArgs ra{cache->ctx_len, c.at<float2>(L.rope), B, k, d.head_dim, d.rope_theta};
    DF_CHECK(launch_rope_table(ra, stream));
    rope_tab = ra.tab;
  }
  const int hq_dh = d.n_q_heads * d.head_dim;
  const size_t layer_cache = size_t(B) * d.n_kv_heads * d.cache_slots * d.head_dim * e;
  auto gain = [&](const void* base, int l) { return static_cast<const char*>(base) + size_t(l) * D * e; };

  if (zero_counters) {
    DF_CHECK(launch_fill_zero(c.at<void>(L.counters), L.keys - L.counters, stream));
    DF_CHECK(launch_fill_zero(c.at<void>(L.attn_cnt), L.attn_o - L.attn_cnt, stream));
  }

  EmbedArgs em{};
  em.anchor = cache->anchor;
  em.ctx_len = cache->ctx_len;
  em.embed = w->embed;
  em.mask_embed = w->mask_embed;
  em.gain = w->attn_norm;
  em.h = c.at<float>(L.h);
  em.xa = c.at<void>(L.xa);
  em.ssq = c.at<float>(L.ssq);
  em.batch = B;
  em.block_k = k;
  em.hidden = D;
  em.vocab = d.vocab;
  em.dev_error = cache->dev_error;
  em.row_map = c.row_map;
  em.m_live = c.m_live;
  DF_CHECK(launch_embed(f32, em, stream));

  for (int l = 0; l < d.n_layers; ++l) {
    // persistent mode: the layer's four GEMMs and its attention are collected into one
    // launch of the layer kernel; otherwise each runs as its own kernel
    LayerArgs la{};
    auto stage_gemm = [&](int slot, int epi, GemmArgs ga) -> int {
      if (!persistent) return run_gemm(epi, c, ga, true, stream);
      const GemmPlan gp = plan_gemm(epi, c, ga, true);
      if (gp.tiled || gp.mt != p_mt || gp.m_tiles != 1) return DFLASH_E_UNSUPPORTED;
      // the four GEMMs of a layer overlap in time: each gets its own quarter of the
      // split-K partials and of the arrival counters
      const size_t quarter = partial_bytes(d) / 4 / 256 * 256;
      if (size_t(gp.splits) * ga.M * gp.n_tiles * kBN * 4 > quarter ||
          size_t(gp.m_tiles) * gp.n_tiles > size_t(kGemmCounters / 4))
        return DFLASH_E_UNSUPPORTED;
      ga.partials = c.at<float>(L.partials + slot * quarter);
      ga.counters = c.at<unsigned>(L.counters) + slot * (kGemmCounters / 4);
      la.gemm[slot] = ga;
      la.grid[slot] = stream_grid(gp);
      return DFLASH_OK;
    };
    // RMSNorm + fused QKV projection + RoPE
    GemmArgs a = base_args(c);
    a.A = c.at<void>(L.xa);
    a.M = Mb;
    a.K = D;
    a.S = L.S_d;
    a.W = c.reg(P.qkv[l]);
    a.N = (d.n_q_heads + 2 * d.n_kv_heads) * d.head_dim;
    a.n_tiles = P.qkv[l].tiles;
    a.ssq_in = c.at<float>(L.ssq);
    a.np_in = l == 0 ? 1 : L.np_d;
    a.out = c.at<void>(L.q);
    a.out2 = c.at<void>(L.kb);
    a.out3 = c.at<void>(L.vb);
    a.rows_per_seq = k;
    a.ctx_len = cache->ctx_len;
    a.rope_tab = rope_tab;
    if (int st = stage_gemm(0, EPI_QKV, a)) return st;

    // block attention over window + block
    AttnArgs at{};
    at.q = c.at<void>(L.q);
    at.kb = c.at<void>(L.kb);
    at.vb = c.at<void>(L.vb);
    at.cache_k = static_cast<const char*>(cache->k) + size_t(l) * layer_cache;
    at.cache_v = static_cast<const char*>(cache->v) + size_t(l) * layer_cache;
    at.ctx_len = cache->ctx_len;
    at.out = c.at<void>(L.o);
    at.out_steps = L.S_o;
    at.part_o = c.at<float>(L.attn_o);
    at.part_ml = c.at<float>(L.attn_ml);
    at.counters = c.at<unsigned>(L.attn_cnt);
    at.batch = B;
    at.block_k = k;
    at.n_q_heads = d.n_q_heads;
    at.n_kv_heads = d.n_kv_heads;
    at.head_dim = d.head_dim;
    at.cache_slots = d.cache_slots;
    at.window = d.window;
    at.sink = d.sink;
    at.keys_per_split = L.ap.kps;
    at.block_len = cache->block_len;
    at.max_splits = L.ap.max_splits;
    at.n_rb = L.ap.n_rb;
    at.rows_per_block = L.ap.rows;
    // long full-attention windows over many sequences: contexts may be ragged
    at.balance = L.ap.max_splits == 1 && B >= 16 && B <= kMaxBalanceBatch && d.window > 1024;
    at.seq_row0 = compact ? c.at<int32_t>(L.seq_row0) : nullptr;
    if (!persistent) {
      DF_CHECK(launch_attention(f32, at, stream));
    } else {
      // rows of at most two 16-row tiles per workgroup (256 threads, two key groups)
      const int row_tiles = cdiv(G * k, 16);
      at.rows_per_block = 16 * p_nw;
      at.n_rb = cdiv(row_tiles, p_nw);
      at.balance = 0;  // the dependency signals are per row group in item order
      la.attn = at;
      la.attn_items = B * d.n_kv_heads * at.n_rb * at.max_splits;
      la.merge_items = at.max_splits > 1 ? B * d.n_kv_heads * at.n_rb * at.rows_per_block : 0;  // one row each
    }

    // output projection + residual; produces the MLP's RMSNorm input
    a = base_args(c);
    a.A = c.at<void>(L.o);
    a.M = Mb;
    a.K = hq_dh;
    a.S = L.S_o;
    a.W = c.reg(P.o[l]);
    a.N = D;
    a.n_tiles = P.o[l].tiles;
    a.h = c.at<float>(L.h);
    a.out = c.at<void>(persistent ? L.xa2 : L.xa);
    a.out_steps = L.S_d;
    a.gain = gain(w->mlp_norm, l);
    a.ssq_out = c.at<float>(persistent ? L.ssq2 : L.ssq);
    a.np_out = L.np_d;
    if (int st = stage_gemm(1, EPI_RESID, a)) return st;

    // RMSNorm + gate/up projection + SwiGLU
    a = base_args(c);
    a.A = c.at<void>(persistent ? L.xa2 : L.xa);
    a.M = Mb;
    a.K = D;
    a.S = L.S_d;
    a.W = c.reg(P.gu[l]);
    a.N = F;
    a.n_tiles = P.gu[l].tiles;
    a.ssq_in = c.at<float>(persistent ? L.ssq2 : L.ssq);
    a.np_in = L.np_d;
    a.out = c.at<void>(L.act);
    a.out_steps = L.S_f;
    if (int st = stage_gemm(2, EPI_SWIGLU, a)) return st;

    // down projection + residual; produces the next RMSNorm input
    a = base_args(c);
    a.A = c.at<void>(L.act);
    a.M = Mb;
    a.K = F;
    a.S = L.S_f;
    a.W = c.reg(P.down[l]);
    a.N = D;
    a.n_tiles = P.down[l].tiles;
    a.h = c.at<float>(L.h);
    a.out = c.at<void>(L.xa);
    a.out_steps = L.S_d;
    a.gain = l + 1 < d.n_layers ? gain(w->attn_norm, l + 1) : w->final_norm;
    a.ssq_out = c.at<float>(L.ssq);
    a.np_out = L.np_d;
    if (int st = stage_gemm(3, EPI_RESID, a)) return st;

    if (persistent) {
      la.sig = c.at<unsigned>(L.sig) + size_t(l) * kSigWords;
      la.dev_error = cache->dev_error;
      la.group = G;
      la.tiles_per_head = d.head_dim / kBN;
      la.o_tiles = la.grid[1].x > 0 ? P.o[l].tiles : 0;
      la.fin_need = la.merge_items > 0 ? B * la.attn.n_rb * la.attn.rows_per_block : B * la.attn.n_rb;
      int items = std::max(la.attn_items, la.merge_items);
      for (const PhaseGrid& pg : la.grid) items = std::max(items, pg.x * pg.y * pg.z);
      DF_CHECK(launch_layer_persistent(la, p_mt, p_nw, std::min(items, p_capacity), stream));
    }
  }

  // final RMSNorm + LM head + split-vocab argmax
  GemmArgs a = base_args(c);
  a.A = c.at<void>(L.xa);
  a.M = Mb;
  a.K = D;
  a.S = L.S_d;
  a.W = c.reg(P.lm);
  a.N = d.vocab;
  a.n_tiles = P.lm.tiles;
  a.ssq_in = c.at<float>(L.ssq);
  a.np_in = L.np_d;
  a.keys = c.at<unsigned long long>(L.keys);
  a.draft = draft;
  a.logits = logits_out;
  a.block_len = cache->block_len;
  a.rows_per_seq = d.block_k;
  const int epi = smp != nullptr ? EPI_SAMPLE : EPI_ARGMAX;
  // one key (and with sampling one (max, sum) pair) per row and column tile
  const GemmPlan hp = gemm_plan(d, epi, a.M, a.n_tiles, a.S, false, partial_bytes(d));
  a.n_parts = hp.tiled ? cdiv(a.n_tiles, tile_cols(hp.mt) / kBN) : a.n_tiles;
  if (smp != nullptr) {
    a.inv_temp = 1.f / smp->temperature;
    a.seed = smp->seed;
    a.step = smp->step;
    a.step_dev = reinterpret_cast<const unsigned long long*>(smp->step_dev);
    a.lse_part = c.at<float2>(L.lse_part);
  }
  if (ev0) DF_CHECK(hipEventRecord(ev0, stream));
  if (int st = run_gemm(epi, c, a, false, stream)) return st;
  if (ev1) DF_CHECK(hipEventRecord(ev1, stream));
  HeadFinalizeArgs f;
  f.keys = a.keys;
  f.part = smp != nullptr ? a.lse_part : nullptr;
  f.n_parts = a.n_parts;
  f.rows = a.M;
  f.rows_per_seq = d.block_k;
  f.draft = draft;
  f.lse = smp != nullptr ? lse_out : nullptr;
  f.block_len = cache->block_len;
  f.seq_row0 = compact ? c.at<int32_t>(L.seq_row0) : nullptr;
  DF_CHECK(launch_head_finalize(f, stream));
  return DFLASH_OK;
}

// ---------------------------------------------------------------------------
// No-allocation draft step: the workspace is a static device array of the library
// (one per GPU, held until the process ends) instead of a caller's buffer.
// ---------------------------------------------------------------------------
constexpr size_t kScratchBytes = DFLASH_NOALLOC_SCRATCH_BYTES;
constexpr int kMaxDevices = 64;

}  // namespace

static __device__ __align__(256) unsigned char scratch[kScratchBytes];

namespace {

// Device address of `scratch` on the current device, looked up once per device
// (each device holds its own copy of the array).  The host-side name of the array is
// only a stand-in and never reaches a kernel.
void* scratch_ptr(int* status) {
  static std::mutex mu;
  static void* ptrs[kMaxDevices];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) {
    *status = DFLASH_E_HIP;
    return nullptr;
  }
  std::lock_guard<std::mutex> lock(mu);
  if (ptrs[dev] == nullptr) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || p == nullptr) {
      *status = DFLASH_E_HIP;
      return nullptr;
    }
    ptrs[dev] = p;
  }
  *status = DFLASH_OK;
  return ptrs[dev];
}

}  // namespace

extern "C" {

size_t dflash_workspace_bytes(const dflash_dims* dims) {
  if (!dims_ok(dims)) return 0;
  return layout(*dims).total;
}

size_t dflash_packed_bytes(const dflash_dims* dims) {
  PackLayout P;
  if (!dims_ok(dims) || !pack_layout(*dims, P)) return 0;
  return P.total;
}

const char* dflash_status_string(int status) {
  switch (status) {
    case DFLASH_OK: return "ok";
    case DFLASH_E_INVALID: return "invalid argument";
    case DFLASH_E_UNSUPPORTED: return "unsupported configuration";
    case DFLASH_E_WORKSPACE: return "workspace missing or too small";
    case DFLASH_E_HIP: return "HIP runtime error";
    case DFLASH_E_TOO_LARGE: return "workspace of these dims exceeds the no-allocation scratch";
    default: return "unknown status";
  }
}

int dflash_pack_weights(const dflash_dims* dims, const dflash_weights* w, void* packed,
                        size_t packed_bytes, uint32_t* dev_error, hipStream_t stream) {
  if (!dims_ok(dims) || w == nullptr || packed == nullptr || !aligned16(packed)) return DFLASH_E_INVALID;
  const dflash_dims& d = *dims;
  PackLayout P;
  if (!pack_layout(d, P)) return DFLASH_E_UNSUPPORTED;
  if (packed_bytes < P.total) return DFLASH_E_INVALID;
  const void* src[] = {w->fuse_w, w->w_qkv, w->w_o, w->w_gate_up, w->w_down, w->lm_head};
  for (const void* p : src)
    if (p == nullptr || !aligned16(p)) return DFLASH_E_INVALID;
  if (dev_error == nullptr) return DFLASH_E_INVALID;
  const bool f32 = is_f32(d);
  const size_t e = elem(d);
  char* base = static_cast<char*>(packed);
  const int D = d.hidden, F = d.ffn;
  const int qkv_rows = (d.n_q_heads + 2 * d.n_kv_heads) * d.head_dim;
  const int hq_dh = d.n_q_heads * d.head_dim;
  auto pack = [&](const Region& r, const void* srcp, int K, int N, int kind, int dst_f16) {
    PackArgs a{};
    a.src = srcp;
    a.K = K;
    a.N = N;
    a.n_tiles = r.tiles;
    a.S = r.S;
    a.kind = kind;
    a.head_dim = d.head_dim;
    a.ffn = F;
    a.dst = base + r.off;
    a.dst_f16 = dst_f16;
    a.dev_error = dev_error;
    return launch_pack(f32, a, stream);
  };
  auto layer = [&](const void* p, size_t elems, int l) { return static_cast<const char*>(p) + size_t(l) * elems * e; };
  DF_CHECK(pack(P.fuse, w->fuse_w, d.n_taps * d.tap_dim, D, PACK_PLAIN, 0));
  for (int l = 0; l < d.n_layers; ++l) {
    DF_CHECK(pack(P.qkv[l], layer(w->w_qkv, size_t(qkv_rows) * D, l), D, qkv_rows, PACK_HEADS, 1));
    DF_CHECK(pack(P.o[l], layer(w->w_o, size_t(D) * hq_dh, l), hq_dh, D, PACK_PLAIN, 1));
    DF_CHECK(pack(P.gu[l], layer(w->w_gate_up, size_t(2) * F * D, l), D, F, PACK_SWIGLU, 1));
    DF_CHECK(pack(P.down[l], layer(w->w_down, size_t(D) * F, l), F, D, PACK_PLAIN, 1));
  }
  DF_CHECK(pack(P.lm, w->lm_head, D, d.vocab, PACK_PLAIN, 1));
  return DFLASH_OK;
}

int dflash_fuse_inject(const dflash_dims* dims, const dflash_weights* w, const void* taps,
                       const int32_t* n_rows, int32_t n_max, int32_t commit,
                       const dflash_cache* cache, void* workspace, size_t workspace_bytes,
                       hipStream_t stream) {
  if (!dims_ok(dims) || w == nullptr || cache == nullptr) return DFLASH_E_INVALID;
  const dflash_dims& d = *dims;
  if (taps == nullptr || !aligned16(taps) || n_rows == nullptr || !aligned4(n_rows)) return DFLASH_E_INVALID;
  if (n_max < 1 || n_max > d.max_inject_rows || (commit != 0 && commit != 1)) return DFLASH_E_INVALID;
  if (!w->fuse_norm || !w->packed || !aligned16(w->fuse_norm) || !aligned16(w->packed)) return DFLASH_E_INVALID;
  if (!cache->k || !cache->v || !aligned16(cache->k) || !aligned16(cache->v)) return DFLASH_E_INVALID;
  if (!cache->ctx_len || !cache->dev_error) return DFLASH_E_INVALID;
  PackLayout P;
  if (!pack_layout(d, P)) return DFLASH_E_UNSUPPORTED;
  const Layout L = layout(d);
  if (workspace == nullptr || !aligned16(workspace) || workspace_bytes < L.total) return DFLASH_E_WORKSPACE;

  Ctx c{d, L, P, static_cast<char*>(workspace), static_cast<const char*>(w->packed), cache->dev_error};
  const int D = d.hidden;
  const int Mi = d.batch * n_max;
  const int K = d.n_taps * d.tap_dim;
  const int tph = d.head_dim / kBN;
  // both GEMMs on the tiled kernel: only the n_rows[b] rows of each sequence are
  // multiplied (compacted), not n_max, and the injection epilogue reads the rows'
  // rotation angles from a table
  const float2* rope_tab = nullptr;
  if (use_tiled(d, Mi)) {
    CompactArgs ca;
    ca.counts = n_rows;
    ca.seq_row0 = c.at<int32_t>(L.seq_row0);
    ca.row_map = c.at<int32_t>(L.row_map);
    ca.batch = d.batch;
    ca.rows_per_seq = n_max;
    ca.dev_error = cache->dev_error;
    ca.err_bit = DFLASH_DEVERR_ROWS;
    DF_CHECK(launch_compact_rows(ca, stream));
    c.m_live = ca.seq_row0 + d.batch;
    c.row_map = ca.row_map;
    RopeTabArgs ra{cache->ctx_len, c.at<float2>(L.rope), d.batch, n_max, d.head_dim, d.rope_theta};
    DF_CHECK(launch_rope_table(ra, stream));
    rope_tab = ra.tab;
  }

  GemmArgs a = base_args(c);
  a.A = taps;
  a.lda = K;
  a.M = Mi;
  a.K = K;
  a.S = P.fuse.S;
  a.W = c.reg(P.fuse);
  a.N = D;
  a.n_tiles = P.fuse.tiles;
  a.out = c.at<void>(L.cu);
  a.out_steps = L.S_d;
  a.gain = w->fuse_norm;
  a.ssq_out = c.at<float>(L.ssq_c);
  a.np_out = L.np_d;
  {
    // On the tiled kernel, the verify round's taps are fragment-packed first: the GEMM
    // then streams contiguous 1 KB chunks instead of gathering 16 rows per load.
    GemmArgs probe = a;
    const GemmPlan fp = plan_gemm(EPI_FUSE, c, probe, true);
    if (fp.tiled && !is_f32(d) && n_max <= d.block_k + 1 && a.K == a.S * kKStep) {
      PackTapsArgs pk{taps, c.at<void>(L.taps_pk), K, Mi, a.S, c.row_map, c.m_live};
      DF_CHECK(launch_pack_taps(pk, stream));
      a.A = pk.out;
      a.a_packed = 1;
      a.row_map = nullptr;  // the packed rows are already the compacted ones
    }
  }
  if (int st = run_gemm(EPI_FUSE, c, a, true, stream)) return st;

  // K/V injection: the K and V head tiles of every layer's packed QKV region
  a = base_args(c);
  a.A = c.at<void>(L.cu);
  a.M = Mi;
  a.K = D;
  a.S = L.S_d;
  a.W = c.reg(P.qkv[0]);
  a.layer_tiles = P.qkv[0].tiles;
  a.inj_tile0 = d.n_q_heads * tph;
  a.inj_tiles = 2 * d.n_kv_heads * tph;
  a.N = d.n_layers * 2 * d.n_kv_heads * d.head_dim;
  a.n_tiles = d.n_layers * a.inj_tiles;
  a.ssq_in = c.at<float>(L.ssq_c);
  a.np_in = L.np_d;
  a.rows_per_seq = n_max;
  a.ctx_len = cache->ctx_len;
  a.n_rows = n_rows;
  a.cache_k = cache->k;
  a.cache_v = cache->v;
  a.rope_tab = rope_tab;
  if (int st = run_gemm(EPI_INJECT, c, a, true, stream)) return st;

  if (commit) DF_CHECK(launch_commit_rows(cache->ctx_len, n_rows, d.batch, n_max, cache->dev_error, stream));
  return DFLASH_OK;
}

int dflash_draft_step(const dflash_dims* dims, const dflash_weights* w, const dflash_cache* cache,
                      int32_t* draft, float* logits_out, void* workspace, size_t workspace_bytes,
                      hipStream_t stream) {
  return draft_impl(dims, w, cache, nullptr, draft, logits_out, nullptr, workspace, workspace_bytes, stream,
                    nullptr, nullptr);
}

int dflash_draft_step_sampled(const dflash_dims* dims, const dflash_weights* w, const dflash_cache* cache,
                              const dflash_sampling* sampling, int32_t* draft, float* logits_out,
                              float* lse_out, void* workspace, size_t workspace_bytes, hipStream_t stream) {
  if (sampling == nullptr) return DFLASH_E_INVALID;
  return draft_impl(dims, w, cache, sampling, draft, logits_out, lse_out, workspace, workspace_bytes, stream,
                    nullptr, nullptr);
}

int dflash_draft_step_noalloc(const dflash_dims* dims, const dflash_weights* w, const dflash_cache* cache,
                              int32_t* draft, float* logits_out, hipStream_t stream) {
  if (!dims_ok(dims)) return DFLASH_E_INVALID;
  if (layout(*dims).total > kScratchBytes) return DFLASH_E_TOO_LARGE;
  int st = DFLASH_OK;
  void* ws = scratch_ptr(&st);
  if (st != DFLASH_OK) return st;
  return draft_impl(dims, w, cache, nullptr, draft, logits_out, nullptr, ws, kScratchBytes, stream, nullptr,
                    nullptr, true);
}

int dflash_draft_step_persistent(const dflash_dims* dims, const dflash_weights* w, const dflash_cache* cache,
                                 int32_t* draft, float* logits_out, void* workspace, size_t workspace_bytes,
                                 hipStream_t stream) {
  return draft_impl(dims, w, cache, nullptr, draft, logits_out, nullptr, workspace, workspace_bytes, stream, nullptr,
                    nullptr, false, true);
}

int dflash_draft_step_timed(const dflash_dims* dims, const dflash_weights* w,
                            const dflash_cache* cache, int32_t* draft, float* logits_out,
                            void* workspace, size_t workspace_bytes, hipStream_t stream,
                            hipEvent_t head_begin, hipEvent_t head_end) {
  return draft_impl(dims, w, cache, nullptr, draft, logits_out, nullptr, workspace, workspace_bytes, stream,
                    head_begin, head_end);
}

int dflash_draft_step_sampled_timed(const dflash_dims* dims, const dflash_weights* w,
                                    const dflash_cache* cache, const dflash_sampling* sampling,
                                    int32_t* draft, float* logits_out, float* lse_out, void* workspace,
                                    size_t workspace_bytes, hipStream_t stream, hipEvent_t head_begin,
                                    hipEvent_t head_end) {
  if (sampling == nullptr) return DFLASH_E_INVALID;
  return draft_impl(dims, w, cache, sampling, draft, logits_out, lse_out, workspace, workspace_bytes, stream,
                    head_begin, head_end);
}

int dflash_verify_commit(const dflash_dims* dims, const int32_t* draft, const int32_t* target,
                         const dflash_cache* cache, int32_t* accept_len, int32_t* out_tokens,
                         hipStream_t stream) {
  if (!dims_ok(dims) || cache == nullptr) return DFLASH_E_INVALID;
  if (!draft || !target || !accept_len || !out_tokens || !cache->ctx_len || !cache->anchor ||
      !cache->dev_error)
    return DFLASH_E_INVALID;
  if (!aligned4(draft) || !aligned4(target) || !aligned4(accept_len) || !aligned4(out_tokens))
    return DFLASH_E_INVALID;
  VerifyArgs v{};
  v.draft = draft;
  v.target = target;
  v.ctx_len = cache->ctx_len;
  v.anchor = cache->anchor;
  v.accept_len = accept_len;
  v.out_tokens = out_tokens;
  v.dev_error = cache->dev_error;
  v.block_len = cache->block_len;
  v.batch = dims->batch;
  v.block_k = dims->block_k;
  v.vocab = dims->vocab;
  if (!aligned4(cache->block_len)) return DFLASH_E_INVALID;
  DF_CHECK(launch_verify(v, stream));
  return DFLASH_OK;
}

int dflash_verify_sampled(const dflash_dims* dims, const dflash_sampling* sampling, const int32_t* draft,
                          const float* draft_logits, const float* draft_lse, const float* target_logits,
                          const dflash_cache* cache, int32_t* accept_len, int32_t* out_tokens,
                          void* workspace, size_t workspace_bytes, hipStream_t stream) {
  if (!dims_ok(dims) || cache == nullptr || !sampling_ok(sampling)) return DFLASH_E_INVALID;
  if (!draft || !draft_logits || !draft_lse || !target_logits || !accept_len || !out_tokens ||
      !cache->ctx_len || !cache->anchor || !cache->dev_error)
    return DFLASH_E_INVALID;
  if (!aligned4(draft) || !aligned16(draft_logits) || !aligned4(draft_lse) || !aligned16(target_logits) ||
      !aligned4(accept_len) || !aligned4(out_tokens) || !aligned4(cache->block_len))
    return DFLASH_E_INVALID;
  const dflash_dims& d = *dims;
  const Layout L = layout(d);
  if (workspace == nullptr || !aligned16(workspace) || workspace_bytes < L.total) return DFLASH_E_WORKSPACE;
  char* ws = static_cast<char*>(workspace);
  VerifySampledArgs v{};
  v.draft = draft;
  v.draft_logits = draft_logits;
  v.draft_lse = draft_lse;
  v.target_logits = target_logits;
  v.block_len = cache->block_len;
  v.ctx_len = cache->ctx_len;
  v.anchor = cache->anchor;
  v.accept_len = accept_len;
  v.out_tokens = out_tokens;
  v.dev_error = cache->dev_error;
  v.part = reinterpret_cast<float2*>(ws + L.v_part);
  v.counters = reinterpret_cast<unsigned*>(ws + L.v_cnt);
  v.row_lse = reinterpret_cast<float*>(ws + L.v_rowlse);
  v.decision = reinterpret_cast<float4*>(ws + L.v_dec);
  v.keys = reinterpret_cast<unsigned long long*>(ws + L.v_keys);
  v.batch = d.batch;
  v.block_k = d.block_k;
  v.vocab = d.vocab;
  v.n_chunks = L.v_chunks;
  v.n_chunks_emit = verify_chunks(d.batch, d.vocab);
  v.inv_temp = 1.f / sampling->temperature;
  v.seed = sampling->seed;
  v.step = sampling->step;
  v.step_dev = reinterpret_cast<const unsigned long long*>(sampling->step_dev);
  DF_CHECK(launch_verify_sampled(v, stream));
  return DFLASH_OK;
}

int dflash_adapt_block_len(const dflash_dims* dims, const dflash_adapt_params* params, const int32_t* accept_len,
                           const dflash_cache* cache, float* ema, int32_t* off_left, hipStream_t stream) {
  if (!dims_ok(dims) || params == nullptr || cache == nullptr) return DFLASH_E_INVALID;
  if (!accept_len || !cache->block_len || !cache->dev_error || !ema || !off_left) return DFLASH_E_INVALID;
  if (!aligned4(accept_len) || !aligned4(cache->block_len) || !aligned4(ema) || !aligned4(off_left))
    return DFLASH_E_INVALID;
  const dflash_adapt_params& p = *params;
  if (!(p.alpha > 0.f && p.alpha <= 1.f) || p.cooldown < 1 || !std::isfinite(p.theta_down) ||
      !std::isfinite(p.theta_off) || !std::isfinite(p.theta_up))
    return DFLASH_E_INVALID;
  AdaptArgs a{};
  a.accept_len = accept_len;
  a.block_len = cache->block_len;
  a.ema = ema;
  a.off_left = off_left;
  a.dev_error = cache->dev_error;
  a.batch = dims->batch;
  a.block_k = dims->block_k;
  a.cooldown = p.cooldown;
  a.alpha = p.alpha;
  a.theta_down = p.theta_down;
  a.theta_off = p.theta_off;
  a.theta_up = p.theta_up;
  DF_CHECK(launch_adapt(a, stream));
  return DFLASH_OK;
}

int dflash_debug_poison(const dflash_dims* dims, const dflash_cache* cache, void* workspace,
                        size_t workspace_bytes, int32_t what, hipStream_t stream) {
  if (!dims_ok(dims) || (what & ~(DFLASH_POISON_RING | DFLASH_POISON_WORKSPACE)) != 0) return DFLASH_E_INVALID;
  const dflash_dims& d = *dims;
  if (what & DFLASH_POISON_RING) {
    if (cache == nullptr || !cache->k || !cache->v || !cache->ctx_len || !aligned16(cache->k) ||
        !aligned16(cache->v) || !aligned4(cache->ctx_len))
      return DFLASH_E_INVALID;
    PoisonRingArgs a{};
    a.cache_k = cache->k;
    a.cache_v = cache->v;
    a.ctx_len = cache->ctx_len;
    a.n_layers = d.n_layers;
    a.batch = d.batch;
    a.n_kv_heads = d.n_kv_heads;
    a.cache_slots = d.cache_slots;
    a.sink = d.sink;
    a.n_dead = d.cache_slots - d.sink - d.window;
    a.row_bytes = static_cast<int>(d.head_dim * elem(d));
    DF_CHECK(launch_poison_ring(a, stream));
  }
  if (what & DFLASH_POISON_WORKSPACE) {
    const Layout L = layout(d);
    if (workspace == nullptr || !aligned16(workspace) || workspace_bytes < L.total) return DFLASH_E_WORKSPACE;
    // every region in workspace order; the arrival counters and the zero-initialised
    // keys of the sampled verification carry state between calls (zero) and are kept
    struct R { size_t off; bool keep; };
    const R regions[] = {{L.h, false}, {L.xa, false}, {L.ssq, false}, {L.q, false}, {L.kb, false},
                         {L.vb, false}, {L.o, false}, {L.act, false}, {L.cu, false}, {L.ssq_c, false},
                         {L.partials, false}, {L.counters, true}, {L.keys, false}, {L.attn_cnt, true},
                         {L.attn_o, false}, {L.attn_ml, false}, {L.lse_part, false}, {L.v_part, false},
                         {L.v_cnt, true}, {L.v_rowlse, false}, {L.v_dec, false}, {L.v_keys, true},
                         {L.xa2, false}, {L.ssq2, false}, {L.sig, true}, {L.row_map, false},
                         {L.seq_row0, false}, {L.total, true}};
    char* ws = static_cast<char*>(workspace);
    for (size_t i = 0; i + 1 < sizeof(regions) / sizeof(regions[0]); ++i) {
      if (regions[i].keep) continue;
      DF_CHECK(launch_fill_ones(ws + regions[i].off, (regions[i + 1].off - regions[i].off) / 16 * 16, stream));
    }
  }
  return DFLASH_OK;
}

}  // extern "C"
