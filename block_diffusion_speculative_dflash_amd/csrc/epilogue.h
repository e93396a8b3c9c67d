// Fused GEMM epilogues shared by the weight-streaming and the tiled GEMM.
//
// Input: one 64-column output tile in LDS, tile[r][c] = sum_k A[m0 + r, k] *
// W[64 * tile_n + c, k] for r < BM, and rs[r], the RMSNorm factor of A row m0 + r
// (1 when the rows are not normalised).  The epilogue applies what the method does
// next and writes the next GEMM's operand already fragment-packed:
//   FUSE    u * rs * fuse_norm gain (packed) + per-tile sum of (u * rs)^2
//   RESID   h += tile * rs, next RMSNorm input h * gain (packed) + per-tile sum of h^2
//   SWIGLU  silu(gate) * up, both scaled by rs (tile columns: 32 gate, 32 up)
//   QKV     q / k / v rows with RoPE on q and k (tile columns: 32 rotation pairs)
//   INJECT  RoPE on K, scatter of K and V rows into their cache slots (positions
//           below the sink keep slot = position, the rest ring over C - sink)
// The split-vocab argmax differs between the two GEMMs and lives with each.
// Values stored in fp16 (bf16 drafters) saturate at the fp16 range and set the
// overflow bit of g.dev_error (see to_act); the fp32 residual stream is unaffected.
#pragma once

#include "common.h"
#include "gemm.h"

namespace dflash {

// Rows m >= m_end are skipped (g.M, or the live rows of compacted blocks).
// hres: RESID only, the residual tile prefetched by the caller (row pass `it` of
// this thread, 8 columns), or nullptr to read it here.  COH: the outputs (and the
// residual read here) are device-coherent, for a consumer inside the same launch.
template <typename TIN, int EPI, int BM, int NT, bool COH = false>
__device__ __forceinline__ void epilogue_tile(const GemmArgs& g, const float (*tile)[kBN + 4], const float* rs,
                                              int tile_n, int m0, int m_end, const float (*hres)[8]) {
  typedef typename ActOf<TIN>::type TA;
  const int tid = threadIdx.x;
  bool bad = false;
  if constexpr (EPI == EPI_FUSE || EPI == EPI_RESID) {
    // 8 threads per row, 8 consecutive columns each: one packed 8-element store
    constexpr int RPP = NT / 8;  // rows per pass
    TA* out = static_cast<TA*>(g.out);
    const TIN* gain = static_cast<const TIN*>(g.gain);
    const int c8 = tid & 7;
#pragma unroll
    for (int it = 0; it < (BM + RPP - 1) / RPP; ++it) {
      const int r = (tid >> 3) + RPP * it;
      const int m = m0 + r;
      const int n0 = tile_n * kBN + c8 * 8;
      float ss = 0.f;
      if (r < BM && m < m_end && n0 < g.N) {
        TA* dst = out + pa_index(m, n0, g.out_steps);
        float x[8];
        float hv[8];
        if constexpr (EPI == EPI_RESID) {
          if (hres != nullptr) {
#pragma unroll
            for (int j = 0; j < 8; ++j) hv[j] = hres[it][j];
          } else {
            const float4* hp = reinterpret_cast<const float4*>(g.h + static_cast<size_t>(m) * g.N + n0);
            const float4 h0 = get16<COH, float4>(hp), h1 = get16<COH, float4>(hp + 1);
            hv[0] = h0.x; hv[1] = h0.y; hv[2] = h0.z; hv[3] = h0.w;
            hv[4] = h1.x; hv[5] = h1.y; hv[6] = h1.z; hv[7] = h1.w;
          }
        }
        typedef TA TA8 __attribute__((ext_vector_type(8)));
        TA8 y;
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          x[j] = tile[r][c8 * 8 + j] * rs[r];
          if constexpr (EPI == EPI_RESID) x[j] += hv[j];
          ss += x[j] * x[j];
          y[j] = to_act<TA>(x[j] * to_f32(gain[n0 + j]), bad);
          if constexpr (!COH) dst[j] = y[j];
        }
        if constexpr (COH) coherent_store16(dst, y);  // 8 fp16 activations = 16 bytes
        if constexpr (EPI == EPI_RESID) {
          float4* hp = reinterpret_cast<float4*>(g.h + static_cast<size_t>(m) * g.N + n0);
          put16<COH>(hp, make_float4(x[0], x[1], x[2], x[3]));
          put16<COH>(hp + 1, make_float4(x[4], x[5], x[6], x[7]));
        }
      }
      ss += __shfl_xor(ss, 1, kWave);
      ss += __shfl_xor(ss, 2, kWave);
      ss += __shfl_xor(ss, 4, kWave);
      if (c8 == 0 && r < BM && m < m_end) put<COH>(&g.ssq_out[static_cast<size_t>(m) * g.np_out + tile_n], ss);
    }
  } else if constexpr (EPI == EPI_SWIGLU) {
    TA* act = static_cast<TA*>(g.out);
    for (int idx = tid; idx < BM * 32; idx += NT) {
      const int r = idx >> 5, p = idx & 31, m = m0 + r;
      const int j = tile_n * 32 + p;
      if (m >= m_end) continue;
      // columns past ffn are the down projection's K padding: written as zeros, so
      // the product never depends on what the workspace held before
      float y = 0.f;
      if (j < g.ffn) {
        const float gv = tile[r][p] * rs[r];
        const float uv = tile[r][p + 32] * rs[r];
        y = gv / (1.f + expf(-gv)) * uv;
      }
      put<COH>(&act[pa_index(m, j, g.out_steps)], to_act<TA>(y, bad));
    }
  } else if constexpr (EPI == EPI_QKV || EPI == EPI_INJECT) {
    const int dh = g.head_dim, half = dh / 2;
    const int tph = dh / kBN;
    const int sub = tile_n % tph;
    const int p = tid & 31;  // constant per thread: NT is a multiple of 32
    const int d1 = sub * 32 + p;
    const double inv_freq = rope_inv_freq(d1, dh, g.theta);
    int kind, head, layer = 0;  // kind 0 = q, 1 = k, 2 = v
    if constexpr (EPI == EPI_QKV) {
      const int hd = tile_n / tph;
      kind = hd < g.n_q_heads ? 0 : (hd < g.n_q_heads + g.n_kv_heads ? 1 : 2);
      head = kind == 0 ? hd : (kind == 1 ? hd - g.n_q_heads : hd - g.n_q_heads - g.n_kv_heads);
    } else {
      layer = tile_n / g.inj_tiles;
      const int hd = (tile_n % g.inj_tiles) / tph;
      kind = hd < g.n_kv_heads ? 1 : 2;
      head = kind == 1 ? hd : hd - g.n_kv_heads;
    }
    for (int idx = tid; idx < BM * 32; idx += NT) {
      const int r = idx >> 5, m = m0 + r;
      if (m >= m_end) continue;
      int b = m / g.rows_per_seq, i = m % g.rows_per_seq;
      if (g.row_map != nullptr) {
        const int e = g.row_map[m];
        b = e / g.rows_per_seq;
        i = e % g.rows_per_seq;
      }
      int n_valid = g.rows_per_seq;
      if constexpr (EPI == EPI_INJECT) {
        const int nr = g.n_rows[b];
        if ((nr < 0 || nr > g.rows_per_seq) && i == 0 && p == 0) atomicOr(g.dev_error, kErrRows);
        n_valid = min(max(nr, 0), g.rows_per_seq);
      }
      if (i >= n_valid) continue;
      const int pos = max(g.ctx_len[b], 0) + i;
      // A call with more than C - s ring rows for one sequence: rows i and
      // i + (C - s) share a slot, and writes in position order leave the later one,
      // so the earlier row is not written at all (no two writers race on a slot).
      if constexpr (EPI == EPI_INJECT)
        if (pos >= g.sink && i + (g.cache_slots - g.sink) < n_valid) continue;
      const float x1 = tile[r][p] * rs[r], x2 = tile[r][p + 32] * rs[r];
      float y1 = x1, y2 = x2;
      if (kind != 2) {
        float sn, cs;
        rope_sincos(pos, inv_freq, &sn, &cs);
        y1 = x1 * cs - x2 * sn;
        y2 = x2 * cs + x1 * sn;
      }
      TA* dst;
      if constexpr (EPI == EPI_QKV) {
        if (kind == 0) dst = static_cast<TA*>(g.out) + (static_cast<size_t>(m) * g.n_q_heads + head) * dh;
        else dst = static_cast<TA*>(kind == 1 ? g.out2 : g.out3) + (static_cast<size_t>(m) * g.n_kv_heads + head) * dh;
      } else {
        const int slot = pos < g.sink ? pos : g.sink + (pos - g.sink) % (g.cache_slots - g.sink);
        dst = static_cast<TA*>(kind == 1 ? g.cache_k : g.cache_v) +
              (((static_cast<size_t>(layer) * g.batch + b) * g.n_kv_heads + head) * g.cache_slots + slot) * dh;
      }
      put<COH>(&dst[d1], to_act<TA>(y1, bad));
      put<COH>(&dst[d1 + half], to_act<TA>(y2, bad));
    }
  }
  report_overflow(bad, g.dev_error);
}

}  // namespace dflash
