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
#include "philox.h"

namespace dflash {

// Targets of one thread's rows in the QKV / INJECT epilogue with the angle table
// (4 threads per row; pass `it` covers row (tid >> 2) + (NT / 4) * it of the tile).
// They are the same for every 64-column subtile of a tile, so a caller that runs
// several subtiles computes them once (epilogue_rows) and hands them in.
template <int BM, int NT>
struct EpiRows {
  static constexpr int RPP = NT / 4, IT = (BM + RPP - 1) / RPP;
  int b[IT], i[IT], pos[IT];
  bool live[IT];
};

// Which rows a QKV / INJECT call writes: row m is (sequence b, block row i) at
// position max(ctx_len[b], 0) + i.  Returns false for rows it skips.  `lead`: the
// thread that reports out-of-range row counts.
template <int EPI>
__device__ __forceinline__ bool epilogue_row_target(const GemmArgs& g, int m, bool lead, int& b, int& i, int& pos) {
  b = m / g.rows_per_seq;
  i = m % g.rows_per_seq;
  if (g.row_map != nullptr) {
    const int e = g.row_map[m];
    b = e / g.rows_per_seq;
    i = e % g.rows_per_seq;
  }
  int n_valid = g.rows_per_seq;
  if constexpr (EPI == EPI_INJECT) {
    const int nr = g.n_rows[b];
    if ((nr < 0 || nr > g.rows_per_seq) && i == 0 && lead) atomicOr(g.dev_error, kErrRows);
    n_valid = min(max(nr, 0), g.rows_per_seq);
  }
  if (i >= n_valid) return false;
  pos = max(g.ctx_len[b], 0) + i;
  // A call with more than C - s ring rows for one sequence: rows i and i + (C - s)
  // share a slot, and writes in position order leave the later one, so the earlier
  // row is not written at all (no two writers race on a slot).
  if constexpr (EPI == EPI_INJECT)
    if (pos >= g.sink && i + (g.cache_slots - g.sink) < n_valid) return false;
  return true;
}

template <int EPI, int BM, int NT>
__device__ __forceinline__ void epilogue_rows(const GemmArgs& g, int m0, int m_end, EpiRows<BM, NT>& er) {
  const int tid = threadIdx.x;
#pragma unroll
  for (int it = 0; it < EpiRows<BM, NT>::IT; ++it) {
    const int r = (tid >> 2) + EpiRows<BM, NT>::RPP * it, m = m0 + r;
    int b = 0, i = 0, pos = 0;
    er.live[it] = r < BM && m < m_end && epilogue_row_target<EPI>(g, m, (tid & 3) == 0, b, i, pos);
    er.b[it] = b;
    er.i[it] = i;
    er.pos[it] = pos;
  }
}

// Rows m >= m_end are skipped (g.M, or the live rows of compacted blocks).
// hres: RESID only, the residual tile prefetched by the caller (row pass `it` of
// this thread, 8 columns), or nullptr to read it here.  COH: the outputs (and the
// residual read here) are device-coherent, for a consumer inside the same launch.
// ROWS: QKV / INJECT with the angle table, `rows` holds the rows' targets from
// epilogue_rows; otherwise they are found here.
template <typename TIN, int EPI, int BM, int NT, bool COH = false, bool ROWS = false>
__device__ __forceinline__ void epilogue_tile(const GemmArgs& g, const float (*tile)[kBN + 4], const float* rs,
                                              int tile_n, int m0, int m_end, const float (*hres)[8],
                                              EpiRows<BM, NT> rows = EpiRows<BM, NT>{}) {
  typedef typename ActOf<TIN>::type TA;
  const int tid = threadIdx.x;
  bool bad = false;
  typedef TA TA8 __attribute__((ext_vector_type(8)));
  if constexpr (EPI == EPI_FUSE || EPI == EPI_RESID) {
    // 8 threads per row, 8 consecutive columns each: one packed 8-element store.
    // The gains (the same columns in every pass) and the residual rows of all
    // passes are loaded before anything is computed, so their latencies overlap.
    constexpr int RPP = NT / 8;  // rows per pass
    constexpr int IT = (BM + RPP - 1) / RPP;
    TA* out = static_cast<TA*>(g.out);
    const TIN* gain = static_cast<const TIN*>(g.gain);
    const int c8 = tid & 7;
    const int n0 = tile_n * kBN + c8 * 8;
    const bool col_ok = n0 < g.N;
    float gn[8];  // several passes: loaded once, up front
    if constexpr (IT > 1) {
#pragma unroll
      for (int j = 0; j < 8; ++j) gn[j] = col_ok ? to_f32(gain[n0 + j]) : 0.f;
    }
    float hv[EPI == EPI_RESID ? IT : 1][8];
    if constexpr (EPI == EPI_RESID) {
#pragma unroll
      for (int it = 0; it < IT; ++it) {
        const int r = (tid >> 3) + RPP * it, m = m0 + r;
        if (hres != nullptr) {
#pragma unroll
          for (int j = 0; j < 8; ++j) hv[it][j] = hres[it][j];
        } else if (r < BM && m < m_end && col_ok) {
          const float4* hp = reinterpret_cast<const float4*>(g.h + static_cast<size_t>(m) * g.N + n0);
          const float4 h0 = get16<COH, float4>(hp), h1 = get16<COH, float4>(hp + 1);
          hv[it][0] = h0.x; hv[it][1] = h0.y; hv[it][2] = h0.z; hv[it][3] = h0.w;
          hv[it][4] = h1.x; hv[it][5] = h1.y; hv[it][6] = h1.z; hv[it][7] = h1.w;
        }
      }
    }
#pragma unroll
    for (int it = 0; it < IT; ++it) {
      const int r = (tid >> 3) + RPP * it;
      const int m = m0 + r;
      float ss = 0.f;
      if (r < BM && m < m_end && col_ok) {
        float x[8];
        TA8 y;
        const float f = rs[r];
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          x[j] = tile[r][c8 * 8 + j] * f;
          if constexpr (EPI == EPI_RESID) x[j] += hv[it][j];
          ss += x[j] * x[j];
          y[j] = to_act<TA>(x[j] * (IT > 1 ? gn[j] : to_f32(gain[n0 + j])), bad);
        }
        put16<COH>(out + pa_index(m, n0, g.out_steps), y);  // 8 activations, 16 bytes (fp16)
        if constexpr (EPI == EPI_RESID) {
          float4* hp = reinterpret_cast<float4*>(g.h + static_cast<size_t>(m) * g.N + n0);
          put16<COH>(hp, make_float4(x[0], x[1], x[2], x[3]));
          put16<COH>(hp + 1, make_float4(x[4], x[5], x[6], x[7]));
        }
      }
      ss = dpp_sum8(ss);
      if (c8 == 0 && r < BM && m < m_end) put<COH>(&g.ssq_out[static_cast<size_t>(m) * g.np_out + tile_n], ss);
    }
  } else if constexpr (EPI == EPI_SWIGLU) {
    // 4 threads per row, 8 consecutive (gate, up) pairs each: one packed 16-byte store
    constexpr int RPP = NT / 4;
    TA* act = static_cast<TA*>(g.out);
    const int p0 = (tid & 3) * 8;
    const int j0 = tile_n * 32 + p0;
#pragma unroll
    for (int it = 0; it < (BM + RPP - 1) / RPP; ++it) {
      const int r = (tid >> 2) + RPP * it, m = m0 + r;
      if (r >= BM || m >= m_end) continue;
      const float f = rs[r];
      const float4 ga = *reinterpret_cast<const float4*>(&tile[r][p0]);
      const float4 gb = *reinterpret_cast<const float4*>(&tile[r][p0 + 4]);
      const float4 ua = *reinterpret_cast<const float4*>(&tile[r][p0 + 32]);
      const float4 ub = *reinterpret_cast<const float4*>(&tile[r][p0 + 36]);
      const float gv[8] = {ga.x, ga.y, ga.z, ga.w, gb.x, gb.y, gb.z, gb.w};
      const float uv[8] = {ua.x, ua.y, ua.z, ua.w, ub.x, ub.y, ub.z, ub.w};
      TA8 y;
#pragma unroll
      for (int q = 0; q < 8; ++q) {
        // columns past ffn are the down projection's K padding: written as zeros, so
        // the product never depends on what the workspace held before
        float v = 0.f;
        if (j0 + q < g.ffn) {
          const float gq = gv[q] * f, uq = uv[q] * f;
          v = gq * __builtin_amdgcn_rcpf(1.f + __builtin_amdgcn_exp2f(-gq * kLog2e)) * uq;
        }
        y[q] = to_act<TA>(v, bad);
      }
      put16<COH>(act + pa_index(m, j0, g.out_steps), y);
    }
  } else if constexpr (EPI == EPI_QKV || EPI == EPI_INJECT) {
    const int dh = g.head_dim, half = dh / 2;
    const int tph = dh / kBN;
    const int sub = tile_n % tph;
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
    auto row_target = [&](int m, int lead, int& b, int& i, int& pos) -> bool {
      return epilogue_row_target<EPI>(g, m, lead != 0, b, i, pos);
    };
    auto row_dst = [&](int m, int b, int pos) -> TA* {
      if constexpr (EPI == EPI_QKV) {
        if (kind == 0) return static_cast<TA*>(g.out) + (static_cast<size_t>(m) * g.n_q_heads + head) * dh;
        return static_cast<TA*>(kind == 1 ? g.out2 : g.out3) + (static_cast<size_t>(m) * g.n_kv_heads + head) * dh;
      } else {
        const int slot = pos < g.sink ? pos : g.sink + (pos - g.sink) % (g.cache_slots - g.sink);
        return static_cast<TA*>(kind == 1 ? g.cache_k : g.cache_v) +
               (((static_cast<size_t>(layer) * g.batch + b) * g.n_kv_heads + head) * g.cache_slots + slot) * dh;
      }
    };
    if (g.rope_tab != nullptr) {
      // 4 threads per row, 8 consecutive rotation pairs each, (sin, cos) from the
      // table: two 16-byte stores per row quarter.  Row targets and angles of every
      // pass are loaded first, so their latencies overlap.
      constexpr int RPP = NT / 4;
      constexpr int IT = (BM + RPP - 1) / RPP;
      const int p0 = (tid & 3) * 8, d0 = sub * 32 + p0;
      EpiRows<BM, NT> er = rows;
      if constexpr (!ROWS) epilogue_rows<EPI, BM, NT>(g, m0, m_end, er);
      float4 sc[IT][4];
#pragma unroll
      for (int it = 0; it < IT; ++it) {
        const int b = er.b[it], i = er.i[it];
        if (er.live[it] && kind != 2) {
          const float4* tp = reinterpret_cast<const float4*>(g.rope_tab + (static_cast<size_t>(b) * g.rows_per_seq + i) * half + d0);
#pragma unroll
          for (int q = 0; q < 4; ++q) sc[it][q] = tp[q];
        }
      }
#pragma unroll
      for (int it = 0; it < IT; ++it) {
        if (!er.live[it]) continue;
        const int r = (tid >> 2) + RPP * it, m = m0 + r;
        const float f = rs[r];
        float x1[8], x2[8];
#pragma unroll
        for (int q = 0; q < 8; q += 4) {
          const float4 a4 = *reinterpret_cast<const float4*>(&tile[r][p0 + q]);
          const float4 b4 = *reinterpret_cast<const float4*>(&tile[r][p0 + 32 + q]);
          x1[q] = a4.x * f; x1[q + 1] = a4.y * f; x1[q + 2] = a4.z * f; x1[q + 3] = a4.w * f;
          x2[q] = b4.x * f; x2[q + 1] = b4.y * f; x2[q + 2] = b4.z * f; x2[q + 3] = b4.w * f;
        }
        TA8 y1, y2;
#pragma unroll
        for (int q = 0; q < 8; ++q) {
          float v1 = x1[q], v2 = x2[q];
          if (kind != 2) {
            const float4 t = sc[it][q >> 1];
            const float sn = (q & 1) ? t.z : t.x, cs = (q & 1) ? t.w : t.y;
            v1 = x1[q] * cs - x2[q] * sn;
            v2 = x2[q] * cs + x1[q] * sn;
          }
          y1[q] = to_act<TA>(v1, bad);
          y2[q] = to_act<TA>(v2, bad);
        }
        TA* dst = row_dst(m, er.b[it], er.pos[it]);
        put16<COH>(dst + d0, y1);
        put16<COH>(dst + d0 + half, y2);
      }
    } else {
      const int p = tid & 31;  // constant per thread: NT is a multiple of 32
      const int d1 = sub * 32 + p;
      const double inv_freq = rope_inv_freq(d1, dh, g.theta);
      for (int idx = tid; idx < BM * 32; idx += NT) {
        const int r = idx >> 5, m = m0 + r;
        if (m >= m_end) continue;
        int b, i, pos;
        if (!row_target(m, p == 0, b, i, pos)) continue;
        const float x1 = tile[r][p] * rs[r], x2 = tile[r][p + 32] * rs[r];
        float y1 = x1, y2 = x2;
        if (kind != 2) {
          float sn, cs;
          rope_sincos(pos, inv_freq, &sn, &cs);
          y1 = x1 * cs - x2 * sn;
          y2 = x2 * cs + x1 * sn;
        }
        TA* dst = row_dst(m, b, pos);
        put<COH>(&dst[d1], to_act<TA>(y1, bad));
        put<COH>(&dst[d1 + half], to_act<TA>(y2, bad));
      }
    }
  }
  report_overflow(bad, g.dev_error);
}

}  // namespace dflash
