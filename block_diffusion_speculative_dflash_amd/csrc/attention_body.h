// Device bodies of block attention and of the key-split merge (one workgroup's
// work item each), shared by the standalone kernels (attention.hip) and the
// persistent layer kernel (persist.hip).  The algorithm is described in
// attention.hip.
#pragma once

#include "common.h"
#include "internal.h"

namespace dflash {

constexpr int kRows = 64;  // row stride of the split partials
constexpr int kKC = 32;    // keys per chunk (one MFMA reduction step of P V)

template <typename T> struct VPad;
template <> struct VPad<f16> { static constexpr int value = 16; };   // 288-byte rows: 8 rows on disjoint banks
template <> struct VPad<float> { static constexpr int value = 4; };  // 16-byte rows

// Reductions over the four lanes l, l^16, l^32, l^48 that hold one query row, with
// the gfx950 lane-swap instructions (VALU, no LDS round trip).  Called with the same
// value as both operands, a swap leaves each lane holding its own value and its
// partner's, so the pairwise max / sum is the same in both lanes.
__device__ __forceinline__ float pair_max16(float x) {
  const unsigned u = __float_as_uint(x);
  const auto r = __builtin_amdgcn_permlane16_swap(u, u, false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float pair_max32(float x) {
  const unsigned u = __float_as_uint(x);
  const auto r = __builtin_amdgcn_permlane32_swap(u, u, false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float pair_sum16(float x) {
  const unsigned u = __float_as_uint(x);
  const auto r = __builtin_amdgcn_permlane16_swap(u, u, false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}
__device__ __forceinline__ float pair_sum32(float x) {
  const unsigned u = __float_as_uint(x);
  const auto r = __builtin_amdgcn_permlane32_swap(u, u, false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}
__device__ __forceinline__ float quad_max(float x) { return pair_max32(pair_max16(x)); }
__device__ __forceinline__ float quad_sum(float x) { return pair_sum32(pair_sum16(x)); }

constexpr float kLazy = 8.f;  // largest allowed growth of a row maximum before the O rescale

// Workgroup = NW x KG wavefronts: wave w takes row tile w % NW and key group w / NW.
// The workgroup walks its key split in rounds of KG chunks of 32 keys; in a round,
// key group kg computes on chunk kg, so KG independent online-softmax streams share
// every SIMD.  At the end the KG partial states (max, sum, O) of each row tile merge
// in LDS, pairwise in a fixed tree order.
// Ragged contexts: the workgroups of one kv head are dispatched to one XCD in slot order
// and spread over its CUs breadth first, so a CU holds slots c and c + B/2.  Slot i of
// the first half takes the sequence of rank i by context length (longest first, ties by
// index), slot i of the second half rank 3B/2 - 1 - i: each CU pairs a long context with
// a short one.  A permutation of the sequences, so results do not depend on it.
// The context lengths go through LDS once; the host enables this for B <= kMaxBalanceBatch.
__device__ __forceinline__ int balanced_sequence(const AttnArgs& a, int slot) {
  __shared__ int seq_s;
  __shared__ int len_s[kMaxBalanceBatch];
  const int B = a.batch, half = (B + 1) / 2;
  const int want = slot < half ? slot : (B - 1) - (slot - half);
  for (int t = threadIdx.x; t < B; t += blockDim.x) len_s[t] = a.ctx_len[t];
  __syncthreads();
  for (int t = threadIdx.x; t < B; t += blockDim.x) {
    const int lt = len_s[t];
    int rank = 0;
    for (int s = 0; s < B; ++s) {
      const int ls = len_s[s];
      rank += (ls > lt || (ls == lt && s < t)) ? 1 : 0;
    }
    if (rank == want) seq_s = t;
  }
  __syncthreads();
  return seq_s;
}

// LDS of one attention workgroup.
template <typename T, int DH, int NW, int KG>
struct AttnLds {
  static constexpr int VS = DH + VPad<T>::value;
  static constexpr int XH = KG > 1 ? KG / 2 : 1;  // merge slots
  __attribute__((aligned(16))) T kv[KG][2][kKC][VS];  // [chunk of the round][K, V][key][dim]
  float xm[XH][NW][64], xl[XH][NW][64];
};

// 4 fp16 values (8 bytes) or 4 floats of one output row.
template <bool COH, typename T>
__device__ __forceinline__ void put4(T* dst, float a, float b, float c, float d) {
  if constexpr (COH && sizeof(T) == 2) {
    typedef T T4 __attribute__((ext_vector_type(4)));
    T4 v;
    v[0] = from_f32<T>(a);
    v[1] = from_f32<T>(b);
    v[2] = from_f32<T>(c);
    v[3] = from_f32<T>(d);
    __hip_atomic_store(reinterpret_cast<unsigned long long*>(dst), __builtin_bit_cast(unsigned long long, v),
                       __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  } else if constexpr (COH) {
    coherent_store16(dst, make_float4(a, b, c, d));
  } else {
    dst[0] = from_f32<T>(a);
    dst[1] = from_f32<T>(b);
    dst[2] = from_f32<T>(c);
    dst[3] = from_f32<T>(d);
  }
}

// One workgroup's work item (the kernel's blockIdx.x).  COH: q, the block's K/V rows
// and the outputs are read / written device-coherently (producer and consumer inside
// one launch).
template <typename T, int DH, int NW, int KG, bool COH>
__device__ __forceinline__ void attention_body(const AttnArgs& a, int item, AttnLds<T, DH, NW, KG>& lds) {
  constexpr int KS = DH / 32;  // MFMA reduction steps over the head dimension (S^T)
  constexpr int DT = DH / 16;  // 16-dim output tiles (O^T)
  constexpr int VS = DH + VPad<T>::value;
  constexpr int NT = 64 * NW * KG;
  constexpr int VPR = DH * static_cast<int>(sizeof(T)) / 16;  // 16-byte pieces per row
  constexpr int HALF = kKC * VPR;                             // pieces of K (or V) per chunk
  constexpr int PIECES = 2 * HALF * KG;                       // pieces per round
  constexpr int PPL = (PIECES + NT - 1) / NT;                 // pieces per thread per round
  constexpr int XH = KG > 1 ? KG / 2 : 1;                     // merge slots
  auto& kv = lds.kv;
  auto& xm = lds.xm;
  auto& xl = lds.xl;
  static_assert(KG == 1 || XH * NW * DT * 4 * 64 * sizeof(float) <= sizeof(lds.kv), "merge buffer");

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // uniform per wavefront
  const int rt = wave % NW, kg = wave / NW;                   // row tile, key group
  const int q4 = lane >> 4, l16 = lane & 15;
  const int split = item % a.max_splits;
  item /= a.max_splits;
  const int rb = item % a.n_rb;
  item /= a.n_rb;
  const int g = item % a.n_kv_heads;
  const int b = a.balance ? balanced_sequence(a, item / a.n_kv_heads) : item / a.n_kv_heads;
  const int k = a.block_k, G = a.n_q_heads / a.n_kv_heads;
  const int rr0 = rt * 16;                   // this wavefront's rows within the row block
  const int r0 = rb * a.rows_per_block;      // first row of the row block
  const int nr = min(a.rows_per_block, G * k - r0);  // rows of the row block
  const T* qg = static_cast<const T*>(a.q);
  // first row of sequence b in q, kb, vb and out (compacted blocks: only its live rows)
  const int rowb = a.seq_row0 != nullptr ? a.seq_row0[b] : b * k;

  // Q^T fragments (B operand), resident for the whole key loop: row rr0 + l16.  Their
  // loads do not depend on the context length, so they go out first.
  Frag<T> qf[KS];
  {
    const int rr = rr0 + l16;
    const int r = r0 + (rr < nr ? rr : 0);
    const T* qrow = qg + ((static_cast<size_t>(rowb) + r % k) * a.n_q_heads + g * G + r / k) * DH;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      if constexpr (COH) qf[ks].v = coherent_load16<decltype(qf[ks].v)>(qrow + ks * 32 + 8 * q4);
      else qf[ks].load(qrow + ks * 32 + 8 * q4);
    }
  }

  // key list: the sink positions 0..n_sink-1, the window positions ws..P-1, the
  // sequence's kb block rows
  const int P = max(a.ctx_len[b], 0);
  const int n_sink = min(a.sink, P);
  const int ws = max(n_sink, P - a.window);
  const int n_ctx = n_sink + (P - ws);
  const int kb = a.block_len != nullptr ? min(max(a.block_len[b], 0), k) : k;
  const int n_keys = n_ctx + kb;
  const int n_split_b = (n_keys + a.keys_per_split - 1) / a.keys_per_split;
  if (split >= n_split_b) return;  // uniform per workgroup
  const int j0 = split * a.keys_per_split;
  const int j1 = min(n_keys, j0 + a.keys_per_split);
  const T* kbg = static_cast<const T*>(a.kb);
  const T* vbg = static_cast<const T*>(a.vb);
  const size_t seq_base = (static_cast<size_t>(b) * a.n_kv_heads + g) * a.cache_slots;
  const T* ck = static_cast<const T*>(a.cache_k) + seq_base * DH;
  const T* cv = static_cast<const T*>(a.cache_v) + seq_base * DH;
  // slots: sink position p in slot p; later positions p in slot s + (p - s) mod R
  const int sk = a.sink, R = a.cache_slots - a.sink;
  const int wrel0 = P > sk ? (ws - sk) % R : 0;  // ring offset of the first window position
  const int blk_stride = a.n_kv_heads * DH;
  const T* kblk = kbg + (static_cast<size_t>(rowb) * a.n_kv_heads + g) * DH;
  const T* vblk = vbg + (static_cast<size_t>(rowb) * a.n_kv_heads + g) * DH;
  // key j's row: sink slot j, ring slot of window key j, or block row j - n_ctx;
  // selects only (no branch), so the unrolled loads stay in flight together
  auto key_ptr = [&](int j, const T* ring, const T* blk) -> const T* {
    const int t = max(wrel0 + j - n_sink, 0);  // window keys: < 2R
    const int sl = j < n_sink ? j : sk + (t >= R ? t - R : t);
    const uintptr_t pr = reinterpret_cast<uintptr_t>(ring + sl * DH);
    const uintptr_t pb = reinterpret_cast<uintptr_t>(blk + max(j - n_ctx, 0) * blk_stride);
    const uintptr_t m = uintptr_t(0) - static_cast<uintptr_t>(j < n_ctx);
    return reinterpret_cast<const T*>((pr & m) | (pb & ~m));
  };

  // scores in log2 units: softmax(s / sqrt(dh)) = 2^(s * log2(e) / sqrt(dh) - max)
  const float scale2 = 1.4426950408889634f / sqrtf(static_cast<float>(DH));
  f32x4 o[DT];  // O^T: lane holds dims dt*16 + 4*q4 + r of row rr0 + l16
#pragma unroll
  for (int dt = 0; dt < DT; ++dt) o[dt] = f32x4{0.f, 0.f, 0.f, 0.f};
  float m_run = -INFINITY, l_run = 0.f;

  // cooperative round load: piece p covers chunk p / (2 HALF) of the round, K if
  // (p / HALF) is even, else V, key (p % HALF) / VPR, 16-byte piece p % VPR of that
  // row.  Past j1 (and past the last piece) valid rows are re-loaded, and the stores
  // of pieces past the last are skipped.  The next round's loads are in flight while
  // this round is computed.
  f32x4 st[PPL];
  auto load = [&](int c0) {
#pragma unroll
    for (int i = 0; i < PPL; ++i) {
      const int p = min(tid + NT * i, PIECES - 1);
      const int cg = p / (2 * HALF), h = (p / HALF) % 2, pp = p % HALF;
      const int j = min(c0 + cg * kKC + pp / VPR, j1 - 1);
      const T* row = h == 0 ? key_ptr(j, ck, kblk) : key_ptr(j, cv, vblk);
      st[i] = get16<COH, f32x4>(reinterpret_cast<const f32x4*>(row) + pp % VPR);
    }
  };
  auto store = [&]() {
#pragma unroll
    for (int i = 0; i < PPL; ++i) {
      const int p = tid + NT * i;
      if (PIECES % NT == 0 || p < PIECES) {
        const int cg = p / (2 * HALF), h = (p / HALF) % 2, pp = p % HALF;
        reinterpret_cast<f32x4*>(&kv[cg][h][pp / VPR][0])[pp % VPR] = st[i];
      }
    }
  };
  // keys c .. c + 31 from this key group's chunk of the round
  auto chunk = [&](int c) {
    // S^T = K Q^T from the chunk's K rows
    f32x4 s[2];
#pragma unroll
    for (int kt = 0; kt < 2; ++kt) {
      s[kt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        Frag<T> kf;
        kf.load(&kv[kg][0][kt * 16 + l16][ks * 32 + 8 * q4]);
        Frag<T>::mma(s[kt], kf, qf[ks]);
      }
    }
    // online softmax of row rr0 + l16 over this lane's 8 keys and its 3 partner lanes
    float x[2][4];
#pragma unroll
    for (int kt = 0; kt < 2; ++kt)
#pragma unroll
      for (int r = 0; r < 4; ++r) x[kt][r] = s[kt][r] * scale2;
    if (c + kKC > j1) {
#pragma unroll
      for (int kt = 0; kt < 2; ++kt)
#pragma unroll
        for (int r = 0; r < 4; ++r)
          if (c + kt * 16 + 4 * q4 + r >= j1) x[kt][r] = -INFINITY;
    }
    float mx = -INFINITY;
#pragma unroll
    for (int kt = 0; kt < 2; ++kt)
#pragma unroll
      for (int r = 0; r < 4; ++r) mx = fmaxf(mx, x[kt][r]);
    mx = quad_max(mx);  // finite: key c < j1 is valid for every row
    // lazy reference: the running maximum moves only when a score passes it by more
    // than kLazy (log2 units), so p <= 2^kLazy and most chunks skip the O rescale; the
    // softmax is unchanged since numerator and denominator share the reference
    const float m_new = mx > m_run + kLazy ? mx : m_run;  // m_run = -inf on the first chunk
    const float corr = __builtin_amdgcn_exp2f(m_run - m_new);  // 0 on the first chunk
    Frag<T> pf;
    float ps = 0.f;
#pragma unroll
    for (int kt = 0; kt < 2; ++kt)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const float p = __builtin_amdgcn_exp2f(x[kt][r] - m_new);
        ps += p;
        pf.v[4 * kt + r] = from_f32<T>(p);
      }
    ps = quad_sum(ps);
    l_run = l_run * corr + ps;
    m_run = m_new;
    if (__any(corr != 1.f)) {
#pragma unroll
      for (int dt = 0; dt < DT; ++dt) o[dt] *= corr;
    }
    // O^T += V^T P^T; V^T operand: dim dt*16 + l16, keys {4*q4 + t, 16 + 4*q4 + t}
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) {
      Frag<T> vf;
      if constexpr (sizeof(T) == 2) {
        // transposing LDS reads: in each 16-lane group, result lane i, slot j takes
        // element i % 4 of the 8 bytes source lane 4j + i/4 points at, so lane (q4, m)
        // points at row 4*q4 + m/4 (then + 16), dims dt*16 + 4*(m % 4)
        typedef __fp16 h4 __attribute__((__vector_size__(4 * sizeof(__fp16))));
        const h4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4f16(
            (__attribute__((address_space(3))) h4*)&kv[kg][1][4 * q4 + (l16 >> 2)][dt * 16 + 4 * (l16 & 3)]);
        const h4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4f16(
            (__attribute__((address_space(3))) h4*)&kv[kg][1][16 + 4 * q4 + (l16 >> 2)][dt * 16 + 4 * (l16 & 3)]);
#pragma unroll
        for (int t = 0; t < 4; ++t) {
          vf.v[t] = static_cast<T>(lo[t]);
          vf.v[4 + t] = static_cast<T>(hi[t]);
        }
      } else {
#pragma unroll
        for (int t = 0; t < 8; ++t) vf.v[t] = kv[kg][1][(t < 4 ? 0 : 12) + 4 * q4 + t][dt * 16 + l16];
      }
      Frag<T>::mma(o[dt], vf, pf);
    }
  };

  const int n_rounds = (j1 - j0 + KG * kKC - 1) / (KG * kKC);
  load(j0);
  for (int r = 0; r < n_rounds; ++r) {
    const int c0 = j0 + r * KG * kKC;
    if (r > 0) __syncthreads();  // the previous round's chunks are no longer read
    store();
    __syncthreads();  // this round's rows are visible
    if (r + 1 < n_rounds) load(c0 + KG * kKC);  // uniform per workgroup
    const int c = c0 + kg * kKC;
    if (c < j1) chunk(c);  // uniform per wavefront
  }

  if constexpr (KG > 1) {
    // merge the key groups of each row tile: in step `half`, groups half .. 2 half - 1
    // hand their state to groups 0 .. half - 1 through LDS (kv is free by then)
    float* xo = reinterpret_cast<float*>(&kv[0][0][0][0]);  // [XH][NW][DT * 4][64]
#pragma unroll
    for (int half = KG / 2; half >= 1; half /= 2) {
      __syncthreads();
      if (kg >= half && kg < 2 * half) {
        const int sl = kg - half;
        float* dst = xo + ((sl * NW + rt) * DT * 4) * 64 + lane;
#pragma unroll
        for (int dt = 0; dt < DT; ++dt)
#pragma unroll
          for (int j = 0; j < 4; ++j) dst[(dt * 4 + j) * 64] = o[dt][j];
        xm[sl][rt][lane] = m_run;
        xl[sl][rt][lane] = l_run;
      }
      __syncthreads();
      if (kg < half) {
        const float mo = xm[kg][rt][lane], lo = xl[kg][rt][lane];
        const float mn = fmaxf(m_run, mo);
        // a group without keys has m = -inf, l = 0, O = 0
        const float ca = m_run == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(m_run - mn);
        const float cb = mo == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(mo - mn);
        const float* src = xo + ((kg * NW + rt) * DT * 4) * 64 + lane;
#pragma unroll
        for (int dt = 0; dt < DT; ++dt)
#pragma unroll
          for (int j = 0; j < 4; ++j) o[dt][j] = o[dt][j] * ca + src[(dt * 4 + j) * 64] * cb;
        l_run = l_run * ca + lo * cb;
        m_run = mn;
      }
    }
  }
  if (kg != 0) return;

  // output: lane -> row rr0 + l16, dims dt*16 + 4*q4 .. +3
  const int rr = rr0 + l16;
  if (rr >= nr) return;
  const size_t grp = (static_cast<size_t>(b) * a.n_kv_heads + g) * a.n_rb + rb;
  const int r = r0 + rr, hl = r / k, i = r % k;
  if (n_split_b == 1) {
    if (a.seq_row0 != nullptr && i >= kb) return;  // compacted: the row does not exist
    T* out = static_cast<T*>(a.out);
    const float inv = 1.f / l_run;
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) {
      T* dst = out + pa_index(rowb + i, (g * G + hl) * DH + dt * 16 + 4 * q4, a.out_steps);
      put4<COH>(dst, o[dt][0] * inv, o[dt][1] * inv, o[dt][2] * inv, o[dt][3] * inv);
    }
  } else {
    float* po = a.part_o + ((grp * a.max_splits + split) * kRows + rr) * DH;
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) put16<COH>(po + dt * 16 + 4 * q4, make_float4(o[dt][0], o[dt][1], o[dt][2], o[dt][3]));
    if (q4 == 0) {
      float* pml = a.part_ml + ((grp * a.max_splits + split) * kRows + rr) * 2;
      put<COH>(pml, m_run);
      put<COH>(pml + 1, l_run);
    }
  }
}

// Merge of the key splits of every (sequence, kv head, row block) whose keys were
// split; sequences with one split were finished by the attention kernel itself.
// Thread t of a workgroup takes 4 head dims ((t % (DH/4)) * 4) of row
// (t / (DH/4)) / NSUB of the workgroup's rows, and the splits s = (t / (DH/4)) % NSUB
// (mod NSUB).  Each thread loads SPT of its splits at once (the first SPT before the
// sequence's split count is known: the partial buffers hold max_splits entries, and
// entries past the count are selected away), folds them into its own (max, sum, O) with the usual
// rescaling, and the NSUB subsets combine in a fixed order, so the result does not
// depend on scheduling.
template <int DH, int NSUB>
struct MergeLds {
  static constexpr int TPR = DH / 4, RPW = kThreads / (TPR * NSUB);
  float red_m[RPW][NSUB];
  float4 red_o[RPW][NSUB][TPR];
  float red_l[RPW][NSUB];
};

template <typename T, int DH, int NSUB, bool COH>
__device__ __forceinline__ void merge_body(const AttnArgs& a, int item, MergeLds<DH, NSUB>& lds) {
  constexpr int TPR = DH / 4, RPW = kThreads / (TPR * NSUB);  // threads per row-subset, rows per workgroup
  constexpr int SPT = 8;                                      // splits per thread in flight
  auto& red_m = lds.red_m;
  auto& red_o = lds.red_o;
  auto& red_l = lds.red_l;
  const int rows = a.rows_per_block;
  const int wg_per_grp = (rows + RPW - 1) / RPW;
  const int grp_i = item / wg_per_grp;
  const int rb = grp_i % a.n_rb, g = (grp_i / a.n_rb) % a.n_kv_heads, b = grp_i / (a.n_rb * a.n_kv_heads);
  const int k = a.block_k, G = a.n_q_heads / a.n_kv_heads;
  const int t = threadIdx.x, dq = t % TPR, sub = (t / TPR) % NSUB, rw = t / (TPR * NSUB);
  const int r0 = rb * rows;
  const int rr = (item % wg_per_grp) * RPW + rw;
  const bool valid = rr < min(rows, G * k - r0);
  const int rrc = valid ? rr : 0;
  const size_t grp = (static_cast<size_t>(b) * a.n_kv_heads + g) * a.n_rb + rb;
  const float* ml_base = a.part_ml + (grp * a.max_splits * kRows + rrc) * 2;
  const float* o_base = a.part_o + (grp * a.max_splits * kRows + rrc) * DH + 4 * dq;
  float m_loc = -INFINITY, l_loc = 0.f;
  float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
  float2 ml[SPT];
  float4 ov[SPT];
  auto fetch = [&](int s0) {  // this thread's splits s0, s0 + NSUB, ... (clamped into the buffers)
#pragma unroll
    for (int i = 0; i < SPT; ++i) {
      const int s = min(s0 + NSUB * i, a.max_splits - 1);
      if constexpr (COH) ml[i] = coherent_load2(ml_base + static_cast<size_t>(s) * kRows * 2);
      else ml[i] = *reinterpret_cast<const float2*>(ml_base + static_cast<size_t>(s) * kRows * 2);
      ov[i] = get16<COH, float4>(o_base + static_cast<size_t>(s) * kRows * DH);
    }
  };
  // folds the fetched splits below n_split_b into (m_loc, l_loc, acc); selects, not
  // branches, so that every fetch load stays unconditional and in flight
  auto fold = [&](int s0, int n_split_b) {
    float mv[SPT];
    float m_new = m_loc;
#pragma unroll
    for (int i = 0; i < SPT; ++i) {
      mv[i] = s0 + NSUB * i < n_split_b ? ml[i].x : -INFINITY;
      m_new = fmaxf(m_new, mv[i]);
    }
    const bool any = m_new != -INFINITY;  // split maxima are finite
    const float corr = any ? __builtin_amdgcn_exp2f(m_loc - m_new) : 1.f;  // log2 units
    l_loc *= corr;
    acc.x *= corr;
    acc.y *= corr;
    acc.z *= corr;
    acc.w *= corr;
#pragma unroll
    for (int i = 0; i < SPT; ++i) {
      const bool ok = mv[i] != -INFINITY;
      const float w = ok ? __builtin_amdgcn_exp2f(mv[i] - m_new) : 0.f;
      const float4 v = ok ? ov[i] : make_float4(0.f, 0.f, 0.f, 0.f);
      l_loc += (ok ? ml[i].y : 0.f) * w;
      acc.x += v.x * w;
      acc.y += v.y * w;
      acc.z += v.z * w;
      acc.w += v.w * w;
    }
    m_loc = m_new;
  };
  fetch(sub);
  asm volatile("" ::: "memory");  // the first loads go out before the context length is read
  const int P = max(a.ctx_len[b], 0);
  const int n_sink = min(a.sink, P);
  const int kb = a.block_len != nullptr ? min(max(a.block_len[b], 0), k) : k;
  const int n_keys = n_sink + (P - max(n_sink, P - a.window)) + kb;
  const int n_split_b = (n_keys + a.keys_per_split - 1) / a.keys_per_split;
  fold(sub, n_split_b);
  for (int s0 = sub + NSUB * SPT; s0 < n_split_b; s0 += NSUB * SPT) {  // more than NSUB * SPT splits
    fetch(s0);
    fold(s0, n_split_b);
  }
  if (n_split_b <= 1) return;  // uniform per workgroup (0: no keys, the rows lie outside any block)
  red_o[rw][sub][dq] = acc;
  if (dq == 0) {
    red_m[rw][sub] = m_loc;
    red_l[rw][sub] = l_loc;
  }
  __syncthreads();
  if (sub != 0 || !valid) return;
  float M = -INFINITY;
#pragma unroll
  for (int i = 0; i < NSUB; ++i) M = fmaxf(M, red_m[rw][i]);
  float4 o = make_float4(0.f, 0.f, 0.f, 0.f);
  float Lt = 0.f;
#pragma unroll
  for (int i = 0; i < NSUB; ++i) {
    const float mi = red_m[rw][i];
    if (mi == -INFINITY) continue;  // a subset without splits
    const float w = __builtin_amdgcn_exp2f(mi - M);
    const float4 v = red_o[rw][i][dq];
    o.x += v.x * w;
    o.y += v.y * w;
    o.z += v.z * w;
    o.w += v.w * w;
    Lt += red_l[rw][i] * w;
  }
  const int r = r0 + rr, hl = r / k, i = r % k;
  if (a.seq_row0 != nullptr && i >= kb) return;  // compacted: the row does not exist
  T* dst = static_cast<T*>(a.out) + pa_index((a.seq_row0 != nullptr ? a.seq_row0[b] : b * k) + i,
                                             (g * G + hl) * DH + 4 * dq, a.out_steps);
  const float inv = 1.f / Lt;
  put4<COH>(dst, o.x * inv, o.y * inv, o.z * inv, o.w * inv);
}

}  // namespace dflash
