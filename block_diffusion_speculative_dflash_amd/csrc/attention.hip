// Block attention on MFMA: every query row of the block attends to the last
// min(P, W) committed positions (the layer's K/V ring) and to all k block rows,
// with no causal mask inside the block (hotdry blog: one forward fills the whole
// masked block, all-SWA drafter with window W; zhihu answer §4: parallel decoding
// inside a block).
//
// Workgroup = (key split, kv head g, sequence b, row block).  Its query rows are
// the G = Hq/Hkv query heads of group g times the k block rows (up to 64, RT tiles
// of 16).  The four wavefronts take interleaved chunks of 32 keys; per chunk a
// wavefront computes S = Q K^T with 16x16x32 MFMA (K fragments load straight from
// the key rows), updates an online softmax (row max / sum across the 16 lanes that
// share a row), stages P and the chunk's V (transposed) in its own LDS, and adds
// P V with MFMA.  The four wavefronts' (max, sum, O) are merged in a fixed order.
// When one sequence's keys are split over several workgroups (long full-attention
// contexts at small batch), each writes its unnormalised partial and a second
// kernel merges them in split order; either way the result does not depend on
// scheduling.
#include "common.h"
#include "internal.h"

namespace dflash {

constexpr int kRows = 64;  // row stride of the split partials (RT <= 4 tiles of 16 per workgroup)
constexpr int kKC = 32;    // keys per wavefront chunk (one MFMA K step for P V)
constexpr int kPad = 8;    // LDS row padding (elements)

// lgkmcnt(0) only (gfx9 s_waitcnt encoding, vmcnt and expcnt left at their maxima):
// this wavefront's LDS writes are complete before its other lanes read them.
__device__ __forceinline__ void lds_written() {
  __builtin_amdgcn_s_waitcnt(0xC07F);
  __builtin_amdgcn_wave_barrier();
}

template <typename T, int DH, int RT>
struct __attribute__((aligned(16))) AttnSmem {
  union {
    struct {
      T vt[4][DH][kKC + kPad];      // per wavefront: V chunk transposed [dh][key]
      T p[4][RT * 16][kKC + kPad];  // per wavefront: probabilities [row][key]
    } loop;
    float o[RT * 16][DH + 4];       // merge of the four wavefronts
  } u;
  float ml[4][RT * 16][2];          // per wavefront (row max, row sum)
};

template <typename T, int DH, int RT>
__global__ __launch_bounds__(kThreads) void attention_kernel(AttnArgs a) {
  constexpr int KS = DH / 32;  // MFMA K steps over the head dimension (Q K^T)
  constexpr int DT = DH / 16;  // 16-wide output column tiles (P V)
  __shared__ AttnSmem<T, DH, RT> sm;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int split = blockIdx.x, g = blockIdx.y;
  const int b = blockIdx.z / a.n_rb, rb = blockIdx.z % a.n_rb;
  const int k = a.block_k, G = a.n_q_heads / a.n_kv_heads;
  const int P = max(a.ctx_len[b], 0);
  const int n_ctx = min(P, a.window);
  const int n_keys = n_ctx + k;
  const int n_split_b = (n_keys + a.keys_per_split - 1) / a.keys_per_split;
  if (split >= n_split_b) return;
  const int j0 = split * a.keys_per_split;
  const int j1 = min(n_keys, j0 + a.keys_per_split);
  const int r0 = rb * RT * 16;
  const int nr = min(RT * 16, G * k - r0);

  const T* qg = static_cast<const T*>(a.q);
  const T* kbg = static_cast<const T*>(a.kb);
  const T* vbg = static_cast<const T*>(a.vb);
  const size_t seq_base = (static_cast<size_t>(b) * a.n_kv_heads + g) * a.cache_slots;
  const T* ck = static_cast<const T*>(a.cache_k) + seq_base * DH;
  const T* cv = static_cast<const T*>(a.cache_v) + seq_base * DH;
  // row j of this sequence's key list: the window (ring slots), then the block
  auto key_row = [&](int j, const T* ring, const T* blk) -> const T* {
    if (j < n_ctx) return ring + static_cast<size_t>((P - n_ctx + j) % a.cache_slots) * DH;
    return blk + ((static_cast<size_t>(b) * k + (j - n_ctx)) * a.n_kv_heads + g) * DH;
  };

  // Q fragments, resident for the whole key loop: row rt*16 + lane%16
  Frag<T> qf[RT][KS];
#pragma unroll
  for (int rt = 0; rt < RT; ++rt) {
    const int rr = rt * 16 + (lane & 15);
    const bool ok = rr < nr;
    const int r = r0 + (ok ? rr : 0);
    const T* qrow = qg + ((static_cast<size_t>(b) * k + r % k) * a.n_q_heads + g * G + r / k) * DH;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      qf[rt][ks].load(qrow + ks * 32 + 8 * (lane >> 4));
      if (!ok) qf[rt][ks].zero();
    }
  }

  const float scale = 1.f / sqrtf(static_cast<float>(DH));
  f32x4 o[RT][DT];
  float m_run[RT][4], l_run[RT][4];
#pragma unroll
  for (int rt = 0; rt < RT; ++rt) {
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) o[rt][dt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int r = 0; r < 4; ++r) { m_run[rt][r] = -INFINITY; l_run[rt][r] = 0.f; }
  }

  T(*vt)[kKC + kPad] = sm.u.loop.vt[wave];
  T(*pp)[kKC + kPad] = sm.u.loop.p[wave];
  // K fragments of keys c + kt*16 + lane%16 and this lane's V slice (key c + lane/2,
  // half the head dim); past j1 a valid row is loaded and masked later.
  constexpr int VE = DH / 2 / 8;  // V fragments per lane
  Frag<T> kf[2][KS], vr[VE], kf_n[2][KS], vr_n[VE];
  auto load_chunk = [&](int c, Frag<T>(&kk)[2][KS], Frag<T>(&vv)[VE]) {
#pragma unroll
    for (int kt = 0; kt < 2; ++kt) {
      const T* krow = key_row(min(c + kt * 16 + (lane & 15), j1 - 1), ck, kbg);
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) kk[kt][ks].load(krow + ks * 32 + 8 * (lane >> 4));
    }
    const T* vrow = key_row(min(c + (lane >> 1), j1 - 1), cv, vbg) + (lane & 1) * (DH / 2);
#pragma unroll
    for (int e = 0; e < VE; ++e) vv[e].load(vrow + 8 * e);
  };
  int c0 = j0 + wave * kKC;
  if (c0 < j1) load_chunk(c0, kf, vr);
  for (; c0 < j1; c0 += 4 * kKC) {
    const int cn = c0 + 4 * kKC;
    if (cn < j1) load_chunk(cn, kf_n, vr_n);  // next chunk in flight during this one
    // V chunk -> LDS, transposed: [dh][key]
    {
      const int jj = lane >> 1, h0 = (lane & 1) * (DH / 2);
      const bool ok = c0 + jj < j1;
#pragma unroll
      for (int e = 0; e < VE; ++e)
#pragma unroll
        for (int i = 0; i < 8; ++i) vt[h0 + 8 * e + i][jj] = ok ? vr[e].v[i] : from_f32<T>(0.f);
    }
    // S = Q K^T, scaled, masked
    f32x4 s[RT][2];
#pragma unroll
    for (int rt = 0; rt < RT; ++rt)
#pragma unroll
      for (int kt = 0; kt < 2; ++kt) {
        s[rt][kt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) Frag<T>::mma(s[rt][kt], qf[rt][ks], kf[kt][ks]);
      }
    const bool kv0 = c0 + (lane & 15) < j1, kv1 = c0 + 16 + (lane & 15) < j1;
    // online softmax; this lane holds rows rt*16 + 4*(lane/16) + r, key column lane%16
#pragma unroll
    for (int rt = 0; rt < RT; ++rt)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const float x0 = kv0 ? s[rt][0][r] * scale : -INFINITY;
        const float x1 = kv1 ? s[rt][1][r] * scale : -INFINITY;
        float mx = fmaxf(x0, x1);
#pragma unroll
        for (int off = 1; off < 16; off <<= 1) mx = fmaxf(mx, __shfl_xor(mx, off, kWave));
        const float m_new = fmaxf(m_run[rt][r], mx);
        const float corr = expf(m_run[rt][r] - m_new);  // 0 on the first chunk
        const float p0 = expf(x0 - m_new), p1 = expf(x1 - m_new);
        float ps = p0 + p1;
#pragma unroll
        for (int off = 1; off < 16; off <<= 1) ps += __shfl_xor(ps, off, kWave);
        l_run[rt][r] = l_run[rt][r] * corr + ps;
        m_run[rt][r] = m_new;
#pragma unroll
        for (int dt = 0; dt < DT; ++dt) o[rt][dt][r] *= corr;
        const int row = rt * 16 + 4 * (lane >> 4) + r;
        pp[row][lane & 15] = from_f32<T>(p0);
        pp[row][16 + (lane & 15)] = from_f32<T>(p1);
      }
    lds_written();
    // O += P V: A = P rows (lane%16), keys 8*(lane/16)..; B = V^T dims (lane%16)
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) {
      Frag<T> vf;
      vf.load(&vt[dt * 16 + (lane & 15)][8 * (lane >> 4)]);
#pragma unroll
      for (int rt = 0; rt < RT; ++rt) {
        Frag<T> pf;
        pf.load(&pp[rt * 16 + (lane & 15)][8 * (lane >> 4)]);
        Frag<T>::mma(o[rt][dt], pf, vf);
      }
    }
    lds_written();
#pragma unroll
    for (int kt = 0; kt < 2; ++kt)
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) kf[kt][ks] = kf_n[kt][ks];
#pragma unroll
    for (int e = 0; e < VE; ++e) vr[e] = vr_n[e];
  }

  // merge the four wavefronts: global row max M, weights exp(m_w - M)
  if ((lane & 15) == 0) {
#pragma unroll
    for (int rt = 0; rt < RT; ++rt)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int row = rt * 16 + 4 * (lane >> 4) + r;
        sm.ml[wave][row][0] = m_run[rt][r];
        sm.ml[wave][row][1] = l_run[rt][r];
      }
  }
  __syncthreads();
  float wf[RT][4];
#pragma unroll
  for (int rt = 0; rt < RT; ++rt)
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int row = rt * 16 + 4 * (lane >> 4) + r;
      float M = -INFINITY;
      for (int w = 0; w < 4; ++w) M = fmaxf(M, sm.ml[w][row][0]);
      wf[rt][r] = m_run[rt][r] == -INFINITY ? 0.f : expf(m_run[rt][r] - M);
    }
  for (int w = 0; w < 4; ++w) {
    if (wave == w) {
#pragma unroll
      for (int rt = 0; rt < RT; ++rt)
#pragma unroll
        for (int dt = 0; dt < DT; ++dt)
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const int row = rt * 16 + 4 * (lane >> 4) + r, col = dt * 16 + (lane & 15);
            const float v = o[rt][dt][r] * wf[rt][r];
            sm.u.o[row][col] = (w == 0 ? 0.f : sm.u.o[row][col]) + v;
          }
    }
    __syncthreads();
  }

  // rows: thread -> row tid/4, a quarter of the head dimension
  const int rr = tid >> 2, qd = tid & 3;
  constexpr int DQ = DH / 4;
  if (rr >= nr) return;
  float M = -INFINITY, L = 0.f;
  for (int w = 0; w < 4; ++w) M = fmaxf(M, sm.ml[w][rr][0]);
  for (int w = 0; w < 4; ++w) {
    const float mw = sm.ml[w][rr][0];
    if (mw != -INFINITY) L += sm.ml[w][rr][1] * expf(mw - M);
  }
  const int r = r0 + rr, hl = r / k, i = r % k;
  if (n_split_b == 1) {
    T* out = static_cast<T*>(a.out);
    const int m = b * k + i;
    const int col0 = (g * G + hl) * DH + qd * DQ;
    const float inv = 1.f / L;
#pragma unroll
    for (int c = 0; c < DQ; c += 8) {
      T* dst = out + pa_index(m, col0 + c, a.out_steps);
#pragma unroll
      for (int j = 0; j < 8; ++j) dst[j] = from_f32<T>(sm.u.o[rr][qd * DQ + c + j] * inv);
    }
  } else {
    const size_t grp = (static_cast<size_t>(b) * a.n_kv_heads + g) * a.n_rb + rb;
    float* po = a.part_o + ((grp * a.max_splits + split) * kRows + rr) * DH + qd * DQ;
#pragma unroll
    for (int d = 0; d < DQ; ++d) po[d] = sm.u.o[rr][qd * DQ + d];
    if (qd == 0) {
      float* pml = a.part_ml + ((grp * a.max_splits + split) * kRows + rr) * 2;
      pml[0] = M;
      pml[1] = L;
    }
  }
}

// Merge of the key splits of every (sequence, kv head, row block) whose keys were
// split, in split order; sequences with one split were finished by the attention
// kernel itself.
template <typename T, int DH>
__global__ __launch_bounds__(kThreads) void attention_merge_kernel(AttnArgs a) {
  // blockIdx.x picks 32 head dims; thread -> row tid/4, 8 of those dims
  const int g = blockIdx.y, b = blockIdx.z / a.n_rb, rb = blockIdx.z % a.n_rb;
  const int k = a.block_k, G = a.n_q_heads / a.n_kv_heads;
  const int P = max(a.ctx_len[b], 0);
  const int n_keys = min(P, a.window) + k;
  const int n_split_b = (n_keys + a.keys_per_split - 1) / a.keys_per_split;
  if (n_split_b == 1) return;
  const int rr = threadIdx.x >> 2;
  const int d0 = blockIdx.x * 32 + (threadIdx.x & 3) * 8;
  const int rows = a.rows_per_block;
  const int r0 = rb * rows;
  if (rr >= min(rows, G * k - r0)) return;
  const size_t grp = (static_cast<size_t>(b) * a.n_kv_heads + g) * a.n_rb + rb;
  float M = -INFINITY;
  for (int s = 0; s < n_split_b; ++s) M = fmaxf(M, a.part_ml[((grp * a.max_splits + s) * kRows + rr) * 2]);
  float acc[8];
#pragma unroll
  for (int d = 0; d < 8; ++d) acc[d] = 0.f;
  float L = 0.f;
  for (int s = 0; s < n_split_b; ++s) {
    const float* pml = a.part_ml + ((grp * a.max_splits + s) * kRows + rr) * 2;
    const float w = expf(pml[0] - M);
    L += pml[1] * w;
    const float* po = a.part_o + ((grp * a.max_splits + s) * kRows + rr) * DH + d0;
#pragma unroll
    for (int d = 0; d < 8; ++d) acc[d] += po[d] * w;
  }
  const int r = r0 + rr, hl = r / k, i = r % k;
  T* dst = static_cast<T*>(a.out) + pa_index(b * k + i, (g * G + hl) * DH + d0, a.out_steps);
  const float inv = 1.f / L;
#pragma unroll
  for (int j = 0; j < 8; ++j) dst[j] = from_f32<T>(acc[j] * inv);
}

template <typename T, int DH, int RT>
static void launch_rt(const AttnArgs& a, hipStream_t s) {
  const dim3 grid(a.max_splits, a.n_kv_heads, a.batch * a.n_rb);
  hipLaunchKernelGGL((attention_kernel<T, DH, RT>), grid, dim3(kThreads), 0, s, a);
}

template <typename T, int DH>
static hipError_t launch_dh(const AttnArgs& a, hipStream_t s) {
  switch (a.rows_per_block / 16) {
    case 1: launch_rt<T, DH, 1>(a, s); break;
    case 2: launch_rt<T, DH, 2>(a, s); break;
    case 3: launch_rt<T, DH, 3>(a, s); break;
    default: launch_rt<T, DH, 4>(a, s); break;
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || a.max_splits == 1) return e;
  const dim3 grid(DH / 32, a.n_kv_heads, a.batch * a.n_rb);
  hipLaunchKernelGGL((attention_merge_kernel<T, DH>), grid, dim3(kThreads), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_attention(bool f32, const AttnArgs& a, hipStream_t stream) {
  if (a.head_dim == 128) return f32 ? launch_dh<float, 128>(a, stream) : launch_dh<f16, 128>(a, stream);
  if (a.head_dim == 64) return f32 ? launch_dh<float, 64>(a, stream) : launch_dh<f16, 64>(a, stream);
  return hipErrorInvalidValue;
}

}  // namespace dflash
