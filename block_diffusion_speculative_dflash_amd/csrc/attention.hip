// Block attention on MFMA: every query row of the block attends to the last
// min(P, W) committed positions (the layer's K/V ring) and to all k block rows,
// with no causal mask inside the block (hotdry blog: one forward fills the whole
// masked block, all-SWA drafter with window W; zhihu answer §4: parallel decoding
// inside a block).
//
// Work item = one wavefront = (sequence b, kv head g, row block, key split).  The
// rows of kv head g are its G = Hq/Hkv query heads times the k block rows; a row
// block is up to RT tiles of 16 of them.  The four wavefronts of a workgroup are
// independent items; there is no workgroup barrier.
//
// Everything is computed transposed so that one query row lives in one lane:
//   S^T = K Q^T     A = 16 keys x 32 head dims (straight from the key rows),
//                   B = Q^T; lane l gets the scores of row l%16 for keys 4*(l/16)+r
//   softmax         running max / sum per lane; across keys: in-lane, then the four
//                   lanes of a row (xor 16, 32)
//   O^T += V^T P^T  B = P^T straight from the score registers: its 32 reduction
//                   slots are keys {4q..4q+3, 16+4q..16+4q+3} for lane group q, and
//                   A = V^T uses the same key order, gathered from the chunk's V rows
//                   staged in this wavefront's LDS
// so the row statistics scale the output accumulators without any data exchange.
// When one sequence's keys are split over several items (long full-attention
// contexts at small batch), each writes its unnormalised partial and a second kernel
// merges them in split order; either way the result does not depend on scheduling.
#include "common.h"
#include "internal.h"

namespace dflash {

constexpr int kRows = 64;  // row stride of the split partials
constexpr int kKC = 32;    // keys per chunk (one MFMA reduction step of P V)

template <typename T> struct VPad;
template <> struct VPad<f16> { static constexpr int value = 8; };    // 16-byte rows
template <> struct VPad<float> { static constexpr int value = 4; };  // 16-byte rows

// lgkmcnt(0) only (gfx9 s_waitcnt encoding, vmcnt and expcnt left at their maxima):
// this wavefront's LDS writes are complete before its other lanes read them.
__device__ __forceinline__ void lds_written() {
  __builtin_amdgcn_s_waitcnt(0xC07F);
  __builtin_amdgcn_wave_barrier();
}

template <typename T, int DH, int RT>
__global__ __launch_bounds__(kThreads, 2) void attention_kernel(AttnArgs a) {
  constexpr int KS = DH / 32;  // MFMA reduction steps over the head dimension (S^T)
  constexpr int DT = DH / 16;  // 16-dim output tiles (O^T)
  constexpr int VS = DH + VPad<T>::value;
  __shared__ __attribute__((aligned(16))) T vl[4][kKC][VS];

  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int q4 = lane >> 4, l16 = lane & 15;
  int item = blockIdx.x * 4 + wave;
  const int split = item % a.max_splits;
  item /= a.max_splits;
  const int rb = item % a.n_rb;
  item /= a.n_rb;
  const int g = item % a.n_kv_heads, b = item / a.n_kv_heads;
  if (b >= a.batch) return;
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
  const int C = a.cache_slots;
  const int slot0 = (P - n_ctx) % C;  // ring slot of key 0 (n_ctx < C)
  const int blk_stride = a.n_kv_heads * DH;
  const T* kblk = kbg + (static_cast<size_t>(b) * k * a.n_kv_heads + g) * DH;
  const T* vblk = vbg + (static_cast<size_t>(b) * k * a.n_kv_heads + g) * DH;
  // key j's row: ring slot slot0 + j (mod C) of the window, then block row j - n_ctx;
  // selects only (no branch), so the unrolled loads stay in flight together
  auto key_ptr = [&](int j, const T* ring, const T* blk) -> const T* {
    const int sl = slot0 + j;
    const uintptr_t pr = reinterpret_cast<uintptr_t>(ring + (sl >= C ? sl - C : sl) * DH);
    const uintptr_t pb = reinterpret_cast<uintptr_t>(blk + (j - n_ctx) * blk_stride);
    const uintptr_t m = uintptr_t(0) - static_cast<uintptr_t>(j < n_ctx);
    return reinterpret_cast<const T*>((pr & m) | (pb & ~m));
  };

  // Q^T fragments (B operand), resident for the whole key loop: row rt*16 + l16
  Frag<T> qf[RT][KS];
#pragma unroll
  for (int rt = 0; rt < RT; ++rt) {
    const int rr = rt * 16 + l16;
    const int r = r0 + (rr < nr ? rr : 0);
    const T* qrow = qg + ((static_cast<size_t>(b) * k + r % k) * a.n_q_heads + g * G + r / k) * DH;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) qf[rt][ks].load(qrow + ks * 32 + 8 * q4);
  }

  const float scale = 1.f / sqrtf(static_cast<float>(DH));
  f32x4 o[RT][DT];  // O^T: lane holds dims dt*16 + 4*q4 + r of row rt*16 + l16
  float m_run[RT], l_run[RT];
#pragma unroll
  for (int rt = 0; rt < RT; ++rt) {
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) o[rt][dt] = f32x4{0.f, 0.f, 0.f, 0.f};
    m_run[rt] = -INFINITY;
    l_run[rt] = 0.f;
  }

  T(*vw)[VS] = vl[wave];
  // K fragments of keys c + kt*16 + l16; V pieces: VPR lanes per row, RPL rows per
  // load (1 KB contiguous).  Past j1 the last valid row is loaded and masked later.
  constexpr int VR = kKC * DH * static_cast<int>(sizeof(T)) / (64 * 16);  // 16-byte pieces per lane
  constexpr int VPR = DH * static_cast<int>(sizeof(T)) / 16;               // 16-byte pieces per row
  constexpr int RPL = 64 / VPR;                                            // rows per load
  const int vrow0 = lane / VPR, vpiece = lane % VPR;
  Frag<T> kfa[2][KS], kfb[2][KS];
  f32x4 va[VR], vb[VR];  // raw 16-byte pieces (any element type)

#define DFLASH_LOAD_CHUNK(c, KF, VV)                                                          \
  {                                                                                           \
    _Pragma("unroll") for (int kt = 0; kt < 2; ++kt) {                                        \
      const int j_ = min((c) + kt * 16 + l16, j1 - 1);                                        \
      const T* krow_ = key_ptr(j_, ck, kblk);                                                 \
      _Pragma("unroll") for (int ks = 0; ks < KS; ++ks) KF[kt][ks].load(krow_ + ks * 32 + 8 * q4); \
    }                                                                                         \
    _Pragma("unroll") for (int e = 0; e < VR; ++e) {                                          \
      const int j_ = min((c) + e * RPL + vrow0, j1 - 1);                                      \
      const T* vrow_ = key_ptr(j_, cv, vblk);                                                 \
      VV[e] = reinterpret_cast<const f32x4*>(vrow_)[vpiece];                                  \
    }                                                                                         \
  }

#define DFLASH_PROCESS_CHUNK(c, KF, VV)                                                       \
  {                                                                                           \
    _Pragma("unroll") for (int e = 0; e < VR; ++e)                                            \
      reinterpret_cast<f32x4*>(&vw[e * RPL + vrow0][0])[vpiece] = VV[e];                      \
    f32x4 s_[2][RT];                                                                          \
    _Pragma("unroll") for (int kt = 0; kt < 2; ++kt)                                          \
      _Pragma("unroll") for (int rt = 0; rt < RT; ++rt) {                                     \
        s_[kt][rt] = f32x4{0.f, 0.f, 0.f, 0.f};                                               \
        _Pragma("unroll") for (int ks = 0; ks < KS; ++ks) Frag<T>::mma(s_[kt][rt], KF[kt][ks], qf[rt][ks]); \
      }                                                                                       \
    Frag<T> pf_[RT];                                                                          \
    _Pragma("unroll") for (int rt = 0; rt < RT; ++rt) {                                       \
      float x_[2][4];                                                                         \
      float mx_ = -INFINITY;                                                                  \
      _Pragma("unroll") for (int kt = 0; kt < 2; ++kt)                                        \
        _Pragma("unroll") for (int r = 0; r < 4; ++r) {                                       \
          const bool valid_ = (c) + kt * 16 + 4 * q4 + r < j1;                                \
          x_[kt][r] = valid_ ? s_[kt][rt][r] * scale : -INFINITY;                             \
          mx_ = fmaxf(mx_, x_[kt][r]);                                                        \
        }                                                                                     \
      mx_ = fmaxf(mx_, __shfl_xor(mx_, 16, kWave));                                           \
      mx_ = fmaxf(mx_, __shfl_xor(mx_, 32, kWave));                                           \
      const float m_new_ = fmaxf(m_run[rt], mx_);                                             \
      const float corr_ = expf(m_run[rt] - m_new_);                                           \
      float ps_ = 0.f;                                                                        \
      _Pragma("unroll") for (int kt = 0; kt < 2; ++kt)                                        \
        _Pragma("unroll") for (int r = 0; r < 4; ++r) {                                       \
          const float p_ = expf(x_[kt][r] - m_new_);                                          \
          ps_ += p_;                                                                          \
          pf_[rt].v[4 * kt + r] = from_f32<T>(p_);                                            \
        }                                                                                     \
      ps_ += __shfl_xor(ps_, 16, kWave);                                                      \
      ps_ += __shfl_xor(ps_, 32, kWave);                                                      \
      l_run[rt] = l_run[rt] * corr_ + ps_;                                                    \
      m_run[rt] = m_new_;                                                                     \
      _Pragma("unroll") for (int dt = 0; dt < DT; ++dt) o[rt][dt] *= corr_;                   \
    }                                                                                         \
    lds_written();                                                                            \
    _Pragma("unroll") for (int dt = 0; dt < DT; ++dt) {                                       \
      Frag<T> vf_;                                                                            \
      _Pragma("unroll") for (int t = 0; t < 8; ++t)                                           \
        vf_.v[t] = vw[(t < 4 ? 0 : 12) + 4 * q4 + t][dt * 16 + l16];                          \
      _Pragma("unroll") for (int rt = 0; rt < RT; ++rt) Frag<T>::mma(o[rt][dt], vf_, pf_[rt]); \
    }                                                                                         \
    lds_written();                                                                            \
  }

  // Two register sets in turn: the loads of the next chunk are in flight while this
  // one is processed, and nothing is copied between the sets.  Per chunk: S^T = K Q^T,
  // online softmax of row rt*16 + l16 over this lane's 8 keys and its 3 partner lanes
  // (the running max stays finite: key c < j1 is valid for every row), then
  // O^T += V^T P^T with V^T gathered as dim dt*16 + l16, keys {4*q4 + t, 16 + 4*q4 + t}.
  DFLASH_LOAD_CHUNK(j0, kfa, va)
  for (int c = j0; c < j1; c += 2 * kKC) {
    if (c + kKC < j1) DFLASH_LOAD_CHUNK(c + kKC, kfb, vb)
    DFLASH_PROCESS_CHUNK(c, kfa, va)
    if (c + kKC >= j1) break;
    if (c + 2 * kKC < j1) DFLASH_LOAD_CHUNK(c + 2 * kKC, kfa, va)
    DFLASH_PROCESS_CHUNK(c + kKC, kfb, vb)
  }
#undef DFLASH_LOAD_CHUNK
#undef DFLASH_PROCESS_CHUNK

  // output: lane -> row rt*16 + l16, dims dt*16 + 4*q4 .. +3
  const size_t grp = (static_cast<size_t>(b) * a.n_kv_heads + g) * a.n_rb + rb;
#pragma unroll
  for (int rt = 0; rt < RT; ++rt) {
    const int rr = rt * 16 + l16;
    if (rr >= nr) continue;
    const int r = r0 + rr, hl = r / k, i = r % k;
    if (n_split_b == 1) {
      T* out = static_cast<T*>(a.out);
      const float inv = 1.f / l_run[rt];
#pragma unroll
      for (int dt = 0; dt < DT; ++dt) {
        T* dst = out + pa_index(b * k + i, (g * G + hl) * DH + dt * 16 + 4 * q4, a.out_steps);
#pragma unroll
        for (int j = 0; j < 4; ++j) dst[j] = from_f32<T>(o[rt][dt][j] * inv);
      }
    } else {
      float* po = a.part_o + ((grp * a.max_splits + split) * kRows + rr) * DH;
#pragma unroll
      for (int dt = 0; dt < DT; ++dt)
        *reinterpret_cast<float4*>(po + dt * 16 + 4 * q4) =
            make_float4(o[rt][dt][0], o[rt][dt][1], o[rt][dt][2], o[rt][dt][3]);
      if (q4 == 0) {
        float* pml = a.part_ml + ((grp * a.max_splits + split) * kRows + rr) * 2;
        pml[0] = m_run[rt];
        pml[1] = l_run[rt];
      }
    }
  }
}

// Merge of the key splits of every (sequence, kv head, row block) whose keys were
// split; sequences with one split were finished by the attention kernel itself.
// One workgroup per row: thread t takes 4 head dims ((t % (DH/4)) * 4) and the
// splits s = t / (DH/4) (mod NSUB); the NSUB subsets combine in a fixed order, so
// the result does not depend on scheduling.
template <typename T, int DH>
__global__ __launch_bounds__(kThreads) void attention_merge_kernel(AttnArgs a) {
  constexpr int TPR = DH / 4, NSUB = kThreads / TPR;
  __shared__ float red_m[NSUB];
  __shared__ float4 red_o[NSUB][TPR];
  __shared__ float red_l[NSUB];
  const int rows = a.rows_per_block;
  const int rr = blockIdx.x % rows, grp_i = blockIdx.x / rows;
  const int rb = grp_i % a.n_rb, g = (grp_i / a.n_rb) % a.n_kv_heads, b = grp_i / (a.n_rb * a.n_kv_heads);
  const int k = a.block_k, G = a.n_q_heads / a.n_kv_heads;
  const int P = max(a.ctx_len[b], 0);
  const int n_keys = min(P, a.window) + k;
  const int n_split_b = (n_keys + a.keys_per_split - 1) / a.keys_per_split;
  const int r0 = rb * rows;
  if (n_split_b == 1 || rr >= min(rows, G * k - r0)) return;  // uniform per workgroup
  const int t = threadIdx.x, dq = t % TPR, sub = t / TPR;
  const size_t grp = (static_cast<size_t>(b) * a.n_kv_heads + g) * a.n_rb + rb;
  auto ml = [&](int s) { return a.part_ml + ((grp * a.max_splits + s) * kRows + rr) * 2; };
  float mloc = -INFINITY;
  for (int s = sub; s < n_split_b; s += NSUB) mloc = fmaxf(mloc, ml(s)[0]);
  if (dq == 0) red_m[sub] = mloc;
  __syncthreads();
  float M = -INFINITY;
#pragma unroll
  for (int i = 0; i < NSUB; ++i) M = fmaxf(M, red_m[i]);
  float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
  float L = 0.f;
  for (int s = sub; s < n_split_b; s += NSUB) {
    const float* pm = ml(s);
    const float w = expf(pm[0] - M);
    L += pm[1] * w;
    const float4 v = *reinterpret_cast<const float4*>(a.part_o + ((grp * a.max_splits + s) * kRows + rr) * DH + 4 * dq);
    acc.x += v.x * w;
    acc.y += v.y * w;
    acc.z += v.z * w;
    acc.w += v.w * w;
  }
  red_o[sub][dq] = acc;
  if (dq == 0) red_l[sub] = L;
  __syncthreads();
  if (sub != 0) return;
  float4 o = red_o[0][dq];
  float Lt = red_l[0];
#pragma unroll
  for (int i = 1; i < NSUB; ++i) {
    const float4 v = red_o[i][dq];
    o.x += v.x;
    o.y += v.y;
    o.z += v.z;
    o.w += v.w;
    Lt += red_l[i];
  }
  const int r = r0 + rr, hl = r / k, i = r % k;
  T* dst = static_cast<T*>(a.out) + pa_index(b * k + i, (g * G + hl) * DH + 4 * dq, a.out_steps);
  const float inv = 1.f / Lt;
  dst[0] = from_f32<T>(o.x * inv);
  dst[1] = from_f32<T>(o.y * inv);
  dst[2] = from_f32<T>(o.z * inv);
  dst[3] = from_f32<T>(o.w * inv);
}

template <typename T, int DH, int RT>
static void launch_rt(const AttnArgs& a, hipStream_t s) {
  const long long items = static_cast<long long>(a.batch) * a.n_kv_heads * a.n_rb * a.max_splits;
  hipLaunchKernelGGL((attention_kernel<T, DH, RT>), dim3(static_cast<unsigned>((items + 3) / 4)), dim3(kThreads), 0,
                     s, a);
}

template <typename T, int DH>
static hipError_t launch_dh(const AttnArgs& a, hipStream_t s) {
  switch (a.rows_per_block / 16) {
    case 1: launch_rt<T, DH, 1>(a, s); break;
    case 2: launch_rt<T, DH, 2>(a, s); break;
    default: return hipErrorInvalidValue;
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || a.max_splits == 1) return e;
  const long long wgs = static_cast<long long>(a.batch) * a.n_kv_heads * a.n_rb * a.rows_per_block;
  hipLaunchKernelGGL((attention_merge_kernel<T, DH>), dim3(static_cast<unsigned>(wgs)), dim3(kThreads), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_attention(bool f32, const AttnArgs& a, hipStream_t stream) {
  if (a.head_dim == 128) return f32 ? launch_dh<float, 128>(a, stream) : launch_dh<f16, 128>(a, stream);
  if (a.head_dim == 64) return f32 ? launch_dh<float, 64>(a, stream) : launch_dh<f16, 64>(a, stream);
  return hipErrorInvalidValue;
}

}  // namespace dflash
