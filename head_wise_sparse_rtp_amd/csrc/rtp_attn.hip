// Split-K softmax attention partials and their merge.
//
// Method: Full Attention Strikes Back (xllm-io.github.io paper review), section 三,
// 核心公式: exact softmax attention of the query over the selected keys/values (the
// sparse-attention equation) for retrieval heads; section 五 (test configuration) and
// the gist.science summary, section 1: local heads attend over a window plus sinks.
//
// A work item holds a slice of the token set and produces (m, l, acc): the running max
// of the base-2 scaled logits, sum of 2^(s - m), and the 2^(s - m)-weighted value sum.
// A second pass merges the slices of a head.  Layout per row of a wave: 16 lanes share
// one key/value row (8 dims per lane, a 16-byte fp16 load), 4 rows per wave step.
#include "rtp_internal.h"

namespace rtp {

namespace {

typedef _Float16 h8 __attribute__((ext_vector_type(8)));

template <typename KT>
struct Vec8;

template <>
struct Vec8<f16> {
  h8 v;
  __device__ __forceinline__ void load(const f16* __restrict__ p) {
    v = *reinterpret_cast<const h8*>(p);
  }
  __device__ __forceinline__ float at(int i) const { return static_cast<float>(v[i]); }
};

template <>
struct Vec8<float> {
  float4 a, b;
  __device__ __forceinline__ void load(const float* __restrict__ p) {
    a = reinterpret_cast<const float4*>(p)[0];
    b = reinterpret_cast<const float4*>(p)[1];
  }
  __device__ __forceinline__ float at(int i) const {
    const float4& x = i < 4 ? a : b;
    switch (i & 3) {
      case 0: return x.x;
      case 1: return x.y;
      case 2: return x.z;
      default: return x.w;
    }
  }
};

template <>
struct Vec8<bf16s> {
  uint4 v;  // 8 bfloat16 values, two per word
  __device__ __forceinline__ void load(const bf16s* __restrict__ p) {
    v = *reinterpret_cast<const uint4*>(p);
  }
  __device__ __forceinline__ float at(int i) const {
    const int j = i >> 1;
    const uint32_t w = j == 0 ? v.x : (j == 1 ? v.y : (j == 2 ? v.z : v.w));
    return bf16_to_f((i & 1) ? (w >> 16) : (w & 0xFFFFu));
  }
};

__device__ __forceinline__ int clamp_len(const int32_t* seq_lens, int b, int Lmax) {
  int L = seq_lens[b];
  return L < 0 ? 0 : (L > Lmax ? Lmax : L);
}

// sum over the 16 lanes of a row group
__device__ __forceinline__ float group16_sum(float v) {
  v += __shfl_xor(v, 8, 64);
  v += __shfl_xor(v, 4, 64);
  v += __shfl_xor(v, 2, 64);
  v += __shfl_xor(v, 1, 64);
  return v;
}

struct SoftState {
  float m, l, acc[8];
};

__device__ __forceinline__ void soft_init(SoftState& s) {
  s.m = -INFINITY;
  s.l = 0.0f;
#pragma unroll
  for (int i = 0; i < 8; i++) s.acc[i] = 0.0f;
}

// online update with logit s2 (base-2 units) and value row v
template <typename KT>
__device__ __forceinline__ void soft_update(SoftState& st, float s2, const Vec8<KT>& v) {
  const float mn = fmaxf(st.m, s2);
  const float a = st.m == -INFINITY ? 0.0f : __builtin_amdgcn_exp2f(st.m - mn);
  const float bt = __builtin_amdgcn_exp2f(s2 - mn);
  st.l = st.l * a + bt;
#pragma unroll
  for (int i = 0; i < 8; i++) st.acc[i] = st.acc[i] * a + bt * v.at(i);
  st.m = mn;
}

// merge state o (from another lane group / wave) into s
__device__ __forceinline__ void soft_merge(SoftState& s, float om, float ol, const float* oacc) {
  const float mn = fmaxf(s.m, om);
  if (mn == -INFINITY) return;
  const float a = s.m == -INFINITY ? 0.0f : __builtin_amdgcn_exp2f(s.m - mn);
  const float c = om == -INFINITY ? 0.0f : __builtin_amdgcn_exp2f(om - mn);
  s.l = s.l * a + ol * c;
#pragma unroll
  for (int i = 0; i < 8; i++) s.acc[i] = s.acc[i] * a + oacc[i] * c;
  s.m = mn;
}

// combine the four 16-lane groups of a wave (result valid in every lane)
__device__ __forceinline__ void wave_combine(SoftState& s) {
#pragma unroll
  for (int off = 16; off <= 32; off <<= 1) {
    float oacc[8];
    const float om = __shfl_xor(s.m, off, 64);
    const float ol = __shfl_xor(s.l, off, 64);
#pragma unroll
    for (int i = 0; i < 8; i++) oacc[i] = __shfl_xor(s.acc[i], off, 64);
    soft_merge(s, om, ol, oacc);
  }
}

template <typename KT>
__device__ __forceinline__ void load_q8(const KT* __restrict__ qrow, int li, float (&q)[8],
                                        float scale2) {
  Vec8<KT> v;
  v.load(qrow + li * 8);
#pragma unroll
  for (int i = 0; i < 8; i++) q[i] = v.at(i) * scale2;
}

// ---------------------------------------------------------------------------
// sparse partials: each wave takes work items (row bh, split) in a grid-stride loop;
// item covers sel_idx[bh, split*kSplit : +kSplit] (clipped to the set size).
// ---------------------------------------------------------------------------
template <typename KT>
__global__ __launch_bounds__(kThreads) void k_sparse_partial(
    const KT* __restrict__ q, const KT* __restrict__ K, const KT* __restrict__ V,
    const int32_t* __restrict__ sel_idx, const int32_t* __restrict__ sel_count, int cap,
    HeadMap map, int Hq, int Hr, int G, int Lmax, float scale2, int BH, int maxs,
    float* __restrict__ pm, float* __restrict__ pl, float* __restrict__ pacc) {
  const int lane = threadIdx.x & 63;
  const int grp = lane >> 4;
  const int li = lane & 15;
  const int wave = (blockIdx.x * kThreads + threadIdx.x) >> 6;
  const int nwaves = (gridDim.x * kThreads) >> 6;
  const int H = Hr * G;
  const long long total = (long long)BH * maxs;
  for (long long it = wave; it < total; it += nwaves) {
    const int bh = (int)(it % BH);
    const int split = (int)(it / BH);
    int n = sel_count[bh];
    n = n < 0 ? 0 : (n > cap ? cap : n);
    const int start = split * kSplit;
    if (start >= n) continue;
    const int end = min(start + kSplit, n);
    const int b = bh / H;
    const int h = bh % H;
    const int kr = h / G;
    const int g = h % G;
    float qv[8];
    load_q8<KT>(q + ((size_t)b * Hq + (size_t)map.kv[kr] * G + g) * kD, li, qv, scale2);
    const KT* Kb = K + ((size_t)b * Hr + kr) * (size_t)Lmax * kD;
    const KT* Vb = V + ((size_t)b * Hr + kr) * (size_t)Lmax * kD;
    const int32_t* ids = sel_idx + (size_t)bh * cap;
    SoftState st;
    soft_init(st);
    for (int r0 = start; r0 < end; r0 += 16) {
      // issue the loads of 4 steps (16 rows) before any use
      Vec8<KT> kk[4], vv[4];
      bool act[4];
#pragma unroll
      for (int u = 0; u < 4; u++) {
        const int ri = r0 + u * 4 + grp;
        int tok = ri < end ? ids[ri] : -1;
        act[u] = tok >= 0 && tok < Lmax;
        if (act[u]) {
          kk[u].load(Kb + (size_t)tok * kD + li * 8);
          vv[u].load(Vb + (size_t)tok * kD + li * 8);
        }
      }
#pragma unroll
      for (int u = 0; u < 4; u++) {
        float d = 0.0f;
        if (act[u]) {
#pragma unroll
          for (int i = 0; i < 8; i++) d = __builtin_fmaf(qv[i], kk[u].at(i), d);
        }
        d = group16_sum(d);
        if (act[u]) soft_update<KT>(st, d, vv[u]);
      }
    }
    wave_combine(st);
    const size_t o = (size_t)bh * maxs + split;
    if (lane == 0) {
      pm[o] = st.m;
      pl[o] = st.l;
    }
    if (lane < 16) {
#pragma unroll
      for (int i = 0; i < 8; i++) pacc[o * kD + li * 8 + i] = st.acc[i];
    }
  }
}

// ---------------------------------------------------------------------------
// window partials: block = (split, local KV head x head group, b); GG query heads
// share each ring row.  Rows of the split are window-set entries e in
// [split*kWinSplit, +kWinSplit): e < ns -> sink position e, else position
// max(sinks, L - window) + (e - ns); slot = pos (sink) or sinks + pos mod window.
// ---------------------------------------------------------------------------
template <typename KT, int GG>
__global__ __launch_bounds__(kThreads) void k_window_partial(
    const KT* __restrict__ q, const KT* __restrict__ K, const KT* __restrict__ V,
    const int32_t* __restrict__ seq_lens, HeadMap map, int Hq, int Hl, int G, int ngrp,
    int window, int sinks, float scale2, int maxs, float* __restrict__ pm,
    float* __restrict__ pl, float* __restrict__ pacc) {
  __shared__ float sm[kThreads / 64][GG], sl[kThreads / 64][GG];
  __shared__ float sacc[kThreads / 64][GG][kD];
  const int lane = threadIdx.x & 63;
  const int wv = threadIdx.x >> 6;
  const int grp = lane >> 4;
  const int li = lane & 15;
  const int split = blockIdx.x;
  const int kl = blockIdx.y / ngrp;
  const int g0 = (blockIdx.y % ngrp) * GG;
  const int b = blockIdx.z;
  const int ring = sinks + window;
  int L = seq_lens[b];
  L = L < 0 ? 0 : L;
  const int ns = min(sinks, L);
  const int wstart = max(sinks, L - window);
  const int nwin = ns + max(0, L - wstart);
  const int e0 = split * kWinSplit;
  const int e1 = min(e0 + kWinSplit, nwin);
  const int H = Hl * G;

  float qv[GG][8];
#pragma unroll
  for (int gg = 0; gg < GG; gg++) {
    const int g = min(g0 + gg, G - 1);
    load_q8<KT>(q + ((size_t)b * Hq + (size_t)map.kv[kl] * G + g) * kD, li, qv[gg], scale2);
  }
  SoftState st[GG];
#pragma unroll
  for (int gg = 0; gg < GG; gg++) soft_init(st[gg]);

  const KT* Kb = K + ((size_t)b * Hl + kl) * (size_t)ring * kD;
  const KT* Vb = V + ((size_t)b * Hl + kl) * (size_t)ring * kD;
  // each wave takes rows e0 + wv*4 + grp + 16*k
  for (int e = e0 + wv * 4 + grp; e - grp < e1; e += 16) {
    const bool act = e < e1;
    Vec8<KT> kk, vv;
    if (act) {
      const int pos = e < ns ? e : wstart + (e - ns);
      const int slot = pos < sinks ? pos : sinks + pos % window;
      kk.load(Kb + (size_t)slot * kD + li * 8);
      vv.load(Vb + (size_t)slot * kD + li * 8);
    }
#pragma unroll
    for (int gg = 0; gg < GG; gg++) {
      float d = 0.0f;
      if (act) {
#pragma unroll
        for (int i = 0; i < 8; i++) d = __builtin_fmaf(qv[gg][i], kk.at(i), d);
      }
      d = group16_sum(d);
      if (act) soft_update<KT>(st[gg], d, vv);
    }
  }
#pragma unroll
  for (int gg = 0; gg < GG; gg++) {
    wave_combine(st[gg]);
    if (lane == 0) {
      sm[wv][gg] = st[gg].m;
      sl[wv][gg] = st[gg].l;
    }
    if (lane < 16) {
#pragma unroll
      for (int i = 0; i < 8; i++) sacc[wv][gg][li * 8 + i] = st[gg].acc[i];
    }
  }
  __syncthreads();
  // thread t: head gg = t / 32 (when GG*32 <= 256), dims 4*(t%32) .. +4
  for (int idx = threadIdx.x; idx < GG * 32; idx += kThreads) {
    const int gg = idx / 32;
    const int d0 = (idx % 32) * 4;
    if (g0 + gg >= G) continue;
    float M = -INFINITY;
    for (int k = 0; k < kThreads / 64; k++) M = fmaxf(M, sm[k][gg]);
    float l = 0.0f, a[4] = {0.0f, 0.0f, 0.0f, 0.0f};
    if (M != -INFINITY) {
      for (int k = 0; k < kThreads / 64; k++) {
        if (sm[k][gg] == -INFINITY) continue;
        const float f = __builtin_amdgcn_exp2f(sm[k][gg] - M);
        l += sl[k][gg] * f;
#pragma unroll
        for (int i = 0; i < 4; i++) a[i] += sacc[k][gg][d0 + i] * f;
      }
    }
    const size_t o = ((size_t)(b * H + kl * G + g0 + gg)) * maxs + split;
    if (d0 == 0) {
      pm[o] = M;
      pl[o] = l;
    }
#pragma unroll
    for (int i = 0; i < 4; i++) pacc[o * kD + d0 + i] = a[i];
  }
}

// ---------------------------------------------------------------------------
// merge: one block (128 threads, one per dim) per (row, b)
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(kD) void k_merge(const float* __restrict__ pm,
                                              const float* __restrict__ pl,
                                              const float* __restrict__ pacc, int maxs,
                                              const int32_t* __restrict__ sel_count, int cap,
                                              HeadMap map, int Hq, int Hrows_kv, int G,
                                              float* __restrict__ out, float* __restrict__ lse) {
  const int row = blockIdx.x;  // kr * G + g
  const int b = blockIdx.y;
  const int H = Hrows_kv * G;
  const size_t bh = (size_t)b * H + row;
  int ns = maxs;
  if (sel_count) {
    int n = sel_count[bh];
    n = n < 0 ? 0 : (n > cap ? cap : n);
    ns = (n + kSplit - 1) / kSplit;
  }
  const int d = threadIdx.x;
  float M = -INFINITY;
  for (int s = 0; s < ns; s++) M = fmaxf(M, pm[bh * maxs + s]);
  float l = 0.0f, a = 0.0f;
  if (M != -INFINITY) {
    for (int s = 0; s < ns; s++) {
      const float ms = pm[bh * maxs + s];
      if (ms == -INFINITY) continue;
      const float f = __builtin_amdgcn_exp2f(ms - M);
      l += pl[bh * maxs + s] * f;
      a += pacc[(bh * maxs + s) * kD + d] * f;
    }
  }
  const int kr = row / G;
  const int g = row % G;
  const size_t orow = (size_t)b * Hq + (size_t)map.kv[kr] * G + g;
  out[orow * kD + d] = l > 0.0f ? a / l : 0.0f;
  if (lse && d == 0) lse[orow] = l > 0.0f ? (M + __log2f(l)) * 0.69314718055994531f : -INFINITY;
}

}  // namespace

static constexpr float kLog2ef = 1.4426950408889634f;

hipError_t launch_sparse_partial(const void* q, const void* K, const void* V, int kv_dtype,
                                 const int32_t* sel_idx, const int32_t* sel_count, int cap,
                                 const HeadMap& map, int B, int Hq, int Hr, int G, int Lmax,
                                 float scale_attn, const AttnPartials& pa, int maxs,
                                 hipStream_t st) {
  const int BH = B * Hr * G;
  const long long items = (long long)BH * maxs;
  long long blocks = (items + 3) / 4;
  if (blocks > 2048) blocks = 2048;
  if (blocks < 1) blocks = 1;
  const float scale2 = scale_attn * kLog2ef;
  if (kv_dtype == 1) {
    k_sparse_partial<f16><<<(int)blocks, kThreads, 0, st>>>(
        (const f16*)q, (const f16*)K, (const f16*)V, sel_idx, sel_count, cap, map, Hq, Hr, G,
        Lmax, scale2, BH, maxs, pa.m, pa.l, pa.acc);
  } else if (kv_dtype == 2) {
    k_sparse_partial<bf16s><<<(int)blocks, kThreads, 0, st>>>(
        (const bf16s*)q, (const bf16s*)K, (const bf16s*)V, sel_idx, sel_count, cap, map, Hq, Hr,
        G, Lmax, scale2, BH, maxs, pa.m, pa.l, pa.acc);
  } else {
    k_sparse_partial<float><<<(int)blocks, kThreads, 0, st>>>(
        (const float*)q, (const float*)K, (const float*)V, sel_idx, sel_count, cap, map, Hq, Hr,
        G, Lmax, scale2, BH, maxs, pa.m, pa.l, pa.acc);
  }
  return hipGetLastError();
}

hipError_t launch_window_partial(const void* q, const void* K, const void* V, int kv_dtype,
                                 const int32_t* seq_lens, const HeadMap& map, int B, int Hq,
                                 int Hl, int G, int window, int sinks, float scale_attn,
                                 const AttnPartials& pa, int maxs, hipStream_t st) {
  const int GG = G >= 8 ? 8 : (G >= 4 ? 4 : (G >= 2 ? 2 : 1));
  const int ngrp = (G + GG - 1) / GG;
  dim3 grid(maxs, Hl * ngrp, B);
  const float scale2 = scale_attn * kLog2ef;
#define RTP_WIN(KT, GGV)                                                                       \
  k_window_partial<KT, GGV><<<grid, kThreads, 0, st>>>(                                       \
      (const KT*)q, (const KT*)K, (const KT*)V, seq_lens, map, Hq, Hl, G, ngrp, window, sinks, \
      scale2, maxs, pa.m, pa.l, pa.acc)
  if (kv_dtype == 1) {
    switch (GG) {
      case 8: RTP_WIN(f16, 8); break;
      case 4: RTP_WIN(f16, 4); break;
      case 2: RTP_WIN(f16, 2); break;
      default: RTP_WIN(f16, 1); break;
    }
  } else if (kv_dtype == 2) {
    switch (GG) {
      case 8: RTP_WIN(bf16s, 8); break;
      case 4: RTP_WIN(bf16s, 4); break;
      case 2: RTP_WIN(bf16s, 2); break;
      default: RTP_WIN(bf16s, 1); break;
    }
  } else {
    switch (GG) {
      case 8: RTP_WIN(float, 8); break;
      case 4: RTP_WIN(float, 4); break;
      case 2: RTP_WIN(float, 2); break;
      default: RTP_WIN(float, 1); break;
    }
  }
#undef RTP_WIN
  return hipGetLastError();
}

hipError_t launch_merge(const AttnPartials& pa, int maxs, const int32_t* sel_count, int cap,
                        const HeadMap& map, int B, int Hq, int Hrows_kv, int G, float* out,
                        float* lse, hipStream_t st) {
  dim3 grid(Hrows_kv * G, B);
  k_merge<<<grid, kD, 0, st>>>(pa.m, pa.l, pa.acc, maxs, sel_count, cap, map, Hq, Hrows_kv, G,
                               out, lse);
  return hipGetLastError();
}

}  // namespace rtp
