// Indexer score and chunked 256-bin histogram partials.
//
// Method: Full Attention Strikes Back (xllm-io.github.io paper review), section 三:
// the indexer score of the adaptive-sparse-attention equations, and the sort-free
// top-p of 硬件感知解码内核 (a 256-bin histogram per head, 1 KB, independent of L).
//
// Bins live on a global grid of cells g = floor(z / w).  A chunk of tokens anchors
// its partial histogram at its own top cell A_c; partials merge exactly by integer
// shifts once the global top cell is known, so one pass over the keys suffices.
//
// Mass of a token in chunk bin j < 255 (relative to exp((A_c + 1) w)):
//     exp(z - (A_c + 1) w) = exp(-j w) * x,   x = exp(z - (g + 1) w) in (e^-w, 1]
// x * 2^24 is an integer after fp32 rounding (x >= 0.5), so the per-bin sums of
// x * 2^24 accumulate EXACTLY in 64-bit LDS counters: the histogram does not depend
// on the order of the atomics.  Tokens 255 or more cells below A_c go to the last
// bin with their extra factor exp(-(A_c - g - 255) w) folded into x.
#include "rtp_internal.h"

namespace rtp {

namespace {

typedef _Float16 h8 __attribute__((ext_vector_type(8)));

// 16 indexer features of one token, kept in the storage type until used.
template <typename KT>
struct Row16;

template <>
struct Row16<f16> {
  h8 a, b;
  __device__ __forceinline__ void load(const f16* __restrict__ p) {
    const h8* q = reinterpret_cast<const h8*>(p);
    a = q[0];
    b = q[1];
  }
  __device__ __forceinline__ float at(int i) const {
    return i < 8 ? static_cast<float>(a[i]) : static_cast<float>(b[i - 8]);
  }
};

template <>
struct Row16<float> {
  float4 v[4];
  __device__ __forceinline__ void load(const float* __restrict__ p) {
    const float4* q = reinterpret_cast<const float4*>(p);
#pragma unroll
    for (int i = 0; i < 4; i++) v[i] = q[i];
  }
  __device__ __forceinline__ float at(int i) const {
    const float4& x = v[i >> 2];
    switch (i & 3) {
      case 0: return x.x;
      case 1: return x.y;
      case 2: return x.z;
      default: return x.w;
    }
  }
};

template <>
struct Row16<bf16s> {
  uint4 a, b;  // 16 bfloat16 values, two per word
  __device__ __forceinline__ void load(const bf16s* __restrict__ p) {
    const uint4* q = reinterpret_cast<const uint4*>(p);
    a = q[0];
    b = q[1];
  }
  __device__ __forceinline__ float at(int i) const {
    const uint4& x = i < 8 ? a : b;
    const int j = (i & 7) >> 1;
    const uint32_t w = j == 0 ? x.x : (j == 1 ? x.y : (j == 2 ? x.z : x.w));
    return bf16_to_f((i & 1) ? (w >> 16) : (w & 0xFFFFu));
  }
};

// fp32 fused multiply-add chain over the 16 features, in index order.
template <typename KT>
__device__ __forceinline__ float fma_chain(const float* q, const Row16<KT>& k) {
  float a = 0.0f;
#pragma unroll
  for (int i = 0; i < kR; i++) a = __builtin_fmaf(q[i], k.at(i), a);
  return a;
}

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, 64));
  return v;
}

__device__ __forceinline__ int clamp_len(const int32_t* seq_lens, int b, int Lmax) {
  int L = seq_lens[b];
  return L < 0 ? 0 : (L > Lmax ? Lmax : L);
}

// ---------------------------------------------------------------------------
// rtp_index_score: z[b, kr*G+g, n] = fl32(scale * chain(q_idx, k_idx[n]))
// ---------------------------------------------------------------------------
template <typename KT, int GG, int TPT>
__global__ __launch_bounds__(kThreads) void k_index_score(
    const float* __restrict__ q_idx, const KT* __restrict__ k_idx,
    const int32_t* __restrict__ seq_lens, int Hr, int G, int Lmax, int ngrp, float scale,
    float* __restrict__ z) {
  const int b = blockIdx.z;
  const int kr = blockIdx.y / ngrp;
  const int g0 = (blockIdx.y % ngrp) * GG;
  const int L = clamp_len(seq_lens, b, Lmax);
  const int base = blockIdx.x * (kThreads * TPT);
  if (base >= L) return;
  const int Hq = Hr * G;
  float q[GG][kR];
#pragma unroll
  for (int gg = 0; gg < GG; gg++) {
    const int g = g0 + gg;
#pragma unroll
    for (int i = 0; i < kR; i++)
      q[gg][i] = g < G ? q_idx[((size_t)b * Hq + (size_t)kr * G + g) * kR + i] : 0.0f;
  }
  const KT* kb = k_idx + ((size_t)b * Hr + kr) * (size_t)Lmax * kR;
  Row16<KT> rows[TPT];
#pragma unroll
  for (int t = 0; t < TPT; t++) {
    const int n = base + t * kThreads + threadIdx.x;
    if (n < L) rows[t].load(kb + (size_t)n * kR);
  }
#pragma unroll
  for (int t = 0; t < TPT; t++) {
    const int n = base + t * kThreads + threadIdx.x;
    if (n >= L) continue;
#pragma unroll
    for (int gg = 0; gg < GG; gg++) {
      const int g = g0 + gg;
      if (g < G) {
        const float a = fma_chain<KT>(q[gg], rows[t]);
        z[((size_t)b * Hq + (size_t)kr * G + g) * Lmax + n] = a * scale;
      }
    }
  }
}

// ---------------------------------------------------------------------------
// chunk histogram partials
//   MODE 0: logits read from z [B, H, Lmax]; rows blockIdx.y*GG .. +GG
//   MODE 1: logits computed from q_idx / k_idx; rows kr*G + g0 + gg
// Outputs per (row, chunk): part_A (top cell), part_mass[256], packed codes.
// ---------------------------------------------------------------------------
constexpr int kCopies = 2;   // lanes alternate between histogram copies
constexpr int kPad = 1;      // u64 padding per 256-bin row (spreads LDS banks)

template <int MODE, typename KT, int GG, int TPT>
__global__ __launch_bounds__(kThreads) void k_hist(
    const float* __restrict__ zin, const float* __restrict__ q_idx,
    const KT* __restrict__ k_idx, const int32_t* __restrict__ seq_lens, HeadMap map, int H,
    int Hq, int Hr, int G, int Lmax, int ngrp, float yscale, float inv_w, float c_log2,
    double w, int nchunk, float* __restrict__ part_mass, int32_t* __restrict__ part_A,
    uint32_t* __restrict__ codes) {
  constexpr int TC = kThreads * TPT;
  __shared__ unsigned long long hist[kCopies * GG * (kNB + kPad)];
  __shared__ float smax[GG][kThreads / 64];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wv = tid >> 6;
  const int chunk = blockIdx.x;
  const int b = blockIdx.z;
  int row0, nrows, kr = 0;
  if (MODE == 0) {
    row0 = blockIdx.y * GG;
    nrows = min(GG, H - row0);
  } else {
    kr = blockIdx.y / ngrp;
    const int g0 = (blockIdx.y % ngrp) * GG;
    row0 = kr * G + g0;
    nrows = min(GG, G - g0);
  }
  const int L = clamp_len(seq_lens, b, Lmax);
  const int base = chunk * TC;
  const size_t rowb = (size_t)b * H + row0;
  if (base >= L) {
    if (tid < nrows) part_A[(rowb + tid) * nchunk + chunk] = kEmptyCell;
    return;
  }

  // ---- pass 1: logits in cell units y = z / w, and the chunk's top cell ----
  float y[TPT][GG];
  float ymax[GG];
#pragma unroll
  for (int gg = 0; gg < GG; gg++) ymax[gg] = -INFINITY;

  if (MODE == 0) {
#pragma unroll
    for (int t = 0; t < TPT; t++) {
      const int n = base + t * kThreads + tid;
#pragma unroll
      for (int gg = 0; gg < GG; gg++) {
        float v = -INFINITY;
        if (n < L && gg < nrows) v = zin[(rowb + gg) * Lmax + n] * inv_w;
        y[t][gg] = v;
        ymax[gg] = fmaxf(ymax[gg], v);
      }
    }
  } else {
    const KT* kb = k_idx + ((size_t)b * Hr + kr) * (size_t)Lmax * kR;
    Row16<KT> rows[TPT];
#pragma unroll
    for (int t = 0; t < TPT; t++) {
      const int n = base + t * kThreads + tid;
      if (n < L) rows[t].load(kb + (size_t)n * kR);
    }
#pragma unroll
    for (int gg = 0; gg < GG; gg++) {
      float q[kR];
      const int g = row0 - kr * G + gg;
      const size_t qrow = ((size_t)b * Hq + (size_t)map.kv[kr] * G + g) * kR;
#pragma unroll
      for (int i = 0; i < kR; i++) q[i] = gg < nrows ? q_idx[qrow + i] : 0.0f;
#pragma unroll
      for (int t = 0; t < TPT; t++) {
        const int n = base + t * kThreads + tid;
        // y = fl32(a * scale) / w exactly: w is a power of two, so scaling the
        // product by 1/w before or after rounding gives the same fp32 value.
        float v = fma_chain<KT>(q, rows[t]) * yscale;
        if (n >= L || gg >= nrows) v = -INFINITY;
        y[t][gg] = v;
        ymax[gg] = fmaxf(ymax[gg], v);
      }
    }
  }

#pragma unroll
  for (int gg = 0; gg < GG; gg++) {
    const float m = wave_max(ymax[gg]);
    if (lane == 0) smax[gg][wv] = m;
  }
  for (int i = tid; i < kCopies * GG * (kNB + kPad); i += kThreads) hist[i] = 0ull;
  __syncthreads();
  int Ac[GG];
#pragma unroll
  for (int gg = 0; gg < GG; gg++) {
    float m = smax[gg][0];
#pragma unroll
    for (int k = 1; k < kThreads / 64; k++) m = fmaxf(m, smax[gg][k]);
    Ac[gg] = gg < nrows ? (int)floorf(m) : 0;
  }

  // ---- pass 2: exact per-bin mass accumulation and bin codes ----
  const int copy = lane & (kCopies - 1);
  uint32_t cw[GG];
#pragma unroll
  for (int gg = 0; gg < GG; gg++) cw[gg] = 0u;
#pragma unroll
  for (int t = 0; t < TPT; t++) {
    const int n = base + t * kThreads + tid;
#pragma unroll
    for (int gg = 0; gg < GG; gg++) {
      uint32_t j = 255u;
      if (n < L && gg < nrows) {
        const float yv = y[t][gg];
        const float gf = floorf(yv);
        const int diff = Ac[gg] - (int)gf;
        j = (uint32_t)min(diff, 255);
        float arg = __builtin_fmaf(yv - gf, c_log2, -c_log2);
        if (diff > 255) arg -= (float)(diff - 255) * c_log2;
        const float e = __builtin_amdgcn_exp2f(arg) * 16777216.0f;
        const unsigned long long xi = (unsigned long long)(uint32_t)e;
        atomicAdd(&hist[(copy * GG + gg) * (kNB + kPad) + j], xi);
      }
      cw[gg] |= j << (8 * (t & 3));
    }
    if ((t & 3) == 3) {
#pragma unroll
      for (int gg = 0; gg < GG; gg++) {
        if (gg < nrows)
          codes[((rowb + gg) * nchunk + chunk) * (size_t)(TC / 4) + (t >> 2) * kThreads + tid] =
              cw[gg];
        cw[gg] = 0u;
      }
    }
  }
  __syncthreads();

  // ---- write the chunk partial: mu_j = 2^-24 * exp(-j w) * sum ----
  const int j = tid;
  const double binf = exp(-(double)j * w) * 5.9604644775390625e-08;  // 2^-24
#pragma unroll
  for (int gg = 0; gg < GG; gg++) {
    if (gg < nrows) {
      unsigned long long s = 0ull;
#pragma unroll
      for (int c = 0; c < kCopies; c++) s += hist[(c * GG + gg) * (kNB + kPad) + j];
      part_mass[((rowb + gg) * nchunk + chunk) * kNB + j] = (float)((double)s * binf);
      if (j == 0) part_A[(rowb + gg) * nchunk + chunk] = Ac[gg];
    }
  }
}

template <int MODE, typename KT, int GG>
hipError_t hist_dispatch_tpt(dim3 grid, const ChunkGeom& cg, hipStream_t st, const float* zin,
                             const float* q_idx, const void* k_idx, const int32_t* seq_lens,
                             const HeadMap& map, int H, int Hq, int Hr, int G, int Lmax, int ngrp,
                             float yscale, float inv_w, float c_log2, double w,
                             const SelectBufs& sb) {
  const KT* kp = static_cast<const KT*>(k_idx);
#define RTP_HIST_LAUNCH(T)                                                                      \
  k_hist<MODE, KT, GG, T><<<grid, kThreads, 0, st>>>(zin, q_idx, kp, seq_lens, map, H, Hq, Hr, \
                                                     G, Lmax, ngrp, yscale, inv_w, c_log2, w,  \
                                                     cg.nchunk, sb.part_mass, sb.part_A,       \
                                                     sb.codes)
  if (cg.tpt == 4)
    RTP_HIST_LAUNCH(4);
  else
    RTP_HIST_LAUNCH(8);
#undef RTP_HIST_LAUNCH
  return hipGetLastError();
}

int pick_gg(int G) { return G >= 8 ? 8 : (G >= 4 ? 4 : (G >= 2 ? 2 : 1)); }

}  // namespace

// chunk geometry: 2048-token chunks, halved while that leaves fewer than 256 blocks
ChunkGeom chunk_geom(int64_t units, int64_t Lmax) {
  ChunkGeom cg;
  int tpt = 8;
  while (tpt > 4 && units * ((Lmax + kThreads * tpt - 1) / (kThreads * tpt)) < 256) tpt >>= 1;
  cg.tpt = tpt;
  cg.tc = kThreads * tpt;
  cg.nchunk = (int)((Lmax + cg.tc - 1) / cg.tc);
  cg.nsplit = (cg.nchunk + kMerge1 - 1) / kMerge1;
  return cg;
}

hipError_t launch_index_score(const float* q_idx, const void* k_idx, int k_dtype,
                              const int32_t* seq_lens, int B, int Hr, int G, int Lmax,
                              float scale_idx, float* z, hipStream_t st) {
  const int GG = pick_gg(G);
  const int ngrp = (G + GG - 1) / GG;
  constexpr int TPT = 8;
  dim3 grid((Lmax + kThreads * TPT - 1) / (kThreads * TPT), Hr * ngrp, B);
#define RTP_SCORE_LAUNCH(KT, GGV)                                                              \
  k_index_score<KT, GGV, TPT><<<grid, kThreads, 0, st>>>(                                    \
      q_idx, static_cast<const KT*>(k_idx), seq_lens, Hr, G, Lmax, ngrp, scale_idx, z)
  if (k_dtype == 1) {
    switch (GG) {
      case 8: RTP_SCORE_LAUNCH(f16, 8); break;
      case 4: RTP_SCORE_LAUNCH(f16, 4); break;
      case 2: RTP_SCORE_LAUNCH(f16, 2); break;
      default: RTP_SCORE_LAUNCH(f16, 1); break;
    }
  } else if (k_dtype == 2) {
    switch (GG) {
      case 8: RTP_SCORE_LAUNCH(bf16s, 8); break;
      case 4: RTP_SCORE_LAUNCH(bf16s, 4); break;
      case 2: RTP_SCORE_LAUNCH(bf16s, 2); break;
      default: RTP_SCORE_LAUNCH(bf16s, 1); break;
    }
  } else {
    switch (GG) {
      case 8: RTP_SCORE_LAUNCH(float, 8); break;
      case 4: RTP_SCORE_LAUNCH(float, 4); break;
      case 2: RTP_SCORE_LAUNCH(float, 2); break;
      default: RTP_SCORE_LAUNCH(float, 1); break;
    }
  }
#undef RTP_SCORE_LAUNCH
  return hipGetLastError();
}

static constexpr double kLog2e = 1.4426950408889634;

// With counts, the mass exponent is zero: every token adds exactly 2^24 to its bin and
// the partial holds exact token counts (bins still come from the cells of width w).
hipError_t launch_hist_from_z(const float* z, const int32_t* seq_lens, int B, int H, int Lmax,
                              float bin_width, bool counts, const ChunkGeom& cg,
                              const SelectBufs& sb, hipStream_t st) {
  HeadMap map{};
  dim3 grid(cg.nchunk, H, B);
  const float inv_w = 1.0f / bin_width;
  const float c = counts ? 0.0f : (float)(bin_width * kLog2e);
  const double wm = counts ? 0.0 : (double)bin_width;
  return hist_dispatch_tpt<0, float, 1>(grid, cg, st, z, nullptr, nullptr, seq_lens, map, H, H,
                                        0, 1, Lmax, 1, 0.0f, inv_w, c, wm, sb);
}

hipError_t launch_hist_from_kidx(const float* q_idx, const void* k_idx, int k_dtype,
                                 const int32_t* seq_lens, const HeadMap& map, int B, int Hq,
                                 int Hr, int G, int Lmax, float scale_idx, float bin_width,
                                 bool counts, const ChunkGeom& cg, const SelectBufs& sb,
                                 hipStream_t st) {
  const int GG = pick_gg(G);
  const int ngrp = (G + GG - 1) / GG;
  dim3 grid(cg.nchunk, Hr * ngrp, B);
  const float inv_w = 1.0f / bin_width;
  const float yscale = scale_idx * inv_w;
  const float c = counts ? 0.0f : (float)(bin_width * kLog2e);
  const double wm = counts ? 0.0 : (double)bin_width;
  const int H = Hr * G;
#define RTP_HK(KT, GGV)                                                                        \
  hist_dispatch_tpt<1, KT, GGV>(grid, cg, st, nullptr, q_idx, k_idx, seq_lens, map, H, Hq, Hr, \
                                G, Lmax, ngrp, yscale, inv_w, c, wm, sb)
  if (k_dtype == 1) {
    switch (GG) {
      case 8: return RTP_HK(f16, 8);
      case 4: return RTP_HK(f16, 4);
      case 2: return RTP_HK(f16, 2);
      default: return RTP_HK(f16, 1);
    }
  }
  if (k_dtype == 2) {
    switch (GG) {
      case 8: return RTP_HK(bf16s, 8);
      case 4: return RTP_HK(bf16s, 4);
      case 2: return RTP_HK(bf16s, 2);
      default: return RTP_HK(bf16s, 1);
    }
  }
  switch (GG) {
    case 8: return RTP_HK(float, 8);
    case 4: return RTP_HK(float, 4);
    case 2: return RTP_HK(float, 2);
    default: return RTP_HK(float, 1);
  }
#undef RTP_HK
}

}  // namespace rtp
