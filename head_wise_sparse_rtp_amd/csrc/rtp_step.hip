// Decode step for fp16 caches in four launches per layer.
//
//   K1 stage A  indexer-score/histogram blocks (retrieval KV heads) and window-attention
//               blocks (local KV heads) in one grid; both write partial results.
//   K2 stage T  threshold sums: per (head, range of 32 chunks) the suffix sums of the
//               chunk histograms are shifted to the head's top cell and added; extra
//               blocks merge the window partials into the local heads' outputs.
//   K3 stage B  per (retrieval KV head, 8192-token slice): find b* from the range sums
//               (coarse then fine search over the 256 bins), select the tokens whose bin
//               is within the threshold, gather the K/V rows of the union over the query
//               heads and run masked softmax attention on the matrix cores.
//   K4 stage M  merge the slice partials of every retrieval query head.
// Blocks of one launch never wait for or read each other's results: on gfx950 a
// device-scope release fence writes back and invalidates the whole L2 of the XCD, so
// cross-block hand-offs go through kernel boundaries instead.
//
// Method: Full Attention Strikes Back (xllm-io.github.io paper review), section 三:
// the indexer score and sparse-attention equations (核心公式) and the sort-free 256-bin
// histogram top-p (硬件感知解码内核); section 五 (test configuration) for the window
// of local heads.  The pages' kernels target another GPU; the tiling here is for
// 64-wide wavefronts and 16x16x32 fp16 MFMA on gfx950.
//
// Attention tile (one wavefront, 32 cache rows):
//   S^T = K_tile (32 x 128) . Q^T (128 x 16 heads) as two 16-row tiles of 4 MFMAs; the
//   accumulator layout gives lane l the logits of head l%16 for rows 4*(l/16)+t,
//   which is exactly the A-operand layout of P for O += P . V (8 MFMAs, one per 16
//   output columns).  Output column c of MFMA nb holds head-dim 8*c + nb, so each lane
//   loads 16 contiguous bytes of each V row it needs.
#include "rtp_internal.h"

#include <algorithm>

namespace rtp {

namespace {

typedef _Float16 h8 __attribute__((ext_vector_type(8)));
typedef float f4 __attribute__((ext_vector_type(4)));

constexpr int kAttnG = 16;        // head columns of the MFMA tile
constexpr int kStep = 32;         // cache rows per wavefront step
constexpr int kWinRows = 128;     // window rows per window block (4 waves x 1 step)
constexpr int kBChunks = 4;       // histogram chunks per stage-B block
constexpr int kBGroup = 16;       // stage-B blocks merged per first-level group

__device__ __forceinline__ f4 mfma32(h8 a, h8 b, f4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ int clamp_len(const int32_t* seq_lens, int b, int Lmax) {
  int L = seq_lens[b];
  return L < 0 ? 0 : (L > Lmax ? Lmax : L);
}

// ---------------------------------------------------------------------------
// MFMA attention engine
// ---------------------------------------------------------------------------
struct AttnState {
  float m;     // running max (base-2 logits) of head lane%16
  float l;     // this lane's share of sum 2^(s - m) for head lane%16
  f4 o[8];     // o[nb][t]: head 4*(lane/16)+t, dim 8*(lane%16)+nb
};

__device__ __forceinline__ void attn_init(AttnState& s) {
  s.m = -INFINITY;
  s.l = 0.0f;
#pragma unroll
  for (int nb = 0; nb < 8; nb++) s.o[nb] = f4{0.0f, 0.0f, 0.0f, 0.0f};
}

// B operand of S^T = K . Q^T: head lane%16, dims 32*(lane/16) + 8*s + {0..7}
__device__ __forceinline__ void load_qop(const f16* __restrict__ qhead0, int G, h8 (&qop)[4]) {
  const int lane = threadIdx.x & 63;
  const int h = lane & 15;
  const int gq = lane >> 4;
  if (h < G) {
    const h8* p = reinterpret_cast<const h8*>(qhead0 + (size_t)h * kD + 32 * gq);
#pragma unroll
    for (int s = 0; s < 4; s++) qop[s] = p[s];
  } else {
#pragma unroll
    for (int s = 0; s < 4; s++) qop[s] = h8{0, 0, 0, 0, 0, 0, 0, 0};
  }
}

struct StepLoads {
  h8 k[2][4];  // [tile][s]: K row (tile*16 + lane%16), dims 32*gq + 8*s ..
  h8 v[8];     // [u]: V row of k-slot u (u<4: tile0 row 4gq+u; else tile1 row 4gq+u-4)
};

// rows[i] for i in 0..31 supplied through `row_of(i)` (already clamped to a valid row)
template <class RowOf>
__device__ __forceinline__ void step_load(const f16* __restrict__ Kb, const f16* __restrict__ Vb,
                                          RowOf row_of, StepLoads& ld) {
  const int lane = threadIdx.x & 63;
  const int c = lane & 15;
  const int gq = lane >> 4;
#pragma unroll
  for (int t = 0; t < 2; t++) {
    const int r = row_of(t * 16 + c);
    const h8* p = reinterpret_cast<const h8*>(Kb + (size_t)r * kD + 32 * gq);
#pragma unroll
    for (int s = 0; s < 4; s++) ld.k[t][s] = p[s];
  }
#pragma unroll
  for (int u = 0; u < 8; u++) {
    const int i = (u < 4) ? (4 * gq + u) : (16 + 4 * gq + (u - 4));
    const int r = row_of(i);
    ld.v[u] = *reinterpret_cast<const h8*>(Vb + (size_t)r * kD + 8 * c);
  }
}

// One step over 32 rows.  active(i, h) says whether row i takes part for head h
// (rows past the end and unselected rows are masked to -inf).
template <class Active>
__device__ __forceinline__ void step_compute(const StepLoads& ld, const h8 (&qop)[4], float scale2,
                                             Active active, AttnState& st) {
  const int lane = threadIdx.x & 63;
  const int h = lane & 15;
  const int gq = lane >> 4;
  f4 s0 = f4{0.0f, 0.0f, 0.0f, 0.0f}, s1 = s0;
#pragma unroll
  for (int s = 0; s < 4; s++) {
    s0 = mfma32(ld.k[0][s], qop[s], s0);
    s1 = mfma32(ld.k[1][s], qop[s], s1);
  }
  float sc[8];
#pragma unroll
  for (int t = 0; t < 4; t++) {
    sc[t] = active(4 * gq + t, h) ? s0[t] * scale2 : -INFINITY;
    sc[4 + t] = active(16 + 4 * gq + t, h) ? s1[t] * scale2 : -INFINITY;
  }
  float mx = sc[0];
#pragma unroll
  for (int i = 1; i < 8; i++) mx = fmaxf(mx, sc[i]);
  mx = fmaxf(mx, __shfl_xor(mx, 16, 64));
  mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
  const float mn = fmaxf(st.m, mx);
  const float alpha = (mn == -INFINITY) ? 1.0f : __builtin_amdgcn_exp2f(st.m - mn);
  // P = hi + lo in fp16 keeps the weights at about fp32 accuracy through the fp16 MFMA
  h8 pa, pb;
  float psum = 0.0f;
#pragma unroll
  for (int i = 0; i < 8; i++) {
    const float pv = (sc[i] == -INFINITY) ? 0.0f : __builtin_amdgcn_exp2f(sc[i] - mn);
    psum += pv;
    const f16 hi = (f16)pv;
    pa[i] = hi;
    pb[i] = (f16)(pv - (float)hi);
  }
  st.l = st.l * alpha + psum;
  st.m = mn;
  // rescale the output rows (heads 4gq+t) by their heads' alpha
  float at[4];
#pragma unroll
  for (int t = 0; t < 4; t++) at[t] = __shfl(alpha, 4 * gq + t, 64);
#pragma unroll
  for (int nb = 0; nb < 8; nb++) {
#pragma unroll
    for (int t = 0; t < 4; t++) st.o[nb][t] *= at[t];
  }
#pragma unroll
  for (int nb = 0; nb < 8; nb++) {
    h8 vb;
#pragma unroll
    for (int u = 0; u < 8; u++) vb[u] = ld.v[u][nb];
    st.o[nb] = mfma32(pa, vb, st.o[nb]);
    st.o[nb] = mfma32(pb, vb, st.o[nb]);
  }
}

// Combine the NWV wavefronts of a block into per-head partials (unnormalised), written
// to out_m/out_l/out_acc for heads < G.  Waves pass through LDS four at a time;
// lds >= 4*(32+2048) floats.
template <int NWV>
__device__ void block_combine(AttnState& st, int G, float* lds, float* out_m, float* out_l,
                              float* out_acc) {
  const int lane = threadIdx.x & 63;
  const int wv = threadIdx.x >> 6;
  const int h = lane & 15;
  const int gq = lane >> 4;
  float l = st.l;
  l += __shfl_xor(l, 16, 64);
  l += __shfl_xor(l, 32, 64);
  // item of this thread (threads 0..255): head th, dims d0..d0+7
  const int th = threadIdx.x >> 4;
  const int d0 = (threadIdx.x & 15) * 8;
  const bool item = threadIdx.x < 256 && th < G;
  float M = -INFINITY, L = 0.0f, a[8] = {0, 0, 0, 0, 0, 0, 0, 0};
  for (int wg = 0; wg < (NWV + 3) / 4; wg++) {
    if (wv / 4 == wg) {
      float* wm = lds + (wv % 4) * (32 + 2048);
      float* wl = wm + 16;
      float* wacc = wm + 32;
      if (lane < 16) {
        wm[h] = st.m;
        wl[h] = l;
      }
#pragma unroll
      for (int nb = 0; nb < 8; nb++) {
#pragma unroll
        for (int t = 0; t < 4; t++) wacc[(4 * gq + t) * kD + 8 * h + nb] = st.o[nb][t];
      }
    }
    __syncthreads();
    if (item) {
      const int nw = min(4, NWV - 4 * wg);
      float Mn = M;
      for (int w = 0; w < nw; w++) Mn = fmaxf(Mn, lds[w * (32 + 2048) + th]);
      if (Mn != -INFINITY) {
        const float fo = (M == -INFINITY) ? 0.0f : __builtin_amdgcn_exp2f(M - Mn);
        L *= fo;
#pragma unroll
        for (int i = 0; i < 8; i++) a[i] *= fo;
        for (int w = 0; w < nw; w++) {
          const float* base = lds + w * (32 + 2048);
          const float mw = base[th];
          if (mw == -INFINITY) continue;
          const float f = __builtin_amdgcn_exp2f(mw - Mn);
          L += base[16 + th] * f;
#pragma unroll
          for (int i = 0; i < 8; i++) a[i] += base[32 + th * kD + d0 + i] * f;
        }
        M = Mn;
      }
    }
    __syncthreads();
  }
  if (item) {
    if (d0 == 0) {
      out_m[th] = M;
      out_l[th] = L;
    }
    float4* dst = reinterpret_cast<float4*>(out_acc + th * kD + d0);
    dst[0] = make_float4(a[0], a[1], a[2], a[3]);
    dst[1] = make_float4(a[4], a[5], a[6], a[7]);
  }
}

// Merge the n split partials of one head g (pm/pl [n][G], pacc [n][G][128], optional
// per-split counts) into out / lse / count.  Block of 256 threads: 32 dim-groups of 4
// x 8 split subsets; every load of a thread is issued before any is used; the sums run
// in a fixed order, so the result is deterministic.
__device__ void merge_head(const float* __restrict__ pm, const float* __restrict__ pl,
                           const float* __restrict__ pacc, const int32_t* __restrict__ pcnt,
                           int n, int G, int g, float* __restrict__ out, float* __restrict__ lse,
                           int32_t* __restrict__ count_out, size_t orow, float* lds) {
  float* wk = lds;                         // [n] weights 2^(m_k - M)
  float* red = lds + n;                    // [256]
  float* racc = red + kThreads;            // [8][128]
  const int tid = threadIdx.x;
  float mloc = -INFINITY;
  for (int k = tid; k < n; k += kThreads) {
    const float m = pm[(size_t)k * G + g];
    wk[k] = m;
    mloc = fmaxf(mloc, m);
  }
  red[tid] = mloc;
  __syncthreads();
  for (int s = kThreads / 2; s > 0; s >>= 1) {
    if (tid < s) red[tid] = fmaxf(red[tid], red[tid + s]);
    __syncthreads();
  }
  const float M = red[0];
  __syncthreads();
  float lloc = 0.0f;
  int cloc = 0;
  for (int k = tid; k < n; k += kThreads) {
    const float m = wk[k];
    const float f = (m == -INFINITY) ? 0.0f : __builtin_amdgcn_exp2f(m - M);
    wk[k] = f;
    lloc += pl[(size_t)k * G + g] * f;
    if (pcnt) cloc += pcnt[(size_t)k * G + g];
  }
  red[tid] = lloc;
  __syncthreads();
  for (int s = kThreads / 2; s > 0; s >>= 1) {
    if (tid < s) red[tid] += red[tid + s];
    __syncthreads();
  }
  const float Lsum = red[0];
  __syncthreads();
  if (count_out) {
    int* ired = reinterpret_cast<int*>(red);
    ired[tid] = cloc;
    __syncthreads();
    for (int s = kThreads / 2; s > 0; s >>= 1) {
      if (tid < s) ired[tid] += ired[tid + s];
      __syncthreads();
    }
    if (tid == 0) count_out[orow] = ired[0];
    __syncthreads();
  }
  const int dg = tid & 31;
  const int sub = tid >> 5;
  float4 a = make_float4(0.f, 0.f, 0.f, 0.f);
  for (int k0 = sub; k0 < n; k0 += 8 * 8) {
    float4 x[8];
#pragma unroll
    for (int u = 0; u < 8; u++) {
      const int k = min(k0 + 8 * u, n - 1);
      x[u] = reinterpret_cast<const float4*>(pacc + ((size_t)k * G + g) * kD)[dg];
    }
#pragma unroll
    for (int u = 0; u < 8; u++) {
      const float f = (k0 + 8 * u < n) ? wk[k0 + 8 * u] : 0.0f;
      a.x += x[u].x * f; a.y += x[u].y * f; a.z += x[u].z * f; a.w += x[u].w * f;
    }
  }
  reinterpret_cast<float4*>(racc + sub * kD)[dg] = a;
  __syncthreads();
  if (tid < kD) {
    float v = 0.0f;
#pragma unroll
    for (int s2 = 0; s2 < 8; s2++) v += racc[s2 * kD + tid];
    out[orow * kD + tid] = Lsum > 0.0f ? v / Lsum : 0.0f;
  }
  if (tid == 0 && lse) lse[orow] = Lsum > 0.0f ? (M + __log2f(Lsum)) * 0.69314718055994531f : -INFINITY;
}

// ---------------------------------------------------------------------------
// histogram block (retrieval): same arithmetic as the chunk-histogram kernel of
// rtp_score.hip, followed by suffix sums of the bin masses.
// ---------------------------------------------------------------------------
constexpr int kCopies = 2;
constexpr int kPad = 1;

struct StageAParams {
  const int32_t* seq_lens;
  int B, Hq, G, Lmax;
  const float* q_idx;
  const f16* k_idx;
  HeadMap ret;
  int Hret, nchunk, ngg;
  float yscale, c_log2;
  double w;
  float* suf;
  int32_t* partA;
  uint32_t* codes;
};

struct WinParams {
  const int32_t* seq_lens;
  int Hq, G;
  const f16* q;
  const f16* K_loc;
  const f16* V_loc;
  HeadMap loc;
  int Hloc, window, sinks, nws;
  float scale2;
  float* wpm;
  float* wpl;
  float* wpacc;
};

// Token t (0..3) of thread tid in a chunk is chunk*TC + t*NT + tid; the 4 bin codes of a
// thread are packed into code word `tid` of the chunk (byte t).
template <int GG, int NT>
__device__ void hist_block(const StageAParams& P, int hb, unsigned char* smem) {
  constexpr int TPT = 4;
  constexpr int TC = NT * TPT;
  constexpr int NWV = NT / 64;
  unsigned long long* hist = reinterpret_cast<unsigned long long*>(smem);
  float* smax = reinterpret_cast<float*>(smem + sizeof(unsigned long long) * kCopies * GG * (kNB + kPad));
  float* sq = smax + GG * NWV;  // q_idx of the GG heads, [GG][16]
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wv = tid >> 6;
  const int chunk = hb % P.nchunk;
  const int grp = (hb / P.nchunk) % P.ngg;
  const int kr = (hb / (P.nchunk * P.ngg)) % P.Hret;
  const int b = hb / (P.nchunk * P.ngg * P.Hret);
  const int G = P.G;
  const int g0 = grp * GG;
  const int nrows = min(GG, G - g0);
  const int H = P.Hret * G;
  const size_t rowb = (size_t)b * H + (size_t)kr * G + g0;
  const int L = clamp_len(P.seq_lens, b, P.Lmax);
  const int base = chunk * TC;
  if (base >= L) {
    if (tid < nrows) P.partA[(rowb + tid) * P.nchunk + chunk] = kEmptyCell;
    return;
  }
  const bool full = base + TC <= L;
  // k_idx rows of this thread's tokens, all loads in flight
  const f16* kb = P.k_idx + ((size_t)b * P.Hret + kr) * (size_t)P.Lmax * kR;
  h8 ra[TPT], rb[TPT];
#pragma unroll
  for (int t = 0; t < TPT; t++) {
    int n = base + t * NT + tid;
    n = n < L ? n : base;  // past the end: re-read a valid row, masked below
    const h8* p = reinterpret_cast<const h8*>(kb + (size_t)n * kR);
    ra[t] = p[0];
    rb[t] = p[1];
  }
  if (tid < GG * kR) {
    const int gg = tid / kR;
    sq[tid] = gg < nrows ? P.q_idx[((size_t)b * P.Hq + (size_t)P.ret.kv[kr] * G + g0 + gg) * kR +
                                   (tid % kR)]
                         : 0.0f;
  }
  for (int i = tid; i < kCopies * GG * (kNB + kPad); i += NT) hist[i] = 0ull;
  __syncthreads();

  // ---- pass 1: y = fl32(a * scale) / w (exact: w is a power of two) and the top cell
  float y[TPT][GG];
#pragma unroll
  for (int gg = 0; gg < GG; gg++) {
    float q[kR];
#pragma unroll
    for (int i = 0; i < kR; i++) q[i] = sq[gg * kR + i];
    float ym = -INFINITY;
#pragma unroll
    for (int t = 0; t < TPT; t++) {
      float a = 0.0f;
#pragma unroll
      for (int i = 0; i < 8; i++) a = __builtin_fmaf(q[i], (float)ra[t][i], a);
#pragma unroll
      for (int i = 0; i < 8; i++) a = __builtin_fmaf(q[8 + i], (float)rb[t][i], a);
      float v = a * P.yscale;
      if (!full && base + t * NT + tid >= L) v = -INFINITY;
      y[t][gg] = v;
      ym = fmaxf(ym, v);
    }
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) ym = fmaxf(ym, __shfl_xor(ym, o, 64));
    if (lane == 0) smax[gg * NWV + wv] = ym;
  }
  __syncthreads();
  float Acf[GG];
#pragma unroll
  for (int gg = 0; gg < GG; gg++) {
    float m = smax[gg * NWV];
#pragma unroll
    for (int k = 1; k < NWV; k++) m = fmaxf(m, smax[gg * NWV + k]);
    Acf[gg] = floorf(m);
  }

  // ---- pass 2: exact per-bin sums of x * 2^24, x = exp(z - (g+1) w), and the bin codes
  const int copy = lane & (kCopies - 1);
  const float c = P.c_log2;
  unsigned long long* hrow = hist + copy * GG * (kNB + kPad);
#pragma unroll
  for (int gg = 0; gg < GG; gg++) {
    if (gg >= nrows) break;
    uint32_t cw = 0u;
#pragma unroll
    for (int t = 0; t < TPT; t++) {
      const float yv = y[t][gg];
      const bool valid = full || (base + t * NT + tid < L);
      const float gf = floorf(yv);
      const float diff = Acf[gg] - gf;          // exact: integral and below 2^24
      const float jf = fminf(diff, 255.0f);
      float arg = __builtin_fmaf(__builtin_amdgcn_fractf(yv), c, -c);
      if (diff > 255.0f) arg = __builtin_fmaf(-(diff - 255.0f), c, arg);  // deep tail
      const float e = __builtin_amdgcn_exp2f(arg) * 16777216.0f;
      const uint32_t j = valid ? (uint32_t)jf : 255u;
      const uint32_t xi = valid ? (uint32_t)e : 0u;
      atomicAdd(&hrow[gg * (kNB + kPad) + j], (unsigned long long)xi);
      cw |= j << (8 * t);
    }
    P.codes[((rowb + gg) * P.nchunk + chunk) * (size_t)(TC / 4) + tid] = cw;
  }
  __syncthreads();
  // suffix sums of the bin masses, one head per wavefront pass: lane k owns bins 4k..4k+3
  for (int gg = wv; gg < nrows; gg += NWV) {
    double mloc[4];
#pragma unroll
    for (int u = 0; u < 4; u++) {
      const int j = 4 * lane + u;
      unsigned long long sum = 0ull;
#pragma unroll
      for (int cp = 0; cp < kCopies; cp++) sum += hist[(cp * GG + gg) * (kNB + kPad) + j];
      mloc[u] = (double)sum * 5.9604644775390625e-08 * exp(-(double)j * P.w);
    }
    const double part = mloc[0] + mloc[1] + mloc[2] + mloc[3];
    double sc = part;  // inclusive suffix scan over lanes
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
      const double oth = __shfl_down(sc, o, 64);
      if (lane + o < 64) sc += oth;
    }
    double acc = sc - part;
    float* dst = P.suf + ((rowb + gg) * P.nchunk + chunk) * kNB;
    float4 outv;
    acc += mloc[3]; outv.w = (float)acc;
    acc += mloc[2]; outv.z = (float)acc;
    acc += mloc[1]; outv.y = (float)acc;
    acc += mloc[0]; outv.x = (float)acc;
    reinterpret_cast<float4*>(dst)[lane] = outv;
    if (lane == 0) {
      float m = smax[gg * NWV];
      for (int k = 1; k < NWV; k++) m = fmaxf(m, smax[gg * NWV + k]);
      P.partA[(rowb + gg) * P.nchunk + chunk] = (int)floorf(m);
    }
  }
}

// ---------------------------------------------------------------------------
// window block (local): 4 wavefronts x 32 entries of the window set -> one partial
// ---------------------------------------------------------------------------
__device__ void window_block(const WinParams& P, int wb, float* lds) {
  const int wsplit = wb % P.nws;
  const int kl = (wb / P.nws) % P.Hloc;
  const int b = wb / (P.nws * P.Hloc);
  const int G = P.G;
  const int ring = P.sinks + P.window;
  int L = P.seq_lens[b];
  L = L < 0 ? 0 : L;
  const int ns = min(P.sinks, L);
  const int wstart = max(P.sinks, L - P.window);
  const int nwin = ns + max(0, L - wstart);
  const int wv = threadIdx.x >> 6;
  const f16* Kb = P.K_loc + ((size_t)b * P.Hloc + kl) * (size_t)ring * kD;
  const f16* Vb = P.V_loc + ((size_t)b * P.Hloc + kl) * (size_t)ring * kD;
  h8 qop[4];
  load_qop(P.q + ((size_t)b * P.Hq + (size_t)P.loc.kv[kl] * G) * kD, G, qop);
  AttnState st;
  attn_init(st);
  const int e0 = wsplit * kWinRows + wv * kStep;
  const int sinks = P.sinks, window = P.window;
  auto slot_of = [&](int e) {
    e = e < nwin ? e : 0;  // rows past the end read entry 0 (masked below)
    const int pos = e < ns ? e : wstart + (e - ns);
    return pos < sinks ? pos : sinks + pos % window;
  };
  if (nwin > 0 && e0 < nwin) {
    StepLoads ld;
    step_load(Kb, Vb, [&](int i) { return slot_of(e0 + i); }, ld);
    step_compute(ld, qop, P.scale2, [&](int i, int h) { return e0 + i < nwin; }, st);
  }
  const size_t prow = ((size_t)(b * P.Hloc + kl) * P.nws + wsplit) * G;
  block_combine<kThreads / 64>(st, G, lds, P.wpm + prow, P.wpl + prow, P.wpacc + prow * kD);
}

template <int GG, int NT>
__global__ __launch_bounds__(NT, 2) void k_stage_a(StageAParams P) {
  extern __shared__ __align__(16) unsigned char smem[];
  hist_block<GG, NT>(P, blockIdx.x, smem);
}

// ---------------------------------------------------------------------------
// stage T: threshold range sums (block (range, row), thread = global bin J):
//   SUF_J(range) = sum_{c in range} suf_c[max(J - s_c, 0)] * exp(-s_c w),  s_c = A - A_c
// over 32 chunks (coalesced: lanes read consecutive bins of one chunk).
// ---------------------------------------------------------------------------
constexpr int kTRange = 32;  // chunks per stage-T block

struct StageTParams {
  const float* suf;
  const int32_t* partA;
  int nchunk, nrange;
  float c_log2;
  double* tpart;
  int32_t* Aglob;
};

__global__ __launch_bounds__(kThreads) void k_stage_t(StageTParams P) {
  __shared__ int sAi[kThreads / 64];
  __shared__ int sAc[kTRange];
  const int row = blockIdx.x / P.nrange;
  const int rg = blockIdx.x % P.nrange;
  const int J = threadIdx.x;
  const int lane = J & 63;
  const int wv = J >> 6;
  const int32_t* pa = P.partA + (size_t)row * P.nchunk;
  int A = kEmptyCell;
  for (int c = J; c < P.nchunk; c += kThreads) A = max(A, pa[c]);
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) A = max(A, __shfl_xor(A, o, 64));
  if (lane == 0) sAi[wv] = A;
  const int c0 = rg * kTRange;
  const int nc = min(kTRange, P.nchunk - c0);
  if (J < nc) sAc[J] = pa[c0 + J];
  __syncthreads();
  A = max(max(sAi[0], sAi[1]), max(sAi[2], sAi[3]));
  double acc = 0.0;
  if (A != kEmptyCell) {
    float x[kTRange];
    float f[kTRange];
#pragma unroll
    for (int i = 0; i < kTRange; i++) {
      const int Ac = i < nc ? sAc[i] : kEmptyCell;
      const long long s = (Ac == kEmptyCell) ? (1ll << 40) : (long long)A - (long long)Ac;
      f[i] = s > 4096 ? 0.0f : __builtin_amdgcn_exp2f(-(float)s * P.c_log2);
      const int jj = s > 4096 ? 0 : max(J - (int)s, 0);
      x[i] = P.suf[((size_t)row * P.nchunk + c0 + (i < nc ? i : 0)) * kNB + jj];
    }
#pragma unroll
    for (int i = 0; i < kTRange; i++) acc += (double)x[i] * (double)f[i];
  }
  P.tpart[((size_t)row * P.nrange + rg) * kNB + J] = acc;
  if (rg == 0 && J == 0) P.Aglob[row] = A;
}

// ---------------------------------------------------------------------------
// stage B: threshold search + selection + masked MFMA attention over the union of the
// selected rows of a retrieval KV head within an 8192-token slice -> one partial
// ---------------------------------------------------------------------------
struct StageBParams {
  const int32_t* seq_lens;
  int B, Hq, G, Lmax, Hret, nchunk, tc, nblk, nrange;
  double p;
  const f16* q;
  const f16* K_ret;
  const f16* V_ret;
  HeadMap ret;
  float scale2;
  const int32_t* partA;
  const uint32_t* codes;
  const double* tpart;
  const int32_t* Aglob;
  int32_t* bstar;
  float* p1m;
  float* p1l;
  float* p1acc;
  int32_t* p1cnt;
  int want_count;
  int nret_blocks;  // blocks past this index run window attention
  WinParams win;
};

// sum over the ranges of SUF_J for head row `row` (fixed order)
__device__ __forceinline__ double suf_at(const double* __restrict__ tpart, size_t row, int nrange,
                                         int J) {
  if (J >= kNB) return 0.0;
  double s = 0.0;
  for (int r0 = 0; r0 < nrange; r0 += 8) {
    double y[8];
#pragma unroll
    for (int u = 0; u < 8; u++)
      y[u] = r0 + u < nrange ? tpart[(row * nrange + r0 + u) * kNB + J] : 0.0;
#pragma unroll
    for (int u = 0; u < 8; u++) s += y[u];
  }
  return s;
}

// Code word w of a chunk holds the bins of tokens w + q*(TC/4), q = 0..3 (byte q).  Thread
// tid of this kernel takes words tid + i*256, i < NW, i.e. TPT = 4*NW tokens per chunk.
template <int TPT, int GMAX>
__device__ void select_attend_block(const StageBParams& P, unsigned char* smem);

template <int TPT, int GMAX>
__global__ __launch_bounds__(kThreads) void k_stage_b(StageBParams P) {
  extern __shared__ __align__(16) unsigned char smem[];
  if ((int)blockIdx.x < P.nret_blocks)
    select_attend_block<TPT, GMAX>(P, smem);
  else
    window_block(P.win, blockIdx.x - P.nret_blocks, reinterpret_cast<float*>(smem));
}

template <int TPT, int GMAX>
__device__ void select_attend_block(const StageBParams& P, unsigned char* smem) {
  constexpr int TC = kThreads * TPT;
  constexpr int NW = TPT / 4;  // code words per thread per chunk and head
  auto tok_of = [&](int chunk, int t) {  // t = 4*i + q
    return chunk * TC + (threadIdx.x + (t >> 2) * kThreads) + (t & 3) * (TC / 4);
  };
  __shared__ int s_tau[kBChunks][kAttnG];
  __shared__ int s_A[kAttnG], s_bs[kAttnG], s_m[kAttnG];
  __shared__ double s_suf[kAttnG][17];
  __shared__ int s_wsum[kThreads / 64];
  __shared__ int s_cnt[kAttnG];
  int32_t* ltok = reinterpret_cast<int32_t*>(smem);
  uint16_t* lmask = reinterpret_cast<uint16_t*>(smem + sizeof(int32_t) * kBChunks * TC);
  float* lds = reinterpret_cast<float*>(smem);

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wv = tid >> 6;
  const int blk = blockIdx.x % P.nblk;
  const int kr = (blockIdx.x / P.nblk) % P.Hret;
  const int b = blockIdx.x / (P.nblk * P.Hret);
  const int G = P.G;
  const int H = P.Hret * G;
  const size_t row0 = (size_t)b * H + (size_t)kr * G;
  const int L = clamp_len(P.seq_lens, b, P.Lmax);
  const int chunk0 = blk * kBChunks;
  const f16* Kb = P.K_ret + ((size_t)b * P.Hret + kr) * (size_t)P.Lmax * kD;
  const f16* Vb = P.V_ret + ((size_t)b * P.Hret + kr) * (size_t)P.Lmax * kD;

  // ---- phase 0: inputs of the selection; the code words do not depend on b*, so all of
  // them are in flight while b* is searched
  h8 qop[4];
  load_qop(P.q + ((size_t)b * P.Hq + (size_t)P.ret.kv[kr] * G) * kD, G, qop);
  uint32_t cw[kBChunks][GMAX][NW];
#pragma unroll
  for (int c = 0; c < kBChunks; c++) {
    const int chunk = min(chunk0 + c, P.nchunk - 1);
#pragma unroll
    for (int g = 0; g < GMAX; g++) {
      const int gg = g < G ? g : 0;
      const uint32_t* cp = P.codes + ((row0 + gg) * P.nchunk + chunk) * (size_t)(TC / 4) + tid;
#pragma unroll
      for (int w = 0; w < NW; w++) cw[c][g][w] = cp[w * kThreads];
    }
  }
  if (tid < kBChunks * kAttnG) {
    const int c = tid / kAttnG, g = tid % kAttnG;
    const int chunk = chunk0 + c;
    s_tau[c][g] = (g < G && chunk < P.nchunk) ? P.partA[(row0 + g) * P.nchunk + chunk] : kEmptyCell;
  }
  if (tid < kAttnG) {
    s_A[tid] = tid < G ? P.Aglob[row0 + tid] : kEmptyCell;
    s_cnt[tid] = 0;
  }
  // coarse search: SUF at bins 16k (k = 0..15); thread (g, k)
  const int sg = tid >> 4, sk = tid & 15;
  if (sg < G && P.p < 1.0) s_suf[sg][sk] = suf_at(P.tpart, row0 + sg, P.nrange, 16 * sk);
  __syncthreads();
  if (tid < kAttnG) {
    int m = 16;  // C_J >= pZ first happens for J in [16(m-1), 16m - 1]
    if (tid < G && P.p < 1.0) {
      const double Z = s_suf[tid][0];
      for (int k = 15; k >= 1; k--)
        if (Z - s_suf[tid][k] >= P.p * Z) m = k;
    }
    s_m[tid] = m;
  }
  __syncthreads();
  // fine search: SUF_{J+1} for J in [16(m-1), 16m-1]
  if (sg < G && P.p < 1.0) {
    const int J1 = 16 * (s_m[sg] - 1) + 1 + sk;
    s_suf[sg][sk + 1] = suf_at(P.tpart, row0 + sg, P.nrange, J1);
  }
  __syncthreads();
  if (tid < kAttnG) {
    int bs = kNB - 1;
    if (tid < G && P.p < 1.0) {
      const double Z = suf_at(P.tpart, row0 + tid, P.nrange, 0);
      const int Jlo = 16 * (s_m[tid] - 1);
      for (int i = 15; i >= 0; i--)
        if (Jlo + i < kNB - 1 && Z - s_suf[tid][i + 1] >= P.p * Z) bs = Jlo + i;
    }
    s_bs[tid] = bs;
    if (blk == 0 && tid < G) P.bstar[row0 + tid] = bs;
  }
  __syncthreads();
  // chunk threshold code tau: tokens with code <= tau are selected (256: all, -1: none)
  int tau = -1;
  if (tid < kBChunks * kAttnG) {
    const int c = tid / kAttnG, g = tid % kAttnG;
    const int Ac = s_tau[c][g];
    const int A = s_A[g];
    const int bs = s_bs[g];
    if (g < G && A != kEmptyCell && Ac != kEmptyCell && (chunk0 + c) * TC < L) {
      if (bs >= kNB - 1) {
        tau = 256;
      } else {
        const long long t = (long long)bs - ((long long)A - (long long)Ac);
        tau = t < 0 ? -1 : (int)t;
      }
    }
  }
  __syncthreads();
  if (tid < kBChunks * kAttnG) s_tau[tid / kAttnG][tid % kAttnG] = tau;
  __syncthreads();

  // ---- phase 1: union of the selected tokens (per-token head masks), compacted in LDS
  uint32_t mk[kBChunks][TPT];
  int mine = 0;
#pragma unroll
  for (int c = 0; c < kBChunks; c++) {
#pragma unroll
    for (int t = 0; t < TPT; t++) mk[c][t] = 0u;
#pragma unroll
    for (int g = 0; g < GMAX; g++) {
      const int tg = s_tau[c][g];
      if (tg < 0) continue;
#pragma unroll
      for (int t = 0; t < TPT; t++) {
        const int code = (cw[c][g][t >> 2] >> (8 * (t & 3))) & 255;
        if (tg == 256 || code <= tg) mk[c][t] |= 1u << g;
      }
    }
#pragma unroll
    for (int t = 0; t < TPT; t++) {
      if (tok_of(chunk0 + c, t) >= L) mk[c][t] = 0u;
      mine += mk[c][t] != 0u;
    }
  }
#pragma unroll
  for (int g = 0; g < GMAX; g++) {
    if (g >= G || !P.want_count) break;
    int cg = 0;
#pragma unroll
    for (int c = 0; c < kBChunks; c++)
#pragma unroll
      for (int t = 0; t < TPT; t++) cg += (mk[c][t] >> g) & 1u;
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) cg += __shfl_xor(cg, o, 64);
    if (lane == 0 && cg) atomicAdd(&s_cnt[g], cg);
  }
  int incl = mine;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int v = __shfl_up(incl, o, 64);
    if (lane >= o) incl += v;
  }
  if (lane == 63) s_wsum[wv] = incl;
  __syncthreads();
  int woff = 0, U = 0;
#pragma unroll
  for (int i = 0; i < kThreads / 64; i++) {
    if (i < wv) woff += s_wsum[i];
    U += s_wsum[i];
  }
  int pos = woff + incl - mine;
#pragma unroll
  for (int c = 0; c < kBChunks; c++) {
#pragma unroll
    for (int t = 0; t < TPT; t++) {
      if (mk[c][t]) {
        ltok[pos] = tok_of(chunk0 + c, t);
        lmask[pos] = (uint16_t)mk[c][t];
        pos++;
      }
    }
  }
  __syncthreads();

  // ---- phase 2: masked MFMA attention over the listed rows; wavefront wv takes steps
  // wv, wv+4, ...; two steps' loads are in flight before the first is used
  AttnState st;
  attn_init(st);
  const int nsteps = (U + kStep - 1) / kStep;
  for (int s0 = wv; s0 < nsteps; s0 += 2 * (kThreads / 64)) {
    const int s1 = s0 + kThreads / 64;
    StepLoads ld0, ld1;
    const int e0 = s0 * kStep, e1 = s1 * kStep;
    step_load(Kb, Vb, [&](int i) { return ltok[e0 + i < U ? e0 + i : 0]; }, ld0);
    if (s1 < nsteps) step_load(Kb, Vb, [&](int i) { return ltok[e1 + i < U ? e1 + i : 0]; }, ld1);
    step_compute(ld0, qop, P.scale2,
                 [&](int i, int h) { return e0 + i < U && ((lmask[e0 + i < U ? e0 + i : 0] >> h) & 1u); },
                 st);
    if (s1 < nsteps)
      step_compute(ld1, qop, P.scale2,
                   [&](int i, int h) { return e1 + i < U && ((lmask[e1 + i < U ? e1 + i : 0] >> h) & 1u); },
                   st);
  }
  __syncthreads();

  // ---- phase 3: block partial
  const size_t s1p = ((size_t)(b * P.Hret + kr) * P.nblk + blk) * G;
  block_combine<kThreads / 64>(st, G, lds, P.p1m + s1p, P.p1l + s1p, P.p1acc + s1p * kD);
  if (tid < G) P.p1cnt[s1p + tid] = s_cnt[tid];
}

// ---------------------------------------------------------------------------
// stage M: merge the slice partials of every retrieval query head, then (blocks past
// them) the window partials of every local query head
// ---------------------------------------------------------------------------
struct StageMParams {
  const float* p1m;
  const float* p1l;
  const float* p1acc;
  const int32_t* p1cnt;
  const int32_t* Aglob;
  const int32_t* bstar;
  int nblk, Hret, G, Hq, nret;
  HeadMap ret;
  // window
  const float* wpm;
  const float* wpl;
  const float* wpacc;
  int nws, Hloc;
  HeadMap loc;
  float* out;
  float* lse;
  int32_t* count_out;
  int32_t* thresh_out;
};

__global__ __launch_bounds__(kThreads) void k_stage_m(StageMParams P) {
  extern __shared__ __align__(16) float mlds[];
  const int G = P.G;
  if ((int)blockIdx.x >= P.nret) {
    const int wm = blockIdx.x - P.nret;
    const int g = wm % G;
    const int kl = (wm / G) % P.Hloc;
    const int b = wm / (G * P.Hloc);
    const size_t p0 = (size_t)(b * P.Hloc + kl) * P.nws * G;
    merge_head(P.wpm + p0, P.wpl + p0, P.wpacc + p0 * kD, nullptr, P.nws, G, g, P.out, P.lse,
               nullptr, (size_t)b * P.Hq + (size_t)P.loc.kv[kl] * G + g, mlds);
    return;
  }
  const int g = blockIdx.x % G;
  const int kr = (blockIdx.x / G) % P.Hret;
  const int b = blockIdx.x / (G * P.Hret);
  const size_t p0 = (size_t)(b * P.Hret + kr) * P.nblk * G;
  const size_t orow = (size_t)b * P.Hq + (size_t)P.ret.kv[kr] * G + g;
  merge_head(P.p1m + p0, P.p1l + p0, P.p1acc + p0 * kD, P.p1cnt + p0, P.nblk, G, g, P.out, P.lse,
             P.count_out, orow, mlds);
  if (P.thresh_out && threadIdx.x == 0) {
    const size_t row = (size_t)b * P.Hret * G + (size_t)kr * G + g;
    const int A = P.Aglob[row];
    P.thresh_out[orow * 2 + 0] = A == kEmptyCell ? 0 : A;
    P.thresh_out[orow * 2 + 1] = A == kEmptyCell ? 0 : P.bstar[row];
  }
}

}  // namespace

// ---------------------------------------------------------------------------
// host side
// ---------------------------------------------------------------------------
bool step_fused_supported(int kv_dtype, int G, int Hloc, int window, int sinks) {
  if (kv_dtype != 1 || G > kAttnG) return false;
  // the window merge keeps one weight per split in LDS
  if (Hloc > 0 && (window + sinks + kWinRows - 1) / kWinRows > 8192) return false;
  return true;
}

StepFusedPlan plan_step_fused(WsPlanner& wp, int B, int Hq, int G, int Lmax, int Hret, int Hloc,
                              int window, int sinks) {
  (void)Hq;
  StepFusedPlan sp{};
  sp.G = G;
  sp.Hret = Hret;
  sp.Hloc = Hloc;
  const int H = Hret * G;
  // 2048-token chunks (stage-A blocks of 512 threads) unless that leaves fewer than 256
  // histogram blocks; then 1024-token chunks (256 threads)
  {
    const int64_t units = (int64_t)B * (Hret > 0 ? Hret : 1);
    sp.tc = units * ((Lmax + 2047) / 2048) >= 256 ? 2048 : 1024;
    sp.nt = sp.tc / 4;
    sp.tpt = sp.tc / kThreads;
  }
  if (Hret > 0) {
    sp.nchunk = (Lmax + sp.tc - 1) / sp.tc;
    sp.nblk = (sp.nchunk + kBChunks - 1) / kBChunks;
    sp.nrange = (sp.nchunk + kTRange - 1) / kTRange;
    sp.suf = wp.take<float>((size_t)B * H * sp.nchunk * kNB);
    sp.partA = wp.take<int32_t>((size_t)B * H * sp.nchunk);
    sp.codes = wp.take<uint32_t>((size_t)B * H * sp.nchunk * (sp.tc / 4));
    sp.bstar = wp.take<int32_t>((size_t)B * H);
    sp.Aglob = wp.take<int32_t>((size_t)B * H);
    sp.tpart = wp.take<double>((size_t)B * H * sp.nrange * kNB);
    const size_t n1 = (size_t)B * Hret * sp.nblk * G;
    sp.p1m = wp.take<float>(n1);
    sp.p1l = wp.take<float>(n1);
    sp.p1acc = wp.take<float>(n1 * kD);
    sp.p1cnt = wp.take<int32_t>(n1);
  }
  if (Hloc > 0) {
    sp.nws = (window + sinks + kWinRows - 1) / kWinRows;
    const size_t nw = (size_t)B * Hloc * sp.nws * G;
    sp.wpm = wp.take<float>(nw);
    sp.wpl = wp.take<float>(nw);
    sp.wpacc = wp.take<float>(nw * kD);
  }
  sp.bytes = (wp.off + 255) & ~size_t(255);
  if (sp.bytes == 0) sp.bytes = 256;
  return sp;
}

template <typename T>
static T* at(char* ws, size_t off) {
  return reinterpret_cast<T*>(ws + off);
}

hipError_t launch_step_fused(const StepFusedPlan& sp, char* ws, const StepFusedArgs& a,
                             hipStream_t st, hipEvent_t* ev) {
  const int G = sp.G;
  const int B = a.B;
  const int H = sp.Hret * G;
  auto rec = [&](int i) {
    if (ev && ev[i]) (void)hipEventRecord(ev[i], st);
  };
  const float scale2 = a.scale_attn * 1.4426950408889634f;
  const float c_log2 = (float)((double)a.bin_width * 1.4426950408889634);
  hipError_t e = hipSuccess;
  rec(0);
  // ---- K1: indexer score + chunk histograms
  StageAParams P{};
  if (sp.Hret > 0) {
    const int GG = G > 4 ? 8 : (G > 2 ? 4 : (G > 1 ? 2 : 1));
    P.seq_lens = a.seq_lens;
    P.B = B;
    P.Hq = a.Hq;
    P.G = G;
    P.Lmax = a.Lmax;
    P.q_idx = a.q_idx;
    P.k_idx = static_cast<const f16*>(a.k_idx);
    P.ret = a.ret;
    P.Hret = sp.Hret;
    P.nchunk = sp.nchunk;
    P.ngg = (G + GG - 1) / GG;
    P.yscale = a.scale_idx / a.bin_width;
    P.c_log2 = c_log2;
    P.w = (double)a.bin_width;
    P.suf = at<float>(ws, sp.suf);
    P.partA = at<int32_t>(ws, sp.partA);
    P.codes = at<uint32_t>(ws, sp.codes);
    const int nA = B * sp.Hret * P.ngg * sp.nchunk;
    const size_t ldsA = sizeof(unsigned long long) * kCopies * 8 * (kNB + kPad) + 1024;
#define RTP_STAGE_A(GGV, NTV) k_stage_a<GGV, NTV><<<nA, NTV, ldsA, st>>>(P)
    if (sp.nt == 256) {
      switch (GG) {
        case 8: RTP_STAGE_A(8, 256); break;
        case 4: RTP_STAGE_A(4, 256); break;
        case 2: RTP_STAGE_A(2, 256); break;
        default: RTP_STAGE_A(1, 256); break;
      }
    } else {
      switch (GG) {
        case 8: RTP_STAGE_A(8, 512); break;
        case 4: RTP_STAGE_A(4, 512); break;
        case 2: RTP_STAGE_A(2, 512); break;
        default: RTP_STAGE_A(1, 512); break;
      }
    }
#undef RTP_STAGE_A
    e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  rec(1);
  // ---- K2: threshold range sums
  StageTParams T{};
  if (sp.Hret > 0) {
    T.suf = P.suf;
    T.partA = P.partA;
    T.nchunk = sp.nchunk;
    T.nrange = sp.nrange;
    T.c_log2 = c_log2;
    T.tpart = at<double>(ws, sp.tpart);
    T.Aglob = at<int32_t>(ws, sp.Aglob);
    k_stage_t<<<B * H * sp.nrange, kThreads, 0, st>>>(T);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  rec(2);
  // ---- K3: selection + sparse attention (retrieval) and window attention (local)
  StageBParams Q{};
  Q.seq_lens = a.seq_lens;
  Q.B = B;
  Q.Hq = a.Hq;
  Q.G = G;
  Q.Lmax = a.Lmax;
  Q.Hret = sp.Hret;
  Q.scale2 = scale2;
  Q.nret_blocks = 0;
  if (sp.Hret > 0) {
    Q.nchunk = sp.nchunk;
    Q.tc = sp.tc;
    Q.nblk = sp.nblk;
    Q.nrange = sp.nrange;
    Q.p = a.p;
    Q.q = static_cast<const f16*>(a.q);
    Q.K_ret = static_cast<const f16*>(a.K_ret);
    Q.V_ret = static_cast<const f16*>(a.V_ret);
    Q.ret = a.ret;
    Q.partA = P.partA;
    Q.codes = P.codes;
    Q.tpart = T.tpart;
    Q.Aglob = T.Aglob;
    Q.bstar = at<int32_t>(ws, sp.bstar);
    Q.p1m = at<float>(ws, sp.p1m);
    Q.p1l = at<float>(ws, sp.p1l);
    Q.p1acc = at<float>(ws, sp.p1acc);
    Q.p1cnt = at<int32_t>(ws, sp.p1cnt);
    Q.want_count = a.count_out != nullptr;
    Q.nret_blocks = B * sp.Hret * sp.nblk;
  }
  int nwin_blocks = 0;
  if (sp.Hloc > 0) {
    WinParams& W = Q.win;
    W.seq_lens = a.seq_lens;
    W.Hq = a.Hq;
    W.G = G;
    W.q = static_cast<const f16*>(a.q);
    W.K_loc = static_cast<const f16*>(a.K_loc);
    W.V_loc = static_cast<const f16*>(a.V_loc);
    W.loc = a.loc;
    W.Hloc = sp.Hloc;
    W.window = a.window;
    W.sinks = a.sinks;
    W.nws = sp.nws;
    W.scale2 = scale2;
    W.wpm = at<float>(ws, sp.wpm);
    W.wpl = at<float>(ws, sp.wpl);
    W.wpacc = at<float>(ws, sp.wpacc);
    nwin_blocks = B * sp.Hloc * sp.nws;
  }
  const size_t ldsB = std::max<size_t>(4 * (32 + 2048) * sizeof(float),
                                       (sizeof(int32_t) + sizeof(uint16_t)) * kBChunks * sp.tc);
  const int nB = Q.nret_blocks + nwin_blocks;
  if (sp.tpt == 4) {
    if (G <= 8)
      k_stage_b<4, 8><<<nB, kThreads, ldsB, st>>>(Q);
    else
      k_stage_b<4, 16><<<nB, kThreads, ldsB, st>>>(Q);
  } else {
    if (G <= 8)
      k_stage_b<8, 8><<<nB, kThreads, ldsB, st>>>(Q);
    else
      k_stage_b<8, 16><<<nB, kThreads, ldsB, st>>>(Q);
  }
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  // ---- K4: merges
  StageMParams M{};
  M.G = G;
  M.Hq = a.Hq;
  M.out = a.out;
  M.lse = a.lse;
  M.nret = sp.Hret > 0 ? B * sp.Hret * G : 0;
  if (sp.Hret > 0) {
    M.p1m = Q.p1m;
    M.p1l = Q.p1l;
    M.p1acc = Q.p1acc;
    M.p1cnt = Q.p1cnt;
    M.Aglob = Q.Aglob;
    M.bstar = Q.bstar;
    M.nblk = sp.nblk;
    M.Hret = sp.Hret;
    M.ret = a.ret;
    M.count_out = a.count_out;
    M.thresh_out = a.thresh_out;
  }
  const int nwm = sp.Hloc > 0 ? B * sp.Hloc * G : 0;
  if (sp.Hloc > 0) {
    M.wpm = Q.win.wpm;
    M.wpl = Q.win.wpl;
    M.wpacc = Q.win.wpacc;
    M.nws = sp.nws;
    M.Hloc = sp.Hloc;
    M.loc = a.loc;
  }
  const int nmax = std::max(sp.Hret > 0 ? sp.nblk : 0, sp.Hloc > 0 ? sp.nws : 0);
  const size_t ldsM = sizeof(float) * ((size_t)nmax + kThreads + 8 * kD);
  k_stage_m<<<M.nret + nwm, kThreads, ldsM, st>>>(M);
  e = hipGetLastError();
  rec(3);
  return e;
}

}  // namespace rtp
