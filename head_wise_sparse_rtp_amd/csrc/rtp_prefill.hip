// Prefill of a prompt: causal attention of every prompt position (dense for retrieval
// heads, sliding window plus sinks for local heads), and the decode state the prompt
// leaves (indexer keys of the retrieval heads, their K/V rows, the local heads' rings).
//
// Method: Full Attention Strikes Back (xllm-io.github.io paper review), section 五
// (efficiency evaluation: prefill with local heads windowed and retrieval heads dense;
// test configuration: window 8192, 4 sinks) and section 三, 核心公式 (the indexer
// projection to r = 16 dims before RoPE).
//
// Attention: block (sequence, KV head, tile of 16 query positions), eight wavefronts;
// wavefront w takes query head kv*G + w (then w + 8, ... in further passes) and runs the
// decode step's MFMA tile with the tile's 16 positions as its columns: S^T = K . Q^T over
// 32 keys per step, an online softmax per position, O += P . V, and a per-(key, position)
// mask for causality and the window.  The block stages each step's 32 K and V rows in
// LDS once for all its wavefronts (two buffers, rows padded to 272 bytes; the next step's
// global loads are in flight during this step's MFMAs).  The tile's keys are its sinks
// followed by one contiguous run ending at its last position.  Longer tiles (later
// positions) are launched first.
//
// Both kernels take the element type (fp16 or bf16) as a template parameter.  fp16
// prompts enter P as one fp16 operand; bf16 prompts as a bf16 hi + lo pair (one bf16
// operand would cost up to 2^-9 relative per weight).
#include "rtp_attn_tile.h"

namespace rtp {

namespace {

constexpr int kPQ = 16;  // query positions per tile (the MFMA tile's columns)
constexpr int kPW = 8;   // wavefronts per attention block (query heads of one KV head)
constexpr int kPR = 64;  // prompt rows per cache block

__device__ __forceinline__ int clamp_len_p(const int32_t* seq_lens, int b, int Lmax) {
  const int L = seq_lens[b];
  return L < 0 ? 0 : (L > Lmax ? Lmax : L);
}

constexpr int kKS = kD + 8;  // LDS row stride of a staged K/V tile (elements): 272 bytes

// a value written to a cache of element type T (round to nearest even), as its bits
template <typename T>
__device__ __forceinline__ uint16_t cache_bits(float x);
template <>
__device__ __forceinline__ uint16_t cache_bits<f16>(float x) {
  return __builtin_bit_cast(uint16_t, (f16)x);
}
template <>
__device__ __forceinline__ uint16_t cache_bits<bf16e>(float x) {
  return f_to_bf16(x);
}

// One 32-row step from the staged tile, in the layout of the decode step's tile: the K
// operands first (S^T = K . Q^T), the V operands only after the S MFMAs, so that the two
// are never live together; P enters O += P . V as one fp16 operand (relative error 2^-11
// per weight, against the decode step's hi + lo pair), or as a bf16 hi + lo pair.
template <typename T, class Active>
__device__ __forceinline__ void step_lds(const T* Kl, const T* Vl, const v8<T> (&qop)[4],
                                         float scale2, Active active, AttnState& st) {
  constexpr bool kPair = __is_same(T, bf16e);
  const int lane = threadIdx.x & 63;
  const int c = lane & 15;
  const int gq = lane >> 4;
  f4 s0 = f4{0.0f, 0.0f, 0.0f, 0.0f}, s1 = s0;
#pragma unroll
  for (int s = 0; s < 4; s++) {
    const v8<T> k0 = *reinterpret_cast<const v8<T>*>(Kl + c * kKS + 8 * gq + 32 * s);
    const v8<T> k1 = *reinterpret_cast<const v8<T>*>(Kl + (16 + c) * kKS + 8 * gq + 32 * s);
    s0 = mfma32(k0, qop[s], s0);
    s1 = mfma32(k1, qop[s], s1);
  }
  v8<T> vv[8];
#pragma unroll
  for (int u = 0; u < 8; u++) {
    const int i = (u < 4) ? (4 * gq + u) : (16 + 4 * gq + (u - 4));
    vv[u] = *reinterpret_cast<const v8<T>*>(Vl + i * kKS + 8 * c);
  }
  float sc[8];
#pragma unroll
  for (int t = 0; t < 4; t++) {
    sc[t] = active(4 * gq + t, c) ? s0[t] * scale2 : -INFINITY;
    sc[4 + t] = active(16 + 4 * gq + t, c) ? s1[t] * scale2 : -INFINITY;
  }
  float mx = sc[0];
#pragma unroll
  for (int i = 1; i < 8; i++) mx = fmaxf(mx, sc[i]);
  mx = fmaxf(mx, __shfl_xor(mx, 16, 64));
  mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
  const float mn = fmaxf(st.m, mx);
  const float alpha = (mn == -INFINITY) ? 1.0f : __builtin_amdgcn_exp2f(st.m - mn);
  v8<T> pa, pb;
  float psum = 0.0f;
#pragma unroll
  for (int i = 0; i < 8; i++) {
    const float pv = (sc[i] == -INFINITY) ? 0.0f : __builtin_amdgcn_exp2f(sc[i] - mn);
    psum += pv;
    pa[i] = (T)pv;
    if constexpr (kPair) pb[i] = (T)(pv - (float)pa[i]);
  }
  st.l = st.l * alpha + psum;
  st.m = mn;
  // the output rows need rescaling only when some column's maximum moved
  if (__ballot(alpha != 1.0f) != 0ull) {
    float at[4];
#pragma unroll
    for (int t = 0; t < 4; t++) at[t] = __shfl(alpha, 4 * gq + t, 64);
#pragma unroll
    for (int nb = 0; nb < 8; nb++)
#pragma unroll
      for (int t = 0; t < 4; t++) st.o[nb][t] *= at[t];
  }
#pragma unroll
  for (int nb = 0; nb < 8; nb++) {
    v8<T> vb;
#pragma unroll
    for (int u = 0; u < 8; u++) vb[u] = vv[u][nb];
    st.o[nb] = mfma32(pa, vb, st.o[nb]);
    if constexpr (kPair) st.o[nb] = mfma32(pb, vb, st.o[nb]);
  }
}

template <typename T>
__global__ __launch_bounds__(kPW * 64, 4) void k_prefill_attn(PrefillArgs A) {
  // two buffers of a 32-row K tile and V tile
  __shared__ __align__(16) T kvs[2][2][kStep * kKS];
  const int qt = A.ntile - 1 - (int)(blockIdx.x % A.ntile);
  const int kv = (blockIdx.x / A.ntile) % A.Hkv;
  const int b = blockIdx.x / (A.ntile * A.Hkv);
  const int L = clamp_len_p(A.seq_lens, b, A.Lmax);
  const int t0 = qt * kPQ;
  if (t0 >= L) return;
  const int ncol = min(kPQ, L - t0);
  const int tend = t0 + ncol;
  const bool ret = A.is_ret[kv] != 0;
  const int sinks = A.sinks, window = A.window;
  // entries e < ns are the sink keys e, later entries the keys kstart + (e - ns)
  const int ns = ret ? 0 : min(sinks, tend);
  const int kstart = ret ? 0 : max(ns, t0 + 1 - window);
  const int nent = ns + max(0, tend - kstart);
  const int nsteps = (nent + kStep - 1) / kStep;
  const T* Kb = static_cast<const T*>(A.K) + ((size_t)b * A.Hkv + kv) * (size_t)A.Lmax * kD;
  const T* Vb = static_cast<const T*>(A.V) + ((size_t)b * A.Hkv + kv) * (size_t)A.Lmax * kD;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wv = tid >> 6;
  const int c = lane & 15;
  const int gq = lane >> 4;
  auto key_of = [&](int e) { return e < ns ? e : kstart + (e - ns); };
  // staging: thread tid moves 16 bytes of K and of V: row tid/16, piece tid%16
  const int srow = tid >> 4, spiece = tid & 15;
  auto fetch = [&](int step, u4& kx, u4& vx) {
    const int e = step * kStep + srow;
    const size_t r = (size_t)key_of(e < nent ? e : 0);
    kx = reinterpret_cast<const u4*>(Kb + r * kD)[spiece];
    vx = reinterpret_cast<const u4*>(Vb + r * kD)[spiece];
  };
  auto store = [&](int buf, const u4& kx, const u4& vx) {
    reinterpret_cast<u4*>(&kvs[buf][0][srow * kKS])[spiece] = kx;
    reinterpret_cast<u4*>(&kvs[buf][1][srow * kKS])[spiece] = vx;
  };
  // every wavefront takes one query head per pass; all take part in the staging
  for (int g0 = 0; g0 < A.G; g0 += kPW) {
    const int g = g0 + wv;
    const bool has = g < A.G;
    const int h = kv * A.G + (has ? g : 0);
    v8<T> qop[4];
    load_qop<T>(static_cast<const T*>(A.q) + ((size_t)(b * A.Hq + h) * A.Lmax + t0) * kD,
                has ? ncol : 0, qop);
    AttnState st;
    attn_init(st);
    u4 kx, vx;
    fetch(0, kx, vx);
    store(0, kx, vx);
    __syncthreads();
    for (int s = 0; s < nsteps; s++) {
      const int buf = s & 1;
      if (s + 1 < nsteps) fetch(s + 1, kx, vx);  // in flight during this step's MFMAs
      if (has) {
        const int e0 = s * kStep;
        // a full step: every key exists, lies at or before the tile's first position and
        // (local heads) is a sink or inside every column's window; keys grow with e
        const int ehi = e0 + kStep - 1;
        bool full = ehi < nent && ncol == kPQ && key_of(ehi) <= t0;
        if (!ret && ehi >= ns) full = full && key_of(max(e0, ns)) >= tend - window;
        step_lds(kvs[buf][0], kvs[buf][1], qop, A.scale2,
                 [&](int i, int col) {
                   if (full) return true;
                   const int e = e0 + i;
                   if (e >= nent || col >= ncol) return false;
                   const int n = key_of(e), t = t0 + col;
                   return n <= t && (ret || n < sinks || n > t - window);
                 },
                 st);
      }
      if (s + 1 < nsteps) store(buf ^ 1, kx, vx);
      __syncthreads();
    }
    if (has) {
      // lane (gq, c) holds positions 4gq+t, dims 8c + nb; every position attends to
      // itself, so its sum is positive
      float l = st.l;
      l += __shfl_xor(l, 16, 64);
      l += __shfl_xor(l, 32, 64);
#pragma unroll
      for (int t = 0; t < 4; t++) {
        const int col = 4 * gq + t;
        const float lc = __shfl(l, col, 64);
        if (col < ncol) {
          const float r = 1.0f / lc;
          float4* dst = reinterpret_cast<float4*>(
              A.out + ((size_t)(b * A.Hq + h) * A.Lmax + t0 + col) * kD + 8 * c);
          dst[0] = make_float4(st.o[0][t] * r, st.o[1][t] * r, st.o[2][t] * r, st.o[3][t] * r);
          dst[1] = make_float4(st.o[4][t] * r, st.o[5][t] * r, st.o[6][t] * r, st.o[7][t] * r);
        }
      }
    }
  }
}

// Decode state of the prompt: block (sequence, KV head, kPR prompt rows), 256 threads.
// Retrieval heads: k_idx rows = fp32 fma chains over the 128 pre-RoPE inputs in order
// (weights and inputs staged in LDS), rounded to the cache dtype; K/V rows copied.  Local
// heads: rows of the final window set copied to their ring slots.  Rows move as 16-byte
// pieces of 2-byte elements, whatever their type.
template <typename T>
__global__ __launch_bounds__(256) void k_prefill_cache(PrefillArgs A) {
  __shared__ __align__(16) float ws[kD * kR];
  __shared__ __align__(16) float xs[kPR][kD + 4];
  const int nchunk = (A.Lmax + kPR - 1) / kPR;
  const int ch = blockIdx.x % nchunk;
  const int kv = (blockIdx.x / nchunk) % A.Hkv;
  const int b = blockIdx.x / (nchunk * A.Hkv);
  const int L = clamp_len_p(A.seq_lens, b, A.Lmax);
  const int n0 = ch * kPR;
  if (n0 >= L) return;
  const int nr = min(kPR, L - n0);
  const int tid = threadIdx.x;
  const int kr = A.rank[kv];
  const uint16_t* Kb = static_cast<const uint16_t*>(A.K) + ((size_t)b * A.Hkv + kv) * (size_t)A.Lmax * kD;
  const uint16_t* Vb = static_cast<const uint16_t*>(A.V) + ((size_t)b * A.Hkv + kv) * (size_t)A.Lmax * kD;
  if (!A.is_ret[kv]) {
    if (!A.K_loc) return;
    const int ring = A.sinks + A.window;
    const int wstart = max(A.sinks, L - A.window);
    uint16_t* Kr = static_cast<uint16_t*>(A.K_loc) + ((size_t)b * A.Hloc + kr) * (size_t)ring * kD;
    uint16_t* Vr = static_cast<uint16_t*>(A.V_loc) + ((size_t)b * A.Hloc + kr) * (size_t)ring * kD;
    // 16 threads per row, 16 bytes each
    for (int i = tid; i < nr * 16; i += 256) {
      const int n = n0 + i / 16, p = i % 16;
      if (n >= A.sinks && n < wstart) continue;  // not in the final window set
      const int slot = n < A.sinks ? n : A.sinks + n % A.window;
      reinterpret_cast<u4*>(Kr + (size_t)slot * kD)[p] = reinterpret_cast<const u4*>(Kb + (size_t)n * kD)[p];
      reinterpret_cast<u4*>(Vr + (size_t)slot * kD)[p] = reinterpret_cast<const u4*>(Vb + (size_t)n * kD)[p];
    }
    return;
  }
  if (A.K_ret) {
    uint16_t* Kd = static_cast<uint16_t*>(A.K_ret) + ((size_t)b * A.Hret + kr) * (size_t)A.Lmax * kD;
    uint16_t* Vd = static_cast<uint16_t*>(A.V_ret) + ((size_t)b * A.Hret + kr) * (size_t)A.Lmax * kD;
    for (int i = tid; i < nr * 16; i += 256) {
      const size_t n = n0 + i / 16;
      const int p = i % 16;
      reinterpret_cast<u4*>(Kd + n * kD)[p] = reinterpret_cast<const u4*>(Kb + n * kD)[p];
      reinterpret_cast<u4*>(Vd + n * kD)[p] = reinterpret_cast<const u4*>(Vb + n * kD)[p];
    }
  }
  if (!A.k_idx) return;
  const float* W = A.Wk + (size_t)kr * kD * kR;
  for (int i = tid; i < kD * kR / 4; i += 256)
    reinterpret_cast<float4*>(ws)[i] = reinterpret_cast<const float4*>(W)[i];
  const float* kp = A.k_pre + (((size_t)b * A.Hkv + kv) * A.Lmax + n0) * kD;
  for (int i = tid; i < nr * (kD / 4); i += 256) {
    const int rr = i / (kD / 4), p = i % (kD / 4);
    reinterpret_cast<float4*>(&xs[rr][0])[p] = reinterpret_cast<const float4*>(kp + (size_t)rr * kD)[p];
  }
  __syncthreads();
  uint16_t* kd = static_cast<uint16_t*>(A.k_idx) + (((size_t)b * A.Hret + kr) * A.Lmax + n0) * kR;
  for (int o = tid; o < nr * kR; o += 256) {
    const int rr = o / kR, i = o % kR;
    float a = 0.0f;
#pragma unroll 16
    for (int cc = 0; cc < kD; cc++) a = __builtin_fmaf(xs[rr][cc], ws[cc * kR + i], a);
    kd[(size_t)rr * kR + i] = cache_bits<T>(a);
  }
}

}  // namespace

hipError_t launch_prefill(const PrefillArgs& a, int kv_dtype, hipStream_t st) {
  const int nchunk = (a.Lmax + kPR - 1) / kPR;
  const bool bf = kv_dtype == 2;
  if (a.k_idx || a.K_ret || a.K_loc) {
    if (bf)
      k_prefill_cache<bf16e><<<a.B * a.Hkv * nchunk, 256, 0, st>>>(a);
    else
      k_prefill_cache<f16><<<a.B * a.Hkv * nchunk, 256, 0, st>>>(a);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  if (bf)
    k_prefill_attn<bf16e><<<a.B * a.Hkv * a.ntile, kPW * 64, 0, st>>>(a);
  else
    k_prefill_attn<f16><<<a.B * a.Hkv * a.ntile, kPW * 64, 0, st>>>(a);
  return hipGetLastError();
}

}  // namespace rtp
