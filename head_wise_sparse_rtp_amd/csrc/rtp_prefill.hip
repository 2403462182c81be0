// Prefill of a prompt: causal attention of every prompt position (dense for retrieval
// heads, sliding window plus sinks for local heads), and the decode state the prompt
// leaves (indexer keys of the retrieval heads, their K/V rows, the local heads' rings).
//
// Method: Full Attention Strikes Back (xllm-io.github.io paper review), section 五
// (efficiency evaluation: prefill with local heads windowed and retrieval heads dense;
// test configuration: window 8192, 4 sinks) and section 三, 核心公式 (the indexer
// projection to r = 16 dims before RoPE).
//
// Attention: block (sequence, KV head, tile of 16 query positions), four wavefronts; each
// wavefront takes query heads kv*G + w, w + 4, ... and runs the decode step's MFMA tile
// with the tile's 16 positions as its columns: S^T = K . Q^T over 32 keys per step, an
// online softmax per position, O += P . V, and a per-(key, position) mask for causality
// and the window.  The tile's keys are its sinks followed by one contiguous run ending at
// its last position.  Longer tiles (later positions) are launched first.
#include "rtp_attn_tile.h"

namespace rtp {

namespace {

constexpr int kPQ = 16;  // query positions per tile (the MFMA tile's columns)
constexpr int kPW = 4;   // wavefronts per attention block
constexpr int kPR = 64;  // prompt rows per cache block

__device__ __forceinline__ int clamp_len_p(const int32_t* seq_lens, int b, int Lmax) {
  const int L = seq_lens[b];
  return L < 0 ? 0 : (L > Lmax ? Lmax : L);
}

__global__ __launch_bounds__(kPW * 64, 2) void k_prefill_attn(PrefillArgs A) {
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
  const f16* Kb = A.K + ((size_t)b * A.Hkv + kv) * (size_t)A.Lmax * kD;
  const f16* Vb = A.V + ((size_t)b * A.Hkv + kv) * (size_t)A.Lmax * kD;
  const int lane = threadIdx.x & 63;
  const int wv = threadIdx.x >> 6;
  const int c = lane & 15;
  const int gq = lane >> 4;
  auto key_of = [&](int e) { return e < ns ? e : kstart + (e - ns); };
  for (int g = wv; g < A.G; g += kPW) {
    const int h = kv * A.G + g;
    h8 qop[4];
    load_qop(A.q + ((size_t)(b * A.Hq + h) * A.Lmax + t0) * kD, ncol, qop);
    AttnState st;
    attn_init(st);
    for (int s0 = 0; s0 < nsteps; s0 += 2) {
      const int s1 = s0 + 1;
      const int e0 = s0 * kStep, e1 = s1 * kStep;
      StepLoads ld0, ld1;
      step_load(Kb, Vb, [&](int i) { return key_of(e0 + i < nent ? e0 + i : 0); }, ld0);
      if (s1 < nsteps) step_load(Kb, Vb, [&](int i) { return key_of(e1 + i < nent ? e1 + i : 0); }, ld1);
      auto active = [&](int e, int col) {
        if (e >= nent || col >= ncol) return false;
        const int n = key_of(e), t = t0 + col;
        return n <= t && (ret || n < sinks || n > t - window);
      };
      step_compute(ld0, qop, A.scale2, [&](int i, int col) { return active(e0 + i, col); }, st);
      if (s1 < nsteps)
        step_compute(ld1, qop, A.scale2, [&](int i, int col) { return active(e1 + i, col); }, st);
    }
    // lane (gq, c) holds positions 4gq+t, dims 8c + nb; every position attends to itself,
    // so its sum is positive
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

// Decode state of the prompt: block (sequence, KV head, kPR prompt rows), 256 threads.
// Retrieval heads: k_idx rows = fp32 fma chains over the 128 pre-RoPE inputs in order
// (weights and inputs staged in LDS), rounded to the cache dtype; K/V rows copied.  Local
// heads: rows of the final window set copied to their ring slots.
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
  const f16* Kb = A.K + ((size_t)b * A.Hkv + kv) * (size_t)A.Lmax * kD;
  const f16* Vb = A.V + ((size_t)b * A.Hkv + kv) * (size_t)A.Lmax * kD;
  if (!A.is_ret[kv]) {
    if (!A.K_loc) return;
    const int ring = A.sinks + A.window;
    const int wstart = max(A.sinks, L - A.window);
    f16* Kr = A.K_loc + ((size_t)b * A.Hloc + kr) * (size_t)ring * kD;
    f16* Vr = A.V_loc + ((size_t)b * A.Hloc + kr) * (size_t)ring * kD;
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
    f16* Kd = A.K_ret + ((size_t)b * A.Hret + kr) * (size_t)A.Lmax * kD;
    f16* Vd = A.V_ret + ((size_t)b * A.Hret + kr) * (size_t)A.Lmax * kD;
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
  f16* kd = A.k_idx + (((size_t)b * A.Hret + kr) * A.Lmax + n0) * kR;
  for (int o = tid; o < nr * kR; o += 256) {
    const int rr = o / kR, i = o % kR;
    float a = 0.0f;
#pragma unroll 16
    for (int cc = 0; cc < kD; cc++) a = __builtin_fmaf(xs[rr][cc], ws[cc * kR + i], a);
    kd[(size_t)rr * kR + i] = (f16)a;
  }
}

}  // namespace

hipError_t launch_prefill(const PrefillArgs& a, hipStream_t st) {
  const int nchunk = (a.Lmax + kPR - 1) / kPR;
  if (a.k_idx || a.K_ret || a.K_loc) {
    k_prefill_cache<<<a.B * a.Hkv * nchunk, 256, 0, st>>>(a);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  k_prefill_attn<<<a.B * a.Hkv * a.ntile, kPW * 64, 0, st>>>(a);
  return hipGetLastError();
}

}  // namespace rtp
