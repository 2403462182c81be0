// Prefill of a prompt: causal attention of every prompt position (dense for retrieval
// heads, sliding window plus sinks for local heads), and the decode state the prompt
// leaves (indexer keys of the retrieval heads, their K/V rows, the local heads' rings).
//
// Method: Full Attention Strikes Back (xllm-io.github.io paper review), section 五
// (efficiency evaluation: prefill with local heads windowed and retrieval heads dense;
// test configuration: window 8192, 4 sinks) and section 三, 核心公式 (the indexer
// projection to r = 16 dims before RoPE).
//
// Attention: block (sequence, KV head, tile of 32 query positions), eight wavefronts;
// wavefront w takes query head kv*G + w (then w + 8, ... in further passes) and runs the
// decode step's MFMA tile twice, with positions t0..t0+15 and t0+16..t0+31 as the columns
// of its two sets: S^T = K . Q^T over 32 keys per step, an online softmax per position,
// O += P . V, and a per-(key, position) mask for causality and the window.  Each K and V
// operand read from LDS serves both sets, which halves the LDS bytes per flop.  The block
// stages 128 keys (bf16: 64) of K and V in LDS per barrier, once for all its wavefronts
// (two buffers, rows padded to 272 bytes; the next stage's global loads are in flight
// during this stage's MFMAs).  The tile's keys are its sinks followed by one contiguous run
// ending at its last position.  Longer tiles (later positions) are launched first.
//
// Both kernels take the element type (fp16 or bf16) as a template parameter.  fp16
// prompts enter P as one fp16 operand; bf16 prompts as a bf16 hi + lo pair (one bf16
// operand would cost up to 2^-9 relative per weight).
#include "rtp_attn_tile.h"

namespace rtp {

namespace {

constexpr int kPQ = 32;  // query positions per tile: two sets of the MFMA tile's 16 columns
constexpr int kPW = 8;   // wavefronts per attention block (query heads of one KV head)
constexpr int kPR = 64;  // prompt rows per cache block

__device__ __forceinline__ int clamp_len_p(const int32_t* seq_lens, int b, int Lmax) {
  const int L = seq_lens[b];
  return L < 0 ? 0 : (L > Lmax ? Lmax : L);
}

constexpr int kKS = kD + 16;  // LDS row stride of a staged K/V tile (elements): 288 bytes
// K/V rows staged per block barrier: 32-row steps per barrier x 32 (fp16: 4, bf16: 2, whose
// weight pairs leave no registers for more staging)
template <typename T>
constexpr int stage_rows() {
  return __is_same(T, bf16e) ? 64 : 128;
}

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

// Running state of one set of 16 query columns: max (base 2) of column lane%16, the row
// sums and the output rows in the MFMA output layout (lane (c, gq): positions 4gq+t).  The
// row sums come from one more MFMA per step, P times a ones operand, so they add exactly
// the rounded weights the output rows add, and need neither VALU adds nor shuffles.
struct PfState {
  float m;
  f4 lsum;   // lsum[t]: sum of the weights of position 4*(lane/16)+t
  f4 o[8];   // o[nb][t]: position 4*(lane/16)+t, head-dim 16 nb + lane%16
};

__device__ __forceinline__ void pf_init(PfState& s) {
  s.m = -INFINITY;
  s.lsum = f4{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
  for (int nb = 0; nb < 8; nb++) s.o[nb] = f4{0.0f, 0.0f, 0.0f, 0.0f};
}

// Online-softmax update of one set of 16 query columns from its two 16 x 16 tiles of
// S^T (keys 0-15 and 16-31 of the step): the set's running max, the rescale of its output
// rows and sums when it moves, and P in the operand type (fp16: one
// part, relative error 2^-11 per weight; bf16: a hi + lo pair).  The maximum is taken on
// the raw products (the scale is positive) and each weight is exp2(fma(s, scale2, -m));
// a column with no active key so far takes m = 0 there, so its masked products (-inf)
// give exactly 0.
template <typename T, class Active>
__device__ __forceinline__ void softmax_set(const f4& s0, const f4& s1, float scale2, bool full,
                                            Active active, PfState& st, v8<T>& pa, v8<T>& pb) {
  constexpr bool kPair = __is_same(T, bf16e);
  const int lane = threadIdx.x & 63;
  const int c = lane & 15;
  const int gq = lane >> 4;
  float r[8];
#pragma unroll
  for (int t = 0; t < 4; t++) {
    r[t] = s0[t];
    r[4 + t] = s1[t];
  }
  if (!full) {  // (uniform) steps that need the causal / window mask
#pragma unroll
    for (int t = 0; t < 4; t++) {
      if (!active(4 * gq + t, c)) r[t] = -INFINITY;
      if (!active(16 + 4 * gq + t, c)) r[4 + t] = -INFINITY;
    }
  }
  float mx = r[0];
#pragma unroll
  for (int i = 1; i < 8; i++) mx = fmaxf(mx, r[i]);
  mx = col_max(mx) * scale2;  // this step's maximum, base 2
  // the running maximum moves (and the rows and sums are rescaled) only when some column's
  // step maximum exceeds it by more than 8, so every weight stays below 2^8 (far inside
  // the fp16/bf16 operand and fp32 accumulator ranges); a first active key always moves it
  if (__ballot(mx > st.m + 8.0f) != 0ull) {
    const float mn = fmaxf(st.m, mx);
    const float alpha = (mn == -INFINITY) ? 1.0f : __builtin_amdgcn_exp2f(st.m - mn);
    st.m = mn;
    float at[4];
#pragma unroll
    for (int t = 0; t < 4; t++) at[t] = __shfl(alpha, 4 * gq + t, 64);
#pragma unroll
    for (int t = 0; t < 4; t++) st.lsum[t] *= at[t];
#pragma unroll
    for (int nb = 0; nb < 8; nb++)
#pragma unroll
      for (int t = 0; t < 4; t++) st.o[nb][t] *= at[t];
  }
  const float mref = (st.m == -INFINITY) ? 0.0f : st.m;
#pragma unroll
  for (int i = 0; i < 8; i++) {
    const float pv = __builtin_amdgcn_exp2f(__builtin_fmaf(r[i], scale2, -mref));
    pa[i] = (T)pv;
    if constexpr (kPair) pb[i] = (T)(pv - (float)pa[i]);
  }
}

// B operand of O += P . V for output columns 16 nb .. 16 nb + 15 (head-dims), read with
// the transposing LDS load: inside each group of 16 lanes (one k-group kg), output lane i
// receives element i%4 of the 4 halfs that lane 4k + i/4 of the group addressed, for
// k = 0..3.  Lane j of the group therefore addresses row 4 kg + j/4 (+16 for the second
// read), dims 16 nb + 4 (j%4) .. +3; lane i then holds dim 16 nb + i of rows 4 kg + k and
// 16 + 4 kg + k, which are exactly the key rows of its P operand's k-slots.
typedef short s4v __attribute__((ext_vector_type(4)));
template <typename T>
__device__ __forceinline__ v8<T> v_operand_tr(const T* Vl, int nb) {
  const int lane = threadIdx.x & 63;
  const int j = lane & 15;
  const int row = 4 * (lane >> 4) + (j >> 2);
  const int col = 16 * nb + 4 * (j & 3);
  typedef __attribute__((address_space(3))) s4v* lds_s4;
  const s4v lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s4)(Vl + row * kKS + col));
  const s4v hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s4)(Vl + (row + 16) * kKS + col));
  return __builtin_bit_cast(v8<T>, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
}

// One 32-row step from the staged tile for two sets of 16 query columns (positions
// t0..t0+15 and t0+16..t0+31 of one head), in the layout of the decode step's tile: each
// K operand read from LDS feeds the S MFMAs of both sets, and each V operand both sets'
// O += P . V; the V operands are read only after the S MFMAs, so that K and V registers are
// never live together.
template <typename T, class ActA, class ActB>
__device__ __forceinline__ void step_lds(const T* Kl, const T* Vl, const v8<T> (&qa)[4],
                                          const v8<T> (&qb)[4], float scale2, bool full,
                                          ActA act_a, ActB act_b, PfState& sa, PfState& sb) {
  constexpr bool kPair = __is_same(T, bf16e);
  const int lane = threadIdx.x & 63;
  const int c = lane & 15;
  const int gq = lane >> 4;
  f4 s0a = f4{0.0f, 0.0f, 0.0f, 0.0f}, s1a = s0a, s0b = s0a, s1b = s0a;
  // the S MFMAs issue at a raised wave priority: while one wavefront of a SIMD issues
  // them, the other's softmax fills the VALU (64K fp16 prompt 16.0 -> 15.2 ms)
  __builtin_amdgcn_s_setprio(2);
#pragma unroll
  for (int s = 0; s < 4; s++) {
    const v8<T> k0 = *reinterpret_cast<const v8<T>*>(Kl + c * kKS + 8 * gq + 32 * s);
    const v8<T> k1 = *reinterpret_cast<const v8<T>*>(Kl + (16 + c) * kKS + 8 * gq + 32 * s);
    s0a = mfma32(k0, qa[s], s0a);
    s1a = mfma32(k1, qa[s], s1a);
    s0b = mfma32(k0, qb[s], s0b);
    s1b = mfma32(k1, qb[s], s1b);
  }
  __builtin_amdgcn_s_setprio(0);
  v8<T> paa, pba, pab, pbb;
  softmax_set<T>(s0a, s1a, scale2, full, act_a, sa, paa, pba);
  softmax_set<T>(s0b, s1b, scale2, full, act_b, sb, pab, pbb);
  // output columns of MFMA nb are head-dims 16 nb .. 16 nb + 15
#pragma unroll
  for (int nb = 0; nb < 8; nb++) {
    const v8<T> vb = v_operand_tr<T>(Vl, nb);
    sa.o[nb] = mfma32(paa, vb, sa.o[nb]);
    sb.o[nb] = mfma32(pab, vb, sb.o[nb]);
    if constexpr (kPair) {
      sa.o[nb] = mfma32(pba, vb, sa.o[nb]);
      sb.o[nb] = mfma32(pbb, vb, sb.o[nb]);
    }
  }
  // the row sums: P times ones
  v8<T> ones;
#pragma unroll
  for (int i = 0; i < 8; i++) ones[i] = (T)1.0f;
  sa.lsum = mfma32(paa, ones, sa.lsum);
  sb.lsum = mfma32(pab, ones, sb.lsum);
  if constexpr (kPair) {
    sa.lsum = mfma32(pba, ones, sa.lsum);
    sb.lsum = mfma32(pbb, ones, sb.lsum);
  }
}

// write the normalised rows of one column set (positions p0 + col, col < ncol)
__device__ __forceinline__ void store_set(const PfState& st, float* out_head, int p0, int ncol) {
  const int lane = threadIdx.x & 63;
  const int c = lane & 15;
  const int gq = lane >> 4;
  // lane (gq, c) holds positions 4gq+t, dims 16 nb + c, and their sums; every position
  // attends to itself, so its sum is positive
#pragma unroll
  for (int t = 0; t < 4; t++) {
    const int col = 4 * gq + t;
    if (col < ncol) {
      const float r = 1.0f / st.lsum[t];
      float* dst = out_head + (size_t)(p0 + col) * kD + c;
#pragma unroll
      for (int nb = 0; nb < 8; nb++) dst[16 * nb] = st.o[nb][t] * r;
    }
  }
}

template <typename T>
__global__ __launch_bounds__(kPW * 64, 2) void k_prefill_attn(PrefillArgs A) {
  constexpr int kSR = stage_rows<T>();
  // two buffers of a kSR-row K tile and V tile (kSR / 32 steps per block barrier)
  __shared__ __align__(16) T kvs[2][2][kSR * kKS];
  const int qt = A.ntile - 1 - (int)(blockIdx.x % A.ntile);
  const int kv = (blockIdx.x / A.ntile) % A.Hkv;
  const int b = blockIdx.x / (A.ntile * A.Hkv);
  const int L = clamp_len_p(A.seq_lens, b, A.Lmax);
  const int t0 = qt * kPQ;
  if (t0 >= L) return;
  const int ncol = min(kPQ, L - t0);
  const int ncol_a = min(kPQ / 2, ncol);
  const int ncol_b = ncol - ncol_a;
  const int tend = t0 + ncol;
  const bool ret = A.is_ret[kv] != 0;
  const int sinks = A.sinks, window = A.window;
  // entries e < ns are the sink keys e, later entries the keys kstart + (e - ns)
  const int ns = ret ? 0 : min(sinks, tend);
  const int kstart = ret ? 0 : max(ns, t0 + 1 - window);
  const int nent = ns + max(0, tend - kstart);
  const int nstages = (nent + kSR - 1) / kSR;
  const T* Kb = static_cast<const T*>(A.K) + ((size_t)b * A.Hkv + kv) * (size_t)A.Lmax * kD;
  const T* Vb = static_cast<const T*>(A.V) + ((size_t)b * A.Hkv + kv) * (size_t)A.Lmax * kD;
  const int tid = threadIdx.x;
  const int wv = tid >> 6;
  auto key_of = [&](int e) { return e < ns ? e : kstart + (e - ns); };
  // staging: thread tid moves 16 bytes of K and of V in each of the rows tid/16 + 32 r,
  // piece tid%16
  constexpr int kRPT = kSR / 32;  // rows per thread
  const int srow = tid >> 4, spiece = tid & 15;
  auto fetch = [&](int stage, u4 (&kx)[kRPT], u4 (&vx)[kRPT]) {
#pragma unroll
    for (int r = 0; r < kRPT; r++) {
      const int e = stage * kSR + srow + 32 * r;
      const size_t row = (size_t)key_of(e < nent ? e : 0);
      kx[r] = reinterpret_cast<const u4*>(Kb + row * kD)[spiece];
      vx[r] = reinterpret_cast<const u4*>(Vb + row * kD)[spiece];
    }
  };
  auto store = [&](int buf, const u4 (&kx)[kRPT], const u4 (&vx)[kRPT]) {
#pragma unroll
    for (int r = 0; r < kRPT; r++) {
      reinterpret_cast<u4*>(&kvs[buf][0][(srow + 32 * r) * kKS])[spiece] = kx[r];
      reinterpret_cast<u4*>(&kvs[buf][1][(srow + 32 * r) * kKS])[spiece] = vx[r];
    }
  };
  // every wavefront takes one query head per pass; all take part in the staging
  for (int g0 = 0; g0 < A.G; g0 += kPW) {
    const int g = g0 + wv;
    const bool has = g < A.G;
    const int h = kv * A.G + (has ? g : 0);
    const T* qh = static_cast<const T*>(A.q) + (size_t)(b * A.Hq + h) * A.Lmax * kD;
    v8<T> qa[4], qb[4];
    load_qop<T>(qh + (size_t)t0 * kD, has ? ncol_a : 0, qa);
    load_qop<T>(qh + (size_t)(t0 + kPQ / 2) * kD, has ? ncol_b : 0, qb);
    PfState sa, sb;
    pf_init(sa);
    pf_init(sb);
    u4 kx[kRPT], vx[kRPT];
    fetch(0, kx, vx);
    store(0, kx, vx);
    __syncthreads();
    for (int s = 0; s < nstages; s++) {
      const int buf = s & 1;
      if (s + 1 < nstages) fetch(s + 1, kx, vx);  // in flight during this stage's MFMAs
#pragma unroll
      for (int sub = 0; sub < kRPT; sub++) {
        const int e0 = s * kSR + sub * kStep;
        if (!has || e0 >= nent) continue;
        // a full step: every key exists, lies at or before the tile's first position and
        // (local heads) is a sink or inside every column's window; keys grow with e
        const int ehi = e0 + kStep - 1;
        bool full = ehi < nent && ncol == kPQ && key_of(ehi) <= t0;
        if (!ret && ehi >= ns) full = full && key_of(max(e0, ns)) >= tend - window;
        auto act = [&](int i, int col, int p0, int nc) {
          const int e = e0 + i;
          if (e >= nent || col >= nc) return false;
          const int n = key_of(e), t = p0 + col;
          return n <= t && (ret || n < sinks || n > t - window);
        };
        step_lds<T>(kvs[buf][0] + sub * kStep * kKS, kvs[buf][1] + sub * kStep * kKS, qa, qb,
                     A.scale2, full, [&](int i, int col) { return act(i, col, t0, ncol_a); },
                     [&](int i, int col) { return act(i, col, t0 + kPQ / 2, ncol_b); }, sa, sb);
      }
      if (s + 1 < nstages) store(buf ^ 1, kx, vx);
      __syncthreads();
    }
    if (has) {
      float* oh = A.out + (size_t)(b * A.Hq + h) * A.Lmax * kD;
      store_set(sa, oh, t0, ncol_a);
      store_set(sb, oh, t0 + kPQ / 2, ncol_b);
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

hipError_t launch_prefill(const PrefillArgs& args, int kv_dtype, hipStream_t st) {
  PrefillArgs a = args;
  a.ntile = (a.Lmax + kPQ - 1) / kPQ;
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
