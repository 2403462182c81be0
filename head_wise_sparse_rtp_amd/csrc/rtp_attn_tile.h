// MFMA attention tile shared by the decode step and the prefill: one wavefront scores 32
// cache rows against 16 query columns (query heads in decode, query positions in prefill)
// with S^T = K . Q^T on 16x16x32 fp16 MFMAs, keeps an online softmax per column, and
// accumulates O += P . V on the same instruction.
//
// Method: Full Attention Strikes Back (xllm-io.github.io paper review), section 三,
// 核心公式: softmax attention over a set of cached rows.  The accumulator layout of S^T
// gives lane l the logits of column l%16 for rows 4*(l/16)+t, which is exactly the
// A-operand layout of P for O += P . V (8 MFMAs, one per 16 output columns).  Output
// column c of MFMA nb holds head-dim 8*c + nb, so each lane loads 16 contiguous bytes of
// each V row it needs.
#pragma once

#include "rtp_internal.h"

namespace rtp {

typedef _Float16 h8 __attribute__((ext_vector_type(8)));
// operand vectors of the MFMA tile for an element type: _Float16 (fp16 caches) or
// __bf16 (bfloat16 caches); h8 is v8<f16>
typedef __bf16 bf16e;
template <typename T>
struct V8T {
  typedef T type __attribute__((ext_vector_type(8)));
};
template <typename T>
using v8 = typename V8T<T>::type;
typedef float f4 __attribute__((ext_vector_type(4)));
typedef uint32_t u4 __attribute__((ext_vector_type(4)));

constexpr int kAttnG = 16;               // head columns of the MFMA tile
constexpr int kStep = 32;                // cache rows per wavefront step
__device__ __forceinline__ f4 mfma32(h8 a, h8 b, f4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f4 mfma32(v8<bf16e> a, v8<bf16e> b, f4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

// max over the four lanes of one MFMA column (lanes l, l^16, l^32, l^48), on the VALU:
// each permlane swap leaves a lane its own value and its partner's, in some order
__device__ __forceinline__ float col_max(float v) {
  const auto p = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  v = fmaxf(__uint_as_float(p[0]), __uint_as_float(p[1]));
  const auto q = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return fmaxf(__uint_as_float(q[0]), __uint_as_float(q[1]));
}

// ---------------------------------------------------------------------------
// MFMA attention engine
// ---------------------------------------------------------------------------
struct AttnState {
  float m;     // running max (base-2 logits) of head lane%16
  float l;     // this lane's share of sum 2^(s - m) for head lane%16
  f4 o[8];     // o[nb][t]: head 4*(lane/16)+t, dim 8*(lane%16)+nb (the prefill's tile
               // maps dim 16*nb + lane%16 instead)
};

__device__ __forceinline__ void attn_init(AttnState& s) {
  s.m = -INFINITY;
  s.l = 0.0f;
#pragma unroll
  for (int nb = 0; nb < 8; nb++) s.o[nb] = f4{0.0f, 0.0f, 0.0f, 0.0f};
}

// B operand of S^T = K . Q^T: head lane%16, dims 32*s + 8*(lane/16) + {0..7} in the MFMA
// of slice s (any assignment of dims to k-slots works if K uses the same one; this one lets
// the four lanes of a K row read 64 contiguous bytes per load)
template <typename T>
__device__ __forceinline__ void load_qop(const T* __restrict__ qhead0, int G, v8<T> (&qop)[4]) {
  const int lane = threadIdx.x & 63;
  const int h = lane & 15;
  const int gq = lane >> 4;
  if (h < G) {
    const v8<T>* p = reinterpret_cast<const v8<T>*>(qhead0 + (size_t)h * kD + 8 * gq);
#pragma unroll
    for (int s = 0; s < 4; s++) qop[s] = p[4 * s];
  } else {
#pragma unroll
    for (int s = 0; s < 4; s++)
#pragma unroll
      for (int i = 0; i < 8; i++) qop[s][i] = (T)0.0f;
  }
}

template <typename T>
struct StepLoads {
  v8<T> k[2][4];  // [tile][s]: K row (tile*16 + lane%16), dims 32*s + 8*gq ..
  v8<T> v[8];     // [u]: V row of k-slot u (u<4: tile0 row 4gq+u; else tile1 row 4gq+u-4)
};

// rows[i] for i in 0..31 supplied through `row_of(i)` (already clamped to a valid row);
// NTL: nontemporal loads (rows that nothing reads again soon)
template <bool NTL = false, typename T, class RowOf>
__device__ __forceinline__ void step_load(const T* __restrict__ Kb, const T* __restrict__ Vb,
                                          RowOf row_of, StepLoads<T>& ld) {
  const int lane = threadIdx.x & 63;
  const int c = lane & 15;
  const int gq = lane >> 4;
#pragma unroll
  for (int t = 0; t < 2; t++) {
    const int r = row_of(t * 16 + c);
    const v8<T>* p = reinterpret_cast<const v8<T>*>(Kb + (size_t)r * kD + 8 * gq);
#pragma unroll
    for (int s = 0; s < 4; s++) ld.k[t][s] = NTL ? __builtin_nontemporal_load(p + 4 * s) : p[4 * s];
  }
#pragma unroll
  for (int u = 0; u < 8; u++) {
    const int i = (u < 4) ? (4 * gq + u) : (16 + 4 * gq + (u - 4));
    const int r = row_of(i);
    const v8<T>* pv = reinterpret_cast<const v8<T>*>(Vb + (size_t)r * kD + 8 * c);
    ld.v[u] = NTL ? __builtin_nontemporal_load(pv) : *pv;
  }
}

// One step over 32 rows.  active(i, h) says whether row i takes part for head h
// (rows past the end and unselected rows are masked to -inf).
template <typename T, class Active>
__device__ __forceinline__ void step_compute(const StepLoads<T>& ld, const v8<T> (&qop)[4],
                                             float scale2, Active active, AttnState& st) {
  const int lane = threadIdx.x & 63;
  const int h = lane & 15;
  const int gq = lane >> 4;
  f4 s0 = f4{0.0f, 0.0f, 0.0f, 0.0f}, s1 = s0;
#pragma unroll
  for (int s = 0; s < 4; s++) {
    s0 = mfma32(ld.k[0][s], qop[s], s0);
    s1 = mfma32(ld.k[1][s], qop[s], s1);
  }
  // the maximum is taken on the raw products (the scale is positive) and each weight is
  // exp2(fma(s, scale2, -m)); a head with no active row so far takes m = 0 there, so its
  // masked products (-inf) give exactly 0
  float r[8];
#pragma unroll
  for (int t = 0; t < 4; t++) {
    r[t] = active(4 * gq + t, h) ? s0[t] : -INFINITY;
    r[4 + t] = active(16 + 4 * gq + t, h) ? s1[t] : -INFINITY;
  }
  float mx = r[0];
#pragma unroll
  for (int i = 1; i < 8; i++) mx = fmaxf(mx, r[i]);
  mx = col_max(mx);
  const float mn = fmaxf(st.m, mx * scale2);
  const float alpha = (mn == -INFINITY) ? 1.0f : __builtin_amdgcn_exp2f(st.m - mn);
  const float mref = (mn == -INFINITY) ? 0.0f : mn;
  // P = hi + lo in the operand type keeps the weights at about fp32 accuracy (fp16: 22
  // bits, bf16: 16 bits) through the 16-bit MFMA
  v8<T> pa, pb;
  float psum = 0.0f;
#pragma unroll
  for (int i = 0; i < 8; i++) {
    const float pv = __builtin_amdgcn_exp2f(__builtin_fmaf(r[i], scale2, -mref));
    psum += pv;
    const T hi = (T)pv;
    pa[i] = hi;
    pb[i] = (T)(pv - (float)hi);
  }
  st.l = st.l * alpha + psum;
  st.m = mn;
  // rescale the output rows (heads 4gq+t) by their heads' alpha, when some head's maximum
  // moved
  if (__ballot(alpha != 1.0f) != 0ull) {
    float at[4];
#pragma unroll
    for (int t = 0; t < 4; t++) at[t] = __shfl(alpha, 4 * gq + t, 64);
#pragma unroll
    for (int nb = 0; nb < 8; nb++) {
#pragma unroll
      for (int t = 0; t < 4; t++) st.o[nb][t] *= at[t];
    }
  }
#pragma unroll
  for (int nb = 0; nb < 8; nb++) {
    v8<T> vb;
#pragma unroll
    for (int u = 0; u < 8; u++) vb[u] = ld.v[u][nb];
    st.o[nb] = mfma32(pa, vb, st.o[nb]);
    st.o[nb] = mfma32(pb, vb, st.o[nb]);
  }
}

}  // namespace rtp
