// Cache update of one decode step: indexer projections of the new token and the append
// of its K/V rows.
//
// Method: Full Attention Strikes Back (xllm-io.github.io paper review), section 三,
// 核心公式: the indexer compares W^Q_h q^pre with W^K_h k^pre, both projected to r = 16
// dims before RoPE; retrieval heads keep the whole cache and local heads a window plus
// sinks (section 五, test configuration).
//
// Block (sequence b, KV head kv, output group u), one wavefront.  For a retrieval head,
// group u < G projects query head kv*G + u and group u = G the key; each block stages its
// 128 x 16 weight matrix and its input row in LDS with every load in flight, then lanes
// 0..15 each run one fp32 fused-multiply-add chain over the 128 inputs in order.  The key
// row is stored in the cache's dtype (round to nearest even).  Group G also copies the new
// K/V rows: to position L - 1 of a retrieval head, or to the position's ring slot of a
// local head (whose other groups have nothing to do).
#include "rtp_internal.h"

namespace rtp {

namespace {

__device__ __forceinline__ int clamp_len(const int32_t* seq_lens, int b, int Lmax) {
  int L = seq_lens[b];
  return L < 0 ? 0 : (L > Lmax ? Lmax : L);
}

template <typename KT>
__device__ __forceinline__ KT to_cache(float x);
template <>
__device__ __forceinline__ f16 to_cache<f16>(float x) {
  return (f16)x;
}
template <>
__device__ __forceinline__ float to_cache<float>(float x) {
  return x;
}
template <>
__device__ __forceinline__ bf16s to_cache<bf16s>(float x) {
  return f_to_bf16(x);
}

template <typename KT>
__global__ __launch_bounds__(64) void k_append_project(AppendArgs A) {
  __shared__ __align__(16) float ws[kD * kR];  // W[c][i]
  __shared__ __align__(16) float xs[kD];       // the input row
  const int G = A.G;
  const int u = blockIdx.x % (G + 1);
  const int kv = (blockIdx.x / (G + 1)) % A.Hkv;
  const int b = blockIdx.x / ((G + 1) * A.Hkv);
  const int lane = threadIdx.x;
  const int L = clamp_len(A.seq_lens, b, A.Lmax);
  if (L < 1) return;
  const int n = L - 1;
  const int kr = A.rank[kv];
  const bool ret = A.is_ret[kv] != 0;
  if (!ret && u < G) return;
  if (u == G) {
    const KT* knew = static_cast<const KT*>(A.k_new) + ((size_t)b * A.Hkv + kv) * kD;
    const KT* vnew = static_cast<const KT*>(A.v_new) + ((size_t)b * A.Hkv + kv) * kD;
    size_t row;
    KT *Kc, *Vc;
    if (ret) {
      row = ((size_t)b * A.Hret + kr) * (size_t)A.Lmax + n;
      Kc = static_cast<KT*>(A.K_ret);
      Vc = static_cast<KT*>(A.V_ret);
    } else {
      const int slot = n < A.sinks ? n : A.sinks + n % A.window;
      row = ((size_t)b * A.Hloc + kr) * (size_t)(A.sinks + A.window) + slot;
      Kc = static_cast<KT*>(A.K_loc);
      Vc = static_cast<KT*>(A.V_loc);
    }
    for (int c = lane; c < kD; c += 64) {
      Kc[row * kD + c] = knew[c];
      Vc[row * kD + c] = vnew[c];
    }
    if (!ret) return;
  }
  const float* W = u < G ? A.Wq + ((size_t)kv * G + u) * kD * kR : A.Wk + (size_t)kr * kD * kR;
  const float* x = u < G ? A.q_pre + ((size_t)b * A.Hq + (size_t)kv * G + u) * kD
                         : A.k_pre + ((size_t)b * A.Hkv + kv) * kD;
  float4 wv[kD * kR / 4 / 64];
#pragma unroll
  for (int j = 0; j < kD * kR / 4 / 64; j++) wv[j] = reinterpret_cast<const float4*>(W)[lane + 64 * j];
  const float2 xv = reinterpret_cast<const float2*>(x)[lane];
#pragma unroll
  for (int j = 0; j < kD * kR / 4 / 64; j++) reinterpret_cast<float4*>(ws)[lane + 64 * j] = wv[j];
  reinterpret_cast<float2*>(xs)[lane] = xv;
  __syncthreads();
  if (lane >= kR) return;
  const int i = lane;
  float a = 0.0f;
#pragma unroll 16
  for (int c = 0; c < kD; c++) a = __builtin_fmaf(xs[c], ws[c * kR + i], a);
  if (u < G)
    A.q_idx[((size_t)b * A.Hq + (size_t)kv * G + u) * kR + i] = a;
  else
    static_cast<KT*>(A.k_idx)[(((size_t)b * A.Hret + kr) * (size_t)A.Lmax + n) * kR + i] =
        to_cache<KT>(a);
}

}  // namespace

hipError_t launch_append_project(const AppendArgs& a, int kv_dtype, hipStream_t st) {
  const dim3 grid(a.B * a.Hkv * (a.G + 1));
  if (kv_dtype == 1)
    k_append_project<f16><<<grid, 64, 0, st>>>(a);
  else if (kv_dtype == 2)
    k_append_project<bf16s><<<grid, 64, 0, st>>>(a);
  else
    k_append_project<float><<<grid, 64, 0, st>>>(a);
  return hipGetLastError();
}

}  // namespace rtp
