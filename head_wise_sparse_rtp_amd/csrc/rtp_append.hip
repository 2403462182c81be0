// Cache update of one decode step: indexer projections of the new token and the append
// of its K/V rows.
//
// Method: Full Attention Strikes Back (xllm-io.github.io paper review), section 三,
// 核心公式: the indexer compares W^Q_h q^pre with W^K_h k^pre, both projected to r = 16
// dims before RoPE; retrieval heads keep the whole cache and local heads a window plus
// sinks (section 五, test configuration).
//
// Block (sequence b, KV head kv), 128 threads.  For a retrieval head the block computes
// the G query projections and the key projection as fp32 fused-multiply-add chains over
// the 128 inputs in order (one chain per thread and output feature; the inputs are
// staged in LDS, the weights are read 16 contiguous floats per input row), stores the
// key row in the cache's dtype (round to nearest even), and copies the new K/V rows to
// position L - 1.  A local head's block copies the rows to the position's ring slot.
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

template <typename KT>
__global__ __launch_bounds__(kD) void k_append_project(AppendArgs A) {
  extern __shared__ float xs[];  // [G + 1][128]: q_pre rows of the KV head's query heads, k_pre
  const int kv = blockIdx.x % A.Hkv;
  const int b = blockIdx.x / A.Hkv;
  const int tid = threadIdx.x;
  const int L = clamp_len(A.seq_lens, b, A.Lmax);
  if (L < 1) return;
  const int n = L - 1;
  const int G = A.G;
  const KT* knew = static_cast<const KT*>(A.k_new) + ((size_t)b * A.Hkv + kv) * kD;
  const KT* vnew = static_cast<const KT*>(A.v_new) + ((size_t)b * A.Hkv + kv) * kD;
  const int kr = A.rank[kv];
  if (!A.is_ret[kv]) {
    const int slot = n < A.sinks ? n : A.sinks + n % A.window;
    const size_t row = ((size_t)b * A.Hloc + kr) * (size_t)(A.sinks + A.window) + slot;
    static_cast<KT*>(A.K_loc)[row * kD + tid] = knew[tid];
    static_cast<KT*>(A.V_loc)[row * kD + tid] = vnew[tid];
    return;
  }
  const size_t row = ((size_t)b * A.Hret + kr) * (size_t)A.Lmax + n;
  static_cast<KT*>(A.K_ret)[row * kD + tid] = knew[tid];
  static_cast<KT*>(A.V_ret)[row * kD + tid] = vnew[tid];
  const float* qp = A.q_pre + ((size_t)b * A.Hq + (size_t)kv * G) * kD;
  for (int i = tid; i < G * kD; i += kD) xs[i] = qp[i];
  xs[G * kD + tid] = A.k_pre[((size_t)b * A.Hkv + kv) * kD + tid];
  __syncthreads();
  // output (u, i): u < G is query head kv*G + u, u = G the key; i the feature
  for (int o = tid; o < (G + 1) * kR; o += kD) {
    const int u = o / kR, i = o % kR;
    const float* W = u < G ? A.Wq + ((size_t)kv * G + u) * kD * kR : A.Wk + (size_t)kr * kD * kR;
    const float* x = xs + u * kD;
    float a = 0.0f;
    for (int c = 0; c < kD; c++) a = __builtin_fmaf(x[c], W[c * kR + i], a);
    if (u < G)
      A.q_idx[((size_t)b * A.Hq + (size_t)kv * G + u) * kR + i] = a;
    else
      static_cast<KT*>(A.k_idx)[row * kR + i] = to_cache<KT>(a);
  }
}

}  // namespace

hipError_t launch_append_project(const AppendArgs& a, int kv_dtype, hipStream_t st) {
  const size_t lds = sizeof(float) * (size_t)(a.G + 1) * kD;
  const dim3 grid(a.B * a.Hkv);
  if (kv_dtype == 1)
    k_append_project<f16><<<grid, kD, lds, st>>>(a);
  else
    k_append_project<float><<<grid, kD, lds, st>>>(a);
  return hipGetLastError();
}

}  // namespace rtp
