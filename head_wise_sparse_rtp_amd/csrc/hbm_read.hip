// Streaming-read ceiling of the device's HBM, as a scale for the decode kernels'
// bandwidth: every byte of a large buffer is read once with 16-byte vector loads, UNROLL
// loads in flight per thread, and folded into one word per thread so that no load can be
// dropped.  Two access orders: grid-stride (each load instruction of a wavefront covers
// 1 KB, and a thread's loads lie a grid apart) and span (each block streams its own
// contiguous share of the buffer in tiles of 256 * UNROLL vectors, one load instruction of
// the block covering 4 KB, as an attention block streams its rows).  Not part of librtp;
// the benchmark loads this library on its own.
#include <hip/hip_runtime.h>

#include <cstddef>
#include <cstdint>

namespace {

typedef uint32_t u4v __attribute__((ext_vector_type(4)));

template <int UNROLL, bool NT>
__global__ __launch_bounds__(256) void k_read(const u4v* __restrict__ src, size_t n16,
                                              uint32_t* __restrict__ sink) {
  const size_t stride = (size_t)gridDim.x * blockDim.x;
  size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
  uint32_t acc = 0u;
  for (; i + (UNROLL - 1) * stride < n16; i += UNROLL * stride) {
    u4v v[UNROLL];
#pragma unroll
    for (int u = 0; u < UNROLL; u++)
      v[u] = NT ? __builtin_nontemporal_load(src + i + u * stride) : src[i + u * stride];
#pragma unroll
    for (int u = 0; u < UNROLL; u++) acc ^= v[u].x ^ v[u].y ^ v[u].z ^ v[u].w;
  }
  for (; i < n16; i += stride) {
    const u4v v = src[i];
    acc ^= v.x ^ v.y ^ v.z ^ v.w;
  }
  sink[(size_t)blockIdx.x * blockDim.x + threadIdx.x] = acc;
}

template <int UNROLL, bool NT>
__global__ __launch_bounds__(256) void k_read_span(const u4v* __restrict__ src, size_t n16,
                                                   uint32_t* __restrict__ sink) {
  const size_t b = blockIdx.x, nb = gridDim.x;
  const size_t beg = n16 * b / nb, end = n16 * (b + 1) / nb;
  size_t i = beg;
  uint32_t acc = 0u;
  for (; i + 256 * UNROLL <= end; i += 256 * UNROLL) {
    u4v v[UNROLL];
#pragma unroll
    for (int u = 0; u < UNROLL; u++) {
      const u4v* p = src + i + u * 256 + threadIdx.x;
      v[u] = NT ? __builtin_nontemporal_load(p) : *p;
    }
#pragma unroll
    for (int u = 0; u < UNROLL; u++) acc ^= v[u].x ^ v[u].y ^ v[u].z ^ v[u].w;
  }
  for (i += threadIdx.x; i < end; i += 256) {
    const u4v v = src[i];
    acc ^= v.x ^ v.y ^ v.z ^ v.w;
  }
  sink[b * 256 + threadIdx.x] = acc;
}

}  // namespace

extern "C" {

// Reads bytes (a multiple of 16) from the 16-byte aligned device buffer src with `blocks`
// blocks of 256 threads.  variant 0..3: grid-stride order, 4 or 8 loads in flight per
// thread, plain or nontemporal; 4..7: span order, 8 or 16 loads in flight, plain or
// nontemporal.  sink holds blocks * 256 words.  Returns the hipError_t of the launch, or
// hipErrorInvalidValue (1) for an unknown variant.
int hbm_read(const void* src, size_t bytes, uint32_t* sink, int blocks, int variant,
             void* stream) {
  const u4v* s = static_cast<const u4v*>(src);
  const size_t n16 = bytes / 16;
  hipStream_t st = static_cast<hipStream_t>(stream);
  switch (variant) {
    case 0: k_read<4, false><<<blocks, 256, 0, st>>>(s, n16, sink); break;
    case 1: k_read<8, false><<<blocks, 256, 0, st>>>(s, n16, sink); break;
    case 2: k_read<4, true><<<blocks, 256, 0, st>>>(s, n16, sink); break;
    case 3: k_read<8, true><<<blocks, 256, 0, st>>>(s, n16, sink); break;
    case 4: k_read_span<8, false><<<blocks, 256, 0, st>>>(s, n16, sink); break;
    case 5: k_read_span<16, false><<<blocks, 256, 0, st>>>(s, n16, sink); break;
    case 6: k_read_span<8, true><<<blocks, 256, 0, st>>>(s, n16, sink); break;
    case 7: k_read_span<16, true><<<blocks, 256, 0, st>>>(s, n16, sink); break;
    default: return (int)hipErrorInvalidValue;
  }
  return (int)hipGetLastError();
}

}  // extern "C"
