// rtp_decode_step_noalloc: the decode step on a fixed scratch array of the library's own,
// for callers that cannot allocate (graph capture, serving loops, harnesses that forbid
// allocation).  The array is a file-scope device variable; its address on each device is
// resolved once, with that device current, through hipGetSymbolAddress, and only that
// address is handed to the kernels (in host code the variable's name is not a device
// address).
#include "rtp_internal.h"

#include <mutex>

namespace {

constexpr size_t kScratchBytes = size_t(64) << 20;  // 64 MiB per device
constexpr int kMaxDevices = 64;

__device__ __align__(256) unsigned char scratch[kScratchBytes];

std::mutex g_mu;
void* g_scratch[kMaxDevices];  // device address of `scratch` per device (null: not resolved)

// The current device's address of `scratch`, resolved on its first use on that device.
rtp_status scratch_ptr(void** out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess) return RTP_EHIP;
  if (dev < 0 || dev >= kMaxDevices) return RTP_EUNSUPPORTED;
  std::lock_guard<std::mutex> lock(g_mu);
  if (!g_scratch[dev]) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || p == nullptr)
      return RTP_EHIP;
    g_scratch[dev] = p;
  }
  *out = g_scratch[dev];
  return RTP_OK;
}

}  // namespace

extern "C" rtp_status rtp_decode_step_noalloc(const rtp_layer_desc* d, void* stream) {
  // an invalid descriptor plans to 0 bytes: the step itself then reports why, before any
  // device call
  const size_t need = rtp_decode_step_workspace_size(d);
  if (need == 0) return rtp::decode_step_impl(d, nullptr, 0, stream, nullptr);
  if (need > kScratchBytes) return RTP_ESCRATCH;
  void* ws = nullptr;
  const rtp_status s = scratch_ptr(&ws);
  if (s != RTP_OK) return s;
  return rtp::decode_step_impl(d, ws, kScratchBytes, stream, nullptr);
}
