// Allocation-free MLP backward, for callers that cannot allocate device memory
// (code under HIP graph capture, tight serving loops, harnesses that forbid
// hipMalloc). It runs the same four products as tp_mlp_bwd, with the bf16 dU
// scratch of [M, f] elements held in a file-scope device array instead of a
// caller workspace.
//
// The array `scratch` is a host-side stand-in in host code: its device address
// is looked up once per device (hipGetSymbolAddress, with that device current)
// and only that address is ever passed to a kernel. Every call on one device
// shares the array, so calls that overlap in time on one device race; nothing
// in it has to start at zero (the dU product writes every element it later
// reads). The products run one output tile per workgroup (no stream-K area).
#include <hip/hip_runtime.h>

#include <mutex>

#include "api_internal.hpp"
#include "tpshard.h"

#define TP_API extern "C" __attribute__((visibility("default")))

namespace {

constexpr size_t kScratchBytes = size_t(80) << 20;  // 80 MiB per device
constexpr int kMaxDevices = 64;

static __device__ __align__(256) unsigned char scratch[kScratchBytes];

std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

// Device address of `scratch` on the current device, looked up on first use.
tp_status scratch_on_current_device(const char* fn, void** out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return tps::api_fail(TP_ERR_HIP, "%s: hipGetDevice: %s", fn, hipGetErrorString(e));
  if (dev < 0 || dev >= kMaxDevices)
    return tps::api_fail(TP_ERR_UNSUPPORTED, "%s: device %d outside the %d devices supported", fn, dev, kMaxDevices);
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !p)
      return tps::api_fail(TP_ERR_HIP, "%s: hipGetSymbolAddress(scratch) on device %d: %s", fn, dev,
                           hipGetErrorString(e));
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return TP_OK;
}

}  // namespace

TP_API size_t tp_mlp_bwd_noalloc_max_bytes(void) { return kScratchBytes; }

TP_API tp_status tp_mlp_bwd_noalloc(int64_t M, int64_t h, int64_t f, const void* X, const void* A_i, const void* B_i,
                                    const void* U_i, const void* Y_i, const void* dZ, float* dX_i, float* dA_i,
                                    float* dB_i, void* stream) {
  const char* fn = "tp_mlp_bwd_noalloc";
  tp_status st = tps::mlp_bwd_validate(fn, M, h, f, X, A_i, B_i, U_i, Y_i, dZ, dX_i, dA_i, dB_i);
  if (st != TP_OK) return st;
  if (M > 0 && (!U_i || !Y_i))
    return tps::api_fail(TP_ERR_INVALID_ARG, "%s: U_i and Y_i are required (no activation recompute)", fn);
  const double need = (double)M * (double)f * 2.0;
  if (need > (double)kScratchBytes)
    return tps::api_fail(TP_ERR_UNSUPPORTED, "%s: dU of %lld x %lld bf16 exceeds the %zu-byte scratch", fn,
                         (long long)M, (long long)f, kScratchBytes);
  void* dU = nullptr;
  if (M > 0) {
    st = scratch_on_current_device(fn, &dU);
    if (st != TP_OK) return st;
  }
  return tps::mlp_bwd_products(fn, M, h, f, X, A_i, B_i, U_i, Y_i, dZ, dX_i, dA_i, dB_i,
                               static_cast<uint16_t*>(dU), nullptr, static_cast<hipStream_t>(stream));
}
