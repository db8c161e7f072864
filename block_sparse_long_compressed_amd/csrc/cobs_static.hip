// Decode step for callers that cannot allocate device memory (code under HIP graph
// capture, tight serving loops, harnesses that forbid hipMalloc).  The workspace of
// cobs_sparse_attn_decode lives in a file-scope device array of fixed size instead
// of a caller buffer; everything else is the same entry point.
//
// Each device holds its own copy of `scratch` until the process ends.  In host code
// the array's name only stands in for the symbol: its device address is looked up once
// per device (hipGetSymbolAddress, with that device current) and only that address is
// handed to kernels.  The first call on a device zero-fills the array with a kernel on
// the caller's stream (the counters in it must start at zero; every completed step
// leaves them zero again).
#include <hip/hip_runtime.h>

#include <mutex>

#include "cobs.h"

static __device__ __align__(256) unsigned char scratch[COBS_STATIC_SCRATCH_BYTES];

namespace {

constexpr int kMaxDevices = 64;
std::mutex g_mu;
void* g_scratch_ptr[kMaxDevices];     // device address of `scratch` per device, once looked up

__global__ void k_zero_fill(uint4* p, size_t n) {
  for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += (size_t)gridDim.x * blockDim.x)
    p[i] = make_uint4(0u, 0u, 0u, 0u);
}

}  // namespace

namespace cobs {
// The device address of this device's array, or null before its first call.
void* static_scratch_of_current_device() {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return nullptr;
  std::lock_guard<std::mutex> lock(g_mu);
  return g_scratch_ptr[dev];
}
}  // namespace cobs

extern "C" cobs_status cobs_sparse_attn_decode_static(const cobs_params* p, int32_t batch, int32_t max_len,
                                                      const int32_t* seq_lens, const void* Q, const void* K,
                                                      const void* V, const void* mu, const void* so, const void* kc,
                                                      const void* vc, const float* gates, const int32_t* sel_in,
                                                      int32_t* sel_out, float* out, void* stream) {
  const cobs_status st = cobs_validate_params(p);
  if (st != COBS_OK) return st;
  const size_t need = cobs_workspace_bytes(p, batch, max_len, 1);
  if (need == 0) return COBS_ERR_INVALID_ARG;
  if (need > COBS_STATIC_SCRATCH_BYTES) return COBS_ERR_WORKSPACE;
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return COBS_ERR_HIP;
  void* ptr = nullptr;
  bool first = false;
  {
    std::lock_guard<std::mutex> lock(g_mu);
    if (!g_scratch_ptr[dev]) {
      if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess || !ptr) return COBS_ERR_HIP;
      g_scratch_ptr[dev] = ptr;
      first = true;
    }
    ptr = g_scratch_ptr[dev];
  }
  if (first) {
    hipLaunchKernelGGL(k_zero_fill, dim3(1024), dim3(256), 0, (hipStream_t)stream, static_cast<uint4*>(ptr),
                       (size_t)COBS_STATIC_SCRATCH_BYTES / sizeof(uint4));
    if (hipGetLastError() != hipSuccess) return COBS_ERR_HIP;
  }
  return cobs_sparse_attn_decode(p, batch, max_len, seq_lens, Q, K, V, mu, so, kc, vc, gates, sel_in, sel_out, out,
                                 ptr, COBS_STATIC_SCRATCH_BYTES, stream);
}
