// noalloc.hip -- moe_stack_pass_noalloc: moe_stack_pass with its workspace
// in a file-scope device array instead of a caller's buffer, for callers
// that cannot allocate device memory (code under HIP graph capture, tight
// serving loops, harnesses that forbid hipMalloc).
//
// The array `scratch` is a host-side stand-in in host code: its device
// address is looked up once per device with hipGetSymbolAddress (each GPU
// holds its own copy at its own address) and only that address is passed
// on.  The array is zero when the code object is loaded; its first 256
// bytes hold the routing's arrival counters, which every call leaves at
// zero, and the first call on each device also clears them with a fill
// kernel on the call's stream.  The rest needs no initialisation: every
// call writes what it reads there.  Every call on one device shares that
// device's array, so calls that can overlap on one device (other streams,
// other host threads) race and must be serialised by the caller.
#include <hip/hip_runtime.h>

#include <mutex>

#include "moe_verify.h"

namespace {

static __device__ __align__(256) unsigned char scratch[MOE_NOALLOC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;

struct DeviceScratch {
  std::mutex mu;
  void *ptr[kMaxDevices] = {};
  bool cleared[kMaxDevices] = {};
};

DeviceScratch &device_scratch() {
  static DeviceScratch d;
  return d;
}

__global__ void clear_head_kernel(unsigned *head) { head[threadIdx.x] = 0u; }

}  // namespace

extern "C" int moe_stack_pass_noalloc(const moe_shape *shape, int32_t n_layers,
                                      const moe_stack_weights *weights, const float *x,
                                      int32_t n_tokens, int32_t engine, int32_t *topk_idx,
                                      float *topk_w, float *y, int32_t *n_unique,
                                      void *stream) {
  // validation and the size this call needs, before any device work
  size_t need = 0;
  int rc = moe_stack_pass(shape, n_layers, weights, x, n_tokens, engine, topk_idx, topk_w, y,
                          n_unique, nullptr, &need, nullptr);
  if (rc != MOE_OK) return rc;
  if (need > (size_t)MOE_NOALLOC_SCRATCH_BYTES) return MOE_ERR_WORKSPACE;

  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return MOE_ERR_HIP;
  hipStream_t st = (hipStream_t)stream;
  void *ptr = nullptr;
  {
    DeviceScratch &ds = device_scratch();
    std::lock_guard<std::mutex> lk(ds.mu);
    if (!ds.ptr[dev]) {
      void *p = nullptr;
      if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return MOE_ERR_HIP;
      ds.ptr[dev] = p;
    }
    ptr = ds.ptr[dev];
    if (!ds.cleared[dev]) {
      hipLaunchKernelGGL(clear_head_kernel, dim3(1), dim3(64), 0, st, (unsigned *)ptr);
      if (hipGetLastError() != hipSuccess) return MOE_ERR_HIP;
      ds.cleared[dev] = true;
    }
  }
  size_t have = (size_t)MOE_NOALLOC_SCRATCH_BYTES;
  return moe_stack_pass(shape, n_layers, weights, x, n_tokens, engine, topk_idx, topk_w, y,
                        n_unique, ptr, &have, stream);
}
