// The HIP runtime calls of the host code (fx_api.cpp reaches the device only through
// these and the kernel launchers).
#include <hip/hip_runtime.h>

#include "fx_plan.h"

namespace fx {

int dev_current(int* device) { return hipGetDevice(device); }

int dev_alloc(void** ptr, size_t bytes) { return hipMalloc(ptr, bytes); }

int dev_free(void* ptr) { return hipFree(ptr); }

int dev_upload(void* dst, const void* src, size_t bytes) {
  return hipMemcpy(dst, src, bytes, hipMemcpyHostToDevice);
}

int dev_zero(void* dst, size_t bytes) { return hipMemset(dst, 0, bytes); }

int dev_take_error(uint32_t* dev_word, uint32_t* host_word) {
  hipError_t e = hipDeviceSynchronize();
  if (e == hipSuccess) e = hipMemcpy(host_word, dev_word, 4, hipMemcpyDeviceToHost);
  if (e == hipSuccess) e = hipMemset(dev_word, 0, 4);
  return e;
}

}  // namespace fx
