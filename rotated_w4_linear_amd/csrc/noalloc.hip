// Static device scratch for paro_w4_linear_noalloc: the workspace of the W4
// linear (arrival counters, then partial sums or the transformed activations)
// in a file-scope device array, for callers that cannot allocate device memory.
// Each device the library runs on holds its own copy of the array until the
// process ends. Host code never uses the array's name as an address: its
// device address is looked up once per device (hipGetSymbolAddress, with
// that device current, in paro_device_init) and kept here.
#include <atomic>
#include <string>

#include "paro_internal.h"

namespace paro {
namespace {

static __device__ __align__(256) unsigned char scratch[kNoallocScratchBytes];

std::atomic<void*> g_scratch_ptr[kMaxDevices];

__global__ void zero_words_kernel(uint32_t* __restrict__ p, int n) {
  for (int i = blockIdx.x * blockDim.x + threadIdx.x; i < n; i += gridDim.x * blockDim.x) p[i] = 0u;
}

}  // namespace

int noalloc_scratch_setup(int dev) {
  if (dev < 0 || dev >= kMaxDevices) return PARO_ERR_UNSUPPORTED;
  if (g_scratch_ptr[dev].load(std::memory_order_acquire)) return PARO_OK;
  void* ptr = nullptr;
  hipError_t e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
  if (e != hipSuccess || !ptr) {
    set_error(std::string("device init: hipGetSymbolAddress(scratch): ") + hipGetErrorString(e));
    return PARO_ERR_HIP;
  }
  // the arrival counters must start at zero (every completed call leaves
  // them zero again)
  hipLaunchKernelGGL(zero_words_kernel, dim3(16), dim3(256), 0, 0, (uint32_t*)ptr,
                     (int)(kDecodeCounterBytes / 4));
  e = hipGetLastError();
  if (e == hipSuccess) e = hipDeviceSynchronize();
  if (e != hipSuccess) {
    set_error(std::string("device init: clearing the scratch counters: ") + hipGetErrorString(e));
    return PARO_ERR_HIP;
  }
  g_scratch_ptr[dev].store(ptr, std::memory_order_release);
  return PARO_OK;
}

void* noalloc_scratch(int dev) {
  if (dev < 0 || dev >= kMaxDevices) return nullptr;
  return g_scratch_ptr[dev].load(std::memory_order_acquire);
}

}  // namespace paro
