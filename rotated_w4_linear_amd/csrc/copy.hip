// A plain device copy at the rate HBM sustains for a read stream and a write
// stream of equal size: the measured ceiling the memory-bound kernels of this
// library (the activation transform, the small-batch linear) are compared
// with, next to the 8 TB/s datasheet peak. Each lane moves 16-byte chunks with
// buffer loads and stores; a lane issues U loads before its first store, so
// U x 16 bytes per lane are in flight; workgroups stride over the buffer.
#include "paro_internal.h"

namespace paro {
namespace {

constexpr int kRsrcWord3 = 0x00020000;  // gfx9 buffer resource word 3

template <int U>
__global__ __launch_bounds__(256) void stream_copy_kernel(const uint8_t* __restrict__ src,
                                                          uint8_t* __restrict__ dst, int64_t chunks) {
  // chunks: number of 16-byte chunks; bytes beyond 2^31 per launch are
  // covered by the host splitting the copy
  const __amdgpu_buffer_rsrc_t rs =
      __builtin_amdgcn_make_buffer_rsrc((void*)src, (short)0, (int)(chunks * 16), kRsrcWord3);
  const __amdgpu_buffer_rsrc_t rd =
      __builtin_amdgcn_make_buffer_rsrc((void*)dst, (short)0, (int)(chunks * 16), kRsrcWord3);
  const int64_t step = (int64_t)gridDim.x * 256 * U;
  for (int64_t c0 = (int64_t)blockIdx.x * 256 * U + threadIdx.x; c0 < chunks; c0 += step) {
    typedef uint32_t u4 __attribute__((ext_vector_type(4)));
    u4 v[U];
#pragma unroll
    for (int u = 0; u < U; ++u)  // out-of-range offsets read 0 and store nothing (buffer bounds)
      v[u] = __builtin_amdgcn_raw_buffer_load_b128(rs, (int)((c0 + 256 * u) * 16), 0, 0);
#pragma unroll
    for (int u = 0; u < U; ++u) __builtin_amdgcn_raw_buffer_store_b128(v[u], rd, (int)((c0 + 256 * u) * 16), 0, 0);
  }
}

}  // namespace

hipError_t launch_stream_copy(const void* src, void* dst, size_t bytes, int blocks, hipStream_t stream) {
  constexpr size_t kMax = size_t(1) << 30;  // bytes per launch (buffer offsets are 32-bit)
  for (size_t off = 0; off < bytes; off += kMax) {
    const size_t n = bytes - off < kMax ? bytes - off : kMax;
    hipLaunchKernelGGL(stream_copy_kernel<4>, dim3((unsigned)blocks), dim3(256), 0, stream,
                       (const uint8_t*)src + off, (uint8_t*)dst + off, (int64_t)(n / 16));
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

}  // namespace paro
