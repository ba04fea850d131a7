// Measured ceilings the kernels of this library are compared with, next to
// the datasheet peaks:
//  * a plain device copy at the rate HBM sustains for a read stream and a
//    write stream of equal size (for the activation transform and the
//    small-batch linear). Each lane moves 16-byte chunks with buffer loads and
//    stores; a lane issues U loads before its first store, so U x 16 bytes per
//    lane are in flight; workgroups stride over the buffer;
//  * a loop of fp16 MFMAs on register operands (for the prefill GEMM): the
//    rate the matrix cores sustain under the chip's power limit, which with
//    random operands sits well below the clock-limited datasheet figure.
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

// One wavefront per SIMD (256 lanes per workgroup): each wavefront keeps 2 x 8
// accumulator tiles of v_mfma_f32_32x32x16_f16 and runs `iters` rounds of 16
// independent MFMAs on operands read once from src (n8 vectors of 8 halfs);
// every lane then writes the sum of its 256 accumulators, so no MFMA is dead.
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(1)))
void mfma_loop_kernel(const _Float16* __restrict__ src, int n8, float* __restrict__ out, int iters) {
  typedef _Float16 h8 __attribute__((ext_vector_type(8)));
  typedef float f16v __attribute__((ext_vector_type(16)));
  const int tid = blockIdx.x * 256 + threadIdx.x;
  h8 a[2], b[8];
#pragma unroll
  for (int j = 0; j < 2; ++j) a[j] = *(const h8*)(src + 8 * ((tid * 10 + j) % n8));
#pragma unroll
  for (int m = 0; m < 8; ++m) b[m] = *(const h8*)(src + 8 * ((tid * 10 + 2 + m) % n8));
  f16v acc[2][8];
#pragma unroll
  for (int j = 0; j < 2; ++j)
#pragma unroll
    for (int m = 0; m < 8; ++m)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[j][m][e] = 0.0f;
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int m = 0; m < 8; ++m) acc[j][m] = __builtin_amdgcn_mfma_f32_32x32x16_f16(a[j], b[m], acc[j][m], 0, 0, 0);
  }
  float sum = 0.0f;
#pragma unroll
  for (int j = 0; j < 2; ++j)
#pragma unroll
    for (int m = 0; m < 8; ++m)
#pragma unroll
      for (int e = 0; e < 16; ++e) sum += acc[j][m][e];
  out[tid] = sum;
}

}  // namespace

hipError_t launch_mfma_loop(const void* src, int64_t n8, float* out, int blocks, int iters, hipStream_t stream) {
  hipLaunchKernelGGL(mfma_loop_kernel, dim3((unsigned)blocks), dim3(256), 0, stream, (const _Float16*)src, (int)n8,
                     out, iters);
  return hipGetLastError();
}

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
