// Layer-wise output loss of the quantized, transformed layer and its
// straight-through gradients with respect to the angles and channel scales:
// the objective the paper notes minimise to learn the transform ("损失函数 /
// 训练策略": L = ||Q(D)(X') - D(X)||, per layer, with the angles and scales
// optimised first). Here L is the squared Frobenius norm
//   L = sum_{m,n} (Y_q[m][n] - Y[m][n])^2,
//   Y_q = the 4-bit layer on X' = X T^-1 (paro_rotate, then the W4 linear;
//         fp16 as the product stores them),
//   Y   = X W^T, the layer in its original fp16 weights.
// Gradients pass through the quantizer unchanged (training through Q reads
// as straight-through): dY = 2 (Y_q - Y), dX' = dY W_hat, dW_hat = dY^T X'
// taken as the gradient of T W, then both transforms' own gradients, summed.
// Because X' (T W)^T = X W^T for every angle and scale, the two sides'
// contributions through T W itself cancel exactly, and the sum equals the
// activation side's gradient for dX' = dY E with E = W_hat - T W the
// quantization error. That form is what is computed: the two cancelling
// terms are each some 30-50 times larger than their sum, so adding them in
// fp32 would lose that much accuracy.
//
// The two dense products (X W^T, and dY E as three bf16 products of split
// operands) are plain GEMMs and go to rocBLAS;
// the rest runs in this library's kernels: the transform, the W4 linear, the
// fp32 transform of W with the quantization error (the quantizer's own pass),
// the loss with its deterministic reduction, and the activation side's
// gradients.
#include <rocblas/rocblas.h>

#include <mutex>

#include "paro_internal.h"

#pragma clang fp contract(off)

namespace paro {
namespace {

constexpr int kLossBlocks = 1024;  // partial sums of the loss (fixed: the order never changes)

// x = hi + lo + (a remainder of about 2^-16 |x|): hi = bf16(x), lo = bf16(x - hi),
// both rounded to nearest even
__device__ __forceinline__ uint16_t bf16_rne(float f) {
  uint32_t u = __builtin_bit_cast(uint32_t, f);
  u += 0x7fffu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

// Block b sums (y_q - y)^2 over elements b, b + B, b + 2B, ... (grid-stride
// by thread, then a fixed tree over the block) into part[b]; with dyh != NULL
// it also writes dY = 2 (y_q - y) as bf16 high and low parts,
// dyh = bf16(dY), dyl = bf16(dY - dyh).
__global__ __launch_bounds__(256) void loss_partial_kernel(const uint16_t* __restrict__ yq,
                                                           const float* __restrict__ y,
                                                           uint16_t* __restrict__ dyh,
                                                           uint16_t* __restrict__ dyl, int64_t n,
                                                           float* __restrict__ part) {
  __shared__ float red[256];
  float acc = 0.f;
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n; i += (int64_t)gridDim.x * 256) {
    const float diff = (float)__builtin_bit_cast(_Float16, yq[i]) - y[i];
    acc += diff * diff;
    if (dyh) {
      const float g = 2.0f * diff;
      const uint16_t h = bf16_rne(g);
      dyh[i] = h;
      dyl[i] = bf16_rne(g - __builtin_bit_cast(float, (uint32_t)h << 16));
    }
  }
  red[threadIdx.x] = acc;
  __syncthreads();
  for (int w = 128; w > 0; w >>= 1) {
    if ((int)threadIdx.x < w) red[threadIdx.x] += red[threadIdx.x + w];
    __syncthreads();
  }
  if (threadIdx.x == 0) part[blockIdx.x] = red[0];
}

// loss = sum of the partial sums (fp64): thread t adds partials t, t + 256,
// ... in order, then a fixed tree over the block
__global__ __launch_bounds__(256) void loss_final_kernel(const float* __restrict__ part, int nb,
                                                         float* __restrict__ loss) {
  __shared__ double red[256];
  double s = 0.0;
  for (int b = threadIdx.x; b < nb; b += 256) s += (double)part[b];
  red[threadIdx.x] = s;
  __syncthreads();
  for (int w = 128; w > 0; w >>= 1) {
    if ((int)threadIdx.x < w) red[threadIdx.x] += red[threadIdx.x + w];
    __syncthreads();
  }
  if (threadIdx.x == 0) loss[0] = (float)red[0];
}

__global__ __launch_bounds__(256) void fill_zero_kernel(float* __restrict__ a, int64_t n) {
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n; i += (int64_t)gridDim.x * 256)
    a[i] = 0.f;
}

unsigned grid_for(int64_t n) {
  const int64_t b = (n + 255) / 256;
  return (unsigned)std::max<int64_t>(1, std::min<int64_t>(b, 16384));
}

size_t a256(size_t b) { return (b + 255) & ~(size_t)255; }

int fail(hipError_t e, const char* what) {
  set_error(std::string(what) + ": " + hipGetErrorString(e));
  return PARO_ERR_HIP;
}

// rocBLAS handle per device, created on first use and kept for the process
rocblas_handle blas_handle(int device) {
  static std::mutex mu;
  static rocblas_handle handles[64] = {};
  std::lock_guard<std::mutex> lock(mu);
  if (device < 0 || device >= 64) return nullptr;
  if (!handles[device] && rocblas_create_handle(&handles[device]) != rocblas_status_success) {
    handles[device] = nullptr;
  }
  return handles[device];
}

struct LossLayout {
  size_t xr, yq, y, w4, part, dxr, qw, sc, zr, flag, bw, dth, dal, yh, yl, eh, el, total;
};

LossLayout loss_layout(const paro_rotation* r, int64_t M, int64_t N, int64_t d, bool grad) {
  LossLayout L{};
  size_t off = 0;
  auto take = [&](size_t bytes) {
    const size_t o = off;
    off += a256(bytes);
    return o;
  };
  // the W4 linear's workspace first: its arrival counters then sit at offset 0
  // for every M and N, so a workspace reused with other sizes still finds
  // them zero
  L.w4 = take(paro_w4_linear_workspace_size(nullptr, M, N, d));
  L.xr = take((size_t)M * d * 2);
  L.yq = take((size_t)M * N * 2);
  L.y = take((size_t)M * N * 4);
  L.part = take((size_t)kLossBlocks * 4);
  if (grad) {
    L.dxr = take((size_t)M * d * 4);
    L.qw = take((size_t)N * (d / 2));
    L.sc = take((size_t)N * (d / r->group) * 2);
    L.zr = take((size_t)N * (d / r->group));
    L.flag = take(4);
    L.bw = take(rotate_backward_scratch_bytes(r, M));
    L.dth = take((size_t)r->K * (size_t)(d / 2) * 4);
    L.dal = take((size_t)d * 4);
    L.yh = take((size_t)M * N * 2);
    L.yl = take((size_t)M * N * 2);
    L.eh = take((size_t)N * d * 2);
    L.el = take((size_t)N * d * 2);
  }
  L.total = off;
  return L;
}

}  // namespace

size_t layer_loss_scratch_bytes(const paro_rotation* r, int64_t M, int64_t N, int64_t d, bool grad) {
  return loss_layout(r, M, N, d, grad).total;
}

int run_layer_loss(const paro_rotation* r, const uint16_t* x, const uint16_t* w, const uint8_t* qw,
                   const uint16_t* sc, const uint8_t* zr, int64_t M, int64_t N, int64_t d, int group,
                   float* loss, float* dtheta, float* dalpha, void* ws, hipStream_t stream) {
  const bool grad = dtheta != nullptr || dalpha != nullptr;
  const LossLayout L = loss_layout(r, M, N, d, grad);
  char* base = (char*)ws;
  uint16_t* xr = (uint16_t*)(base + L.xr);
  uint16_t* yq = (uint16_t*)(base + L.yq);
  float* y = (float*)(base + L.y);
  float* part = (float*)(base + L.part);
  hipError_t e = launch_rotate(r, x, xr, M, stream);
  if (e != hipSuccess) return fail(e, "paro_layer_loss: transform");
  int st = paro_w4_linear(nullptr, xr, qw, sc, zr, nullptr, yq, M, N, d, group, base + L.w4,
                          paro_w4_linear_workspace_size(nullptr, M, N, d), stream);
  if (st != PARO_OK) return st;
  int dev = 0;
  if ((e = hipGetDevice(&dev)) != hipSuccess) return fail(e, "paro_layer_loss: hipGetDevice");
  rocblas_handle h = blas_handle(dev);
  if (!h || rocblas_set_stream(h, stream) != rocblas_status_success) {
    set_error("paro_layer_loss: rocBLAS handle");
    return PARO_ERR_HIP;
  }
  const float one = 1.0f, zero = 0.0f;
  // Y (column-major N x M, ld N) = W (stored [N][d]: column-major d x N, transposed) * X^T
  if (rocblas_gemm_ex(h, rocblas_operation_transpose, rocblas_operation_none, (rocblas_int)N,
                      (rocblas_int)M, (rocblas_int)d, &one, w, rocblas_datatype_f16_r, (rocblas_int)d, x,
                      rocblas_datatype_f16_r, (rocblas_int)d, &zero, y, rocblas_datatype_f32_r,
                      (rocblas_int)N, y, rocblas_datatype_f32_r, (rocblas_int)N, rocblas_datatype_f32_r,
                      rocblas_gemm_algo_standard, 0, 0) != rocblas_status_success) {
    set_error("paro_layer_loss: rocBLAS X W^T");
    return PARO_ERR_HIP;
  }
  uint16_t* yh = grad ? (uint16_t*)(base + L.yh) : nullptr;
  uint16_t* yl = grad ? (uint16_t*)(base + L.yl) : nullptr;
  hipLaunchKernelGGL(loss_partial_kernel, dim3(kLossBlocks), dim3(256), 0, stream, yq, y, yh, yl,
                     M * N, part);
  hipLaunchKernelGGL(loss_final_kernel, dim3(1), dim3(256), 0, stream, part, kLossBlocks, loss);
  if ((e = hipGetLastError()) != hipSuccess) return fail(e, "paro_layer_loss: loss");
  if (!grad) return PARO_OK;

  float* dxr = (float*)(base + L.dxr);
  uint16_t* eh = (uint16_t*)(base + L.eh);
  uint16_t* el = (uint16_t*)(base + L.el);
  // The quantizer's pass over T W (its codes go to scratch) writes the
  // quantization error E = W_hat - T W, as bf16 high and low parts
  if ((e = launch_quantize(r, w, N, d, group, (uint8_t*)(base + L.qw), (uint16_t*)(base + L.sc),
                           (uint8_t*)(base + L.zr), (int*)(base + L.flag), stream, eh, el)) != hipSuccess)
    return fail(e, "paro_layer_loss: weight transform");
  // dX' (column-major d x M, ld d) = E (column-major d x N) * dY^T (column-major N x M),
  // as three bf16 products with fp32 accumulation: E_hi dY_hi + E_hi dY_lo +
  // E_lo dY_hi carries about 16 bits of each operand (relative error ~2^-16),
  // at a fraction of an fp32 GEMM's time, with fp32's range (dY's parts come
  // from the loss kernel, E's from the quantizer)
  const uint16_t* ea[3] = {eh, eh, el};
  const uint16_t* yb[3] = {yh, yl, yh};
  for (int t = 0; t < 3; ++t) {
    if (rocblas_gemm_ex(h, rocblas_operation_none, rocblas_operation_none, (rocblas_int)d, (rocblas_int)M,
                        (rocblas_int)N, &one, ea[t], rocblas_datatype_bf16_r, (rocblas_int)d, yb[t],
                        rocblas_datatype_bf16_r, (rocblas_int)N, t ? &one : &zero, dxr,
                        rocblas_datatype_f32_r, (rocblas_int)d, dxr, rocblas_datatype_f32_r,
                        (rocblas_int)d, rocblas_datatype_f32_r, rocblas_gemm_algo_standard, 0,
                        0) != rocblas_status_success) {
      set_error("paro_layer_loss: rocBLAS dY E");
      return PARO_ERR_HIP;
    }
  }
  float* dth = dtheta ? dtheta : (float*)(base + L.dth);  // a NULL output still needs a place
  float* dal = dalpha ? dalpha : (float*)(base + L.dal);
  if ((e = launch_rotate_backward(r, 0, x, dxr, nullptr, dth, dal, M, base + L.bw, stream)) !=
      hipSuccess)
    return fail(e, "paro_layer_loss: transform gradients");
  return PARO_OK;
}

hipError_t launch_fill_zero(float* a, int64_t n, hipStream_t stream) {
  if (n <= 0 || !a) return hipSuccess;
  hipLaunchKernelGGL(fill_zero_kernel, dim3(grid_for(n)), dim3(256), 0, stream, a, n);
  return hipGetLastError();
}

}  // namespace paro
