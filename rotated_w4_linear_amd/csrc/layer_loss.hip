// Layer-wise output loss of the quantized, transformed layer and its
// straight-through gradients with respect to the angles and channel scales:
// the objective the paper notes minimise to learn the transform ("损失函数 /
// 训练策略": L = ||Q(D)(X') - D(X)||, per layer, with the angles and scales
// optimised first). Here L is the squared Frobenius norm
//   L = sum_{m,n} (Y_q[m][n] - Y[m][n])^2,
//   Y_q = the 4-bit layer on X' = X T^-1 (paro_rotate, then the W4 linear;
//         fp16 as the product stores them),
//   Y   = X W^T, the layer in its original fp16 weights (fp32 sums).
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
// Every step runs in this library's kernels: the transform, the W4 linear,
// X W^T on the matrix cores with the loss and dY (fp16) in its epilogue, a
// fixed-order reduction of the per-tile loss sums, the quantizer's own pass
// over T W writing E in fp16, E transposed, dY E on the matrix cores (fp32
// out), and the activation side's transform gradients. fp16 operands for dY E
// cost nothing measurable: dY already carries the fp16 rounding of Y_q, whose
// relative size against Y_q - Y is tens of times larger than fp16's own.
#include <algorithm>

#include "paro_internal.h"

#pragma clang fp contract(off)

namespace paro {
namespace {

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

// dY and E^T keep the contraction (N) padded to a multiple of 64 with zeros
int64_t pad64(int64_t n) { return (n + 63) & ~int64_t(63); }

struct LossLayout {
  size_t w4, xr, yq, part, dxr, qw, sc, zr, flag, bw, dth, dal, dy, e, et, total;
};

LossLayout loss_layout(const paro_rotation* r, int64_t M, int64_t N, int64_t d, bool grad) {
  LossLayout L{};
  size_t off = 0;
  auto take = [&](size_t bytes) {
    const size_t o = off;
    off += a256(bytes);
    return o;
  };
  // the W4 linear's workspace first, never shorter than its arrival
  // counters: they then sit at offset 0 for every M and N, so a workspace
  // reused with other sizes still finds them zero
  L.w4 = take(std::max(paro_w4_linear_workspace_size(nullptr, M, N, d), kDecodeCounterBytes));
  L.xr = take((size_t)M * d * 2);
  L.yq = take((size_t)M * N * 2);
  L.part = take((size_t)nt_tiles(M, N) * 4);
  if (grad) {
    const size_t np = (size_t)pad64(N);
    L.dxr = take((size_t)M * d * 4);
    L.qw = take((size_t)N * (d / 2));
    L.sc = take((size_t)N * (d / r->group) * 2);
    L.zr = take((size_t)N * (d / r->group));
    L.flag = take(4);
    L.bw = take(rotate_backward_scratch_bytes(r, M));
    L.dth = take((size_t)r->K * (size_t)(d / 2) * 4);
    L.dal = take((size_t)d * 4);
    L.dy = take((size_t)M * np * 2);
    L.e = take((size_t)N * d * 2);
    L.et = take((size_t)d * np * 2);
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
  float* part = (float*)(base + L.part);
  uint16_t* dy = grad ? (uint16_t*)(base + L.dy) : nullptr;
  const int64_t np = pad64(N);
  hipError_t e = launch_rotate(r, x, xr, M, stream);
  if (e != hipSuccess) return fail(e, "paro_layer_loss: transform");
  int st = paro_w4_linear(nullptr, xr, qw, sc, zr, nullptr, yq, M, N, d, group, base + L.w4,
                          paro_w4_linear_workspace_size(nullptr, M, N, d), stream);
  if (st != PARO_OK) return st;
  // X W^T with the loss and dY in the epilogue, then the fixed-order sum
  if ((e = launch_nt_gemm_loss(x, w, M, N, d, yq, dy, np, part, stream)) != hipSuccess)
    return fail(e, "paro_layer_loss: X W^T");
  hipLaunchKernelGGL(loss_final_kernel, dim3(1), dim3(256), 0, stream, part, nt_tiles(M, N), loss);
  if ((e = hipGetLastError()) != hipSuccess) return fail(e, "paro_layer_loss: loss");
  if (!grad) return PARO_OK;

  float* dxr = (float*)(base + L.dxr);
  uint16_t* err = (uint16_t*)(base + L.e);
  uint16_t* et = (uint16_t*)(base + L.et);
  // The quantizer's pass over T W (its codes go to scratch) writes the
  // quantization error E = W_hat - T W in fp16; E^T [d][pad64(N)]
  if ((e = launch_quantize(r, w, N, d, group, (uint8_t*)(base + L.qw), (uint16_t*)(base + L.sc),
                           (uint8_t*)(base + L.zr), (int*)(base + L.flag), stream, err)) != hipSuccess)
    return fail(e, "paro_layer_loss: weight transform");
  if ((e = launch_transpose_pad(err, N, d, et, np, stream)) != hipSuccess)
    return fail(e, "paro_layer_loss: E transpose");
  // dX' [M][d] = dY [M][N] E [N][d] (fp32)
  if ((e = launch_nt_gemm_f32(dy, np, et, np, M, d, np, dxr, d, stream)) != hipSuccess)
    return fail(e, "paro_layer_loss: dY E");
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
