// C ABI of the rotated W4G128 linear library (declarations and argument
// contracts in include/paro.h).
#include <cstring>
#include <string>

#include "paro_internal.h"

namespace paro {

static thread_local std::string g_last_error;

void set_error(const std::string& msg) { g_last_error = msg; }

namespace {

bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

int hip_fail(hipError_t e, const char* what) {
  set_error(std::string(what) + ": " + hipGetErrorString(e));
  return PARO_ERR_HIP;
}

template <typename T>
int upload(T** dst, const std::vector<T>& src) {
  *dst = nullptr;
  if (src.empty()) return PARO_OK;
  hipError_t e = hipMalloc((void**)dst, src.size() * sizeof(T));
  if (e != hipSuccess) {
    *dst = nullptr;
    return hip_fail(e, "hipMalloc");
  }
  e = hipMemcpy(*dst, src.data(), src.size() * sizeof(T), hipMemcpyHostToDevice);
  if (e != hipSuccess) return hip_fail(e, "hipMemcpy");
  return PARO_OK;
}

void free_rotation(paro_rotation* r) {
  if (!r) return;
  if (r->d_table) (void)hipFree(r->d_table);
  if (r->d_wt_pairs) (void)hipFree(r->d_wt_pairs);
  if (r->d_wt_c) (void)hipFree(r->d_wt_c);
  if (r->d_wt_s) (void)hipFree(r->d_wt_s);
  if (r->d_alpha) (void)hipFree(r->d_alpha);
  if (r->d_bw) (void)hipFree(r->d_bw);
  delete r;
}

}  // namespace
}  // namespace paro

using namespace paro;

extern "C" {

const char* paro_status_string(int status) {
  switch (status) {
    case PARO_OK: return "PARO_OK";
    case PARO_ERR_NULL: return "PARO_ERR_NULL";
    case PARO_ERR_SHAPE: return "PARO_ERR_SHAPE";
    case PARO_ERR_PAIRING: return "PARO_ERR_PAIRING";
    case PARO_ERR_VALUE: return "PARO_ERR_VALUE";
    case PARO_ERR_ALIGN: return "PARO_ERR_ALIGN";
    case PARO_ERR_UNSUPPORTED: return "PARO_ERR_UNSUPPORTED";
    case PARO_ERR_WORKSPACE: return "PARO_ERR_WORKSPACE";
    case PARO_ERR_HIP: return "PARO_ERR_HIP";
    default: return "PARO_ERR_UNKNOWN";
  }
}

const char* paro_last_error(void) { return g_last_error.c_str(); }

int paro_rotation_plan_host(int64_t d, int32_t group, int32_t K, const int32_t* pairs,
                            const float* theta, const float* alpha, void* out, size_t out_bytes,
                            size_t* needed, int32_t layout[5]) {
  RotPlanHost plan;
  int st = build_rotation_plan(d, group, K, pairs, theta, alpha, &plan);
  if (st != PARO_OK) return st;
  const size_t bytes = plan.table.size() * sizeof(uint32_t);
  if (needed) *needed = bytes;
  if (layout) {
    layout[0] = plan.lay.seg_ch;
    layout[1] = plan.lay.ppl;
    layout[2] = plan.lay.words;
    layout[3] = plan.lay.fast ? 1 : 0;
    layout[4] = plan.lay.stages;
  }
  if (out) {
    if (out_bytes < bytes) {
      set_error("output buffer too small for the plan image");
      return PARO_ERR_WORKSPACE;
    }
    std::memcpy(out, plan.table.data(), bytes);
  }
  return PARO_OK;
}

int paro_device_init(void) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_fail(e, "paro_device_init: hipGetDevice");
  if (dev >= kMaxDevices) {
    set_error("paro_device_init: device ordinal too large");
    return PARO_ERR_UNSUPPORTED;
  }
  int st = xcd_dispatch_probe(dev);
  if (st == PARO_OK) st = noalloc_scratch_setup(dev);
  return st;
}

int paro_rotation_create(int64_t d, int32_t group, int32_t K, const int32_t* pairs,
                         const float* theta, const float* alpha, paro_rotation** out) {
  if (!out) {
    set_error("out is NULL");
    return PARO_ERR_NULL;
  }
  *out = nullptr;
  RotPlanHost plan;
  int st = build_rotation_plan(d, group, K, pairs, theta, alpha, &plan);
  if (st != PARO_OK) return st;
  paro_rotation* r = new paro_rotation();
  std::memset(r, 0, sizeof(*r));
  r->d = d;
  r->group = group;
  r->K = K;
  r->lay = plan.lay;
  hipError_t e = hipGetDevice(&r->device);
  if (e != hipSuccess) {
    free_rotation(r);
    return hip_fail(e, "hipGetDevice");
  }
  if ((st = paro_device_init()) != PARO_OK) {
    free_rotation(r);
    return st;
  }
  if ((st = upload(&r->d_table, plan.table)) != PARO_OK ||
      (st = upload(&r->d_wt_pairs, plan.wt_pairs)) != PARO_OK ||
      (st = upload(&r->d_wt_c, plan.wt_c)) != PARO_OK ||
      (st = upload(&r->d_wt_s, plan.wt_s)) != PARO_OK ||
      (st = upload(&r->d_alpha, plan.alpha)) != PARO_OK ||
      (st = upload(&r->d_bw, plan.bw)) != PARO_OK) {
    free_rotation(r);
    return st;
  }
  *out = r;
  return PARO_OK;
}

void paro_rotation_destroy(paro_rotation* r) { free_rotation(r); }

int paro_rotation_info(const paro_rotation* r, int64_t* d, int32_t* group, int32_t* K) {
  if (!r) {
    set_error("rotation handle is NULL");
    return PARO_ERR_NULL;
  }
  if (d) *d = r->d;
  if (group) *group = r->group;
  if (K) *K = r->K;
  return PARO_OK;
}

int paro_rotate(const paro_rotation* r, const uint16_t* x, uint16_t* y, int64_t M,
                hipStream_t stream) {
  if (!r) {
    set_error("paro_rotate: NULL handle");
    return PARO_ERR_NULL;
  }
  if (M < 0 || M > INT32_MAX) {
    set_error("paro_rotate: M must be in [0, 2^31 - 1]");
    return PARO_ERR_SHAPE;
  }
  if (M == 0) return PARO_OK;
  if (!x || !y) {
    set_error("paro_rotate: NULL tensor");
    return PARO_ERR_NULL;
  }
  if (!aligned16(x) || !aligned16(y)) {
    set_error("paro_rotate: x and y must be 16-byte aligned");
    return PARO_ERR_ALIGN;
  }
  hipError_t e = launch_rotate(r, x, y, M, stream);
  if (e != hipSuccess) return hip_fail(e, "paro_rotate launch");
  return PARO_OK;
}

int paro_quantize_weights(const paro_rotation* r, const uint16_t* w, int64_t N, int64_t d,
                          int32_t group, uint8_t* qweight, uint16_t* scales, uint8_t* zeros,
                          hipStream_t stream) {
  if (!w || !qweight || !scales || !zeros) {
    set_error("paro_quantize_weights: NULL tensor");
    return PARO_ERR_NULL;
  }
  if (N < 0 || d <= 0 || group <= 0) {
    set_error("paro_quantize_weights: bad sizes");
    return PARO_ERR_SHAPE;
  }
  if (group != 64 && group != 128 && group != 256) {
    set_error("paro_quantize_weights: group must be 64, 128 or 256");
    return PARO_ERR_UNSUPPORTED;
  }
  if (d % group) {
    set_error("paro_quantize_weights: d must be a multiple of group");
    return PARO_ERR_SHAPE;
  }
  if (r && (r->d != d || r->group != group)) {
    set_error("paro_quantize_weights: d/group differ from the rotation plan");
    return PARO_ERR_SHAPE;
  }
  if (!aligned16(w)) {
    set_error("paro_quantize_weights: w must be 16-byte aligned");
    return PARO_ERR_ALIGN;
  }
  if (N == 0) return PARO_OK;
  int* flag = nullptr;
  hipError_t e = hipMalloc((void**)&flag, sizeof(int));
  if (e != hipSuccess) return hip_fail(e, "hipMalloc(flag)");
  e = hipMemsetAsync(flag, 0, sizeof(int), stream);
  if (e == hipSuccess) e = launch_quantize(r, w, N, d, group, qweight, scales, zeros, flag, stream);
  int hflag = 0;
  if (e == hipSuccess) e = hipMemcpyAsync(&hflag, flag, sizeof(int), hipMemcpyDeviceToHost, stream);
  if (e == hipSuccess) e = hipStreamSynchronize(stream);
  (void)hipFree(flag);
  if (e != hipSuccess) return hip_fail(e, "paro_quantize_weights");
  if (hflag) {
    set_error("paro_quantize_weights: non-finite transformed weight or group scale");
    return PARO_ERR_VALUE;
  }
  return PARO_OK;
}

size_t paro_w4_linear_workspace_size(const paro_rotation* r, int64_t M, int64_t N, int64_t d) {
  if (M <= 0 || N <= 0 || d <= 0) return 0;
  auto round256 = [](size_t b) { return (b + 255) & ~(size_t)255; };
  if (M <= kDecodeMaxM) {
    size_t bytes = kDecodeCounterBytes;
    const size_t ksl = (size_t)((d / 128 + 3) / 4);
    if (ksl > 1) bytes += round256(ksl * (size_t)M * (size_t)N * 4);
    if (r && !decode_fuses_rotation(r, M, N, d)) bytes += round256((size_t)M * (size_t)d * 2);
    return bytes;
  }
  const size_t split = plan_w4_gemm(M, N, d).partial_bytes;
  if (!r && !split) return 0;
  return kDecodeCounterBytes + (r ? round256((size_t)M * (size_t)d * 2) : 0) + split;
}

}  // extern "C"

namespace paro {
namespace {

// Argument checks shared by paro_w4_linear and paro_w4_linear_noalloc
// (everything but the workspace). Returns PARO_OK, or an error with the
// message set; *noop is set when M == 0 (nothing to do).
int check_w4_linear(const char* fn, const paro_rotation* r, const uint16_t* x,
                    const uint8_t* qweight, const uint16_t* scales, const uint8_t* zeros,
                    const uint16_t* bias, const uint16_t* y, int64_t M, int64_t N, int64_t d,
                    int32_t group, bool* noop) {
  *noop = false;
  const std::string f(fn);
  if (M < 0 || N <= 0 || d <= 0) {
    set_error(f + ": bad sizes");
    return PARO_ERR_SHAPE;
  }
  if (group != 64 && group != 128 && group != 256) {
    set_error(f + ": group must be 64, 128 or 256");
    return PARO_ERR_UNSUPPORTED;
  }
  if (N % 16 || d % 128 || d % group) {
    set_error(f + ": N must be a multiple of 16, d of 128 and of group");
    return PARO_ERR_SHAPE;
  }
  // (the kernels address one tile of rows with 32-bit byte offsets)
  if (N > (int64_t(1) << 30) || d > (int64_t(1) << 22) || M > (int64_t(1) << 31) / 2) {
    set_error(f + ": sizes too large (N <= 2^30, d <= 2^22, M < 2^30)");
    return PARO_ERR_UNSUPPORTED;
  }
  if (r && (r->d != d || r->group != group)) {
    set_error(f + ": d or group differs from the rotation plan");
    return PARO_ERR_SHAPE;
  }
  if (M == 0) {
    *noop = true;
    return PARO_OK;
  }
  if (!x || !qweight || !scales || !zeros || !y) {
    set_error(f + ": NULL tensor");
    return PARO_ERR_NULL;
  }
  if (!aligned16(x) || !aligned16(qweight) || !aligned16(y) || (bias && ((uintptr_t)bias & 7))) {
    set_error(f + ": x, qweight, y must be 16-byte aligned (bias 8-byte)");
    return PARO_ERR_ALIGN;
  }
  if (M <= kDecodeMaxM && (uint64_t)((d / 128 + 3) / 4) * (uint64_t)M * (uint64_t)N * 4 >= (1ull << 31)) {
    set_error(f + ": ceil(d / 512) * M * N * 4 must be below 2^31 for M <= 64");
    return PARO_ERR_UNSUPPORTED;
  }
  return PARO_OK;
}

// The smallest workspace paro_w4_linear runs with: as reported for M <= 64,
// the transformed activations (and the counters before them) for M > 64; the
// stream-K partial tiles of the large-batch kernel only speed the call up.
size_t w4_linear_min_workspace(const paro_rotation* r, int64_t M, int64_t N, int64_t d) {
  if (M <= kDecodeMaxM || M <= 0) return paro_w4_linear_workspace_size(r, M, N, d);
  if (!r) return 0;
  return kDecodeCounterBytes + (((size_t)M * (size_t)d * 2 + 255) & ~(size_t)255);
}

// The launches of the W4 linear on a checked workspace ws of ws_bytes bytes
// (at least w4_linear_min_workspace; NULL when that is 0).
int run_w4_linear(const paro_rotation* r, const uint16_t* x, const uint8_t* qweight,
                  const uint16_t* scales, const uint8_t* zeros, const uint16_t* bias, uint16_t* y,
                  int64_t M, int64_t N, int64_t d, int32_t group, char* ws, size_t ws_bytes,
                  hipStream_t stream) {
  hipError_t e = hipSuccess;
  if (M <= kDecodeMaxM) {
    const paro_rotation* fused = r;
    const uint16_t* xin = x;
    if (r && !decode_fuses_rotation(r, M, N, d)) {
      // stand-alone transform into the workspace tail, then the plain kernel
      uint16_t* xr = (uint16_t*)(ws + ws_bytes - (((size_t)M * (size_t)d * 2 + 255) & ~(size_t)255));
      e = launch_rotate(r, x, xr, M, stream);
      if (e != hipSuccess) return hip_fail(e, "paro_w4_linear rotate launch");
      xin = xr;
      fused = nullptr;
    }
    e = launch_w4_decode(xin, qweight, scales, zeros, bias, y, M, N, d, group, fused, ws, stream);
  } else {
    const uint16_t* xin = x;
    const size_t xbytes = r ? (((size_t)M * (size_t)d * 2 + 255) & ~(size_t)255) : 0;
    if (r) {
      uint16_t* xr = (uint16_t*)(ws + kDecodeCounterBytes);
      e = launch_rotate(r, x, xr, M, stream);
      if (e != hipSuccess) return hip_fail(e, "paro_w4_linear rotate launch");
      xin = xr;
    }
    // split-k partial tiles after the counters and X', when the workspace holds them
    const GemmPlan plan = plan_w4_gemm(M, N, d);
    const bool split = plan.partial_bytes && ws && ws_bytes >= kDecodeCounterBytes + xbytes + plan.partial_bytes;
    e = launch_w4_gemm(xin, qweight, scales, zeros, bias, y, M, N, d, group, split ? (uint32_t*)ws : nullptr,
                       split ? (float*)(ws + kDecodeCounterBytes + xbytes) : nullptr, stream);
  }
  if (e != hipSuccess) return hip_fail(e, "paro_w4_linear launch");
  return PARO_OK;
}

}  // namespace
}  // namespace paro

extern "C" {

int paro_w4_linear(const paro_rotation* r, const uint16_t* x, const uint8_t* qweight,
                   const uint16_t* scales, const uint8_t* zeros, const uint16_t* bias,
                   uint16_t* y, int64_t M, int64_t N, int64_t d, int32_t group,
                   void* workspace, size_t workspace_bytes, hipStream_t stream) {
  bool noop = false;
  int st = check_w4_linear("paro_w4_linear", r, x, qweight, scales, zeros, bias, y, M, N, d, group,
                           &noop);
  if (st != PARO_OK || noop) return st;
  const size_t need = w4_linear_min_workspace(r, M, N, d);
  if (need && (!workspace || workspace_bytes < need)) {
    set_error("paro_w4_linear: workspace missing or smaller than the minimum (see paro_w4_linear_workspace_size)");
    return PARO_ERR_WORKSPACE;
  }
  if (workspace && ((uintptr_t)workspace & 255)) {
    set_error("paro_w4_linear: workspace must be 256-byte aligned");
    return PARO_ERR_ALIGN;
  }
  return run_w4_linear(r, x, qweight, scales, zeros, bias, y, M, N, d, group, (char*)workspace,
                       workspace ? workspace_bytes : 0, stream);
}

int paro_w4_linear_noalloc(const paro_rotation* r, const uint16_t* x, const uint8_t* qweight,
                           const uint16_t* scales, const uint8_t* zeros, const uint16_t* bias,
                           uint16_t* y, int64_t M, int64_t N, int64_t d, int32_t group,
                           hipStream_t stream) {
  bool noop = false;
  int st = check_w4_linear("paro_w4_linear_noalloc", r, x, qweight, scales, zeros, bias, y, M, N, d,
                           group, &noop);
  if (st != PARO_OK || noop) return st;
  const size_t need = w4_linear_min_workspace(r, M, N, d);
  if (need > kNoallocScratchBytes) {
    set_error("paro_w4_linear_noalloc: these sizes need " + std::to_string(need) +
              " bytes of workspace, more than the static scratch's " +
              std::to_string(kNoallocScratchBytes));
    return PARO_ERR_WORKSPACE;
  }
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_fail(e, "paro_w4_linear_noalloc: hipGetDevice");
  char* ws = (char*)noalloc_scratch(dev);
  if (!ws) {
    set_error("paro_w4_linear_noalloc: paro_device_init has not run on this device");
    return PARO_ERR_UNSUPPORTED;
  }
  return run_w4_linear(r, x, qweight, scales, zeros, bias, y, M, N, d, group, ws, kNoallocScratchBytes, stream);
}


size_t paro_rotation_backward_workspace_size(const paro_rotation* r, int64_t M) {
  if (!r || M <= 0) return 0;
  return (paro::rotate_backward_scratch_bytes(r, M) + 255) & ~(size_t)255;
}

int paro_rotation_backward(const paro_rotation* r, int32_t side, const uint16_t* x,
                           const float* gy, float* gx, float* dtheta, float* dalpha, int64_t M,
                           void* workspace, size_t workspace_bytes, hipStream_t stream) {
  using namespace paro;
  if (!r) {
    set_error("paro_rotation_backward: NULL rotation");
    return PARO_ERR_NULL;
  }
  if (side != PARO_SIDE_ACTIVATION && side != PARO_SIDE_WEIGHT) {
    set_error("paro_rotation_backward: side must be PARO_SIDE_ACTIVATION or PARO_SIDE_WEIGHT");
    return PARO_ERR_VALUE;
  }
  if (M < 0 || M >= (int64_t(1) << 31)) {
    set_error("paro_rotation_backward: M must be in [0, 2^31)");
    return PARO_ERR_SHAPE;
  }
  if (!dalpha || (r->K > 0 && !dtheta) || (M > 0 && (!x || !gy))) {
    set_error("paro_rotation_backward: NULL tensor");
    return PARO_ERR_NULL;
  }
  if (((uintptr_t)x & 3) || ((uintptr_t)gy & 7) || ((uintptr_t)gx & 7) || ((uintptr_t)dtheta & 3) ||
      ((uintptr_t)dalpha & 3)) {
    set_error("paro_rotation_backward: x must be 4-byte aligned, gy and gx 8-byte aligned");
    return PARO_ERR_ALIGN;
  }
  const size_t need = paro_rotation_backward_workspace_size(r, M);
  if (need && (!workspace || workspace_bytes < need)) {
    set_error("paro_rotation_backward: workspace missing or smaller than "
              "paro_rotation_backward_workspace_size");
    return PARO_ERR_WORKSPACE;
  }
  if (need && ((uintptr_t)workspace & 255)) {
    set_error("paro_rotation_backward: workspace must be 256-byte aligned");
    return PARO_ERR_ALIGN;
  }
  hipError_t e = launch_rotate_backward(r, side == PARO_SIDE_WEIGHT, x, gy, gx, dtheta, dalpha, M,
                                        workspace, stream);
  if (e != hipSuccess) return hip_fail(e, "paro_rotation_backward launch");
  return PARO_OK;
}

size_t paro_layer_loss_workspace_size(const paro_rotation* r, int64_t M, int64_t N, int64_t d,
                                      int32_t with_gradients) {
  if (!r || M <= 0 || N <= 0 || d != r->d) return 0;
  return paro::layer_loss_scratch_bytes(r, M, N, d, with_gradients != 0);
}

int paro_layer_loss(const paro_rotation* r, const uint16_t* x, const uint16_t* w,
                    const uint8_t* qweight, const uint16_t* scales, const uint8_t* zeros, int64_t M,
                    int64_t N, int64_t d, int32_t group, float* loss, float* dtheta, float* dalpha,
                    void* workspace, size_t workspace_bytes, hipStream_t stream) {
  using namespace paro;
  if (!r || !loss) {
    set_error("paro_layer_loss: NULL rotation or loss");
    return PARO_ERR_NULL;
  }
  if (M < 0 || N <= 0 || d != r->d || group != r->group || N % 16 || M >= (int64_t(1) << 30) ||
      N >= (int64_t(1) << 30)) {
    set_error("paro_layer_loss: sizes (d and group of the plan, N % 16 == 0, 0 <= M, N < 2^30)");
    return PARO_ERR_SHAPE;
  }
  const bool grad = dtheta || dalpha;
  if (M == 0) {  // no rows: zero loss and gradients
    hipError_t e = launch_fill_zero(loss, 1, stream);
    if (e == hipSuccess && dtheta) e = launch_fill_zero(dtheta, (int64_t)r->K * (d / 2), stream);
    if (e == hipSuccess && dalpha) e = launch_fill_zero(dalpha, d, stream);
    return e == hipSuccess ? PARO_OK : hip_fail(e, "paro_layer_loss");
  }
  if (!x || !w || !qweight || !scales || !zeros) {
    set_error("paro_layer_loss: NULL tensor");
    return PARO_ERR_NULL;
  }
  if (!aligned16(x) || !aligned16(w) || !aligned16(qweight) || ((uintptr_t)loss & 3) ||
      ((uintptr_t)dtheta & 3) || ((uintptr_t)dalpha & 3)) {
    set_error("paro_layer_loss: x, w, qweight must be 16-byte aligned");
    return PARO_ERR_ALIGN;
  }
  const size_t need = layer_loss_scratch_bytes(r, M, N, d, grad);
  if (!workspace || workspace_bytes < need) {
    set_error("paro_layer_loss: workspace missing or smaller than paro_layer_loss_workspace_size");
    return PARO_ERR_WORKSPACE;
  }
  if ((uintptr_t)workspace & 255) {
    set_error("paro_layer_loss: workspace must be 256-byte aligned");
    return PARO_ERR_ALIGN;
  }
  return run_layer_loss(r, x, w, qweight, scales, zeros, M, N, d, group, loss, dtheta, dalpha,
                        workspace, stream);
}

int paro_stream_copy(const void* src, void* dst, size_t bytes, int32_t blocks, hipStream_t stream) {
  if (bytes == 0) return PARO_OK;
  if (!src || !dst) {
    set_error("paro_stream_copy: NULL pointer");
    return PARO_ERR_NULL;
  }
  if (!aligned16(src) || !aligned16(dst) || (bytes & 15)) {
    set_error("paro_stream_copy: pointers must be 16-byte aligned and bytes a multiple of 16");
    return PARO_ERR_ALIGN;
  }
  if (blocks < 1 || blocks > (1 << 20)) {
    set_error("paro_stream_copy: blocks must be in [1, 2^20]");
    return PARO_ERR_SHAPE;
  }
  hipError_t e = launch_stream_copy(src, dst, bytes, blocks, stream);
  if (e != hipSuccess) return hip_fail(e, "paro_stream_copy launch");
  return PARO_OK;
}

int paro_mfma_loop(const void* src, int64_t n, float* out, int32_t blocks, int32_t iters, hipStream_t stream) {
  if (!src || !out) {
    set_error("paro_mfma_loop: NULL pointer");
    return PARO_ERR_NULL;
  }
  if (!aligned16(src) || ((uintptr_t)out & 3)) {
    set_error("paro_mfma_loop: src must be 16-byte aligned, out 4-byte aligned");
    return PARO_ERR_ALIGN;
  }
  if (n < 8 || n % 8 || n > (int64_t(1) << 30) || blocks < 1 || blocks > (1 << 16) || iters < 0) {
    set_error("paro_mfma_loop: n a multiple of 8 in [8, 2^30], blocks in [1, 2^16], iters >= 0");
    return PARO_ERR_SHAPE;
  }
  hipError_t e = launch_mfma_loop(src, n / 8, out, blocks, iters, stream);
  if (e != hipSuccess) return hip_fail(e, "paro_mfma_loop launch");
  return PARO_OK;
}

}  // extern "C"
