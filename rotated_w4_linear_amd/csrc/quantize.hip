// gfx950 kernel for the offline weight transform T W and W4 group quantization.
//
// Method: ParoQuant paper notes, section "关键设计" (W scaled by alpha, then the
// K independent-rotation stages) and "损失函数 / 训练策略" / "主实验" (int4
// weights with a per-group scale s and zero z, group 128). The quantizer
// formula is not on the pages; this library uses asymmetric min/max
// round-to-nearest over 15 steps with the range widened to include zero, an
// fp16 scale and an integer zero, in a fixed fp32 order of operations so that
// codes, scales and zeros are reproducible bit for bit:
//   u_k = fl(w_k alpha_k); per pair u_i = fl(fl(c a) - fl(s b)), u_j = fl(fl(s a) + fl(c b));
//   s32 = fl(fl(max(0,max u) - min(0,min u)) / 15); s16 = fp16_rne(s32) (0 -> 1.0);
//   z = clamp(rint(fl(-mn / s16)), 0, 15); q = clamp(rint(fl(u / s16)) + z, 0, 15).
// The file is compiled without floating-point contraction.
//
// One wavefront owns one (output row, group): the group lives in a
// wave-private LDS slice, each lane updates its own pairs per stage, and
// min/max are wave reductions (exact in any order).
#include <cmath>

#include "paro_internal.h"

#pragma clang fp contract(off)

namespace paro {
namespace {

// Wave-wide min, max and or, exact in any order: within each row of 16 lanes
// by DPP moves (lane i with i ^ 1, i ^ 2, its mirror in the half row and in
// the row), then the four rows' values read from lanes 0, 16, 32 and 48.
__device__ __forceinline__ int dpp_row(int v, int ctrl_step) {
  switch (ctrl_step) {
    case 0: return __builtin_amdgcn_mov_dpp(v, 0xB1, 0xF, 0xF, false);   // quad_perm [1, 0, 3, 2]
    case 1: return __builtin_amdgcn_mov_dpp(v, 0x4E, 0xF, 0xF, false);   // quad_perm [2, 3, 0, 1]
    case 2: return __builtin_amdgcn_mov_dpp(v, 0x141, 0xF, 0xF, false);  // row_half_mirror
    default: return __builtin_amdgcn_mov_dpp(v, 0x140, 0xF, 0xF, false); // row_mirror
  }
}
__device__ __forceinline__ float wave_min(float v) {
#pragma unroll
  for (int k = 0; k < 4; ++k) v = fminf(v, __builtin_bit_cast(float, dpp_row(__builtin_bit_cast(int, v), k)));
  const int b = __builtin_bit_cast(int, v);
  return fminf(fminf(__builtin_bit_cast(float, __builtin_amdgcn_readlane(b, 0)),
                     __builtin_bit_cast(float, __builtin_amdgcn_readlane(b, 16))),
               fminf(__builtin_bit_cast(float, __builtin_amdgcn_readlane(b, 32)),
                     __builtin_bit_cast(float, __builtin_amdgcn_readlane(b, 48))));
}
__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int k = 0; k < 4; ++k) v = fmaxf(v, __builtin_bit_cast(float, dpp_row(__builtin_bit_cast(int, v), k)));
  const int b = __builtin_bit_cast(int, v);
  return fmaxf(fmaxf(__builtin_bit_cast(float, __builtin_amdgcn_readlane(b, 0)),
                     __builtin_bit_cast(float, __builtin_amdgcn_readlane(b, 16))),
               fmaxf(__builtin_bit_cast(float, __builtin_amdgcn_readlane(b, 32)),
                     __builtin_bit_cast(float, __builtin_amdgcn_readlane(b, 48))));
}
__device__ __forceinline__ int wave_or(int v) {
#pragma unroll
  for (int k = 0; k < 4; ++k) v |= dpp_row(v, k);
  return __builtin_amdgcn_readlane(v, 0) | __builtin_amdgcn_readlane(v, 16) |
         __builtin_amdgcn_readlane(v, 32) | __builtin_amdgcn_readlane(v, 48);
}

__global__ __launch_bounds__(256) void quantize_kernel(
    const uint16_t* __restrict__ w, int64_t N, int64_t d, int G, int K,
    const uint32_t* __restrict__ wt_pairs, const float* __restrict__ wt_c,
    const float* __restrict__ wt_s, const float* __restrict__ alpha, uint8_t* __restrict__ qweight,
    uint16_t* __restrict__ scales, uint8_t* __restrict__ zeros, int* __restrict__ flag,
    float* __restrict__ uout) {
  __shared__ float buf[4][256];
  const int lane = threadIdx.x & 63;
  // wave-uniform: the item, row and group stay in scalar registers, and every
  // table and row address is a scalar base plus the lane's offset
  const int wid = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int64_t groups = d / G;
  const int64_t total = N * groups;
  float* u = buf[wid];
  const int half = G / 2;
  // Each lane reads its weights as dwords (two consecutive fp16), and the
  // next item's are requested before the current one is transformed.
  // Items item0, item0 + stride, ...: (row, group) advances by (sn, sg) with
  // a carry, so no item needs a division.
  const int64_t stride = (int64_t)gridDim.x * 4;
  const int64_t sn = stride / groups, sg = stride - sn * groups;
  uint32_t nxt[2] = {0u, 0u};
  auto fetch = [&](int64_t item, int64_t n, int64_t g) {
    if (item >= total) return;
    const uint32_t* wr = (const uint32_t*)(w + n * d + g * G);
#pragma unroll
    for (int r = 0; r < 2; ++r)
      if (lane + 64 * r < half) nxt[r] = wr[lane + 64 * r];
  };
  const int64_t item0 = (int64_t)blockIdx.x * 4 + wid;
  int64_t n = item0 / groups, g = item0 - (item0 / groups) * groups;
  fetch(item0, n, g);
  for (int64_t item = item0; item < total; item += stride) {
    const uint32_t cur[2] = {nxt[0], nxt[1]};
    int64_t nn = n + sn, ng = g + sg;
    if (ng >= groups) {
      ng -= groups;
      ++nn;
    }
    fetch(item + stride, nn, ng);
#pragma unroll
    for (int r = 0; r < 2; ++r) {
      const int k2 = lane + 64 * r;
      if (k2 < half) {
        float v0 = (float)__builtin_bit_cast(_Float16, (uint16_t)(cur[r] & 0xffffu));
        float v1 = (float)__builtin_bit_cast(_Float16, (uint16_t)(cur[r] >> 16));
        if (alpha) {
          v0 = v0 * alpha[g * G + 2 * k2];
          v1 = v1 * alpha[g * G + 2 * k2 + 1];
        }
        u[2 * k2] = v0;
        u[2 * k2 + 1] = v1;
      }
    }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    for (int t = 0; t < K; ++t) {
      const size_t base = ((size_t)g * K + t) * half;
      for (int p = lane; p < half; p += 64) {
        const uint32_t ij = wt_pairs[base + p];
        const int i = (int)(ij & 0xffffu), j = (int)(ij >> 16);
        const float c = wt_c[base + p], s = wt_s[base + p];
        const float a = u[i], b = u[j];
        const float ca = c * a, sb = s * b, sa = s * a, cb = c * b;
        u[i] = ca - sb;
        u[j] = sa + cb;
      }
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    }
    if (uout) {  // the transformed row itself (fp32), for the layer loss's gradients
      for (int k = lane; k < G; k += 64) uout[n * d + g * G + k] = u[k];
    }
    float mn = 0.0f, mx = 0.0f;
    int bad = 0;
    for (int k = lane; k < G; k += 64) {
      const float v = u[k];
      bad |= !__builtin_isfinite(v);
      mn = fminf(mn, v);
      mx = fmaxf(mx, v);
    }
    mn = wave_min(mn);
    mx = wave_max(mx);
    bad = wave_or(bad);
    const float range = mx - mn;
    const float s32 = range / 15.0f;
    _Float16 s16 = (_Float16)s32;
    float sq = (float)s16;
    if (bad || !__builtin_isfinite(sq)) {
      if (lane == 0) atomicOr(flag, 1);
    }
    if (sq == 0.0f) {
      s16 = (_Float16)1.0f;
      sq = 1.0f;
    }
    const float negmn = -mn;
    const float zf = fminf(fmaxf(rintf(negmn / sq), 0.0f), 15.0f);
    for (int b = lane; b < half; b += 64) {
      const float q0f = fminf(fmaxf(rintf(u[2 * b] / sq) + zf, 0.0f), 15.0f);
      const float q1f = fminf(fmaxf(rintf(u[2 * b + 1] / sq) + zf, 0.0f), 15.0f);
      const uint32_t q0 = (uint32_t)q0f, q1 = (uint32_t)q1f;
      qweight[n * (d / 2) + g * half + b] = (uint8_t)(q0 | (q1 << 4));
    }
    if (lane == 0) {
      scales[n * groups + g] = __builtin_bit_cast(uint16_t, s16);
      zeros[n * groups + g] = (uint8_t)zf;
    }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    n = nn;
    g = ng;
  }
}

}  // namespace

hipError_t launch_quantize(const paro_rotation* r, const uint16_t* w, int64_t N, int64_t d,
                           int group, uint8_t* qweight, uint16_t* scales, uint8_t* zeros,
                           int* d_flag, hipStream_t stream, float* uout) {
  const int64_t total = N * (d / group);
  if (total == 0) return hipSuccess;
  int64_t blocks = (total + 3) / 4;
  if (blocks > 16384) blocks = 16384;
  hipLaunchKernelGGL(quantize_kernel, dim3((unsigned)blocks), dim3(256), 0, stream, w, N, d, group,
                     r ? r->K : 0, r ? r->d_wt_pairs : nullptr, r ? r->d_wt_c : nullptr,
                     r ? r->d_wt_s : nullptr, r ? r->d_alpha : nullptr, qweight, scales, zeros,
                     d_flag, uout);
  return hipGetLastError();
}

}  // namespace paro
