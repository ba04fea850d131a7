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
// One wavefront owns one or two (output row, group) items at a time: each
// group lives in a wave-private LDS slice, each lane updates its own pairs per
// stage, and min/max are wave reductions (exact in any order).
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

// NI: items per wavefront step. Two for groups of up to 128 channels: the
// two items' stage chains (dependent LDS round trips) then overlap. One for
// groups of 256 channels, whose slice fills the wavefront's 256 floats.
// Slot r (0, 1) of a lane is pair `lane` of item r (NI = 2; item r's slice at
// u + 128 r) or pair lane + 64 r of the one item (NI = 1).
template <int NI>
__global__ __launch_bounds__(256) void quantize_kernel(
    const uint16_t* __restrict__ w, int64_t N, int64_t d, int G, int K,
    const uint32_t* __restrict__ wt_pairs, const float* __restrict__ wt_c,
    const float* __restrict__ wt_s, const float* __restrict__ alpha, uint8_t* __restrict__ qweight,
    uint16_t* __restrict__ scales, uint8_t* __restrict__ zeros, int* __restrict__ flag,
    uint16_t* __restrict__ err) {
  __shared__ float buf[4][256];
  constexpr int SL = 128;  // floats between the two items' slices (NI = 2)
  const int lane = threadIdx.x & 63;
  // wave-uniform: items, rows and groups stay in scalar registers, and every
  // table and row address is a scalar base plus the lane's offset
  const int wid = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int64_t groups = d / G;
  const int64_t total = N * groups;
  float* u = buf[wid];
  const int half = G / 2;
  auto item_of = [](int r) { return NI == 2 ? r : 0; };
  auto pair_of = [&](int r) { return NI == 2 ? lane : lane + 64 * r; };
  // A step takes items item, item + 1 (NI = 2): the second is the next group
  // of the same row, or group 0 of the next row.
  auto second = [&](int64_t n, int64_t g, int64_t& n1, int64_t& g1) {
    g1 = g + 1;
    n1 = n;
    if (g1 == groups) {
      g1 = 0;
      ++n1;
    }
  };
  // Each lane reads its weights as dwords (two consecutive fp16), and the
  // next step's are requested before the current one is transformed. Steps
  // item0, item0 + stride, ...: (row, group) advances by (sn, sg) with a
  // carry, so no step needs a division.
  const int64_t stride = (int64_t)gridDim.x * 4 * NI;
  const int64_t sn = stride / groups, sg = stride - sn * groups;
  uint32_t nxt[2] = {0u, 0u};
  auto fetch = [&](int64_t item, int64_t n, int64_t g) {
    int64_t n1, g1;
    second(n, g, n1, g1);
#pragma unroll
    for (int r = 0; r < 2; ++r) {
      const int q = item_of(r), p = pair_of(r);
      if (item + q < total && p < half)
        nxt[r] = ((const uint32_t*)(w + (q ? n1 : n) * d + (q ? g1 : g) * G))[p];
    }
  };
  const int64_t item0 = ((int64_t)blockIdx.x * 4 + wid) * NI;
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
    int64_t n1, g1;
    second(n, g, n1, g1);
    const int ni = (NI == 2 && item + 1 < total) ? 2 : 1;  // items of this step
#pragma unroll
    for (int r = 0; r < 2; ++r) {
      const int q = item_of(r), p = pair_of(r);
      if (p < half) {
        const int64_t gq = q ? g1 : g;
        float v0 = (float)__builtin_bit_cast(_Float16, (uint16_t)(cur[r] & 0xffffu));
        float v1 = (float)__builtin_bit_cast(_Float16, (uint16_t)(cur[r] >> 16));
        if (alpha) {
          v0 = v0 * alpha[gq * G + 2 * p];
          v1 = v1 * alpha[gq * G + 2 * p + 1];
        }
        u[SL * q + 2 * p] = v0;
        u[SL * q + 2 * p + 1] = v1;
      }
    }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    for (int t = 0; t < K; ++t) {
#pragma unroll
      for (int r = 0; r < 2; ++r) {
        const int q = item_of(r), p = pair_of(r);
        if (p < half) {
          const size_t e = ((size_t)(q ? g1 : g) * K + t) * half + p;
          const uint32_t ij = wt_pairs[e];
          const int i = SL * q + (int)(ij & 0xffffu), j = SL * q + (int)(ij >> 16);
          const float c = wt_c[e], s = wt_s[e];
          const float a = u[i], b = u[j];
          const float ca = c * a, sb = s * b, sa = s * a, cb = c * b;
          u[i] = ca - sb;
          u[j] = sa + cb;
        }
      }
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    }
    // per item: min / max / non-finite over the wave, scale, zero, codes
    float mn[NI], mx[NI];
    int bad[NI];
#pragma unroll
    for (int q = 0; q < NI; ++q) {
      mn[q] = 0.0f;
      mx[q] = 0.0f;
      bad[q] = 0;
      if (q < ni) {
        const int64_t nq = q ? n1 : n, gq = q ? g1 : g;
        for (int k = lane; k < G; k += 64) {
          const float v = u[SL * q + k];
          bad[q] |= !__builtin_isfinite(v);
          mn[q] = fminf(mn[q], v);
          mx[q] = fmaxf(mx[q], v);
        }
      }
    }
#pragma unroll
    for (int q = 0; q < NI; ++q) {
      mn[q] = wave_min(mn[q]);
      mx[q] = wave_max(mx[q]);
      bad[q] = wave_or(bad[q]);
    }
#pragma unroll
    for (int q = 0; q < NI; ++q) {
      if (q < ni) {
        const int64_t nq = q ? n1 : n, gq = q ? g1 : g;
        const float range = mx[q] - mn[q];
        const float s32 = range / 15.0f;
        _Float16 s16 = (_Float16)s32;
        float sq = (float)s16;
        if (bad[q] || !__builtin_isfinite(sq)) {
          if (lane == 0) atomicOr(flag, 1);
        }
        if (sq == 0.0f) {
          s16 = (_Float16)1.0f;
          sq = 1.0f;
        }
        const float negmn = -mn[q];
        const float zf = fminf(fmaxf(rintf(negmn / sq), 0.0f), 15.0f);
        for (int b = lane; b < half; b += 64) {
          // byte b of the group: byte b % 4 of the word of channels 8 (b / 4) ..
          // + 7, which holds channels c0 and c0 + 2 (low, high nibble) with
          // c0 = 0, 4, 1, 5 for bytes 0 .. 3 (even channels in the word's low
          // half, odd ones in its high half)
          const int c0 = 8 * (b >> 2) + ((b & 1) << 2) + ((b >> 1) & 1);
          const float u0 = u[SL * q + c0], u1 = u[SL * q + c0 + 2];
          const float q0f = fminf(fmaxf(rintf(u0 / sq) + zf, 0.0f), 15.0f);
          const float q1f = fminf(fmaxf(rintf(u1 / sq) + zf, 0.0f), 15.0f);
          const uint32_t q0 = (uint32_t)q0f, q1 = (uint32_t)q1f;
          qweight[nq * (d / 2) + gq * half + b] = (uint8_t)(q0 | (q1 << 4));
          if (err) {
            // the quantization error E = (q - z) s - T W ((q - z) s is exact in
            // fp32), rounded once to fp16
            uint16_t* e = err + nq * d + gq * G + c0;
            e[0] = __builtin_bit_cast(uint16_t, (_Float16)((q0f - zf) * sq - u0));
            e[2] = __builtin_bit_cast(uint16_t, (_Float16)((q1f - zf) * sq - u1));
          }
        }
        if (lane == 0) {
          scales[nq * groups + gq] = __builtin_bit_cast(uint16_t, s16);
          zeros[nq * groups + gq] = (uint8_t)zf;
        }
      }
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
                           int* d_flag, hipStream_t stream, uint16_t* err) {
  const int64_t total = N * (d / group);
  if (total == 0) return hipSuccess;
  const int ni = group <= 128 ? 2 : 1;
  int64_t blocks = (total + 4 * ni - 1) / (4 * ni);
  if (blocks > 16384) blocks = 16384;
  auto kern = ni == 2 ? quantize_kernel<2> : quantize_kernel<1>;
  hipLaunchKernelGGL(kern, dim3((unsigned)blocks), dim3(256), 0, stream, w, N, d, group,
                     r ? r->K : 0, r ? r->d_wt_pairs : nullptr, r ? r->d_wt_c : nullptr,
                     r ? r->d_wt_s : nullptr, r ? r->d_alpha : nullptr, qweight, scales, zeros,
                     d_flag, err);
  return hipGetLastError();
}

}  // namespace paro
