// gfx950 kernel for the online activation transform X' = X T^-1.
//
// Method: ParoQuant paper notes, section "关键设计" (independent Givens
// rotations on disjoint channel pairs inside each group, K stages, channel
// scaling) and "亮点与洞察" (all stages fused into one launch, activations
// and rotation parameters kept on chip); CSDN article section 3.1 (token,
// channel-group and pair parallelism).
//
// Mapping on CDNA4: one wavefront owns one 128- (or 256-) channel segment of
// a batch of tokens. Lane v holds the two members of one pair in fp32 VGPRs
// (two pairs per lane for 256-channel segments). Every stage is two fused
// multiply-adds per lane and token: the per-pair cosine/sine factors are
// deferred into per-channel scales that the host folds into the coefficients
// and applies once at the end. Between stages each lane keeps one of its two
// channels and fetches the other member of its next pair from another lane's
// register through a per-wave LDS tile that interleaves four tokens per
// 16-byte slot (b128 writes and reads, bank-conflict-free slots planned on the
// host). HBM traffic is one coalesced dword load and one dword store per lane
// and token; the schedule tables are read once per wavefront.
#include <cstring>

#include "paro_internal.h"

namespace paro {
namespace {

typedef float f4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ float half_lo(uint32_t v) {
  return (float)__builtin_bit_cast(_Float16, (uint16_t)(v & 0xffffu));
}
__device__ __forceinline__ float half_hi(uint32_t v) {
  return (float)__builtin_bit_cast(_Float16, (uint16_t)(v >> 16));
}
__device__ __forceinline__ uint32_t half_bits(float f) {
  return (uint32_t)__builtin_bit_cast(uint16_t, (_Float16)f);
}
__device__ __forceinline__ float as_f(uint32_t u) { return __builtin_bit_cast(float, u); }

// PPL: pairs per lane (1: 128-channel segments, 2: 256-channel segments).
// KMAX: compile-time bound on the number of stages (runtime K <= KMAX).
// FAST: factored two-FMA stage form (else the general 2x2 form).
template <int PPL, int KMAX, bool FAST>
__global__ __launch_bounds__(256) void rotate_kernel(const uint32_t* x, uint32_t* y,
                                                     const uint32_t* __restrict__ tab, int64_t M,
                                                     int64_t row_dw, int segs, int K, int tpw) {
  constexpr int NV = 64 * PPL;             // virtual lanes (pairs) per segment
  constexpr int T = PPL == 1 ? 8 : 4;      // tokens per batch
  constexpr int NQ = T / 4;                // 4-token LDS quads per batch
  constexpr int C = FAST ? 2 : 4;          // coefficients per stage
  constexpr bool TREG = KMAX <= 8;         // keep the whole schedule in VGPRs
  constexpr int KR = TREG ? KMAX : 0;
  __shared__ f4 lds_all[4][NQ * NV > 0 ? NQ * NV : 1];

  const int lane = threadIdx.x & 63;
  const int wid = threadIdx.x >> 6;
  const int64_t gw = (int64_t)blockIdx.x * 4 + wid;
  const int seg = (int)(gw % segs);
  const int64_t tok0 = (gw / segs) * (int64_t)tpw;
  if (tok0 >= M) return;
  const int64_t tok1 = (tok0 + tpw < M) ? tok0 + tpw : M;
  const int W = 1 + 2 * (K + 1) + C * K + 4;
  const uint32_t* tb = tab + (size_t)seg * W * NV + lane;
  char* lds = (char*)&lds_all[wid][0];
  const int ff = 3 + 2 * K + C * K;

  uint32_t ldsel[PPL], stoff[PPL], stsel[PPL];
  float lamX[PPL], lamB[PPL];
  uint32_t wr[KR + 1][PPL], rd[KR + 1][PPL];
  float cf[KR > 0 ? KR : 1][C][PPL];
#pragma unroll
  for (int h = 0; h < PPL; ++h) {
    ldsel[h] = tb[64 * h];
    lamX[h] = as_f(tb[(size_t)(ff + 0) * NV + 64 * h]);
    lamB[h] = as_f(tb[(size_t)(ff + 1) * NV + 64 * h]);
    stoff[h] = tb[(size_t)(ff + 2) * NV + 64 * h];
    stsel[h] = tb[(size_t)(ff + 3) * NV + 64 * h];
    if constexpr (TREG) {
#pragma unroll
      for (int tau = 0; tau <= KR; ++tau) {
        if (tau <= K) {
          wr[tau][h] = tb[(size_t)(1 + 2 * tau) * NV + 64 * h];
          rd[tau][h] = tb[(size_t)(2 + 2 * tau) * NV + 64 * h];
        }
      }
#pragma unroll
      for (int t = 0; t < KR; ++t) {
        if (t < K) {
#pragma unroll
          for (int e = 0; e < C; ++e) cf[t][e][h] = as_f(tb[(size_t)(3 + 2 * K + C * t + e) * NV + 64 * h]);
        }
      }
    }
  }

  auto wr_off = [&](int tau, int h) -> uint32_t {
    if constexpr (TREG) return wr[tau][h];
    else return tb[(size_t)(1 + 2 * tau) * NV + 64 * h];
  };
  auto rd_off = [&](int tau, int h) -> uint32_t {
    if constexpr (TREG) return rd[tau][h];
    else return tb[(size_t)(2 + 2 * tau) * NV + 64 * h];
  };
  auto coef = [&](int t, int e, int h) -> float {
    if constexpr (TREG) return cf[t][e][h];
    else return as_f(tb[(size_t)(3 + 2 * K + C * t + e) * NV + 64 * h]);
  };

  const int64_t seg_dw = (int64_t)seg * NV;
  float X[PPL][T], B[PPL][T];

  auto exchange = [&](int tau) {
#pragma unroll
    for (int q = 0; q < NQ; ++q) {
#pragma unroll
      for (int h = 0; h < PPL; ++h) {
        f4 v = {B[h][4 * q], B[h][4 * q + 1], B[h][4 * q + 2], B[h][4 * q + 3]};
        *(f4*)(lds + q * NV * 16 + wr_off(tau, h)) = v;
      }
    }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
#pragma unroll
    for (int q = 0; q < NQ; ++q) {
#pragma unroll
      for (int h = 0; h < PPL; ++h) {
        f4 v = *(const f4*)(lds + q * NV * 16 + rd_off(tau, h));
        B[h][4 * q] = v.x;
        B[h][4 * q + 1] = v.y;
        B[h][4 * q + 2] = v.z;
        B[h][4 * q + 3] = v.w;
      }
    }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  };

  for (int64_t t0 = tok0; t0 < tok1; t0 += T) {
    // ---- load (natural channel pairs), keep one member in X --------------------
#pragma unroll
    for (int i = 0; i < T; ++i) {
      const int64_t tok = t0 + i;
#pragma unroll
      for (int h = 0; h < PPL; ++h) {
        uint32_t v = 0;
        if (tok < tok1) v = x[tok * row_dw + seg_dw + 64 * h + lane];
        v = __builtin_amdgcn_perm(v, v, ldsel[h]);
        X[h][i] = half_lo(v);
        B[h][i] = half_hi(v);
      }
    }
    if constexpr (KMAX > 0) {
      exchange(0);
#pragma unroll
      for (int t = 0; t < KMAX; ++t) {
        if (t < K) {
#pragma unroll
          for (int h = 0; h < PPL; ++h) {
#pragma unroll
            for (int i = 0; i < T; ++i) {
              const float a = X[h][i], b = B[h][i];
              if constexpr (FAST) {
                X[h][i] = __builtin_fmaf(coef(t, 0, h), b, a);
                B[h][i] = __builtin_fmaf(coef(t, 1, h), a, b);
              } else {
                X[h][i] = __builtin_fmaf(coef(t, 1, h), b, coef(t, 0, h) * a);
                B[h][i] = __builtin_fmaf(coef(t, 2, h), a, coef(t, 3, h) * b);
              }
            }
          }
          exchange(t + 1);
        }
      }
    }
    // ---- apply the deferred scales, round to fp16, store the natural pair -------
#pragma unroll
    for (int i = 0; i < T; ++i) {
      const int64_t tok = t0 + i;
      if (tok < tok1) {
        char* row = (char*)(y + tok * row_dw + seg_dw);
#pragma unroll
        for (int h = 0; h < PPL; ++h) {
          const uint32_t ux = half_bits(X[h][i] * lamX[h]);
          const uint32_t ub = half_bits(B[h][i] * lamB[h]);
          *(uint32_t*)(row + stoff[h]) = __builtin_amdgcn_perm(ub, ux, stsel[h]);
        }
      }
    }
  }
}

template <int PPL, int KMAX, bool FAST>
hipError_t launch_t(const paro_rotation* r, const uint16_t* x, uint16_t* y, int64_t M,
                    hipStream_t stream) {
  const int segs = (int)(r->d / r->lay.seg_ch);
  constexpr int T = PPL == 1 ? 8 : 4;
  // about 4096 wavefronts in flight over the 256 CUs; tokens per wave a multiple of T
  int64_t per = (M * segs + 4095) / 4096;
  int64_t tpw = ((per + T - 1) / T) * T;
  if (tpw < T) tpw = T;
  const int64_t chunks = (M + tpw - 1) / tpw;
  const int64_t waves = chunks * segs;
  const int64_t blocks = (waves + 3) / 4;
  hipLaunchKernelGGL((rotate_kernel<PPL, KMAX, FAST>), dim3((unsigned)blocks), dim3(256), 0, stream,
                     (const uint32_t*)x, (uint32_t*)y, r->d_table, M, r->d / 2, segs, r->K,
                     (int)tpw);
  return hipGetLastError();
}

template <int PPL, bool FAST>
hipError_t launch_k(const paro_rotation* r, const uint16_t* x, uint16_t* y, int64_t M,
                    hipStream_t stream) {
  const int K = r->K;
  if (K == 0) return launch_t<PPL, 0, true>(r, x, y, M, stream);
  if (K <= 1) return launch_t<PPL, 1, FAST>(r, x, y, M, stream);
  if (K <= 2) return launch_t<PPL, 2, FAST>(r, x, y, M, stream);
  if (K <= 4) return launch_t<PPL, 4, FAST>(r, x, y, M, stream);
  if (K <= 8) return launch_t<PPL, 8, FAST>(r, x, y, M, stream);
  if (K <= 16) return launch_t<PPL, 16, FAST>(r, x, y, M, stream);
  return launch_t<PPL, 32, FAST>(r, x, y, M, stream);
}

}  // namespace

hipError_t launch_rotate(const paro_rotation* r, const uint16_t* x, uint16_t* y, int64_t M,
                         hipStream_t stream) {
  if (M == 0) return hipSuccess;
  if (r->lay.ppl == 1) {
    return r->lay.fast ? launch_k<1, true>(r, x, y, M, stream) : launch_k<1, false>(r, x, y, M, stream);
  }
  return r->lay.fast ? launch_k<2, true>(r, x, y, M, stream) : launch_k<2, false>(r, x, y, M, stream);
}

}  // namespace paro
