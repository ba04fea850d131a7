// gfx950 kernels for the W4G128 linear layer on rotated activations:
//   Y[m][n] = sum_k X'[m][k] (q[n][k] - z[n][k/128]) s[n][k/128] + b[n]
// (CSDN article section 2.1: Y = (X T^-1)(T W) + b; paper notes "主实验":
// 4-bit weights, group 128).
//
// Both kernels use the gfx950 MFMA v_mfma_f32_16x16x32_f16 with the
// dequantized weights as operand A (16 output channels x 32 k) and the
// activations as operand B (32 k x 16 tokens), so each lane's accumulator
// holds four consecutive output channels of one token and the epilogue stores
// 8 bytes per lane. Dequantization: two nibbles are spread into the mantissas
// of two fp16 1024.0 values with v_perm, (1024 + q) - (1024 + z) = q - z is
// exact in packed fp16, and one packed multiply by the fp16 scale rounds once.
//
//  * decode (M <= 16): weight streaming. A workgroup owns 16 output channels
//    and all of d; its four wavefronts split d, each lane streams 16 bytes of
//    packed weights per group, and the partial 16x16 tiles are summed through
//    LDS. Rows of X' beyond M are zero operands.
//  * prefill (M > 16): a 128x128 output tile per workgroup, k-tiles of 64
//    staged through double-buffered, padded LDS (conflict-free 16-byte
//    reads), weights dequantized once per tile on the way into LDS.
#include "paro_internal.h"

#pragma clang fp contract(off)

namespace paro {
namespace {

typedef _Float16 h8 __attribute__((ext_vector_type(8)));
typedef _Float16 h2 __attribute__((ext_vector_type(2)));
typedef float f4 __attribute__((ext_vector_type(4)));
typedef uint32_t u4 __attribute__((ext_vector_type(4)));

// Eight 4-bit codes (k0 in bits 0..3, ..., k7 in bits 28..31) -> eight fp16
// values (q - z) * s in k order.
__device__ __forceinline__ h8 dequant8(uint32_t w, h2 zz, h2 ss) {
  const uint32_t lo = w & 0x0F0F0F0Fu;         // q0 q2 q4 q6 (one per byte)
  const uint32_t hi = (w >> 4) & 0x0F0F0F0Fu;  // q1 q3 q5 q7
  uint32_t p[4];
  p[0] = __builtin_amdgcn_perm(hi, lo, 0x0C040C00u) | 0x64006400u;
  p[1] = __builtin_amdgcn_perm(hi, lo, 0x0C050C01u) | 0x64006400u;
  p[2] = __builtin_amdgcn_perm(hi, lo, 0x0C060C02u) | 0x64006400u;
  p[3] = __builtin_amdgcn_perm(hi, lo, 0x0C070C03u) | 0x64006400u;
  h8 out;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    h2 v = __builtin_bit_cast(h2, p[i]);
    v = (v - zz) * ss;
    out[2 * i] = v.x;
    out[2 * i + 1] = v.y;
  }
  return out;
}

__device__ __forceinline__ h2 splat2(_Float16 v) { return h2{v, v}; }

// --------------------------------------------------------------------------
// decode: M <= 16
// --------------------------------------------------------------------------
__global__ __launch_bounds__(256) void w4_gemv_kernel(const uint16_t* __restrict__ x,
                                                      const uint8_t* __restrict__ qw,
                                                      const uint16_t* __restrict__ sc,
                                                      const uint8_t* __restrict__ zr,
                                                      const uint16_t* __restrict__ bias,
                                                      uint16_t* __restrict__ y, int M, int N, int d) {
  __shared__ f4 red[4][64];
  const int lane = threadIdx.x & 63;
  const int wid = threadIdx.x >> 6;
  const int n0 = blockIdx.x * 16;
  const int groups = d >> 7;
  const int gpw = (groups + 3) >> 2;
  const int g0 = wid * gpw;
  const int g1 = min(groups, g0 + gpw);
  const int n = n0 + (lane & 15);
  const int kq = lane >> 4;
  const int m = lane & 15;
  const uint8_t* wrow = qw + (size_t)n * (d >> 1) + kq * 16;
  const uint16_t* xrow = x + (size_t)m * d + kq * 32;
  f4 acc = {0.f, 0.f, 0.f, 0.f};
  for (int g = g0; g < g1; ++g) {
    const u4 wv = *(const u4*)(wrow + (size_t)g * 64);
    const _Float16 s = __builtin_bit_cast(_Float16, sc[(size_t)n * groups + g]);
    const _Float16 zf = (_Float16)(1024.0f + (float)zr[(size_t)n * groups + g]);
    const h2 ss = splat2(s), zz = splat2(zf);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const h8 a = dequant8(wv[i], zz, ss);
      h8 b = {};
      if (m < M) b = *(const h8*)(xrow + (size_t)g * 128 + 8 * i);
      acc = __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, acc, 0, 0, 0);
    }
  }
  red[wid][lane] = acc;
  __syncthreads();
  if (wid == 0) {
    f4 t = red[0][lane] + red[1][lane] + red[2][lane] + red[3][lane];
    if (m < M) {
      const int nb = n0 + 4 * kq;
      uint16_t o[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        float v = t[e];
        if (bias) v += (float)__builtin_bit_cast(_Float16, bias[nb + e]);
        o[e] = __builtin_bit_cast(uint16_t, (_Float16)v);
      }
      uint2 pk;
      pk.x = (uint32_t)o[0] | ((uint32_t)o[1] << 16);
      pk.y = (uint32_t)o[2] | ((uint32_t)o[3] << 16);
      *(uint2*)(y + (size_t)m * N + nb) = pk;
    }
  }
}

// --------------------------------------------------------------------------
// prefill: M > 16
// --------------------------------------------------------------------------
constexpr int BN = 128, BM = 128, BK = 64, LDK = BK + 8;  // LDS row: 72 halfs = 144 bytes

__global__ __launch_bounds__(256, 2) void w4_gemm_kernel(const uint16_t* __restrict__ x,
                                                         const uint8_t* __restrict__ qw,
                                                         const uint16_t* __restrict__ sc,
                                                         const uint8_t* __restrict__ zr,
                                                         const uint16_t* __restrict__ bias,
                                                         uint16_t* __restrict__ y, int M, int N,
                                                         int d, int nblk) {
  __shared__ __attribute__((aligned(16))) _Float16 Wl[2][BN * LDK];
  __shared__ __attribute__((aligned(16))) _Float16 Xl[2][BM * LDK];
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wid = tid >> 6;
  const int wn = wid & 1, wm = wid >> 1;
  const int nb = blockIdx.x % nblk;
  const int mb = blockIdx.x / nblk;
  const int n0 = nb * BN, m0 = mb * BM;
  const int groups = d >> 7;
  const int KT = d / BK;

  // global -> register assignments
  const int wl_n = tid >> 1, wl_kh = tid & 1;  // weights: one row, 32 codes
  const bool wl_ok = n0 + wl_n < N;
  const uint8_t* wl_ptr = qw + (size_t)(wl_ok ? n0 + wl_n : 0) * (d >> 1) + wl_kh * 16;
  const int xl_c = tid & 7;                    // activations: 4 rows, 8 halfs each
  const int xl_r = tid >> 3;                   // rows xl_r + 32 j

  u4 wreg;
  u4 xreg[4];
  auto gload = [&](int kt) {
    const int k0 = kt * BK;
    wreg = wl_ok ? *(const u4*)(wl_ptr + (k0 >> 1)) : u4{0u, 0u, 0u, 0u};
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int mrow = m0 + xl_r + 32 * j;
      xreg[j] = mrow < M ? *(const u4*)(x + (size_t)mrow * d + k0 + 8 * xl_c) : u4{0u, 0u, 0u, 0u};
    }
  };
  auto lstore = [&](int kt, int buf) {
    const int g = (kt * BK) >> 7;
    _Float16 s = (_Float16)0.0f, zf = (_Float16)1024.0f;
    if (wl_ok) {
      s = __builtin_bit_cast(_Float16, sc[(size_t)(n0 + wl_n) * groups + g]);
      zf = (_Float16)(1024.0f + (float)zr[(size_t)(n0 + wl_n) * groups + g]);
    }
    const h2 ss = splat2(s), zz = splat2(zf);
    _Float16* wdst = &Wl[buf][wl_n * LDK + wl_kh * 32];
#pragma unroll
    for (int i = 0; i < 4; ++i) *(h8*)(wdst + 8 * i) = dequant8(wreg[i], zz, ss);
#pragma unroll
    for (int j = 0; j < 4; ++j) *(u4*)(&Xl[buf][(xl_r + 32 * j) * LDK + 8 * xl_c]) = xreg[j];
  };

  f4 acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = f4{0.f, 0.f, 0.f, 0.f};

  gload(0);
  lstore(0, 0);
  __syncthreads();
  const int fr = lane & 15, fk = 8 * (lane >> 4);
  for (int kt = 0; kt < KT; ++kt) {
    const int buf = kt & 1;
    if (kt + 1 < KT) gload(kt + 1);
#pragma unroll
    for (int ks = 0; ks < BK / 32; ++ks) {
      h8 a[4], b[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) a[i] = *(const h8*)(&Wl[buf][(wn * 64 + 16 * i + fr) * LDK + ks * 32 + fk]);
#pragma unroll
      for (int j = 0; j < 4; ++j) b[j] = *(const h8*)(&Xl[buf][(wm * 64 + 16 * j + fr) * LDK + ks * 32 + fk]);
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_f16(a[i], b[j], acc[i][j], 0, 0, 0);
    }
    if (kt + 1 < KT) lstore(kt + 1, buf ^ 1);
    __syncthreads();
  }

  // epilogue: lane holds C[n = base + 4*(lane/16) + e][m = base + lane%16]
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int m = m0 + wm * 64 + 16 * j + fr;
    if (m >= M) continue;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int n = n0 + wn * 64 + 16 * i + 4 * (lane >> 4);
      if (n >= N) continue;
      uint16_t o[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        float v = acc[i][j][e];
        if (bias) v += (float)__builtin_bit_cast(_Float16, bias[n + e]);
        o[e] = __builtin_bit_cast(uint16_t, (_Float16)v);
      }
      uint2 pk;
      pk.x = (uint32_t)o[0] | ((uint32_t)o[1] << 16);
      pk.y = (uint32_t)o[2] | ((uint32_t)o[3] << 16);
      *(uint2*)(y + (size_t)m * N + n) = pk;
    }
  }
}

}  // namespace

hipError_t launch_w4_linear(const uint16_t* x, const uint8_t* qweight, const uint16_t* scales,
                            const uint8_t* zeros, const uint16_t* bias, uint16_t* y, int64_t M,
                            int64_t N, int64_t d, hipStream_t stream) {
  if (M == 0) return hipSuccess;
  if (M <= 16) {
    hipLaunchKernelGGL(w4_gemv_kernel, dim3((unsigned)(N / 16)), dim3(256), 0, stream, x, qweight,
                       scales, zeros, bias, y, (int)M, (int)N, (int)d);
    return hipGetLastError();
  }
  const int nblk = (int)((N + BN - 1) / BN);
  const int64_t mblk = (M + BM - 1) / BM;
  hipLaunchKernelGGL(w4_gemm_kernel, dim3((unsigned)(nblk * mblk)), dim3(256), 0, stream, x, qweight,
                     scales, zeros, bias, y, (int)M, (int)N, (int)d, nblk);
  return hipGetLastError();
}

}  // namespace paro
