// gfx950 dense fp16 products of the layer-wise loss (paper notes, "损失函数 /
// 训练策略": the layer's output error ||Q(D)(X') - D(X)|| and, for learning the
// angles and scales, its gradient):
//   * Y = X W^T of the layer in its original fp16 weights, with the loss
//     folded into the epilogue: each workgroup reads Y_q at its outputs, adds
//     (Y_q - Y)^2 over its tile in a fixed order into one partial sum, and
//     writes dY = 2 (Y_q - Y) in fp16 (Y itself never goes to memory);
//   * dX' = dY E (E = W_hat - T W, the quantization error) with fp32 output,
//     on E transposed by a tiled LDS transpose.
// Both are "NT" products C[m][n] = sum_k A[m][k] B[n][k] of row-major fp16
// operands whose k is contiguous, fp32 accumulation on the matrix cores
// (v_mfma_f32_32x32x16_f16).
//
// Tiling: a workgroup of four wavefronts owns a 128 (m) x 128 (n) tile, each
// wavefront 64 x 64 (2 x 2 accumulator tiles). k-tiles of 64 of both operands
// go from global memory straight into LDS by load-to-LDS DMA (16 bytes per
// lane), into two stages: the DMA of k-tile kt + 1 runs while kt is
// multiplied. In a stage, row r holds its 8 chunks of 16 bytes with chunk c at
// position c ^ ((r >> 1) & 7), so the operand reads (16 consecutive rows at one
// chunk) hit 16 distinct 16-byte positions modulo 16, which a gfx950 16-byte
// LDS read serves without bank conflicts; DMA writes land lane-contiguously,
// so the swizzle is applied by choosing which source chunk each lane fetches.
// Operand A (rows m) is the MFMA's first operand and B (rows n) its second, so
// each accumulator register holds 32 consecutive n of one m across a
// half-wavefront: stores of C are 128-byte (fp32) or 64-byte (fp16) runs.
// Workgroup b runs on XCD b % 8; XCD x owns the n-blocks x, x + 8, ... and
// walks them in super-blocks of 8 m-blocks, so the workgroups resident on one
// XCD share A and B k-tiles in its L2.
#include "paro_internal.h"

#pragma clang fp contract(off)

namespace paro {
namespace {

typedef _Float16 h8 __attribute__((ext_vector_type(8)));
typedef float f16v __attribute__((ext_vector_type(16)));
typedef __attribute__((address_space(3))) void lds_void;

constexpr int DG_M = 128, DG_N = 128, DG_K = 64;
constexpr int kRsrcWord3 = 0x00020000;  // gfx9 buffer resource word 3
constexpr int kWaitVmLgkm0 = 0x70;      // s_waitcnt vmcnt(0) lgkmcnt(0)

enum { EPI_STORE_F32 = 0, EPI_LOSS = 1 };

__device__ __forceinline__ uint16_t f16_bits(float f) {
  return __builtin_bit_cast(uint16_t, (_Float16)f);
}

// EPI_STORE_F32: c[m * ldc + n] = acc (fp32).
// EPI_LOSS: part[tile] = sum over the tile of (yq[m][n] - acc)^2 (fixed
// order), and with dy != NULL dy[m * ldd + n] = fp16(2 (yq - acc)) for n < N,
// 0 for N <= n < ldd.
template <int EPI>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2)))
void nt_gemm_kernel(const uint16_t* __restrict__ a, int lda, const uint16_t* __restrict__ b,
                    int ldb, int M, int N, int K, int mblk, int nblk, float* __restrict__ c, int ldc,
                    const uint16_t* __restrict__ yq, uint16_t* __restrict__ dy, int ldd,
                    float* __restrict__ part) {
  __shared__ __attribute__((aligned(1024))) _Float16 A0[DG_M * DG_K], A1[DG_M * DG_K];
  __shared__ __attribute__((aligned(1024))) _Float16 B0[DG_N * DG_K], B1[DG_N * DG_K];
  __shared__ float red[256];
  const int tid = threadIdx.x, lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = w & 1, wn = w >> 1;
  const int xcd = blockIdx.x & 7, idx = blockIdx.x >> 3;
  const int nbx = (nblk - xcd + 7) >> 3;
  if (nbx <= 0) return;
  const int mg = idx / (8 * nbx), rem = idx - mg * 8 * nbx;
  const int nb = xcd + 8 * (rem / 8);
  const int mb = mg * 8 + (rem & 7);
  if (mb >= mblk) return;
  const int m0 = mb * DG_M, n0 = nb * DG_N;
  const int KT = K / DG_K;
  const int l32 = lane & 31, g = lane >> 5;

  // buffer resources based at the tile's first rows; rows past M or N are
  // clamped to the last row (their results are never stored)
  const __amdgpu_buffer_rsrc_t ra = __builtin_amdgcn_make_buffer_rsrc(
      (void*)(a + (size_t)m0 * lda), (short)0, min(M - m0, DG_M) * lda * 2, kRsrcWord3);
  const __amdgpu_buffer_rsrc_t rb = __builtin_amdgcn_make_buffer_rsrc(
      (void*)(b + (size_t)n0 * ldb), (short)0, min(N - n0, DG_N) * ldb * 2, kRsrcWord3);
  // DMA c of wavefront w fills tile rows 8 (4 w + c) .. + 7: the lane at
  // position l % 8 of row l / 8 fetches the source chunk (l % 8) ^ swizzle
  uint32_t aoff[4], boff[4];
#pragma unroll
  for (int cc = 0; cc < 4; ++cc) {
    const int r = 8 * (4 * w + cc) + (lane >> 3);
    const int ch = (lane & 7) ^ ((r >> 1) & 7);
    aoff[cc] = (uint32_t)(min(r, M - 1 - m0) * lda + 8 * ch) * 2u;
    boff[cc] = (uint32_t)(min(r, N - 1 - n0) * ldb + 8 * ch) * 2u;
  }
  auto dma = [&](int kt, _Float16* as, _Float16* bs) {
#pragma unroll
    for (int cc = 0; cc < 4; ++cc)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(ra, (lds_void*)&as[(4 * w + cc) * 64 * 8], 16, aoff[cc],
                                               kt * DG_K * 2, 0, 0);
#pragma unroll
    for (int cc = 0; cc < 4; ++cc)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rb, (lds_void*)&bs[(4 * w + cc) * 64 * 8], 16, boff[cc],
                                               kt * DG_K * 2, 0, 0);
  };

  f16v acc[2][2];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.0f;

  // MFMA step i contracts, for lane half g, chunk 4 g + i of each row (k =
  // 8 (4 g + i) .. + 7), the same mapping on both operands
  auto step = [&](int kt, const _Float16* as, const _Float16* bs, _Float16* an, _Float16* bn) {
    dma(min(kt + 1, KT - 1), an, bn);
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      h8 av[2], bv[2];
#pragma unroll
      for (int t = 0; t < 2; ++t) {
        const int ra_ = 64 * wm + 32 * t + l32;
        const int rb_ = 64 * wn + 32 * t + l32;
        av[t] = *(const h8*)(as + ra_ * DG_K + 8 * ((4 * g + i) ^ ((ra_ >> 1) & 7)));
        bv[t] = *(const h8*)(bs + rb_ * DG_K + 8 * ((4 * g + i) ^ ((rb_ >> 1) & 7)));
      }
#pragma unroll
      for (int mm = 0; mm < 2; ++mm)
#pragma unroll
        for (int nn = 0; nn < 2; ++nn)
          acc[mm][nn] = __builtin_amdgcn_mfma_f32_32x32x16_f16(av[mm], bv[nn], acc[mm][nn], 0, 0, 0);
    }
    __builtin_amdgcn_sched_barrier(0);
    __builtin_amdgcn_s_waitcnt(kWaitVmLgkm0);
    __builtin_amdgcn_s_barrier();
  };

  dma(0, A0, B0);
  __builtin_amdgcn_s_waitcnt(kWaitVmLgkm0);
  __builtin_amdgcn_s_barrier();
  for (int kt = 0; kt < KT; kt += 2) {
    step(kt, A0, B0, A1, B1);
    if (kt + 1 < KT) step(kt + 1, A1, B1, A0, B0);
  }

  // acc[mm][nn][e] = C[m = m0 + 64 wm + 32 mm + 8 (e / 4) + 4 g + e % 4][n = n0 + 64 wn + 32 nn + l32]
  if constexpr (EPI == EPI_STORE_F32) {
#pragma unroll
    for (int mm = 0; mm < 2; ++mm)
#pragma unroll
      for (int nn = 0; nn < 2; ++nn) {
        const int n = n0 + 64 * wn + 32 * nn + l32;
#pragma unroll
        for (int e = 0; e < 16; ++e) {
          const int m = m0 + 64 * wm + 32 * mm + 8 * (e >> 2) + 4 * g + (e & 3);
          if (m < M && n < N) c[(size_t)m * ldc + n] = acc[mm][nn][e];
        }
      }
  } else {
    float s = 0.0f;
#pragma unroll
    for (int mm = 0; mm < 2; ++mm)
#pragma unroll
      for (int nn = 0; nn < 2; ++nn) {
        const int n = n0 + 64 * wn + 32 * nn + l32;
#pragma unroll
        for (int e = 0; e < 16; ++e) {
          const int m = m0 + 64 * wm + 32 * mm + 8 * (e >> 2) + 4 * g + (e & 3);
          if (m < M) {
            if (n < N) {
              const float v = (float)__builtin_bit_cast(_Float16, yq[(size_t)m * N + n]) - acc[mm][nn][e];
              s += v * v;
              if (dy) dy[(size_t)m * ldd + n] = f16_bits(2.0f * v);
            } else if (dy && n < ldd) {
              dy[(size_t)m * ldd + n] = 0;
            }
          }
        }
      }
    // the tile's sum in a fixed order: per lane above, then a fixed tree
    red[tid] = s;
    __syncthreads();
    for (int h = 128; h > 0; h >>= 1) {
      if (tid < h) red[tid] += red[tid + h];
      __syncthreads();
    }
    if (tid == 0) part[mb * nblk + nb] = red[0];
  }
}

// out[cidx][ridx] = in[ridx][cidx] for a [R][C] fp16 matrix, out row stride
// ldo >= R with zeros in columns R .. ldo - 1. 64 x 64 tiles through LDS (one
// padding half per row against bank conflicts); reads and writes of 4 bytes
// per lane, 128 bytes per row segment.
__global__ __launch_bounds__(256) void transpose_pad_kernel(const uint16_t* __restrict__ in, int R,
                                                            int C, uint16_t* __restrict__ out, int ldo) {
  __shared__ uint16_t t[64][66];
  const int tr = blockIdx.y * 64, tc = blockIdx.x * 64;  // tile of in: rows tr.., cols tc..
  const int tid = threadIdx.x;
  const int cx = 2 * (tid & 31), ry = tid >> 5;  // two columns per lane, 8 rows per pass
#pragma unroll
  for (int p = 0; p < 8; ++p) {
    const int r = ry + 8 * p;
    const int gr = tr + r, gc = tc + cx;
    uint32_t v = 0;
    if (gr < R && gc < C) v = *(const uint32_t*)(in + (size_t)gr * C + gc);  // C even
    t[r][cx] = (uint16_t)v;
    t[r][cx + 1] = (uint16_t)(v >> 16);
  }
  __syncthreads();
#pragma unroll
  for (int p = 0; p < 8; ++p) {
    const int oc = ry + 8 * p;          // row of out (a column of in)
    const int orow = tc + oc, ocol = tr + cx;
    if (orow < C && ocol < ldo) {
      const uint32_t v = (uint32_t)t[cx][oc] | ((uint32_t)t[cx + 1][oc] << 16);  // zero past R
      *(uint32_t*)(out + (size_t)orow * ldo + ocol) = v;
    }
  }
}

template <int EPI>
hipError_t launch_nt(const uint16_t* a, int lda, const uint16_t* b, int ldb, int M, int N, int K,
                     float* c, int ldc, const uint16_t* yq, uint16_t* dy, int ldd, float* part,
                     hipStream_t stream) {
  const int mblk = (M + DG_M - 1) / DG_M, nblk = (N + DG_N - 1) / DG_N;
  const int64_t nbp = (nblk + 7) / 8;
  const int64_t blocks = 8 * nbp * (((int64_t)mblk + 7) / 8) * 8;
  hipLaunchKernelGGL((nt_gemm_kernel<EPI>), dim3((unsigned)blocks), dim3(256), 0, stream, a, lda, b,
                     ldb, M, N, K, mblk, nblk, c, ldc, yq, dy, ldd, part);
  return hipGetLastError();
}

}  // namespace

int nt_tiles(int64_t M, int64_t N) {
  return (int)(((M + DG_M - 1) / DG_M) * ((N + DG_N - 1) / DG_N));
}

hipError_t launch_nt_gemm_f32(const uint16_t* a, int64_t lda, const uint16_t* b, int64_t ldb,
                              int64_t M, int64_t N, int64_t K, float* c, int64_t ldc,
                              hipStream_t stream) {
  if (M == 0 || N == 0) return hipSuccess;
  return launch_nt<EPI_STORE_F32>(a, (int)lda, b, (int)ldb, (int)M, (int)N, (int)K, c, (int)ldc,
                                  nullptr, nullptr, 0, nullptr, stream);
}

hipError_t launch_nt_gemm_loss(const uint16_t* x, const uint16_t* w, int64_t M, int64_t N, int64_t d,
                               const uint16_t* yq, uint16_t* dy, int64_t ldd, float* part,
                               hipStream_t stream) {
  if (M == 0 || N == 0) return hipSuccess;
  return launch_nt<EPI_LOSS>(x, (int)d, w, (int)d, (int)M, (int)N, (int)d, nullptr, 0, yq, dy,
                             (int)ldd, part, stream);
}

hipError_t launch_transpose_pad(const uint16_t* in, int64_t R, int64_t C, uint16_t* out, int64_t ldo,
                                hipStream_t stream) {
  if (R == 0 || C == 0) return hipSuccess;
  const dim3 grid((unsigned)((C + 63) / 64), (unsigned)((ldo + 63) / 64));
  hipLaunchKernelGGL(transpose_pad_kernel, grid, dim3(256), 0, stream, in, (int)R, (int)C, out, (int)ldo);
  return hipGetLastError();
}

}  // namespace paro
