// gfx950 kernel for the W4G128 linear layer on rotated activations with
// many tokens (prefill, M > 16):
//   Y[m][n] = sum_k X'[m][k] (q[n][k] - z[n][k/128]) s[n][k/128] + b[n]
// (CSDN article section 2.1: Y = (X T^-1)(T W) + b; paper notes "主实验":
// 4-bit weights, group 128). Here the layer is a dense contraction and runs
// on the matrix cores. Dequantization: two nibbles are spread into the
// mantissas of two fp16 1024.0 values with v_perm, (1024 + q) - (1024 + z) =
// q - z is exact in packed fp16, and one packed multiply by the fp16 scale
// rounds once.
#include "paro_internal.h"
#include "w4_common.h"

#pragma clang fp contract(off)

namespace paro {
namespace {

using namespace w4;

// --------------------------------------------------------------------------
// prefill (M > 16): MFMA v_mfma_f32_32x32x16_f16 with the dequantized weights
// as operand A (32 output channels x 16 k) and X' as operand B (16 k x 32
// tokens). A wavefront owns a 64 (n) x 128 (m) tile: 2 x 4 accumulator tiles,
// 128 fp32 per lane, so two wavefronts fit on a SIMD and one's dequantization
// overlaps the other's MFMAs. A group of four wavefronts shares a 128 (m) x
// 256 (n) workgroup tile through double-buffered LDS:
//  * X' tile [128 rows][8 chunks of 8 halfs]; chunk c of row r stored at
//    position c ^ ((r >> 1) & 7);
//  * packed int4 weight tile [256 rows][2 halves of 16 bytes]; half h of row r
//    at position h ^ ((r >> 3) & 1).
// A gfx950 16-byte LDS read is conflict-free when every 16 consecutive lanes
// address positions distinct modulo 16, a 16-byte write when every 8 consecutive
// lanes do modulo 8: the operand reads take 16 consecutive rows at a fixed
// chunk, which these swizzles spread over all 16 positions, and the staging
// writes are lane-contiguous. Global loads are staged through registers one
// k-tile ahead of the LDS buffer being written, so every load has a whole
// multiply phase to land before its data is needed. Each
// wavefront dequantizes its own 64 rows in registers.
// With KS = 2 two groups of four wavefronts split k in halves inside the
// workgroup (for layers with few output tiles) and add their accumulators
// through LDS at the end.
//
// k order inside an MFMA: for a 64-wide k-tile, lane l (row n = l % 32,
// half g = l / 32) takes the codes 32 g .. 32 g + 31 of its row; MFMA step
// i (0..3) uses codes 32 g + 8 i .. + 7, so the four steps together contract
// k = 8 i + {0..7, 32..39}, and X' is read with the same mapping.
// --------------------------------------------------------------------------
typedef float f16v __attribute__((ext_vector_type(16)));

constexpr int GB_M = 128, GB_N = 256, GB_K = 64;
constexpr int GB_XSTAGE = GB_M * GB_K;  // halfs per X' buffer (16 KB)
constexpr int GB_WSTAGE = GB_N * 2;     // 16-byte chunks per weight buffer (8 KB)

template <int KS>
__global__ __launch_bounds__(256 * KS) __attribute__((amdgpu_waves_per_eu(2, 2)))
void w4_gemm_kernel(const uint16_t* __restrict__ x, const uint8_t* __restrict__ qw,
                    const uint16_t* __restrict__ sc, const uint8_t* __restrict__ zr,
                    const uint16_t* __restrict__ bias, uint16_t* __restrict__ y, int M, int N,
                    int d, int mblk, int nblk) {
  __shared__ __attribute__((aligned(1024))) _Float16 Xl[KS][2][GB_XSTAGE];
  __shared__ __attribute__((aligned(1024))) u4 Wl[KS][2][GB_WSTAGE];
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int kg = tid >> 8;          // k half (KS = 2)
  const int w = (tid >> 6) & 3;     // wavefront inside the group
  // XCD-aware tile order: workgroup b runs on XCD b % 8. XCD x owns the
  // n-blocks [x nbp, (x + 1) nbp) and walks them in super-blocks of 8 m-blocks
  // x all its n-blocks, so the ~64 workgroups resident on one XCD share both
  // their X' and their weight k-tiles through its L2.
  const int nbp = (nblk + 7) >> 3;
  const int xcd = blockIdx.x & 7, idx = blockIdx.x >> 3;
  const int nbx = min(nbp, nblk - xcd * nbp);
  if (nbx <= 0) return;
  const int mg = idx / (8 * nbx), rem = idx - mg * 8 * nbx;
  const int nb = xcd * nbp + rem / 8;
  const int mb = mg * 8 + (rem & 7);
  if (mb >= mblk) return;
  const int m0 = mb * GB_M;
  const int nw0 = nb * GB_N;       // workgroup's first output channel
  const int n0 = nw0 + 64 * w;     // this wavefront's first output channel
  const int groups = d >> 7;
  const int KT = (d / GB_K) / KS;  // k-tiles per group of wavefronts
  const int kt0 = kg * KT;
  const int l32 = lane & 31, g = lane >> 5;

  // scales / zeros of the lane's rows n0 + 32 j + l32 (rows past N: zero scale)
  uint32_t soff[2];
  bool wok[2];
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const int n = n0 + 32 * j + l32;
    wok[j] = n < N;
    soff[j] = (uint32_t)(wok[j] ? n : N - 1) * (uint32_t)groups;
  }
  // X' staging: chunk c of wavefront w covers tile rows 8 (4 w + c) .. + 7; the
  // lane at position l % 8 of row l / 8 carries the source chunk (l % 8) ^ swizzle
  uint32_t xoff[4];
#pragma unroll
  for (int c = 0; c < 4; ++c) {
    const int r = 8 * (4 * w + c) + (lane >> 3);
    const int row = min(m0 + r, M - 1);  // rows past M are never stored
    xoff[c] = (uint32_t)row * (uint32_t)d + 8u * ((lane & 7) ^ ((r >> 1) & 7));
  }
  // weight staging: chunk c of wavefront w covers tile rows 32 (2 w + c) .. + 31
  uint32_t woff[2];
#pragma unroll
  for (int c = 0; c < 2; ++c) {
    const int r = 32 * (2 * w + c) + (lane >> 1);
    const int row = min(nw0 + r, N - 1);
    woff[c] = (uint32_t)row * (uint32_t)(d >> 1) + 16u * ((lane & 1) ^ ((r >> 3) & 1));
  }

  u4 xr[4], wr[2];
  uint32_t sraw[2], zraw[2];
  h2 ss[2], zz[2], ss_n[2], zz_n[2];
  auto load_regs = [&](int kt) {  // k-tile kt of this group's range: X', codes, scales
    const int kglob = kt0 + kt;
#pragma unroll
    for (int c = 0; c < 4; ++c) xr[c] = *(const u4*)(x + xoff[c] + kglob * GB_K);
#pragma unroll
    for (int c = 0; c < 2; ++c) wr[c] = *(const u4*)(qw + woff[c] + kglob * (GB_K / 2));
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      sraw[j] = sc[soff[j] + (kglob >> 1)];
      zraw[j] = zr[soff[j] + (kglob >> 1)];
    }
  };
  auto store_regs = [&](int buf) {
#pragma unroll
    for (int c = 0; c < 4; ++c) *(u4*)&Xl[kg][buf][((4 * w + c) * 64 + lane) * 8] = xr[c];
#pragma unroll
    for (int c = 0; c < 2; ++c) Wl[kg][buf][(2 * w + c) * 64 + lane] = wr[c];
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const _Float16 s = wok[j] ? __builtin_bit_cast(_Float16, (uint16_t)sraw[j]) : (_Float16)0.0f;
      ss_n[j] = splat2(s);
      zz_n[j] = splat2((_Float16)(1024.0f + (float)zraw[j]));
    }
  };

  f16v acc[2][4];
#pragma unroll
  for (int j = 0; j < 2; ++j)
#pragma unroll
    for (int mm = 0; mm < 4; ++mm)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[j][mm][e] = 0.0f;

  // Iteration kt: write the staged k-tile kt + 1 to the buffer last read in
  // iteration kt - 1 (its loads were issued a whole iteration ago), issue the
  // loads of k-tile kt + 2, multiply k-tile kt, then one barrier. The loop is
  // branch-free: past the last tile it writes a buffer nobody reads again and
  // reloads the last tile.
  load_regs(0);
  store_regs(0);
  load_regs(min(1, KT - 1));
  __syncthreads();
  for (int kt = 0; kt < KT; ++kt) {
    const int buf = kt & 1;
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      ss[j] = ss_n[j];
      zz[j] = zz_n[j];
    }
    store_regs(buf ^ 1);
    load_regs(min(kt + 2, KT - 1));
    const _Float16* xb = &Xl[kg][buf][0];
    u4 wf[2];
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int r = 64 * w + 32 * j + l32;
      wf[j] = Wl[kg][buf][2 * r + (g ^ ((r >> 3) & 1))];
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      h8 a[2], b[4];
#pragma unroll
      for (int j = 0; j < 2; ++j) a[j] = dequant8(wf[j][i], zz[j], ss[j]);
#pragma unroll
      for (int mm = 0; mm < 4; ++mm) {
        const int r = 32 * mm + l32;
        b[mm] = *(const h8*)(xb + r * GB_K + 8 * ((4 * g + i) ^ ((r >> 1) & 7)));
      }
#pragma unroll
      for (int j = 0; j < 2; ++j)
#pragma unroll
        for (int mm = 0; mm < 4; ++mm)
          acc[j][mm] = __builtin_amdgcn_mfma_f32_32x32x16_f16(a[j], b[mm], acc[j][mm], 0, 0, 0);
    }
    __syncthreads();
  }

  if constexpr (KS == 2) {
    // the second k half hands its partial sums to the first through LDS, one
    // 64 KB half of the accumulators at a time
    float* red = (float*)&Xl[0][0][0];
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      if (kg == 1) {
#pragma unroll
        for (int mm = 0; mm < 4; ++mm)
#pragma unroll
          for (int e = 0; e < 16; ++e) red[((w * 4 + mm) * 16 + e) * 64 + lane] = acc[j][mm][e];
      }
      __syncthreads();
      if (kg == 0) {
#pragma unroll
        for (int mm = 0; mm < 4; ++mm)
#pragma unroll
          for (int e = 0; e < 16; ++e) acc[j][mm][e] += red[((w * 4 + mm) * 16 + e) * 64 + lane];
      }
      __syncthreads();
    }
    if (kg == 1) return;
  }

  // epilogue: acc[j][mm][e] = C[n = n0 + 32 j + 8 (e/4) + 4 g + e%4][m = m0 + 32 mm + l32]
#pragma unroll
  for (int j = 0; j < 2; ++j) {
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int n = n0 + 32 * j + 8 * q + 4 * g;
      if (n >= N) continue;
      float bv[4] = {0.f, 0.f, 0.f, 0.f};
      if (bias) {
        const uint2 braw = *(const uint2*)(bias + n);
        bv[0] = half_lo(braw.x);
        bv[1] = half_hi(braw.x);
        bv[2] = half_lo(braw.y);
        bv[3] = half_hi(braw.y);
      }
#pragma unroll
      for (int mm = 0; mm < 4; ++mm) {
        const int m = m0 + 32 * mm + l32;
        if (m >= M) continue;
        uint2 pk;
        pk.x = half_bits(acc[j][mm][4 * q + 0] + bv[0]) | (half_bits(acc[j][mm][4 * q + 1] + bv[1]) << 16);
        pk.y = half_bits(acc[j][mm][4 * q + 2] + bv[2]) | (half_bits(acc[j][mm][4 * q + 3] + bv[3]) << 16);
        *(uint2*)(y + (size_t)m * N + n) = pk;
      }
    }
  }
}

}  // namespace

hipError_t launch_w4_gemm(const uint16_t* x, const uint8_t* qweight, const uint16_t* scales,
                          const uint8_t* zeros, const uint16_t* bias, uint16_t* y, int64_t M,
                          int64_t N, int64_t d, hipStream_t stream) {
  if (M == 0) return hipSuccess;
  const int nblk = (int)((N + GB_N - 1) / GB_N);
  const int mblk = (int)((M + GB_M - 1) / GB_M);
  const int64_t tiles = (int64_t)nblk * mblk;
  // 8 XCDs, each with its n-block range walked in super-blocks of 8 m-blocks
  const int64_t nbp = (nblk + 7) / 8;
  const int64_t blocks = 8 * nbp * (((int64_t)mblk + 7) / 8) * 8;
  // too few tiles to give every SIMD two wavefronts: split k inside the workgroup
  if (tiles < 512 && (d / GB_K) % 2 == 0 && d / GB_K >= 4) {
    hipLaunchKernelGGL(w4_gemm_kernel<2>, dim3((unsigned)blocks), dim3(512), 0, stream, x, qweight,
                       scales, zeros, bias, y, (int)M, (int)N, (int)d, mblk, nblk);
  } else {
    hipLaunchKernelGGL(w4_gemm_kernel<1>, dim3((unsigned)blocks), dim3(256), 0, stream, x, qweight,
                       scales, zeros, bias, y, (int)M, (int)N, (int)d, mblk, nblk);
  }
  return hipGetLastError();
}

}  // namespace paro
