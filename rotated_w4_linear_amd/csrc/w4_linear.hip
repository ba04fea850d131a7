// gfx950 kernel for the W4G128 linear layer on rotated activations with
// many tokens (prefill, M > 16):
//   Y[m][n] = sum_k X'[m][k] (q[n][k] - z[n][k/G]) s[n][k/G] + b[n]
// (CSDN article section 2.1: Y = (X T^-1)(T W) + b; paper notes "主实验":
// 4-bit weights, group G = 128; 64 and 256 are taken as well, each 64-channel
// k-tile reading the one group it lies in). Here the layer is a dense contraction and runs
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
// 256 (n) workgroup tile.
//
// Staging: every operand of a k-tile of 64 (X' tile, packed codes, the
// tile's group scale and zero of each row) goes from global memory straight
// into LDS with load-to-LDS DMA (16 bytes per lane for X' and codes), into
// two stages: the DMA of k-tile kt + 1 runs while k-tile kt is multiplied,
// and nothing is staged through registers. Each stage is its own LDS object,
// so the compiler sees that the stage being filled never aliases the one
// being read; the kernel waits for the DMA counter itself (s_waitcnt) before
// the one barrier per k-tile.
//  * X' tile [128 rows][8 chunks of 8 halfs]; chunk c of row r stored at
//    position c ^ ((r >> 1) & 7);
//  * packed int4 weight tile [256 rows][2 halves of 16 bytes]; half h of row r
//    at position h ^ ((r >> 3) & 1).
// A gfx950 16-byte LDS read is conflict-free when every 16 consecutive lanes
// address positions distinct modulo 16: the operand reads take 16 consecutive
// rows at a fixed chunk, which these swizzles spread over all 16 positions.
// DMA writes land lane-contiguously, so the swizzle is applied by choosing
// which source chunk each lane fetches. Each wavefront dequantizes its own 64
// rows in registers.
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
typedef __attribute__((address_space(3))) void lds_void;

constexpr int GB_N = 256, GB_K = 64;
constexpr int GB_WSTAGE = GB_N * 2;     // 16-byte chunks per weight stage (8 KB)
constexpr int kRsrcWord3 = 0x00020000;  // gfx9 buffer resource word 3
// s_waitcnt immediate (gfx9 encoding): vmcnt(0) lgkmcnt(0), expcnt untouched
constexpr int kWaitVmLgkm0 = 0x70;
// Output tiles (at 128 tokens) below which 64-token tiles are used: measured
// on MI355X, 64-token tiles win at 128 tiles (1024 x 4096 -> 4096: 699
// against 581 TFLOP/s) and lose at 256 (2048 x 4096 -> 4096: 760 against 918).
constexpr int64_t kHalfTileBelow = 256;

// MT: 32-token m tiles per wavefront (4: 128-token workgroup tiles; 2: 64,
// for layers with few output tiles).
template <int KS, int MT>
__global__ __launch_bounds__(256 * KS) __attribute__((amdgpu_waves_per_eu(2)))
void w4_gemm_kernel(const uint16_t* __restrict__ x, const uint8_t* __restrict__ qw,
                    const uint16_t* __restrict__ sc, const uint8_t* __restrict__ zr,
                    const uint16_t* __restrict__ bias, uint16_t* __restrict__ y, int M, int N,
                    int d, int gsh, int mblk, int nblk) {
  constexpr int GB_M = 32 * MT;           // tokens per workgroup tile
  constexpr int GB_XSTAGE = GB_M * GB_K;  // halfs per X' stage (16 KB at MT = 4)
  __shared__ __attribute__((aligned(1024))) _Float16 X0[KS][GB_XSTAGE], X1[KS][GB_XSTAGE];
  __shared__ __attribute__((aligned(1024))) u4 W0[KS][GB_WSTAGE], W1[KS][GB_WSTAGE];
  __shared__ __attribute__((aligned(16))) uint32_t S0[KS][GB_N], S1[KS][GB_N];
  __shared__ __attribute__((aligned(16))) uint32_t Z0[KS][GB_N], Z1[KS][GB_N];
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int kg = __builtin_amdgcn_readfirstlane(tid >> 8);     // k half (KS = 2)
  const int w = __builtin_amdgcn_readfirstlane((tid >> 6) & 3);  // wavefront inside the group
  // XCD-aware tile order: workgroup b runs on XCD b % 8. XCD x owns the
  // n-blocks x, x + 8, ... and walks them in super-blocks of 8 m-blocks x all
  // its n-blocks, so the workgroups resident on one XCD share both their X'
  // and their weight k-tiles through its L2.
  const int xcd = blockIdx.x & 7, idx = blockIdx.x >> 3;
  const int nbx = (nblk - xcd + 7) >> 3;
  if (nbx <= 0) return;
  const int mg = idx / (8 * nbx), rem = idx - mg * 8 * nbx;
  const int nb = xcd + 8 * (rem / 8);
  const int mb = mg * 8 + (rem & 7);
  if (mb >= mblk) return;
  const int m0 = mb * GB_M;
  const int nw0 = nb * GB_N;       // workgroup's first output channel
  const int n0 = nw0 + 64 * w;     // this wavefront's first output channel
  const int groups = d >> (6 + gsh);  // quantization groups of 64 << gsh channels per row
  const int KT = (d / GB_K) / KS;  // k-tiles per group of wavefronts
  const int kt0 = kg * KT;
  const int l32 = lane & 31, g = lane >> 5;

  // Buffer resources based at this tile's first row (byte offsets < 2^31,
  // checked on the host); rows past M or N are clamped to the last row.
  const __amdgpu_buffer_rsrc_t rx = __builtin_amdgcn_make_buffer_rsrc(
      (void*)(x + (size_t)m0 * d), (short)0, min(M - m0, GB_M) * d * 2, kRsrcWord3);
  const __amdgpu_buffer_rsrc_t rw = __builtin_amdgcn_make_buffer_rsrc(
      (void*)(qw + (size_t)nw0 * (d >> 1)), (short)0, min(N - nw0, GB_N) * (d >> 1), kRsrcWord3);
  const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(
      (void*)(sc + (size_t)nw0 * groups), (short)0, min(N - nw0, GB_N) * groups * 2, kRsrcWord3);
  const __amdgpu_buffer_rsrc_t rz = __builtin_amdgcn_make_buffer_rsrc(
      (void*)(zr + (size_t)nw0 * groups), (short)0, min(N - nw0, GB_N) * groups, kRsrcWord3);
  // X' DMA c of wavefront w fills tile rows 8 (MT w + c) .. + 7; the lane at
  // position l % 8 of row l / 8 fetches the source chunk (l % 8) ^ swizzle
  // (arrays the lambdas below capture are sized for MT = 4: the host pass of
  // hipcc cannot instantiate lambdas capturing arrays of template-dependent
  // size)
  uint32_t xoff[4];
#pragma unroll
  for (int c = 0; c < MT; ++c) {
    const int r = 8 * (MT * w + c) + (lane >> 3);
    const int row = min(r, M - 1 - m0);
    xoff[c] = (uint32_t)(row * d + 8 * ((lane & 7) ^ ((r >> 1) & 7))) * 2u;
  }
  // code DMA c of wavefront w fills tile rows 32 (2 w + c) .. + 31
  uint32_t woff[2];
#pragma unroll
  for (int c = 0; c < 2; ++c) {
    const int r = 32 * (2 * w + c) + (lane >> 1);
    const int row = min(r, N - 1 - nw0);
    woff[c] = (uint32_t)(row * (d >> 1) + 16 * ((lane & 1) ^ ((r >> 3) & 1)));
  }
  // group scale and zero: lane l of wavefront w fetches row 64 w + l
  const uint32_t szrow = (uint32_t)(min(64 * w + lane, N - 1 - nw0) * groups);

  // the DMA of one k-tile: ten load-to-LDS instructions per lane
  auto dma = [&](int kt, _Float16* xs, u4* ws, uint32_t* ss_l, uint32_t* zs_l) {
    const int kglob = kt0 + kt;
    const uint32_t gi = (uint32_t)(kglob >> gsh);  // the k-tile's group (64-channel k-tiles)
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (lds_void*)&ss_l[64 * w], 2, (szrow + gi) * 2u, 0, 0, 0);
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rz, (lds_void*)&zs_l[64 * w], 1, szrow + gi, 0, 0, 0);
#pragma unroll
    for (int c = 0; c < MT; ++c)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rx, (lds_void*)&xs[(MT * w + c) * 64 * 8], 16, xoff[c],
                                               kglob * GB_K * 2, 0, 0);
#pragma unroll
    for (int c = 0; c < 2; ++c)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rw, (lds_void*)&ws[(2 * w + c) * 64], 16, woff[c],
                                               kglob * (GB_K / 2), 0, 0);
  };

  f16v acc[2][4];  // m tiles mm < MT used
#pragma unroll
  for (int j = 0; j < 2; ++j)
#pragma unroll
    for (int mm = 0; mm < MT; ++mm)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[j][mm][e] = 0.0f;

  // One k-tile from stage (xs, ws, ss_l, zs_l) while the DMA of the next
  // k-tile fills the other stage, then wait for that DMA and one barrier.
  // Past the last tile the DMA reloads the last tile into a stage nobody reads.
  auto step = [&](int kt, const _Float16* xb, const u4* wl, const uint32_t* ss_l,
                  const uint32_t* zs_l, _Float16* xn, u4* wn, uint32_t* sn, uint32_t* zn) {
    dma(min(kt + 1, KT - 1), xn, wn, sn, zn);
    __builtin_amdgcn_sched_barrier(0);
    u4 wf[2];
    h2 ss[2], zz[2];
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int r = 64 * w + 32 * j + l32;
      wf[j] = wl[2 * r + (g ^ ((r >> 3) & 1))];
      const bool ok = nw0 + r < N;
      ss[j] = splat2(ok ? __builtin_bit_cast(_Float16, (uint16_t)(ss_l[r] & 0xffffu)) : (_Float16)0.0f);
      zz[j] = splat2((_Float16)(1024.0f + (float)(zs_l[r] & 0xffu)));
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      h8 a[2], b[MT];
#pragma unroll
      for (int j = 0; j < 2; ++j) a[j] = dequant8(wf[j][i], zz[j], ss[j]);
#pragma unroll
      for (int mm = 0; mm < MT; ++mm) {
        const int r = 32 * mm + l32;
        b[mm] = *(const h8*)(xb + r * GB_K + 8 * ((4 * g + i) ^ ((r >> 1) & 7)));
      }
#pragma unroll
      for (int j = 0; j < 2; ++j)
#pragma unroll
        for (int mm = 0; mm < MT; ++mm)
          acc[j][mm] = __builtin_amdgcn_mfma_f32_32x32x16_f16(a[j], b[mm], acc[j][mm], 0, 0, 0);
    }
    __builtin_amdgcn_sched_barrier(0);
    __builtin_amdgcn_s_waitcnt(kWaitVmLgkm0);
    __builtin_amdgcn_s_barrier();
  };

  dma(0, &X0[kg][0], &W0[kg][0], &S0[kg][0], &Z0[kg][0]);
  __builtin_amdgcn_s_waitcnt(kWaitVmLgkm0);
  __builtin_amdgcn_s_barrier();
  for (int kt = 0; kt < KT; kt += 2) {
    step(kt, &X0[kg][0], &W0[kg][0], &S0[kg][0], &Z0[kg][0], &X1[kg][0], &W1[kg][0], &S1[kg][0], &Z1[kg][0]);
    if (kt + 1 < KT) step(kt + 1, &X1[kg][0], &W1[kg][0], &S1[kg][0], &Z1[kg][0], &X0[kg][0], &W0[kg][0], &S0[kg][0], &Z0[kg][0]);
  }

  if constexpr (KS == 2) {
    // the second k half hands its partial sums to the first through LDS (the
    // X' stages 0 of both halves: 32 KB at MT = 4, 16 KB at MT = 2), PM m
    // tiles of one n tile (16 KB per m tile) at a time
    constexpr int PM = MT / 2;
    float* red = (float*)&X0[0][0];
#pragma unroll
    for (int j = 0; j < 2; ++j) {
#pragma unroll
      for (int h = 0; h < MT / PM; ++h) {
        if (kg == 1) {
#pragma unroll
          for (int mm = 0; mm < PM; ++mm)
#pragma unroll
            for (int e = 0; e < 16; ++e) red[((w * PM + mm) * 16 + e) * 64 + lane] = acc[j][PM * h + mm][e];
        }
        __syncthreads();
        if (kg == 0) {
#pragma unroll
          for (int mm = 0; mm < PM; ++mm)
#pragma unroll
            for (int e = 0; e < 16; ++e) acc[j][PM * h + mm][e] += red[((w * PM + mm) * 16 + e) * 64 + lane];
        }
        __syncthreads();
      }
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
      for (int mm = 0; mm < MT; ++mm) {
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

template <int KS, int MT>
void launch_gemm(unsigned blocks, hipStream_t stream, const uint16_t* x, const uint8_t* qweight,
                 const uint16_t* scales, const uint8_t* zeros, const uint16_t* bias, uint16_t* y,
                 int64_t M, int64_t N, int64_t d, int gsh, int mblk, int nblk) {
  hipLaunchKernelGGL((w4_gemm_kernel<KS, MT>), dim3(blocks), dim3(256 * KS), 0, stream, x, qweight,
                     scales, zeros, bias, y, (int)M, (int)N, (int)d, gsh, mblk, nblk);
}

}  // namespace

hipError_t launch_w4_gemm(const uint16_t* x, const uint8_t* qweight, const uint16_t* scales,
                          const uint8_t* zeros, const uint16_t* bias, uint16_t* y, int64_t M,
                          int64_t N, int64_t d, int group, hipStream_t stream) {
  if (M == 0) return hipSuccess;
  const int gsh = group == 64 ? 0 : group == 128 ? 1 : 2;
  const int nblk = (int)((N + GB_N - 1) / GB_N);
  // 64-token tiles when 128-token ones would leave most SIMDs without work
  const bool half = (int64_t)nblk * ((M + 127) / 128) < kHalfTileBelow;
  const int gbm = half ? 64 : 128;
  const int mblk = (int)((M + gbm - 1) / gbm);
  const int64_t tiles = (int64_t)nblk * mblk;
  // 8 XCDs, each owning every 8th n-block, walked in super-blocks of 8 m-blocks
  const int64_t nbp = (nblk + 7) / 8;
  const int64_t blocks = 8 * nbp * (((int64_t)mblk + 7) / 8) * 8;
  // too few tiles to give every SIMD two wavefronts: split k inside the workgroup
  const bool ks2 = tiles < 512 && (d / GB_K) % 2 == 0 && d / GB_K >= 4;
  const unsigned g = (unsigned)blocks;
  if (half && ks2) launch_gemm<2, 2>(g, stream, x, qweight, scales, zeros, bias, y, M, N, d, gsh, mblk, nblk);
  else if (half) launch_gemm<1, 2>(g, stream, x, qweight, scales, zeros, bias, y, M, N, d, gsh, mblk, nblk);
  else if (ks2) launch_gemm<2, 4>(g, stream, x, qweight, scales, zeros, bias, y, M, N, d, gsh, mblk, nblk);
  else launch_gemm<1, 4>(g, stream, x, qweight, scales, zeros, bias, y, M, N, d, gsh, mblk, nblk);
  return hipGetLastError();
}

}  // namespace paro
