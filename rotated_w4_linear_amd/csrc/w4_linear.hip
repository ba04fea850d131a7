// gfx950 kernel for the W4G128 linear layer on rotated activations with
// many tokens (prefill, M > 16):
//   Y[m][n] = sum_k X'[m][k] (q[n][k] - z[n][k/G]) s[n][k/G] + b[n]
// (CSDN article section 2.1: Y = (X T^-1)(T W) + b; paper notes "主实验":
// 4-bit weights, group G = 128; 64 and 256 are taken as well, each 64-channel
// k-tile reading the one group it lies in). Here the layer is a dense contraction and runs
// on the matrix cores. Dequantization (w4_common.h): two codes at a time are
// masked into the mantissas of a pair of fp16 1024.0 values with one
// v_and_or_b32, (1024 + q) - (1024 + z) = q - z is exact in packed fp16, and
// one packed multiply by the fp16 scale rounds once.
#include <algorithm>

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
// buffer access cache bits: sc0 (skip the per-CU cache) for loads of data
// another workgroup stored; sc0 | sc1 (memory-side) where workgroups may sit
// on different XCDs
constexpr int kAuxL2R = 1;
constexpr int kAuxSysW = 17;
// s_waitcnt immediate (gfx9 encoding): vmcnt(0) lgkmcnt(0), expcnt untouched
constexpr int kWaitVmLgkm0 = 0x70;
// lgkmcnt(0) alone (vmcnt and expcnt at their maxima)
constexpr int kWaitLgkm0 = 0xC07F;
// Output tiles (at 128 tokens) below which 64-token tiles are used: measured
// on MI355X, 64-token tiles win at 128 tiles (1024 x 4096 -> 4096: 699
// against 581 TFLOP/s) and lose at 256 (2048 x 4096 -> 4096: 760 against 918).
constexpr int64_t kHalfTileBelow = 256;
// 64-token tiles below which the tiles are also narrowed to 128 channels, so
// that every CU gets a workgroup
constexpr int64_t kNarrowTileBelow = 256;
// k-tiles per group of wavefronts below which the 64 x 128-tile kernel does
// not split k further across workgroups
constexpr int64_t kMinNarrowSplitKT = 4;
// 256 x 256 tiles (at 256 tokens) from which the wide kernel is used: measured
// on MI355X, 4096 x 4096 -> 4096 (256 tiles): 128 against 135 us; 2048 x
// 14336 -> 4096 (128 tiles) runs 372 against 288 us
constexpr int64_t kWideMinTiles = 256;
// Stream-K (the wide kernel with the tiles' k-tiles shared out evenly among
// the workgroups of each XCD) when each workgroup's range holds at least
// kMinSplitKT k-tiles: the partial tiles (256 KB per piece, written and read
// back) pay off only on long ranges. Measured on MI355X with uniform splits:
// 2048 x 14336 -> 4096 (two splits of 112 k-tiles) 242 against 292 us for the
// 128 x 256-tile kernel; 2048 x 4096 -> 4096 (two of 32) 88 against 73 us,
// 2048 x 4096 -> 1024 (eight of 8) 102 against 48 us
constexpr int64_t kMinSplitKT = 48;
// k-tiles a stream-K range is charged for cutting tiles at unequal k (see
// plan_w4_gemm)
constexpr int64_t kSkMisaligned = 20;
// n tiles of 32 channels per wavefront in the wide kernel
constexpr int kWideWN = 2;

// MT: 32-token m tiles per wavefront (4: 128-token workgroup tiles; 2: 64,
// for layers with few output tiles). NT: 32-channel n tiles per wavefront (2:
// 256-channel workgroup tiles; 1: 128, for layers with fewer still). SPLIT: k
// also split across ksplit workgroups per tile (consecutive slots of one
// XCD), which meet through fp32 partial tiles; the last to arrive adds them
// in split order.
template <int KS, int MT, int NT, bool SPLIT>
__global__ __launch_bounds__(256 * KS) __attribute__((amdgpu_waves_per_eu(2)))
void w4_gemm_kernel(const uint16_t* __restrict__ x, const uint8_t* __restrict__ qw,
                    const uint16_t* __restrict__ sc, const uint8_t* __restrict__ zr,
                    const uint16_t* __restrict__ bias, uint16_t* __restrict__ y, int M, int N,
                    int d, int gsh, int mblk, int nblk, int ksplit, float* __restrict__ part,
                    uint32_t* __restrict__ cnt, int sys, int mmaj) {
  constexpr int GB_M = 32 * MT;           // tokens per workgroup tile
  constexpr int GN = 128 * NT;            // output channels per workgroup tile
  constexpr int GB_XSTAGE = GB_M * GB_K;  // halfs per X' stage (16 KB at MT = 4)
  __shared__ __attribute__((aligned(1024))) _Float16 X0[KS][GB_XSTAGE], X1[KS][GB_XSTAGE];
  __shared__ __attribute__((aligned(1024))) u4 W0[KS][GB_WSTAGE], W1[KS][GB_WSTAGE];
  __shared__ __attribute__((aligned(16))) uint32_t S0[KS][GB_N], S1[KS][GB_N];
  __shared__ __attribute__((aligned(16))) uint32_t Z0[KS][GB_N], Z1[KS][GB_N];
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int kg = __builtin_amdgcn_readfirstlane(tid >> 8);     // k group (KS > 1)
  const int w = __builtin_amdgcn_readfirstlane((tid >> 6) & 3);  // wavefront inside the group
  // XCD-aware tile order: workgroup b runs on XCD b % 8. XCD x owns the
  // n-blocks x, x + 8, ... and walks them in super-blocks of 8 m-blocks x all
  // its n-blocks, so the workgroups resident on one XCD share both their X'
  // and their weight k-tiles through its L2; or (mmaj, layers with a large X'
  // and N < 4 M) XCD x owns the m-blocks x, x + 8, ... and all n-blocks, so
  // that it reads only its eighth of X'.
  const int xcd = blockIdx.x & 7, idx0 = blockIdx.x >> 3;
  if (!SPLIT) ksplit = 1;
  const int ks = idx0 % ksplit, idx = idx0 / ksplit;
  int mb, nb;
  if (mmaj) {
    // XCD x owns the m-blocks x, x + 8, ... and all n-blocks of each
    const int mi = idx / nblk;
    mb = xcd + 8 * mi;
    nb = idx - mi * nblk;
    if (mb >= mblk) return;
  } else {
    const int nbx = (nblk - xcd + 7) >> 3;
    if (nbx <= 0) return;
    const int mg = idx / (8 * nbx), rem = idx - mg * 8 * nbx;
    nb = xcd + 8 * (rem / 8);
    mb = mg * 8 + (rem & 7);
    if (mb >= mblk) return;
  }
  const int m0 = mb * GB_M;
  const int nw0 = nb * GN;         // workgroup's first output channel
  const int n0 = nw0 + 32 * NT * w;  // this wavefront's first output channel
  const int groups = d >> (6 + gsh);  // quantization groups of 64 << gsh channels per row
  const int KT = (d / GB_K) / (KS * ksplit);  // k-tiles per group of wavefronts
  const int kt0 = (ks * KS + kg) * KT;
  const int l32 = lane & 31, g = lane >> 5;

  // Buffer resources based at this tile's first row (byte offsets < 2^31,
  // checked on the host); rows past M or N are clamped to the last row.
  const __amdgpu_buffer_rsrc_t rx = __builtin_amdgcn_make_buffer_rsrc(
      (void*)(x + (size_t)m0 * d), (short)0, min(M - m0, GB_M) * d * 2, kRsrcWord3);
  const __amdgpu_buffer_rsrc_t rw = __builtin_amdgcn_make_buffer_rsrc(
      (void*)(qw + (size_t)nw0 * (d >> 1)), (short)0, min(N - nw0, GN) * (d >> 1), kRsrcWord3);
  const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(
      (void*)(sc + (size_t)nw0 * groups), (short)0, min(N - nw0, GN) * groups * 2, kRsrcWord3);
  const __amdgpu_buffer_rsrc_t rz = __builtin_amdgcn_make_buffer_rsrc(
      (void*)(zr + (size_t)nw0 * groups), (short)0, min(N - nw0, GN) * groups, kRsrcWord3);
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
  // code DMA c of wavefront w fills tile rows 32 (NT w + c) .. + 31
  uint32_t woff[2];
#pragma unroll
  for (int c = 0; c < NT; ++c) {
    const int r = 32 * (NT * w + c) + (lane >> 1);
    const int row = min(r, N - 1 - nw0);
    woff[c] = (uint32_t)(row * (d >> 1) + 16 * ((lane & 1) ^ ((r >> 3) & 1)));
  }
  // group scale and zero: lane l of wavefront w fetches row 64 w + l (NT = 1:
  // wavefronts 0 and 1 fetch the 128 rows)
  const bool szw = NT == 2 || w < 2;
  const uint32_t szrow = (uint32_t)(min(64 * w + lane, N - 1 - nw0) * groups);

  // the DMA of one k-tile: MT + NT + 2 load-to-LDS instructions per lane
  auto dma = [&](int kt, _Float16* xs, u4* ws, uint32_t* ss_l, uint32_t* zs_l) {
    const int kglob = kt0 + kt;
    const uint32_t gi = (uint32_t)(kglob >> gsh);  // the k-tile's group (64-channel k-tiles)
    if (szw) {
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (lds_void*)&ss_l[64 * w], 2, (szrow + gi) * 2u, 0, 0, 0);
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rz, (lds_void*)&zs_l[64 * w], 1, szrow + gi, 0, 0, 0);
    }
#pragma unroll
    for (int c = 0; c < MT; ++c)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rx, (lds_void*)&xs[(MT * w + c) * 64 * 8], 16, xoff[c],
                                               kglob * GB_K * 2, 0, 0);
#pragma unroll
    for (int c = 0; c < NT; ++c)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rw, (lds_void*)&ws[(NT * w + c) * 64], 16, woff[c],
                                               kglob * (GB_K / 2), 0, 0);
  };

  const uint32_t one = fp16_1024_pair();
  f16v acc[2][4];  // n tiles j < NT and m tiles mm < MT used
#pragma unroll
  for (int j = 0; j < NT; ++j)
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
    h2 ss[2], zz[2], ss16[2], zz16[2];
#pragma unroll
    for (int j = 0; j < NT; ++j) {
      const int r = 32 * NT * w + 32 * j + l32;
      wf[j] = wl[2 * r + (g ^ ((r >> 3) & 1))];
      // (rows past N read the last row's scale, clamped by the DMA; never stored)
      ss[j] = splat2(__builtin_bit_cast(_Float16, (uint16_t)(ss_l[r] & 0xffffu)));
      ss16[j] = ss[j] * splat2((_Float16)0.0625f);
      const float zf = (float)(zs_l[r] & 0xffu);
      zz[j] = splat2((_Float16)(1024.0f + zf));
      zz16[j] = splat2((_Float16)(1024.0f + 16.0f * zf));
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      h8 a[2], b[MT];
#pragma unroll
      for (int j = 0; j < NT; ++j) a[j] = dequant8(wf[j][i], zz[j], ss[j], zz16[j], ss16[j], one);
#pragma unroll
      for (int mm = 0; mm < MT; ++mm) {
        const int r = 32 * mm + l32;
        b[mm] = *(const h8*)(xb + r * GB_K + 8 * ((4 * g + i) ^ ((r >> 1) & 7)));
      }
#pragma unroll
      for (int j = 0; j < NT; ++j)
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

  if constexpr (KS > 1) {
    // the k groups add their partial sums pairwise through LDS, (0 + 1) +
    // (2 + 3): in the round of span s, group kg = r + s hands its sums to
    // group r (r a multiple of 2 s) through the X' stages 0 of groups r and
    // r + 1 (32 KB at MT = 4, 16 KB at MT = 2), PM m tiles of one n tile
    // (16 KB per m tile) at a time
    constexpr int PM = MT / 2;
#pragma unroll
    for (int span = 1; span < KS; span *= 2) {
      const int pos = kg & (2 * span - 1);
      float* red = (float*)&X0[kg - pos][0];
#pragma unroll
      for (int j = 0; j < NT; ++j) {
#pragma unroll
        for (int h = 0; h < MT / PM; ++h) {
          if (pos == span) {
#pragma unroll
            for (int mm = 0; mm < PM; ++mm)
#pragma unroll
              for (int e = 0; e < 16; ++e) red[((w * PM + mm) * 16 + e) * 64 + lane] = acc[j][PM * h + mm][e];
          }
          __syncthreads();
          if (pos == 0) {
#pragma unroll
            for (int mm = 0; mm < PM; ++mm)
#pragma unroll
              for (int e = 0; e < 16; ++e) acc[j][PM * h + mm][e] += red[((w * PM + mm) * 16 + e) * 64 + lane];
          }
          __syncthreads();
        }
      }
    }
    if constexpr (!SPLIT) {
      if (kg != 0) return;
    }
  }

  if constexpr (SPLIT) {
    // Split k across workgroups: group 0 of every workgroup of the tile stores
    // its fp32 partial tile ([w][f][lane] 16-byte chunks, GB_M x GN floats)
    // and the workgroup counts itself in; the last to arrive adds the partial
    // tiles in split order (so the sum does not depend on the order of
    // arrival), resets the counter and runs the epilogue. The workgroups of a
    // tile share an XCD: plain stores, an L2 atomic and loads that skip the
    // per-CU cache suffice; where the dispatch rule is not established (sys)
    // they go through memory. Every wavefront takes part in the barriers.
    __shared__ uint32_t s_last;
    const int tile = mb * nblk + nb;
    constexpr int NF = NT * MT * 4;  // 16-byte chunks per lane
    auto rsrc = [&](int k2) {
      return __builtin_amdgcn_make_buffer_rsrc(
          (void*)(part + ((size_t)tile * ksplit + k2) * (size_t)(GB_M * GN)), (short)0, GB_M * GN * 4, kRsrcWord3);
    };
    if (kg == 0) {
      const __amdgpu_buffer_rsrc_t rmine = rsrc(ks);
#pragma unroll
      for (int f = 0; f < NF; ++f) {
        const int j = f / (MT * 4), mm = (f / 4) % MT, q = f % 4;
        const u4 v = __builtin_bit_cast(u4, f4{acc[j][mm][4 * q], acc[j][mm][4 * q + 1], acc[j][mm][4 * q + 2],
                                               acc[j][mm][4 * q + 3]});
        const int off = ((w * NF + f) * 64 + lane) * 16;
        if (sys) __builtin_amdgcn_raw_buffer_store_b128(v, rmine, off, 0, kAuxSysW);
        else __builtin_amdgcn_raw_buffer_store_b128(v, rmine, off, 0, 0);
      }
    }
    __builtin_amdgcn_s_waitcnt(0);  // this wavefront's stores have reached L2 / memory
    __syncthreads();
    if (tid == 0) {
      uint32_t old;
      if (sys) old = __hip_atomic_fetch_add(&cnt[tile], 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);
      else old = __hip_atomic_fetch_add(&cnt[tile], 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      s_last = old == (uint32_t)(ksplit - 1);
    }
    __syncthreads();
    if (!s_last || kg != 0) return;
#pragma unroll
    for (int f = 0; f < NF; ++f) {
      const int j = f / (MT * 4), mm = (f / 4) % MT, q = f % 4;
      const int off = ((w * NF + f) * 64 + lane) * 16;
      f4 t = {0.f, 0.f, 0.f, 0.f};
      for (int k2 = 0; k2 < ksplit; ++k2) {
        const f4 v = __builtin_bit_cast(f4, sys ? __builtin_amdgcn_raw_buffer_load_b128(rsrc(k2), off, 0, kAuxSysW)
                                                : __builtin_amdgcn_raw_buffer_load_b128(rsrc(k2), off, 0, kAuxL2R));
        t = k2 == 0 ? v : t + v;
      }
#pragma unroll
      for (int e = 0; e < 4; ++e) acc[j][mm][4 * q + e] = t[e];
    }
    if (tid == 0) {
      if (sys) __hip_atomic_store(&cnt[tile], 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);
      else __hip_atomic_store(&cnt[tile], 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
  }

  // epilogue: acc[j][mm][e] = C[n = n0 + 32 j + 8 (e/4) + 4 g + e%4][m = m0 + 32 mm + l32].
  // Each wavefront stages its 32 NT (n) x 64 (m) output blocks through an LDS
  // region of its own (the operand stages are free after the last barrier) as
  // fp16 rows of 32 NT outputs (CR = 4 NT 16-byte chunks), chunk c of row r at
  // position c ^ (r % CR), and then stores whole rows: lane l writes chunk
  // l % CR of row l / CR of each group of 64 / CR rows.
  {
    constexpr int CR = 4 * NT, RB = 16 * CR;
    uint8_t* stage = w == 0 ? (uint8_t*)&X0[0][0] : w == 1 ? (uint8_t*)&X1[0][0]
                   : w == 2 ? (uint8_t*)&W0[0][0] : (uint8_t*)&W1[0][0];
    constexpr int PASSES = MT / 2;  // 64 tokens per pass
#pragma unroll
    for (int ps = 0; ps < PASSES; ++ps) {
#pragma unroll
      for (int j = 0; j < NT; ++j) {
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int nl = 32 * j + 8 * q + 4 * g;  // local output channel of e = 4 q
          float b4[4] = {0.f, 0.f, 0.f, 0.f};
          if (bias && n0 + nl < N) {
            const uint2 braw = *(const uint2*)(bias + n0 + nl);
            b4[0] = half_lo(braw.x);
            b4[1] = half_hi(braw.x);
            b4[2] = half_lo(braw.y);
            b4[3] = half_hi(braw.y);
          }
#pragma unroll
          for (int t = 0; t < 2; ++t) {
            const int mm = 2 * ps + t;
            const int rl = 32 * t + l32;  // row of the staged block
            uint2 pk;
            pk.x = half_bits(acc[j][mm][4 * q + 0] + b4[0]) | (half_bits(acc[j][mm][4 * q + 1] + b4[1]) << 16);
            pk.y = half_bits(acc[j][mm][4 * q + 2] + b4[2]) | (half_bits(acc[j][mm][4 * q + 3] + b4[3]) << 16);
            const int c = nl >> 3;  // 16-byte chunk, 8-byte half (nl >> 2) & 1
            *(uint2*)(stage + rl * RB + ((c ^ (rl % CR)) << 4) + (((nl >> 2) & 1) << 3)) = pk;
          }
        }
      }
      // (the region is this wavefront's own: its LDS accesses complete in order)
#pragma unroll
      for (int rr = 0; rr < CR; ++rr) {
        const int rl = (64 / CR) * rr + lane / CR, c = lane % CR;
        const u4 v = *(const u4*)(stage + rl * RB + ((c ^ (rl % CR)) << 4));
        const int m = m0 + 64 * ps + rl, n = n0 + 8 * c;
        if (m < M && n < N) *(u4*)(y + (size_t)m * N + n) = v;
      }
    }
  }
}

// --------------------------------------------------------------------------
// prefill, layers with many output tiles: 256 (m) x 256 (n) workgroup tiles
// and one wavefront per SIMD with 256 fp32 accumulators per lane. The
// wavefront tile is 64 (n) x 256 (m) (WN = 2): each dequantized weight
// fragment feeds eight MFMAs, half the vector work per MFMA of the 64 x 128
// wavefront tiles above (measured on the MLP layer: 868 against 911 us for
// 128 x 128 wavefront tiles, WN = 4). The wavefront's own instruction stream
// overlaps the next step's dequantization with the current MFMAs. Staging,
// swizzles, the k order and the dequantization are those of w4_gemm_kernel;
// the X' stage holds 256 rows (32 KB).
// --------------------------------------------------------------------------
constexpr int GW_M = 256;
constexpr int GW_XSTAGE = GW_M * GB_K;  // halfs per X' stage (32 KB)
// groups per row up to which the wide kernel keeps all scales and zeros of its
// tile in LDS (48 KB at 64; a multiple of 16 groups, scales and zeros 16-byte
// aligned)
constexpr int kPanelGroups = 64;
// stream-K workgroups per XCD at most (one workgroup per CU: 256 CUs in 8
// XCDs)
constexpr int kSkSlots = 32;
// wide-kernel modes
constexpr int kModeTile = 0, kModeSkOne = 1, kModeSkMany = 2;

// Instruction order inside a scheduling region of 16 MFMAs: the region's ND
// LDS reads first, the first NW MFMAs alone (while those reads return), then
// each MFMA followed by up to NV vector instructions (the next step's
// dequantization); the first NG MFMAs are each followed by one global load
// (the DMA of a k-tile), so that issuing the loads, which holds the
// wavefront's in-order issue, overlaps running MFMAs.
// One chunk of four MFMAs: the chunk's ND LDS reads first, then each MFMA
// followed by up to NV vector instructions and, for the first NG, one global
// load with the scalar write of its LDS address (M0) before it.
template <int ND, int NV, int NG>
__device__ __forceinline__ void sched_chunk() {
  if constexpr (ND > 0) __builtin_amdgcn_sched_group_barrier(0x100, ND, 0);
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
    if constexpr (NV > 0) __builtin_amdgcn_sched_group_barrier(0x002, NV, 0);
    if (k < NG) {
      __builtin_amdgcn_sched_group_barrier(0x004, 1, 0);
      __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);
    }
  }
}

template <int ND, int NW, int NV, int NG>
__device__ __forceinline__ void sched_order() {
  __builtin_amdgcn_sched_group_barrier(0x100, ND, 0);
#pragma unroll
  for (int k = 0; k < 16; ++k) {
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
    if (k >= NW) __builtin_amdgcn_sched_group_barrier(0x002, NV, 0);
    if (k < NG) {
      __builtin_amdgcn_sched_group_barrier(0x004, 1, 0);  // the load's M0 write
      __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);
    }
  }
}

// WN: 32-channel n tiles per wavefront (4: 128 (n) x 128 (m) wavefront tiles,
// 2: 64 (n) x 256 (m)); MTW = 16 / WN m tiles of 32 tokens.
// MODE: kModeTile, one tile per workgroup; kModeSkOne and kModeSkMany,
// stream-K (separate instantiations, so that the reduction's and the segment
// loop's registers do not weigh on the others). Stream-K: the grid is `slots` (<= kSkSlots) workgroups
// per XCD. The tiles of XCD x (its n-blocks x, x + 8, ... in the
// data-parallel order) are laid end to end as one sequence of k-tiles, and
// workgroup j of the XCD takes the j-th of `slots` equal ranges of it (even
// lengths): whole tiles,
// plus at most one partial tile at each end. The pieces of a partial tile
// meet through fp32 partial tiles in the workspace; the last to arrive adds
// them in k order and runs the epilogue.
template <int WN, bool PANEL, int MODE>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(1)))
void w4_gemm_wide_kernel(const uint16_t* __restrict__ x, const uint8_t* __restrict__ qw,
                         const uint16_t* __restrict__ sc, const uint8_t* __restrict__ zr,
                         const uint16_t* __restrict__ bias, uint16_t* __restrict__ y, int M, int N,
                         int d, int gsh, int mblk, int nblk, int slots, float* __restrict__ part,
                         uint32_t* __restrict__ cnt, int sys) {
  __shared__ __attribute__((aligned(1024))) _Float16 X0[GW_XSTAGE], X1[GW_XSTAGE];
  __shared__ __attribute__((aligned(1024))) u4 W0[GB_WSTAGE], W1[GB_WSTAGE];
  __shared__ __attribute__((aligned(16))) uint32_t S0[GB_N], S1[GB_N], Z0[GB_N], Z1[GB_N];
  // PANEL: the tile's scales and zeros of the groups a segment's k-tiles span
  // (from the 8-aligned group below its first), loaded once per segment and
  // stored group-major ([group][256 rows]), so that the 32 rows one read
  // spans are consecutive in LDS
  __shared__ __attribute__((aligned(1024))) uint16_t SPT[PANEL ? GB_N * kPanelGroups : 8];
  __shared__ __attribute__((aligned(1024))) uint8_t ZPT[PANEL ? GB_N * kPanelGroups : 16];
  __shared__ uint32_t s_last;
  constexpr bool SK = MODE != kModeTile;
  const int tid_k = threadIdx.x;
  const int w = __builtin_amdgcn_readfirstlane(tid_k >> 6);  // wavefront 0..3
  constexpr int MTW = 16 / WN, NWAV = 8 / WN;               // m tiles; wavefronts along n
  const int wn = w % NWAV, wm = w / NWAV;                   // the wavefront's n and m blocks
  // XCD-aware tile order, as in w4_gemm_kernel
  const int xcd = blockIdx.x & 7;
  const int nbx = (nblk - xcd + 7) >> 3;
  if (nbx <= 0) return;
  const int groups = d >> (6 + gsh);
  const int L = d / GB_K;  // k-tiles per tile
  const uint32_t one = fp16_1024_pair();
  // SK: range j of this XCD's sequence of k-tiles starts at rstart(j)
  // (`slots` ranges of H / slots k-tile pairs, rounded down); owner(u) is
  // the range holding k-tile u (the host keeps every range non-empty)
  const int jw = blockIdx.x >> 3;
  const int64_t H = SK ? (int64_t)nbx * mblk * L / 2 : 1;
  auto rstart = [&](int j) -> int64_t { return 2 * (((int64_t)j * H) / slots); };
  auto owner = [&](int64_t u) -> int {
    int j = (int)min((int64_t)slots - 1, (u / 2) * slots / H);
    while (j + 1 < slots && rstart(j + 1) <= u) ++j;
    while (j > 0 && rstart(j) > u) --j;
    return j;
  };

  // One segment: k-tiles kt0 .. kt0 + KT - 1 (KT even) of tile (mb, nb), the
  // XCD's tile tl; first: the workgroup's first segment
  auto segment = [&](const int mb, const int nb, const int kt0, const int KT, const int tl, const bool first) {
  // the lane index through an opaque copy, so that nothing derived from it is
  // hoisted out of the segment loop and held (spilled) across the k-loop
  int tid_o = tid_k;
  asm volatile("" : "+v"(tid_o));
  const int tid = tid_o, lane = tid & 63, l32 = lane & 31, g = lane >> 5;
  const int m0 = mb * GW_M;
  const int nw0 = nb * GB_N;
  const int pg0 = PANEL ? ((kt0 >> gsh) & ~7) : 0;  // first group of the panel

  // buffer resources at the tile's first row (byte offsets < 2^31: d <= 2^21,
  // checked on the host); rows past M or N are clamped to the last row
  const __amdgpu_buffer_rsrc_t rx = __builtin_amdgcn_make_buffer_rsrc(
      (void*)(x + (size_t)m0 * d), (short)0, min(M - m0, GW_M) * d * 2, kRsrcWord3);
  const __amdgpu_buffer_rsrc_t rw = __builtin_amdgcn_make_buffer_rsrc(
      (void*)(qw + (size_t)nw0 * (d >> 1)), (short)0, min(N - nw0, GB_N) * (d >> 1), kRsrcWord3);
  const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(
      (void*)(sc + (size_t)nw0 * groups), (short)0, min(N - nw0, GB_N) * groups * 2, kRsrcWord3);
  const __amdgpu_buffer_rsrc_t rz = __builtin_amdgcn_make_buffer_rsrc(
      (void*)(zr + (size_t)nw0 * groups), (short)0, min(N - nw0, GB_N) * groups, kRsrcWord3);
  // X' DMA c (0..7) of wavefront w fills tile rows 8 (8 w + c) .. + 7
  uint32_t xoff[8];
#pragma unroll
  for (int c = 0; c < 8; ++c) {
    const int r = 8 * (8 * w + c) + (lane >> 3);
    const int row = min(r, M - 1 - m0);
    xoff[c] = (uint32_t)(row * d + 8 * ((lane & 7) ^ ((r >> 1) & 7))) * 2u;
  }
  // code DMA c (0..1) of wavefront w fills tile rows 32 (2 w + c) .. + 31
  uint32_t woff[2];
#pragma unroll
  for (int c = 0; c < 2; ++c) {
    const int r = 32 * (2 * w + c) + (lane >> 1);
    const int row = min(r, N - 1 - nw0);
    woff[c] = (uint32_t)(row * (d >> 1) + 16 * ((lane & 1) ^ ((r >> 3) & 1)));
  }
  // group scale and zero: lane l of wavefront w fetches row 64 w + l
  const uint32_t szrow = (uint32_t)(min(64 * w + lane, N - 1 - nw0) * groups);

  // the DMA of one k-tile: twelve load-to-LDS instructions per lane (ten
  // with PANEL: no scale and zero); dma3(q) issues instructions 3 q .. 3 q + 2
  auto dma3 = [&](int q, int ktl, _Float16* xs, u4* ws, uint32_t* ss_l, uint32_t* zs_l) {
    const int kt = kt0 + ktl;  // global k-tile
    const uint32_t gi = (uint32_t)(kt >> gsh);
#pragma unroll
    for (int c0 = 3 * q; c0 < 3 * q + 3; ++c0) {
      const int c = c0 + (PANEL ? 2 : 0);
      if (c >= 12) break;
      if (c == 0)
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (lds_void*)&ss_l[64 * w], 2, (szrow + gi) * 2u, 0, 0, 0);
      else if (c == 1)
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rz, (lds_void*)&zs_l[64 * w], 1, szrow + gi, 0, 0, 0);
      else if (c < 10)
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rx, (lds_void*)&xs[(8 * w + c - 2) * 64 * 8], 16, xoff[c - 2],
                                                 kt * GB_K * 2, 0, 0);
      else
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rw, (lds_void*)&ws[(2 * w + c - 10) * 64], 16, woff[c - 10],
                                                 kt * (GB_K / 2), 0, 0);
    }
  };
  auto dma = [&](int kt, _Float16* xs, u4* ws, uint32_t* ss_l, uint32_t* zs_l) {
#pragma unroll
    for (int q = 0; q < 4; ++q) dma3(q, kt, xs, ws, ss_l, zs_l);
  };

  // (arrays are sized for the largest WN and MTW and used up to WN, MTW: the
  // host pass of hipcc cannot instantiate lambdas capturing arrays of
  // template-dependent size)
  f16v acc[4][8];  // [n tile j][m tile mm]
#pragma unroll
  for (int j = 0; j < WN; ++j)
#pragma unroll
    for (int mm = 0; mm < MTW; ++mm)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[j][mm][e] = 0.0f;

  // A k-tile's per-row operands: the 32 codes of each of the wavefront's WN
  // n tiles and their group's scale and zero, in the forms dequant8 takes.
  struct Params {
    u4 wf[4];
    h2 ss[4], zz[4], ss16[4], zz16[4];
  };
  // the LDS reads of the operands (raw scale and zero words), then their
  // conversion
  struct Raw {
    u4 wf[4];
    uint32_t s[4], z[4];
  };
  auto read_raw = [&](int ktl, const u4* wl, const uint32_t* ss_l, const uint32_t* zs_l, Raw& q) {
    const int gi = (kt0 + ktl) >> gsh;
#pragma unroll
    for (int j = 0; j < WN; ++j) {
      const int r = 32 * WN * wn + 32 * j + l32;
      q.wf[j] = wl[2 * r + (g ^ ((r >> 3) & 1))];
      if constexpr (PANEL) {
        q.s[j] = SPT[(gi - pg0) * GB_N + r];
        q.z[j] = ZPT[(gi - pg0) * GB_N + r];
      } else {
        q.s[j] = ss_l[r];
        q.z[j] = zs_l[r];
      }
    }
  };
  auto convert = [&](const Raw& q, Params& p) {
#pragma unroll
    for (int j = 0; j < WN; ++j) {
      p.wf[j] = q.wf[j];
      p.ss[j] = splat2(__builtin_bit_cast(_Float16, (uint16_t)(q.s[j] & 0xffffu)));
      p.ss16[j] = p.ss[j] * splat2((_Float16)0.0625f);
      const float zf = (float)(q.z[j] & 0xffu);
      p.zz[j] = splat2((_Float16)(1024.0f + zf));
      p.zz16[j] = splat2((_Float16)(1024.0f + 16.0f * zf));
    }
  };
  auto load_params = [&](int kt, const u4* wl, const uint32_t* ss_l, const uint32_t* zs_l, Params& p) {
    Raw q;
    read_raw(kt, wl, ss_l, zs_l, q);
    convert(q, p);
  };
  // X' fragments of MFMA step i (0..3) of a k-tile for the MTW m tiles
  auto read_b = [&](const _Float16* xb, int i, h8* bf) {
#pragma unroll
    for (int mm = 0; mm < MTW; ++mm) {
      const int r = 32 * MTW * wm + 32 * mm + l32;
      bf[mm] = *(const h8*)(xb + r * GB_K + 8 * ((4 * g + i) ^ ((r >> 1) & 7)));
    }
  };
  auto deq = [&](const Params& p, int i, h8* af) {
#pragma unroll
    for (int j = 0; j < WN; ++j) af[j] = dequant8(p.wf[j][i], p.zz[j], p.ss[j], p.zz16[j], p.ss16[j], one);
  };
  auto mma = [&](const h8* af, const h8* bf) {
#pragma unroll
    for (int j = 0; j < WN; ++j)
#pragma unroll
      for (int mm = 0; mm < MTW; ++mm)
        acc[j][mm] = __builtin_amdgcn_mfma_f32_32x32x16_f16(af[j], bf[mm], acc[j][mm], 0, 0, 0);
  };
  // MFMAs 4 q .. 4 q + 3 of the 16 of one step (j major)
  auto mma4 = [&](int q, const h8* af, const h8* bf) {
#pragma unroll
    for (int f = 4 * q; f < 4 * q + 4; ++f)
      acc[f / MTW][f % MTW] = __builtin_amdgcn_mfma_f32_32x32x16_f16(af[f / MTW], bf[f % MTW], acc[f / MTW][f % MTW], 0, 0, 0);
  };
  // Pipeline: while the MFMAs of step i of k-tile kt run, the wavefront reads
  // and dequantizes the operands of step i + 1. After step 2 it waits for the
  // DMA of k-tile kt + 1 and the barrier, so that step 3 overlaps the first
  // operands of kt + 1 (read from the other stage). Past that barrier every
  // wavefront has read all it needs of k-tile kt, so the DMA of kt + 2 into
  // kt's stage goes out there, a whole k-tile before it is waited for; past
  // the last tile it reloads the last tile, which is read but not used.
  Params P, Pn;
  h8 a[4], b[8], an[4], bn[8];
  auto tile = [&](int kt, _Float16* xb, u4* wl, uint32_t* sb, uint32_t* zb, const _Float16* xn,
                  const u4* wnx, const uint32_t* sn, const uint32_t* zn) {
#pragma unroll
    for (int i = 0; i < 3; ++i) {
      read_b(xb, i + 1, bn);
      deq(P, i + 1, an);
      mma(a, b);
      sched_order<MTW, 0, WN + 1, 0>();
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int t = 0; t < 8; ++t) {
        if (t < WN) a[t] = an[t];
        if (t < MTW) b[t] = bn[t];
      }
    }
    __builtin_amdgcn_s_waitcnt(kWaitVmLgkm0);
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_sched_barrier(0);
    // step 3 in four chunks of four MFMAs, each with three of the twelve
    // loads of the DMA of kt + 2 and a share of kt + 1's operand work
    const int kd = min(kt + 2, KT - 1);
    Raw raw;
    read_raw(kt + 1, wnx, sn, zn, raw);
    read_b(xn, 0, bn);
    mma4(0, a, b);
    dma3(0, kd, xb, wl, sb, zb);
    sched_chunk<MTW + 3 * WN, 0, 3>();
    __builtin_amdgcn_sched_barrier(0);
    convert(raw, Pn);
    mma4(1, a, b);
    dma3(1, kd, xb, wl, sb, zb);
    sched_chunk<0, 3 * WN, 3>();
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int j = 0; j < WN / 2; ++j) an[j] = dequant8(Pn.wf[j][0], Pn.zz[j], Pn.ss[j], Pn.zz16[j], Pn.ss16[j], one);
    mma4(2, a, b);
    dma3(2, kd, xb, wl, sb, zb);
    sched_chunk<0, (13 * WN / 2 + 3) / 4, 3>();
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int j = WN / 2; j < WN; ++j) an[j] = dequant8(Pn.wf[j][0], Pn.zz[j], Pn.ss[j], Pn.zz16[j], Pn.ss16[j], one);
    mma4(3, a, b);
    dma3(3, kd, xb, wl, sb, zb);
    sched_chunk<0, (13 * WN / 2 + 3) / 4, 3>();
    __builtin_amdgcn_sched_barrier(0);
    P = Pn;
#pragma unroll
    for (int t = 0; t < 8; ++t) {
      if (t < WN) a[t] = an[t];
      if (t < MTW) b[t] = bn[t];
    }
  };

  if constexpr (PANEL) {
    // lane l of wavefront w loads the scales (fp16) and zeros (bytes) of the
    // panel's pg groups of tile row 64 w + l, its own row, in 16-byte pieces
    // (the last piece may run into the next groups or row, which are stored
    // but never read; past the tile's rows it reads zero), and stores them
    // group-major
    const __amdgpu_buffer_rsrc_t rsp = __builtin_amdgcn_make_buffer_rsrc(
        (void*)(sc + (size_t)nw0 * groups), (short)0, min(N - nw0, GB_N) * groups * 2, kRsrcWord3);
    const __amdgpu_buffer_rsrc_t rzp = __builtin_amdgcn_make_buffer_rsrc(
        (void*)(zr + (size_t)nw0 * groups), (short)0, min(N - nw0, GB_N) * groups, kRsrcWord3);
    const int rr = 64 * w + lane;
    const int pg = ((kt0 + KT - 1) >> gsh) - pg0 + 1;  // at most kPanelGroups (checked on the host)
    u4 sv[kPanelGroups / 8], zv[kPanelGroups / 16];
#pragma unroll
    for (int c = 0; c < kPanelGroups / 8; ++c)
      if (c < (pg + 7) / 8)
        sv[c] = __builtin_bit_cast(u4, __builtin_amdgcn_raw_buffer_load_b128(rsp, (rr * groups + pg0) * 2 + 16 * c, 0, 0));
#pragma unroll
    for (int c = 0; c < kPanelGroups / 16; ++c)
      if (c < (pg + 15) / 16)
        zv[c] = __builtin_bit_cast(u4, __builtin_amdgcn_raw_buffer_load_b128(rzp, rr * groups + pg0 + 16 * c, 0, 0));
#pragma unroll
    for (int c = 0; c < kPanelGroups / 8; ++c)
      if (c < (pg + 7) / 8) {
#pragma unroll
        for (int t = 0; t < 8; ++t) SPT[(8 * c + t) * GB_N + rr] = (uint16_t)(sv[c][t >> 1] >> (16 * (t & 1)));
      }
#pragma unroll
    for (int c = 0; c < kPanelGroups / 16; ++c)
      if (c < (pg + 15) / 16) {
#pragma unroll
        for (int t = 0; t < 16; ++t) ZPT[(16 * c + t) * GB_N + rr] = (uint8_t)(zv[c][t >> 2] >> (8 * (t & 3)));
      }
  }
  dma(0, X0, W0, S0, Z0);
  __builtin_amdgcn_s_waitcnt(kWaitVmLgkm0);
  __builtin_amdgcn_s_barrier();
  dma(min(1, KT - 1), X1, W1, S1, Z1);
  load_params(0, W0, S0, Z0, P);
  read_b(X0, 0, b);
  deq(P, 0, a);
  for (int kt = 0; kt < KT; kt += 2) {  // KT even (checked on the host)
    tile(kt, X0, W0, S0, Z0, X1, W1, S1, Z1);
    tile(kt + 1, X1, W1, S1, Z1, X0, W0, S0, Z0);
  }
  // the last tile's step 3 read a stage that the epilogue below overwrites
  __builtin_amdgcn_s_waitcnt(kWaitVmLgkm0);
  __builtin_amdgcn_s_barrier();

  if constexpr (SK) {
    if (KT != L) {
      // A partial tile: the workgroup stores its fp32 partial tile (wavefront
      // w's 256 accumulators per lane as [w][64 groups of 4][lane], 256 KB) in
      // its slot (0: its first segment, 1: its last; only those two can be
      // partial) and counts itself in on the counter of the tile's first
      // range; the last piece to arrive adds the pieces in range order (so
      // the sum does not depend on the order of arrival), resets the counter
      // and runs the epilogue. The ranges of a tile are those of one XCD, so
      // plain stores, an L2 atomic and loads that skip the per-CU cache
      // suffice; where the dispatch rule is not established (sys) they go
      // through memory.
      const size_t tile_floats = (size_t)GW_M * GB_N;
      auto rsrc = [&](int j, int slot) {
        return __builtin_amdgcn_make_buffer_rsrc(
            (void*)(part + ((size_t)(xcd * kSkSlots + j) * 2 + slot) * tile_floats), (short)0,
            (int)(tile_floats * 4), kRsrcWord3);
      };
      const __amdgpu_buffer_rsrc_t rmine = rsrc(jw, first ? 0 : 1);
#pragma unroll
      for (int f = 0; f < 64; ++f) {
        const int j = f >> 5, mm = (f >> 2) & 7, q = f & 3;
        const u4 v = __builtin_bit_cast(u4, f4{acc[j][mm][4 * q], acc[j][mm][4 * q + 1], acc[j][mm][4 * q + 2],
                                               acc[j][mm][4 * q + 3]});
        const int off = ((w * 64 + f) * 64 + lane) * 16;
        if (sys) __builtin_amdgcn_raw_buffer_store_b128(v, rmine, off, 0, kAuxSysW);
        else __builtin_amdgcn_raw_buffer_store_b128(v, rmine, off, 0, 0);
      }
      const int ja = owner((int64_t)tl * L);
      const int pieces = owner((int64_t)tl * L + L - 1) - ja + 1;
      const int ctr = xcd * slots + ja;
      __builtin_amdgcn_s_waitcnt(0);  // this wavefront's stores have reached L2 / memory
      __syncthreads();
      if (tid == 0) {
        uint32_t old;
        if (sys) old = __hip_atomic_fetch_add(&cnt[ctr], 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);
        else old = __hip_atomic_fetch_add(&cnt[ctr], 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        s_last = old == (uint32_t)(pieces - 1);
      }
      __syncthreads();
      if (!s_last) return;
      // the first piece is range ja's first segment if the tile is the first
      // of that range, else its last
      const int slot0 = rstart(ja) / L == tl ? 0 : 1;
      // 16 groups of 4 accumulators at a time, summed in range order from the
      // stored partial tiles (this workgroup's own included)
#pragma unroll
      for (int f0 = 0; f0 < 64; f0 += 16) {
        f4 r[16];
        for (int p = 0; p < pieces; ++p) {
          const __amdgpu_buffer_rsrc_t rk = rsrc(ja + p, p == 0 ? slot0 : 0);
          f4 v[16];
#pragma unroll
          for (int e = 0; e < 16; ++e) {
            const int off = ((w * 64 + f0 + e) * 64 + lane) * 16;
            v[e] = __builtin_bit_cast(f4, sys ? __builtin_amdgcn_raw_buffer_load_b128(rk, off, 0, kAuxSysW)
                                              : __builtin_amdgcn_raw_buffer_load_b128(rk, off, 0, kAuxL2R));
          }
#pragma unroll
          for (int e = 0; e < 16; ++e) r[e] = p == 0 ? v[e] : r[e] + v[e];
        }
#pragma unroll
        for (int e = 0; e < 16; ++e) {
          const int f = f0 + e, j = f >> 5, mm = (f >> 2) & 7, q = f & 3;
#pragma unroll
          for (int c = 0; c < 4; ++c) acc[j][mm][4 * q + c] = r[e][c];
        }
      }
      if (tid == 0) {
        if (sys) __hip_atomic_store(&cnt[ctr], 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);
        else __hip_atomic_store(&cnt[ctr], 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      }
    }
  }

  // epilogue: acc[j][mm][e] = C[n = n0 + 32 j + 8 (e/4) + 4 g + e%4][m = mw0 + 32 mm + l32],
  // staged per wavefront through an 8 KB LDS region of its own (a quarter of
  // the X' stage 0, free after the last barrier) in 64 x 64 blocks, as in
  // w4_gemm_kernel
  const int n0 = nw0 + 32 * WN * wn, mw0 = m0 + 32 * MTW * wm;
  uint8_t* stage = (uint8_t*)X0 + 8192 * w;
#pragma unroll
  for (int jh = 0; jh < WN / 2; ++jh) {
#pragma unroll
    for (int ps = 0; ps < MTW / 2; ++ps) {
#pragma unroll
      for (int jj = 0; jj < 2; ++jj) {
        const int j = 2 * jh + jj;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int nl = 32 * jj + 8 * q + 4 * g;  // channel of e = 4 q inside the 64-channel block
          const int n = n0 + 64 * jh + nl;
          float b4[4] = {0.f, 0.f, 0.f, 0.f};
          if (bias && n < N) {
            const uint2 braw = *(const uint2*)(bias + n);
            b4[0] = half_lo(braw.x);
            b4[1] = half_hi(braw.x);
            b4[2] = half_lo(braw.y);
            b4[3] = half_hi(braw.y);
          }
#pragma unroll
          for (int t = 0; t < 2; ++t) {
            const int mm = 2 * ps + t;
            const int rl = 32 * t + l32;
            uint2 pk;
            pk.x = half_bits(acc[j][mm][4 * q + 0] + b4[0]) | (half_bits(acc[j][mm][4 * q + 1] + b4[1]) << 16);
            pk.y = half_bits(acc[j][mm][4 * q + 2] + b4[2]) | (half_bits(acc[j][mm][4 * q + 3] + b4[3]) << 16);
            const int c = nl >> 3;
            *(uint2*)(stage + rl * 128 + ((c ^ (rl & 7)) << 4) + (((nl >> 2) & 1) << 3)) = pk;
          }
        }
      }
#pragma unroll
      for (int rr = 0; rr < 8; ++rr) {
        const int rl = 8 * rr + (lane >> 3), c = lane & 7;
        const u4 v = *(const u4*)(stage + rl * 128 + ((c ^ (rl & 7)) << 4));
        const int m = mw0 + 64 * ps + rl, n = n0 + 64 * jh + 8 * c;
        if (m < M && n < N) *(u4*)(y + (size_t)m * N + n) = v;
      }
    }
  }
  };

  if constexpr (!SK) {
    // one tile per workgroup: XCD x walks all of its n-blocks for each
    // m-block in turn, so that the tiles resident on it at once span few
    // m-blocks. An X' block (256 rows) is four times the bytes of a weight
    // block, so sharing X' blocks saves more L2 misses than sharing weight
    // blocks (MLP 8192 x 4096 -> 14336: 0.792 -> 0.783 ms against super-blocks
    // of 8 m-blocks, fewer misses at the same work)
    const int idx = blockIdx.x >> 3;
    const int mb = idx / nbx;
    const int nb = xcd + 8 * (idx - mb * nbx);
    if (mb >= mblk) return;
    segment(mb, nb, 0, L, 0, true);
  } else {
    // the XCD's tile t, its n-blocks walked in super-blocks of 8 m-blocks
    // (the last super-block may hold fewer)
    int64_t u = rstart(jw);
    const int64_t ue = rstart(jw + 1);
    const int tfirst = (int)(u / L);
    if constexpr (MODE == kModeSkOne) {
      // every range lies in one tile (checked on the host)
      const int t = tfirst;
      const int sb = t / (8 * nbx);
      const int rows = min(8, mblk - 8 * sb);
      const int rem = t - sb * 8 * nbx;
      segment(8 * sb + rem % rows, xcd + 8 * (rem / rows), (int)(u - (int64_t)t * L), (int)(ue - u), t, true);
    } else {
      while (u < ue) {
        const int t = (int)(u / L);
        const int k0 = (int)(u - (int64_t)t * L);
        const int k1 = (int)min((int64_t)L, k0 + (ue - u));
        const int sb = t / (8 * nbx);
        const int rows = min(8, mblk - 8 * sb);
        const int rem = t - sb * 8 * nbx;
        segment(8 * sb + rem % rows, xcd + 8 * (rem / rows), k0, k1 - k0, t, t == tfirst);
        u += k1 - k0;
        if (u < ue) {
          // the epilogue's LDS reads before the next segment's DMA and panel
          // (an LDS wait and a barrier: __syncthreads would also wait for the
          // epilogue's global stores)
          __builtin_amdgcn_s_waitcnt(kWaitLgkm0);
          __builtin_amdgcn_s_barrier();
        }
      }
    }
  }
}

template <int KS, int MT, int NT>
void launch_gemm(unsigned blocks, hipStream_t stream, const uint16_t* x, const uint8_t* qweight,
                 const uint16_t* scales, const uint8_t* zeros, const uint16_t* bias, uint16_t* y,
                 int64_t M, int64_t N, int64_t d, int gsh, int mblk, int nblk, int mmaj) {
  hipLaunchKernelGGL((w4_gemm_kernel<KS, MT, NT, false>), dim3(blocks), dim3(256 * KS), 0, stream, x, qweight,
                     scales, zeros, bias, y, (int)M, (int)N, (int)d, gsh, mblk, nblk, 1, nullptr, nullptr, 0,
                     mmaj);
}

// Smaller-tile kernel geometry, as launch_w4_gemm chooses it: 64-token tiles
// when 128-token ones would leave most SIMDs without work, 128-channel ones
// when even those leave CUs without a workgroup; k split two or four ways
// inside the workgroup; and (nsplit > 1) across workgroups when the tiles do
// not fill the CUs.
struct SmallGemm {
  int nblk256, mblk, nblk, ksin, nsplit;
  bool half, narrow;
  int64_t tiles;
};
SmallGemm small_gemm(int64_t M, int64_t N, int64_t d) {
  SmallGemm g;
  g.nblk256 = (int)((N + GB_N - 1) / GB_N);
  g.half = (int64_t)g.nblk256 * ((M + 127) / 128) < kHalfTileBelow;
  const int gbm = g.half ? 64 : 128;
  g.mblk = (int)((M + gbm - 1) / gbm);
  g.narrow = g.half && (int64_t)g.nblk256 * g.mblk < kNarrowTileBelow;
  g.nblk = g.narrow ? (int)((N + GB_N / 2 - 1) / (GB_N / 2)) : g.nblk256;
  g.tiles = (int64_t)g.nblk * g.mblk;
  const int64_t kt = d / GB_K;
  const bool ks2 = g.tiles < 512 && kt % 2 == 0 && kt >= 4;
  const bool ks4 = g.narrow && kt % 4 == 0 && kt >= 16;
  g.ksin = ks4 ? 4 : ks2 ? 2 : 1;
  // with 64 x 128 tiles (and k split four ways inside) that leave CUs idle:
  // up to 4 workgroups per tile, each group of wavefronts keeping at least
  // kMinNarrowSplitKT k-tiles
  g.nsplit = 1;
  if (g.narrow && g.ksin == 4)
    while (g.nsplit < 4 && g.tiles * 2 * g.nsplit <= 256 && kt % (g.ksin * 2 * g.nsplit) == 0 &&
           kt / (g.ksin * 2 * g.nsplit) >= kMinNarrowSplitKT && g.tiles <= (int64_t)(kDecodeCounterBytes / 4))
      g.nsplit *= 2;
  return g;
}

}  // namespace

GemmPlan plan_w4_gemm(int64_t M, int64_t N, int64_t d) {
  GemmPlan p;
  const int64_t nblk = (N + GB_N - 1) / GB_N, mblkw = (M + GW_M - 1) / GW_M;
  const int64_t tiles = nblk * mblkw, kt = d / GB_K;
  if (M <= kDecodeMaxM || d > (int64_t(1) << 21) || kt % 2 || d < 4 * GB_K) return p;
  // one tile per workgroup from kWideMinTiles tiles (stream-K measured slower
  // there: 2048 x 4096 -> 14336, 448 tiles, 252 against 223 us, the
  // workgroups of an XCD no longer reading the same k-tiles at the same
  // time); below, stream-K when every XCD holds n-blocks
  if (tiles >= kWideMinTiles) {
    p.wide = true;
    return p;
  }
  const int64_t nbmin = nblk / 8, nbmax = (nblk + 7) / 8;
  // Workgroups per XCD: the fewest k-tiles per range on the busiest XCD,
  // counting kSkMisaligned more for ranges that do not cut the tiles into
  // equal pieces (nor hold whole tiles): their pieces start at different k,
  // so the workgroups of an XCD stop sharing k-tiles in L2 (measured: 1300 x
  // 8192 -> 4096, 96 tiles of 128 k-tiles, 123 us with ranges of 48 against
  // 113 with 24 workgroups per XCD taking half tiles). Every range keeps at
  // least two k-tiles on the least busy XCD and kMinSplitKT on the busiest;
  // ranges of whole tiles (one tile per workgroup on fewer workgroups than
  // CUs) are not taken, nor misaligned ones on fewer than 3/4 of the CUs.
  int best = 0;
  int64_t best_cost = 0;
  for (int sl = kSkSlots; nbmin >= 1 && sl >= kSkSlots / 2; sl -= 4) {
    const int64_t units = nbmax * mblkw * kt;
    if (nbmin * mblkw * kt < 2 * sl) continue;
    const int64_t U = (units + sl - 1) / sl;
    if (U < kMinSplitKT || U % kt == 0) continue;  // (whole tiles: fewer workgroups than CUs)
    const bool aligned = units % (2 * sl) == 0 && kt % U == 0;
    if (!aligned && sl < kSkSlots * 3 / 4) continue;
    const int64_t cost = U + (aligned ? 0 : kSkMisaligned);
    if (!best || cost < best_cost) {
      best = sl;
      best_cost = cost;
    }
  }
  if (best) {
    p.wide = p.sk = true;
    p.sk_slots = best;
    p.partial_bytes = (size_t)8 * kSkSlots * 2 * GW_M * GB_N * 4;
    return p;
  }
  const SmallGemm g = small_gemm(M, N, d);
  if (g.nsplit > 1) {
    p.nsplit = g.nsplit;
    p.partial_bytes = (size_t)g.tiles * g.nsplit * 64 * 128 * 4;
  }
  return p;
}

namespace {
// A stream-K split's most groups per segment panel (from the 8-aligned group
// below a segment's first k-tile's: whole tiles span all of a row's groups,
// partial ones lie at the ends of the ranges), and whether every range lies
// in one tile.
void sk_shape(int64_t nblk, int64_t mblkw, int64_t L, int gsh, int slots, int64_t* panel_groups, bool* one_tile) {
  auto span = [&](int64_t kt0, int64_t KT) { return ((kt0 + KT - 1) >> gsh) - ((kt0 >> gsh) & ~int64_t(7)) + 1; };
  int64_t most = 0;
  bool one = true;
  for (int64_t x = 0; x < 8; ++x) {
    const int64_t nbx = (nblk - x + 7) / 8;
    if (nbx <= 0) continue;
    const int64_t H = nbx * mblkw * L / 2;
    for (int64_t j = 0; j < slots; ++j) {
      const int64_t s = 2 * (j * H / slots), e = 2 * ((j + 1) * H / slots);
      if (e <= s) continue;
      const int64_t t = s / L, k0 = s - t * L, te = (e - 1) / L;
      one = one && te == t;
      most = std::max(most, span(k0, std::min(L - k0, e - s)));
      if (te > t) most = std::max(most, span(0, e - te * L));
      if (te > t + 1 || (te > t && k0 == 0)) most = std::max(most, span(0, L));
    }
  }
  *panel_groups = most;
  *one_tile = one;
}
}  // namespace

hipError_t launch_w4_gemm(const uint16_t* x, const uint8_t* qweight, const uint16_t* scales,
                          const uint8_t* zeros, const uint16_t* bias, uint16_t* y, int64_t M,
                          int64_t N, int64_t d, int group, uint32_t* cnt, float* part, hipStream_t stream) {
  if (M == 0) return hipSuccess;
  const int gsh = group == 64 ? 0 : group == 128 ? 1 : 2;
  const SmallGemm sg = small_gemm(M, N, d);
  const int nblk256 = sg.nblk256, mblk = sg.mblk, nblk = sg.nblk;
  const bool half = sg.half, narrow = sg.narrow;
  // 8 XCDs, each owning every 8th n-block, walked in super-blocks of 8 m-blocks
  const int64_t nbp = (nblk + 7) / 8;
  const int64_t blocks = 8 * nbp * (((int64_t)mblk + 7) / 8) * 8;
  const bool ks2 = sg.ksin == 2, ks4 = sg.ksin == 4;
  // The smaller-tile kernel's XCD order. By n-blocks, every XCD reads all of
  // X' (2 M d bytes) and an eighth of the weights; by m-blocks, an eighth of
  // X' and all of the weights (N d / 2 bytes), which is less when N < 4 M.
  // Where X' is at least 8 MiB (twice an XCD's L2) the saved re-reads show:
  // plain GEMM, 2048 x 4096 -> 1024 35.5 -> 32.0 us, 1024 x 4096 -> 1024
  // 26.3 -> 24.8, 4096 x 4096 -> 1024 102 -> 56; 2048 x 4096 -> 4096 the same
  // (76.5 us); with X' in L2 (2048 x 1024 -> 1024, 4 MiB) by n-blocks stays
  // faster (14.1 against 16.1 us). At least 8 m-blocks, so that every XCD
  // gets one.
  const int mmaj = mblk >= 8 && N < 4 * M && 2 * M * d >= (int64_t(8) << 20);
  const unsigned g = mmaj ? 8u * (unsigned)((mblk + 7) / 8) * (unsigned)nblk : (unsigned)blocks;
  // layers with many 256 x 256 tiles take the one-wavefront-per-SIMD kernel,
  // one tile per workgroup when the tiles fill whole rounds of one workgroup
  // per CU, else stream-K when the workspace holds the partial tiles
  const GemmPlan plan = plan_w4_gemm(M, N, d);
  if (plan.wide && (!plan.sk || (cnt && part))) {
    const int mblkw = (int)((M + GW_M - 1) / GW_M);
    const int64_t L = d / GB_K;
    const int64_t groups = d >> (6 + gsh);
    const int sys = plan.sk && !xcd_dispatch_is_round_robin();
    // the scale and zero panel: at most kPanelGroups groups per segment;
    // rows of a multiple of 8 groups, scales 16-byte and zeros 8-byte aligned
    int64_t pgs = groups;
    bool one_tile = false;
    if (plan.sk) sk_shape(nblk256, mblkw, L, gsh, plan.sk_slots, &pgs, &one_tile);
    const bool panel = pgs <= kPanelGroups && groups % 8 == 0 && ((uintptr_t)scales & 15) == 0 &&
                       ((uintptr_t)zeros & 7) == 0;
    const int64_t bw = plan.sk ? 8 * plan.sk_slots : 8 * ((nblk256 + 7) / 8) * (int64_t)mblkw;
    auto go = [&](auto kernel) {
      hipLaunchKernelGGL(kernel, dim3((unsigned)bw), dim3(256), 0, stream, x, qweight, scales, zeros, bias, y,
                         (int)M, (int)N, (int)d, gsh, mblkw, nblk256, plan.sk_slots, part, cnt, sys);
    };
    if (plan.sk && one_tile) {
      if (panel) go(w4_gemm_wide_kernel<kWideWN, true, kModeSkOne>);
      else go(w4_gemm_wide_kernel<kWideWN, false, kModeSkOne>);
    } else if (plan.sk) {
      if (panel) go(w4_gemm_wide_kernel<kWideWN, true, kModeSkMany>);
      else go(w4_gemm_wide_kernel<kWideWN, false, kModeSkMany>);
    } else {
      if (panel) go(w4_gemm_wide_kernel<kWideWN, true, kModeTile>);
      else go(w4_gemm_wide_kernel<kWideWN, false, kModeTile>);
    }
    return hipGetLastError();
  }
  if (ks4 && sg.nsplit > 1 && cnt && part) {
    const int sys = !xcd_dispatch_is_round_robin();
    hipLaunchKernelGGL((w4_gemm_kernel<4, 2, 1, true>), dim3(g * (unsigned)sg.nsplit), dim3(1024), 0, stream, x,
                       qweight, scales, zeros, bias, y, (int)M, (int)N, (int)d, gsh, mblk, nblk, sg.nsplit, part,
                       cnt, sys, mmaj);
  } else if (ks4) launch_gemm<4, 2, 1>(g, stream, x, qweight, scales, zeros, bias, y, M, N, d, gsh, mblk, nblk, mmaj);
  else if (narrow && ks2) launch_gemm<2, 2, 1>(g, stream, x, qweight, scales, zeros, bias, y, M, N, d, gsh, mblk, nblk, mmaj);
  else if (narrow) launch_gemm<1, 2, 1>(g, stream, x, qweight, scales, zeros, bias, y, M, N, d, gsh, mblk, nblk, mmaj);
  else if (half && ks2) launch_gemm<2, 2, 2>(g, stream, x, qweight, scales, zeros, bias, y, M, N, d, gsh, mblk, nblk, mmaj);
  else if (half) launch_gemm<1, 2, 2>(g, stream, x, qweight, scales, zeros, bias, y, M, N, d, gsh, mblk, nblk, mmaj);
  else if (ks2) launch_gemm<2, 4, 2>(g, stream, x, qweight, scales, zeros, bias, y, M, N, d, gsh, mblk, nblk, mmaj);
  else launch_gemm<1, 4, 2>(g, stream, x, qweight, scales, zeros, bias, y, M, N, d, gsh, mblk, nblk, mmaj);
  return hipGetLastError();
}

}  // namespace paro
