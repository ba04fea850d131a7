// gfx950 kernel for the W4G128 linear layer with few tokens (decode, M <= 64),
// with the online activation transform fused in:
//   Y[m][n] = sum_k X'[m][k] (q[n][k] - z[n][k/G]) s[n][k/G] + b[n],
//   X' = X T^-1
// (G = 128; 64 and 256 as well: each lane's 32 codes of a segment lie in one
// group)
// (CSDN article section 2.1: Y = (X T^-1)(T W) + b; paper notes "关键设计"
// for the rotation and "主实验" for the 4-bit, group-128 weights).
//
// With at most 16 tokens the layer is a stream over the packed weights, so
// the kernel is organised around keeping HBM busy:
//  * a workgroup owns a k-slice of 512 input channels (four 128-channel
//    groups) and 128 output channels (64 for layers where 128 would leave
//    CUs idle). Each wavefront first loads the activations (and schedule) of
//    segment w of the slice, then issues all of its weight loads (32 or 16
//    rows x 512 k);
//  * while the weights are in flight, wavefront w rotates its segment for
//    all tokens in registers (the per-lane machinery of the stand-alone
//    rotation: K stages, K + 1 LDS exchanges) and writes X' into a shared,
//    swizzled LDS tile; without a plan it copies X there;
//  * the weights are dequantized in registers group by group as they land
//    and multiplied on the matrix cores (v_mfma_f32_16x16x32_f16: 16 output
//    channels x 32 k x 16 tokens; columns past M are ignored);
//  * k-slices meet through fp32 partial sums in the workspace; the last
//    workgroup of an n-block to arrive (an atomic arrival counter, reset to
//    zero by that workgroup) adds them in k-slice order, adds the bias and
//    rounds to fp16, so the result does not depend on arrival order.
// Partial sums and counters must be coherent between the workgroups of one
// n-block. MI355X's L2 is per XCD and not coherent across XCDs, and an
// agent-scope fence (write-back of the whole L2) costs more than the layer.
// Workgroup b is dispatched to XCD b % 8, and all k-slices of an n-block get
// equal b % 8, so they meet in one L2: plain stores, an L2 atomic and loads
// that skip the per-CU L1 suffice. paro_device_init (which
// paro_rotation_create runs too) checks that dispatch rule once per device
// with a probe kernel that reads each workgroup's XCC id; where it does not
// hold, or on a device that was never checked, the partial sums and the
// counter go through memory-side (system scope) stores, loads and atomics
// instead. The kernel launch itself only reads the recorded result.
// The rotation is recomputed by each of the N / 128 n-blocks that read a
// segment: with few tokens this is ALU work hidden under the weight loads.
//
// Dequantization (w4_common.h): two codes at a time are masked into the
// mantissas of a pair of fp16 1024.0 values, (v - (1024 + z)) = q - z is
// exact, and one packed multiply by the fp16 scale rounds once; the codes of
// a word come out in channel order, and X' is stored in LDS in channel order.
#include <atomic>
#include <mutex>
#include <string>
#include <vector>

#include "paro_internal.h"
#include "rotate_core.h"
#include "w4_common.h"

#pragma clang fp contract(off)

namespace paro {
namespace {

using namespace w4;

constexpr int DK_SEGS = 4;                 // 128-channel groups per k-slice
constexpr int DK_TOK = 16;                 // token columns of the MFMA tile
constexpr int kRsrcWord3 = 0x00020000;     // gfx9 buffer resource word 3
constexpr int kAuxL2 = 1;                  // sc0: skip the per-CU cache
constexpr int kAuxSys = 17;                // sc0 | sc1: memory-side coherence

// Byte offset in the X' tile of channel k (local to the 512-wide slice) of
// token m: chunk k / 8 at position (k / 8) ^ m, half k % 8 inside it.
__device__ __forceinline__ int xl_offset(int m, int k) {
  const int c = k >> 3;
  return (m * 64 + (c ^ m)) * 16 + 2 * (k & 7);
}

// T: token rows staged and rotated (4 for M <= 4, else 16); MFMA columns past
// T read tile rows that were never written and are ignored like those past M.
// TJ: 16-row tiles per wavefront (the workgroup owns 64 TJ output channels).
// TB: blocks of 16 token columns (T = 16; M up to 16 TB): the blocks'
// activations are transformed one after the other, and every dequantized
// weight fragment feeds TB MFMAs.
// At least four wavefronts per SIMD with one block (registers within 128):
// with the transform at T = 16 the kernel took 117 VGPRs and 16 AGPRs, three
// wavefronts per SIMD, and layers with more than 768 workgroups (gate/up-proj
// at M = 16: 896) then ran in two rounds.
template <bool ROT, int KMAX, bool KEXACT, bool FAST, int T, int TJ, bool SZV, int TB>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(TB == 1 ? 4 : 2))) void w4_decode_kernel(
    const uint16_t* __restrict__ x, const uint8_t* __restrict__ qw,
    const uint16_t* __restrict__ sc, const uint8_t* __restrict__ zr,
    const uint16_t* __restrict__ bias, uint16_t* __restrict__ y, int M, int N, int d,
    const uint32_t* __restrict__ tab, int K, float* part, uint32_t* cnt, int ksl, int nbl,
    int nb_base, int sys, int gsh) {
  // X' tile: [16 TB tokens][64 chunks of 16 bytes]; chunk c of token m is
  // stored at position c ^ m, so the 16 tokens of one MFMA operand read land
  // on 16 distinct 16-byte positions.
  __shared__ u4 xl[DK_TOK * TB * 64];
  // the transform's exchange slots; with four token blocks they share the
  // LDS of the last block's rows (written only after every wavefront's last
  // transform), so that two workgroups fit a CU
  constexpr bool XCH_IN_XL = ROT && TB == 4;
  __shared__ rot::f4 xch_own[ROT && !XCH_IN_XL ? 4 * (T / 4) * 64 : 1];
  rot::f4* xch = XCH_IN_XL ? (rot::f4*)&xl[DK_TOK * (TB - 1) * 64] : xch_own;
  __shared__ int s_last;

  constexpr int NB = 64 * TJ;  // output channels per workgroup
  const int tid = threadIdx.x, lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int xcd = blockIdx.x & 7, j8 = blockIdx.x >> 3;
  const int nb = xcd + 8 * (j8 / ksl);  // n-block inside this launch
  const int ks = j8 % ksl;              // k-slice
  if (nb >= nbl) return;
  const int nbg = nb_base + nb;
  const int groups = d >> 7;            // 128-channel segments
  const int sgr = d >> (6 + gsh);       // quantization groups (64 << gsh channels) per row
  const int g0 = ks * DK_SEGS;
  const int nq = min(DK_SEGS, groups - g0);
  const int r = lane & 15, kq = lane >> 4;
  const int rb = nbg * NB + 16 * TJ * w;  // this wavefront's first output channel
  char* xlb = (char*)xl;

  // ---- 1. activations of segment g0 + w (token rows past M repeat M - 1) ---
  // (in a slice cut short by the end of d, wavefronts without a segment
  // process a copy of the last one into their own, never read, part of the
  // tile: no branch lets the compiler sink these loads behind the weights)
  // (every token block's activations before the weights: loads complete in
  // order, so a block requested after the weights would wait for all of them)
  const int seg = min(g0 + w, groups - 1);
  uint32_t raw[TB][T];
  rot::Lane<1, KMAX, KEXACT, FAST> L;
  {
    const uint32_t* xs = (const uint32_t*)(x + seg * 128) + lane;
#pragma unroll
    for (int tb = 0; tb < TB; ++tb)
#pragma unroll
      for (int i = 0; i < T; ++i) raw[tb][i] = xs[(size_t)min(16 * tb + i, M - 1) * (size_t)(d >> 1)];
    if constexpr (ROT) L.load(tab, seg, K, lane);
  }
  __builtin_amdgcn_sched_barrier(0);

  // ---- 2. packed weights and group parameters: rows rb + 16 j + r ----------
  // lane (r, kq) holds bytes 16 kq .. 16 kq + 15 of group g0 + q of its row,
  // i.e. codes 128 (g0 + q) + 32 kq + 8 i + e for MFMA step i. All loads are
  // issued here, group by group, without waiting: groups past the end of d
  // re-read the last group (never used) and the scale and zero are converted
  // only when their group is multiplied. With SZV (the number of groups is a
  // multiple of four, so every slice has four groups and a row's four scales
  // and four zeros start 8- and 4-byte aligned) they come in as one 8-byte and
  // one 4-byte load per row instead of eight 2- and 1-byte loads: small loads
  // cost as much issue and queue time as 16-byte ones.
  u4 wv[TJ][DK_SEGS];
  uint32_t sraw[TJ][DK_SEGS], zraw[TJ][DK_SEGS];
  const uint8_t* wrow[TJ];
  size_t grow[TJ];
#pragma unroll
  for (int j = 0; j < TJ; ++j) {
    const int nc = min(rb + 16 * j + r, N - 1);  // rows past N are never stored
    wrow[j] = qw + (size_t)nc * (size_t)(d >> 1) + 16 * kq;
    grow[j] = (size_t)nc * sgr;
  }
  if constexpr (SZV) {  // (group 128: sgr == groups)
    uint2 s4[TJ];
    uint32_t z4[TJ];
#pragma unroll
    for (int j = 0; j < TJ; ++j) {
      s4[j] = *(const uint2*)(sc + grow[j] + g0);
      z4[j] = *(const uint32_t*)(zr + grow[j] + g0);
    }
#pragma unroll
    for (int q = 0; q < DK_SEGS; ++q)
#pragma unroll
      for (int j = 0; j < TJ; ++j) wv[j][q] = *(const u4*)(wrow[j] + 64 * (g0 + q));
#pragma unroll
    for (int q = 0; q < DK_SEGS; ++q)
#pragma unroll
      for (int j = 0; j < TJ; ++j) {
        sraw[j][q] = ((q < 2 ? s4[j].x : s4[j].y) >> (16 * (q & 1))) & 0xffffu;
        zraw[j][q] = (z4[j] >> (8 * q)) & 0xffu;
      }
  } else {
#pragma unroll
    for (int q = 0; q < DK_SEGS; ++q) {
      const int g = min(g0 + q, groups - 1);
      const int gq = ((g << 7) + 32 * kq) >> (6 + gsh);  // this lane's 32 codes share one group
#pragma unroll
      for (int j = 0; j < TJ; ++j) {
        wv[j][q] = *(const u4*)(wrow[j] + 64 * g);
        sraw[j][q] = sc[grow[j] + gq];
        zraw[j][q] = zr[grow[j] + gq];
      }
    }
  }
  // keep every load above ahead of the first use of the activations: the
  // in-order load counter would otherwise hold the weight loads back
  __builtin_amdgcn_sched_barrier(0);

  // ---- 3. X' of the segment into the LDS tile (block by block) --------------
#pragma unroll
  for (int tb = 0; tb < TB; ++tb) {
    uint32_t pk[T];
    int k0;  // slice-local channel of the low half of this lane's pair
    if constexpr (ROT) {
      float X[1][T], B[1][T];
#pragma unroll
      for (int i = 0; i < T; ++i) L.unpack(raw[tb][i], 0, X[0][i], B[0][i]);
      L.template run<T>(X, B, (char*)&xch[w * (T / 4) * 64]);
#pragma unroll
      for (int i = 0; i < T; ++i) pk[i] = L.pack(X[0][i], B[0][i], 0);
      k0 = 128 * w + (int)(L.stoff[0] >> 1);
      if (XCH_IN_XL && tb == TB - 1) __syncthreads();  // every wavefront is done with the slots
    } else {
#pragma unroll
      for (int i = 0; i < T; ++i) pk[i] = raw[tb][i];
      k0 = 128 * w + 2 * lane;
    }
    // (k0 is even: the lane's two channels are adjacent halves of one chunk)
#pragma unroll
    for (int i = 0; i < T; ++i) *(uint32_t*)(xlb + xl_offset(16 * tb + i, k0)) = pk[i];
  }
  __syncthreads();

  // ---- 4. dequantize and multiply, group by group as the weights land -------
  const uint32_t one = fp16_1024_pair();
  f4 acc[TB][TJ];
#pragma unroll
  for (int tb = 0; tb < TB; ++tb)
#pragma unroll
    for (int j = 0; j < TJ; ++j) acc[tb][j] = f4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int q = 0; q < DK_SEGS; ++q) {
    if (q < nq) {
      h2 ss[TJ], zz[TJ], ss16[TJ], zz16[TJ];
#pragma unroll
      for (int j = 0; j < TJ; ++j) {
        ss[j] = splat2(__builtin_bit_cast(_Float16, (uint16_t)sraw[j][q]));
        ss16[j] = ss[j] * splat2((_Float16)0.0625f);
        zz[j] = splat2((_Float16)(1024.0f + (float)zraw[j][q]));
        zz16[j] = splat2((_Float16)(1024.0f + 16.0f * (float)zraw[j][q]));
      }
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        h8 b[TB];
#pragma unroll
        for (int tb = 0; tb < TB; ++tb) {
          const int m = 16 * tb + r;
          b[tb] = *(const h8*)(xlb + (m * 64 + ((16 * q + 4 * kq + i) ^ m)) * 16);
        }
#pragma unroll
        for (int j = 0; j < TJ; ++j) {
          const h8 a = dequant8(wv[j][q][i], zz[j], ss[j], zz16[j], ss16[j], one);
#pragma unroll
          for (int tb = 0; tb < TB; ++tb)
            acc[tb][j] = __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b[tb], acc[tb][j], 0, 0, 0);
        }
      }
    }
  }

  // ---- 5. acc[tb][j][e] = Y[n = rb + 16 j + 4 kq + e][m = 16 tb + r] ------------
  auto store_y = [&](int m, int n, f4 v) {
    if (bias) {
      const uint2 braw = *(const uint2*)(bias + n);
      v[0] += half_lo(braw.x);
      v[1] += half_hi(braw.x);
      v[2] += half_lo(braw.y);
      v[3] += half_hi(braw.y);
    }
    uint2 o;
    o.x = half_bits(v[0]) | (half_bits(v[1]) << 16);
    o.y = half_bits(v[2]) | (half_bits(v[3]) << 16);
    *(uint2*)(y + (size_t)m * N + n) = o;
  };
  if (ksl == 1) {
#pragma unroll
    for (int tb = 0; tb < TB; ++tb)
#pragma unroll
      for (int j = 0; j < TJ; ++j) {
        const int n = rb + 16 * j + 4 * kq, m = 16 * tb + r;
        if (m < M && n < N) store_y(m, n, acc[tb][j]);
      }
    return;
  }
  // partial sums: [k-slice][M][N] fp32; offsets in bytes from part (< 2^31,
  // checked on the host)
  const __amdgpu_buffer_rsrc_t rp =
      __builtin_amdgcn_make_buffer_rsrc((void*)part, (short)0, 0x7fffffff, kRsrcWord3);
#pragma unroll
  for (int tb = 0; tb < TB; ++tb)
#pragma unroll
    for (int j = 0; j < TJ; ++j) {
      const int n = rb + 16 * j + 4 * kq, m = 16 * tb + r;
      if (m < M && n < N) {
        const int off = (int)((((size_t)ks * M + m) * N + n) * 4);
        const u4 v = __builtin_bit_cast(u4, acc[tb][j]);
        if (sys) __builtin_amdgcn_raw_buffer_store_b128(v, rp, off, 0, kAuxSys);
        else __builtin_amdgcn_raw_buffer_store_b128(v, rp, off, 0, 0);
      }
    }
  __builtin_amdgcn_s_waitcnt(0);  // this wavefront's stores have reached L2 / memory
  __syncthreads();
  if (tid == 0) {
    uint32_t old;
    if (sys) old = __hip_atomic_fetch_add(&cnt[nb], 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);
    else old = __hip_atomic_fetch_add(&cnt[nb], 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    s_last = old == (uint32_t)(ksl - 1);
  }
  __syncthreads();
  if (!s_last) return;

  // ---- 6. last k-slice to arrive: sum the k-slices, bias, fp16 --------------
  // The order of the additions is fixed (it does not depend on which slice
  // arrived last). Each four-output item's slices are added in slice order by
  // one thread, loads issued eight slices at a time. With more than eight
  // slices (one round of loads no longer covers them) and few items per
  // n-block (at most 128), groups of consecutive slices are instead summed in
  // parallel, each in slice order, and the group sums added in group order.
  const int slice_bytes = M * N * 4;
  const int items = M * (NB / 4);
  auto sum_slices = [&](int off0, int s0, int s1) {
    f4 acc = {0.f, 0.f, 0.f, 0.f};
    for (int k2 = s0; k2 < s1; k2 += 8) {
      u4 v[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        const int off = off0 + min(k2 + u, s1 - 1) * slice_bytes;
        v[u] = sys ? __builtin_amdgcn_raw_buffer_load_b128(rp, off, 0, kAuxSys)
                   : __builtin_amdgcn_raw_buffer_load_b128(rp, off, 0, kAuxL2);
      }
#pragma unroll
      for (int u = 0; u < 8; ++u)
        if (k2 + u < s1) acc = (k2 + u == s0) ? __builtin_bit_cast(f4, v[u]) : acc + __builtin_bit_cast(f4, v[u]);
    }
    return acc;
  };
  if (ksl > 8 && 2 * items <= 256) {
    const int spg = (ksl + min(ksl, 256 / items) - 1) / min(ksl, 256 / items);  // slices per group
    const int ng = (ksl + spg - 1) / spg;                                       // groups
    f4* red = (f4*)xl;  // [group][item]; the X' tile is no longer read
    if (tid < items * ng) {
      const int item = tid % items, gi = tid / items;
      const int m = item / (NB / 4);
      const int n = nbg * NB + 4 * (item % (NB / 4));
      f4 g = {0.f, 0.f, 0.f, 0.f};
      if (n < N) g = sum_slices((int)(((size_t)m * N + n) * 4), gi * spg, min(gi * spg + spg, ksl));
      red[gi * items + item] = g;
    }
    __syncthreads();
    if (tid < items) {
      const int m = tid / (NB / 4);
      const int n = nbg * NB + 4 * (tid % (NB / 4));
      if (n < N) {
        f4 t = red[tid];
        for (int gi = 1; gi < ng; ++gi) t += red[gi * items + tid];
        store_y(m, n, t);
      }
    }
  } else {
    for (int it = tid; it < items; it += 256) {
      const int m = it / (NB / 4);
      const int n = nbg * NB + 4 * (it % (NB / 4));
      if (n >= N) continue;
      store_y(m, n, sum_slices((int)(((size_t)m * N + n) * 4), 0, ksl));
    }
  }
  if (tid == 0) {
    if (sys) __hip_atomic_store(&cnt[nb], 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);
    else __hip_atomic_store(&cnt[nb], 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
}

// Reads the XCC id of the XCD each workgroup runs on (hardware register 20,
// bits 0..3).
__global__ void xcc_probe_kernel(uint32_t* out) {
  if (threadIdx.x == 0) out[blockIdx.x] = __builtin_amdgcn_s_getreg((3 << 11) | 20) & 0xFu;
}

// Per device: 0 = not probed, 1 = workgroup b runs on the XCD of every other
// workgroup with the same b % 8 and the eight classes use eight XCDs (the
// round-robin dispatch the kernel relies on), 2 = it does not.
std::atomic<int> g_xcd_state[kMaxDevices];

}  // namespace

int xcd_dispatch_probe(int dev) {
  if (dev < 0 || dev >= kMaxDevices) return PARO_ERR_UNSUPPORTED;
  static std::mutex mu;
  std::lock_guard<std::mutex> lock(mu);
  if (g_xcd_state[dev].load(std::memory_order_acquire) != 0) return PARO_OK;
  constexpr int kBlocks = 4096;
  uint32_t* d_out = nullptr;
  hipError_t e = hipMalloc(&d_out, kBlocks * sizeof(uint32_t));
  if (e != hipSuccess) {
    set_error(std::string("device init: hipMalloc: ") + hipGetErrorString(e));
    return PARO_ERR_HIP;
  }
  std::vector<uint32_t> h(kBlocks, 0xFFFFFFFFu);
  hipLaunchKernelGGL(xcc_probe_kernel, dim3(kBlocks), dim3(64), 0, 0, d_out);
  e = hipGetLastError();
  if (e == hipSuccess) e = hipMemcpy(h.data(), d_out, kBlocks * sizeof(uint32_t), hipMemcpyDeviceToHost);
  (void)hipFree(d_out);
  if (e != hipSuccess) {  // nothing is cached: a later call probes again
    set_error(std::string("device init: XCD probe: ") + hipGetErrorString(e));
    return PARO_ERR_HIP;
  }
  bool ok = true;
  uint32_t seen = 0;
  for (int b = 0; b < kBlocks; ++b) {
    if (h[b] != h[b & 7]) ok = false;
    if (h[b] < 32) seen |= 1u << h[b];
    else ok = false;
  }
  if (__builtin_popcount(seen) != 8) ok = false;
  g_xcd_state[dev].store(ok ? 1 : 2, std::memory_order_release);
  return PARO_OK;
}

// The hot path only reads what the probe recorded; a device never probed
// takes the memory-side path, which is correct under any dispatch.
bool xcd_dispatch_is_round_robin() {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return false;
  return g_xcd_state[dev].load(std::memory_order_acquire) == 1;
}

namespace {

template <bool ROT, int KMAX, bool KEXACT, bool FAST, int T, int TJ, bool SZV, int TB>
hipError_t launch_t(const uint16_t* x, const uint8_t* qw, const uint16_t* sc, const uint8_t* zr,
                    const uint16_t* bias, uint16_t* y, int M, int N, int d, int gsh,
                    const paro_rotation* r, void* ws, hipStream_t stream) {
  const int ksl = (d / 128 + DK_SEGS - 1) / DK_SEGS;
  const int nbl_all = (N + 64 * TJ - 1) / (64 * TJ);
  uint32_t* cnt = (uint32_t*)ws;
  float* part = (float*)((char*)ws + kDecodeCounterBytes);
  const uint32_t* tab = r ? r->d_table : nullptr;
  const int K = r ? r->lay.stages : 0;
  constexpr int kMaxNb = (int)(kDecodeCounterBytes / 4);
  const int sys = ksl > 1 && !xcd_dispatch_is_round_robin();
  for (int nb0 = 0; nb0 < nbl_all; nb0 += kMaxNb) {
    const int nbl = min(kMaxNb, nbl_all - nb0);
    const unsigned blocks = 8u * (unsigned)ksl * (unsigned)((nbl + 7) / 8);
    hipLaunchKernelGGL((w4_decode_kernel<ROT, KMAX, KEXACT, FAST, T, TJ, SZV, TB>), dim3(blocks), dim3(256), 0,
                       stream, x, qw, sc, zr, bias, y, M, N, d, tab, K, part, cnt, ksl, nbl, nb0,
                       sys, gsh);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

template <int T, int TJ, bool SZV, int TB>
hipError_t launch_plan(const uint16_t* x, const uint8_t* qw, const uint16_t* sc, const uint8_t* zr,
                       const uint16_t* bias, uint16_t* y, int m, int n, int k, int gsh,
                       const paro_rotation* r, void* ws, hipStream_t stream) {
  if (!r) return launch_t<false, 0, true, true, T, TJ, SZV, TB>(x, qw, sc, zr, bias, y, m, n, k, gsh, r, ws, stream);
  if (r->lay.stages == 0) return launch_t<true, 0, true, true, T, TJ, SZV, TB>(x, qw, sc, zr, bias, y, m, n, k, gsh, r, ws, stream);
  if (r->lay.fast) {
    if (r->lay.stages == 8) return launch_t<true, 8, true, true, T, TJ, SZV, TB>(x, qw, sc, zr, bias, y, m, n, k, gsh, r, ws, stream);
    return launch_t<true, 8, false, true, T, TJ, SZV, TB>(x, qw, sc, zr, bias, y, m, n, k, gsh, r, ws, stream);
  }
  return launch_t<true, 8, false, false, T, TJ, SZV, TB>(x, qw, sc, zr, bias, y, m, n, k, gsh, r, ws, stream);
}

}  // namespace

bool decode_fuses_rotation(const paro_rotation* r) {
  return r == nullptr || (r->lay.ppl == 1 && r->lay.stages <= 8);
}

// Beyond 16 tokens the N / 128 workgroups that each transform the same
// k-slice make the fused transform the larger cost, and one stand-alone
// transform (4-5 us) before the plain kernel is cheaper: from 33 tokens on
// every layer, from 17 on layers of at least 2^25 weights. Measured,
// graph-replayed, fused against transform-then-plain: 64 tokens, 4096 ->
// 14336 51.4 against 38.8 us, 14336 -> 4096 72.4 against 57.3, 4096 -> 4096
// 21.6 against about 18.4; 32 tokens, 4096 -> 4096 13.7 against about 15.
bool decode_fuses_rotation(const paro_rotation* r, int64_t M, int64_t N, int64_t d) {
  return decode_fuses_rotation(r) && (M <= 16 || (M <= 32 && N * d < (int64_t(1) << 25)));
}

hipError_t launch_w4_decode(const uint16_t* x, const uint8_t* qweight, const uint16_t* scales,
                            const uint8_t* zeros, const uint16_t* bias, uint16_t* y, int64_t M,
                            int64_t N, int64_t d, int group, const paro_rotation* r, void* ws,
                            hipStream_t stream) {
  if (M == 0) return hipSuccess;
  const int m = (int)M, n = (int)N, k = (int)d;
  const int gsh = group == 64 ? 0 : group == 128 ? 1 : 2;
  // 64-channel workgroups when 128-channel ones would not give two per CU;
  // but with the transform fused and more than 4 tokens, every workgroup's
  // transform of its k-slice (an LDS-bound chain of exchanges) sits on the
  // critical path, and 128-channel workgroups halve how often each segment is
  // transformed (4096 -> 4096 at M = 16: 10.9 -> 10.0 us measured), unless
  // they would leave half the CUs idle (4096 -> 1024 at M = 16: 8.74 -> 7.76
  // us with 64-channel workgroups)
  const int64_t wg128 = ((N + 127) / 128) * ((d / 128 + DK_SEGS - 1) / DK_SEGS);
  const bool small = M <= 4;
  const bool tj1 = wg128 < 384 && (small || r == nullptr || wg128 < 128);
  // full slices and aligned bases: vector scale / zero loads
  const bool szv = group == 128 && (d / 128) % DK_SEGS == 0 && ((uintptr_t)scales & 7) == 0 &&
                   ((uintptr_t)zeros & 3) == 0;
  // token blocks of 16 beyond 16 tokens
  const int tb = M <= 16 ? 1 : M <= 32 ? 2 : 4;
#define PARO_DECODE_PLAN(T_, TJ_, SZV_, TB_) \
  launch_plan<T_, TJ_, SZV_, TB_>(x, qweight, scales, zeros, bias, y, m, n, k, gsh, r, ws, stream)
  if (tb == 1) {
    if (szv) {
      if (tj1) return small ? PARO_DECODE_PLAN(4, 1, true, 1) : PARO_DECODE_PLAN(16, 1, true, 1);
      return small ? PARO_DECODE_PLAN(4, 2, true, 1) : PARO_DECODE_PLAN(16, 2, true, 1);
    }
    if (tj1) return small ? PARO_DECODE_PLAN(4, 1, false, 1) : PARO_DECODE_PLAN(16, 1, false, 1);
    return small ? PARO_DECODE_PLAN(4, 2, false, 1) : PARO_DECODE_PLAN(16, 2, false, 1);
  }
  if (tb == 2) {
    if (szv) return tj1 ? PARO_DECODE_PLAN(16, 1, true, 2) : PARO_DECODE_PLAN(16, 2, true, 2);
    return tj1 ? PARO_DECODE_PLAN(16, 1, false, 2) : PARO_DECODE_PLAN(16, 2, false, 2);
  }
  if (szv) return tj1 ? PARO_DECODE_PLAN(16, 1, true, 4) : PARO_DECODE_PLAN(16, 2, true, 4);
  return tj1 ? PARO_DECODE_PLAN(16, 1, false, 4) : PARO_DECODE_PLAN(16, 2, false, 4);
#undef PARO_DECODE_PLAN
}

}  // namespace paro
