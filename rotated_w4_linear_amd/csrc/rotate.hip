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
// and token, the loads one batch ahead of the arithmetic; the schedule tables
// are read once per wavefront. Each load instruction covers one contiguous
// 256-byte piece of a row. The last exchange leaves every lane some natural
// pair of its segment, which it stores in place: for 128-channel segments
// one store instruction still covers 256 contiguous bytes. For 256-channel
// segments a lane's two pairs may lie anywhere in 512 bytes, and stores
// spread that way cost 15% at K = 1; there one more exchange, of the packed
// fp16 output words, first gives every virtual lane the natural pair of its
// own index (6-14% faster over the sweep; for 128-channel segments that
// exchange costs more than it saves: prefill MLP 36.5 -> 38.3 us).
#include <cstring>

#include "paro_internal.h"
#include "rotate_core.h"

namespace paro {
namespace {

using rot::f4;

// Word 3 of a gfx9 buffer resource: 32-bit data format, no swizzle.
constexpr int kRsrcWord3 = 0x00020000;

// PPL, KMAX, KEXACT, FAST: see rot::Lane. T: tokens per batch (a multiple of
// 4: one LDS quad holds 4 tokens). A wavefront owns segment gw % segs of the
// token chunk gw / segs (tpw tokens).
// perm: the store permutation of the plan ([segs][NV][2] words after the
// segments' schedules), used by 256-channel segments.
template <int PPL, int KMAX, bool KEXACT, bool FAST, int T>
__global__ __launch_bounds__(256) void rotate_kernel(const uint16_t* x, uint16_t* y,
                                                     const uint32_t* __restrict__ tab,
                                                     const uint32_t* __restrict__ perm, int M,
                                                     int64_t row, int segs, int K, int tpw) {
  using L = rot::Lane<PPL, KMAX, KEXACT, FAST>;
  constexpr int NV = L::NV;
  constexpr int SEG = 2 * NV;  // channels per segment
  __shared__ f4 lds_all[4][T / 4 * NV];

  const int lane = threadIdx.x & 63;
  // wave-uniform: keeps the token and address arithmetic in scalar registers
  const int wid = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int64_t gw = (int64_t)blockIdx.x * 4 + wid;
  const int seg = (int)(gw % segs);
  const int64_t tok0l = (gw / segs) * (int64_t)tpw;
  if (tok0l >= M) return;
  const int tok0 = (int)tok0l;
  const int tok1 = (tok0 + tpw < M) ? tok0 + tpw : M;
  char* lds = (char*)&lds_all[wid][0];

  L sch;
  sch.load(tab, seg, K, lane);
  // the store permutation's LDS write and read offsets of each virtual lane
  // (without stages every lane still holds the natural pair it loaded)
  constexpr bool PERM = PPL == 2 && KMAX > 0;
  uint32_t pw[PPL], pr[PPL];
  if constexpr (PERM) {
#pragma unroll
    for (int h = 0; h < PPL; ++h) {
      const uint2 pv = *(const uint2*)(perm + ((size_t)seg * NV + 64 * h + lane) * 2);
      pw[h] = pv.x;
      pr[h] = pv.y;
    }
  }

  const uint16_t* xseg = x + (int64_t)seg * SEG;
  uint16_t* yseg = y + (int64_t)seg * SEG;

  // Raw fp16 pairs of one batch. The next batch is loaded while the current
  // one is rotated so that a wavefront always has HBM reads in flight; loads
  // past the end of the chunk re-read its last token (in bounds, cached).
  // Buffer instructions take the token row as a scalar offset from a
  // wave-uniform base, so addressing costs no vector instructions.
  const uint32_t rowb = (uint32_t)row * 2u;  // bytes per token row
  typedef uint32_t Raw[PPL][T];
  Raw raw;
  auto load = [&](int t0, Raw& nxt) {
    const int tl = (t0 < tok1) ? t0 : tok1 - 1;
    const __amdgpu_buffer_rsrc_t rs =
        __builtin_amdgcn_make_buffer_rsrc((void*)(xseg + (int64_t)tl * row), (short)0, 0x7fffffff, kRsrcWord3);
#pragma unroll
    for (int i = 0; i < T; ++i) {
      const int di = (tl + i < tok1) ? i : tok1 - 1 - tl;
#pragma unroll
      for (int h = 0; h < PPL; ++h)
        nxt[h][i] = __builtin_amdgcn_raw_buffer_load_b32(rs, 4 * (64 * h + lane), di * rowb, 0);
    }
  };

  load(tok0, raw);
  for (int t0 = tok0; t0 < tok1; t0 += T) {
    float X[PPL][T], B[PPL][T];
#pragma unroll
    for (int i = 0; i < T; ++i)
#pragma unroll
      for (int h = 0; h < PPL; ++h) sch.unpack(raw[h][i], h, X[h][i], B[h][i]);
    load(t0 + T, raw);
    sch.template run<T>(X, B, lds);
    uint32_t pk[PPL][T];
#pragma unroll
    for (int i = 0; i < T; ++i)
#pragma unroll
      for (int h = 0; h < PPL; ++h) pk[h][i] = sch.pack(X[h][i], B[h][i], h);
    if constexpr (PERM) {
      // natural pair w to virtual lane w, four tokens per 16-byte slot as in
      // the exchanges
#pragma unroll
      for (int q = 0; q < T / 4; ++q) {
#pragma unroll
        for (int h = 0; h < PPL; ++h) {
          const rot::u4 v = {pk[h][4 * q], pk[h][4 * q + 1], pk[h][4 * q + 2], pk[h][4 * q + 3]};
          *(rot::u4*)(lds + q * NV * 16 + pw[h]) = v;
        }
      }
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
#pragma unroll
      for (int q = 0; q < T / 4; ++q) {
#pragma unroll
        for (int h = 0; h < PPL; ++h) {
          const rot::u4 v = *(const rot::u4*)(lds + q * NV * 16 + pr[h]);
          pk[h][4 * q] = v.x;
          pk[h][4 * q + 1] = v.y;
          pk[h][4 * q + 2] = v.z;
          pk[h][4 * q + 3] = v.w;
        }
      }
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    }
    const __amdgpu_buffer_rsrc_t rs =
        __builtin_amdgcn_make_buffer_rsrc((void*)(yseg + (int64_t)t0 * row), (short)0, 0x7fffffff, kRsrcWord3);
#pragma unroll
    for (int i = 0; i < T; ++i) {
      if (t0 + i < tok1) {
#pragma unroll
        for (int h = 0; h < PPL; ++h)
          __builtin_amdgcn_raw_buffer_store_b32(pk[h][i], rs, PERM ? 4 * (64 * h + lane) : sch.stoff[h],
                                                i * rowb, 0);
      }
    }
  }
}

// Tokens per wavefront, a multiple of the batch size T: about target_waves
// wavefronts, or (cap) at most target_waves of them, so that a launch sized
// to one round of resident wavefronts leaves no few stragglers to a second
// round (8192 x 5120, 256-channel segments, K = 8: 4100 wavefronts of 40
// tokens took 44.9 us, against 43.0 with 8200 of 20 tokens and 42.1 with
// 3740 of 44).
inline int64_t tokens_per_wave(int64_t M, int segs, int T, int64_t target_waves, bool cap) {
  int64_t per;
  if (cap) {
    const int64_t chunks = target_waves / segs > 0 ? target_waves / segs : 1;
    per = (M + chunks - 1) / chunks;
  } else {
    per = (M * segs + target_waves - 1) / target_waves;
  }
  int64_t tpw = ((per + T - 1) / T) * T;
  return tpw < T ? T : tpw;
}

template <int PPL, int KMAX, bool KEXACT, bool FAST, int T>
hipError_t launch_t(const paro_rotation* r, const uint16_t* x, uint16_t* y, int64_t M,
                    hipStream_t stream, int64_t target_waves, bool cap) {
  const int segs = (int)(r->d / r->lay.seg_ch);
  const int64_t tpw = tokens_per_wave(M, segs, T, target_waves, cap);
  const int64_t chunks = (M + tpw - 1) / tpw;
  const int64_t waves = chunks * segs;
  const int64_t blocks = (waves + 3) / 4;
  hipLaunchKernelGGL((rotate_kernel<PPL, KMAX, KEXACT, FAST, T>), dim3((unsigned)blocks),
                     dim3(256), 0, stream, x, y, r->d_table, r->d_table + rot_perm_base(segs, r->lay),
                     (int)M, r->d, segs, r->lay.stages, (int)tpw);
  return hipGetLastError();
}

// About 8192 wavefronts per launch (32 per CU) measured best on MI355X for
// the 8192-token workloads. 256-channel segments from three stages on hold
// 79 (K = 4) to 110 (K = 8) VGPRs, six to four wavefronts per SIMD; there at
// most 4096 wavefronts of more tokens each (8192 x 4096, K = 8: 34.4 -> 33.2
// us; the other widths and K = 4 within 0.5%). With fewer stages more
// wavefronts stay ahead (K = 1, d = 4096: 27.1 against 28.8 us with 4096).
constexpr int64_t kTargetWaves = 8192;
constexpr int64_t kMaxWaves256 = 4096;

template <int PPL>
hipError_t launch_ppl(const paro_rotation* r, const uint16_t* x, uint16_t* y, int64_t M,
                      hipStream_t stream) {
  constexpr int T = PPL == 1 ? 8 : 4;
  const int K = r->lay.stages;  // stages the schedule executes
  const bool cap = PPL == 2 && K >= 3;
  const int64_t tw = cap ? kMaxWaves256 : kTargetWaves;
  if (K == 0) return launch_t<PPL, 0, true, true, T>(r, x, y, M, stream, tw, cap);
  if (r->lay.fast) {
    switch (K) {
      case 1: return launch_t<PPL, 1, true, true, T>(r, x, y, M, stream, tw, cap);
      case 2: return launch_t<PPL, 2, true, true, T>(r, x, y, M, stream, tw, cap);
      case 3: return launch_t<PPL, 3, true, true, T>(r, x, y, M, stream, tw, cap);
      case 4: return launch_t<PPL, 4, true, true, T>(r, x, y, M, stream, tw, cap);
      case 5: return launch_t<PPL, 5, true, true, T>(r, x, y, M, stream, tw, cap);
      case 6: return launch_t<PPL, 6, true, true, T>(r, x, y, M, stream, tw, cap);
      case 7: return launch_t<PPL, 7, true, true, T>(r, x, y, M, stream, tw, cap);
      case 8: return launch_t<PPL, 8, true, true, T>(r, x, y, M, stream, tw, cap);
      default: break;
    }
    if (K <= 16) return launch_t<PPL, 16, false, true, T>(r, x, y, M, stream, tw, cap);
    return launch_t<PPL, 32, false, true, T>(r, x, y, M, stream, tw, cap);
  }
  if (K <= 8) return launch_t<PPL, 8, false, false, T>(r, x, y, M, stream, tw, cap);
  if (K <= 16) return launch_t<PPL, 16, false, false, T>(r, x, y, M, stream, tw, cap);
  return launch_t<PPL, 32, false, false, T>(r, x, y, M, stream, tw, cap);
}

}  // namespace

hipError_t launch_rotate(const paro_rotation* r, const uint16_t* x, uint16_t* y, int64_t M,
                         hipStream_t stream) {
  if (M == 0) return hipSuccess;
  return r->lay.ppl == 1 ? launch_ppl<1>(r, x, y, M, stream) : launch_ppl<2>(r, x, y, M, stream);
}

}  // namespace paro
