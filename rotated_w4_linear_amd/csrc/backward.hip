// gfx950 kernels for the gradients of the transform, the step that learns the
// angles and channel scales (paper notes, "损失函数 / 训练策略": both are fitted
// by minimising the layer-wise output loss, which needs them).
//
// For one row r (a token of X, or a row of W in the [N][d] layout) the
// transform is v_0 = r / alpha (activations, X' = X T^-1) or r * alpha
// (weights, T W), then stage t of K applies the pair update
// (v_i, v_j) <- (c v_i - s v_j, s v_i + c v_j) (CSDN article, section 2.2).
// Given g = dL/d(output) per row:
//   * walking stage t back, the pair's gradient becomes
//     (c g_i + s g_j, -s g_i + c g_j) and the angle collects
//     g'_j v'_i - g'_i v'_j from the stage's outputs v' and their gradient g';
//   * the stage's inputs are recovered from its outputs by the inverse (the
//     transpose), so the forward values of the stages are never stored;
//   * at the end dr = g_0 / alpha (or g_0 * alpha) and alpha collects
//     -g_0 r / alpha^2 (or g_0 r).
//
// Work split: a wavefront (one per workgroup) owns one segment of 128
// channels (256 for groups of 256) and one chunk of rows, which it walks in
// batches of BT rows (batch_rows). Lane l owns the segment's pair slots
// l * PPL .. + PPL - 1 of every stage (the pairs of a stage lie inside the
// segment, so every exchange stays inside the wavefront) and the natural
// channels 2 (l + 64 q) + {0, 1}. A batch sits in LDS channel-major in planes
// of four rows: the four rows of channel c in 16-byte slot c of a plane,
// values and gradients in two arrays. The host places the pairs on the lanes
// so that every 16 consecutive lanes touch channels distinct modulo 16 and
// every 8 distinct modulo 8, which makes the 16-byte accesses free of bank
// conflicts. LDS accesses of one wavefront complete in order, so a stage
// reads what the previous stage wrote without a barrier. Angle sums stay in
// LDS per wavefront, scale sums in registers; each chunk writes its partial
// sums to scratch, and a second kernel adds the chunks in chunk order, so the
// result does not depend on scheduling.
#include <algorithm>

#include "paro_internal.h"

#pragma clang fp contract(off)

namespace paro {
namespace {

// Rows per batch (a multiple of 4) for segments of 128 * PPL channels: eight
// rows for 128-channel segments (measured 7% faster than four at 8192 x 4096,
// K = 8: the table entries, addresses and angle sums of a stage serve twice
// the rows), four for 256-channel segments (eight measured no faster there).
__host__ __device__ constexpr int batch_rows(int ppl) { return ppl == 1 ? 8 : 4; }
// Wavefronts per launch (measured at 8192 x 4096, K = 8, over 2048..6144):
// 4096 for 128-channel segments, 3072 for 256-channel segments (170 against
// 192 us at 4096).
constexpr int64_t target_waves(int seg_ch) { return seg_ch == 128 ? 4096 : 3072; }

typedef float f4v __attribute__((ext_vector_type(4)));

__device__ __forceinline__ float h_lo(uint32_t v) {
  return (float)__builtin_bit_cast(_Float16, (uint16_t)(v & 0xffffu));
}
__device__ __forceinline__ float h_hi(uint32_t v) {
  return (float)__builtin_bit_cast(_Float16, (uint16_t)(v >> 16));
}

// BT floats of one channel: BT / 4 16-byte LDS accesses, one per plane of
// four rows (planes qs floats apart)
template <int BT>
__device__ __forceinline__ void lds_get(const float* p, int qs, float (&o)[BT]) {
#pragma unroll
  for (int k = 0; k < BT / 4; ++k) {
    const f4v a = *(const f4v*)(p + qs * k);
#pragma unroll
    for (int r = 0; r < 4; ++r) o[4 * k + r] = a[r];
  }
}
template <int BT>
__device__ __forceinline__ void lds_put(float* p, int qs, const float (&o)[BT]) {
#pragma unroll
  for (int k = 0; k < BT / 4; ++k) *(f4v*)(p + qs * k) = f4v{o[4 * k], o[4 * k + 1], o[4 * k + 2], o[4 * k + 3]};
}

template <int PPL>
__global__ __launch_bounds__(64) void rotate_backward_kernel(
    const uint16_t* __restrict__ x, const float* gy, float* gx,  // gx may be gy
    const uint4* __restrict__ tab, const float* __restrict__ alpha, int M, int d, int K,
    int segs, int chunk, int nchunks, int weight_side, float* __restrict__ part_th,
    float* __restrict__ part_al) {
  constexpr int S = 128 * PPL;  // channels per segment
  constexpr int NP = S / 2;     // pair slots per stage
  extern __shared__ float lds[];
  constexpr int BT = batch_rows(PPL);
  constexpr int QS = 4 * S;     // floats per plane of four rows
  float* v = lds;               // [BT / 4][S][4] values
  float* g = v + S * BT;        // [BT / 4][S][4] gradients
  float* th = g + S * BT;       // [K][NP] angle sums of this chunk
  const int lane = threadIdx.x;
  const int seg = blockIdx.x % segs, ch = blockIdx.x / segs;
  if (ch >= nchunks) return;
  const int m0 = ch * chunk, m1 = min(M, m0 + chunk);
  for (int e = lane; e < K * NP; e += 64) th[e] = 0.f;

  float sc[PPL][2], dacc[PPL][2];
#pragma unroll
  for (int q = 0; q < PPL; ++q)
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const float a = alpha[(size_t)seg * S + 2 * (lane + 64 * q) + h];
      sc[q][h] = weight_side ? a : 1.0f / a;
      dacc[q][h] = 0.f;
    }
  const uint4* tseg = tab + (size_t)seg * K * NP;

  for (int mb = m0; mb < m1; mb += BT) {
    const int nt = min(BT, m1 - mb);
    // ---- the batch's rows of the segment (rows past the chunk repeat its
    // last row with a zero gradient, so they add nothing)
    uint32_t xr[BT][PPL];
    float gr[BT][PPL][2];
#pragma unroll
    for (int i = 0; i < BT; ++i) {
      const size_t row = (size_t)(mb + min(i, nt - 1)) * (size_t)d + (size_t)seg * S;
#pragma unroll
      for (int q = 0; q < PPL; ++q) {
        const int c0 = 2 * (lane + 64 * q);
        xr[i][q] = *(const uint32_t*)(x + row + c0);
        const float2 gg = *(const float2*)(gy + row + c0);
        gr[i][q][0] = i < nt ? gg.x : 0.f;
        gr[i][q][1] = i < nt ? gg.y : 0.f;
      }
    }
#pragma unroll
    for (int q = 0; q < PPL; ++q)
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const int c = 2 * (lane + 64 * q) + h;
        float vv[BT], gg[BT];
#pragma unroll
        for (int i = 0; i < BT; ++i) {
          vv[i] = (h ? h_hi(xr[i][q]) : h_lo(xr[i][q])) * sc[q][h];
          gg[i] = gr[i][q][h];
        }
        lds_put(v + c * 4, QS, vv);
        lds_put(g + c * 4, QS, gg);
      }

    // ---- forward: the stages' outputs, then backward: angle sums, gradients
    // and inputs of each stage. The table entries of two consecutive stages
    // are held in two register sets, each reloaded right after its use, so a
    // stage's entries are requested two stages ahead (requests past the end
    // are clamped to the last stage and unused). K == 0: there is no table,
    // and no entry may be read.
    auto fetch = [&](uint4 (&e)[PPL], int t) {
#pragma unroll
      for (int q = 0; q < PPL; ++q) e[q] = tseg[(size_t)t * NP + lane * PPL + q];
    };
    auto fwd_stage = [&](const uint4 (&en)[PPL]) {
#pragma unroll
      for (int q = 0; q < PPL; ++q) {
        const uint4 e = en[q];
        const int i = (int)(e.x & 0xffffu), j = (int)(e.x >> 16);
        const float c = __builtin_bit_cast(float, e.y), s = __builtin_bit_cast(float, e.z);
        float a[BT], b[BT], na[BT], nb[BT];
        lds_get(v + i * 4, QS, a);
        lds_get(v + j * 4, QS, b);
#pragma unroll
        for (int r = 0; r < BT; ++r) {
          na[r] = __builtin_fmaf(c, a[r], -(s * b[r]));
          nb[r] = __builtin_fmaf(s, a[r], c * b[r]);
        }
        lds_put(v + i * 4, QS, na);
        lds_put(v + j * 4, QS, nb);
      }
    };
    auto bwd_stage = [&](int t, const uint4 (&en)[PPL]) {
#pragma unroll
      for (int q = 0; q < PPL; ++q) {
        const uint4 e = en[q];
        const int i = (int)(e.x & 0xffffu), j = (int)(e.x >> 16);
        const float c = __builtin_bit_cast(float, e.y), s = __builtin_bit_cast(float, e.z);
        float vi[BT], vj[BT], gi[BT], gj[BT], o1[BT], o2[BT];
        lds_get(v + i * 4, QS, vi);
        lds_get(v + j * 4, QS, vj);
        lds_get(g + i * 4, QS, gi);
        lds_get(g + j * 4, QS, gj);
        float acc = th[t * NP + lane * PPL + q];
#pragma unroll
        for (int r = 0; r < BT; ++r) acc = __builtin_fmaf(-gi[r], vj[r], __builtin_fmaf(gj[r], vi[r], acc));
        th[t * NP + lane * PPL + q] = acc;
#pragma unroll
        for (int r = 0; r < BT; ++r) {
          o1[r] = __builtin_fmaf(c, gi[r], s * gj[r]);
          o2[r] = __builtin_fmaf(c, gj[r], -(s * gi[r]));
        }
        lds_put(g + i * 4, QS, o1);
        lds_put(g + j * 4, QS, o2);
#pragma unroll
        for (int r = 0; r < BT; ++r) {
          o1[r] = __builtin_fmaf(c, vi[r], s * vj[r]);
          o2[r] = __builtin_fmaf(c, vj[r], -(s * vi[r]));
        }
        lds_put(v + i * 4, QS, o1);
        lds_put(v + j * 4, QS, o2);
      }
    };
    if (K > 0) {
      // stage pairs without a branch inside, so that the loads of the two
      // sets stay in flight across the loop's back edge; an odd K ends with
      // one more stage
      uint4 ea[PPL], eb[PPL];
      fetch(ea, 0);
      fetch(eb, min(1, K - 1));
      int t = 0;
#pragma unroll 1
      for (; t + 1 < K; t += 2) {
        fwd_stage(ea);
        fetch(ea, min(t + 2, K - 1));
        fwd_stage(eb);
        fetch(eb, min(t + 3, K - 1));
      }
      if (t < K) fwd_stage(ea);
      fetch(ea, K - 1);
      fetch(eb, max(K - 2, 0));
      t = K - 1;
#pragma unroll 1
      for (; t >= 1; t -= 2) {
        bwd_stage(t, ea);
        fetch(ea, max(t - 2, 0));
        bwd_stage(t - 1, eb);
        fetch(eb, max(t - 3, 0));
      }
      if (t == 0) bwd_stage(0, ea);
    }

    // ---- input gradients and the scales' sums
#pragma unroll
    for (int q = 0; q < PPL; ++q) {
      const int c0 = 2 * (lane + 64 * q);
      float g0[BT], g1[BT];
      lds_get(g + c0 * 4, QS, g0);
      lds_get(g + (c0 + 1) * 4, QS, g1);
#pragma unroll
      for (int i = 0; i < BT; ++i) {
        if (i < nt) {
          dacc[q][0] += g0[i] * h_lo(xr[i][q]);
          dacc[q][1] += g1[i] * h_hi(xr[i][q]);
          if (gx) {
            const size_t row = (size_t)(mb + i) * (size_t)d + (size_t)seg * S;
            *(float2*)(gx + row + c0) = float2{g0[i] * sc[q][0], g1[i] * sc[q][1]};
          }
        }
      }
    }
  }

  // ---- this chunk's partial sums
  float* pt = part_th + ((size_t)ch * segs + seg) * (size_t)K * NP;
  for (int e = lane; e < K * NP; e += 64) pt[e] = th[e];
#pragma unroll
  for (int q = 0; q < PPL; ++q)
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const size_t c = (size_t)seg * S + 2 * (lane + 64 * q) + h;
      const float a = alpha[c];
      part_al[(size_t)ch * d + c] = weight_side ? dacc[q][h] : -dacc[q][h] / (a * a);
    }
}

// Sum of n partial sums at stride `stride`, in order, eight loads in flight.
__device__ __forceinline__ float sum_chunks(const float* p, size_t stride, int n) {
  float acc = 0.f;
  for (int c = 0; c < n; c += 8) {
    float v[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) v[u] = c + u < n ? p[(size_t)(c + u) * stride] : 0.f;
#pragma unroll
    for (int u = 0; u < 8; ++u)
      if (c + u < n) acc += v[u];
  }
  return acc;
}

// dtheta[flat pair index] and dalpha[channel]: the chunks' partial sums added
// in chunk order
__global__ __launch_bounds__(64) void rotate_backward_reduce(
    const float* __restrict__ part_th, const float* __restrict__ part_al,
    const uint4* __restrict__ tab, int nth, int d, int nchunks, float* __restrict__ dtheta,
    float* __restrict__ dalpha) {
  const int e = blockIdx.x * 64 + threadIdx.x;
  if (e < nth) {
    const float acc = sum_chunks(part_th + e, (size_t)nth, nchunks);
    const uint32_t w = tab[e].w;  // bit 31: the pair is stored the other way round
    dtheta[w & 0x7fffffffu] = (w >> 31) ? -acc : acc;
  } else if (e < nth + d) {
    const int k = e - nth;
    dalpha[k] = sum_chunks(part_al + k, (size_t)d, nchunks);
  }
}

struct ChunkPlan {
  int segs, chunk, nchunks;
};

ChunkPlan chunk_plan(const paro_rotation* r, int64_t M) {
  const int S = r->lay.seg_ch;
  const int BT = batch_rows(S / 128);
  ChunkPlan p;
  p.segs = (int)(r->d / S);
  if (M <= 0) {
    p.chunk = BT;
    p.nchunks = 0;
    return p;
  }
  // about target_waves(S) wavefronts, chunks a multiple of BT rows
  const int64_t batches = (M + BT - 1) / BT;
  int64_t want = (target_waves(S) + p.segs - 1) / p.segs;
  want = std::max<int64_t>(1, std::min(want, batches));
  const int64_t per = (batches + want - 1) / want;
  p.chunk = (int)(per * BT);
  p.nchunks = (int)((M + p.chunk - 1) / p.chunk);
  return p;
}

}  // namespace

size_t rotate_backward_scratch_bytes(const paro_rotation* r, int64_t M) {
  const ChunkPlan p = chunk_plan(r, M);
  return (size_t)p.nchunks * ((size_t)r->K * (size_t)(r->d / 2) + (size_t)r->d) * 4;
}

hipError_t launch_rotate_backward(const paro_rotation* r, int weight_side, const uint16_t* x,
                                  const float* gy, float* gx, float* dtheta, float* dalpha,
                                  int64_t M, void* part, hipStream_t stream) {
  const ChunkPlan p = chunk_plan(r, M);
  const int S = r->lay.seg_ch, K = r->K, d = (int)r->d;
  const int nth = K * (d / 2);
  float* part_th = (float*)part;
  float* part_al = part_th + (size_t)p.nchunks * nth;
  if (p.nchunks > 0) {
    const size_t lds = ((size_t)2 * S * batch_rows(S / 128) + (size_t)K * (S / 2)) * sizeof(float);
    const unsigned blocks = (unsigned)((int64_t)p.segs * p.nchunks);
    if (S == 128)
      hipLaunchKernelGGL(rotate_backward_kernel<1>, dim3(blocks), dim3(64), lds, stream, x, gy, gx,
                         (const uint4*)r->d_bw, r->d_alpha, (int)M, d, K, p.segs, p.chunk,
                         p.nchunks, weight_side, part_th, part_al);
    else
      hipLaunchKernelGGL(rotate_backward_kernel<2>, dim3(blocks), dim3(64), lds, stream, x, gy, gx,
                         (const uint4*)r->d_bw, r->d_alpha, (int)M, d, K, p.segs, p.chunk,
                         p.nchunks, weight_side, part_th, part_al);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  const unsigned rb = (unsigned)((nth + d + 63) / 64);
  hipLaunchKernelGGL(rotate_backward_reduce, dim3(rb), dim3(64), 0, stream, part_th, part_al,
                     (const uint4*)r->d_bw, nth, d, p.nchunks, dtheta, dalpha);
  return hipGetLastError();
}

}  // namespace paro
