// Per-wavefront rotation machinery shared by the stand-alone activation
// transform and the fused small-batch linear.
//
// Method: ParoQuant paper notes, section "关键设计" (K stages of independent
// Givens rotations on disjoint channel pairs inside each group, then the
// channel scaling) and "亮点与洞察" (all stages applied on chip in one pass).
//
// One wavefront owns one segment of 128 (PPL = 1) or 256 (PPL = 2) channels
// of a batch of T tokens. Virtual lane v = lane + 64 h (h < PPL) holds the two
// members of one pair in fp32 registers X (kept channel) and B (fetched
// channel). A stage is two fused multiply-adds per virtual lane and token (the
// factored form: per-pair cosine/sine factors are deferred into per-channel
// scales that the host folded into the coefficients and into the final
// scales), or the general 2x2 form for pairs whose factored form would lose
// range. Between consecutive pairings every virtual lane keeps X and fetches
// its next partner from another lane's B through a per-wavefront LDS tile that
// interleaves four tokens per 16-byte slot; the slots are planned on the host
// so that both the writes and the reads are free of bank conflicts.
//
// Schedule table image (built by the host plan): per segment and virtual lane
// NW words (the fields, padded to a multiple of four), four consecutive
// fields of a lane side by side: field f of virtual lane v is word
// ((f / 4) NV + v) 4 + f % 4, so a lane fetches four fields with one 16-byte
// load and a wavefront's such load is 1 KB contiguous. Field 0 is the load
// selector, 1 + 2 tau / 2 + 2 tau the LDS write / read byte offsets of
// exchange tau (tau = 0..K), then C words per stage, then the final scales of
// X and B, the store byte offset of the natural pair and the store selector.
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>

namespace paro {
namespace rot {

typedef float f4 __attribute__((ext_vector_type(4)));
typedef uint32_t u4 __attribute__((ext_vector_type(4)));
typedef _Float16 h2 __attribute__((ext_vector_type(2)));

__device__ __forceinline__ float as_f(uint32_t u) { return __builtin_bit_cast(float, u); }
__device__ __forceinline__ float half_lo(uint32_t v) {
  return (float)__builtin_bit_cast(_Float16, (uint16_t)(v & 0xffffu));
}
__device__ __forceinline__ float half_hi(uint32_t v) {
  return (float)__builtin_bit_cast(_Float16, (uint16_t)(v >> 16));
}

// PPL: pairs per lane. KMAX: compile-time stage count; with KEXACT the runtime
// K equals KMAX, otherwise K <= KMAX. FAST: factored form (else general 2x2).
template <int PPL, int KMAX, bool KEXACT, bool FAST>
struct Lane {
  static constexpr int NV = 64 * PPL;      // virtual lanes (pairs) per segment
  static constexpr int C = FAST ? 2 : 4;   // coefficients per stage
  static constexpr bool TREG = KMAX <= 8;  // whole schedule held in VGPRs
  static constexpr int KR = TREG ? KMAX : 0;

  const uint32_t* tb;  // this lane's first quad in the segment's table
  int K;
  uint32_t ldsel[PPL], stoff[PPL], stsel[PPL];
  float lamX[PPL], lamB[PPL];
  uint32_t wr[KR + 1][PPL], rd[KR + 1][PPL];
  float cf[KR > 0 ? KR : 1][C][PPL];

  static __host__ __device__ constexpr int nfields(int K) { return 1 + 2 * (K + 1) + C * K + 4; }
  static __host__ __device__ constexpr int fields(int K) { return (nfields(K) + 3) & ~3; }

  // field f of virtual lane lane + 64 h
  __device__ __forceinline__ uint32_t word(int f, int h) const {
    return tb[(size_t)(f >> 2) * (NV * 4) + 256 * h + (f & 3)];
  }

  __device__ __forceinline__ void load(const uint32_t* tab, int seg, int K_, int lane) {
    K = KEXACT ? KMAX : K_;
    tb = tab + (size_t)seg * fields(K) * NV + 4 * lane;
    if constexpr (KEXACT && TREG) {
      // the whole schedule with fields(K) / 4 16-byte loads per virtual lane
      constexpr int NQ = fields(KMAX) / 4;
      constexpr int ff = 3 + 2 * KMAX + C * KMAX;
#pragma unroll
      for (int h = 0; h < PPL; ++h) {
        uint32_t wv[4 * NQ];
#pragma unroll
        for (int q = 0; q < NQ; ++q) {
          const u4 v = *(const u4*)(tb + (size_t)q * (NV * 4) + 256 * h);
          wv[4 * q] = v.x;
          wv[4 * q + 1] = v.y;
          wv[4 * q + 2] = v.z;
          wv[4 * q + 3] = v.w;
        }
        ldsel[h] = wv[0];
#pragma unroll
        for (int tau = 0; tau <= KR; ++tau) {
          wr[tau][h] = wv[1 + 2 * tau];
          rd[tau][h] = wv[2 + 2 * tau];
        }
#pragma unroll
        for (int t = 0; t < KR; ++t)
#pragma unroll
          for (int e = 0; e < C; ++e) cf[t][e][h] = as_f(wv[3 + 2 * KMAX + C * t + e]);
        lamX[h] = as_f(wv[ff]);
        lamB[h] = as_f(wv[ff + 1]);
        stoff[h] = wv[ff + 2];
        stsel[h] = wv[ff + 3];
      }
    } else {
      const int ff = 3 + 2 * K + C * K;
#pragma unroll
      for (int h = 0; h < PPL; ++h) {
        ldsel[h] = word(0, h);
        lamX[h] = as_f(word(ff + 0, h));
        lamB[h] = as_f(word(ff + 1, h));
        stoff[h] = word(ff + 2, h);
        stsel[h] = word(ff + 3, h);
        if constexpr (TREG) {
#pragma unroll
          for (int tau = 0; tau <= KR; ++tau) {
            if (tau <= K) {
              wr[tau][h] = word(1 + 2 * tau, h);
              rd[tau][h] = word(2 + 2 * tau, h);
            }
          }
#pragma unroll
          for (int t = 0; t < KR; ++t) {
            if (t < K) {
#pragma unroll
              for (int e = 0; e < C; ++e) cf[t][e][h] = as_f(word(3 + 2 * K + C * t + e, h));
            }
          }
        }
      }
    }
  }

  __device__ __forceinline__ uint32_t wr_off(int tau, int h) const {
    if constexpr (TREG) return wr[tau][h];
    else return word(1 + 2 * tau, h);
  }
  __device__ __forceinline__ uint32_t rd_off(int tau, int h) const {
    if constexpr (TREG) return rd[tau][h];
    else return word(2 + 2 * tau, h);
  }
  __device__ __forceinline__ float coef(int t, int e, int h) const {
    if constexpr (TREG) return cf[t][e][h];
    else return as_f(word(3 + 2 * K + C * t + e, h));
  }

  // Raw fp16 pair word of the natural pair (v) -> fp32 (kept, fetched).
  __device__ __forceinline__ void unpack(uint32_t raw, int h, float& X, float& B) const {
    const uint32_t v = __builtin_amdgcn_perm(raw, raw, ldsel[h]);
    X = half_lo(v);
    B = half_hi(v);
  }

  // Final scales and one fp16 rounding each; the returned word is the natural
  // pair (even channel in the low half) that belongs at byte offset stoff[h].
  __device__ __forceinline__ uint32_t pack(float X, float B, int h) const {
    const h2 pk = {(_Float16)(X * lamX[h]), (_Float16)(B * lamB[h])};
    const uint32_t u = __builtin_bit_cast(uint32_t, pk);
    return __builtin_amdgcn_perm(u, u, stsel[h]);
  }

  // All K stages and K + 1 exchanges on a batch of T tokens (T % 4 == 0);
  // lds is this wavefront's exchange tile of T / 4 * NV 16-byte slots.
  template <int T>
  __device__ __forceinline__ void run(float (&X)[PPL][T], float (&B)[PPL][T], char* lds) const {
    constexpr int NQ = T / 4;
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
    if constexpr (KMAX > 0) {
      exchange(0);
#pragma unroll
      for (int t = 0; t < KMAX; ++t) {
        if (KEXACT || t < K) {
#pragma unroll
          for (int h = 0; h < PPL; ++h) {
#pragma unroll
            for (int i = 0; i < T; ++i) {
              const float a = X[h][i], b = B[h][i];
              if constexpr (FAST) {
                B[h][i] = __builtin_fmaf(coef(t, 1, h), a, b);
                X[h][i] = __builtin_fmaf(coef(t, 0, h), b, a);
              } else {
                B[h][i] = __builtin_fmaf(coef(t, 2, h), a, coef(t, 3, h) * b);
                X[h][i] = __builtin_fmaf(coef(t, 1, h), b, coef(t, 0, h) * a);
              }
            }
          }
          exchange(t + 1);
        }
      }
    }
  }
};

}  // namespace rot
}  // namespace paro
