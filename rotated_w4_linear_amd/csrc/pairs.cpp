// Host-side choice of the channel pairs of the K independent-rotation stages
// (the inputs paro_rotation_create takes), and sparsification of a plan to
// its strongest rotations. The pages name three strategies:
//  * random pairs with de-duplication (paper notes, "局限与展望": the authors'
//    pair selection is random plus de-duplication);
//  * pairs of channels whose values differ strongly (CSDN article, section
//    2.2: pairs with a large numeric difference are preferred, for saliency);
//  * keeping only the top 10% of the channel pairs (paper notes, "核心观察":
//    a sparse rotation with the top-10% pairs matches the full one).
// Their exact rules are not on the pages; the readings implemented here are
// stated at each function. Random numbers come from SplitMix64 (Steele, Lea
// and Flood, "Fast splittable pseudorandom number generators", 2014), a
// counter-based generator whose definition is public, so that a reference
// implementation elsewhere reproduces every draw.
#include <algorithm>
#include <cmath>
#include <cstring>
#include <numeric>
#include <string>
#include <vector>

#include "paro_internal.h"

namespace paro {
namespace {

// draws of a whole stage's pairing before paro_pairs_random gives up
constexpr int kPairAttempts = 4096;

// SplitMix64: the state advances by the golden-ratio increment and each
// output is the state passed through two xor-shift-multiply rounds.
struct SplitMix64 {
  uint64_t x;
  uint64_t next() {
    uint64_t z = (x += 0x9E3779B97F4A7C15ull);
    z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
    z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
    return z ^ (z >> 31);
  }
};

bool group_ok(int64_t d, int32_t group, int32_t K, const char* fn, int kmax) {
  if (group < 2 || group % 2 || d <= 0 || d % group || d > (int64_t(1) << 24)) {
    set_error(std::string(fn) + ": group must be even and divide d (d <= 2^24)");
    return false;
  }
  if (K < 0 || K > kmax) {
    set_error(std::string(fn) + ": K out of range for this group size");
    return false;
  }
  return true;
}

}  // namespace
}  // namespace paro

using namespace paro;

extern "C" {

/* Random pairs, no pair repeated across the stages of a group (reading in
 * include/paro.h). */
int paro_pairs_random(int64_t d, int32_t group, int32_t K, uint64_t seed, int32_t* pairs) {
  if (!pairs && K > 0) {
    set_error("paro_pairs_random: pairs is NULL");
    return PARO_ERR_NULL;
  }
  if (!group_ok(d, group, K, "paro_pairs_random", group - 1)) return PARO_ERR_SHAPE;
  SplitMix64 rng{seed};
  const int G = group, H = group / 2;
  std::vector<uint8_t> used((size_t)G * G);
  std::vector<int> perm(G);
  for (int64_t g = 0; g < d / G; ++g) {
    std::fill(used.begin(), used.end(), 0);
    for (int t = 0; t < K; ++t) {
      bool done = false;
      for (int attempt = 0; attempt < kPairAttempts && !done; ++attempt) {
        std::iota(perm.begin(), perm.end(), 0);
        for (int i = G - 1; i >= 1; --i) {  // Fisher-Yates
          const int j = (int)(rng.next() % (uint64_t)(i + 1));
          std::swap(perm[i], perm[j]);
        }
        done = true;
        for (int i = 0; i < G && done; i += 2) {
          const int a = perm[i];
          int k = i + 1;
          while (k < G && used[(size_t)a * G + perm[k]]) ++k;
          if (k == G) {
            done = false;  // every remaining partner of a was used: draw again
          } else {
            std::swap(perm[i + 1], perm[k]);
          }
        }
      }
      if (!done) {
        set_error("paro_pairs_random: no pairing without repeated pairs found");
        return PARO_ERR_VALUE;
      }
      for (int p = 0; p < H; ++p) {
        const int a = perm[2 * p], b = perm[2 * p + 1];
        used[(size_t)a * G + b] = used[(size_t)b * G + a] = 1;
        int32_t* dst = pairs + ((size_t)t * (size_t)(d / 2) + (size_t)g * H + p) * 2;
        dst[0] = (int32_t)(g * G + a);
        dst[1] = (int32_t)(g * G + b);
      }
    }
  }
  return PARO_OK;
}

/* Pairs of strongly differing channels (reading in include/paro.h). */
int paro_pairs_by_gap(int64_t d, int32_t group, int32_t K, const float* score, int32_t* pairs) {
  if (!score || (!pairs && K > 0)) {
    set_error("paro_pairs_by_gap: NULL argument");
    return PARO_ERR_NULL;
  }
  if (!group_ok(d, group, K, "paro_pairs_by_gap", group / 2)) return PARO_ERR_SHAPE;
  for (int64_t k = 0; k < d; ++k) {
    if (!std::isfinite(score[k])) {
      set_error("paro_pairs_by_gap: non-finite score");
      return PARO_ERR_VALUE;
    }
  }
  const int G = group, H = group / 2;
  std::vector<int> rank(G);
  for (int64_t g = 0; g < d / G; ++g) {
    const float* s = score + g * G;
    std::iota(rank.begin(), rank.end(), 0);
    std::stable_sort(rank.begin(), rank.end(), [&](int a, int b) { return s[a] > s[b]; });
    for (int t = 0; t < K; ++t) {
      for (int i = 0; i < H; ++i) {
        const int hi = rank[i];                        // i-th largest
        const int lo = rank[G - 1 - (i + t) % H];      // ((i + t) mod H)-th smallest
        int32_t* dst = pairs + ((size_t)t * (size_t)(d / 2) + (size_t)g * H + i) * 2;
        dst[0] = (int32_t)(g * G + hi);
        dst[1] = (int32_t)(g * G + lo);
      }
    }
  }
  return PARO_OK;
}

/* Keep the n_keep strongest rotations of a plan (reading in include/paro.h). */
int paro_sparsify_angles(int64_t d, int32_t K, const float* theta, int64_t n_keep, float* theta_out) {
  const int64_t P = (int64_t)K * (d / 2);
  if ((P > 0 && (!theta || !theta_out))) {
    set_error("paro_sparsify_angles: NULL argument");
    return PARO_ERR_NULL;
  }
  if (d <= 0 || d % 2 || K < 0 || n_keep < 0 || n_keep > P) {
    set_error("paro_sparsify_angles: sizes (d even, K >= 0, 0 <= n_keep <= K d / 2)");
    return PARO_ERR_SHAPE;
  }
  for (int64_t i = 0; i < P; ++i) {
    if (!std::isfinite(theta[i])) {
      set_error("paro_sparsify_angles: non-finite angle");
      return PARO_ERR_VALUE;
    }
  }
  std::vector<int64_t> idx(P);
  std::iota(idx.begin(), idx.end(), 0);
  std::stable_sort(idx.begin(), idx.end(),
                   [&](int64_t a, int64_t b) { return std::fabs(theta[a]) > std::fabs(theta[b]); });
  std::vector<float> out(P, 0.0f);
  for (int64_t r = 0; r < n_keep; ++r) out[idx[r]] = theta[idx[r]];
  if (P) std::memcpy(theta_out, out.data(), (size_t)P * sizeof(float));
  return PARO_OK;
}

}  // extern "C"
