// Internal declarations shared by the host library and the gfx950 kernels.
#pragma once

#include <hip/hip_runtime.h>

#include <cstddef>
#include <cstdint>
#include <string>
#include <vector>

#include "../../include/paro.h"

namespace paro {

// ---------------------------------------------------------------------------
// Rotation schedule for the activation kernel.
//
// The d channels are cut into segments of 128 channels (groups of 64 or 128:
// one or two groups per segment) or 256 channels (group 256). One wavefront
// processes one segment of a token: "virtual lane" v (0 .. SEG/2-1) holds two
// channels, in registers X and Y; with 256-channel segments a hardware lane
// holds two virtual lanes (v = lane and v = lane + 64).
//
// Between two consecutive pairings (the natural pairing {2v, 2v+1} before
// stage 0 and after stage K-1, and the K stages in between) every virtual
// lane keeps one of its two channels (in X) and fetches the other member of
// its next pair from the Y register of another virtual lane, through a
// per-wave LDS tile. The two pairings together form disjoint even cycles, so
// a "keep one, fetch one" assignment always exists.
//
// Table image per segment: NW fields (padded with zero words to a multiple of
// four) for each of NV virtual lanes, four fields interleaved per lane so that
// a lane loads four consecutive fields with one 16-byte load and a wavefront's
// load is one contiguous 1 KB: field f of virtual lane v is word
// ((f / 4) * NV + v) * 4 + f % 4 of the segment. Field order:
//   0                 load selector (v_perm byte selector putting the kept
//                     channel of the natural pair in the low half)
//   1 + 2*tau         LDS byte offset the lane writes its Y to, tau = 0..K
//   2 + 2*tau         LDS byte offset the lane reads its fetched value from
//   3 + 2*K + c*t + e stage t coefficient e (c = 2 for the factored form,
//                     4 for the general 2x2 form)
//   then              final scale of X, final scale of the fetched value,
//                     store byte offset of the natural pair, store selector.
// After all segments' images: the store permutation, [segs][NV][2] words.
// Virtual lane v ends the last exchange holding the natural pair q(v) (the
// pair at the store byte offset above); word 0 of lane v is the LDS byte
// offset it writes its packed output word to, word 1 the offset virtual lane
// v reads natural pair v from (slots planned like an exchange's).
// ---------------------------------------------------------------------------
struct RotPlanLayout {
  int seg_ch = 128;      // channels per segment
  int ppl = 1;           // virtual lanes per hardware lane
  int nv = 64;           // virtual lanes per segment
  int coef = 2;          // coefficients per stage (2 factored, 4 general)
  int words = 0;         // words per virtual lane (fields rounded up to four)
  int stages = 0;        // stages the activation schedule executes (<= K)
  bool fast = true;      // factored two-FMA stage form
};

inline int rot_field_count(int K, int coef) { return 1 + 2 * (K + 1) + coef * K + 4; }
// words per virtual lane in the image: the field count rounded up to four
inline int rot_words(int K, int coef) { return (rot_field_count(K, coef) + 3) & ~3; }

// first word of the store permutation, and the whole image, in words
inline size_t rot_perm_base(int64_t segs, const RotPlanLayout& lay) { return (size_t)segs * lay.words * lay.nv; }
inline size_t rot_table_words(int64_t segs, const RotPlanLayout& lay) {
  return rot_perm_base(segs, lay) + (size_t)segs * lay.nv * 2;
}

struct RotPlanHost {
  RotPlanLayout lay;
  std::vector<uint32_t> table;  // [segs][words / 4][nv][4], then [segs][nv][2]
  // canonical fp32 tables for the weight transform, per group, stage, pair:
  // local (i | j << 16), c bits, s bits
  std::vector<uint32_t> wt_pairs;  // [groups][K][G/2]
  std::vector<float> wt_c, wt_s;   // [groups][K][G/2]
  std::vector<float> alpha;        // [d]
  // gradient kernel: per segment, stage, lane slot: (i | j << 16, c bits,
  // s bits, flat pair index)
  std::vector<uint32_t> bw;        // [segs][K][seg_ch / 2][4]
};

// Validates arguments and builds the schedule. Returns a paro_status.
int build_rotation_plan(int64_t d, int32_t group, int32_t K, const int32_t* pairs,
                        const float* theta, const float* alpha, RotPlanHost* out);

void set_error(const std::string& msg);

// Gradients of the transform (activation side: X' = X T^-1; weight side:
// rows of T W). part is scratch of rotate_backward_scratch_bytes(r, M).
size_t rotate_backward_scratch_bytes(const paro_rotation* r, int64_t M);
hipError_t launch_rotate_backward(const paro_rotation* r, int weight_side, const uint16_t* x,
                                  const float* gy, float* gx, float* dtheta, float* dalpha,
                                  int64_t M, void* part, hipStream_t stream);

// Layer-wise output loss and its straight-through angle/scale gradients
// (layer_loss.hip): scratch bytes, the whole computation, and a zero fill.
size_t layer_loss_scratch_bytes(const paro_rotation* r, int64_t M, int64_t N, int64_t d, bool grad);
int run_layer_loss(const paro_rotation* r, const uint16_t* x, const uint16_t* w, const uint8_t* qw,
                   const uint16_t* sc, const uint8_t* zr, int64_t M, int64_t N, int64_t d, int group,
                   float* loss, float* dtheta, float* dalpha, void* ws, hipStream_t stream);
hipError_t launch_fill_zero(float* a, int64_t n, hipStream_t stream);

}  // namespace paro

struct paro_rotation {
  int64_t d;
  int32_t group;
  int32_t K;
  int device;
  paro::RotPlanLayout lay;
  uint32_t* d_table;    // device copy of RotPlanHost::table
  uint32_t* d_wt_pairs; // device canonical weight-transform tables
  float* d_wt_c;
  float* d_wt_s;
  float* d_alpha;
  uint32_t* d_bw;       // device copy of RotPlanHost::bw
};

namespace paro {
// Kernel launchers (defined in the .hip files). Return hipError_t of the launch.
hipError_t launch_rotate(const paro_rotation* r, const uint16_t* x, uint16_t* y, int64_t M,
                         hipStream_t stream);
// err (NULL or 4-byte aligned): also writes the quantization error
// E = W_hat - T W [N][d] (W_hat = (q - z) s, T W in the canonical fp32 order)
// rounded to fp16
hipError_t launch_quantize(const paro_rotation* r, const uint16_t* w, int64_t N, int64_t d,
                           int group, uint8_t* qweight, uint16_t* scales, uint8_t* zeros,
                           int* d_flag, hipStream_t stream, uint16_t* err = nullptr);
// Dense fp16 "NT" products (dense_gemm.hip), C[m][n] = sum_k A[m][k] B[n][k]
// with fp32 accumulation; K % 64 == 0, row strides in elements, 16-byte
// aligned rows.
//  * launch_nt_gemm_f32: C fp32 [M][ldc].
//  * launch_nt_gemm_loss: A = x [M][d], B = w [N][d]; part[nt_tiles(M, N)]
//    receives the per-tile sums of (yq - x w^T)^2 (yq fp16 [M][N]) and, with dy
//    != NULL, dy [M][ldd] = fp16(2 (yq - x w^T)), zero in columns N .. ldd - 1.
//  * launch_transpose_pad: out [C][ldo] = in^T for in fp16 [R][C] (C even,
//    ldo even, ldo >= R), zero in columns R .. ldo - 1.
int nt_tiles(int64_t M, int64_t N);
// Plain device copy (copy.hip): bytes % 16 == 0, 16-byte aligned pointers.
hipError_t launch_stream_copy(const void* src, void* dst, size_t bytes, int blocks, hipStream_t stream);
hipError_t launch_mfma_loop(const void* src, int64_t n8, float* out, int blocks, int iters, hipStream_t stream);
hipError_t launch_nt_gemm_f32(const uint16_t* a, int64_t lda, const uint16_t* b, int64_t ldb,
                              int64_t M, int64_t N, int64_t K, float* c, int64_t ldc,
                              hipStream_t stream);
hipError_t launch_nt_gemm_loss(const uint16_t* x, const uint16_t* w, int64_t M, int64_t N, int64_t d,
                               const uint16_t* yq, uint16_t* dy, int64_t ldd, float* part,
                               hipStream_t stream);
hipError_t launch_transpose_pad(const uint16_t* in, int64_t R, int64_t C, uint16_t* out, int64_t ldo,
                                hipStream_t stream);
// Large-batch linear (M > 16) on already transformed activations. The plan
// says whether the 256 x 256-tile kernel runs, and whether stream-K (the
// tiles' k-tiles shared out among the workgroups); a stream-K run needs the
// arrival counters (zero between calls) and partial_bytes of fp32 partial
// tiles, and without them (NULL) the layer takes the smaller-tile kernel.
struct GemmPlan {
  bool wide = false;
  bool sk = false;
  int sk_slots = 0;  // stream-K workgroups per XCD
  int nsplit = 1;    // smaller-tile kernel: workgroups per tile along k
  size_t partial_bytes = 0;
};
GemmPlan plan_w4_gemm(int64_t M, int64_t N, int64_t d);
hipError_t launch_w4_gemm(const uint16_t* x, const uint8_t* qweight, const uint16_t* scales,
                          const uint8_t* zeros, const uint16_t* bias, uint16_t* y, int64_t M,
                          int64_t N, int64_t d, int group, uint32_t* cnt, float* part, hipStream_t stream);
// Whether paro_device_init found workgroup b running on XCD b % 8.
bool xcd_dispatch_is_round_robin();

// Small-batch linear (M <= kDecodeMaxM). With r != NULL the activation transform runs
// inside the kernel (requires decode_fuses_rotation(r)); ws is the workspace:
// kDecodeCounterBytes of arrival counters (zero between calls), then the fp32
// partial sums [ceil(d / 512)][M][N].
constexpr size_t kDecodeCounterBytes = 16384;
constexpr int64_t kDecodeMaxM = 64;
bool decode_fuses_rotation(const paro_rotation* r);
// whether the small-batch call with these sizes fuses it (else the transform
// runs first, into the workspace)
bool decode_fuses_rotation(const paro_rotation* r, int64_t M, int64_t N, int64_t d);
// Devices the library keeps per-device state for (device ordinals below this).
constexpr int kMaxDevices = 64;
// Runs the XCD dispatch probe on device dev (current) once and records the
// result; allocates, launches and synchronizes. Returns a paro_status.
int xcd_dispatch_probe(int dev);

// Static device scratch of paro_w4_linear_noalloc (noalloc.hip): its size,
// the once-per-device look-up of its address (with dev current; clears the
// arrival counters and synchronizes) and the recorded address (NULL before
// set-up).
constexpr size_t kNoallocScratchBytes = (size_t(64) << 20) + kDecodeCounterBytes;
int noalloc_scratch_setup(int dev);
void* noalloc_scratch(int dev);
hipError_t launch_w4_decode(const uint16_t* x, const uint8_t* qweight, const uint16_t* scales,
                            const uint8_t* zeros, const uint16_t* bias, uint16_t* y, int64_t M,
                            int64_t N, int64_t d, int group, const paro_rotation* r, void* ws,
                            hipStream_t stream);
}  // namespace paro
