/*
 * paro.h - C ABI of the MI355X (gfx950) rotated W4G128 linear library.
 *
 * The library implements the inference hot path of ParoQuant (pairwise
 * rotation quantization, arXiv 2511.10645):
 *
 *   Y = X W + b = (X T^-1)(T W) + b                     (CSDN article, section 2.1)
 *   T = (prod_{t=1..K} R(P_t, Theta_t)) diag(alpha)     (paper notes, "关键设计")
 *
 * R(P_t, Theta_t) is one stage of independent Givens rotations: every channel
 * of a quantization group belongs to exactly one pair (i, j) of the stage, and
 * the pair is rotated by its own angle theta with the 2x2 matrix
 * [[cos, -sin], [sin, cos]] acting on (v_i, v_j) (CSDN article, section 2.2):
 *
 *   v_i <- cos(theta) v_i - sin(theta) v_j,   v_j <- sin(theta) v_i + cos(theta) v_j
 *
 * Conventions fixed by this library (the pages leave them open):
 *   - stage 0 of the arrays is applied first;
 *   - activations are divided by alpha and then go through the SAME stages in
 *     the SAME order with the SAME update (this equals x T^-1 for a row x);
 *     weights are multiplied by alpha and then go through the stages;
 *   - W4G128 quantization (paper notes, "主实验"; per-group s and z:
 *     "损失函数 / 训练策略") is asymmetric min/max round-to-nearest-even over
 *     15 steps with the range widened to include 0, an fp16 scale and an
 *     integer zero in [0, 15].
 *
 * Types: fp16 tensors are passed as uint16_t* (IEEE binary16 bit patterns).
 * Every tensor is row-major and contiguous. Device pointers are HIP device
 * memory (for example torch.Tensor.data_ptr() of a ROCm tensor); host
 * pointers are ordinary memory. The caller owns every tensor; a rotation
 * handle owns only the device tables it allocates in paro_rotation_create and
 * frees in paro_rotation_destroy.
 *
 * Errors: every int-returning function returns PARO_OK (0) or a negative
 * paro_status and never throws or aborts. Argument checks run on the host
 * before anything is enqueued, so a failed check enqueues nothing. A failed
 * kernel launch returns PARO_ERR_HIP. Asynchronous device faults surface at
 * the caller's next synchronisation, as with any HIP library.
 * paro_last_error() returns a thread-local message for the last failure.
 *
 * Threads and streams: hot calls (paro_rotate, paro_w4_linear) allocate
 * nothing, do not synchronise and write no global state (they may be captured
 * into a HIP graph); a handle may be used from several threads and streams at
 * once. Per-device set-up that needs allocation and synchronisation happens in
 * paro_device_init, which paro_rotation_create also runs.
 */
#ifndef PARO_H
#define PARO_H

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h> /* hipStream_t */

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  PARO_OK = 0,
  PARO_ERR_NULL = -1,        /* a required pointer is NULL */
  PARO_ERR_SHAPE = -2,       /* sizes inconsistent (d % group, N % 16, negative sizes, ...) */
  PARO_ERR_PAIRING = -3,     /* a stage is not a perfect pairing inside every group */
  PARO_ERR_VALUE = -4,       /* alpha <= 0 or non-finite, theta non-finite, non-finite weights */
  PARO_ERR_ALIGN = -5,       /* a tensor pointer is not 16-byte aligned */
  PARO_ERR_UNSUPPORTED = -6, /* a valid request the library does not implement */
  PARO_ERR_WORKSPACE = -7,   /* workspace missing or too small */
  PARO_ERR_HIP = -8          /* a HIP runtime call failed */
} paro_status;

/* Static string naming a status code. Never NULL. */
const char* paro_status_string(int status);

/* Thread-local detail message of the last failing call on this thread ("" if none). */
const char* paro_last_error(void);

/*
 * Per-device set-up (synchronous; allocates, launches and synchronises on the
 * null stream, so not inside a stream capture). Checks once per device how
 * workgroups are dispatched to the XCDs (the small-batch linear splits k over
 * workgroups that must meet in one XCD's L2) and records the result;
 * idempotent and thread-safe. paro_rotation_create calls it for its device.
 * A device on which it never ran still gives correct results: the
 * small-batch linear then exchanges its partial sums through memory-side
 * (system-scope) accesses, about 15% slower.
 * Errors: PARO_ERR_HIP (nothing is recorded; a later call tries again),
 * PARO_ERR_UNSUPPORTED (device ordinal >= 64).
 */
int paro_device_init(void);

/* Opaque rotation plan: the K stages of pairs/angles plus alpha for one layer,
 * validated and turned into device tables. Immutable after creation. */
typedef struct paro_rotation paro_rotation;

/*
 * Create a rotation plan on the current HIP device (synchronous).
 *
 *   d      number of input channels; d % group == 0; d % 128 == 0;
 *          d <= 2^24.
 *   group  rotation group size: 64, 128 or 256 (pairs never leave a group,
 *          paper notes "关键设计").
 *   K      number of stages, 0 <= K <= 32 (the pages' default is 8).
 *   pairs  host int32 [K][d/2][2], global channel ids. In every stage each
 *          channel appears exactly once and i / group == j / group. The
 *          order of pairs inside a stage is free; the order (i, j) inside a
 *          pair selects the sign as in the update above (swapping i and j is
 *          the same as negating theta). Partial and sparse pairings (only
 *          some pairs rotate; paper notes "核心观察") are expressed with
 *          theta = 0, an exact identity; the activation side then skips the
 *          identities and runs fewer stages where the remaining rotations
 *          allow it (see paro_rotation_plan_host's layout[4]).
 *   theta  host float [K][d/2], radians, finite. The library evaluates
 *          c = (float)cos((double)theta), s = (float)sin((double)theta) on the
 *          host.
 *   alpha  host float [d], finite and > 0.
 *   out    receives the handle.
 *
 * Runs paro_device_init for the current device.
 * Errors: PARO_ERR_NULL, PARO_ERR_SHAPE, PARO_ERR_PAIRING, PARO_ERR_VALUE,
 * PARO_ERR_UNSUPPORTED (group not in {64,128,256}, K > 32, d % 128 != 0,
 * d > 2^24),
 * PARO_ERR_HIP (device allocation or copy failed). The host arrays are only
 * read during the call.
 */
int paro_rotation_create(int64_t d, int32_t group, int32_t K, const int32_t* pairs,
                         const float* theta, const float* alpha, paro_rotation** out);

/* Free the plan's device tables (synchronous). NULL is a no-op. The caller
 * must make sure no enqueued work still uses the handle. */
void paro_rotation_destroy(paro_rotation* r);

/* Read back plan properties (host only; any pointer may be NULL). */
int paro_rotation_info(const paro_rotation* r, int64_t* d, int32_t* group, int32_t* K);

/*
 * Online activation transform X' = X T^-1, row by row
 * (paper notes, "关键设计" and "亮点与洞察": one fused launch for all stages).
 *
 *   x, y   device fp16 [M][d], 16-byte aligned. y == x (in place) is allowed;
 *          any other overlap is undefined.
 *   M      number of token rows, 0 <= M <= 2^31 - 1; M == 0 is a no-op.
 *   stream HIP stream the kernel is enqueued on (0 = the null stream).
 *
 * Arithmetic: fp32 inside, one fp16 round-to-nearest-even per output.
 * Errors: PARO_ERR_NULL, PARO_ERR_SHAPE (M out of range), PARO_ERR_ALIGN,
 * PARO_ERR_HIP.
 */
int paro_rotate(const paro_rotation* r, const uint16_t* x, uint16_t* y, int64_t M,
                hipStream_t stream);

/*
 * Offline weight transform and int4 group quantization: Q(T W) (r != NULL)
 * or Q(W) (r == NULL, plain W4).
 *
 *   w        device fp16 [N][d] (the nn.Linear [out][in] layout, i.e. the
 *            transpose of the math W whose rows are input channels).
 *   group    quantization group along d: 64, 128 or 256; with r != NULL it
 *            must equal the plan's group.
 *   qweight  device uint8 [N][d/2]: each 4 bytes (a little-endian 32-bit
 *            word) hold the codes c0 .. c7 of 8 consecutive channels, the even
 *            channels in the low 16 bits and the odd ones in the high 16 bits,
 *            4 bits each in channel order: bytes c0 | c2 << 4, c4 | c6 << 4,
 *            c1 | c3 << 4, c5 | c7 << 4 (so that two codes at a time unpack
 *            into an fp16 pair with one AND-OR).
 *   scales   device fp16 [N][d/group].
 *   zeros    device uint8 [N][d/group], values 0..15.
 *
 * The result is bit-exact with this arithmetic, in fp32 with every operation
 * rounded on its own (no fused multiply-add):
 *   u_k = w_k * alpha_k; for each stage and pair: a = u_i, b = u_j,
 *   u_i = c*a - s*b, u_j = s*a + c*b (c, s as in paro_rotation_create);
 *   per group: mn = min(0, min u), mx = max(0, max u), s32 = (mx - mn) / 15,
 *   s16 = fp16(s32) (round to nearest even; 0 becomes 1.0),
 *   z = clamp(rint(-mn / s16), 0, 15), q = clamp(rint(u / s16) + z, 0, 15).
 * Synchronises the stream to read a device error flag and returns
 * PARO_ERR_VALUE if some transformed weight or some scale is not finite
 * (the outputs are then unspecified). Allocates a 4-byte flag per call.
 * Errors: also PARO_ERR_NULL, PARO_ERR_SHAPE, PARO_ERR_ALIGN,
 * PARO_ERR_UNSUPPORTED, PARO_ERR_HIP.
 */
int paro_quantize_weights(const paro_rotation* r, const uint16_t* w, int64_t N, int64_t d,
                          int32_t group, uint8_t* qweight, uint16_t* scales, uint8_t* zeros,
                          hipStream_t stream);

/* Bytes of device workspace with which paro_w4_linear runs its fastest
 * kernels for this plan (NULL: plain W4) and these sizes; 0 means the call
 * uses no workspace. For M > 64 on layers with fewer than 256 output tiles of
 * 256 x 256 whose k-tiles can be shared out among the workgroups (stream-K)
 * this includes 128 MiB of fp32 partial tiles (two of 256 KB per workgroup),
 * and on layers whose 64 x 128 tiles leave CUs idle 32 KB per tile and k
 * split; paro_w4_linear also runs, with the smaller-tile kernel unsplit, on
 * the minimum: 16 KiB + M d 2 bytes (rounded up to 256) with a plan, none
 * without. */
size_t paro_w4_linear_workspace_size(const paro_rotation* r, int64_t M, int64_t N, int64_t d);

/*
 * The W4 linear layer on rotated activations (W4G128 in the paper notes'
 * main experiments; groups of 64 and 256 as well, the sizes the CSDN
 * article's section 5.2 compares):
 *   Y[m][n] = sum_k X'[m][k] * (q[n][k] - z[n][k/G]) * s[n][k/G] + bias[n]
 * with X' = X T^-1 when r != NULL (rotated inside the call) and X' = X when
 * r == NULL (plain W4, or activations the caller rotated already).
 *
 *   x        device fp16 [M][d]; qweight/scales/zeros as produced by
 *            paro_quantize_weights with the same group; bias device fp16 [N]
 *            or NULL;
 *   y        device fp16 [M][N] (must not overlap x).
 *   group    G = 64, 128 or 256; other values return PARO_ERR_UNSUPPORTED.
 *            A plan r must have the same d and group (the pairs stay inside
 *            quantization groups), else PARO_ERR_SHAPE.
 *   N % 16 == 0, d % 128 == 0, d % G == 0, M >= 0 (M == 0 is a no-op); N <= 2^30,
 *   d <= 2^22, M < 2^30, else PARO_ERR_UNSUPPORTED.
 *   workspace, workspace_bytes: device memory of
 *            paro_w4_linear_workspace_size(r, M, N, d) bytes, or of at least
 *            the minimum given there (M > 64: then without stream-K),
 *            256-byte aligned (may be NULL when the size in use is 0;
 *            smaller than the minimum: PARO_ERR_WORKSPACE). Its first 16 KiB hold
 *            arrival counters that must be zero before the first call that
 *            uses the workspace (zero-fill it once after allocating it); every
 *            call leaves them zero again. The rest is scratch. Calls that may
 *            run at the same time (different streams) need different
 *            workspaces.
 *
 * Execution: M <= 64 runs one kernel that streams the packed weights (token
 * columns in blocks of 16) and, for plans of group 64 or 128 that execute at
 * most 8 stages, applies the transform to the activations inside the same
 * kernel; other plans rotate into the workspace first. M > 64 rotates into
 * the workspace and then runs
 * a matrix-core kernel: 256 x 256 tiles from 256 such tiles, one per
 * workgroup; with fewer, when every XCD holds n-blocks and k is long enough,
 * the same kernel with each XCD's k-tiles shared out in equal ranges among 16
 * to 32 of its workgroups (stream-K): partial tiles meet through fp32 partial
 * tiles in the workspace (the last piece to arrive adds them in k order),
 * when the workspace holds them; else a kernel with 128 x 256 tiles, or
 * 64 x 256 or 64 x 128 (k split two or four ways inside the workgroup) for
 * layers with few tiles, the latter with k also split across 2 or 4
 * workgroups per tile when the tiles leave CUs idle and the workspace holds
 * their partial tiles.
 *
 * Arithmetic: X' exactly as paro_rotate computes it (fp16); fp32 accumulation
 * of exact fp16 products against the fp16 rounding of each dequantized weight
 * (q - z) * s, in an order that depends on the sizes (and for M > 64 on
 * whether the workspace holds the stream-K partial tiles) but not on timing;
 * fp16 output.
 * Errors: PARO_ERR_NULL, PARO_ERR_SHAPE, PARO_ERR_ALIGN, PARO_ERR_UNSUPPORTED,
 * PARO_ERR_WORKSPACE, PARO_ERR_HIP.
 */
int paro_w4_linear(const paro_rotation* r, const uint16_t* x, const uint8_t* qweight,
                   const uint16_t* scales, const uint8_t* zeros, const uint16_t* bias,
                   uint16_t* y, int64_t M, int64_t N, int64_t d, int32_t group,
                   void* workspace, size_t workspace_bytes, hipStream_t stream);

/*
 * paro_w4_linear for callers that cannot allocate device memory (code under
 * HIP-graph capture, tight serving loops, harnesses that forbid hipMalloc):
 * the same kernels, arguments and result as paro_w4_linear, with the
 * workspace taken from a static device array inside the library instead of a
 * caller's buffer. The call allocates and frees nothing.
 *
 *   Scratch: (64 MiB + 16 KiB) per device, held from the library's load until
 *            the process ends; its address is looked up and its arrival
 *            counters cleared by paro_device_init (paro_rotation_create runs
 *            it), and every completed call leaves the counters zero again.
 *   Limit:   the minimum workspace of paro_w4_linear (see
 *            paro_w4_linear_workspace_size) must not exceed that size (for
 *            example M x d <= 32 Mi elements for a rotated layer with
 *            M > 64), else PARO_ERR_WORKSPACE and nothing is enqueued; the
 *            stream-K partial tiles are used when they fit as well.
 *   Sharing: every call on one device uses that device's single array, so
 *            calls that may run at the same time on one device (several
 *            streams or threads) race and give wrong results: serialise them,
 *            or use paro_w4_linear with a workspace per stream.
 * Errors: those of paro_w4_linear, PARO_ERR_WORKSPACE (too large, see
 * above), PARO_ERR_UNSUPPORTED (paro_device_init has not run on the current
 * device).
 */
int paro_w4_linear_noalloc(const paro_rotation* r, const uint16_t* x, const uint8_t* qweight,
                           const uint16_t* scales, const uint8_t* zeros, const uint16_t* bias,
                           uint16_t* y, int64_t M, int64_t N, int64_t d, int32_t group,
                           hipStream_t stream);

/* Which transform paro_rotation_backward differentiates. */
typedef enum {
  PARO_SIDE_ACTIVATION = 0, /* X' = X T^-1, as paro_rotate computes it */
  PARO_SIDE_WEIGHT = 1      /* the rows of T W in the [N][d] layout, as the quantizer transforms them */
} paro_side;

/* Bytes of device scratch paro_rotation_backward needs for M rows (0 when
 * M <= 0). */
size_t paro_rotation_backward_workspace_size(const paro_rotation* r, int64_t M);

/*
 * Gradients of the transform with respect to its input, its angles and its
 * channel scales: the step that learns theta and alpha by minimising the
 * layer-wise output loss (paper notes, "损失函数 / 训练策略"). For every row r
 * of x (a token for PARO_SIDE_ACTIVATION; a weight row, [N][d] layout, for
 * PARO_SIDE_WEIGHT) the transform is v_0 = r / alpha (activation) or
 * r * alpha (weight), then the K stages in order with the pair update
 * (v_i, v_j) <- (c v_i - s v_j, s v_i + c v_j) (CSDN article, section 2.2).
 * Given gy = dL/d(output):
 *   gx[m][k]     = dL/dr: gy walked back through the transposed stages, then
 *                  divided (activation) or multiplied (weight) by alpha;
 *   dtheta[t][p] = sum over rows of g'_j v'_i - g'_i v'_j, with (i, j) the
 *                  stored pair p of stage t, v' that stage's outputs and g'
 *                  their gradient (d v'_i / d theta = -v'_j,
 *                  d v'_j / d theta = v'_i); pairs with theta = 0 included;
 *   dalpha[k]    = sum over rows of g_0[k] * d v_0[k] / d alpha[k], i.e.
 *                  -g_0 r / alpha^2 (activation) or g_0 r (weight),
 * with g_0 the gradient of v_0.
 *
 *   side     PARO_SIDE_ACTIVATION or PARO_SIDE_WEIGHT, else PARO_ERR_VALUE.
 *   x        device fp16 [M][d] (4-byte aligned): the transform's input.
 *   gy       device fp32 [M][d] (8-byte aligned): gradient of its output.
 *   gx       device fp32 [M][d] (8-byte aligned) or NULL (not computed); may
 *            be gy itself (in place).
 *   dtheta   device fp32 [K][d/2] (may be NULL when K == 0), overwritten.
 *   dalpha   device fp32 [d], overwritten.
 *   M        rows, 0 <= M < 2^31 (M == 0 writes zero gradients).
 *   workspace, workspace_bytes: device scratch of at least
 *            paro_rotation_backward_workspace_size(r, M) bytes, 256-byte
 *            aligned (NULL when that size is 0); calls that may overlap need
 *            different workspaces.
 *
 * Arithmetic: fp32. The stages' inputs are recovered from their outputs by
 * the transposed update instead of being stored. The sums over rows are taken
 * per chunk of rows and the chunks added in a fixed order: the result does
 * not depend on scheduling.
 * Errors: PARO_ERR_NULL, PARO_ERR_VALUE, PARO_ERR_SHAPE, PARO_ERR_ALIGN,
 * PARO_ERR_WORKSPACE, PARO_ERR_HIP.
 */
int paro_rotation_backward(const paro_rotation* r, int32_t side, const uint16_t* x,
                           const float* gy, float* gx, float* dtheta, float* dalpha, int64_t M,
                           void* workspace, size_t workspace_bytes, hipStream_t stream);

/* Bytes of device workspace paro_layer_loss needs (0 for M <= 0, or d not the plan's). */
size_t paro_layer_loss_workspace_size(const paro_rotation* r, int64_t M, int64_t N, int64_t d,
                                      int32_t with_gradients);

/*
 * Layer-wise output loss of the quantized, transformed layer (paper notes,
 * "损失函数 / 训练策略": L = ||Q(D)(X') - D(X)||, minimised per layer to learn
 * the angles and scales), as the squared Frobenius norm
 *   L = sum_{m,n} (Y_q[m][n] - Y[m][n])^2,
 *   Y_q = paro_w4_linear's output (fp16) on X' = paro_rotate(x) with the
 *         4-bit weights (qweight, scales, zeros: Q(T W) from
 *         paro_quantize_weights with this plan), i.e. fp32 sums of X' times
 *         the fp16 rounding of each dequantized weight,
 *   Y   = x w^T with w the original fp16 weights [N][d] (fp32 accumulation).
 * With dtheta and/or dalpha non-NULL also the gradients, passing through the
 * quantizer and the fp16 roundings unchanged (straight-through):
 * dY = 2 (Y_q - Y), dL/dX' = dY W_hat, dL/d(T W) = dY^T X', then both
 * transforms' gradients as paro_rotation_backward computes them (activation
 * side with x, weight side with w), summed. Since X' (T W)^T = X W^T for all
 * angles and scales, that sum equals the activation side's gradient for
 * dL/dX' = dY E, E = W_hat - T W (T W in the quantizer's fp32), which is how
 * it is computed: the two sides' other terms cancel and are each tens of
 * times larger than the result. E comes from the quantizer's own pass over
 * T W, with W_hat from the codes that pass produces; these equal qweight,
 * scales and zeros bit for bit when those are Q(T W) of this plan, as
 * required above. dY and E enter that product rounded to fp16, with fp32
 * sums.
 *
 *   x        device fp16 [M][d], w device fp16 [N][d] (16-byte aligned);
 *   qweight, scales, zeros: as for paro_w4_linear, with the plan's group;
 *   loss     device fp32 [1] (per-tile sums in a fixed order, fp64 at the end);
 *   dtheta   device fp32 [K][d/2] or NULL; dalpha device fp32 [d] or NULL;
 *   N % 16 == 0, 0 <= M, N < 2^30; M == 0 writes zeros.
 *   workspace: at least paro_layer_loss_workspace_size(r, M, N, d, dtheta ||
 *            dalpha) bytes, 256-byte aligned, zero-filled once after
 *            allocation (its first 16 KiB hold paro_w4_linear's arrival
 *            counters for M <= 64, which every call leaves zero, whatever M
 *            and N the workspace is reused with). Calls that may run at the
 *            same time need different workspaces.
 * Every step runs in this library's kernels (the dense products on the
 * matrix cores); the call allocates nothing and does not synchronise.
 * Errors: PARO_ERR_NULL, PARO_ERR_SHAPE, PARO_ERR_ALIGN, PARO_ERR_WORKSPACE,
 * PARO_ERR_HIP, and those of paro_w4_linear.
 */
int paro_layer_loss(const paro_rotation* r, const uint16_t* x, const uint16_t* w,
                    const uint8_t* qweight, const uint16_t* scales, const uint8_t* zeros, int64_t M,
                    int64_t N, int64_t d, int32_t group, float* loss, float* dtheta, float* dalpha,
                    void* workspace, size_t workspace_bytes, hipStream_t stream);

/*
 * Channel-pair selection (host only, synchronous, no GPU): fills pairs
 * [K][d/2][2] with global channel ids in the layout paro_rotation_create
 * takes; every stage is a perfect pairing inside every group of `group`
 * channels (pair p of a stage belongs to group p / (group / 2)).
 *
 * paro_pairs_random: random pairs with de-duplication, the selection the
 * paper notes name ("局限与展望": random plus de-duplication). Reading: for
 * each group in order and each stage in order, draw a uniformly random
 * permutation of the group's channels (Fisher-Yates from the last position
 * down, j = r mod (i + 1) with r the next SplitMix64 output of one stream
 * seeded with `seed`, state += 0x9E3779B97F4A7C15 per output); then for
 * positions i = 0, 2, 4, ... pair the channel at i with the first channel
 * after it not yet paired with it in an earlier stage of the group, which is
 * exchanged with the channel at position i + 1; if none is left, draw the
 * stage again (at most 4096 draws).
 * The pair is stored as (channel at i, its partner). No unordered pair
 * occurs twice in one group. K <= group - 1; near that bound the earlier
 * stages can leave no pairing without repeats (for example 7 stages of a
 * group of 8 need a one-factorization the greedy stages may not extend), and
 * the call returns PARO_ERR_VALUE.
 * Errors: PARO_ERR_NULL, PARO_ERR_SHAPE (group odd or not dividing d, d >
 * 2^24, K out of range), PARO_ERR_VALUE (4096 draws without a pairing).
 */
int paro_pairs_random(int64_t d, int32_t group, int32_t K, uint64_t seed, int32_t* pairs);

/*
 * paro_pairs_by_gap: pairs of channels whose values differ strongly (CSDN
 * article, section 2.2: pairs with a large numeric difference are preferred).
 * score: host float [d], one value per input channel (for example the
 * largest |W| over the output rows). Reading: in each group, rank the
 * channels by score, largest first (ties: lower channel first); stage t
 * pairs the i-th largest with the ((i + t) mod (group / 2))-th smallest, for
 * i = 0 .. group / 2 - 1, stored as (larger, smaller). Stage 0 pairs the
 * largest with the smallest; every pair joins the top and the bottom half of
 * the ranking, which is the largest total score difference a perfect
 * pairing can have, and no pair repeats across stages. K <= group / 2.
 * Errors: PARO_ERR_NULL, PARO_ERR_SHAPE, PARO_ERR_VALUE (non-finite score).
 */
int paro_pairs_by_gap(int64_t d, int32_t group, int32_t K, const float* score, int32_t* pairs);

/*
 * paro_sparsify_angles: keep only the strongest rotations of a plan (paper
 * notes, "核心观察": a sparse rotation keeping the top 10% of the channel
 * pairs matches the full one). theta, theta_out: host float [K][d/2] (may
 * be the same array). Reading: the n_keep pairs with the largest |theta| over
 * the whole plan keep their angle (ties: the earlier stage and pair first),
 * every other pair gets theta = 0, an exact identity. For angles in
 * [-pi, pi], |theta| orders the rotations by their distance from the
 * identity. Errors: PARO_ERR_NULL, PARO_ERR_SHAPE (0 <= n_keep <= K d / 2,
 * d even), PARO_ERR_VALUE (non-finite angle).
 */
int paro_sparsify_angles(int64_t d, int32_t K, const float* theta, int64_t n_keep, float* theta_out);

/*
 * Measurement: a plain device copy dst[0 .. bytes) = src[0 .. bytes) at the
 * rate HBM sustains for one read and one write stream (16-byte buffer loads
 * and stores, 4 per lane in flight, `blocks` workgroups of 256 lanes striding
 * over the buffer). It is the measured ceiling that the memory-bound kernels
 * (paro_rotate, the small-batch paro_w4_linear) are reported against, next to
 * the datasheet peak; it takes no part in the method.
 *   src, dst  device memory, 16-byte aligned, not overlapping;
 *   bytes     a multiple of 16 (0 is a no-op);
 *   blocks    1 .. 2^20.
 * Asynchronous on stream. Errors: PARO_ERR_NULL, PARO_ERR_ALIGN,
 * PARO_ERR_SHAPE, PARO_ERR_HIP.
 */
int paro_stream_copy(const void* src, void* dst, size_t bytes, int32_t blocks, hipStream_t stream);

/*
 * Measurement: fp16 matrix-core throughput with operands in registers. Each
 * of `blocks` workgroups runs one wavefront per SIMD (256 lanes); every
 * wavefront runs `iters` rounds of 16 independent v_mfma_f32_32x32x16_f16
 * (32768 flop each) on operands read once from src, then each lane writes the
 * sum of its 256 fp32 accumulators to out[lane]. With random operands the
 * rate is the ceiling the matrix cores sustain under the chip's power limit,
 * which the prefill linear is reported against next to the datasheet peak; it
 * takes no part in the method. With every operand 1.0, each output is
 * 4096 * iters.
 *   src   device fp16 [n], 16-byte aligned, n a multiple of 8 in [8, 2^30];
 *   out   device float [blocks * 256];
 *   blocks 1 .. 2^16, iters >= 0.
 * Asynchronous on stream. Errors: PARO_ERR_NULL, PARO_ERR_ALIGN,
 * PARO_ERR_SHAPE, PARO_ERR_HIP.
 */
int paro_mfma_loop(const void* src, int64_t n, float* out, int32_t blocks, int32_t iters, hipStream_t stream);

/*
 * Host-only view of the per-segment rotation schedule that
 * paro_rotation_create uploads (for testing the plan logic without a GPU).
 * Fills `out` (host memory of out_bytes) with the exact table image and writes
 * the image size to *needed (out may be NULL to query the size), and the
 * layout descriptor to *layout (may be NULL):
 *   layout[0] = channels per segment (128 or 256),
 *   layout[1] = pairs per lane (1 or 2),
 *   layout[2] = 32-bit words per virtual lane per segment (the schedule's
 *               fields padded to a multiple of 4; the image of a segment is
 *               [layout[2] / 4][virtual lane][4], four consecutive fields of
 *               a lane side by side; after the segments' images comes the
 *               store permutation, [segment][virtual lane][2] words: the LDS
 *               byte offsets at which a lane writes its packed output pair
 *               and from which it reads the natural pair of its own index,
 *               which the activation transform uses for 256-channel
 *               segments),
 *   layout[3] = 1 if the factored two-FMA stage form is used, 0 for the
 *               general 2x2 form,
 *   layout[4] = stages the activation schedule executes: K for a plan
 *               without identities; with pairs of theta == 0 (exact
 *               identities, a partial or sparse pairing) the identities are
 *               dropped and each other rotation goes to the first stage after
 *               the last rotation on either of its channels, which gives the
 *               length of the longest chain of rotations linked by shared
 *               channels (<= K).
 * Runs the same validation as paro_rotation_create and returns its errors;
 * PARO_ERR_WORKSPACE when out is non-NULL and out_bytes is too small.
 */
int paro_rotation_plan_host(int64_t d, int32_t group, int32_t K, const int32_t* pairs,
                            const float* theta, const float* alpha, void* out, size_t out_bytes,
                            size_t* needed, int32_t layout[5]);

#ifdef __cplusplus
}
#endif

#endif /* PARO_H */
