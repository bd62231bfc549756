/*
 * qpn.h - C ABI of libqpn.so, a weight-streaming skinny GEMM for AMD MI355X
 * (gfx950): y[M, N] = x[M, K] * dequant(W)^T with M = 1..16 fp16 activation
 * rows and W held compressed in HBM as NVFP4 or FP8 (E4M3), decoded to fp16
 * in registers right before the matrix-core multiply.
 *
 * Pages cited ([P3]): https://reddlx.com/feed/productivity-ai-news, the post
 * "Four Tesla V100s from 2017 matched my RTX 5090 on single-request Qwen 3.8
 * decode"; section names are that post's headings.
 *
 * Conventions for every entry point:
 *   - All pointers named *_dev are device pointers (hipMalloc'd, or torch CUDA
 *     tensors); the caller owns every buffer. The library allocates no memory.
 *   - `stream` is a hipStream_t (NULL = the default stream). Device work is
 *     enqueued on it and the call returns without waiting, unless stated (the
 *     two pack calls wait for their stream: they report invalid codes).
 *   - Arguments are validated on the host before any HIP call; a failed check
 *     returns a negative qpn_status and enqueues nothing. A failed kernel
 *     launch returns QPN_ERR_HIP. Faults inside kernels surface
 *     asynchronously, as HIP reports them.
 *   - No global mutable state: calls may run concurrently on different
 *     streams as long as their output buffers do not overlap.
 */
#ifndef QPN_H
#define QPN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  QPN_OK = 0,
  QPN_ERR_INVALID_ARG = -1,      /* null / misaligned pointer, bad size or format */
  QPN_ERR_UNSUPPORTED = -2,      /* valid request the library does not implement */
  QPN_ERR_BAD_CODE = -3,         /* pack met invalid E4M3 codes (NaN, sign-set block scale) */
  QPN_ERR_BUFFER_TOO_SMALL = -4, /* packed buffer or workspace below the required size */
  QPN_ERR_HIP = -5               /* a HIP runtime call failed */
} qpn_status;

typedef enum { QPN_FMT_NVFP4 = 1, QPN_FMT_FP8_E4M3 = 2 } qpn_format;

/* Largest number of activation rows per call. A k-step speculative verify
 * round multiplies k+1 rows (k=7 gives the 8 rows of [P3] "What I actually
 * built"); the 16-row matrix-core tile holds up to 16 at no extra cost. */
#define QPN_MAX_M 16

/*
 * A packed weight matrix W[N, K] as qpn_gemm reads it.
 *   format       QPN_FMT_NVFP4 or QPN_FMT_FP8_E4M3.
 *   n, k         logical shape; n >= 0, k >= 0, k % 16 == 0.
 *   packed       device buffer written by qpn_pack_nvfp4 / qpn_pack_fp8 for
 *                the same (format, n, k); 16-byte aligned; opaque layout.
 *   tensor_scale NVFP4: the fp32 per-tensor scale s_t (host value). FP8: unused.
 *   row_scales   FP8: device float[n], the fp32 scale of each output row.
 *                NVFP4: unused (may be NULL).
 * The value of element (n, k) is
 *   NVFP4: E2M1(code[n][k]) * E4M3(block_scale[n][k / 16]) * tensor_scale
 *   FP8:   E4M3(code[n][k]) * row_scales[n]
 */
typedef struct {
  int32_t format;
  int32_t reserved; /* must be 0 */
  int64_t n;
  int64_t k;
  const void* packed;
  float tensor_scale;
  const float* row_scales;
} qpn_weight;

/* Human-readable name of a status code (static storage, never NULL). */
const char* qpn_status_string(qpn_status s);

/* Bytes of device memory the packed form of an [n, k] matrix occupies, or 0
 * when the arguments are invalid (unknown format, n < 0, k < 0, k % 16 != 0).
 * The packed form pads n up to a multiple of 16 and k up to a multiple of 256
 * with zero weights. */
size_t qpn_packed_bytes(int32_t format, int64_t n, int64_t k);

/*
 * Canonical NVFP4 -> packed device layout.
 *   codes_dev        uint8 [n][k/2] row-major; byte j of a row holds element
 *                    2j in its low nibble and 2j+1 in its high nibble (E2M1
 *                    codes s|e1e0|m, OCP MX v1.0).
 *   block_scales_dev uint8 [n][k/16] row-major E4M3FN codes, one per 16
 *                    consecutive elements of a row along k.
 *   packed_dev       output, packed_bytes >= qpn_packed_bytes(NVFP4, n, k),
 *                    16-byte aligned. Every byte of the packed form is written.
 *   bad_codes_dev    a device int32 (4-byte aligned, not NULL) that the call
 *                    uses as its counter: it is cleared, the pack kernels add
 *                    the invalid block-scale codes they find, NaN (0x7F, 0xFF)
 *                    or sign-set (0x80..0xFF: NVFP4 block scales are
 *                    positive), and it holds that count when the call returns.
 * Validation: the call waits for `stream` (pack is an offline, once-per-weight
 * step; do not capture it in a graph) and returns QPN_ERR_BAD_CODE if any
 * invalid code was found. The packed buffer is written all the same, byte for
 * byte (unpack reads it back), but must not be handed to a GEMM: a NaN or
 * negative scale would turn its block's outputs NaN or negate them (it never
 * makes the GEMM fault). Nothing to pack (n == 0 or k == 0): QPN_OK, the
 * counter is not touched.
 * The pages keep published FP4 regions in their own format rather than
 * converting them ([P3] "v1.0 got us here. v1.1 removes its last
 * compromise."); this entry point takes such codes as they are.
 */
qpn_status qpn_pack_nvfp4(const uint8_t* codes_dev, const uint8_t* block_scales_dev,
                          int64_t n, int64_t k, void* packed_dev, size_t packed_bytes,
                          int32_t* bad_codes_dev, void* stream);

/* Canonical FP8 -> packed layout. codes_dev: uint8 [n][k] row-major E4M3FN
 * codes. bad_codes_dev and the validation as for qpn_pack_nvfp4 (the call
 * waits for its stream and returns QPN_ERR_BAD_CODE), counting the NaN codes
 * 0x7F and 0xFF (weights of either sign are valid).
 * The per-row fp32 scales stay in a separate caller-owned array. ([P3] "v1.0
 * got us here. v1.1 removes its last compromise.": FP8 regions keep FP8.) */
qpn_status qpn_pack_fp8(const uint8_t* codes_dev, int64_t n, int64_t k,
                        void* packed_dev, size_t packed_bytes,
                        int32_t* bad_codes_dev, void* stream);

/* Packed -> canonical (the inverse of the two pack calls, for round-trip
 * checks). Outputs have the canonical shapes described above. */
qpn_status qpn_unpack_nvfp4(const void* packed_dev, size_t packed_bytes, int64_t n, int64_t k,
                            uint8_t* codes_dev, uint8_t* block_scales_dev, void* stream);
qpn_status qpn_unpack_fp8(const void* packed_dev, size_t packed_bytes, int64_t n, int64_t k,
                          uint8_t* codes_dev, void* stream);

/*
 * Synthetic-weight quantizers (offline helpers; the pages serve an already
 * quantized checkpoint and do not give a recipe, so the plainest two-level
 * one is used). All arithmetic is fp32, correctly rounded, ties to even.
 *
 * qpn_absmax_f32: out_dev[0] = max |x_dev[i]| over count floats (0 for
 *   count == 0; NaN if any element is NaN). Deterministic.
 * qpn_nvfp4_tensor_scale: host helper, amax / 2688 (= 6 * 448) in fp32, or 1
 *   when that is zero.
 * qpn_quantize_nvfp4: w_dev float [n][k] (finite; k % 16 == 0) and the
 *   tensor scale s_t -> codes_dev uint8 [n][k/2] (canonical nibble order) and
 *   block_scales_dev uint8 [n][k/16]:
 *     sc = E4M3((amax_block / 6) / s_t); d = E4M3value(sc) * s_t;
 *     code = d == 0 ? sign-only zero : E2M1(w / d), saturating at 6.
 * qpn_quantize_fp8: w_dev float [n][k] (finite) -> codes_dev uint8 [n][k]
 *   and row_scales_dev float [n]: s = amax_row / 448 (1 when zero),
 *   code = E4M3(w / s), saturating at 448.
 * Non-finite weights give unspecified codes (never a fault).
 */
qpn_status qpn_absmax_f32(const float* x_dev, int64_t count, float* out_dev, void* stream);
float qpn_nvfp4_tensor_scale(float amax);
qpn_status qpn_quantize_nvfp4(const float* w_dev, int64_t n, int64_t k, float tensor_scale,
                              uint8_t* codes_dev, uint8_t* block_scales_dev, void* stream);
qpn_status qpn_quantize_fp8(const float* w_dev, int64_t n, int64_t k,
                            uint8_t* codes_dev, float* row_scales_dev, void* stream);

/*
 * Offline FP8 -> NVFP4 conversion ([P3] "v1.0 got us here. v1.1 removes its
 * last compromise.": the first version served the checkpoint's FP8 regions
 * by converting them to NVFP4). The FP8 weight (codes uint8 [n][k], no NaN
 * codes; fp32 row scales [n]) stands for w = E4M3(c) * s_n, one fp32
 * multiply per element; those values get the recipe of qpn_quantize_nvfp4.
 *   qpn_fp8_absmax: out_dev[0] = max |w| (0 for an empty weight), for the
 *     tensor scale qpn_nvfp4_tensor_scale(amax).
 *   qpn_requantize_fp8_nvfp4: with that tensor scale (finite, > 0) ->
 *     codes_dev uint8 [n][k/2] and block_scales_dev uint8 [n][k/16] as
 *     qpn_quantize_nvfp4 writes them; pack with qpn_pack_nvfp4.
 * k % 16 == 0. The conversion loses accuracy (E2M1 keeps 1 mantissa bit
 * where E4M3 keeps 3), which is why the pages' second version kept FP8.
 */
qpn_status qpn_fp8_absmax(const uint8_t* codes_dev, const float* row_scales_dev, int64_t n, int64_t k,
                          float* out_dev, void* stream);
qpn_status qpn_requantize_fp8_nvfp4(const uint8_t* fp8_codes_dev, const float* row_scales_dev, int64_t n,
                                    int64_t k, float tensor_scale, uint8_t* codes_dev, uint8_t* block_scales_dev,
                                    void* stream);

/* Device workspace qpn_gemm needs for this weight and row count (0 if none).
 * When K is split over several workgroups the workspace holds one arrival
 * counter per n-tile, an 8 KiB control block (the key slots of
 * qpn_gemm_argmax) and fp32 partial sums. The counters and the control block
 * sit at offsets that depend only on the weight, so one workspace serves
 * calls with any m and epilogue once it is as large as the largest need
 * among them (this and qpn_workspace_bytes_tuned per call; the need is not
 * monotonic in m: a launch without a K split needs none). They must be zero
 * before the first call that uses the workspace (allocate it zeroed); every
 * call leaves them zero again. Calls that run at the same time must not
 * share a workspace. */
size_t qpn_workspace_bytes(const qpn_weight* w, int32_t m);

/*
 * The hot path ([P3] "What I actually built": weights stay compressed while
 * they stream from HBM and each fragment becomes fp16 in registers, with no
 * dequantize-to-fp16 pass).
 *   x_dev     fp16 [m][w->k] row-major, 16-byte aligned.
 *   y_dev     fp16 [m][w->n] row-major output (fully overwritten), 2-byte aligned.
 *   m         0..QPN_MAX_M activation rows (0 or n == 0: nothing to do).
 *   workspace device scratch of at least qpn_workspace_bytes(w, m) bytes
 *             (NULL allowed when that is 0); 16-byte aligned; see above.
 * Accumulation is fp32 over exactly decoded fp16 weights; the result is
 * rounded once to fp16. Deterministic: the same inputs give the same bits.
 * Never synchronizes the stream. Packed weights of 2 GiB or more return
 * QPN_ERR_UNSUPPORTED.
 */
qpn_status qpn_gemm(const void* x_dev, const qpn_weight* w, void* y_dev, int32_t m,
                    void* workspace_dev, size_t workspace_bytes, void* stream);

/*
 * An explicit launch shape for qpn_gemm_tuned (tuning sweeps), and the
 * epilogue. 0 in any shape field means "choose automatically".
 *   split_k          cut K into this many ranges over workgroups (their fp32
 *                    partials are added by the last workgroup to finish);
 *   waves_per_group  4 or 8 wavefronts per workgroup; or 9 for the uneven
 *                    grid: whole_groups workgroups share the n-tiles, one K
 *                    slice each and no K split, the first (n-tiles mod
 *                    whole_groups) of them taking one n-tile more than the
 *                    others, at most 9. It takes NVFP4 weights,
 *                    QPN_EPILOGUE_NONE or QPN_EPILOGUE_F32, the matrix
 *                    cores, depth 2 or 3,
 *                    k_slices and split_k 0 or 1, and 1 <= whole_groups <=
 *                    n-tiles; else QPN_ERR_UNSUPPORTED. With whole_groups =
 *                    the CU count every CU streams the same number of tiles
 *                    to within one, without a split-K tail (qpn_gemm and
 *                    qpn_gemm_f32 pick it for the 34816 x 5120 gate_up
 *                    matrix from 9 rows on);
 *   depth            2, 3, 4, 6 or 8 units of the weight stream in flight per
 *                    wavefront;
 *   k_slices         1, 2, 4 or 8 (at most waves_per_group): wavefronts of
 *                    one workgroup that split one n-tile's K range and add
 *                    their results through LDS;
 *   epilogue         QPN_EPILOGUE_NONE (y as in qpn_gemm), QPN_EPILOGUE_SWIGLU
 *                    (see qpn_gemm_swiglu), QPN_EPILOGUE_F32 (y_dev fp32, see
 *                    qpn_gemm_f32) or QPN_EPILOGUE_ARGMAX (only with
 *                    qpn_gemm_argmax and the workspace / plan queries);
 *   x_stage          how the activation rows reach LDS (0 = automatic):
 *                    QPN_X_STAGE_FULL copies the workgroup's whole K range
 *                    before the weight stream starts (one barrier; LDS of
 *                    2 * m * range bytes, so a long K at large m must be
 *                    split); QPN_X_STAGE_RING keeps three 256-element units
 *                    per K slice in a ring refilled one unit ahead of the
 *                    stream (one barrier per unit; LDS of
 *                    1584 * m * k_slices bytes; needs depth 2..4,
 *                    k_slices * m <= 4 * waves_per_group and 2 * m * k < 2^31);
 *   whole_groups     with split_k > 1, the number of leading groups of
 *                    n-tiles (waves_per_group / k_slices tiles each) that
 *                    still take all of K in one workgroup; only the others
 *                    are split (more than there are = none split). 0: the
 *                    tuned value when split_k is automatic, else all split.
 *                    Whole groups first, then the split ones' ranges: a grid
 *                    that fills the CUs evenly and leaves a short tail of
 *                    small workgroups. A full stage must hold all of K.
 *                    With waves_per_group = 9 it is instead the workgroup
 *                    count of the uneven grid (required there);
 *   valu_dot         0: the matrix cores (v_mfma_f32_16x16x32_f16, the
 *                    default); 1: the VALU packed-dot path instead
 *                    (v_dot2c_f32_f16: each lane adds its row's weight pairs
 *                    times the m activation rows, so its cost grows with m).
 *                    It takes m <= 4, QPN_EPILOGUE_NONE, depth 2..4 and a full
 *                    stage (automatic stage = full; a ring returns
 *                    QPN_ERR_UNSUPPORTED). It exists to measure the MFMA
 *                    choice against; qpn_gemm never picks it. Other values
 *                    return QPN_ERR_INVALID_ARG.
 *   block_columns    one activation row (m == 1) of NVFP4 weights with a full
 *                    stage: 1 on (QPN_ERR_UNSUPPORTED where not possible),
 *                    0 (automatic) and 2 off; qpn_gemm never picks it. The
 *                    matrix cores' 16 output columns then carry the 16
 *                    K-blocks of each 256-element unit instead of activation
 *                    rows (the B operand is the activation row laid out
 *                    block-diagonally), so each E4M3 block scale multiplies
 *                    one fp32 block sum per weight row instead of every
 *                    decoded weight. Other values return QPN_ERR_INVALID_ARG.
 * The result bits depend on split_k, whole_groups, k_slices, valu_dot and
 * block_columns (the summation order), not on the other fields; the uneven
 * grid sums like any launch with k_slices 1 and split_k 1.
 */
typedef enum {
  QPN_EPILOGUE_NONE = 0,
  QPN_EPILOGUE_SWIGLU = 1,
  QPN_EPILOGUE_ARGMAX = 2,
  QPN_EPILOGUE_F32 = 3
} qpn_epilogue;
typedef enum { QPN_X_STAGE_AUTO = 0, QPN_X_STAGE_FULL = 1, QPN_X_STAGE_RING = 2 } qpn_x_stage;

typedef struct {
  int32_t split_k;
  int32_t waves_per_group;
  int32_t depth;
  int32_t k_slices;
  int32_t epilogue;
  int32_t x_stage;
  int32_t whole_groups;
  int32_t valu_dot;
  int32_t block_columns;
} qpn_launch;

/* qpn_gemm with an explicit launch shape (NULL = automatic). A shape that
 * is not possible (an activation stage that does not fit in LDS, a ring
 * outside its limits) returns QPN_ERR_UNSUPPORTED. */
qpn_status qpn_gemm_tuned(const void* x_dev, const qpn_weight* w, void* y_dev, int32_t m,
                          void* workspace_dev, size_t workspace_bytes,
                          const qpn_launch* launch, void* stream);
/* Workspace for qpn_gemm_tuned with this launch shape (0 if none is needed
 * or the shape is not possible). */
size_t qpn_workspace_bytes_tuned(const qpn_weight* w, int32_t m, const qpn_launch* launch);

/* The launch shape qpn_gemm_tuned(w, m, launch) would use, every field
 * resolved (launch NULL = what qpn_gemm uses): written to *resolved. Returns
 * QPN_ERR_UNSUPPORTED for a shape that is not possible; no device work. */
qpn_status qpn_gemm_plan(const qpn_weight* w, int32_t m, const qpn_launch* launch, qpn_launch* resolved);

/*
 * qpn_gemm for callers that cannot allocate device memory (code under HIP
 * graph capture, tight serving loops, harnesses that forbid allocation): the
 * same launch and kernels as qpn_gemm with no workspace argument. The split-K
 * counters and fp32 partial sums go to a scratch array the library holds in
 * device memory, one per GPU it runs on, of QPN_NOALLOC_SCRATCH_BYTES bytes,
 * kept until the process ends. The call allocates nothing.
 *   Arguments and results as in qpn_gemm.
 *   A shape whose launch needs more scratch than that (qpn_workspace_bytes
 *   above QPN_NOALLOC_SCRATCH_BYTES) returns QPN_ERR_BUFFER_TOO_SMALL and
 *   enqueues nothing; QPN_ERR_HIP if the scratch address cannot be taken.
 * Every call on one GPU shares that GPU's scratch: calls that may overlap on
 * one GPU (other streams, other threads) race and must not be issued; calls
 * in order on one stream are safe, and each leaves the counters at zero for
 * the next.
 */
#define QPN_NOALLOC_SCRATCH_BYTES (16u << 20)
qpn_status qpn_gemm_noalloc(const void* x_dev, const qpn_weight* w, void* y_dev, int32_t m, void* stream);

/*
 * The gate_up GEMM of a gated MLP with SwiGLU fused into its epilogue. The
 * weight is the row concatenation [W_gate; W_up] (w->n = 2 * F, F a multiple
 * of 16); with g = x W_gate^T and u = x W_up^T (fp32 accumulators, scaled),
 * the output is
 *   h_dev     fp16 [m][F] row-major, h = silu(g) * u, silu(g) = g / (1 + e^-g),
 *             rounded once to fp16 (fully overwritten), 2-byte aligned,
 * so the N x M gate_up result never goes to memory. Other arguments as in
 * qpn_gemm; the workspace is qpn_workspace_bytes_tuned(w, m, launch) with
 * launch->epilogue = QPN_EPILOGUE_SWIGLU. w->n not a multiple of 32 returns
 * QPN_ERR_INVALID_ARG. (The SwiGLU between the two projections is not
 * described on the pages; this is the common fused gate_up form.)
 */
qpn_status qpn_gemm_swiglu(const void* x_dev, const qpn_weight* w, void* h_dev, int32_t m,
                           void* workspace_dev, size_t workspace_bytes, void* stream);

/*
 * qpn_gemm with an fp32 output: the scaled fp32 accumulators, not rounded.
 * This is what a row-parallel tensor-parallel rank hands to its all-reduce
 * ([P3] "This is a server, not a GEMM screenshot": the pages run 4-way
 * tensor parallelism): with K split over ranks each rank's y is a partial
 * sum, and rounding it to fp16 before the sum would round every rank's
 * part (and could overflow fp16 where the total does not).
 *   y_dev     fp32 [m][w->n] row-major output (fully overwritten), 4-byte
 *             aligned.
 * Other arguments, the workspace and the launch shape as in qpn_gemm, with
 * the same accumulators: y is the scaled accumulator rounded once to fp32,
 * where qpn_gemm rounds it once to fp16. Rounding this y to fp16 so gives
 * qpn_gemm's bits except where y lies exactly halfway between two fp16
 * values.
 * qpn_gemm_tuned with launch->epilogue = QPN_EPILOGUE_F32 is the same call
 * with an explicit shape.
 */
qpn_status qpn_gemm_f32(const void* x_dev, const qpn_weight* w, float* y_dev, int32_t m,
                        void* workspace_dev, size_t workspace_bytes, void* stream);

/*
 * A greedy output head: the GEMM with, per activation row, the index and the
 * value of its largest logit, so the m x N logits never go to memory (for an
 * lm_head at N = 151936 that is 0.3-4.9 MB per step). The logits are the
 * scaled fp32 accumulators (not rounded to fp16); among equal logits the
 * smallest index wins, so the result is deterministic.
 *   idx_dev   int32 [m] output, 4-byte aligned.
 *   val_dev   fp32 [m] output (the largest logits), or NULL.
 *   launch    NULL or a launch shape (its epilogue field 0 or
 *             QPN_EPILOGUE_ARGMAX); other arguments as in qpn_gemm_tuned.
 * The workspace is always needed: qpn_workspace_bytes_tuned(w, m, launch)
 * with launch->epilogue = QPN_EPILOGUE_ARGMAX. It holds 64 x 16 key slots
 * (8 KiB) besides any split-K counters; all must be zero before the first
 * call, and every call leaves them zero. The call enqueues two kernels: the
 * GEMM, whose workgroups fold their best (logit, index) keys into the slots
 * with device-scope atomic max, and a one-workgroup kernel that reads the
 * slots, writes idx and val, and clears them.
 * (The pages speak of a native 4-bit lm_head; folding the greedy argmax into
 * it is a reading of how a verify step uses that head.)
 */
qpn_status qpn_gemm_argmax(const void* x_dev, const qpn_weight* w, int32_t* idx_dev, float* val_dev, int32_t m,
                           void* workspace_dev, size_t workspace_bytes, const qpn_launch* launch, void* stream);

/*
 * The MLP of a decoder layer: h = SwiGLU(x W_gate^T, x W_up^T) as in
 * qpn_gemm_swiglu, then y = h W_down^T as in qpn_gemm ([P3] "What I actually
 * built": the dense layer's gate_up and down projections, streamed back to
 * back), as two GEMM launches or, on request, as ONE launch in which the
 * down workgroups start streaming their weights while the last gate_up
 * workgroups still run and read h as soon as all of it is written.
 *   gate_up   [W_gate; W_up], n = 2 * F (F a multiple of 16), k = K.
 *   down      n = N, k = F.
 *   x_dev     fp16 [m][K], 16-byte aligned.
 *   h_dev     fp16 [m][F] output (the SwiGLU values, as qpn_gemm_swiglu
 *             writes them), 16-byte aligned.
 *   y_dev     fp16 [m][N] output (as qpn_gemm on h), 2-byte aligned.
 *   launch    NULL (automatic) or a launch shape; `launches` (host, may be
 *             NULL) gets the number of kernels enqueued, 1 or 2.
 * Automatic is two launches: on the 27B shapes the one launch measured
 * level with them at m = 1 and slower at m = 2. The one-launch form
 * (launch->fused = 1) needs NVFP4 weights and a grid that fits on the device
 * at once (the call checks the occupancy; the down workgroups stage their K
 * range of h whole, so more rows cut down's K into more ranges and enlarge
 * the grid), else the call returns QPN_ERR_UNSUPPORTED with nothing
 * enqueued. Both forms are within the GEMMs' bounds; y is the down GEMM's on
 * the h the call writes, bit for bit, and where the gate_up launch shapes
 * agree (the 27B shapes at m = 1) h is too but for rare 1-ulp differences of
 * the epilogue's fp32 rounding.
 * The workspace is
 * qpn_mlp_workspace_bytes(gate_up, down, m, launch), 16-byte aligned: the two
 * GEMMs' workspaces, a 128-byte flag line per down workgroup of the
 * one-launch form, and a 256-byte control block at its end (an arrival
 * counter, then at byte 8 a status word the kernel sets to 1, and never
 * clears, if a wait ran past its bound, in which case that call's results
 * are undefined). All of it must be zero before the first call; every call
 * leaves the rest zero. Calls that share a workspace must not run at the
 * same time, and a one-launch call should not share the device with other
 * work that could hold the CUs its gate_up workgroups need (the bounded
 * waits then end the call with the status word set).
 */
typedef struct {
  int32_t fused;        /* 0 automatic (two launches: the faster or equal form as measured),
                           1 one launch or QPN_ERR_UNSUPPORTED, 2 two launches */
  int32_t down_depth;   /* one launch: weight units in flight per down wavefront: 0 auto, 2, 3, 4, 6, 8 */
  int32_t stream_after; /* one launch: gate_up workgroups finished before the down workgroups issue
                           their first weight units: 0 auto (half of them), -1 at once, else the count */
  int32_t reserved;     /* 0 */
} qpn_mlp_launch;

size_t qpn_mlp_workspace_bytes(const qpn_weight* gate_up, const qpn_weight* down, int32_t m,
                               const qpn_mlp_launch* launch);
qpn_status qpn_mlp(const void* x_dev, const qpn_weight* gate_up, const qpn_weight* down, void* h_dev, void* y_dev,
                   int32_t m, void* workspace_dev, size_t workspace_bytes, const qpn_mlp_launch* launch,
                   int32_t* launches, void* stream);

/*
 * Read-only streaming kernel that measures the HBM read ceiling the GEMM is
 * compared against ([P3] "What I actually built": bandwidth is quoted against
 * a measured read-only ceiling). Reads `bytes` (a multiple of 16) from buf_dev
 * with 16-byte non-temporal loads, grid-stride, on `grid` workgroups of 256
 * threads (grid 0 = automatic; qpn_read_ceiling_grid() gives that count),
 * `loads` loads in flight per thread (2, 4 or 8; 0 = 4), and writes one
 * word per wavefront to sink_dev (uint32 [4 * grid]). A sweep over grid and
 * loads gives the best plain read a launch of that size can make.
 */
qpn_status qpn_read_ceiling(const void* buf_dev, size_t bytes, uint32_t* sink_dev,
                            int32_t grid, int32_t loads, void* stream);
int32_t qpn_read_ceiling_grid(void);

#ifdef __cplusplus
}
#endif

#endif /* QPN_H */
