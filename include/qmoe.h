/*
 * qmoe.h -- C ABI of the MI355X (gfx950) low-bit quantized MoE expert FFN.
 *
 * One MoE layer computes, for T tokens x[t] (hidden size H):
 *
 *   route    ids[t][0..k-1] = the k experts with the largest router logits
 *            (ties to the lower expert index, ordered by descending logit);
 *            w[t][j] = softmax of those k logits, so sum_j w[t][j] = 1 (or,
 *            as an option, the selected entries of the softmax over all E
 *            logits: qmoe_topk_weights).
 *   expand   tokens grouped by expert: per-expert row counts, exclusive
 *            offsets and a stable row list of flat slots r = t*k + j.
 *   FC1      a = W1[e] x[t] (+ an optional per-expert bias), W1[e] is [2I][H]
 *            with gate/up rows interleaved: row 2i is gate_i, row 2i+1 is up_i.
 *   SwiGLU   h_i = silu(a[2i]) * a[2i+1],  silu(g) = g / (1 + exp(-g))
 *            (or ReLU, h_i = max(a_i, 0) over a single [I][H] FC1: qmoe_activation).
 *   FC2      o = W2[e] h (+ an optional per-expert bias), W2[e] is [H][I].
 *   combine  y[t] = sum_j w[t][j] * o_(t,j), summed in fp32, rounded once
 *            (nearest-even) to the activation dtype.
 *
 * Weights are block-quantized: every B consecutive weights of a row share a
 * 16-bit scale s (and, for affine formats, a bias b); w = s*q or w = s*q + b.
 *
 * Where each part comes from on the pages:
 *   - onnxruntime pull request 33005 ("[CUDA] Enable SM80+ FP16/BF16 mixed
 *     INT2/INT4 QMoE prefill by default"), Description: the stage order
 *     (routing and expert map, rows expanded by expert, FC1, SwiGLU, FC2,
 *     top-k weighted finalize), an aligned per-call workspace ordered on the
 *     stream, prepacked weights with transposed scales; Current Scope:
 *     FP16/BF16 activations, symmetric codes without zero points, block 64,
 *     interleaved fused SwiGLU, dimensions divisible by 64, at most 256
 *     experts, bounded int-sized routed-row counts, and an error instead of
 *     a larger allocation when scratch does not fit.
 *   - MLX issue 3852 ("2-bit quantized_matmul loses its size advantage over
 *     4-bit at M >= 3"), repro and closing remarks: the dense call
 *     quantized_matmul(x, wq, scales, biases, transpose=True, group_size,
 *     bits) with W as [N][K], affine groups of 128, ternary as affine.
 *   - onnx-genai pull request 1167 ("QMoE gate/up SwiGLU expert-GEMV
 *     occupancy lever"): the fused gate/up SwiGLU expert GEMV and the
 *     separate down-projection GEMV; Parity: f16, bf16 and f32 activations
 *     on the decode GEMV.
 *
 * Canonical input format (what qmoe_prepack / qmoe_linear_prepack read):
 *   codes   [E][N][K*bits/8] bytes; within a byte, fields run LSB-first along
 *           K.  Field u maps to the code q by the qtype:
 *             SYM_INT4     q = u - 8        in [-8, 7]     w = s*q
 *             SYM_INT2     q = u - 2        in [-2, 1]     w = s*q
 *             TERNARY      q = u - 1        in {-1, 0, 1}  w = s*q (u = 3 invalid)
 *             AFFINE_INT2  q = u            in [0, 3]      w = s*q + b
 *             AFFINE_INT4  q = u            in [0, 15]     w = s*q + b
 *   scales  [E][N][K/B] 16-bit patterns of scale_dtype; biases likewise
 *           (affine formats only).
 *
 * Conventions:
 *   - Every pointer argument to a compute call is a DEVICE pointer on the
 *     current HIP device unless stated otherwise; descriptors and size
 *     outputs are host pointers.  `stream` is a hipStream_t (NULL = the
 *     default stream).
 *   - The caller allocates and owns every buffer.  The library never
 *     allocates, frees or synchronizes inside qmoe_forward, qmoe_route and
 *     qmoe_linear; it holds no per-call state between calls.
 *   - Validation runs before any launch: a non-OK status means nothing was
 *     enqueued.  Launch failures return QMOE_ERR_DEVICE.  qmoe_last_error()
 *     gives a thread-local message for the last non-OK status.
 *   - Alignment: packed buffers and workspaces 256 B; x and y 16 B; logits 4 B.
 */
#ifndef QMOE_H_
#define QMOE_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define QMOE_ABI_VERSION 9

typedef enum qmoe_status {
  QMOE_OK = 0,
  QMOE_ERR_INVALID_ARGUMENT = 1, /* null/misaligned pointer, inconsistent shape, bad code */
  QMOE_ERR_UNSUPPORTED = 2,      /* valid request outside what is built (see each call) */
  QMOE_ERR_WORKSPACE_TOO_SMALL = 3,
  QMOE_ERR_DEVICE = 4            /* a HIP call or launch failed */
} qmoe_status;

typedef enum qmoe_dtype {
  QMOE_DTYPE_BF16 = 0,
  QMOE_DTYPE_F16 = 1,
  QMOE_DTYPE_F32 = 2 /* activations only (see qmoe_layer_desc) */
} qmoe_dtype;

typedef enum qmoe_qtype {
  QMOE_QTYPE_SYM_INT4 = 0,
  QMOE_QTYPE_SYM_INT2 = 1,
  QMOE_QTYPE_TERNARY = 2,
  QMOE_QTYPE_AFFINE_INT2 = 3,
  QMOE_QTYPE_AFFINE_INT4 = 4,
  QMOE_QTYPE_TERNARY_B3 = 5 /* ternary in base 3, five weights per byte (MLX issue 3852, closing
                               remarks: a denser ternary storage of about 1.6 bits per weight):
                               each block of B weights takes ceil(B/5) bytes, weight i of the block
                               is base-3 digit i mod 5 (least significant first) of byte i/5,
                               q = digit - 1; a byte holding more than its digits allow (>= 243,
                               or >= 3^(B mod 5) for a block's last byte) is invalid.  Gathered
                               channels only (fc1 and fc2 both); the MoE and dense calls return
                               QMOE_ERR_UNSUPPORTED. */
} qmoe_qtype;

typedef enum qmoe_path {
  QMOE_PATH_AUTO = 0,    /* GEMV kernels when every expert row count can be <= 16 (T <= 16), or in
                            row tiles of <= 16 rows for a layer with no grouped path; else grouped */
  QMOE_PATH_GEMV = 1,    /* register-accumulator GEMV kernels (needs T <= 16, or row tiles) */
  QMOE_PATH_GROUPED = 2  /* grouped MFMA kernels over expert row tiles */
} qmoe_path;

/* One quantized matrix W [rows][cols] = [N][K]. */
typedef struct qmoe_qmatrix_desc {
  int32_t qtype;       /* qmoe_qtype */
  int32_t block;       /* weights per scale along K: 64 or 128 */
  int32_t scale_dtype; /* QMOE_DTYPE_BF16 or QMOE_DTYPE_F16 */
  int32_t reserved;    /* must be 0 */
  int64_t rows;        /* N, a positive multiple of 64 */
  int64_t cols;        /* K, a positive multiple of 64 and of block */
} qmoe_qmatrix_desc;

/* Expert FFN activation.  SWIGLU: FC1 is [2I][H] with interleaved gate/up
   rows and h_i = silu(a[2i]) * a[2i+1].  RELU: the single-matrix FFN of the
   Switch Transformer family (QMoE gotcha page, on the SwitchTransformer
   expert shapes): FC1 is [I][H] and h_i = max(a_i, 0). */
typedef enum qmoe_activation {
  QMOE_ACT_SWIGLU = 0,
  QMOE_ACT_RELU = 1
} qmoe_activation;

/* One MoE layer.  fc1 must be [2*inter][hidden] (SWIGLU) or [inter][hidden]
   (RELU), fc2 [hidden][inter]. */
typedef struct qmoe_layer_desc {
  int32_t num_experts; /* E in [1, 256] */
  int32_t hidden;      /* H */
  int32_t inter;       /* I */
  int32_t act_dtype;   /* QMOE_DTYPE_BF16, F16 or F32: x and y.  F32 (onnx-genai pull request
                          1167, Parity: f16/bf16/f32 decode) is NOT fp32 arithmetic on x: on the
                          GEMV path x enters the matrix cores as two bf16 parts, hi = RNE(x) and
                          lo = RNE(x - hi), about 16 of x's 24 significand bits (relative error
                          below 2^-16 per element); on the grouped path as two f16 parts of
                          x 2^r (r a per-row power of two), about 22 bits.  The products and
                          sums are fp32; y is rounded once to f32.  No expert biases
                          (QMOE_ERR_UNSUPPORTED). */
  qmoe_qmatrix_desc fc1;
  qmoe_qmatrix_desc fc2;
  int32_t activation;  /* qmoe_activation */
  int32_t reserved;    /* must be 0 */
} qmoe_layer_desc;

/* Routing weights of the k selected experts of a token (top-k by logit, ties
   to the lower expert index).  RENORMALIZED: the softmax over the k selected
   logits, so the weights sum to 1.  SOFTMAX_ALL: the softmax over all E
   logits, of which the k selected probabilities are used as they are (for
   k = 1, the top probability of a Switch-style router); they sum to at most 1. */
typedef enum qmoe_topk_weights {
  QMOE_TOPK_RENORMALIZED = 0,
  QMOE_TOPK_SOFTMAX_ALL = 1
} qmoe_topk_weights;

/* Optional controls and diagnostics of qmoe_forward_ex.  Zero-initialise. */
typedef struct qmoe_forward_opts {
  int32_t path;      /* qmoe_path */
  int32_t reserved;  /* must be 0 */
  float *h_out;      /* optional device [T*k][I] fp32: SwiGLU output per slot, slot order t*k+j */
  int32_t *ids_out;  /* optional device [T][k]: routed expert ids */
  float *w_out;      /* optional device [T][k]: routing weights */
  int32_t *counts_out; /* optional device [E]: rows routed to each expert */
  void **events;     /* optional host array of hipEvent_t created with timing: events[2i] /
                        events[2i+1] receive the begin timestamp of the first kernel and the
                        end timestamp of the last kernel of stage i of the plan's stage list
                        (the kernels' own dispatch timestamps, as a kernel trace reports them);
                        a stage whose pair is incomplete is not timed */
  int32_t num_events; /* entries in `events` (0 = none) */
  int32_t reserved2;  /* must be 0 */
  /* Optional per-expert output biases, device, 16-bit values of the layer's
     act_dtype (onnxruntime pull request 33005, Description: an expert bias
     applied after FC1 and before the SwiGLU, and the FC2 bias in the top-k
     finalize).  fc1_bias [E][2I] is in FC1's interleaved row order (row 2i
     gate, 2i+1 up) and is added to FC1's output before the SwiGLU; fc2_bias
     [E][H] is added to each expert's FC2 output before that output is scaled
     by its routing weight.  Null: no bias. */
  const void *fc1_bias;
  const void *fc2_bias;
  int32_t topk_weights; /* qmoe_topk_weights: how the routing weights are formed */
  int32_t reserved3;    /* must be 0 */
  /* Row tiling under a workspace budget (onnxruntime pull request 33005,
     Current Scope: the prefill is row-tiled to keep its temporary scratch
     within a budget, the tile size halved until it fits, full and final
     partial tiles sized explicitly).  0: no limit.
     The tokens run in consecutive tiles of R rows and a final tile of the
     rest.  R starts at T and is halved (rounding up) while it exceeds the
     row bound of the path -- 16 rows when the layer has no grouped path (an
     affine format with more than 80 blocks per row), with
     or without a limit, or when a call with a limit is pinned to the GEMV
     path -- then while the workspace of a full tile or of the final tile
     exceeds workspace_limit bytes.  Each tile takes its own path (auto: by
     its row count).  ws_bytes must hold the tile workspace that
     qmoe_forward_plan reports.  counts_out and events need a single tile
     (QMOE_ERR_UNSUPPORTED otherwise); ids_out, w_out and h_out are written
     as without tiling.  If one row does not fit: QMOE_ERR_WORKSPACE_TOO_SMALL.
     Must not be negative. */
  int64_t workspace_limit;
  /* Configurable SwiGLU (onnxruntime pull request 33005, Description: a
     configurable SwiGLU follows the expert bias; the page names no
     parameters).  swiglu_params = 0: the plain h = silu(g) * u.  1: with
     swiglu_limit > 0 the gate is clipped from above, g = min(g, limit), and
     the up value to [-limit, limit]; then h = g * sigmoid(swiglu_alpha * g) *
     (u + swiglu_beta).  alpha and beta finite, limit finite and >= 0 (0: no
     clipping); SWIGLU layers only (INVALID_ARGUMENT otherwise). */
  int32_t swiglu_params;
  float swiglu_alpha;
  float swiglu_beta;
  float swiglu_limit;
} qmoe_forward_opts;

/* Host-side description of what a forward call would launch (diagnostic). */
typedef struct qmoe_plan {
  int32_t path;          /* the path actually taken */
  int32_t num_launches;  /* kernels enqueued per call */
  int32_t gemv_mmax;     /* GEMV path: bound on the rows of one expert the kernels are built for */
  int32_t gemv_fc1_waves;  /* GEMV path: waves per workgroup (K split) of FC1 */
  int32_t gemv_fc2_waves;
  int32_t max_active;    /* upper bound of active experts the grids are sized for */
  int64_t workspace_bytes;
  char kernels[256];     /* stage names in launch order, comma separated; a stage is one
                            kernel except "route" (one or two kernels); with row tiling,
                            those of a full tile */
  int32_t row_tile;      /* rows of a full tile (T without tiling) */
  int32_t num_tiles;     /* tiles run one after another (1 without tiling); num_launches and
                            workspace_bytes cover all of them */
} qmoe_plan;

/* ABI version (QMOE_ABI_VERSION) and a thread-local message for the last non-OK status. */
int32_t qmoe_abi_version(void);
const char *qmoe_last_error(void);

/* ------------------------------------------------------------------ MoE --- */

/* Bytes of the opaque prepacked buffer for `desc` (host call, no device work).
 * Errors: INVALID_ARGUMENT (null, inconsistent shapes), UNSUPPORTED (qtype,
 * block not in {64,128}, E > 256, dims not multiples of 64, f32 scales). */
qmoe_status qmoe_prepacked_size(const qmoe_layer_desc *desc, size_t *bytes);

/* Rearranges canonical codes and scales (device pointers, layout above) into
 * the prepacked gfx950 layout in `dst` (device, >= qmoe_prepacked_size bytes,
 * 256-B aligned).  Biases are required for affine formats and must be NULL
 * otherwise.  Offline call: it synchronizes `stream` to read back a device
 * error word and returns INVALID_ARGUMENT if a ternary field holds 3.  The
 * sources may be freed afterwards; `dst` is the only persistent artefact. */
qmoe_status qmoe_prepack(const qmoe_layer_desc *desc,
                         const void *fc1_codes, const void *fc1_scales, const void *fc1_biases,
                         const void *fc2_codes, const void *fc2_scales, const void *fc2_biases,
                         void *dst, size_t dst_bytes, void *stream);

/* Runtime scales (onnxruntime pull request 33005, Description: the packed
 * weights and transposed scales are reused, runtime scale inputs included).
 * Rewrites only the scale (and affine bias) sections of a buffer made by
 * qmoe_prepack for the same desc, from canonical scales and biases in the
 * layout above (device pointers; biases required for affine formats and NULL
 * otherwise); the codes are left as they are.  Stream-ordered, no
 * synchronisation: forward calls enqueued after it on `stream` use the new
 * scales, and calls on other streams must be ordered by the caller.  The
 * sources may be freed once the stream has passed this call. */
qmoe_status qmoe_prepack_scales(const qmoe_layer_desc *desc, const void *fc1_scales, const void *fc1_biases,
                                const void *fc2_scales, const void *fc2_biases, void *packed,
                                size_t packed_bytes, void *stream);

/* Worst-case workspace bytes of one forward call with T tokens and top_k
 * (host call).  top_k in [1, min(E, 16)], T >= 0, T*top_k <= INT32_MAX.
 * With row tiling (qmoe_forward_opts.workspace_limit) a call needs only the
 * tile workspace that qmoe_forward_plan reports. */
qmoe_status qmoe_workspace_size(const qmoe_layer_desc *desc, int32_t T, int32_t top_k,
                                size_t *bytes);

/* One MoE layer.  x [T][H] and y [T][H] row-major in act_dtype; logits
 * [T][E] fp32 (finite); packed from qmoe_prepack; ws of at least
 * qmoe_workspace_size bytes.  Asynchronous on `stream`; never allocates,
 * frees or synchronizes.  T = 0 returns OK without launching. */
qmoe_status qmoe_forward(const qmoe_layer_desc *desc, const void *packed, const void *x,
                         const float *logits, int32_t T, int32_t top_k, void *y,
                         void *ws, size_t ws_bytes, void *stream);

/* qmoe_forward with the options of qmoe_forward_opts: path choice,
 * diagnostic outputs, stage events, expert biases, routing-weight mode and
 * row tiling (opts may be NULL: the defaults of qmoe_forward).  UNSUPPORTED
 * if path = GEMV and T > 16 without a workspace limit, and if path = GROUPED
 * for a layer the grouped kernels do not take (an affine format with more
 * than 80 blocks per row). */
qmoe_status qmoe_forward_ex(const qmoe_layer_desc *desc, const void *packed, const void *x,
                            const float *logits, int32_t T, int32_t top_k, void *y,
                            void *ws, size_t ws_bytes, void *stream,
                            const qmoe_forward_opts *opts);

/* For callers that cannot allocate (code under HIP graph capture, tight
 * serving loops, harnesses that forbid hipMalloc): qmoe_forward with the
 * workspace taken from a fixed device array inside the library instead of a
 * caller buffer.  The array holds QMOE_NOALLOC_SCRATCH_BYTES on every GPU the
 * library runs on and stays allocated until the process ends; its device
 * address is looked up once per device on the first call made with that
 * device current.  The call allocates and frees nothing.  A call whose
 * workspace (qmoe_forward_plan's workspace_bytes) exceeds the array returns
 * QMOE_ERR_WORKSPACE_TOO_SMALL before any launch; the layer's own row tiling
 * (wide-affine layers above 16 tokens) applies as in qmoe_forward.
 * All calls on one GPU share the array and it keeps the last call's
 * contents: calls that overlap on one GPU (other streams, other threads)
 * race and must be ordered by the caller.  Everything the kernels read from
 * the workspace is written earlier in the same call, so no clearing is
 * needed between calls.  Arguments and errors otherwise as qmoe_forward. */
#define QMOE_NOALLOC_SCRATCH_BYTES (32u << 20)
qmoe_status qmoe_forward_noalloc(const qmoe_layer_desc *desc, const void *packed, const void *x,
                                 const float *logits, int32_t T, int32_t top_k, void *y, void *stream);

/* Host-only: the launch plan a qmoe_forward_ex call with these arguments would follow. */
qmoe_status qmoe_forward_plan(const qmoe_layer_desc *desc, int32_t T, int32_t top_k,
                              const qmoe_forward_opts *opts, qmoe_plan *plan);

/* Routing alone, with the same kernels as the forward (bit-exact checks),
 * renormalised weights.
 * logits [T][E] fp32 -> ids [T][k] int32, w [T][k] fp32, counts [E],
 * offsets [E+1] (exclusive scan), row_list [T*k] (slots t*k+j grouped by
 * expert, ascending within an expert).  ws >= qmoe_route_workspace_size. */
qmoe_status qmoe_route_workspace_size(int32_t T, int32_t E, int32_t top_k, size_t *bytes);
qmoe_status qmoe_route(int32_t T, int32_t E, int32_t top_k, const float *logits,
                       int32_t *ids, float *w, int32_t *counts, int32_t *offsets,
                       int32_t *row_list, void *ws, size_t ws_bytes, void *stream);

/* Diagnostic: read the prepacked layout back to integer codes.  which = 1
 * for FC1 ([E][fc1.rows][H]), 2 for FC2 ([E][H][I]); codes_out int8, device. */
qmoe_status qmoe_unpack_codes(const qmoe_layer_desc *desc, const void *packed, int32_t which,
                              int8_t *codes_out, void *stream);

/* ---------------------------------------------------- gathered channels --- */

/* Top-k channel selection inside the routed experts (learnaivisually
 * explainer "MoE channel selection, top-k vs calibrated threshold", the
 * channel-selection section): for each token and each of its k routed
 * experts only the listed channels c are computed, channel c being the gate
 * row 2c and the up row 2c+1 of FC1 and column c of the down projection:
 *
 *   y_t = sum_j w_j sum_{c in list(t, j)} silu(g_c(x_t)) u_c(x_t) D_e[:, c]
 *
 * with e = the j-th routed expert and w_j its renormalised routing weight
 * (routing exactly as qmoe_forward).  Choosing the channels (scores,
 * thresholds, calibration) is the caller's; a channel listed twice counts
 * twice.
 *
 * Supported layers: activation SWIGLU, act_dtype BF16 or F16, fc1 and fc2
 * qtypes SYM_INT4, SYM_INT2 or TERNARY (no affine formats), or both
 * TERNARY_B3, no biases, hidden <= 4096 (base-3: hidden <= 2048).
 *
 * Channel-packed buffer: fc1 codes and scales exactly as for qmoe_prepack
 * (canonical [E][2I][H*bits/8] rows, [E][2I][H/block] scales), and the down
 * projection CHANNEL-MAJOR: down_codes [E][I][H*bits/8] (row c holds column c
 * of the [H][I] down matrix, quantized along H in fc2's qtype, fc2.block
 * weights per block) and down_scales [E][I][H/fc2.block] in fc2.scale_dtype.
 * TERNARY_B3 rows hold (H/B) * ceil(B/5) bytes; the packed buffer keeps each
 * of their blocks as one 4-byte aligned record of its digit bytes followed by
 * its scale (16 bytes for B = 64, 28 for B = 128).
 * All sources are device pointers; the call copies them into `dst` (256-byte
 * aligned, >= qmoe_channel_prepacked_size bytes), waits for the stream, and
 * returns QMOE_ERR_INVALID_ARGUMENT if a TERNARY field holds the value 3 or a
 * TERNARY_B3 byte is invalid. */
qmoe_status qmoe_channel_prepacked_size(const qmoe_layer_desc *desc, size_t *bytes);
qmoe_status qmoe_channel_prepack(const qmoe_layer_desc *desc, const void *fc1_codes,
                                 const void *fc1_scales, const void *down_codes,
                                 const void *down_scales, void *dst, size_t dst_bytes,
                                 void *stream);

/* Workspace bytes of qmoe_forward_channels for T tokens, top_k and list
 * length C (host call). */
qmoe_status qmoe_channel_workspace_size(const qmoe_layer_desc *desc, int32_t T, int32_t top_k,
                                        int32_t C, size_t *bytes);

/* x [T][H] (16-byte aligned) and y [T][H] in act_dtype, logits [T][E] fp32,
 * channels [T][top_k][C] int32 (device): the list of token t's j-th routed
 * expert, entries outside [0, I) unused (padding).  1 <= C <= 65536.  Each
 * output is an fp32 sum rounded once (nearest even) to act_dtype; the sum
 * order is fixed, so repeated calls give identical bits.  ws: device,
 * 256-byte aligned, >= qmoe_channel_workspace_size.  Asynchronous on
 * `stream`. */
qmoe_status qmoe_forward_channels(const qmoe_layer_desc *desc, const void *packed, const void *x,
                                  const float *logits, int32_t T, int32_t top_k,
                                  const int32_t *channels, int32_t C, void *y, void *ws,
                                  size_t ws_bytes, void *stream);

/* --------------------------------------------------------------- dense --- */

/* Dense skinny-M quantized matmul y = x W^T (MLX issue 3852, repro):
 * W [N][K] in the canonical format (E = 1), x [M][K] and y [M][N] in
 * x_dtype.  Same error rules as the MoE calls. */
qmoe_status qmoe_linear_prepacked_size(const qmoe_qmatrix_desc *desc, size_t *bytes);
qmoe_status qmoe_linear_prepack(const qmoe_qmatrix_desc *desc, const void *codes,
                                const void *scales, const void *biases, void *dst,
                                size_t dst_bytes, void *stream);
qmoe_status qmoe_linear_workspace_size(const qmoe_qmatrix_desc *desc, int32_t M, size_t *bytes);
/* path: QMOE_PATH_AUTO, GEMV (M <= 32) or GROUPED (MFMA tiles, any M >= 1);
 * x_dtype BF16 or F16. */
qmoe_status qmoe_linear(const qmoe_qmatrix_desc *desc, const void *packed, const void *x,
                        int32_t x_dtype, int32_t M, void *y, void *ws, size_t ws_bytes,
                        int32_t path, void *stream);
qmoe_status qmoe_linear_unpack_codes(const qmoe_qmatrix_desc *desc, const void *packed,
                                     int8_t *codes_out, void *stream);

/* --------------------------------------------------------- diagnostics --- */

/* Read-bandwidth probe: streams `bytes` of device memory at `src` (16-B
 * aligned, bytes a multiple of 16) with one 16-B load per lane per step in a
 * grid-stride sweep of 8 workgroups of 256 threads per compute unit, and
 * writes nothing unless the XOR of all words read equals a fixed value
 * (then one word to sink[0]; sink: device, 4 B).  Its duration over a buffer
 * much larger than the last-level cache is the achievable HBM read rate that
 * the GEMV kernels' effective bandwidth is compared with.  Asynchronous on
 * `stream`. */
qmoe_status qmoe_read_probe(const void *src, size_t bytes, uint32_t *sink, void *stream);

#ifdef __cplusplus
}
#endif

#endif /* QMOE_H_ */
