/*
 * moe.h -- C ABI of the MI355X (gfx950) small-batch W4A16 sigmoid-routed
 * mixture-of-experts layer.
 *
 * The layer (pages: "Day-0 Support for Flint on vLLM", section "Model
 * architecture"; "vLLM Flint" commentary, section "Only 14 of 49 layers
 * retain full-history KV"): a pre-norm MoE block of hidden size H whose
 * router scores 256 routed experts with a sigmoid and keeps the top 6,
 * plus one shared expert; experts are SwiGLU MLPs.  Weights are NVFP4
 * (E2M1 values, one E4M3 scale per 16 elements along K, one FP32 scale
 * per tensor) executed weight-only with BF16 activations (W4A16), or BF16.
 *
 * Conventions for every call:
 *  - Pointers marked "device" are caller-owned device memory (hipMalloc or
 *    torch tensors); the library allocates nothing, keeps no state between
 *    calls and never synchronises.
 *  - `stream` is a hipStream_t (NULL = the default stream).  Calls are
 *    stream-ordered and asynchronous and may be captured into a HIP graph.
 *  - Every argument is validated on the host before anything is enqueued;
 *    on an error nothing is launched and the return value says why.  Faults
 *    during kernel execution surface at the caller's next synchronisation.
 *  - Activations are BF16 (raw 16-bit patterns), row-major [tokens][H].
 *    Device pointers must be 16-byte aligned.  No two of the activations x
 *    and y, the optional top-k outputs and the workspace may share a byte
 *    (checked: INVALID_ARG).
 */
#ifndef MOE_H
#define MOE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum moe_status {
  MOE_OK = 0,
  MOE_ERR_INVALID_ARG = -1, /* null/misaligned pointer, bad size or shape */
  MOE_ERR_UNSUPPORTED = -2, /* valid request outside the fast path's shapes:
                               the caller should use another implementation
                               (the pages' dispatch falls back to standard
                               layers off its fast path) */
  MOE_ERR_WORKSPACE = -3,   /* workspace too small */
  MOE_ERR_HIP = -4          /* a HIP launch or runtime call failed */
} moe_status;

typedef enum moe_wtype {
  MOE_W_BF16 = 0,  /* BF16 weights, row-major [out][in] */
  MOE_W_NVFP4 = 1  /* NVFP4 weights in the runtime layout written by moe_repack_nvfp4 */
} moe_wtype;

/* Shape of one layer.  Routed and shared experts are SwiGLU MLPs:
 *   y = W_down (SiLU(W_gate x) * (W_up x)),  W_gate, W_up: [inter][hidden],
 *   W_down: [hidden][inter].
 * n_experts == 0 describes a dense SwiGLU layer: only the "shared" expert,
 * of width shared_inter, with no router (the first two layers of the model
 * use a dense MLP). */
typedef struct moe_layer_desc {
  int32_t hidden;       /* H */
  int32_t inter;        /* I, intermediate width of each routed expert */
  int32_t shared_inter; /* Is, width of the shared expert; 0 = none */
  int32_t n_experts;    /* E routed experts; 0 = dense layer */
  int32_t top_k;        /* k experts kept per token, 1..8, <= E */
  int32_t wtype;        /* moe_wtype of routed and shared expert weights */
  float norm_eps;       /* RMSNorm epsilon, used when norm_gain != NULL */
} moe_layer_desc;

/* Weights of one layer (all device pointers). */
typedef struct moe_layer_weights {
  const void *router_w;  /* [E][H] BF16 (the router stays BF16 in both modes) */
  const float *router_b; /* [E] FP32 logit offset, or NULL for zero */
  const void *w_gate;    /* E matrices [I][H], back to back */
  const void *w_up;      /* E matrices [I][H] */
  const void *w_down;    /* E matrices [H][I] */
  const float *w_scale;  /* [E][3] FP32 tensor scales (gate, up, down); NVFP4 only */
  const void *sh_gate;   /* [Is][H] */
  const void *sh_up;     /* [Is][H] */
  const void *sh_down;   /* [H][Is] */
  const float *sh_scale; /* [3] FP32 tensor scales; NVFP4 only */
  const void *norm_gain; /* [H] BF16 RMSNorm gain, or NULL: no pre-norm */
} moe_layer_weights;

/* Bytes of one NVFP4 matrix [rows][cols], in either the GGUF-like source
 * layout or the runtime layout (both hold rows*cols/2 nibble bytes plus
 * rows*cols/16 scale bytes).  Returns 0 if rows % 8 or cols % 32 != 0. */
size_t moe_nvfp4_matrix_bytes(int64_t rows, int64_t cols);

/* Load-time lossless repack of NVFP4 matrices ("Day-0 Support for Flint on
 * vLLM", section "Model architecture": the GGUF checkpoint holds NVIDIA
 * NVFP4 blocks in a different byte order and is repacked without loss at
 * load time).
 *  src: device, n_mats matrices [rows][cols] back to back, each row-major
 *       over rows, each row cols/16 blocks of 9 bytes: [E4M3 scale][8 bytes
 *       of nibbles], nibble byte j holding element j (low nibble) and
 *       element j+8 (high nibble) of the block.
 *  dst: device, same size, runtime layout: per matrix a nibble plane
 *       [rows][cols/2] with element 2i
 *       in the low and 2i+1 in the high nibble of byte i, followed by a
 *       scale plane of 16-byte tiles [rows/8][cols/32][8 rows][2 blocks].
 *  nan_scale_count: device int32 or NULL; when given, the number of NaN
 *       E4M3 scale bytes (0x7F, 0xFF) met is ADDED to it.
 * Errors: INVALID_ARG for null src/dst, src == dst, rows % 8, cols % 32,
 * non-positive sizes or misaligned pointers. */
moe_status moe_repack_nvfp4(const void *src, void *dst, int64_t rows, int64_t cols, int64_t n_mats,
                            int32_t *nan_scale_count, void *stream);

/* Inverse of moe_repack_nvfp4 (runtime layout -> GGUF-like blocks); used to
 * prove the repack lossless.  Same arguments and errors, no NaN count. */
moe_status moe_unpack_nvfp4(const void *src, void *dst, int64_t rows, int64_t cols, int64_t n_mats,
                            void *stream);

/* Runtime-layout NVFP4 matrices -> FP32 [n_mats][rows][cols], element =
 * E2M1 * E4M3 block scale * tensor_scale[m] (tensor_scale: device [n_mats]
 * FP32, or NULL for 1), through the same per-element conversions the GEMV
 * kernels use.  For inspection and tests; not on the decode path.
 * Errors: INVALID_ARG as for moe_repack_nvfp4 (dst 16-byte aligned). */
moe_status moe_dequant_nvfp4(const void *src, float *dst, int64_t rows, int64_t cols, int64_t n_mats,
                             const float *tensor_scale, void *stream);

/* Workspace bytes moe_decode_layer needs for batches up to max_batch, or 0
 * if the description is invalid or max_batch is outside the layer's batch
 * range (1..16 with NVFP4 weights, 1..8 with BF16 weights). */
size_t moe_decode_workspace_bytes(const moe_layer_desc *desc, int32_t max_batch);

/* One decode step of the layer for `batch` independent tokens: 1..16 with
 * NVFP4 weights, 1..8 with BF16 weights (the low-latency path the pages
 * describe for up to eight requests: "Day-0 Support for Flint on vLLM",
 * section "Optimizations"; batches of 9..16 run the same matrix-core
 * kernels as 2..8, the tokens filling the 16 columns of their tiles).
 *  x [batch][H] BF16 in; y [batch][H] BF16 out.
 *  Per token: xn = x, or, when norm_gain is given, xn = BF16(x /
 *  sqrt(mean(x^2) + eps) * gain), rounded once from the exact value;
 *  logits l = W_r xn + b (FP32); the top_k experts by logit (ties: lower
 *  index) are kept with weights s_j / sum s, s = sigmoid(l); each selected
 *  expert and the shared expert run as SwiGLU with FP32 accumulation and a
 *  BF16 rounding after each GEMV and after SiLU*up; the outputs are
 *  combined in FP32 as sum_j w_j y_j + y_shared and rounded to BF16; with
 *  `residual` != 0 the result is BF16(x + that).  Only the selected
 *  experts' weights are read.
 *  topk_idx [batch][k] int32, topk_w [batch][k] FP32: optional (NULL)
 *  outputs, in descending score order.
 *  ws: device workspace of ws_bytes >= moe_decode_workspace_bytes(desc,
 *  batch), 256-byte aligned; no zero-fill needed (every call writes what
 *  it reads before reading it; one token with routed experts runs one
 *  kernel per layer, whose blocks hand values to each other through sync
 *  words that the call zeroes first, in a kernel of its own), reusable
 *  across calls and batch sizes.  Its first word reports waits that gave
 *  up (moe_decode_wait_status).
 *  Concurrent calls must not share a workspace.
 * Errors: UNSUPPORTED for batch above the range (use moe_prefill_layer)
 * and for shapes the kernels do not tile (H/32, I/32 and Is/32 must each
 * be at least 2 and either a power of two or at least 64; E at most 1024;
 * Is == I when both routed and shared experts exist; batch * H * 2 <= 64
 * KiB; for batch >= 2 with routed experts, (batch + 1) * E <= 16384); INVALID_ARG for null required
 * pointers, misalignment, top_k outside 1..8 or above E, H or I not a
 * multiple of 32; WORKSPACE; HIP. */
moe_status moe_decode_layer(const moe_layer_desc *desc, const moe_layer_weights *w, const void *x,
                            int32_t batch, int32_t residual, void *y, int32_t *topk_idx, float *topk_w,
                            void *ws, size_t ws_bytes, void *stream);

/* Workspace bytes moe_decode_step needs for n_layers layers (descs[0..n))
 * and batches up to max_batch, or 0 if a description is invalid or the
 * layers' hidden sizes differ. */
size_t moe_decode_step_workspace_bytes(const moe_layer_desc *descs, int32_t n_layers, int32_t max_batch);

/* One decode step of `batch` tokens (1..16; 1..8 if a layer has BF16
 * weights) through a stack of pre-norm
 * residual layers ("vLLM Flint" commentary, section "Only 14 of 49 layers
 * retain full-history KV": 49 pre-norm layers; "Day-0 Support for Flint on
 * vLLM", section "Model architecture": layers 0 and 1 use a dense MLP, the
 * others 256 routed experts plus a shared expert):
 *   x_0 = x;  x_{i+1} = BF16(x_i + layer_i(xn_i)),  y = x_n,
 * where xn_i is BF16(RMSNorm(x_i) * gain_i) when weights[i].norm_gain is
 * set (else x_i) and layer_i is moe_decode_layer's computation (a dense
 * SwiGLU for n_experts == 0).  The activations between layers live in the
 * workspace; the call enqueues every layer's kernels back to back on
 * `stream` (capture it once into a HIP graph to replay a whole step).
 *  descs, weights: host arrays of n_layers entries (read during the call
 *  only); device pointers inside as for moe_decode_layer.
 *  x [batch][H], y [batch][H]: device BF16, disjoint from each other and
 *  from ws.
 *  ws: device, ws_bytes >= moe_decode_step_workspace_bytes(descs, n_layers,
 *  batch), 256-byte aligned; no zero-fill needed, reusable across calls;
 *  its first word reports waits that gave up in any layer of the step
 *  (moe_decode_wait_status).
 * Errors: as moe_decode_layer for each layer (the first failing layer's
 * status); INVALID_ARG for n_layers < 1 or differing hidden sizes. */
moe_status moe_decode_step(const moe_layer_desc *descs, const moe_layer_weights *weights, int32_t n_layers,
                           const void *x, int32_t batch, void *y, void *ws, size_t ws_bytes, void *stream);

/* Workspace bytes moe_decode_step_persistent needs: the step's, plus the
 * per-layer hand-over stages of one persistent launch (about 4.7 MB for
 * the full 256-expert layer at hidden 2048), or 0 as for the step. */
size_t moe_decode_step_persistent_workspace_bytes(const moe_layer_desc *descs, int32_t n_layers,
                                                  int32_t max_batch);

/* moe_decode_step with cross-layer overlap: the same computation, inputs
 * and outputs, bit for bit.  At batch 1, runs of consecutive layers with
 * routed experts and one shape (up to 24 per launch) run in one persistent
 * kernel: a layer's output is handed to the next layer's blocks inside the
 * kernel instead of across a launch, and each block requests its next
 * layer's routing-independent weights (router rows) before that hand-over
 * ("Day-0 Support for Flint on vLLM", section "Optimizations": the
 * low-latency path starts each kernel's weight loads while the previous one
 * runs).  Other layers, and runs whose blocks cannot all be resident on the
 * device at once (checked per call), run as in moe_decode_step.  The
 * persistent kernel's blocks wait on each other, so nothing else should run
 * on the GPU at the same time: a wait that is starved gives up after a
 * bounded time and reports status bit 16 (moe_decode_wait_status).
 *  ws: ws_bytes >= moe_decode_step_persistent_workspace_bytes(descs,
 *  n_layers, batch); otherwise as moe_decode_step.
 * Errors: as moe_decode_step; WORKSPACE; HIP. */
moe_status moe_decode_step_persistent(const moe_layer_desc *descs, const moe_layer_weights *weights,
                                      int32_t n_layers, const void *x, int32_t batch, void *y, void *ws,
                                      size_t ws_bytes, void *stream);

/* Dense projection on one NVFP4 matrix for a small batch: the small-batch
 * dense GEMV the pages run on the same packed NVFP4 weights as the MoE
 * kernel, for the projections outside the MoE blocks (attention QKV and
 * output, the LM head; "Day-0 Support for Flint on vLLM", section
 * "Optimizations").  For t < batch, n < rows:
 *   y[t][n] = BF16( S * sum_k W[n][k] x[t][k] ),
 * W[n][k] = E2M1 * E4M3 block scale, FP32 accumulation, one BF16 rounding.
 *  w: device, one matrix [rows][cols] in the runtime layout written by
 *     moe_repack_nvfp4; tensor_scale: device FP32 S.
 *  x [batch][cols] BF16 in; y [batch][rows] BF16 out; batch 1..8.
 * Errors: INVALID_ARG for null or misaligned pointers, rows % 8 or cols %
 * 32 != 0, batch < 1, y sharing a byte with w, x or the scale; UNSUPPORTED
 * for batch > 8 or a column count the kernels do not tile (cols/32 must be
 * at least 2 and either a power of two or at least 64; one token: cols <=
 * 32768); HIP. */
moe_status moe_gemv_nvfp4(const void *w, const float *tensor_scale, int64_t rows, int64_t cols, const void *x,
                          int32_t batch, void *y, void *stream);

/* Workspace bytes moe_prefill_layer needs for n_tokens tokens (1 ..
 * 4,194,304), or 0 if the description is invalid or n_tokens is out of
 * range.  About (k + 1) * n_tokens * (H + max(I, Is)) * 2 bytes: the
 * expert-sorted intermediate and output rows (342 MB at 8192 tokens for
 * the full layer). */
size_t moe_prefill_workspace_bytes(const moe_layer_desc *desc, int32_t n_tokens);

/* The same layer over n_tokens prompt tokens (prefill; the pages measure
 * 8192-token prefill: "Day-0 Support for Flint on vLLM", section
 * "Optimizations").  Same per-token definition, arguments and outputs as
 * moe_decode_layer, for any n_tokens in 1 .. 4,194,304: x, y [n_tokens][H];
 * topk_idx, topk_w [n_tokens][k] (optional).  The tokens are grouped by
 * selected expert (plus the shared expert over all tokens) and every
 * expert's gate/up and down projections run as matrix products on the
 * matrix cores; each token's result does not depend on the other tokens.
 *  ws: device workspace of ws_bytes >= moe_prefill_workspace_bytes(desc,
 *  n_tokens), 256-byte aligned; no zero-fill needed (every call
 *  initialises what it uses).  Concurrent calls must not share it.
 * Errors: as moe_decode_layer's shape checks (the same tiled shapes);
 * INVALID_ARG for n_tokens < 1, null or misaligned pointers, overlapping
 * buffers;
 * UNSUPPORTED for n_tokens > 4,194,304; WORKSPACE; HIP. */
moe_status moe_prefill_layer(const moe_layer_desc *desc, const moe_layer_weights *w, const void *x,
                             int32_t n_tokens, int32_t residual, void *y, int32_t *topk_idx,
                             float *topk_w, void *ws, size_t ws_bytes, void *stream);

/* moe_decode_layer with its kernels timed: events holds 6 hipEvent_t
 * handles (caller-owned, created with timing enabled) that are attached to
 * the kernel dispatches themselves, so they time the kernels' execution as
 * a kernel trace does: [0]/[1] start and stop of the router kernel, [2]/[3]
 * of the gate/up kernel, [4]/[5] of the down-and-combine kernel.  A batch of
 * one token with routed experts runs the whole layer in one kernel, timed
 * by [2]/[3]; the other pairs are then recorded back to back.  The zeroing
 * of the sync region is not timed.  For measurement of eager calls (not
 * under graph capture).  Errors: as moe_decode_layer; INVALID_ARG for a
 * null events array or handle. */
moe_status moe_decode_layer_timed(const moe_layer_desc *desc, const moe_layer_weights *w, const void *x,
                                  int32_t batch, int32_t residual, void *y, int32_t *topk_idx, float *topk_w,
                                  void *ws, size_t ws_bytes, void *const *events, void *stream);

/* Health of the last moe_decode_layer, moe_decode_step or moe_attn_decode
 * call on a workspace.  The blocks of one MoE kernel hand the router logits
 * and the SwiGLU intermediate to each other through memory, each wait
 * bounded (a wait that never ends would hang the GPU).  A wait that runs
 * out of polls ORs a bit into a status word at the start of the workspace,
 * which every call zeroes first: 1 = the logits, 2 = the intermediate, 4 =
 * the logits of a batch's routing block, 16 = a layer's input in the
 * persistent step.  moe_attn_decode writes bit 8 there
 * (a position out of range).  A non-zero word means that call's outputs
 * must not be used.  This enqueues a copy of the word into status_out (device
 * int32) on `stream`, after the calls enqueued before it.  ws == NULL: the
 * workspace of moe_decode_layer_noalloc on the current device.
 * Errors: INVALID_ARG for a null status_out or misaligned pointers; HIP. */
moe_status moe_decode_wait_status(const void *ws, int32_t *status_out, void *stream);

/* Bytes of the device array moe_decode_layer_noalloc takes its workspace
 * from (one per GPU). */
#define MOE_NOALLOC_SCRATCH_BYTES ((size_t)4 << 20)

/* moe_decode_layer for callers that cannot allocate device memory (code
 * under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc): the same computation, arguments and outputs, with no
 * workspace argument.  The workspace is a fixed array of
 * MOE_NOALLOC_SCRATCH_BYTES in the library's own device memory, one per
 * GPU, held from the library's load until the process ends; its address is
 * looked up once per device, on the first call with that device current.
 * The call allocates nothing (no hipMalloc, hipFree or allocating library
 * routine).  Every call on one GPU shares that GPU's array, which keeps the
 * last call's contents (the call zeroes what must start at zero): calls
 * that overlap in time on one GPU (other streams or threads) race and give
 * wrong results; calls ordered on one stream are safe.
 * moe_decode_wait_status(NULL, ...) reads the array's status word.
 * Errors: as moe_decode_layer; WORKSPACE when the layer at this batch needs
 * more than MOE_NOALLOC_SCRATCH_BYTES of workspace
 * (moe_decode_workspace_bytes(desc, batch); the full 256-expert layer needs
 * about 0.6 MB at batch 8), before any device call; HIP if the array's
 * address cannot be looked up. */
moe_status moe_decode_layer_noalloc(const moe_layer_desc *desc, const moe_layer_weights *w, const void *x,
                                    int32_t batch, int32_t residual, void *y, int32_t *topk_idx, float *topk_w,
                                    void *stream);

/* Host-side validation alone: what moe_decode_layer, moe_decode_step,
 * moe_prefill_layer, moe_repack_nvfp4 (and moe_unpack_nvfp4) and
 * moe_gemv_nvfp4 return for
 * these arguments before anything would be enqueued (MOE_OK: the call
 * would launch).  Nothing is launched, no pointer is dereferenced.  The
 * same checks are built into a host-only library without the HIP runtime. */
moe_status moe_check_decode_layer(const moe_layer_desc *desc, const moe_layer_weights *w, const void *x,
                                  int32_t batch, const void *y, const int32_t *topk_idx, const float *topk_w,
                                  const void *ws, size_t ws_bytes);
moe_status moe_check_decode_step(const moe_layer_desc *descs, const moe_layer_weights *weights, int32_t n_layers,
                                 const void *x, int32_t batch, const void *y, const void *ws, size_t ws_bytes);
moe_status moe_check_decode_step_persistent(const moe_layer_desc *descs, const moe_layer_weights *weights,
                                            int32_t n_layers, const void *x, int32_t batch, const void *y,
                                            const void *ws, size_t ws_bytes);
moe_status moe_check_prefill_layer(const moe_layer_desc *desc, const moe_layer_weights *w, const void *x,
                                   int32_t n_tokens, const void *y, const int32_t *topk_idx, const float *topk_w,
                                   const void *ws, size_t ws_bytes);
moe_status moe_check_repack_nvfp4(const void *src, const void *dst, int64_t rows, int64_t cols, int64_t n_mats);
moe_status moe_check_gemv_nvfp4(const void *w, const float *tensor_scale, int64_t rows, int64_t cols, const void *x,
                                int32_t batch, const void *y);

/* ------------------------------------------------------------------
 * Decode attention beside the MoE blocks ("Day-0 Support for Flint on
 * vLLM", sections "Model architecture" and "Optimizations"; "vLLM Flint"
 * commentary, section "Only 14 of 49 layers retain full-history KV"):
 * GQA with n_q query heads and n_kv K/V heads of 128 (32 and 4 in the
 * model), per-head Q/K RMSNorm, learned attention sinks, BF16 KV cache;
 * sliding-window layers (513 positions, RoPE) and full-context layers (no
 * positional encoding).  The Q/K norm, RoPE and KV write are one kernel
 * (moe_attn_prep); decode attention is moe_attn_decode.
 *
 * Caches (caller-owned device memory, one per layer, `slots` positions per
 * token row; position p lives in slot p % slots, so a window layer keeps a
 * ring and a full-context layer needs slots > every position):
 *   k_cache, v_cache: [batch][n_kv][slots / 32] tiles of 32 slots x 128
 *   BF16 (8 KiB), each tile in the lane order of the matrix-core operands
 *   that read it.  Element d of the slot at offset o (0..31) of its tile is
 *   tile element
 *     keys:   ((((o/4) % 2) * 4 + d/32) * 64 + ((d/8) % 4) * 16 + (o/8) * 4 + o % 4) * 8 + d % 8
 *     values: ((d/16) * 64 + (o/8) * 16 + d % 16) * 8 + o % 8
 *   (integer division).  moe_attn_prep writes the decoded token's slot;
 *   moe_attn_kv_write writes any positions from natural [n_kv][128] rows.
 * Positions `pos` are device int64 [batch] (graph replays may change them),
 * 0 .. 2^40 - 1.
 * ------------------------------------------------------------------ */
typedef struct moe_attn_desc {
  int32_t n_q;        /* query heads; n_q % n_kv == 0 and n_q / n_kv <= 16 */
  int32_t n_kv;       /* K/V heads, >= 1 */
  int32_t head_dim;   /* 128 (the only supported value) */
  int32_t window;     /* 0: full context; W > 0: the last W positions, the
                         current one included; W <= slots */
  int32_t rope;       /* 1: RoPE on q and k at the token's position, 0: none */
  int32_t slots;      /* cache positions per token row, a multiple of 32,
                         at most 2^24 */
  double rope_theta;  /* RoPE base (> 1) when rope == 1 */
  float norm_eps;     /* per-head RMSNorm epsilon, >= 0 */
} moe_attn_desc;

/* Q/K norm, RoPE and KV-cache write for `batch` decode tokens (1..256).
 * For token t at position p = pos[t], with D = 128 and the head vectors of
 * qkv[t] = [q heads (n_q x D) | k heads (n_kv x D) | v heads (n_kv x D)]:
 *   q', k' = per head BF16(x / sqrt(mean(x^2) + eps) * gain)   (q_gain for
 *            q heads, k_gain for k heads; one gain of D shared by the heads)
 *   with rope: element d < D/2 pairs with d + D/2, rotated by the angle
 *            p * theta^(-2d/D): (a, b) -> (BF16(a cos - b sin), BF16(b cos + a sin))
 *   q_out[t] = q' ([n_q][D]); k' and v go to slot p % slots of token row t
 *   of k_cache and v_cache (layouts above).
 *  qkv [batch][(n_q + 2 n_kv) * 128] BF16; q_gain, k_gain [128] BF16;
 *  q_out [batch][n_q][128] BF16; all device, 16-byte aligned.
 * A token whose position is negative, at least 2^40, or not below `slots`
 * in a full-context layer writes nothing to the caches and zeros to q_out.
 * Errors: INVALID_ARG for null or misaligned pointers, batch outside
 * 1..256, a bad description, q_out sharing a byte with an input or a
 * cache; UNSUPPORTED for head_dim != 128, n_q / n_kv > 16 or slots above
 * 2^24; HIP. */
moe_status moe_attn_prep(const moe_attn_desc *desc, const void *qkv, const int64_t *pos, int32_t batch,
                         const void *q_gain, const void *k_gain, void *q_out, void *k_cache, void *v_cache,
                         void *stream);

/* K and V rows into the caches (a prompt's keys and values, a cache
 * restore): for token row b < batch and i < n, the n_kv x 128 key and value
 * rows k_rows[b][i], v_rows[b][i] (BF16, keys already normed and rotated)
 * go to the slot of position pos[b * n + i] (device int64).  Positions out
 * of range (as for moe_attn_prep) are skipped; positions of one token row
 * that share a slot leave one of their rows there, unspecified which.
 *  k_rows, v_rows [batch][n][n_kv][128] BF16; all device, 16-byte aligned
 *  (pos 8-byte).
 * Errors: INVALID_ARG for null or misaligned pointers, n < 1 or above
 * 2^24, batch outside 1..256, a bad description, a cache sharing a byte
 * with an input or the other cache; UNSUPPORTED as moe_attn_prep; HIP. */
moe_status moe_attn_kv_write(const moe_attn_desc *desc, const void *k_rows, const void *v_rows, const int64_t *pos,
                             int32_t n, int32_t batch, void *k_cache, void *v_cache, void *stream);

/* Workspace bytes moe_attn_decode needs for `batch` tokens attending at
 * most max_ctx positions each (0: the layer's bound, window or slots), or 0
 * for invalid arguments.  256 bytes (the status word's line) plus, when the
 * context is long enough to be split over several blocks per head, FP32
 * partial results: batch * n_kv * chunks * (G * 128 + 2 G rounded up to 4)
 * * 4 bytes, G = n_q / n_kv (about 1 MB at one token and 100K positions). */
size_t moe_attn_workspace_bytes(const moe_attn_desc *desc, int32_t batch, int64_t max_ctx);

/* Decode attention of `batch` tokens (1..256) over their caches.  For token
 * t at p = pos[t] and query head h (K/V head g = h / (n_q / n_kv)), over
 * the positions i = lo..p (lo = 0, or p - W + 1 floored at 0 with a window)
 * read from slot i % slots:
 *   s_i = q[t][h] . k_i / sqrt(128),  m = max(s_i, sink_h),
 *   out[t][h] = BF16( sum_i e^(s_i - m) v_i / (sum_i e^(s_i - m) + e^(sink_h - m)) )
 * with sink_h = sinks[h] (a logit that joins the normalisation and
 * contributes no value), or no sink term when sinks == NULL.  FP32
 * arithmetic on the matrix cores (scores and probabilities times values),
 * one BF16 rounding.
 *  q [batch][n_q][128] BF16 (from moe_attn_prep); caches as above;
 *  sinks [n_q] FP32 or NULL; out [batch][n_q][128] BF16; all device.
 *  max_ctx: the most positions any token attends (p + 1, or W with a
 *  window), 0 = the layer's bound; it sizes the grid; a smaller bound
 *  shortens calls at short contexts.
 *  ws: device workspace of ws_bytes >= moe_attn_workspace_bytes(desc,
 *  batch, max_ctx), 256-byte aligned, no zero-fill needed.  Its first word
 *  is the call's status: bit 8 = a token's position was out of range (as for
 *  moe_attn_prep) or attends more than max_ctx positions
 *  (its output rows are zero); moe_decode_wait_status reads it.
 * Errors: INVALID_ARG for null or misaligned pointers, a bad description,
 * batch outside 1..256, max_ctx < 0 or above the layer's bound, out sharing
 * a byte with an input, a cache or ws; UNSUPPORTED as moe_attn_prep;
 * WORKSPACE; HIP. */
moe_status moe_attn_decode(const moe_attn_desc *desc, const void *q, const void *k_cache, const void *v_cache,
                           const int64_t *pos, int32_t batch, int64_t max_ctx, const float *sinks, void *out,
                           void *ws, size_t ws_bytes, void *stream);

/* moe_attn_prep then moe_attn_decode in one kernel (plus the chunk merge
 * when the context is split): the same outputs and cache writes, bit for
 * bit, with no q buffer.  Each block of the decode forms the q heads of its
 * group itself (norm and RoPE while its first cache tiles load), and the
 * block whose share of the context holds the token's position also forms
 * the new k and v, writes them to the cache and uses them from registers.
 * One launch fewer per layer than prep + decode ("Day-0 Support for Flint
 * on vLLM", section "Optimizations": the Q/K norm, RoPE and KV write fused;
 * decode attention with sinks and sliding windows).
 *  Arguments as for moe_attn_prep (qkv, pos, batch, gains, caches) and
 *  moe_attn_decode (max_ctx, sinks, out, ws: ws_bytes >=
 *  moe_attn_workspace_bytes(desc, batch, max_ctx)); status bit 8 as there.
 * Errors: as the two calls; INVALID_ARG also when out, ws or a cache shares
 * a byte with another argument. */
moe_status moe_attn_layer(const moe_attn_desc *desc, const void *qkv, const int64_t *pos, int32_t batch,
                          int64_t max_ctx, const void *q_gain, const void *k_gain, const float *sinks, void *k_cache,
                          void *v_cache, void *out, void *ws, size_t ws_bytes, void *stream);

/* Host-side validation alone of moe_attn_prep, moe_attn_kv_write,
 * moe_attn_decode and moe_attn_layer, as for the calls above. */
moe_status moe_check_attn_prep(const moe_attn_desc *desc, const void *qkv, const int64_t *pos, int32_t batch,
                               const void *q_gain, const void *k_gain, const void *q_out, const void *k_cache,
                               const void *v_cache);
moe_status moe_check_attn_kv_write(const moe_attn_desc *desc, const void *k_rows, const void *v_rows,
                                   const int64_t *pos, int32_t n, int32_t batch, const void *k_cache,
                                   const void *v_cache);
moe_status moe_check_attn_layer(const moe_attn_desc *desc, const void *qkv, const int64_t *pos, int32_t batch,
                                int64_t max_ctx, const void *q_gain, const void *k_gain, const float *sinks,
                                const void *k_cache, const void *v_cache, const void *out, const void *ws,
                                size_t ws_bytes);
moe_status moe_check_attn_decode(const moe_attn_desc *desc, const void *q, const void *k_cache,
                                 const void *v_cache, const int64_t *pos, int32_t batch, int64_t max_ctx,
                                 const float *sinks, const void *out, const void *ws, size_t ws_bytes);

/* Measurement: reads `bytes` (a multiple of 16) of device memory at src
 * once, streaming, with `blocks` blocks of 256 threads (grid-stride, four
 * 16-byte loads in flight per lane); sink: a device int32 that is written
 * only if the folded data equals a fixed constant (it keeps the loads
 * live).  The time of this kernel gives the practical HBM read ceiling the
 * decode kernels are compared with, and its size scales the hardware
 * traffic counters.  Errors: INVALID_ARG for null, misaligned or
 * overlapping pointers, a size not a multiple of 16, blocks outside
 * 1..65536; HIP. */
moe_status moe_probe_hbm_read(const void *src, size_t bytes, int32_t blocks, int32_t *sink, void *stream);

/* Static description of a status code. */
const char *moe_status_string(moe_status s);

/* The HIP runtime's description of the last HIP failure reported as
 * MOE_ERR_HIP on the calling thread ("no HIP error" if none). */
const char *moe_last_error_detail(void);

#ifdef __cplusplus
}
#endif

#endif /* MOE_H */
