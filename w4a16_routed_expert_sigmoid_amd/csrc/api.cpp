// C ABI of the library: argument validation, workspace layout and dispatch.
// Every check runs on the host before anything is enqueued, so each error
// path can be exercised without a GPU.
#include <math.h>
#include <string.h>

#include "../../include/moe.h"
#include "common.h"


using namespace moe;

namespace {

constexpr size_t kAlign = 256;

// The last failing HIP call of this thread, for moe_last_error_detail().
thread_local hipError_t g_last_hip = hipSuccess;

// Stage events set by moe_set_stage_events (per thread).
thread_local hipEvent_t g_stage_events[6];
thread_local bool g_stage_events_on = false;

inline moe_status hip_status(hipError_t e) {
  if (e == hipSuccess) return MOE_OK;
  g_last_hip = e;
  return MOE_ERR_HIP;
}

inline size_t up(size_t v) { return (v + kAlign - 1) / kAlign * kAlign; }
inline bool aligned(const void *p, size_t a) { return ((uintptr_t)p % a) == 0; }

struct WsLayout {
  size_t sync_lines, sync_l, sync_h, sync_bytes;
  size_t logits, xn, n_routed, entry_expert, entry_mask, entry_w, topk_idx, topk_w, h, xcd_l, xcd_h, bytes;
  size_t stage_l, stage_elems;
};

inline int max_routed_of(const moe_layer_desc &d, int B) {
  if (d.n_experts <= 0) return 0;
  int m = B * d.top_k;
  return m < d.n_experts ? m : d.n_experts;
}

inline size_t imax_of(const moe_layer_desc &d) {
  return (size_t)(d.inter > d.shared_inter ? d.inter : d.shared_inter);
}

constexpr size_t kSyncLineBytes = (size_t)kSyncLines * kXcdSlots * 256;

// Bytes of the sync region of a layer at batch B: the ticket and flag
// lines, then the tagged logit words ([B][E]) and the one-token h words.
// Zero for a layer without routed experts.
size_t sync_bytes_of(const moe_layer_desc &d, int B) {
  if (d.n_experts <= 0) return 0;
  const size_t words_h = (size_t)(max_routed_of(d, 1) + 1) * imax_of(d) / 2;
  return kSyncLineBytes + up((size_t)B * d.n_experts * 8) + up(words_h * 8);
}

// Layout of one layer's workspace.  The sync region comes first and takes
// max(sync_cap, this layer's own) bytes, so that the layers of one step,
// which share the workspace, keep their sync words inside one region that
// the step zeroes once.
WsLayout decode_layout(const moe_layer_desc &d, int B, size_t sync_cap = 0) {
  WsLayout L;
  const size_t E = d.n_experts > 0 ? d.n_experts : 0, H = d.hidden, k = d.n_experts > 0 ? d.top_k : 0;
  const size_t Imax = imax_of(d);
  const size_t R = max_routed_of(d, B);
  const size_t own = sync_bytes_of(d, B);
  L.sync_lines = 0;
  L.sync_l = kSyncLineBytes;
  L.sync_h = kSyncLineBytes + up(B * E * 8);
  L.sync_bytes = own > sync_cap ? own : sync_cap;
  size_t o = L.sync_bytes;
  L.logits = o; o += up(B * E * 4);
  L.xn = o; o += up(B * H * 2);
  L.n_routed = o; o += up(4);
  L.entry_expert = o; o += up(R * 4);
  L.entry_mask = o; o += up(R * 4);
  L.entry_w = o; o += up(R * kMaxBatch * 4);
  L.topk_idx = o; o += up(B * k * 4);
  L.topk_w = o; o += up(B * k * 4);
  L.h = o; o += up((R + 1) * B * Imax * 2);
  // one-token stages (also reserved at larger batches, so that a workspace
  // sized for batch b serves every smaller batch)
  const size_t R1 = max_routed_of(d, 1);
  L.stage_l = (E + 63) / 64 * 64;
  L.stage_elems = ((R1 + 1) * Imax + 127) / 128 * 128;
  L.xcd_l = o; o += up(kXcdSlots * L.stage_l * 4);
  L.xcd_h = o; o += up(kXcdSlots * L.stage_elems * 2);
  L.bytes = o;
  return L;
}

// Shape checks shared by the decode calls.  Returns MOE_OK or the error.
moe_status check_desc(const moe_layer_desc *d) {
  if (!d) return MOE_ERR_INVALID_ARG;
  if (d->hidden <= 0 || d->hidden % 32) return MOE_ERR_INVALID_ARG;
  if (d->n_experts < 0 || d->inter < 0 || d->shared_inter < 0) return MOE_ERR_INVALID_ARG;
  if (d->wtype != MOE_W_BF16 && d->wtype != MOE_W_NVFP4) return MOE_ERR_INVALID_ARG;
  if (d->n_experts == 0 && d->shared_inter == 0) return MOE_ERR_INVALID_ARG;
  if (d->n_experts > 0) {
    if (d->inter <= 0 || d->inter % 32) return MOE_ERR_INVALID_ARG;
    if (d->top_k < 1 || d->top_k > kMaxTopK || d->top_k > d->n_experts) return MOE_ERR_INVALID_ARG;
  }
  if (d->shared_inter % 32) return MOE_ERR_INVALID_ARG;
  if (!(d->norm_eps >= 0.0f) || isinf(d->norm_eps)) return MOE_ERR_INVALID_ARG;
  // Shapes the kernels tile.
  if (d->n_experts > kMaxExperts) return MOE_ERR_UNSUPPORTED;
  if (!k_tileable(d->hidden)) return MOE_ERR_UNSUPPORTED;
  if (d->n_experts > 0 && !k_tileable(d->inter)) return MOE_ERR_UNSUPPORTED;
  if (d->shared_inter > 0 && !k_tileable(d->shared_inter)) return MOE_ERR_UNSUPPORTED;
  if (d->n_experts > 0 && d->shared_inter > 0 && d->shared_inter != d->inter) return MOE_ERR_UNSUPPORTED;
  return MOE_OK;
}

moe_status check_weights(const moe_layer_desc *d, const moe_layer_weights *w) {
  if (!w) return MOE_ERR_INVALID_ARG;
  const bool fp4 = d->wtype == MOE_W_NVFP4;
  if (d->n_experts > 0) {
    if (!w->router_w || !w->w_gate || !w->w_up || !w->w_down) return MOE_ERR_INVALID_ARG;
    if (fp4 && !w->w_scale) return MOE_ERR_INVALID_ARG;
    if (!aligned(w->router_w, 16) || !aligned(w->w_gate, 16) || !aligned(w->w_up, 16) ||
        !aligned(w->w_down, 16))
      return MOE_ERR_INVALID_ARG;
    if ((w->router_b && !aligned(w->router_b, 4)) || (w->w_scale && !aligned(w->w_scale, 4)))
      return MOE_ERR_INVALID_ARG;
  }
  if (d->shared_inter > 0) {
    if (!w->sh_gate || !w->sh_up || !w->sh_down) return MOE_ERR_INVALID_ARG;
    if (fp4 && !w->sh_scale) return MOE_ERR_INVALID_ARG;
    if (!aligned(w->sh_gate, 16) || !aligned(w->sh_up, 16) || !aligned(w->sh_down, 16))
      return MOE_ERR_INVALID_ARG;
    if (w->sh_scale && !aligned(w->sh_scale, 4)) return MOE_ERR_INVALID_ARG;
  }
  if (w->norm_gain && !aligned(w->norm_gain, 2)) return MOE_ERR_INVALID_ARG;
  return MOE_OK;
}

}  // namespace

extern "C" {

size_t moe_nvfp4_matrix_bytes(int64_t rows, int64_t cols) {
  if (rows <= 0 || cols <= 0 || rows % 8 || cols % 32) return 0;
  return (size_t)nvfp4_matrix_bytes(rows, cols);
}

static moe_status check_repack(const void *src, void *dst, int64_t rows, int64_t cols, int64_t n_mats) {
  if (!src || !dst || src == dst) return MOE_ERR_INVALID_ARG;
  if (rows <= 0 || cols <= 0 || n_mats <= 0 || rows % 8 || cols % 32) return MOE_ERR_INVALID_ARG;
  if (!aligned(src, 16) || !aligned(dst, 16)) return MOE_ERR_INVALID_ARG;
  // The two ranges must not overlap.
  const uintptr_t s = (uintptr_t)src, t = (uintptr_t)dst;
  const uintptr_t n = (uintptr_t)(n_mats * nvfp4_matrix_bytes(rows, cols));
  if (s < t + n && t < s + n) return MOE_ERR_INVALID_ARG;
  return MOE_OK;
}

moe_status moe_repack_nvfp4(const void *src, void *dst, int64_t rows, int64_t cols, int64_t n_mats,
                            int32_t *nan_scale_count, void *stream) {
  moe_status st = check_repack(src, dst, rows, cols, n_mats);
  if (st != MOE_OK) return st;
  if (nan_scale_count && !aligned(nan_scale_count, 4)) return MOE_ERR_INVALID_ARG;
  return hip_status(launch_repack(src, dst, rows, cols, n_mats, nan_scale_count, (hipStream_t)stream));
}

moe_status moe_unpack_nvfp4(const void *src, void *dst, int64_t rows, int64_t cols, int64_t n_mats,
                            void *stream) {
  moe_status st = check_repack(src, dst, rows, cols, n_mats);
  if (st != MOE_OK) return st;
  return hip_status(launch_unpack(src, dst, rows, cols, n_mats, (hipStream_t)stream));
}

moe_status moe_dequant_nvfp4(const void *src, float *dst, int64_t rows, int64_t cols, int64_t n_mats,
                             const float *tensor_scale, void *stream) {
  if (!src || !dst || (const void *)dst == src) return MOE_ERR_INVALID_ARG;
  if (rows <= 0 || cols <= 0 || n_mats <= 0 || rows % 8 || cols % 32) return MOE_ERR_INVALID_ARG;
  if (!aligned(src, 16) || !aligned(dst, 16)) return MOE_ERR_INVALID_ARG;
  if (tensor_scale && !aligned(tensor_scale, 4)) return MOE_ERR_INVALID_ARG;
  const uintptr_t s = (uintptr_t)src, t = (uintptr_t)dst;
  const uintptr_t ns = (uintptr_t)(n_mats * nvfp4_matrix_bytes(rows, cols)), nt = (uintptr_t)(n_mats * rows * cols * 4);
  if (s < t + nt && t < s + ns) return MOE_ERR_INVALID_ARG;
  return hip_status(launch_dequant(src, dst, rows, cols, n_mats, tensor_scale, (hipStream_t)stream));
}

size_t moe_decode_workspace_bytes(const moe_layer_desc *desc, int32_t max_batch) {
  if (check_desc(desc) != MOE_OK || max_batch < 1 || max_batch > kMaxBatch) return 0;
  return decode_layout(*desc, max_batch).bytes;
}

// Validates one layer call and fills the kernel arguments; nothing is
// launched.  ws_bytes must cover decode_layout(desc, batch).
// sync_cap: the step's common sync region (0: the layer's own); tag: the
// layer's position in the enqueuing call, from 1.
static moe_status prepare_decode(const moe_layer_desc *desc, const moe_layer_weights *w, const void *x,
                                 int32_t batch, int32_t residual, void *y, int32_t *topk_idx, float *topk_w,
                                 void *ws, size_t ws_bytes, DecodeArgs &a, size_t sync_cap = 0,
                                 uint32_t tag = 1) {
  moe_status st = check_desc(desc);
  if (st != MOE_OK) return st;
  if (batch < 1) return MOE_ERR_INVALID_ARG;
  if (batch > kMaxBatch) return MOE_ERR_UNSUPPORTED;
  // The routing kernels stage the batch's activations through 64 KiB.
  if ((size_t)batch * desc->hidden * 2 > 65536) return MOE_ERR_UNSUPPORTED;
  st = check_weights(desc, w);
  if (st != MOE_OK) return st;
  if (!x || !y || !ws || x == y) return MOE_ERR_INVALID_ARG;
  if (!aligned(x, 16) || !aligned(y, 16) || !aligned(ws, kAlign)) return MOE_ERR_INVALID_ARG;
  if ((topk_idx && !aligned(topk_idx, 4)) || (topk_w && !aligned(topk_w, 4))) return MOE_ERR_INVALID_ARG;
  const WsLayout L = decode_layout(*desc, batch, sync_cap);
  if (ws_bytes < L.bytes) return MOE_ERR_WORKSPACE;

  uint8_t *base = (uint8_t *)ws;
  memset(&a, 0, sizeof(a));
  a.tag = tag;
  a.H = desc->hidden;
  a.I = desc->n_experts > 0 ? desc->inter : 0;
  a.Is = desc->shared_inter;
  a.E = desc->n_experts;
  a.k = desc->n_experts > 0 ? desc->top_k : 0;
  a.B = batch;
  a.residual = residual ? 1 : 0;
  a.use_norm = w->norm_gain ? 1 : 0;
  a.max_routed = max_routed_of(*desc, batch);
  a.wtype = desc->wtype;
  a.eps = desc->norm_eps;
  a.x = (const uint16_t *)x;
  a.y = (uint16_t *)y;
  a.router_w = (const uint16_t *)w->router_w;
  a.router_b = w->router_b;
  a.w_gate = (const uint8_t *)w->w_gate;
  a.w_up = (const uint8_t *)w->w_up;
  a.w_down = (const uint8_t *)w->w_down;
  a.w_scale = w->w_scale;
  a.sh_gate = (const uint8_t *)w->sh_gate;
  a.sh_up = (const uint8_t *)w->sh_up;
  a.sh_down = (const uint8_t *)w->sh_down;
  a.sh_scale = w->sh_scale;
  a.norm_gain = (const uint16_t *)w->norm_gain;
  a.ws.logits = (float *)(base + L.logits);
  a.ws.xn = (uint16_t *)(base + L.xn);
  a.ws.n_routed = (int32_t *)(base + L.n_routed);
  a.ws.entry_expert = (int32_t *)(base + L.entry_expert);
  a.ws.entry_mask = (uint32_t *)(base + L.entry_mask);
  a.ws.entry_w = (float *)(base + L.entry_w);
  a.ws.topk_idx = (int32_t *)(base + L.topk_idx);
  a.ws.topk_w = (float *)(base + L.topk_w);
  a.ws.h = (uint16_t *)(base + L.h);
  a.ws.sync_lines = (uint32_t *)(base + L.sync_lines);
  a.ws.sync_l = (uint64_t *)(base + L.sync_l);
  a.ws.sync_h = (uint64_t *)(base + L.sync_h);
  a.ws.xcd_l = (float *)(base + L.xcd_l);
  a.ws.xcd_h = (uint16_t *)(base + L.xcd_h);
  a.ws.stage_l = (int64_t)L.stage_l;
  a.ws.stage_elems = (int64_t)L.stage_elems;
  a.ws.bytes = L.bytes;
  a.out_idx = topk_idx ? topk_idx : a.ws.topk_idx;
  a.out_w = topk_w ? topk_w : a.ws.topk_w;
  return MOE_OK;
}

moe_status moe_decode_layer(const moe_layer_desc *desc, const moe_layer_weights *w, const void *x,
                            int32_t batch, int32_t residual, void *y, int32_t *topk_idx, float *topk_w,
                            void *ws, size_t ws_bytes, void *stream) {
  DecodeArgs a;
  const moe_status st = prepare_decode(desc, w, x, batch, residual, y, topk_idx, topk_w, ws, ws_bytes, a);
  if (st != MOE_OK) return st;
  // With routed experts the hand-overs inside the kernels (the logits; for
  // one token also h) start from a zeroed sync region.
  if (desc->n_experts > 0) {
    const moe_status sc = hip_status(
        launch_sync_clear((uint32_t *)ws, (int64_t)(sync_bytes_of(*desc, batch) / 4), (hipStream_t)stream));
    if (sc != MOE_OK) return sc;
  }
  return hip_status(launch_decode(a, (hipStream_t)stream, g_stage_events_on ? g_stage_events : nullptr));
}

// Step workspace: two activation buffers, then the largest layer workspace.
static size_t step_act_bytes(int32_t hidden, int32_t max_batch) { return up((size_t)max_batch * hidden * 2); }

// The common sync region of a step's layers at batch B.
static size_t step_sync_cap(const moe_layer_desc *descs, int32_t n_layers, int32_t B) {
  size_t cap = 0;
  for (int32_t i = 0; i < n_layers; ++i) {
    const size_t b = sync_bytes_of(descs[i], B);
    cap = b > cap ? b : cap;
  }
  return cap;
}

size_t moe_decode_step_workspace_bytes(const moe_layer_desc *descs, int32_t n_layers, int32_t max_batch) {
  if (!descs || n_layers < 1 || max_batch < 1 || max_batch > kMaxBatch) return 0;
  for (int32_t i = 0; i < n_layers; ++i)
    if (check_desc(&descs[i]) != MOE_OK || descs[i].hidden != descs[0].hidden) return 0;
  const size_t cap = step_sync_cap(descs, n_layers, max_batch);
  size_t layer = 0;
  for (int32_t i = 0; i < n_layers; ++i) {
    const size_t b = decode_layout(descs[i], max_batch, cap).bytes;
    layer = b > layer ? b : layer;
  }
  return 2 * step_act_bytes(descs[0].hidden, max_batch) + layer;
}

moe_status moe_decode_step(const moe_layer_desc *descs, const moe_layer_weights *weights, int32_t n_layers,
                           const void *x, int32_t batch, void *y, void *ws, size_t ws_bytes, void *stream) {
  if (!descs || !weights || n_layers < 1) return MOE_ERR_INVALID_ARG;
  for (int32_t i = 0; i < n_layers; ++i) {
    const moe_status st = check_desc(&descs[i]);
    if (st != MOE_OK) return st;
    if (descs[i].hidden != descs[0].hidden) return MOE_ERR_INVALID_ARG;
  }
  if (batch < 1) return MOE_ERR_INVALID_ARG;
  if (batch > kMaxBatch) return MOE_ERR_UNSUPPORTED;
  if (!x || !y || !ws || x == y) return MOE_ERR_INVALID_ARG;
  if (!aligned(ws, kAlign)) return MOE_ERR_INVALID_ARG;
  const size_t need = moe_decode_step_workspace_bytes(descs, n_layers, batch);
  if (need == 0) return MOE_ERR_INVALID_ARG;
  if (ws_bytes < need) return MOE_ERR_WORKSPACE;
  const size_t act = step_act_bytes(descs[0].hidden, batch);
  uint8_t *a0 = (uint8_t *)ws, *a1 = a0 + act, *lws = a1 + act;
  const size_t lws_bytes = ws_bytes - 2 * act;
  const size_t cap = step_sync_cap(descs, n_layers, batch);
  // Validate every layer before launching anything.
  for (int32_t i = 0; i < n_layers; ++i) {
    const void *in = (i == 0) ? x : ((i & 1) ? (const void *)a0 : (const void *)a1);
    void *out = (i == n_layers - 1) ? y : ((i & 1) ? (void *)a1 : (void *)a0);
    DecodeArgs a;
    const moe_status st = prepare_decode(&descs[i], &weights[i], in, batch, 1, out, nullptr, nullptr, lws,
                                         lws_bytes, a, cap);
    if (st != MOE_OK) return st;
  }
  // The layers' sync words start zeroed, once per step; each layer call
  // then carries its own tag.
  if (cap > 0) {
    const moe_status sc = hip_status(launch_sync_clear((uint32_t *)lws, (int64_t)(cap / 4), (hipStream_t)stream));
    if (sc != MOE_OK) return sc;
  }
  for (int32_t i = 0; i < n_layers; ++i) {
    const void *in = (i == 0) ? x : ((i & 1) ? (const void *)a0 : (const void *)a1);
    void *out = (i == n_layers - 1) ? y : ((i & 1) ? (void *)a1 : (void *)a0);
    DecodeArgs a;
    prepare_decode(&descs[i], &weights[i], in, batch, 1, out, nullptr, nullptr, lws, lws_bytes, a, cap,
                   (uint32_t)i + 1u);
    const moe_status st = hip_status(launch_decode(a, (hipStream_t)stream, nullptr));
    if (st != MOE_OK) return st;
  }
  return MOE_OK;
}

// Prefill workspace, carved in this order (each piece 256-byte aligned).
struct PfLayout {
  size_t xn, logits, topk_idx, topk_w, counts, offsets, cursors, n_tiles, tiles, sorted_tok, pair_pos, h, y, bytes;
  int64_t max_tiles;
};

static constexpr int32_t kMaxPrefillTokens = 1 << 22;

static PfLayout prefill_layout(const moe_layer_desc &d, int64_t T) {
  PfLayout L;
  const int64_t E = d.n_experts > 0 ? d.n_experts : 0, H = d.hidden, k = E > 0 ? d.top_k : 0;
  const int64_t Imax = d.inter > d.shared_inter ? d.inter : d.shared_inter;
  const int64_t P = T * k, rows = P + (d.shared_inter > 0 ? T : 0);
  L.max_tiles = prefill_max_tiles(T, k, E, d.shared_inter > 0);
  size_t o = 0;
  L.xn = o; o += up(T * H * 2);
  L.logits = o; o += up(T * E * 4);
  L.topk_idx = o; o += up(P * 4);
  L.topk_w = o; o += up(P * 4);
  L.counts = o; o += up((E + 1) * 4);
  L.offsets = o; o += up((E + 1) * 4);
  L.cursors = o; o += up((E + 1) * 4);
  L.n_tiles = o; o += up(4);
  L.tiles = o; o += up(L.max_tiles * sizeof(PfTile));
  L.sorted_tok = o; o += up(P * 4);
  L.pair_pos = o; o += up(P * 4);
  L.h = o; o += up(rows * Imax * 2);
  L.y = o; o += up(rows * H * 2);
  L.bytes = o;
  return L;
}

size_t moe_prefill_workspace_bytes(const moe_layer_desc *desc, int32_t n_tokens) {
  if (check_desc(desc) != MOE_OK || n_tokens < 1 || n_tokens > kMaxPrefillTokens) return 0;
  return prefill_layout(*desc, n_tokens).bytes;
}

moe_status moe_prefill_layer(const moe_layer_desc *desc, const moe_layer_weights *w, const void *x,
                             int32_t n_tokens, int32_t residual, void *y, int32_t *topk_idx,
                             float *topk_w, void *ws, size_t ws_bytes, void *stream) {
  moe_status st = check_desc(desc);
  if (st != MOE_OK) return st;
  if (n_tokens < 1) return MOE_ERR_INVALID_ARG;
  if (n_tokens > kMaxPrefillTokens) return MOE_ERR_UNSUPPORTED;
  st = check_weights(desc, w);
  if (st != MOE_OK) return st;
  if (!x || !y || !ws || x == y) return MOE_ERR_INVALID_ARG;
  if (!aligned(x, 16) || !aligned(y, 16) || !aligned(ws, kAlign)) return MOE_ERR_INVALID_ARG;
  if ((topk_idx && !aligned(topk_idx, 4)) || (topk_w && !aligned(topk_w, 4))) return MOE_ERR_INVALID_ARG;
  const PfLayout L = prefill_layout(*desc, n_tokens);
  if (ws_bytes < L.bytes) return MOE_ERR_WORKSPACE;

  uint8_t *base = (uint8_t *)ws;
  PrefillArgs a;
  memset(&a, 0, sizeof(a));
  a.T = n_tokens;
  a.H = desc->hidden;
  a.I = desc->n_experts > 0 ? desc->inter : 0;
  a.Is = desc->shared_inter;
  a.E = desc->n_experts;
  a.k = desc->n_experts > 0 ? desc->top_k : 0;
  a.wtype = desc->wtype;
  a.residual = residual ? 1 : 0;
  a.use_norm = w->norm_gain ? 1 : 0;
  a.P = a.T * a.k;
  a.max_tiles = (int)L.max_tiles;
  a.eps = desc->norm_eps;
  a.x = (const uint16_t *)x;
  a.y = (uint16_t *)y;
  a.router_w = (const uint16_t *)w->router_w;
  a.router_b = w->router_b;
  a.w_gate = (const uint8_t *)w->w_gate;
  a.w_up = (const uint8_t *)w->w_up;
  a.w_down = (const uint8_t *)w->w_down;
  a.w_scale = w->w_scale;
  a.sh_gate = (const uint8_t *)w->sh_gate;
  a.sh_up = (const uint8_t *)w->sh_up;
  a.sh_down = (const uint8_t *)w->sh_down;
  a.sh_scale = w->sh_scale;
  a.norm_gain = (const uint16_t *)w->norm_gain;
  a.out_idx = topk_idx ? topk_idx : (int32_t *)(base + L.topk_idx);
  a.out_w = topk_w ? topk_w : (float *)(base + L.topk_w);
  a.xn = (uint16_t *)(base + L.xn);
  a.logits = (float *)(base + L.logits);
  a.counts = (int32_t *)(base + L.counts);
  a.offsets = (int32_t *)(base + L.offsets);
  a.cursors = (int32_t *)(base + L.cursors);
  a.n_tiles = (int32_t *)(base + L.n_tiles);
  a.tiles = (PfTile *)(base + L.tiles);
  a.sorted_tok = (int32_t *)(base + L.sorted_tok);
  a.pair_pos = (int32_t *)(base + L.pair_pos);
  a.h_rows = (uint16_t *)(base + L.h);
  a.y_rows = (uint16_t *)(base + L.y);
  return hip_status(launch_prefill(a, (hipStream_t)stream));
}

moe_status moe_set_stage_events(void *const *events, int32_t n_events) {
  if (!events || n_events == 0) {
    g_stage_events_on = false;
    return MOE_OK;
  }
  if (n_events != 6) return MOE_ERR_INVALID_ARG;
  for (int i = 0; i < 6; ++i)
    if (!events[i]) return MOE_ERR_INVALID_ARG;
  for (int i = 0; i < 6; ++i) g_stage_events[i] = (hipEvent_t)events[i];
  g_stage_events_on = true;
  return MOE_OK;
}

const char *moe_last_error_detail(void) {
  return g_last_hip == hipSuccess ? "no HIP error" : hipGetErrorString(g_last_hip);
}

const char *moe_status_string(moe_status s) {
  switch (s) {
    case MOE_OK: return "ok";
    case MOE_ERR_INVALID_ARG: return "invalid argument";
    case MOE_ERR_UNSUPPORTED: return "unsupported shape or batch for this path";
    case MOE_ERR_WORKSPACE: return "workspace too small";
    case MOE_ERR_HIP: return "HIP launch or runtime error";
  }
  return "unknown status";
}

}  // extern "C"
