// Host-side validation and workspace layouts of the C ABI (no HIP).  Every
// check runs before anything is enqueued, so each error path is exercised
// on the CPU, with or without the HIP runtime.
#include "validate.h"

#include <math.h>
#include <string.h>

namespace moe {

namespace {

inline size_t up(size_t v) { return (v + kWsAlign - 1) / kWsAlign * kWsAlign; }
inline bool aligned(const void *p, size_t a) { return ((uintptr_t)p % a) == 0; }

constexpr size_t kStatusLine = 256;  // the status word's own line, at byte 0
constexpr size_t kSyncLineBytes = (size_t)kSyncLines * kXcdSlots * 256;

inline size_t imax_of(const moe_layer_desc &d) {
  return (size_t)(d.inter > d.shared_inter ? d.inter : d.shared_inter);
}

// Caller buffers [p, p + n); a null pointer or n == 0 takes no room.
struct Range {
  const void *p;
  size_t n;
};

inline bool overlap(Range a, Range b) {
  if (!a.p || !b.p || a.n == 0 || b.n == 0) return false;
  const uintptr_t s = (uintptr_t)a.p, t = (uintptr_t)b.p;
  return s < t + b.n && t < s + a.n;
}

// No two of the n ranges overlap.
bool disjoint(const Range *r, int n) {
  for (int i = 0; i < n; ++i)
    for (int j = i + 1; j < n; ++j)
      if (overlap(r[i], r[j])) return false;
  return true;
}

}  // namespace

// Largest decode batch of a layer: 16 tokens with NVFP4 weights (the
// matrix-core kernels take the tokens as the 16 columns of their tiles),
// 8 with BF16 weights (per-token dot products on the vector ALUs).
int max_batch_of(const moe_layer_desc &d) { return d.wtype == 1 ? kMaxBatch : kMaxBatchBf16; }

int max_routed_of(const moe_layer_desc &d, int B) {
  if (d.n_experts <= 0) return 0;
  const int m = B * d.top_k;
  return m < d.n_experts ? m : d.n_experts;
}

// Bytes of the sync region of a layer at batch B: the ticket and flag
// lines, then the tagged logit words ([B][E]) and the one-token h words.
// Zero for a layer without routed experts.
size_t sync_bytes_of(const moe_layer_desc &d, int B) {
  if (d.n_experts <= 0) return 0;
  const size_t words_h = (size_t)(max_routed_of(d, 1) + 1) * imax_of(d) / 2;
  const size_t words_y = (size_t)d.hidden / 2;  // the persistent step's layer outputs
  return kSyncLineBytes + up((size_t)B * d.n_experts * 8) + up(words_h * 8) + up(words_y * 8);
}

DecodeLayout decode_layout(const moe_layer_desc &d, int B, size_t sync_cap) {
  DecodeLayout L;
  const size_t E = d.n_experts > 0 ? d.n_experts : 0, H = d.hidden, k = d.n_experts > 0 ? d.top_k : 0;
  const size_t Imax = imax_of(d);
  const size_t R = max_routed_of(d, B);
  const size_t own = sync_bytes_of(d, B);
  const size_t sync = own > sync_cap ? own : sync_cap;
  L.sync_lines = kStatusLine;
  L.sync_l = kStatusLine + kSyncLineBytes;
  L.sync_h = L.sync_l + up(B * E * 8);
  L.sync_y = L.sync_h + up((max_routed_of(d, 1) + 1) * Imax / 2 * 8);
  L.clear_bytes = kStatusLine + sync;
  size_t o = L.clear_bytes;
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
  L.stage_l = (int64_t)((E + 63) / 64 * 64);
  L.stage_elems = (int64_t)(((R1 + 1) * Imax + 127) / 128 * 128);
  L.xcd_l = o; o += up(kXcdSlots * (size_t)L.stage_l * 4);
  L.xcd_h = o; o += up(kXcdSlots * (size_t)L.stage_elems * 2);
  L.bytes = o;
  return L;
}

bool step_layout(const moe_layer_desc *descs, int32_t n_layers, int32_t B, StepLayout &L) {
  if (!descs || n_layers < 1 || B < 1 || B > kMaxBatch) return false;
  for (int32_t i = 0; i < n_layers; ++i)
    if (check_desc(&descs[i]) != MOE_OK || descs[i].hidden != descs[0].hidden || B > max_batch_of(descs[i]))
      return false;
  L.sync_cap = 0;
  for (int32_t i = 0; i < n_layers; ++i) {
    const size_t b = sync_bytes_of(descs[i], B);
    L.sync_cap = b > L.sync_cap ? b : L.sync_cap;
  }
  L.layer_bytes = 0;
  for (int32_t i = 0; i < n_layers; ++i) {
    const size_t b = decode_layout(descs[i], B, L.sync_cap).bytes;
    L.layer_bytes = b > L.layer_bytes ? b : L.layer_bytes;
  }
  const size_t act = up((size_t)B * descs[0].hidden * 2);
  L.act0 = L.layer_bytes;
  L.act1 = L.act0 + act;
  L.bytes = L.act1 + act;
  return true;
}

bool persist_layout(const moe_layer_desc *descs, int32_t n_layers, int32_t B, PersistLayout &L) {
  if (!step_layout(descs, n_layers, B, L.step)) return false;
  L.stage_l = 0;
  L.stage_elems = 0;
  for (int32_t i = 0; i < n_layers; ++i) {
    const DecodeLayout d = decode_layout(descs[i], 1, L.step.sync_cap);
    L.stage_l = d.stage_l > L.stage_l ? d.stage_l : L.stage_l;
    L.stage_elems = d.stage_elems > L.stage_elems ? d.stage_elems : L.stage_elems;
  }
  const size_t H = descs[0].hidden;
  L.off_h = up(kXcdSlots * (size_t)L.stage_l * 4);
  L.off_y = L.off_h + up(kXcdSlots * (size_t)L.stage_elems * 2);
  L.slot_bytes = L.off_y + up(kXcdSlots * H * 2);
  L.stages = L.step.bytes;
  L.bytes = L.stages + (size_t)kPersistMaxLayers * L.slot_bytes;
  return true;
}

int32_t persist_run_end(const moe_layer_desc *descs, const moe_layer_weights *weights, int32_t n_layers,
                        int32_t batch, int32_t i) {
  const moe_layer_desc &d = descs[i];
  if (batch != 1 || d.n_experts <= 0) return i + 1;
  const bool norm = weights[i].norm_gain != nullptr;
  int32_t j = i + 1;
  while (j < n_layers && j - i < kPersistMaxLayers) {
    const moe_layer_desc &e = descs[j];
    if (e.n_experts != d.n_experts || e.hidden != d.hidden || e.inter != d.inter ||
        e.shared_inter != d.shared_inter || e.top_k != d.top_k || e.wtype != d.wtype ||
        (weights[j].norm_gain != nullptr) != norm || (norm && e.norm_eps != d.norm_eps))
      break;
    ++j;
  }
  return j;
}

PfLayout prefill_layout(const moe_layer_desc &d, int64_t T) {
  PfLayout L;
  const int64_t E = d.n_experts > 0 ? d.n_experts : 0, H = d.hidden, k = E > 0 ? d.top_k : 0;
  const int64_t Imax = d.inter > d.shared_inter ? d.inter : d.shared_inter;
  const int64_t P = T * k, rows = P + (d.shared_inter > 0 ? T : 0);
  L.max_tiles = prefill_max_tiles(T, k, E, d.shared_inter > 0, prefill_tile_rows(T, d.wtype));
  size_t o = 0;
  L.xn = o; o += up(T * H * 2);
  L.logits = o; o += up((size_t)prefill_router_logit_rows(T, E, H) * E * 4);
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

moe_status check_decode_call(const moe_layer_desc *desc, const moe_layer_weights *w, const void *x,
                             int32_t batch, const void *y, const int32_t *topk_idx, const float *topk_w,
                             const void *ws, size_t ws_bytes, size_t sync_cap, DecodeLayout *L) {
  moe_status st = check_desc(desc);
  if (st != MOE_OK) return st;
  if (batch < 1) return MOE_ERR_INVALID_ARG;
  if (batch > max_batch_of(*desc)) return MOE_ERR_UNSUPPORTED;
  // The routing kernels stage the batch's activations through 64 KiB, and
  // a batch gate/up block its logits and expert marks through 64 KiB.
  if ((size_t)batch * desc->hidden * 2 > 65536) return MOE_ERR_UNSUPPORTED;
  if (batch > 1 && desc->n_experts > 0 && (size_t)(batch + 1) * desc->n_experts > (size_t)kMaxRouteStage)
    return MOE_ERR_UNSUPPORTED;
  st = check_weights(desc, w);
  if (st != MOE_OK) return st;
  if (!x || !y || !ws) return MOE_ERR_INVALID_ARG;
  if (!aligned(x, 16) || !aligned(y, 16) || !aligned(ws, kWsAlign)) return MOE_ERR_INVALID_ARG;
  if ((topk_idx && !aligned(topk_idx, 4)) || (topk_w && !aligned(topk_w, 4))) return MOE_ERR_INVALID_ARG;
  // The kernels read x while other blocks write y, the top-k outputs and
  // the workspace: none of these may share a byte.
  const size_t act = (size_t)batch * desc->hidden * 2;
  const size_t tk = desc->n_experts > 0 ? (size_t)batch * desc->top_k * 4 : 0;
  const Range r[5] = {{x, act}, {y, act}, {topk_idx, tk}, {topk_w, tk}, {ws, ws_bytes}};
  if (!disjoint(r, 5)) return MOE_ERR_INVALID_ARG;
  const DecodeLayout lay = decode_layout(*desc, batch, sync_cap);
  if (ws_bytes < lay.bytes) return MOE_ERR_WORKSPACE;
  if (L) *L = lay;
  return MOE_OK;
}

moe_status check_step_call(const moe_layer_desc *descs, const moe_layer_weights *weights, int32_t n_layers,
                           const void *x, int32_t batch, const void *y, const void *ws, size_t ws_bytes,
                           StepLayout *L) {
  if (!descs || !weights || n_layers < 1) return MOE_ERR_INVALID_ARG;
  for (int32_t i = 0; i < n_layers; ++i) {
    const moe_status st = check_desc(&descs[i]);
    if (st != MOE_OK) return st;
    if (descs[i].hidden != descs[0].hidden) return MOE_ERR_INVALID_ARG;
  }
  if (batch < 1) return MOE_ERR_INVALID_ARG;
  for (int32_t i = 0; i < n_layers; ++i)
    if (batch > max_batch_of(descs[i])) return MOE_ERR_UNSUPPORTED;
  if (!x || !y || !ws) return MOE_ERR_INVALID_ARG;
  if (!aligned(x, 16) || !aligned(y, 16) || !aligned(ws, kWsAlign)) return MOE_ERR_INVALID_ARG;
  const size_t act = (size_t)batch * descs[0].hidden * 2;
  const Range r[3] = {{x, act}, {y, act}, {ws, ws_bytes}};
  if (!disjoint(r, 3)) return MOE_ERR_INVALID_ARG;
  StepLayout S;
  if (!step_layout(descs, n_layers, batch, S)) return MOE_ERR_INVALID_ARG;
  if (ws_bytes < S.bytes) return MOE_ERR_WORKSPACE;
  // Every layer as the step runs it: its input and output are the caller's
  // x / y or an activation buffer past the layer workspace.
  const uint8_t *base = (const uint8_t *)ws;
  for (int32_t i = 0; i < n_layers; ++i) {
    const void *in = (i == 0) ? x : base + ((i & 1) ? S.act0 : S.act1);
    const void *out = (i == n_layers - 1) ? y : base + ((i & 1) ? S.act1 : S.act0);
    const moe_status st =
        check_decode_call(&descs[i], &weights[i], in, batch, out, nullptr, nullptr, ws, S.layer_bytes, S.sync_cap,
                          nullptr);
    if (st != MOE_OK) return st;
  }
  if (L) *L = S;
  return MOE_OK;
}

moe_status check_step_persistent_call(const moe_layer_desc *descs, const moe_layer_weights *weights,
                                     int32_t n_layers, const void *x, int32_t batch, const void *y, const void *ws,
                                     size_t ws_bytes, PersistLayout *L) {
  // every check of the step (the persistent workspace begins with the step's)
  const moe_status st = check_step_call(descs, weights, n_layers, x, batch, y, ws, ws_bytes, nullptr);
  if (st != MOE_OK) return st;
  PersistLayout P;
  if (!persist_layout(descs, n_layers, batch, P)) return MOE_ERR_INVALID_ARG;
  if (ws_bytes < P.bytes) return MOE_ERR_WORKSPACE;
  if (L) *L = P;
  return MOE_OK;
}

moe_status check_prefill_call(const moe_layer_desc *desc, const moe_layer_weights *w, const void *x,
                              int32_t n_tokens, const void *y, const int32_t *topk_idx, const float *topk_w,
                              const void *ws, size_t ws_bytes, PfLayout *L) {
  moe_status st = check_desc(desc);
  if (st != MOE_OK) return st;
  if (n_tokens < 1) return MOE_ERR_INVALID_ARG;
  if (n_tokens > kMaxPrefillTokens) return MOE_ERR_UNSUPPORTED;
  st = check_weights(desc, w);
  if (st != MOE_OK) return st;
  if (!x || !y || !ws) return MOE_ERR_INVALID_ARG;
  if (!aligned(x, 16) || !aligned(y, 16) || !aligned(ws, kWsAlign)) return MOE_ERR_INVALID_ARG;
  if ((topk_idx && !aligned(topk_idx, 4)) || (topk_w && !aligned(topk_w, 4))) return MOE_ERR_INVALID_ARG;
  const size_t act = (size_t)n_tokens * desc->hidden * 2;
  const size_t tk = desc->n_experts > 0 ? (size_t)n_tokens * desc->top_k * 4 : 0;
  const Range r[5] = {{x, act}, {y, act}, {topk_idx, tk}, {topk_w, tk}, {ws, ws_bytes}};
  if (!disjoint(r, 5)) return MOE_ERR_INVALID_ARG;
  const PfLayout lay = prefill_layout(*desc, n_tokens);
  if (ws_bytes < lay.bytes) return MOE_ERR_WORKSPACE;
  if (L) *L = lay;
  return MOE_OK;
}

moe_status check_gemv_call(const void *w, const float *tensor_scale, int64_t rows, int64_t cols, const void *x,
                           int32_t batch, const void *y) {
  if (!w || !tensor_scale || !x || !y) return MOE_ERR_INVALID_ARG;
  if (rows <= 0 || cols <= 0 || rows % 8 || cols % 32) return MOE_ERR_INVALID_ARG;
  if (batch < 1) return MOE_ERR_INVALID_ARG;
  if (!aligned(w, 16) || !aligned(x, 16) || !aligned(y, 16) || !aligned(tensor_scale, 4)) return MOE_ERR_INVALID_ARG;
  if (batch > kMaxBatchBf16) return MOE_ERR_UNSUPPORTED;
  // one token stages x in 64 KiB of LDS
  if (!k_tileable(cols) || rows > (int64_t)1 << 30 || (batch == 1 && cols > 32768)) return MOE_ERR_UNSUPPORTED;
  // the output may share no byte with an input
  const Range out = {y, (size_t)batch * rows * 2};
  const Range in[3] = {{w, (size_t)nvfp4_matrix_bytes(rows, cols)}, {x, (size_t)batch * cols * 2}, {tensor_scale, 4}};
  for (const Range &r : in)
    if (overlap(out, r)) return MOE_ERR_INVALID_ARG;
  return MOE_OK;
}

moe_status check_attn_desc(const moe_attn_desc *d) {
  if (!d) return MOE_ERR_INVALID_ARG;
  if (d->n_q < 1 || d->n_kv < 1 || d->n_q > 4096 || d->n_q % d->n_kv) return MOE_ERR_INVALID_ARG;
  if (d->head_dim < 1 || d->slots < kAttnTile || d->slots % kAttnTile) return MOE_ERR_INVALID_ARG;
  if (d->window < 0 || d->window > d->slots) return MOE_ERR_INVALID_ARG;
  if (d->rope != 0 && d->rope != 1) return MOE_ERR_INVALID_ARG;
  if (d->rope && !(d->rope_theta > 1.0 && isfinite(d->rope_theta))) return MOE_ERR_INVALID_ARG;
  if (!(d->norm_eps >= 0.0f) || !isfinite(d->norm_eps)) return MOE_ERR_INVALID_ARG;
  if (d->head_dim != kAttnD || d->n_q / d->n_kv > kAttnMaxGroup || d->slots > kAttnMaxSlots)
    return MOE_ERR_UNSUPPORTED;
  return MOE_OK;
}

int64_t attn_span(const moe_attn_desc &d, int64_t max_ctx) {
  const int64_t bound = d.window > 0 ? d.window : d.slots;
  if (max_ctx < 0 || max_ctx > bound) return -1;
  return max_ctx > 0 ? max_ctx : bound;
}

AttnPlan attn_plan_of(const moe_attn_desc &d, int32_t batch, int64_t max_ctx) {
  return attn_plan(attn_span(d, max_ctx), d.window > 0, batch, d.n_kv);
}

size_t attn_partial_offset() { return kStatusLine; }

size_t attn_workspace_bytes(const moe_attn_desc &d, int32_t batch, int64_t max_ctx) {
  const AttnPlan p = attn_plan_of(d, batch, max_ctx);
  size_t b = kStatusLine;
  if (p.chunks > 1)
    b += up((size_t)batch * d.n_kv * p.chunks * (size_t)attn_part_floats(d.n_q / d.n_kv) * sizeof(float));
  return b;
}

namespace {
inline size_t cache_bytes(const moe_attn_desc &d, int32_t batch) {
  return (size_t)batch * d.n_kv * (size_t)d.slots * kAttnD * 2;
}

// Each output range shares no byte with any other range.
bool outputs_disjoint(const Range *r, int n, int n_out) {
  for (int i = 0; i < n_out; ++i)
    for (int j = 0; j < n; ++j)
      if (j != i && overlap(r[i], r[j])) return false;
  return true;
}
}  // namespace

moe_status check_attn_prep_call(const moe_attn_desc *desc, const void *qkv, const int64_t *pos, int32_t batch,
                                const void *q_gain, const void *k_gain, const void *q_out, const void *k_cache,
                                const void *v_cache) {
  const moe_status st = check_attn_desc(desc);
  if (st != MOE_OK) return st;
  if (!qkv || !pos || !q_gain || !k_gain || !q_out || !k_cache || !v_cache) return MOE_ERR_INVALID_ARG;
  if (batch < 1 || batch > kAttnMaxBatch) return MOE_ERR_INVALID_ARG;
  if (!aligned(qkv, 16) || !aligned(pos, 8) || !aligned(q_gain, 16) || !aligned(k_gain, 16) ||
      !aligned(q_out, 16) || !aligned(k_cache, 16) || !aligned(v_cache, 16))
    return MOE_ERR_INVALID_ARG;
  const size_t cb = cache_bytes(*desc, batch);
  const Range r[7] = {{q_out, (size_t)batch * desc->n_q * kAttnD * 2},
                      {k_cache, cb},
                      {v_cache, cb},
                      {qkv, (size_t)batch * (desc->n_q + 2 * desc->n_kv) * kAttnD * 2},
                      {pos, (size_t)batch * 8},
                      {q_gain, kAttnD * 2},
                      {k_gain, kAttnD * 2}};
  return outputs_disjoint(r, 7, 3) ? MOE_OK : MOE_ERR_INVALID_ARG;
}

moe_status check_attn_kv_write_call(const moe_attn_desc *desc, const void *k_rows, const void *v_rows,
                                   const int64_t *pos, int32_t n, int32_t batch, const void *k_cache,
                                   const void *v_cache) {
  const moe_status st = check_attn_desc(desc);
  if (st != MOE_OK) return st;
  if (!k_rows || !v_rows || !pos || !k_cache || !v_cache) return MOE_ERR_INVALID_ARG;
  if (n < 1 || n > (1 << 24) || batch < 1 || batch > kAttnMaxBatch) return MOE_ERR_INVALID_ARG;
  if (!aligned(k_rows, 16) || !aligned(v_rows, 16) || !aligned(pos, 8) || !aligned(k_cache, 16) ||
      !aligned(v_cache, 16))
    return MOE_ERR_INVALID_ARG;
  const size_t cb = cache_bytes(*desc, batch);
  const size_t rows = (size_t)batch * n * desc->n_kv * kAttnD * 2;
  const Range r[5] = {{k_cache, cb}, {v_cache, cb}, {k_rows, rows}, {v_rows, rows}, {pos, (size_t)batch * n * 8}};
  return outputs_disjoint(r, 5, 2) ? MOE_OK : MOE_ERR_INVALID_ARG;
}

moe_status check_attn_layer_call(const moe_attn_desc *desc, const void *qkv, const int64_t *pos, int32_t batch,
                                 int64_t max_ctx, const void *q_gain, const void *k_gain, const float *sinks,
                                 const void *k_cache, const void *v_cache, const void *out, const void *ws,
                                 size_t ws_bytes) {
  const moe_status st = check_attn_desc(desc);
  if (st != MOE_OK) return st;
  if (!qkv || !pos || !q_gain || !k_gain || !k_cache || !v_cache || !out || !ws) return MOE_ERR_INVALID_ARG;
  if (batch < 1 || batch > kAttnMaxBatch) return MOE_ERR_INVALID_ARG;
  if (attn_span(*desc, max_ctx) < 0) return MOE_ERR_INVALID_ARG;
  if (!aligned(qkv, 16) || !aligned(pos, 8) || !aligned(q_gain, 16) || !aligned(k_gain, 16) ||
      !aligned(k_cache, 16) || !aligned(v_cache, 16) || !aligned(out, 16) || !aligned(ws, kWsAlign) ||
      (sinks && !aligned(sinks, 4)))
    return MOE_ERR_INVALID_ARG;
  const size_t cb = cache_bytes(*desc, batch);
  const Range r[9] = {{out, (size_t)batch * desc->n_q * kAttnD * 2},
                      {ws, ws_bytes},
                      {k_cache, cb},
                      {v_cache, cb},
                      {qkv, (size_t)batch * (desc->n_q + 2 * desc->n_kv) * kAttnD * 2},
                      {pos, (size_t)batch * 8},
                      {q_gain, kAttnD * 2},
                      {k_gain, kAttnD * 2},
                      {sinks, sinks ? (size_t)desc->n_q * 4 : 0}};
  if (!outputs_disjoint(r, 9, 4)) return MOE_ERR_INVALID_ARG;
  if (ws_bytes < attn_workspace_bytes(*desc, batch, max_ctx)) return MOE_ERR_WORKSPACE;
  return MOE_OK;
}

moe_status check_attn_decode_call(const moe_attn_desc *desc, const void *q, const void *k_cache, const void *v_cache,
                                  const int64_t *pos, int32_t batch, int64_t max_ctx, const float *sinks,
                                  const void *out, const void *ws, size_t ws_bytes) {
  const moe_status st = check_attn_desc(desc);
  if (st != MOE_OK) return st;
  if (!q || !k_cache || !v_cache || !pos || !out || !ws) return MOE_ERR_INVALID_ARG;
  if (batch < 1 || batch > kAttnMaxBatch) return MOE_ERR_INVALID_ARG;
  if (attn_span(*desc, max_ctx) < 0) return MOE_ERR_INVALID_ARG;
  if (!aligned(q, 16) || !aligned(k_cache, 16) || !aligned(v_cache, 16) || !aligned(pos, 8) ||
      !aligned(out, 16) || !aligned(ws, kWsAlign) || (sinks && !aligned(sinks, 4)))
    return MOE_ERR_INVALID_ARG;
  const size_t cb = cache_bytes(*desc, batch);
  const size_t act = (size_t)batch * desc->n_q * kAttnD * 2;
  const Range r[7] = {{out, act}, {ws, ws_bytes}, {q, act}, {k_cache, cb}, {v_cache, cb},
                      {pos, (size_t)batch * 8}, {sinks, sinks ? (size_t)desc->n_q * 4 : 0}};
  if (!outputs_disjoint(r, 7, 2)) return MOE_ERR_INVALID_ARG;
  if (ws_bytes < attn_workspace_bytes(*desc, batch, max_ctx)) return MOE_ERR_WORKSPACE;
  return MOE_OK;
}

moe_status check_repack_call(const void *src, const void *dst, int64_t rows, int64_t cols, int64_t n_mats) {
  if (!src || !dst) return MOE_ERR_INVALID_ARG;
  if (rows <= 0 || cols <= 0 || n_mats <= 0 || rows % 8 || cols % 32) return MOE_ERR_INVALID_ARG;
  if (!aligned(src, 16) || !aligned(dst, 16)) return MOE_ERR_INVALID_ARG;
  const size_t n = (size_t)(n_mats * nvfp4_matrix_bytes(rows, cols));
  const Range r[2] = {{src, n}, {dst, n}};
  return disjoint(r, 2) ? MOE_OK : MOE_ERR_INVALID_ARG;
}

moe_status check_dequant_call(const void *src, const float *dst, int64_t rows, int64_t cols, int64_t n_mats,
                              const float *tensor_scale) {
  if (!src || !dst) return MOE_ERR_INVALID_ARG;
  if (rows <= 0 || cols <= 0 || n_mats <= 0 || rows % 8 || cols % 32) return MOE_ERR_INVALID_ARG;
  if (!aligned(src, 16) || !aligned(dst, 16)) return MOE_ERR_INVALID_ARG;
  if (tensor_scale && !aligned(tensor_scale, 4)) return MOE_ERR_INVALID_ARG;
  const Range r[2] = {{src, (size_t)(n_mats * nvfp4_matrix_bytes(rows, cols))},
                      {dst, (size_t)(n_mats * rows * cols * 4)}};
  return disjoint(r, 2) ? MOE_OK : MOE_ERR_INVALID_ARG;
}

}  // namespace moe

using namespace moe;

extern "C" {

size_t moe_nvfp4_matrix_bytes(int64_t rows, int64_t cols) {
  if (rows <= 0 || cols <= 0 || rows % 8 || cols % 32) return 0;
  return (size_t)nvfp4_matrix_bytes(rows, cols);
}

size_t moe_decode_workspace_bytes(const moe_layer_desc *desc, int32_t max_batch) {
  if (check_desc(desc) != MOE_OK || max_batch < 1 || max_batch > max_batch_of(*desc)) return 0;
  return decode_layout(*desc, max_batch).bytes;
}

size_t moe_decode_step_workspace_bytes(const moe_layer_desc *descs, int32_t n_layers, int32_t max_batch) {
  StepLayout S;
  return step_layout(descs, n_layers, max_batch, S) ? S.bytes : 0;
}

size_t moe_decode_step_persistent_workspace_bytes(const moe_layer_desc *descs, int32_t n_layers, int32_t max_batch) {
  PersistLayout P;
  if (!descs || n_layers < 1 || max_batch < 1 || max_batch > kMaxBatch) return 0;
  return persist_layout(descs, n_layers, max_batch, P) ? P.bytes : 0;
}

moe_status moe_check_decode_step_persistent(const moe_layer_desc *descs, const moe_layer_weights *weights,
                                            int32_t n_layers, const void *x, int32_t batch, const void *y,
                                            const void *ws, size_t ws_bytes) {
  return check_step_persistent_call(descs, weights, n_layers, x, batch, y, ws, ws_bytes, nullptr);
}

size_t moe_prefill_workspace_bytes(const moe_layer_desc *desc, int32_t n_tokens) {
  if (check_desc(desc) != MOE_OK || n_tokens < 1 || n_tokens > kMaxPrefillTokens) return 0;
  return prefill_layout(*desc, n_tokens).bytes;
}

moe_status moe_check_decode_layer(const moe_layer_desc *desc, const moe_layer_weights *w, const void *x,
                                  int32_t batch, const void *y, const int32_t *topk_idx, const float *topk_w,
                                  const void *ws, size_t ws_bytes) {
  return check_decode_call(desc, w, x, batch, y, topk_idx, topk_w, ws, ws_bytes, 0, nullptr);
}

moe_status moe_check_decode_step(const moe_layer_desc *descs, const moe_layer_weights *weights, int32_t n_layers,
                                 const void *x, int32_t batch, const void *y, const void *ws, size_t ws_bytes) {
  return check_step_call(descs, weights, n_layers, x, batch, y, ws, ws_bytes, nullptr);
}

moe_status moe_check_prefill_layer(const moe_layer_desc *desc, const moe_layer_weights *w, const void *x,
                                   int32_t n_tokens, const void *y, const int32_t *topk_idx, const float *topk_w,
                                   const void *ws, size_t ws_bytes) {
  return check_prefill_call(desc, w, x, n_tokens, y, topk_idx, topk_w, ws, ws_bytes, nullptr);
}

moe_status moe_check_repack_nvfp4(const void *src, const void *dst, int64_t rows, int64_t cols, int64_t n_mats) {
  return check_repack_call(src, dst, rows, cols, n_mats);
}

size_t moe_attn_workspace_bytes(const moe_attn_desc *desc, int32_t batch, int64_t max_ctx) {
  if (check_attn_desc(desc) != MOE_OK || batch < 1 || batch > kAttnMaxBatch) return 0;
  if (attn_span(*desc, max_ctx) < 0) return 0;
  return attn_workspace_bytes(*desc, batch, max_ctx);
}

moe_status moe_check_attn_prep(const moe_attn_desc *desc, const void *qkv, const int64_t *pos, int32_t batch,
                               const void *q_gain, const void *k_gain, const void *q_out, const void *k_cache,
                               const void *v_cache) {
  return check_attn_prep_call(desc, qkv, pos, batch, q_gain, k_gain, q_out, k_cache, v_cache);
}

moe_status moe_check_attn_kv_write(const moe_attn_desc *desc, const void *k_rows, const void *v_rows,
                                   const int64_t *pos, int32_t n, int32_t batch, const void *k_cache,
                                   const void *v_cache) {
  return check_attn_kv_write_call(desc, k_rows, v_rows, pos, n, batch, k_cache, v_cache);
}

moe_status moe_check_attn_layer(const moe_attn_desc *desc, const void *qkv, const int64_t *pos, int32_t batch,
                                int64_t max_ctx, const void *q_gain, const void *k_gain, const float *sinks,
                                const void *k_cache, const void *v_cache, const void *out, const void *ws,
                                size_t ws_bytes) {
  return check_attn_layer_call(desc, qkv, pos, batch, max_ctx, q_gain, k_gain, sinks, k_cache, v_cache, out, ws,
                               ws_bytes);
}

moe_status moe_check_attn_decode(const moe_attn_desc *desc, const void *q, const void *k_cache,
                                 const void *v_cache, const int64_t *pos, int32_t batch, int64_t max_ctx,
                                 const float *sinks, const void *out, const void *ws, size_t ws_bytes) {
  return check_attn_decode_call(desc, q, k_cache, v_cache, pos, batch, max_ctx, sinks, out, ws, ws_bytes);
}

moe_status moe_check_gemv_nvfp4(const void *w, const float *tensor_scale, int64_t rows, int64_t cols, const void *x,
                                int32_t batch, const void *y) {
  return check_gemv_call(w, tensor_scale, rows, cols, x, batch, y);
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
