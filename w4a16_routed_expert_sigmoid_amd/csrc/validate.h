// Host-side argument validation and workspace layouts of the C ABI, in
// plain C++ with no HIP dependency.  libmoe.so compiles this unit next to
// the kernels; the same source also builds alone into a host-only library
// (libmoe_host.so) whose checks run without the HIP runtime.
#pragma once

#include "../../include/moe.h"
#include "attn_shapes.h"
#include "shapes.h"

namespace moe {

// Byte offsets of one layer's decode workspace.  The status word's line
// comes first, then the sync region (the ticket and flag lines, the tagged
// logit words [B][E] and the one-token h words); the call zeroes
// [0, clear_bytes) before its kernels run.
struct DecodeLayout {
  size_t sync_lines, sync_l, sync_h, sync_y, clear_bytes;
  size_t logits, xn, n_routed, entry_expert, entry_mask, entry_w, topk_idx, topk_w, h, xcd_l, xcd_h, bytes;
  int64_t stage_l, stage_elems;
};

// A step's workspace: the largest layer workspace (all layers share its
// status word and sync region), then two activation buffers.
struct StepLayout {
  size_t sync_cap, layer_bytes, act0, act1, bytes;
};

// The persistent step's workspace: the step's, then per-layer stage sets
// (the logits, h and layer-input copies of every XCD) for the layers of one
// launch, so that no block reads a stage address twice in a launch.
struct PersistLayout {
  StepLayout step;
  size_t stages, slot_bytes, bytes;
  int64_t stage_l, stage_elems;  // per-XCD stage sizes (elements), as in DecodeLayout
  size_t off_h, off_y;           // offsets of the h and input stages within a slot
};

// A prefill workspace, carved in this order.
struct PfLayout {
  size_t xn, logits, topk_idx, topk_w, counts, offsets, cursors, n_tiles, tiles, sorted_tok, pair_pos, h, y, bytes;
  int64_t max_tiles;
};

int max_batch_of(const moe_layer_desc &d);
int max_routed_of(const moe_layer_desc &d, int B);
size_t sync_bytes_of(const moe_layer_desc &d, int B);
DecodeLayout decode_layout(const moe_layer_desc &d, int B, size_t sync_cap = 0);
bool step_layout(const moe_layer_desc *descs, int32_t n_layers, int32_t B, StepLayout &L);
bool persist_layout(const moe_layer_desc *descs, int32_t n_layers, int32_t B, PersistLayout &L);
// Layers i .. end - 1 that one persistent launch can run: batch 1, routed
// experts, the shape of layer i, a pre-norm gain on all or none, at most
// kPersistMaxLayers; end == i + 1 means none (the layer runs alone).
int32_t persist_run_end(const moe_layer_desc *descs, const moe_layer_weights *weights, int32_t n_layers,
                        int32_t batch, int32_t i);
PfLayout prefill_layout(const moe_layer_desc &d, int64_t T);

moe_status check_desc(const moe_layer_desc *d);
moe_status check_weights(const moe_layer_desc *d, const moe_layer_weights *w);

// One layer call of `batch` tokens on workspace [ws, ws + ws_bytes) whose
// sync region is sized for sync_cap (0: the layer's own); fills *L.
moe_status check_decode_call(const moe_layer_desc *desc, const moe_layer_weights *w, const void *x,
                             int32_t batch, const void *y, const int32_t *topk_idx, const float *topk_w,
                             const void *ws, size_t ws_bytes, size_t sync_cap, DecodeLayout *L);
moe_status check_step_call(const moe_layer_desc *descs, const moe_layer_weights *weights, int32_t n_layers,
                           const void *x, int32_t batch, const void *y, const void *ws, size_t ws_bytes,
                           StepLayout *L);
moe_status check_step_persistent_call(const moe_layer_desc *descs, const moe_layer_weights *weights,
                                     int32_t n_layers, const void *x, int32_t batch, const void *y, const void *ws,
                                     size_t ws_bytes, PersistLayout *L);
moe_status check_prefill_call(const moe_layer_desc *desc, const moe_layer_weights *w, const void *x,
                              int32_t n_tokens, const void *y, const int32_t *topk_idx, const float *topk_w,
                              const void *ws, size_t ws_bytes, PfLayout *L);
moe_status check_gemv_call(const void *w, const float *tensor_scale, int64_t rows, int64_t cols, const void *x,
                           int32_t batch, const void *y);
// Attention: the description's checks, the positions a token may attend
// (max_ctx, or the layer's bound when 0; -1 when out of range), the chunk
// plan and the workspace size (status line, then the partials when split).
moe_status check_attn_desc(const moe_attn_desc *d);
int64_t attn_span(const moe_attn_desc &d, int64_t max_ctx);
AttnPlan attn_plan_of(const moe_attn_desc &d, int32_t batch, int64_t max_ctx);
size_t attn_partial_offset();
size_t attn_workspace_bytes(const moe_attn_desc &d, int32_t batch, int64_t max_ctx);
moe_status check_attn_prep_call(const moe_attn_desc *desc, const void *qkv, const int64_t *pos, int32_t batch,
                                const void *q_gain, const void *k_gain, const void *q_out, const void *k_cache,
                                const void *v_cache);
moe_status check_attn_kv_write_call(const moe_attn_desc *desc, const void *k_rows, const void *v_rows,
                                   const int64_t *pos, int32_t n, int32_t batch, const void *k_cache,
                                   const void *v_cache);
moe_status check_attn_layer_call(const moe_attn_desc *desc, const void *qkv, const int64_t *pos, int32_t batch,
                                 int64_t max_ctx, const void *q_gain, const void *k_gain, const float *sinks,
                                 const void *k_cache, const void *v_cache, const void *out, const void *ws,
                                 size_t ws_bytes);
moe_status check_attn_decode_call(const moe_attn_desc *desc, const void *q, const void *k_cache, const void *v_cache,
                                  const int64_t *pos, int32_t batch, int64_t max_ctx, const float *sinks,
                                  const void *out, const void *ws, size_t ws_bytes);
moe_status check_repack_call(const void *src, const void *dst, int64_t rows, int64_t cols, int64_t n_mats);
moe_status check_dequant_call(const void *src, const float *dst, int64_t rows, int64_t cols, int64_t n_mats,
                              const float *tensor_scale);

}  // namespace moe
