// C ABI of the library: dispatch of the validated calls to the kernels.
// Argument checks and workspace layouts live in validate.cpp (host-only,
// no HIP); nothing here is enqueued before they pass.
#include <math.h>
#include <string.h>

#include <atomic>
#include <mutex>

#include "../../include/moe.h"
#include "attn.h"
#include "common.h"
#include "validate.h"

using namespace moe;

namespace {

// The last failing HIP call of this thread, for moe_last_error_detail().
thread_local hipError_t g_last_hip = hipSuccess;

inline moe_status hip_status(hipError_t e) {
  if (e == hipSuccess) return MOE_OK;
  g_last_hip = e;
  return MOE_ERR_HIP;
}

// Kernel arguments of one validated layer call.  tag: the layer's position
// in the enqueuing call, from 1.
void fill_decode_args(const moe_layer_desc *desc, const moe_layer_weights *w, const void *x, int32_t batch,
                      int32_t residual, void *y, int32_t *topk_idx, float *topk_w, void *ws,
                      const DecodeLayout &L, uint32_t tag, DecodeArgs &a) {
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
  a.ws.status = (uint32_t *)base;
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
  a.ws.sync_y = (uint64_t *)(base + L.sync_y);
  a.ws.xcd_l = (float *)(base + L.xcd_l);
  a.ws.xcd_h = (uint16_t *)(base + L.xcd_h);
  a.ws.stage_l = L.stage_l;
  a.ws.stage_elems = L.stage_elems;
  a.ws.bytes = L.bytes;
  a.out_idx = topk_idx ? topk_idx : a.ws.topk_idx;
  a.out_w = topk_w ? topk_w : a.ws.topk_w;
}

// One layer call: the status word and sync region are zeroed, then the
// layer's kernels run (events: NULL or the 6 stage events).
moe_status decode_layer(const moe_layer_desc *desc, const moe_layer_weights *w, const void *x, int32_t batch,
                        int32_t residual, void *y, int32_t *topk_idx, float *topk_w, void *ws, size_t ws_bytes,
                        hipEvent_t const *events, hipStream_t stream) {
  DecodeLayout L;
  const moe_status st = check_decode_call(desc, w, x, batch, y, topk_idx, topk_w, ws, ws_bytes, 0, &L);
  if (st != MOE_OK) return st;
  DecodeArgs a;
  fill_decode_args(desc, w, x, batch, residual, y, topk_idx, topk_w, ws, L, 1u, a);
  const moe_status sc = hip_status(launch_sync_clear((uint32_t *)ws, (int64_t)(L.clear_bytes / 4), stream));
  if (sc != MOE_OK) return sc;
  return hip_status(launch_decode(a, stream, events));
}

// Workspace of moe_decode_layer_noalloc: one fixed array in the library's
// device memory, so that call allocates nothing.  Host code never passes
// the array's name to a kernel or a copy (on the host it is only a stand-in
// for the symbol); it uses the device address hipGetSymbolAddress returns,
// looked up once per device with that device current.
static __device__ __align__(256) uint8_t scratch[MOE_NOALLOC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
std::atomic<void *> g_scratch_ptr[kMaxDevices];
std::mutex g_scratch_mu;

// The current device's address of `scratch`.
hipError_t device_scratch(void **out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  void *p = g_scratch_ptr[dev].load(std::memory_order_acquire);
  if (!p) {
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    p = g_scratch_ptr[dev].load(std::memory_order_relaxed);
    if (!p) {
      e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
      if (e != hipSuccess) return e;
      if (!p) return hipErrorInvalidSymbol;
      g_scratch_ptr[dev].store(p, std::memory_order_release);
    }
  }
  *out = p;
  return hipSuccess;
}

}  // namespace

extern "C" {

moe_status moe_repack_nvfp4(const void *src, void *dst, int64_t rows, int64_t cols, int64_t n_mats,
                            int32_t *nan_scale_count, void *stream) {
  moe_status st = check_repack_call(src, dst, rows, cols, n_mats);
  if (st != MOE_OK) return st;
  if (nan_scale_count && ((uintptr_t)nan_scale_count % 4)) return MOE_ERR_INVALID_ARG;
  return hip_status(launch_repack(src, dst, rows, cols, n_mats, nan_scale_count, (hipStream_t)stream));
}

moe_status moe_unpack_nvfp4(const void *src, void *dst, int64_t rows, int64_t cols, int64_t n_mats,
                            void *stream) {
  moe_status st = check_repack_call(src, dst, rows, cols, n_mats);
  if (st != MOE_OK) return st;
  return hip_status(launch_unpack(src, dst, rows, cols, n_mats, (hipStream_t)stream));
}

moe_status moe_dequant_nvfp4(const void *src, float *dst, int64_t rows, int64_t cols, int64_t n_mats,
                             const float *tensor_scale, void *stream) {
  moe_status st = check_dequant_call(src, dst, rows, cols, n_mats, tensor_scale);
  if (st != MOE_OK) return st;
  return hip_status(launch_dequant(src, dst, rows, cols, n_mats, tensor_scale, (hipStream_t)stream));
}

moe_status moe_decode_layer(const moe_layer_desc *desc, const moe_layer_weights *w, const void *x,
                            int32_t batch, int32_t residual, void *y, int32_t *topk_idx, float *topk_w,
                            void *ws, size_t ws_bytes, void *stream) {
  return decode_layer(desc, w, x, batch, residual, y, topk_idx, topk_w, ws, ws_bytes, nullptr,
                      (hipStream_t)stream);
}

moe_status moe_decode_layer_timed(const moe_layer_desc *desc, const moe_layer_weights *w, const void *x,
                                  int32_t batch, int32_t residual, void *y, int32_t *topk_idx, float *topk_w,
                                  void *ws, size_t ws_bytes, void *const *events, void *stream) {
  if (!events) return MOE_ERR_INVALID_ARG;
  hipEvent_t ev[6];
  for (int i = 0; i < 6; ++i) {
    if (!events[i]) return MOE_ERR_INVALID_ARG;
    ev[i] = (hipEvent_t)events[i];
  }
  return decode_layer(desc, w, x, batch, residual, y, topk_idx, topk_w, ws, ws_bytes, ev, (hipStream_t)stream);
}

moe_status moe_decode_step(const moe_layer_desc *descs, const moe_layer_weights *weights, int32_t n_layers,
                           const void *x, int32_t batch, void *y, void *ws, size_t ws_bytes, void *stream) {
  StepLayout S;
  const moe_status st = check_step_call(descs, weights, n_layers, x, batch, y, ws, ws_bytes, &S);
  if (st != MOE_OK) return st;
  uint8_t *base = (uint8_t *)ws;
  // The status word and the layers' common sync region start zeroed, once
  // per step; each layer call then carries its own tag.
  const size_t clear = decode_layout(descs[0], batch, S.sync_cap).clear_bytes;
  moe_status sc = hip_status(launch_sync_clear((uint32_t *)ws, (int64_t)(clear / 4), (hipStream_t)stream));
  if (sc != MOE_OK) return sc;
  for (int32_t i = 0; i < n_layers; ++i) {
    const void *in = (i == 0) ? x : base + ((i & 1) ? S.act0 : S.act1);
    void *out = (i == n_layers - 1) ? y : base + ((i & 1) ? S.act1 : S.act0);
    const DecodeLayout L = decode_layout(descs[i], batch, S.sync_cap);
    DecodeArgs a;
    fill_decode_args(&descs[i], &weights[i], in, batch, 1, out, nullptr, nullptr, ws, L, (uint32_t)i + 1u, a);
    sc = hip_status(launch_decode(a, (hipStream_t)stream, nullptr));
    if (sc != MOE_OK) return sc;
  }
  return MOE_OK;
}

moe_status moe_decode_step_persistent(const moe_layer_desc *descs, const moe_layer_weights *weights,
                                      int32_t n_layers, const void *x, int32_t batch, void *y, void *ws,
                                      size_t ws_bytes, void *stream) {
  PersistLayout P;
  const moe_status st = check_step_persistent_call(descs, weights, n_layers, x, batch, y, ws, ws_bytes, &P);
  if (st != MOE_OK) return st;
  const StepLayout &S = P.step;
  uint8_t *base = (uint8_t *)ws;
  const size_t clear = decode_layout(descs[0], batch, S.sync_cap).clear_bytes;
  moe_status sc = hip_status(launch_sync_clear((uint32_t *)ws, (int64_t)(clear / 4), (hipStream_t)stream));
  if (sc != MOE_OK) return sc;
  // Runs of layers that one persistent launch takes, the others one by
  // one; activations alternate between the two step buffers.
  const void *in = x;
  int32_t n_out = 0;  // outputs written so far
  for (int32_t i = 0; i < n_layers;) {
    int32_t end = persist_run_end(descs, weights, n_layers, batch, i);
    const DecodeLayout L = decode_layout(descs[i], batch, S.sync_cap);
    DecodeArgs a;
    if (end > i + 1) {
      fill_decode_args(&descs[i], &weights[i], in, batch, 1, nullptr, nullptr, nullptr, ws, L, (uint32_t)i + 1u, a);
      bool fits = false;
      sc = hip_status(persist_fits(a, &fits));
      if (sc != MOE_OK) return sc;
      if (!fits) end = i + 1;
    }
    void *out = (end == n_layers) ? y : base + ((n_out & 1) ? S.act1 : S.act0);
    if (end > i + 1) {
      PersistArgs p;
      memset(&p, 0, sizeof(p));
      fill_decode_args(&descs[i], &weights[i], in, batch, 1, out, nullptr, nullptr, ws, L, (uint32_t)i + 1u, p.a);
      p.stages = base + P.stages;
      p.slot_bytes = (int64_t)P.slot_bytes;
      p.off_h = (int64_t)P.off_h;
      p.off_y = (int64_t)P.off_y;
      p.n_layers = end - i;
      for (int32_t j = i; j < end; ++j) {
        const moe_layer_weights &w = weights[j];
        PersistLayer &q = p.L[j - i];
        q.router_w = (const uint16_t *)w.router_w;
        q.router_b = w.router_b;
        q.w_gate = (const uint8_t *)w.w_gate;
        q.w_up = (const uint8_t *)w.w_up;
        q.w_down = (const uint8_t *)w.w_down;
        q.w_scale = w.w_scale;
        q.sh_gate = (const uint8_t *)w.sh_gate;
        q.sh_up = (const uint8_t *)w.sh_up;
        q.sh_down = (const uint8_t *)w.sh_down;
        q.sh_scale = w.sh_scale;
        q.norm_gain = (const uint16_t *)w.norm_gain;
      }
      sc = hip_status(launch_step_b1(p, (hipStream_t)stream));
    } else {
      fill_decode_args(&descs[i], &weights[i], in, batch, 1, out, nullptr, nullptr, ws, L, (uint32_t)i + 1u, a);
      sc = hip_status(launch_decode(a, (hipStream_t)stream, nullptr));
    }
    if (sc != MOE_OK) return sc;
    in = out;
    ++n_out;
    i = end;
  }
  return MOE_OK;
}

moe_status moe_decode_layer_noalloc(const moe_layer_desc *desc, const moe_layer_weights *w, const void *x,
                                    int32_t batch, int32_t residual, void *y, int32_t *topk_idx, float *topk_w,
                                    void *stream) {
  // The size limit first: it needs no device.
  moe_status st = check_desc(desc);
  if (st != MOE_OK) return st;
  if (batch < 1) return MOE_ERR_INVALID_ARG;
  if (batch > kMaxBatch) return MOE_ERR_UNSUPPORTED;
  if (decode_layout(*desc, batch).bytes > MOE_NOALLOC_SCRATCH_BYTES) return MOE_ERR_WORKSPACE;
  void *ws = nullptr;
  st = hip_status(device_scratch(&ws));
  if (st != MOE_OK) return st;
  return decode_layer(desc, w, x, batch, residual, y, topk_idx, topk_w, ws, MOE_NOALLOC_SCRATCH_BYTES, nullptr,
                      (hipStream_t)stream);
}

moe_status moe_decode_wait_status(const void *ws, int32_t *status_out, void *stream) {
  if (!ws) {
    // the array of moe_decode_layer_noalloc on the current device
    void *p = nullptr;
    const moe_status st = hip_status(device_scratch(&p));
    if (st != MOE_OK) return st;
    ws = p;
  }
  if (!status_out || ((uintptr_t)ws % kWsAlign) || ((uintptr_t)status_out % 4)) return MOE_ERR_INVALID_ARG;
  return hip_status(hipMemcpyAsync(status_out, ws, 4, hipMemcpyDeviceToDevice, (hipStream_t)stream));
}

moe_status moe_gemv_nvfp4(const void *w, const float *tensor_scale, int64_t rows, int64_t cols, const void *x,
                          int32_t batch, void *y, void *stream) {
  const moe_status st = check_gemv_call(w, tensor_scale, rows, cols, x, batch, y);
  if (st != MOE_OK) return st;
  GemvArgs g;
  g.w = (const uint8_t *)w;
  g.scale = tensor_scale;
  g.x = (const uint16_t *)x;
  g.y = (uint16_t *)y;
  g.N = (int)rows;
  g.K = (int)cols;
  g.B = batch;
  return hip_status(launch_gemv(g, (hipStream_t)stream));
}

moe_status moe_prefill_layer(const moe_layer_desc *desc, const moe_layer_weights *w, const void *x,
                             int32_t n_tokens, int32_t residual, void *y, int32_t *topk_idx,
                             float *topk_w, void *ws, size_t ws_bytes, void *stream) {
  PfLayout L;
  const moe_status st = check_prefill_call(desc, w, x, n_tokens, y, topk_idx, topk_w, ws, ws_bytes, &L);
  if (st != MOE_OK) return st;
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
  a.tile_rows = prefill_tile_rows(n_tokens, desc->wtype);
  a.rsplit = prefill_router_split(n_tokens, desc->n_experts > 0 ? desc->n_experts : 0, desc->hidden);
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

moe_status moe_attn_prep(const moe_attn_desc *desc, const void *qkv, const int64_t *pos, int32_t batch,
                         const void *q_gain, const void *k_gain, void *q_out, void *k_cache, void *v_cache,
                         void *stream) {
  const moe_status st = check_attn_prep_call(desc, qkv, pos, batch, q_gain, k_gain, q_out, k_cache, v_cache);
  if (st != MOE_OK) return st;
  AttnPrepArgs a;
  a.qkv = (const uint16_t *)qkv;
  a.q_gain = (const uint16_t *)q_gain;
  a.k_gain = (const uint16_t *)k_gain;
  a.pos = pos;
  a.q_out = (uint16_t *)q_out;
  a.k_cache = (uint16_t *)k_cache;
  a.v_cache = (uint16_t *)v_cache;
  a.n_q = desc->n_q;
  a.n_kv = desc->n_kv;
  a.slots = desc->slots;
  a.window = desc->window;
  a.rope = desc->rope;
  a.log2_theta = desc->rope ? log2(desc->rope_theta) : 0.0;
  a.eps = (double)desc->norm_eps;
  return hip_status(launch_attn_prep(a, batch, (hipStream_t)stream));
}

moe_status moe_attn_kv_write(const moe_attn_desc *desc, const void *k_rows, const void *v_rows, const int64_t *pos,
                             int32_t n, int32_t batch, void *k_cache, void *v_cache, void *stream) {
  const moe_status st = check_attn_kv_write_call(desc, k_rows, v_rows, pos, n, batch, k_cache, v_cache);
  if (st != MOE_OK) return st;
  AttnKvWriteArgs a;
  a.k_rows = (const uint16_t *)k_rows;
  a.v_rows = (const uint16_t *)v_rows;
  a.pos = pos;
  a.k_cache = (uint16_t *)k_cache;
  a.v_cache = (uint16_t *)v_cache;
  a.n = n;
  a.n_kv = desc->n_kv;
  a.slots = desc->slots;
  a.window = desc->window;
  return hip_status(launch_attn_kv_write(a, batch, (hipStream_t)stream));
}

moe_status moe_attn_layer(const moe_attn_desc *desc, const void *qkv, const int64_t *pos, int32_t batch,
                          int64_t max_ctx, const void *q_gain, const void *k_gain, const float *sinks, void *k_cache,
                          void *v_cache, void *out, void *ws, size_t ws_bytes, void *stream) {
  const moe_status st = check_attn_layer_call(desc, qkv, pos, batch, max_ctx, q_gain, k_gain, sinks, k_cache,
                                              v_cache, out, ws, ws_bytes);
  if (st != MOE_OK) return st;
  const AttnPlan plan = attn_plan_of(*desc, batch, max_ctx);
  AttnDecodeArgs a;
  memset(&a, 0, sizeof(a));
  a.k_cache = (const uint16_t *)k_cache;
  a.v_cache = (const uint16_t *)v_cache;
  a.pos = pos;
  a.sinks = sinks;
  a.out = (uint16_t *)out;
  a.status = (uint32_t *)ws;
  a.part = plan.chunks > 1 ? (float *)((uint8_t *)ws + attn_partial_offset()) : nullptr;
  a.n_q = desc->n_q;
  a.n_kv = desc->n_kv;
  a.G = desc->n_q / desc->n_kv;
  a.slots = desc->slots;
  a.window = desc->window;
  a.B = batch;
  a.span = plan.span;
  a.tpc = plan.tpc;
  a.chunks = plan.chunks;
  a.fused = 1;
  a.rope = desc->rope;
  a.qkv = (const uint16_t *)qkv;
  a.q_gain = (const uint16_t *)q_gain;
  a.k_gain = (const uint16_t *)k_gain;
  a.log2_theta = desc->rope ? log2(desc->rope_theta) : 0.0;
  a.eps = (double)desc->norm_eps;
  return hip_status(launch_attn_decode(a, (hipStream_t)stream));
}

moe_status moe_attn_decode(const moe_attn_desc *desc, const void *q, const void *k_cache, const void *v_cache,
                           const int64_t *pos, int32_t batch, int64_t max_ctx, const float *sinks, void *out,
                           void *ws, size_t ws_bytes, void *stream) {
  const moe_status st =
      check_attn_decode_call(desc, q, k_cache, v_cache, pos, batch, max_ctx, sinks, out, ws, ws_bytes);
  if (st != MOE_OK) return st;
  const AttnPlan plan = attn_plan_of(*desc, batch, max_ctx);
  AttnDecodeArgs a;
  memset(&a, 0, sizeof(a));
  a.q = (const uint16_t *)q;
  a.k_cache = (const uint16_t *)k_cache;
  a.v_cache = (const uint16_t *)v_cache;
  a.pos = pos;
  a.sinks = sinks;
  a.out = (uint16_t *)out;
  a.status = (uint32_t *)ws;
  a.part = plan.chunks > 1 ? (float *)((uint8_t *)ws + attn_partial_offset()) : nullptr;
  a.n_q = desc->n_q;
  a.n_kv = desc->n_kv;
  a.G = desc->n_q / desc->n_kv;
  a.slots = desc->slots;
  a.window = desc->window;
  a.B = batch;
  a.span = plan.span;
  a.tpc = plan.tpc;
  a.chunks = plan.chunks;
  return hip_status(launch_attn_decode(a, (hipStream_t)stream));
}

moe_status moe_probe_hbm_read(const void *src, size_t bytes, int32_t blocks, int32_t *sink, void *stream) {
  if (!src || !sink || ((uintptr_t)src % 16) || ((uintptr_t)sink % 4)) return MOE_ERR_INVALID_ARG;
  if (bytes == 0 || bytes % 16 || blocks < 1 || blocks > 65536) return MOE_ERR_INVALID_ARG;
  const uintptr_t s = (uintptr_t)src, k = (uintptr_t)sink;
  if (k + 4 > s && k < s + bytes) return MOE_ERR_INVALID_ARG;
  return hip_status(launch_probe_read(src, (int64_t)bytes, blocks, (uint32_t *)sink, (hipStream_t)stream));
}

const char *moe_last_error_detail(void) {
  return g_last_hip == hipSuccess ? "no HIP error" : hipGetErrorString(g_last_hip);
}

}  // extern "C"
