// Internal declarations of the attention kernels (attn.hip) shared with
// the host dispatch (api.cpp).
#pragma once

#include "attn_shapes.h"
#include "common.h"

namespace moe {

struct AttnPrepArgs {
  const uint16_t *qkv, *q_gain, *k_gain;
  const int64_t *pos;
  uint16_t *q_out, *k_cache, *v_cache;
  int n_q, n_kv, slots, window, rope;
  double log2_theta, eps;
};

struct AttnDecodeArgs {
  const uint16_t *q, *k_cache, *v_cache;
  const int64_t *pos;
  const float *sinks;
  uint16_t *out;
  float *part;        // [B][n_kv][chunks] FP32 partials (split plans; attn_part_floats each)
  uint32_t *status;   // the call's status word
  int n_q, n_kv, G, slots, window, B;
  int64_t span;       // most positions a token may attend
  int tpc, chunks;
  // fused (moe_attn_layer): the Q/K norm, RoPE and KV write run in the
  // decode kernel; q is then unused and the caches are written
  int fused, rope;
  const uint16_t *qkv, *q_gain, *k_gain;
  double log2_theta, eps;
};

struct AttnKvWriteArgs {
  const uint16_t *k_rows, *v_rows;  // [B][n][n_kv][128]
  const int64_t *pos;               // [B][n]
  uint16_t *k_cache, *v_cache;
  int n, n_kv, slots, window;
};

hipError_t launch_attn_prep(const AttnPrepArgs &a, int B, hipStream_t stream);
hipError_t launch_attn_kv_write(const AttnKvWriteArgs &a, int B, hipStream_t stream);
hipError_t launch_attn_decode(const AttnDecodeArgs &a, hipStream_t stream);

}  // namespace moe
