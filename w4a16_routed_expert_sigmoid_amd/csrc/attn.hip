// Decode attention beside the MoE blocks ("Day-0 Support for Flint on
// vLLM", sections "Model architecture" and "Optimizations"; "vLLM Flint"
// commentary, section "Only 14 of 49 layers retain full-history KV"): GQA
// 32/4 with head_dim 128, per-head Q/K RMSNorm, learned sinks, sliding-window
// layers with RoPE and full-context layers without it, BF16 KV cache.
//
//   k_attn_prep     one wave per head of a token: per-head RMSNorm (FP64
//                   sum of squares and scale, one BF16 rounding), RoPE of the
//                   pairs (d, d + 64) with FP64 angles (one BF16 rounding),
//                   q out, k and v written into the caches.  The norm, the
//                   rotation and the cache write the pages fuse into one
//                   kernel.
//   k_attn_decode   flash-decoding: a block of 8 waves takes a chunk of
//                   32-position tiles of one (token, KV head); per tile a wave
//                   computes the scores of the group's query heads on the
//                   matrix cores (v_mfma_f32_16x16x32_bf16: 16 positions x
//                   16 head columns x 32 dims), an online base-2 softmax in
//                   FP32, and P V on the matrix cores with P split into two
//                   BF16 terms (hi + lo, about 16 significant bits).  The
//                   block merges its waves through LDS, then writes the
//                   final BF16 output (one chunk) or an FP32 partial.
//   k_attn_combine  merges a token's partials and applies the sink.
//   k_attn_kv_write K/V rows (natural layout) into cache slots.
//
// Cache layout (per token row and KV head): tiles of 32 positions, each
// stored in the lane order of the MFMA operands that read it (attn_k_index,
// attn_v_index), so every operand is one contiguous 1 KiB wave load.  Read
// in the operands' natural layout instead, a 16-lane group would touch 16
// rows per load and the address units, not HBM, would set the pace.  The
// values are stored by dimension within a tile, so the 8 positions a lane
// feeds into P V are 16 contiguous bytes, and the probabilities leave the
// score MFMA already in the lane order that P V takes (see k_attn_decode).
#include "attn.h"

namespace moe {

// Positions lo..pos a token attends; false for a position the layer cannot
// hold or that attends more than `span` positions.
__device__ __forceinline__ bool attn_range(int64_t pos, int window, int slots, int64_t span, int64_t &lo) {
  if (pos < 0 || pos >= kAttnMaxPos) return false;
  if (window > 0) {
    lo = pos - window + 1 > 0 ? pos - window + 1 : 0;
  } else {
    if (pos >= slots) return false;
    lo = 0;
  }
  return pos - lo + 1 <= span;
}

// RoPE angle of the pair (lane, lane + 64) at position pos: its cosine and
// sine, angle = pos * theta^(-2 lane / 128) in FP64.
__device__ __forceinline__ void rope_angle(int64_t pos, int lane, double log2_theta, double &cs, double &sn) {
  const double f = exp2(-(double)lane / 64.0 * log2_theta);
  sincos((double)pos * f, &sn, &cs);
}

// One head (lane holds elements lane and lane + 64): y = BF16(x / sqrt(
// mean(x^2) + eps) * gain) with an FP64 sum of squares (exact per term) and
// scale, then with RoPE (a, b) -> (BF16(a cos - b sin), BF16(b cos + a sin)).
__device__ __forceinline__ void norm_rope_head(uint32_t x0b, uint32_t x1b, const uint16_t *gain, int lane, double eps,
                                               bool rope, double cs, double sn, uint32_t &y0, uint32_t &y1) {
#pragma clang fp contract(off)
  const double x0 = (double)bf16_to_f32(x0b), x1 = (double)bf16_to_f32(x1b);
  double ss = x0 * x0 + x1 * x1;
  ss = group_sum_f64(ss, kWave);
  const double inv = 1.0 / sqrt(ss / (double)kAttnD + eps);
  const double g0 = (double)bf16_to_f32(gain[lane]), g1 = (double)bf16_to_f32(gain[lane + 64]);
  y0 = f64_to_bf16(x0 * inv * g0);
  y1 = f64_to_bf16(x1 * inv * g1);
  if (rope) {
    const double ya = (double)bf16_to_f32(y0), yb = (double)bf16_to_f32(y1);
    y0 = f64_to_bf16(ya * cs - yb * sn);
    y1 = f64_to_bf16(yb * cs + ya * sn);
  }
}

// ---------------------------------------------------------------------------
// Q/K norm + RoPE + KV write.  Grid (ceil(units / 4), B), 4 waves; unit u of
// a token: q heads 0..n_q-1, k heads, then v heads.  Lane l holds elements
// l and l + 64, the RoPE pair.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void k_attn_prep(AttnPrepArgs a) {
  const int b = blockIdx.y;
  const int lane = threadIdx.x & 63;
  const int u = blockIdx.x * 4 + (threadIdx.x >> 6);
  const int units = a.n_q + 2 * a.n_kv;
  if (u >= units) return;
  const int64_t pos = a.pos[b];
  int64_t lo;
  const bool ok = attn_range(pos, a.window, a.slots, (int64_t)1 << 62, lo);
  const int64_t slot = ok ? pos % a.slots : 0;
  const uint16_t *src = a.qkv + ((int64_t)b * units + u) * kAttnD;
  const uint32_t x0b = src[lane], x1b = src[lane + 64];

  // the cache tile of the slot, and the position's offset in it
  const int o = (int)(slot % kAttnTile);
  const int64_t tile = (slot / kAttnTile) * kAttnTileElems;
  if (u >= a.n_q + a.n_kv) {  // v head
    if (!ok) return;
    const int g = u - a.n_q - a.n_kv;
    uint16_t *vt = a.v_cache + ((int64_t)b * a.n_kv + g) * a.slots * kAttnD + tile;
    vt[attn_v_index(o, lane)] = (uint16_t)x0b;
    vt[attn_v_index(o, lane + 64)] = (uint16_t)x1b;
    return;
  }
  const bool is_q = u < a.n_q;
  if (!ok) {
    if (is_q) {
      uint16_t *dq = a.q_out + ((int64_t)b * a.n_q + u) * kAttnD;
      dq[lane] = dq[lane + 64] = 0;
    }
    return;
  }
  double cs = 1.0, sn = 0.0;
  if (a.rope) rope_angle(pos, lane, a.log2_theta, cs, sn);
  uint32_t y0, y1;
  norm_rope_head(x0b, x1b, is_q ? a.q_gain : a.k_gain, lane, a.eps, a.rope != 0, cs, sn, y0, y1);
  if (is_q) {
    uint16_t *dq = a.q_out + ((int64_t)b * a.n_q + u) * kAttnD;
    dq[lane] = (uint16_t)y0;
    dq[lane + 64] = (uint16_t)y1;
  } else {
    uint16_t *kt = a.k_cache + ((int64_t)b * a.n_kv + (u - a.n_q)) * a.slots * kAttnD + tile;
    kt[attn_k_index(o, lane)] = (uint16_t)y0;
    kt[attn_k_index(o, lane + 64)] = (uint16_t)y1;
  }
}

// ---------------------------------------------------------------------------
// K/V rows into the cache layout.  Grid (n, B), 4 waves; wave w writes KV
// heads w, w + 4, ... of row i of token row b, lane l elements l and l + 64.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void k_attn_kv_write(AttnKvWriteArgs a) {
  const int i = blockIdx.x, b = blockIdx.y;
  const int lane = threadIdx.x & 63;
  const int64_t pos = a.pos[(int64_t)b * a.n + i];
  int64_t lo;
  if (!attn_range(pos, a.window, a.slots, (int64_t)1 << 62, lo)) return;
  const int64_t slot = pos % a.slots;
  const int o = (int)(slot % kAttnTile);
  const int64_t tile = (slot / kAttnTile) * kAttnTileElems;
  for (int g = threadIdx.x >> 6; g < a.n_kv; g += 4) {
    const int64_t row = (((int64_t)b * a.n + i) * a.n_kv + g) * kAttnD;
    const int64_t base = ((int64_t)b * a.n_kv + g) * a.slots * kAttnD + tile;
    a.k_cache[base + attn_k_index(o, lane)] = a.k_rows[row + lane];
    a.k_cache[base + attn_k_index(o, lane + 64)] = a.k_rows[row + lane + 64];
    a.v_cache[base + attn_v_index(o, lane)] = a.v_rows[row + lane];
    a.v_cache[base + attn_v_index(o, lane + 64)] = a.v_rows[row + lane + 64];
  }
}

// ---------------------------------------------------------------------------
// Decode attention.  Grid (chunks, n_kv, B), 8 waves.
//
// Lane l = 16 g + r (r = l % 16, g = l / 16).  MFMA 16x16x32 lane layouts:
// A lane l holds row r, k-group g (8 elements); B lane l holds column r,
// k-group g; C lane l value i is row 4g + i, column r.  A dot product only
// needs A and B to pair the same k elements, so any fixed assignment of
// dims (or positions) to a k-group's 8 elements works.
//
// Scores, per 32-position tile and per half tt (0, 1): A = keys of 16
// positions, row r <-> position offset 8 (r / 4) + 4 tt + r % 4; k-step s
// (dims 32 s .. 32 s + 31) gives group g the dims 8 (4 s + g) .. + 8 (the
// cache tile holds exactly this operand as 1 KiB in lane order).  B = q of the
// group's heads, column r = head r (zero beyond G).  So C value i of lane l
// is the score of head r at position offset 8 g + 4 tt + i: each lane holds
// one head's scores at 8 consecutive positions 8 g .. 8 g + 7.
//
// P V, per 16-dim tile dt: out^T[dims][heads] += V^T[dims][32 positions] *
// P[32 positions][heads].  A lane l = value dim dt*16 + r, positions
// 8 g .. 8 g + 7 (16 contiguous bytes of the cache tile); B lane l =
// head r, the same 8 positions: exactly the 8 probabilities the lane holds.
// C lane l value i = dim dt*16 + 4 g + i of head r.
// ---------------------------------------------------------------------------
constexpr float kLog2e = 1.4426950408889634f;

__device__ __forceinline__ u32x4 ld16(const uint16_t *p) { return *reinterpret_cast<const u32x4 *>(p); }

struct AttnTileRegs {
  u32x4 k[2][4];  // keys: half tt, k-step s
  u32x4 v[8];     // transposed values: dim tile dt
};

// Cache tile st of a token row's KV head; each operand is one contiguous
// 1 KiB wave load (lane order of the tile layout).
__device__ __forceinline__ void attn_load_tile(AttnTileRegs &t, const uint16_t *kb, const uint16_t *vb, int st,
                                               int lane) {
  const int64_t off = (int64_t)st * kAttnTileElems + lane * 8;
  const uint16_t *kt = kb + off, *vt = vb + off;
#pragma unroll
  for (int tt = 0; tt < 2; ++tt)
#pragma unroll
    for (int s = 0; s < 4; ++s) t.k[tt][s] = ld16(kt + (tt * 4 + s) * 512);
#pragma unroll
  for (int dt = 0; dt < 8; ++dt) t.v[dt] = ld16(vt + dt * 512);
}

__device__ __forceinline__ f32x4 mfma16(u32x4 a, u32x4 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a), __builtin_bit_cast(bf16x8, b), c,
                                                 0, 0, 0);
}

// Sum / max over the 4 lanes of one head column (lanes r, r+16, r+32, r+48).
__device__ __forceinline__ float col_sum(float v) {
  v += xor_lane<16>(v);
  return v + xor_lane<32>(v);
}
__device__ __forceinline__ float col_max(float v) {
  v = fmaxf(v, xor_lane<16>(v));
  return fmaxf(v, xor_lane<32>(v));
}

constexpr int kAccStride = kAttnD + 4;  // LDS row of one head's accumulator (floats)

// moe_attn_layer: KV head kv's new k (normed, rotated) or v (u = 0 / 1) of
// token b into the cache slot of pos, by one wave; the row also to `row`
// when given.
__device__ inline void fused_kv_unit(const AttnDecodeArgs &a, int b, int kv, int u, int64_t pos, int lane, double cs,
                                     double sn, uint16_t *row) {
  const int64_t slot = pos % a.slots;
  const int o = (int)(slot % kAttnTile);
  const int64_t tile_off = ((int64_t)b * a.n_kv + kv) * a.slots * kAttnD + (slot / kAttnTile) * kAttnTileElems;
  const uint16_t *src = a.qkv + ((int64_t)b * (a.n_q + 2 * a.n_kv) + a.n_q + (int64_t)u * a.n_kv + kv) * kAttnD;
  uint32_t y0 = src[lane], y1 = src[lane + 64];
  if (u == 0) {
    norm_rope_head(y0, y1, a.k_gain, lane, a.eps, a.rope != 0, cs, sn, y0, y1);
    uint16_t *kt = const_cast<uint16_t *>(a.k_cache) + tile_off;
    kt[attn_k_index(o, lane)] = (uint16_t)y0;
    kt[attn_k_index(o, lane + 64)] = (uint16_t)y1;
  } else {
    uint16_t *vt = const_cast<uint16_t *>(a.v_cache) + tile_off;
    vt[attn_v_index(o, lane)] = (uint16_t)y0;
    vt[attn_v_index(o, lane + 64)] = (uint16_t)y1;
  }
  if (row) {
    row[lane] = (uint16_t)y0;
    row[lane + 64] = (uint16_t)y1;
  }
}

// FUSED (moe_attn_layer): before the tiles are used, the block computes its
// group's q heads into LDS (norm and RoPE as k_attn_prep, the same bits),
// and the block whose chunk holds the current position also the new k and
// v, which it writes to the cache and patches into its registers when it
// reaches that tile (its tiles were requested before the write).
template <bool FUSED>
__global__ __launch_bounds__(kAttnWaves * kWave) void k_attn_decode(AttnDecodeArgs a) {
  __shared__ float s_acc[kAttnWaves][kAttnMaxGroup][kAccStride];
  __shared__ float s_m[kAttnWaves][kAttnMaxGroup], s_l[kAttnWaves][kAttnMaxGroup];
  __shared__ __attribute__((aligned(16))) uint16_t s_q[FUSED ? kAttnMaxGroup : 1][kAttnD];
  __shared__ __attribute__((aligned(16))) uint16_t s_kv[FUSED ? 2 : 1][kAttnD];  // the position's k, v

  const int c = blockIdx.x, kv = blockIdx.y, b = blockIdx.z;
  // the wave index as a scalar: tile indices and the edge test stay in
  // scalar registers and branches
  const int lane = threadIdx.x & 63, wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int r = lane & 15, g = lane >> 4;
  const int G = a.G;

  // One chunk per token: this kernel writes the status word (block 0).
  if (a.chunks == 1 && c == 0 && kv == 0 && b == 0 && threadIdx.x < kWave) {
    uint32_t bad = 0;
    for (int t = threadIdx.x; t < a.B; t += kWave) {
      int64_t lo;
      bad |= attn_range(a.pos[t], a.window, a.slots, a.span, lo) ? 0u : (uint32_t)kStatusBadPos;
    }
    bad = wave_max_u32(bad);
    if (threadIdx.x == 0) *a.status = bad;
  }

  const int64_t pos = a.pos[b];
  int64_t lo = 0;
  const bool ok = attn_range(pos, a.window, a.slots, a.span, lo);
  uint16_t *outb = a.out + ((int64_t)b * a.n_q + (int64_t)kv * G) * kAttnD;
  if (!ok) {  // zero output rows (the combine kernel does it for split plans)
    if (a.chunks == 1)
      for (int i = threadIdx.x; i < G * kAttnD / 8; i += blockDim.x)
        reinterpret_cast<u32x4 *>(outb)[i] = u32x4{0, 0, 0, 0};
    if constexpr (FUSED) {
      // a position the cache holds, beyond the context bound: the new k and
      // v are still written, as moe_attn_prep writes them (chunk 0's block)
      int64_t lo2;
      if (c == 0 && wave < 2 && attn_range(pos, a.window, a.slots, (int64_t)1 << 62, lo2)) {
        double cs = 1.0, sn = 0.0;
        if (a.rope) rope_angle(pos, lane, a.log2_theta, cs, sn);
        fused_kv_unit(a, b, kv, wave, pos, lane, cs, sn, nullptr);
      }
    }
    return;
  }
  const int64_t ft = lo / kAttnTile, lt = pos / kAttnTile;
  const int64_t t0 = ft + (int64_t)c * a.tpc;
  if (t0 > lt) return;  // this token needs fewer chunks
  const int64_t t1 = t0 + a.tpc - 1 < lt ? t0 + a.tpc - 1 : lt;
  const uint16_t *kb = a.k_cache + ((int64_t)b * a.n_kv + kv) * a.slots * kAttnD;
  const uint16_t *vb = a.v_cache + ((int64_t)b * a.n_kv + kv) * a.slots * kAttnD;

  // This wave's first tile, requested before anything else (cache tiles
  // follow the tiles: st = t mod (slots / 32), advanced by addition).
  int64_t t = t0 + wave;
  const int nst = a.slots / kAttnTile;
  int sa = 0;
  AttnTileRegs ra, rb;
  if (t <= t1) {
    sa = (int)(t % nst);
    attn_load_tile(ra, kb, vb, sa, lane);
  }

  if constexpr (FUSED) {
    // units: the group's q heads, then (the block holding the position)
    // KV head kv's k and v
    const bool holds_pos = t0 <= lt && lt <= t1;
    const int units = G + (holds_pos ? 2 : 0);
    const uint16_t *row = a.qkv + (int64_t)b * (a.n_q + 2 * a.n_kv) * kAttnD;
    double cs = 1.0, sn = 0.0;
    if (a.rope) rope_angle(pos, lane, a.log2_theta, cs, sn);
    for (int u = wave; u < units; u += kAttnWaves) {
      if (u >= G) {
        fused_kv_unit(a, b, kv, u - G, pos, lane, cs, sn, &s_kv[u - G][0]);
      } else {
        const uint16_t *src = row + (int64_t)(kv * G + u) * kAttnD;
        uint32_t y0, y1;
        norm_rope_head(src[lane], src[lane + 64], a.q_gain, lane, a.eps, a.rope != 0, cs, sn, y0, y1);
        s_q[u][lane] = (uint16_t)y0;
        s_q[u][lane + 64] = (uint16_t)y1;
      }
    }
    __syncthreads();
  }

  // q of head r of the group, dims 8 (4 s + g) .. + 8 for k-step s
  u32x4 qv[4];
  {
    const int hq = r < G ? r : 0;
    const uint16_t *qh = FUSED ? &s_q[hq][0] : a.q + ((int64_t)b * a.n_q + (int64_t)kv * G + hq) * kAttnD;
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      const u32x4 v = ld16(qh + (s * 4 + g) * 8);
      qv[s] = r < G ? v : u32x4{0, 0, 0, 0};
    }
  }
  const float qscale = kLog2e / sqrtf((float)kAttnD);

  f32x4 acc[8];
#pragma unroll
  for (int dt = 0; dt < 8; ++dt) acc[dt] = f32x4{0.f, 0.f, 0.f, 0.f};
  float m_run = -INFINITY, l_run = 0.f;

  // Tiles t0 + wave, t0 + wave + 8, ... of the chunk, two register sets
  // used in turn: the loads of the next tile are in flight while this one
  // is computed (a copy between the sets would wait for them).  Loads are
  // unconditional: past the end they reload the last tile, a cache hit.
  auto tile_step = [&](AttnTileRegs &cur, int64_t t) {
    if constexpr (FUSED) {
      if (t == lt) {
        // the current position's new k and v, into the lanes that hold it
        const int o = (int)(pos - t * kAttnTile);
        const int r_o = ((o >> 3) << 2) | (o & 3);
        if (r == r_o) {
#pragma unroll
          for (int s = 0; s < 4; ++s) {
            const u32x4 nk = *reinterpret_cast<const u32x4 *>(&s_kv[0][(s * 4 + g) * 8]);
            if ((o >> 2) & 1) cur.k[1][s] = nk;
            else cur.k[0][s] = nk;
          }
        }
        if (g == (o >> 3)) {
          const int j = o & 7;
          const uint32_t keep = (j & 1) ? 0x0000FFFFu : 0xFFFF0000u;
#pragma unroll
          for (int dt = 0; dt < 8; ++dt) {
            const uint32_t val = (uint32_t)s_kv[1][dt * 16 + r] << ((j & 1) * 16);
            u32x4 &vv = cur.v[dt];
            if ((j >> 1) == 0) vv.x = (vv.x & keep) | val;
            else if ((j >> 1) == 1) vv.y = (vv.y & keep) | val;
            else if ((j >> 1) == 2) vv.z = (vv.z & keep) | val;
            else vv.w = (vv.w & keep) | val;
          }
        }
      }
    }
    f32x4 sc[2];
#pragma unroll
    for (int tt = 0; tt < 2; ++tt) {
      sc[tt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int s = 0; s < 4; ++s) sc[tt] = mfma16(cur.k[tt][s], qv[s], sc[tt]);
    }
    // positions 32 t + 8 g + j, j = 4 tt + i
    float x[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) x[j] = sc[j >> 2][j & 3] * qscale;
    // A tile that straddles lo or pos (uniform): positions outside lo..pos
    // get no weight, and their values (possibly never written) are zeroed
    // so that 0 * garbage cannot make a NaN.
    u32x4 vmask = {~0u, ~0u, ~0u, ~0u};
    const int64_t tp = t * kAttnTile;
    const bool edge = tp < lo || tp + kAttnTile - 1 > pos;
    if (edge) {
      const int first = (int)(lo - tp > 0 ? lo - tp : 0);                         // 0..31
      const int last = (int)(pos - tp < kAttnTile - 1 ? pos - tp : kAttnTile - 1);  // 0..31
      uint32_t vm[4] = {~0u, ~0u, ~0u, ~0u};
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const int o = g * 8 + j;
        const bool in = o >= first && o <= last;
        x[j] = in ? x[j] : -INFINITY;
        vm[j >> 1] &= in ? ~0u : ((j & 1) ? 0x0000FFFFu : 0xFFFF0000u);
      }
      vmask = u32x4{vm[0], vm[1], vm[2], vm[3]};
    }
    float mx = x[0];
#pragma unroll
    for (int j = 1; j < 8; ++j) mx = fmaxf(mx, x[j]);
    mx = col_max(mx);
    const float m_new = fmaxf(m_run, mx);  // finite: every tile holds a valid position
    const bool rescale = __any(m_new != m_run);  // rare once the maxima settle
    const float alpha = __builtin_amdgcn_exp2f(m_run - m_new);
    float p[8], ps = 0.f;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      p[j] = __builtin_amdgcn_exp2f(x[j] - m_new);
      ps += p[j];
    }
    l_run = l_run * alpha + ps;
    m_run = m_new;
    // P as two BF16 terms
    uint32_t h[4], l[4];
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      h[w] = f32x2_to_bf16x2(p[2 * w], p[2 * w + 1]);
      const float r0 = p[2 * w] - bf16_to_f32(h[w] & 0xFFFFu);
      const float r1 = p[2 * w + 1] - bf16_to_f32(h[w] >> 16);
      l[w] = f32x2_to_bf16x2(r0, r1);
    }
    const u32x4 ph = u32x4{h[0], h[1], h[2], h[3]}, pl = u32x4{l[0], l[1], l[2], l[3]};
    if (rescale) {
#pragma unroll
      for (int dt = 0; dt < 8; ++dt) acc[dt] *= alpha;
    }
    if (edge) {
#pragma unroll
      for (int dt = 0; dt < 8; ++dt) {
        const u32x4 vv = cur.v[dt] & vmask;
        acc[dt] = mfma16(vv, ph, acc[dt]);
        acc[dt] = mfma16(vv, pl, acc[dt]);
      }
    } else {
#pragma unroll
      for (int dt = 0; dt < 8; ++dt) {
        acc[dt] = mfma16(cur.v[dt], ph, acc[dt]);
        acc[dt] = mfma16(cur.v[dt], pl, acc[dt]);
      }
    }
  };
  if (t <= t1) {
    auto advance = [nst](int st) {
      st += kAttnWaves;
      while (st >= nst) st -= nst;
      return st;
    };
    for (;;) {
      const int64_t tb = t + kAttnWaves;
      const int sb = advance(sa);
      attn_load_tile(rb, kb, vb, tb <= t1 ? sb : sa, lane);
      tile_step(ra, t);
      if (tb > t1) break;
      const int64_t ta = tb + kAttnWaves;
      const int sa2 = advance(sb);
      attn_load_tile(ra, kb, vb, ta <= t1 ? sa2 : sb, lane);
      tile_step(rb, tb);
      if (ta > t1) break;
      t = ta;
      sa = sa2;
    }
  }
  l_run = col_sum(l_run);

  // merge the waves
  if (g == 0) {
    s_m[wave][r] = m_run;
    s_l[wave][r] = l_run;
  }
#pragma unroll
  for (int dt = 0; dt < 8; ++dt)
    *reinterpret_cast<f32x4 *>(&s_acc[wave][r][dt * 16 + g * 4]) = acc[dt];
  __syncthreads();

  // thread -> (head n, dims 4 d4 .. + 4)
  for (int idx = threadIdx.x; idx < G * (kAttnD / 4); idx += blockDim.x) {
    const int n = idx / (kAttnD / 4), d = (idx % (kAttnD / 4)) * 4;
    float M = -INFINITY;
#pragma unroll
    for (int w = 0; w < kAttnWaves; ++w) M = fmaxf(M, s_m[w][n]);
    float L = 0.f;
    f32x4 A = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int w = 0; w < kAttnWaves; ++w) {
      const float f = __builtin_amdgcn_exp2f(s_m[w][n] - M);  // 0 for a wave with no tile
      L += f * s_l[w][n];
      A += f * *reinterpret_cast<const f32x4 *>(&s_acc[w][n][d]);
    }
    if (a.chunks == 1) {
      const float sk = a.sinks ? a.sinks[kv * G + n] * kLog2e : -INFINITY;
      const float M2 = fmaxf(M, sk);
      const float f = __builtin_amdgcn_exp2f(M - M2);
      const float inv = 1.0f / (L * f + __builtin_amdgcn_exp2f(sk - M2));
      const f32x4 o = A * (f * inv);
      *reinterpret_cast<uint2 *>(outb + n * kAttnD + d) = uint2{f32x2_to_bf16x2(o[0], o[1]), f32x2_to_bf16x2(o[2], o[3])};
    } else {
      float *pp = a.part + (((int64_t)b * a.n_kv + kv) * a.chunks + c) * attn_part_floats(G);
      *reinterpret_cast<f32x4 *>(pp + n * kAttnD + d) = A;
      if (d == 0) {
        pp[G * kAttnD + n] = M;
        pp[G * kAttnD + G + n] = L;
      }
    }
  }
}

// Grid (n_q, B), 256 threads: merge one query head's chunk partials and
// apply its sink.  Thread (cg, col): column col of 32 four-dim columns,
// chunks cg, cg + 8, ...; the 8 chunk groups are summed through LDS.
constexpr int kCombineThreads = 256;

__global__ __launch_bounds__(kCombineThreads) void k_attn_combine(AttnDecodeArgs a) {
  constexpr int kGroups = kCombineThreads / 32;
  __shared__ float s_m[kCombineThreads / kWave], s_l[kGroups];
  __shared__ f32x4 s_acc[kGroups][32];
  const int h = blockIdx.x, b = blockIdx.y;
  const int G = a.G, kv = h / G, n = h % G;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  if (h == 0 && b == 0 && tid < kWave) {
    uint32_t bad = 0;
    for (int t = tid; t < a.B; t += kWave) {
      int64_t lo;
      bad |= attn_range(a.pos[t], a.window, a.slots, a.span, lo) ? 0u : (uint32_t)kStatusBadPos;
    }
    bad = wave_max_u32(bad);
    if (tid == 0) *a.status = bad;
  }
  const int64_t pos = a.pos[b];
  int64_t lo = 0;
  const bool ok = attn_range(pos, a.window, a.slots, a.span, lo);
  uint16_t *outh = a.out + ((int64_t)b * a.n_q + h) * kAttnD;
  const int cg = tid / 32, col = tid % 32;
  if (!ok) {
    if (tid < 32) *reinterpret_cast<uint2 *>(outh + col * 4) = uint2{0u, 0u};
    return;
  }
  const int64_t tiles = pos / kAttnTile - lo / kAttnTile + 1;
  const int nch = (int)((tiles + a.tpc - 1) / a.tpc);
  const int64_t pf = attn_part_floats(G);
  const float *pb = a.part + ((int64_t)b * a.n_kv + kv) * a.chunks * pf;
  const float sk = a.sinks ? a.sinks[h] * kLog2e : -INFINITY;

  // the largest chunk maximum, and the sink
  float m = -INFINITY;
  for (int ch = tid; ch < nch; ch += kCombineThreads) m = fmaxf(m, pb[ch * pf + G * kAttnD + n]);
  m = fmaxf(m, xor_lane<1>(m));
  m = fmaxf(m, xor_lane<2>(m));
  m = fmaxf(m, xor_lane<4>(m));
  m = fmaxf(m, xor_lane<8>(m));
  m = fmaxf(m, xor_lane<16>(m));
  m = fmaxf(m, xor_lane<32>(m));
  if (lane == 0) s_m[wave] = m;
  __syncthreads();
  float M = sk;
#pragma unroll
  for (int w = 0; w < kCombineThreads / kWave; ++w) M = fmaxf(M, s_m[w]);

  // chunk group cg sums chunks cg, cg + 8, ... (independent loads)
  float L = 0.f;
  f32x4 A = {0.f, 0.f, 0.f, 0.f};
  for (int ch = cg; ch < nch; ch += kGroups) {
    const float *pp = pb + ch * pf;
    const float f = __builtin_amdgcn_exp2f(pp[G * kAttnD + n] - M);
    L += f * pp[G * kAttnD + G + n];
    A += f * *reinterpret_cast<const f32x4 *>(pp + n * kAttnD + col * 4);
  }
  s_acc[cg][col] = A;
  if (col == 0) s_l[cg] = L;
  __syncthreads();
  if (tid < 32) {
    f32x4 S = {0.f, 0.f, 0.f, 0.f};
    float Lt = __builtin_amdgcn_exp2f(sk - M);
#pragma unroll
    for (int c = 0; c < kGroups; ++c) {
      S += s_acc[c][tid];
      Lt += s_l[c];
    }
    const f32x4 o = S * (1.0f / Lt);
    *reinterpret_cast<uint2 *>(outh + tid * 4) = uint2{f32x2_to_bf16x2(o[0], o[1]), f32x2_to_bf16x2(o[2], o[3])};
  }
}

// ---------------------------------------------------------------------------
hipError_t launch_attn_prep(const AttnPrepArgs &a, int B, hipStream_t stream) {
  const int units = a.n_q + 2 * a.n_kv;
  hipLaunchKernelGGL(k_attn_prep, dim3((units + 3) / 4, B), dim3(256), 0, stream, a);
  return hipGetLastError();
}

hipError_t launch_attn_kv_write(const AttnKvWriteArgs &a, int B, hipStream_t stream) {
  hipLaunchKernelGGL(k_attn_kv_write, dim3(a.n, B), dim3(256), 0, stream, a);
  return hipGetLastError();
}

hipError_t launch_attn_decode(const AttnDecodeArgs &a, hipStream_t stream) {
  if (a.fused)
    hipLaunchKernelGGL(k_attn_decode<true>, dim3(a.chunks, a.n_kv, a.B), dim3(kAttnWaves * kWave), 0, stream, a);
  else
    hipLaunchKernelGGL(k_attn_decode<false>, dim3(a.chunks, a.n_kv, a.B), dim3(kAttnWaves * kWave), 0, stream, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || a.chunks == 1) return e;
  hipLaunchKernelGGL(k_attn_combine, dim3(a.n_q, a.B), dim3(kCombineThreads), 0, stream, a);
  return hipGetLastError();
}

}  // namespace moe
