// Small-batch (1..8 tokens) decode path of the sigmoid-routed W4A16 MoE
// layer.  One token with routed experts runs the whole layer in one kernel
// (k_layer_b1), with the logits and h handed between its blocks through
// tagged words in memory.  Batches of 2..8 tokens and the dense layers run
// two to five kernels, their stages separated by kernel boundaries: on
// this GPU a device-scope atomic on one address serialises across blocks,
// an agent-scope fence writes back the L2, and data that many blocks read
// right after another block wrote it must come from memory rather than
// from each XCD's L2.
//
//   k_layer_b1 (one token, routed experts present) router rows, gate/up
//              units and down rows as three kinds of blocks of one kernel
//              (below); k_sync_clear zeroes its sync words once per call.
//   k_norm     (batches of 2..8 tokens with a pre-norm) one block per
//              token: xn = BF16(x * inv * gain), inv from an FP64 sum of
//              squares.
//   k_router   router GEMV l = W_r xn + b in FP32, the batch staged in LDS
//              (a dense layer of one token: only its pre-norm), one row
//              per lane group, each row loaded once for every token; its
//              last block (one wave per token) waits for the batch's
//              logits, published as tagged words, and derives the routing:
//              sigmoid top-k of every token, the sorted list of distinct
//              selected experts with token masks, the combine weights.
//   k_gateup   (dense layers, and batches with BF16 weights) its share of
//              the gate and up GEMVs of one selected (or the shared)
//              expert: FP4 decoded to BF16 in registers, FP32
//              accumulation, BF16 rounding of g and u, h = BF16(SiLU(g) u).
//   k_down     for every 4-row group of the output: the down GEMV of every
//              selected expert and of the shared expert, BF16 rounding per
//              expert, weighted FP32 combine in a fixed order, BF16 output
//              (plus the residual when asked).
//   k_gateup_mm, k_down_mm: the same two stages for batches of 2..8 tokens
//              with NVFP4 weights, on the matrix cores (below).
//
// What is computed follows "Day-0 Support for Flint on vLLM" (sections
// "Model architecture" and "Optimizations"): 256 experts, sigmoid top-6
// plus a shared expert; only the selected experts' weights are read;
// weight-only FP4 with BF16 activations; the reference's rounding points.
#include <hip/hip_ext.h>

#include "common.h"
#include "mm_rows.h"

namespace moe {

// ---------------------------------------------------------------------------
// Wave-level helpers
// ---------------------------------------------------------------------------

// Fold-reduce 4 values over aligned groups of W lanes (W a power of two,
// 2..64): step 1 exchanges two of them with lane ^ 1, step 2 one with
// lane ^ 2, then plain sums over the remaining lane bits; 2 + 1 + (log2(W)
// - 2) lane exchanges instead of 4 * log2(W).  Returns the group total of
// value index `row` = 2*(lane bit 0) + (lane bit 1) (with W == 2 the lane
// also keeps row + 1's total in *second).  Written on scalars so that no
// register array gets a runtime index.
__device__ __forceinline__ float fold4(float v0, float v1, float v2, float v3, int W, int &row, float *second) {
  const int lane = threadIdx.x & (kWave - 1);
  const bool u1 = (lane & 1) != 0, u2 = (lane & 2) != 0;
  // step o = 1: lower lanes keep values 0,1; upper lanes keep 2,3
  const float n0 = (u1 ? v2 : v0) + xor_lane<1>(u1 ? v0 : v2);
  const float n1 = (u1 ? v3 : v1) + xor_lane<1>(u1 ? v1 : v3);
  row = u1 ? 2 : 0;
  if (W <= 2) {
    if (second) *second = n1;
    return n0;
  }
  // step o = 2
  float r = (u2 ? n1 : n0) + xor_lane<2>(u2 ? n0 : n1);
  row += u2 ? 1 : 0;
  if (W > 4) r += xor_lane<4>(r);
  if (W > 8) r += xor_lane<8>(r);
  if (W > 16) r += xor_lane<16>(r);
  if (W > 32) r += xor_lane<32>(r);
  return r;
}

// Orderable 32-bit image of a logit: larger logit -> larger key; NaN ranks
// as -inf; 0 is below every real key and marks "taken / absent".
__device__ __forceinline__ uint32_t topk_key(float l) {
  if (l != l) l = -INFINITY;
  l += 0.0f;  // -0 -> +0: equal logits tie by index
  const uint32_t u = __float_as_uint(l);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

__device__ __forceinline__ float topk_key_logit(uint32_t u) {
  return __uint_as_float((u & 0x80000000u) ? (u & 0x7fffffffu) : ~u);
}

// Top-k experts of one token's logits by one wave: sel[0..k) in descending
// logit order, ties to the lower expert index; selv = their logits.  Lane l
// holds experts l*J .. l*J+J-1 (E <= 64*J), so the lowest expert index with
// a given key is in the lowest lane holding it.  Each round every lane
// first notes the first slot holding its own max and what its keys and max
// are without that slot (work independent of the wave max, which hides it);
// then the wave max of the lanes' maxima, one ballot for the lowest lane
// holding it, and that lane drops its slot.  Results are wave-uniform.
template <int J>
__device__ __forceinline__ void wave_topk(const float *lt, int E, int k, int (&sel)[kMaxTopK],
                                          float (&selv)[kMaxTopK]) {
  const int lane = threadIdx.x & (kWave - 1);
  // Clamped indices keep the J loads unconditional, so they are all in
  // flight together (a load under a bound test is issued and waited for one
  // at a time).
  float lv[J];
#pragma unroll
  for (int j = 0; j < J; ++j) {
    const int e = lane * J + j;
    lv[j] = lt[e < E ? e : E - 1];
  }
  uint32_t key[J];
#pragma unroll
  for (int j = 0; j < J; ++j) key[j] = (lane * J + j < E) ? topk_key(lv[j]) : 0u;
  uint32_t lmax = key[0];
#pragma unroll
  for (int j = 1; j < J; ++j) lmax = max(lmax, key[j]);
#pragma unroll
  for (int r = 0; r < kMaxTopK; ++r) {
    if (r < k) {
      int jm = J - 1;  // some slot holds lmax
#pragma unroll
      for (int j = J - 2; j >= 0; --j) jm = (key[j] == lmax) ? j : jm;
      uint32_t keyx[J], lx = 0u;
#pragma unroll
      for (int j = 0; j < J; ++j) {
        keyx[j] = (j == jm) ? 0u : key[j];
        lx = max(lx, keyx[j]);
      }
      // k <= E, so an untaken real key (> 0) remains and some lane holds m
      const uint32_t m = wave_max_u32(lmax);
      const int L = (int)__builtin_ctzll(__ballot(lmax == m));
      sel[r] = L * J + __builtin_amdgcn_readlane(jm, L);
      selv[r] = topk_key_logit(m);
      const bool mine = lane == L;
#pragma unroll
      for (int j = 0; j < J; ++j) key[j] = mine ? keyx[j] : key[j];
      lmax = mine ? lx : lmax;
    }
  }
}

// The same selection for E <= 256 (four experts per lane), with each
// lane's keys sorted once: every round is then the wave max of the lanes'
// first keys, one ballot for the lowest lane holding it, and that lane
// shifts its list by one.  The sort is odd-even transposition (adjacent
// exchanges on a strict comparison), so equal keys keep their index order
// and a lane's first key is its lowest-index expert among equals.
__device__ __forceinline__ void wave_topk4(const float *lt, int E, int k, int (&sel)[kMaxTopK],
                                           float (&selv)[kMaxTopK]) {
  const int lane = threadIdx.x & (kWave - 1);
  float lv[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int e = lane * 4 + j;
    lv[j] = lt[e < E ? e : E - 1];
  }
  uint32_t key[4];
  int idx[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    // the empty asm keeps the four loads unconditional and in flight
    // together (a load whose value only one side of the bound test uses
    // would otherwise move under that test, one wait per load)
    float l = lv[j];
    asm volatile("" : "+v"(l));
    key[j] = (lane * 4 + j < E) ? topk_key(l) : 0u;
    idx[j] = j;
  }
  auto cx = [&](int p, int q) __attribute__((always_inline)) {
    const bool sw = key[q] > key[p];
    const uint32_t kp = key[p], kq = key[q];
    const int ip = idx[p], iq = idx[q];
    key[p] = sw ? kq : kp;
    key[q] = sw ? kp : kq;
    idx[p] = sw ? iq : ip;
    idx[q] = sw ? ip : iq;
  };
  cx(0, 1); cx(2, 3);
  cx(1, 2);
  cx(0, 1); cx(2, 3);
  cx(1, 2);
#pragma unroll
  for (int r = 0; r < kMaxTopK; ++r) {
    if (r < k) {
      // k <= E, so an untaken real key (> 0) remains and some lane holds m
      const uint32_t m = wave_max_u32(key[0]);
      const int L = (int)__builtin_ctzll(__ballot(key[0] == m));
      sel[r] = L * 4 + __builtin_amdgcn_readlane(idx[0], L);
      selv[r] = topk_key_logit(m);
      const bool mine = lane == L;
      key[0] = mine ? key[1] : key[0];
      key[1] = mine ? key[2] : key[1];
      key[2] = mine ? key[3] : key[2];
      key[3] = mine ? 0u : key[3];
      idx[0] = mine ? idx[1] : idx[0];
      idx[1] = mine ? idx[2] : idx[1];
      idx[2] = mine ? idx[3] : idx[2];
    }
  }
}

__device__ __forceinline__ void wave_topk_any(const float *lt, int E, int k, int (&sel)[kMaxTopK],
                                              float (&selv)[kMaxTopK]) {
  if (E <= 4 * kWave) wave_topk4(lt, E, k, sel, selv);
  else wave_topk<kMaxExperts / kWave>(lt, E, k, sel, selv);
}

// ---------------------------------------------------------------------------
// Chunk math: one lane's 32-element chunk of kRows rows
// ---------------------------------------------------------------------------

constexpr int kRows = 4;  // rows per lane in the expert GEMVs

__device__ __forceinline__ void load16(const uint16_t *p, uint32_t (&x)[16]) {
  const uint4 *q = reinterpret_cast<const uint4 *>(p);
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const uint4 v = q[i];
    x[i * 4 + 0] = v.x;
    x[i * 4 + 1] = v.y;
    x[i * 4 + 2] = v.z;
    x[i * 4 + 3] = v.w;
  }
}

// Raw weights of kRows rows x one chunk as loaded from memory.
struct ChunkRaw {
  uint4 q[kRows][4];    // FP4 uses q[r][0] (16 bytes of nibbles); BF16 all four
  uint32_t scale[kRows];  // FP4: block scales of the row (byte 0: block 2c, byte 1: block 2c+1)
};

// Rows [r0, r0 + kRows) of matrix m (N x K), chunk c; r0 % 4 == 0.
template <int WT>
__device__ __forceinline__ void load_rows(const uint8_t *m, int64_t N, int64_t K, int r0, int c, ChunkRaw &cr) {
  if (WT == 1) {
    const int64_t rowb = K / 2;
    const uint8_t *p = m + (int64_t)r0 * rowb + (int64_t)c * 16;
#pragma unroll
    for (int r = 0; r < kRows; ++r) cr.q[r][0] = *reinterpret_cast<const uint4 *>(p + r * rowb);
    // 16-byte tile of rows 8g..8g+7: this lane's rows are its first or second half
    const uint4 t = *reinterpret_cast<const uint4 *>(m + N * K / 2 + ((int64_t)(r0 >> 3) * (K / 32) + c) * 16);
    const bool second = (r0 & 4) != 0;
    const uint32_t w0 = second ? t.z : t.x, w1 = second ? t.w : t.y;
    cr.scale[0] = w0 & 0xffffu;
    cr.scale[1] = w0 >> 16;
    cr.scale[2] = w1 & 0xffffu;
    cr.scale[3] = w1 >> 16;
  } else {
    const uint16_t *p = reinterpret_cast<const uint16_t *>(m) + (int64_t)r0 * K + (int64_t)c * 32;
#pragma unroll
    for (int r = 0; r < kRows; ++r) {
      const uint4 *q = reinterpret_cast<const uint4 *>(p + r * K);
#pragma unroll
      for (int i = 0; i < 4; ++i) cr.q[r][i] = q[i];
    }
  }
}

// Weights as 16 BF16 pairs per row plus FP32 block scales.
struct ChunkBF {
  uint32_t w[kRows][16];
  float s0[kRows], s1[kRows];
};

template <int WT>
__device__ __forceinline__ void convert_rows(const ChunkRaw &cr, ChunkBF &cb) {
#pragma unroll
  for (int r = 0; r < kRows; ++r) {
    if (WT == 1) {
      const uint32_t nw[4] = {cr.q[r][0].x, cr.q[r][0].y, cr.q[r][0].z, cr.q[r][0].w};
#pragma unroll
      for (int d = 0; d < 4; ++d) {
        cb.w[r][d * 4 + 0] = __builtin_bit_cast(uint32_t, MOE_FP4X2_TO_BF16X2(nw[d], 0));
        cb.w[r][d * 4 + 1] = __builtin_bit_cast(uint32_t, MOE_FP4X2_TO_BF16X2(nw[d], 1));
        cb.w[r][d * 4 + 2] = __builtin_bit_cast(uint32_t, MOE_FP4X2_TO_BF16X2(nw[d], 2));
        cb.w[r][d * 4 + 3] = __builtin_bit_cast(uint32_t, MOE_FP4X2_TO_BF16X2(nw[d], 3));
      }
      cb.s0[r] = e4m3_to_f32(cr.scale[r] & 0xffu);
      cb.s1[r] = e4m3_to_f32(cr.scale[r] >> 8);
    } else {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        cb.w[r][i * 4 + 0] = cr.q[r][i].x;
        cb.w[r][i * 4 + 1] = cr.q[r][i].y;
        cb.w[r][i * 4 + 2] = cr.q[r][i].z;
        cb.w[r][i * 4 + 3] = cr.q[r][i].w;
      }
      cb.s0[r] = 1.f;
      cb.s1[r] = 1.f;
    }
  }
}

// acc[r] += sum over the chunk of W[r][.] * x[.] (block scales applied).
template <int WT>
__device__ __forceinline__ void dot_rows(const ChunkBF &cb, const uint32_t (&x)[16], float (&acc)[kRows]) {
#pragma unroll
  for (int r = 0; r < kRows; ++r) {
    float p0 = 0.f, p1 = 0.f;
#pragma unroll
    for (int i = 0; i < 8; ++i) p0 = dot2_bf16(cb.w[r][i], x[i], p0);
#pragma unroll
    for (int i = 8; i < 16; ++i) p1 = dot2_bf16(cb.w[r][i], x[i], p1);
    acc[r] = (WT == 1) ? fmaf(cb.s0[r], p0, fmaf(cb.s1[r], p1, acc[r])) : acc[r] + (p0 + p1);
  }
}

// ---------------------------------------------------------------------------
// k_router: logits (and the pre-norm)
// ---------------------------------------------------------------------------

// Pre-norm of one token per block (batches of 2..8, where doing it once
// beats doing it in every router block): xn = BF16(x * inv * gain) with
// inv = 1/sqrt(mean(x^2) + eps), the sum of squares exact per term in FP64.
constexpr int kNormThreads = 256;

__global__ __launch_bounds__(kNormThreads) void k_norm(DecodeArgs a) {
  __shared__ double s_part[kNormThreads / kWave];
  const int H = a.H, t = blockIdx.x, n8 = H / 8;
  const int tid = threadIdx.x, lane = tid & (kWave - 1), wave = tid / kWave;
  const uint4 *xr = reinterpret_cast<const uint4 *>(a.x + (int64_t)t * H);
  const uint4 *gr = reinterpret_cast<const uint4 *>(a.norm_gain);
  // This thread's first piece of x and of the gain, loaded together up
  // front and kept for the second pass.
  uint4 x0 = make_uint4(0, 0, 0, 0), g0 = make_uint4(0, 0, 0, 0);
  if (tid < n8) {
    x0 = xr[tid];
    g0 = gr[tid];
  }
  double ss = 0.0;
  for (int i = tid; i < n8; i += kNormThreads) {
    const uint4 v = i == tid ? x0 : xr[i];
    const uint32_t q[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const double lo = bf16_to_f32(q[j] & 0xffffu), hi = bf16_to_f32(q[j] >> 16);
      ss = fma(lo, lo, fma(hi, hi, ss));
    }
  }
  ss = group_sum_f64(ss, kWave);
  if (lane == 0) s_part[wave] = ss;
  __syncthreads();
  double tot = 0.0;
#pragma unroll
  for (int w = 0; w < kNormThreads / kWave; ++w) tot += s_part[w];
  const double inv = 1.0 / sqrt(tot / (double)H + (double)a.eps);
  const float inv_f = (float)inv;
  for (int i = tid; i < n8; i += kNormThreads) {
    const uint4 v = i == tid ? x0 : xr[i], gv = i == tid ? g0 : gr[i];
    reinterpret_cast<uint4 *>(a.ws.xn + (int64_t)t * H)[i] = norm_piece_bf16(v, gv, inv_f, inv);
  }
}

// A value published for other blocks of the same kernel: the
// value's 32 bits with the layer call's tag above them, in one 64-bit
// agent-scope store.  A reader polls the word until it carries its own tag.
__device__ __forceinline__ void publish_tagged(uint64_t *p, uint32_t v, uint32_t tag) {
  __hip_atomic_store(p, (uint64_t)v | ((uint64_t)tag << 32), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

__device__ __forceinline__ uint64_t load_tagged(const uint64_t *p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

__device__ void route_block(const DecodeArgs &a, uint4 *lds);

// Router GEMV, W waves per block (4 for one token, 8 for batches).  The block first brings the batch's
// activations into LDS (at most 64 KiB): xn when k_norm already wrote it
// (xn_ready), else x, normalised there with a pre-norm (the sum of squares
// of each token in FP64 over the whole block, then every element
// BF16(x * inv * gain); block 0 also stores xn for the expert kernels, and
// every block computes the same bits).  Each lane group of LPR lanes then
// owns one router row, loaded once, and takes its dot product with every
// token from LDS; lane j of a group takes the 16-byte pieces j, j + LPR,
// ... of the row, so a wave's LDS and global accesses are contiguous.
constexpr int kRouterWaves = 4;
constexpr int kRouterThreads = kRouterWaves * kWave;
constexpr int kRouteWaves = kMaxBatchBf16;  // BF16 batches: one wave per token in the routing block

// MT: tokens a block handles.  kMaxBatchBf16: the whole batch (BF16
// weights), staged in 32768 / 8 16-byte pieces (B * H <= 32768).  1: one token of a
// batch of two or more, the batch split over blockIdx.y; its stage takes
// at most 16384 / 8 pieces (H <= 16384), and its per-token registers are a
// batch's eighth, so that several blocks fit on a compute unit.
template <int W, int MT>
__global__ __launch_bounds__(W *kWave) void k_router(DecodeArgs a, int xn_ready, int route) {
  constexpr int kRouterWaves = W, kRouterThreads = W * kWave;
  constexpr int XCAP = MT == 1 ? kRouterTokenMaxHidden / 8 : 32768 / 8;
  static_assert(XCAP * 16 >= 32768, "the routing block keeps B * E <= 8192 logits in the stage");
  __shared__ uint4 s_x[XCAP];  // [B][H] BF16
  __shared__ double s_ss[kRouterWaves][MT];
  if (route && blockIdx.x == gridDim.x - 1) {
    route_block(a, s_x);
    return;
  }
  if (a.zero0 && blockIdx.x == 0 && blockIdx.y == 0)
    for (int i = threadIdx.x; i < a.zero_n; i += kRouterThreads) {
      a.zero0[i] = 0;
      a.zero1[i] = 0;
    }
  if (MT == 1) {
    // the batch split over blockIdx.y, one token per block row: a block
    // takes its token's dot products only (a row's 16 pieces per lane
    // instead of 16 per token), the row weights are read once per token
    // from the L2
    const int t = blockIdx.y;
    a.x += (int64_t)t * a.H;
    a.ws.xn += (int64_t)t * a.H;
    a.ws.logits += (int64_t)t * a.E;
    a.B = 1;
  }
  const int H = a.H, E = a.E, B = a.B;
  const int LPR = lanes_per_row(H);
  const int tid = threadIdx.x, lane = tid & (kWave - 1), wave = tid / kWave, lg = lane % LPR;
  const int row = (blockIdx.x * kRouterWaves + wave) * (kWave / LPR) + lane / LPR;
  const int n8 = H / 8;  // 16-byte pieces per token row
  const bool norm_here = a.use_norm && !xn_ready;
  const uint16_t *src = xn_ready ? a.ws.xn : a.x;

  uint4 w0[4];
  float bias;
  if (norm_here && B > 1 && B <= kRouterWaves && n8 <= 8 * kWave) {
    // Batches (H <= 4096): one wave per token.  Wave t loads token t (lane l
    // the 16-byte pieces l, l + 64, ..., at most 8) and its gain, sums the
    // squares in FP64 over its pieces and then across the wave (every lane
    // ends with the same bits), forms 1/sqrt(mean + eps) itself and normalises its pieces into
    // LDS: one cross-lane reduction per wave and no cross-wave step before
    // the normalisation.  The token and the gain are requested before the
    // router row's first pieces: loads complete in issue order, so the norm
    // runs while the router weights are still on their way from memory.
    const int np = (n8 + kWave - 1) / kWave;
    const bool tok = wave < B;
    // (indices clamped into the buffers: every load is unconditional, so
    // the waits before the norm cover the token and the gain only)
    const uint4 *xr = reinterpret_cast<const uint4 *>(a.x + (int64_t)(tok ? wave : 0) * H);
    const uint4 *gr = reinterpret_cast<const uint4 *>(a.norm_gain);
    // a layer without routed experts has no router: its row loads read the
    // token instead (valid memory) and are discarded
    const uint4 *wr = E > 0 ? reinterpret_cast<const uint4 *>(a.router_w + (int64_t)(row < E ? row : E - 1) * H) : xr;
    uint4 xv[8], gv[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) xv[j] = xr[min(lane + j * kWave, n8 - 1)];
#pragma unroll
    for (int j = 0; j < 8; ++j) gv[j] = gr[min(lane + j * kWave, n8 - 1)];
#pragma unroll
    for (int i = 0; i < 4; ++i) w0[i] = wr[min(lg + i * LPR, n8 - 1)];
    // pieces past the token (clamped duplicates) take no part in the sums
#pragma unroll
    for (int j = 0; j < 8; ++j)
      if (!(j < np && lane + j * kWave < n8)) xv[j] = make_uint4(0, 0, 0, 0);
#pragma unroll
    for (int i = 0; i < 4; ++i)
      if (!(row < E && lg + i * LPR < n8)) w0[i] = make_uint4(0, 0, 0, 0);
    bias = (a.router_b && E > 0) ? a.router_b[row < E ? row : E - 1] : 0.f;
    if (row >= E) bias = 0.f;
    if (tok) {
      double ss = 0.0;
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const uint32_t q[4] = {xv[j].x, xv[j].y, xv[j].z, xv[j].w};
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const double lo = bf16_to_f32(q[e] & 0xffffu), hi = bf16_to_f32(q[e] >> 16);
          ss = fma(lo, lo, fma(hi, hi, ss));
        }
      }
      ss = group_sum_f64(ss, kWave);
      const double inv = 1.0 / sqrt(ss / (double)H + (double)a.eps);
      const float inv_f = (float)inv;
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const int i = lane + j * kWave;
        if (j < np && i < n8) {
          const uint4 o = norm_piece_bf16(xv[j], gv[j], inv_f, inv);
          s_x[wave * n8 + i] = o;
          if (blockIdx.x == 0) reinterpret_cast<uint4 *>(a.ws.xn + (int64_t)wave * H)[i] = o;
        }
      }
    }
    __syncthreads();
  } else {
    // Loads in the order they are needed (memory operations complete in
    // issue order): this thread's first piece of every token and of the
    // norm gain (the staging and the norm start as soon as they land), then
    // the first four pieces of this lane's router row and the row's bias,
    // which arrive from memory while the norm runs.
    // (indices clamped into the buffers: every load is unconditional)
    const int tc = tid < n8 ? tid : n8 - 1;
    uint4 v0[MT];
#pragma unroll
    for (int t = 0; t < MT; ++t)
      if (t < B) v0[t] = reinterpret_cast<const uint4 *>(src + (int64_t)t * H)[tc];
    uint4 g0 = make_uint4(0, 0, 0, 0);
    if (norm_here) g0 = reinterpret_cast<const uint4 *>(a.norm_gain)[tc];
    // a layer without routed experts (the pre-norm alone) has no router: its
    // row loads read the token instead (valid memory) and are discarded
    const uint4 *wr = E > 0 ? reinterpret_cast<const uint4 *>(a.router_w + (int64_t)(row < E ? row : E - 1) * H)
                            : reinterpret_cast<const uint4 *>(src);
#pragma unroll
    for (int i = 0; i < 4; ++i) w0[i] = wr[min(lg + i * LPR, n8 - 1)];
#pragma unroll
    for (int i = 0; i < 4; ++i)
      if (!(row < E && lg + i * LPR < n8)) w0[i] = make_uint4(0, 0, 0, 0);
    bias = (a.router_b && E > 0) ? a.router_b[row < E ? row : E - 1] : 0.f;
    if (row >= E) bias = 0.f;

    // 1. activations -> LDS; sums of squares (exact per term in FP64).  A
    // thread's pieces of every token are loaded before any is stored, so the
    // loads are in flight together.
    double ss[MT];
#pragma unroll
    for (int t = 0; t < MT; ++t) ss[t] = 0.0;
    for (int i = tid; i < n8; i += kRouterThreads) {
      uint4 v[MT];
#pragma unroll
      for (int t = 0; t < MT; ++t)
        if (t < B) v[t] = i == tid ? v0[t] : reinterpret_cast<const uint4 *>(src + (int64_t)t * H)[i];
#pragma unroll
      for (int t = 0; t < MT; ++t) {
        if (t >= B) break;
        s_x[t * n8 + i] = v[t];
        if (norm_here) {
          const uint32_t q[4] = {v[t].x, v[t].y, v[t].z, v[t].w};
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            const double lo = bf16_to_f32(q[j] & 0xffffu), hi = bf16_to_f32(q[j] >> 16);
            ss[t] = fma(lo, lo, fma(hi, hi, ss[t]));
          }
        }
      }
    }
    if (norm_here) {
#pragma unroll
      for (int t = 0; t < MT; ++t) {
        if (t >= B) break;
        const double v = group_sum_f64(ss[t], kWave);
        if (lane == 0) s_ss[wave][t] = v;
      }
    }
    __syncthreads();

    // 2. pre-norm in LDS: xn = BF16(x * inv * gain)
    if (norm_here) {
      // one thread per token forms 1/sqrt(mean(x^2) + eps) in FP64
      if (tid < B) {
        double tot = 0.0;
#pragma unroll
        for (int w = 0; w < kRouterWaves; ++w) tot += s_ss[w][tid];
        s_ss[0][tid] = 1.0 / sqrt(tot / (double)H + (double)a.eps);
      }
      __syncthreads();
      double inv[MT];
#pragma unroll
      for (int t = 0; t < MT; ++t) inv[t] = t < B ? s_ss[0][t] : 1.0;
      for (int i = tid; i < n8; i += kRouterThreads) {
        const uint4 gv = i == tid ? g0 : reinterpret_cast<const uint4 *>(a.norm_gain)[i];
        const uint32_t g[4] = {gv.x, gv.y, gv.z, gv.w};
#pragma unroll
        for (int t = 0; t < MT; ++t) {
          if (t >= B) break;
          const float inv_f = (float)inv[t];
          const uint4 o = norm_piece_bf16(s_x[t * n8 + i], gv, inv_f, inv[t]);
          s_x[t * n8 + i] = o;
          if (blockIdx.x == 0) reinterpret_cast<uint4 *>(a.ws.xn + (int64_t)t * H)[i] = o;
        }
      }
      __syncthreads();
    }
  }

  // 3. router row x every token
  if (row >= E) return;
  float acc[MT];
#pragma unroll
  for (int t = 0; t < MT; ++t) acc[t] = 0.f;
  for (int j0 = lg; j0 < n8; j0 += 4 * LPR) {
    uint4 w[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int j = j0 + i * LPR;
      if (j0 == lg) w[i] = w0[i];
      else w[i] = j < n8 ? reinterpret_cast<const uint4 *>(a.router_w + (int64_t)row * H)[j] : make_uint4(0, 0, 0, 0);
    }
#pragma unroll
    for (int t = 0; t < MT; ++t) {
      if (t >= B) break;
      float s = acc[t];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int j = j0 + i * LPR;
        if (j < n8) {
          const uint4 v = s_x[t * n8 + j];
          s = dot2_bf16(w[i].x, v.x, s);
          s = dot2_bf16(w[i].y, v.y, s);
          s = dot2_bf16(w[i].z, v.z, s);
          s = dot2_bf16(w[i].w, v.w, s);
        }
      }
      acc[t] = s;
    }
  }
#pragma unroll
  for (int t = 0; t < MT; ++t) {
    if (t >= B) break;
    const float v = group_sum(acc[t], LPR);
    if (lg == 0) {
      if (route) publish_tagged(a.ws.sync_l + t * E + row, __float_as_uint(v + bias), a.tag);
      else a.ws.logits[t * E + row] = v + bias;
    }
  }
}

// ---------------------------------------------------------------------------
// Routing: top-k per token and the sorted list of distinct experts
// ---------------------------------------------------------------------------

struct Routing {
  int n;                                // distinct selected experts
  int expert[kMaxBatch * kMaxTopK];     // ascending expert id
  uint32_t mask[kMaxBatch * kMaxTopK];  // bit t: token t selected it
  int sel[kMaxBatch][kMaxTopK];         // per token, descending score
  float w[kMaxBatch][kMaxTopK];         // renormalised sigmoid weights
};

// Top-k of every token (one wave per token), its weights, and the sorted
// list of distinct experts, from logits [B][E].  Every caller derives the
// same list from the same logits.
__device__ inline void build_routing(const DecodeArgs &a, const float *logits, Routing &R, uint32_t *s_mark,
                                     int nwaves) {
  const int wave = threadIdx.x / kWave, lane = threadIdx.x & (kWave - 1);
  const bool single = a.B == 1;
  if (!single)
    for (int e = threadIdx.x; e < a.E; e += nwaves * kWave) s_mark[e] = 0u;
  __syncthreads();
  for (int t = wave; t < a.B; t += nwaves) {
    int sel[kMaxTopK];
    float selv[kMaxTopK];
    wave_topk_any(logits + t * a.E, a.E, a.k, sel, selv);
    // lane r < k handles selection r
    int e = sel[0];
    float l = selv[0];
#pragma unroll
    for (int r = 1; r < kMaxTopK; ++r) {
      e = (lane == r) ? sel[r] : e;
      l = (lane == r) ? selv[r] : l;
    }
    // sigmoid from the hardware base-2 exponential and reciprocal (about
    // 1 ulp each); the sum over lanes 0..7 (0 past k), the same bits in
    // each of them
    const float sg = (lane < a.k) ? __builtin_amdgcn_rcpf(1.0f + __builtin_amdgcn_exp2f(-l * 1.44269504088896341f))
                                  : 0.f;
    float sum = sg + xor_lane<1>(sg);
    sum += xor_lane<2>(sum);
    sum += xor_lane<4>(sum);
    if (lane < a.k) {
      R.sel[t][lane] = e;
      R.w[t][lane] = sg / sum;  // a correctly rounded division: one expert gets exactly 1
      if (single) {
        // one token: the distinct list is the selection sorted by index
        int rank = 0;
#pragma unroll
        for (int r = 0; r < kMaxTopK; ++r) rank += (r < a.k && sel[r] < e) ? 1 : 0;
        R.expert[rank] = e;
        R.mask[rank] = 1u;
      } else {
        atomicOr(&s_mark[e], 1u << t);
      }
    }
    if (single && lane == 0) R.n = a.k;
  }
  __syncthreads();
  if (!single) {
    if (wave == 0) {
      int count = 0;
      for (int base = 0; base < a.E; base += kWave) {
        const int e = base + lane;
        const uint32_t m = (e < a.E) ? s_mark[e] : 0u;
        const unsigned long long ball = __ballot(m != 0u);
        if (m) {
          const int slot = count + __popcll(ball & ((1ull << lane) - 1ull));
          R.expert[slot] = e;
          R.mask[slot] = m;
        }
        count += __popcll(ball);
      }
      if (lane == 0) R.n = count;
    }
    __syncthreads();
  }
}

// Top-k outputs, the entry list and the combine weight of every (entry,
// token) pair, for the down kernel.
__device__ inline void publish_routing(const DecodeArgs &a, const Routing &R) {
  const int tid = threadIdx.x;
  for (int i = tid; i < a.B * a.k; i += blockDim.x) {
    const int t = i / a.k, r = i % a.k;
    a.out_idx[i] = R.sel[t][r];
    a.out_w[i] = R.w[t][r];
  }
  for (int i = tid; i < R.n * kMaxBatch; i += blockDim.x) {
    const int j = i / kMaxBatch, t = i % kMaxBatch;
    float w = 0.f;
    if (t < a.B && ((R.mask[j] >> t) & 1u))
      for (int r = 0; r < a.k; ++r)
        if (R.sel[t][r] == R.expert[j]) w = R.w[t][r];
    a.ws.entry_w[i] = w;
    if (t == 0) {
      a.ws.entry_expert[j] = R.expert[j];
      a.ws.entry_mask[j] = R.mask[j];
    }
  }
  if (tid == 0) *a.ws.n_routed = R.n;
}

// ---------------------------------------------------------------------------
// k_gateup: each lane group computes 4 rows of h for one expert
// ---------------------------------------------------------------------------

constexpr int kGateupWaves = 4;

// acc[t][r] += W[r0 + r][chunk c] . x_t[chunk c] for the tokens of `mask`.
template <int WT, int MAXT>
__device__ __forceinline__ void dot_tokens(const ChunkBF &cb, const uint16_t *xs, int H, int c, uint32_t mask, int B,
                                  float (&acc)[MAXT][kRows]) {
  StaticFor<0, MAXT>::run([&](auto tc) __attribute__((always_inline)) {
    constexpr int t = decltype(tc)::value;
    if (t < B && ((mask >> t) & 1u)) {
      uint32_t x[16];
      load16(xs + (int64_t)t * H + c * 32, x);
      dot_rows<WT>(cb, x, acc[t]);
    }
  });
}

// Gate/up GEMVs of block `bid`: 4-row units of the selected experts, then
// of the shared expert, on the activations xs ([B][H] BF16, global memory
// or LDS).  PUB (one token): R already holds the routing, and h is
// published as tagged words for the down blocks of the same kernel.
// Otherwise, with routed experts, the routing kernel wrote the list.
template <int WT, int MAXT, bool PUB>
__device__ __forceinline__ void gateup_block(const DecodeArgs &a, int bid, Routing &R, const uint16_t *xs) {
  static_assert(!PUB || MAXT == 1, "published h is the one-token layout");
  const int H = a.H, I = a.I, B = a.B;
  const int LPR = lanes_per_row(H), C = H / 32;
  const int groups = kGateupWaves * (kWave / LPR);
  const int lane = threadIdx.x & (kWave - 1), lg = lane % LPR;
  const int u = bid * groups + threadIdx.x / LPR;  // 4-row unit of this lane group
  const int routed_units = a.max_routed * (I / kRows);

  if (!PUB && a.E > 0 && bid * groups < routed_units) {
    if (threadIdx.x == 0) R.n = *a.ws.n_routed;
    for (int j = threadIdx.x; j < a.max_routed; j += blockDim.x) {
      R.expert[j] = a.ws.entry_expert[j];
      R.mask[j] = a.ws.entry_mask[j];
    }
    __syncthreads();
  }

  int slot = 0, q = 0, N = 0;
  uint32_t mask = 0;
  const uint8_t *Wg = nullptr, *Wu = nullptr;
  float Sg = 1.f, Su = 1.f;
  if (u < routed_units) {
    slot = u / (I / kRows);
    q = u % (I / kRows);
    if (slot < R.n) {
      const int e = R.expert[slot];
      mask = R.mask[slot];
      N = I;
      const int64_t mb = (WT == 1) ? nvfp4_matrix_bytes(I, H) : (int64_t)I * H * 2;
      Wg = a.w_gate + e * mb;
      Wu = a.w_up + e * mb;
      if (WT == 1) {
        Sg = a.w_scale[3 * e + 0];
        Su = a.w_scale[3 * e + 1];
      }
    }
  } else if (u - routed_units < a.Is / kRows) {
    slot = a.max_routed;
    q = u - routed_units;
    mask = (1u << B) - 1u;
    N = a.Is;
    Wg = a.sh_gate;
    Wu = a.sh_up;
    if (WT == 1) {
      Sg = a.sh_scale[0];
      Su = a.sh_scale[1];
    }
  }

  float ag[MAXT][kRows], au[MAXT][kRows];
#pragma unroll
  for (int t = 0; t < MAXT; ++t)
#pragma unroll
    for (int r = 0; r < kRows; ++r) ag[t][r] = au[t][r] = 0.f;
  if (mask) {
    for (int c = lg; c < C; c += LPR) {
      ChunkRaw rg, ru;
      load_rows<WT>(Wg, N, H, q * kRows, c, rg);
      load_rows<WT>(Wu, N, H, q * kRows, c, ru);
      ChunkBF cb;
      convert_rows<WT>(rg, cb);
      dot_tokens<WT, MAXT>(cb, xs, H, c, mask, B, ag);
      convert_rows<WT>(ru, cb);
      dot_tokens<WT, MAXT>(cb, xs, H, c, mask, B, au);
    }
  }
  // Per token: fold the 4 gate rows, then the 4 up rows, over the lane
  // group; lanes 0..3 of the group end up with one row each (the same row
  // for gate and up), and write h.
  const int Imax = a.I > a.Is ? a.I : a.Is;
  StaticFor<0, MAXT>::run([&](auto tc) __attribute__((always_inline)) {
    constexpr int t = decltype(tc)::value;
    if (t < B) {
      int row;
      float g2 = 0.f, u2 = 0.f;
      const float gs = fold4(ag[t][0], ag[t][1], ag[t][2], ag[t][3], LPR, row, &g2);
      const float us = fold4(au[t][0], au[t][1], au[t][2], au[t][3], LPR, row, &u2);
      if constexpr (PUB) {
        // rows (row, row + 1) in one word: with 2-lane groups a lane holds
        // both; otherwise lanes 0 and 1 of the group (rows 0 and 2) take
        // rows 1 and 3 from lanes 2 and 3
        const uint32_t h0 = f32_to_bf16(silu_mul(round_bf16(gs * Sg), round_bf16(us * Su)));
        uint32_t h1;
        if (LPR == 2) h1 = f32_to_bf16(silu_mul(round_bf16(g2 * Sg), round_bf16(u2 * Su)));
        else h1 = xor_lane<2>(h0);
        if (lg < 2 && mask)
          publish_tagged(a.ws.sync_h + ((int64_t)slot * Imax + q * kRows + row) / 2, h0 | (h1 << 16), a.tag);
      } else if (lg < (LPR == 2 ? 2 : kRows) && ((mask >> t) & 1u)) {
        // with 2-lane groups each lane holds two rows
        for (int k2 = 0; k2 < (LPR == 2 ? 2 : 1); ++k2) {
          const float g = round_bf16((k2 ? g2 : gs) * Sg);
          const float uu = round_bf16((k2 ? u2 : us) * Su);
          const float h = silu_mul(g, uu);
          a.ws.h[((int64_t)slot * B + t) * Imax + q * kRows + row + k2] = (uint16_t)f32_to_bf16(h);
        }
      }
    }
  });
}

template <int WT, int MAXT>
__global__ __launch_bounds__(kGateupWaves *kWave) void k_gateup(DecodeArgs a) {
  __shared__ Routing R;
  gateup_block<WT, MAXT, false>(a, blockIdx.x, R, a.use_norm ? a.ws.xn : a.x);
}

// ---------------------------------------------------------------------------
// Batches of 2..8 tokens with NVFP4 weights: the expert GEMVs on the matrix
// cores (v_mfma_f32_16x16x32_bf16, weights as the 16-row A operand, the
// tokens as the 16 columns of B, padded with zeros).  Each weight element
// is dequantised once, and the per-token work moves from the vector ALUs
// to the matrix cores.
//   Operand layout (checked on the GPU): A lane l holds row l%16, K
//   elements (l/16)*8 .. +8; B lane l holds column l%16, the same K; C lane
//   l value i is row (l/16)*4 + i, column l%16.
//   K order: in a 128-K super-step lane part p = l/16 takes the 32-element
//   chunk c = 4*ss + p (16 contiguous bytes of FP4 per weight row) and MFMA
//   step s uses its elements s*8 .. +8, for A and B alike.
// ---------------------------------------------------------------------------

constexpr int kMmRows = 64;  // gate/up weight rows per block (four 16-row groups)

// Scale pair (blocks 2c, 2c+1) of row n of an N x K NVFP4 matrix.
__device__ __forceinline__ uint32_t scale_pair(const uint8_t *m, int64_t N, int64_t K, int n, int c) {
  return *reinterpret_cast<const uint16_t *>(m + N * K / 2 + ((int64_t)(n >> 3) * (K / 32) + c) * 16 + (n & 7) * 2);
}

// One gate/up work item: rows [row0, row0 + 16 RG) of one entry (a
// selected expert, or the shared one) times the batch's tokens.  RG:
// 16-row groups per item (4, or 2 when the items of 64 rows outnumber the
// blocks).
template <int RG>
__device__ __forceinline__ void gateup_item(const DecodeArgs &a, const Routing &R, float (&s_red)[kMmWaves][32][kWave],
                                            const uint16_t *xs, int item, int groups, int sh_groups) {
  const int H = a.H, B = a.B;
  const int Imax = a.I > a.Is ? a.I : a.Is;
  const bool shared = item < sh_groups;
  const int slot = shared ? a.max_routed : (item - sh_groups) / groups;
  const int row0 = (shared ? item : (item - sh_groups) % groups) * (16 * RG);
  const uint8_t *Wg, *Wu;
  float Sg, Su;
  uint32_t mask;
  int N;
  if (!shared) {
    const int e = R.expert[slot];
    mask = R.mask[slot];
    N = a.I;
    const int64_t mb = nvfp4_matrix_bytes(a.I, H);
    Wg = a.w_gate + e * mb;
    Wu = a.w_up + e * mb;
    Sg = a.w_scale[3 * e + 0];
    Su = a.w_scale[3 * e + 1];
  } else {
    mask = (1u << B) - 1u;
    N = a.Is;
    Wg = a.sh_gate;
    Wu = a.sh_up;
    Sg = a.sh_scale[0];
    Su = a.sh_scale[1];
  }
  if (row0 >= N) return;  // block-uniform
  const int col = threadIdx.x & 15;
  uint16_t *h = a.ws.h + (int64_t)slot * B * Imax;
  mm_rows<RG, true>(H, xs, B, H, col < B ? col : -1, Wg, Wu, Sg, Su, N, row0, mask, s_red,
                    [&](int t, int n, uint32_t v) { h[(int64_t)t * Imax + n] = (uint16_t)v; });
}

// Gate/up of a batch.  With routed experts every block first derives the
// routing from the logits (one wave per token: the top-k, then the sorted
// list of distinct experts), so no separate routing stage runs between the
// router kernel and this one; block 0 also publishes the list, the combine
// weights and the top-k outputs for the down kernel.  Work items are
// (entry, row group) pairs, the shared expert's first (they need no
// routing), then the distinct selected experts'; blocks take items in
// turn.
__global__ __launch_bounds__(kMmWaves *kWave) void k_gateup_mm(DecodeArgs a) {
  __shared__ float s_red[kMmWaves][32][kWave];  // before the first item: the logits and marks of the routing
  __shared__ Routing R;
  const int B = a.B;
  const int Imax = a.I > a.Is ? a.I : a.Is;
  const int tid = threadIdx.x;
  int n_routed = 0;
  if (a.E > 0) {
    float *s_l = &s_red[0][0][0];                                   // [B][E]
    uint32_t *s_mark = reinterpret_cast<uint32_t *>(s_l + B * a.E);  // [E]; (B + 1) E <= 16384 floats
    for (int i = tid; i < B * a.E; i += kMmWaves * kWave) s_l[i] = a.ws.logits[i];
    build_routing(a, s_l, R, s_mark, kMmWaves);  // ends with a barrier
    if (blockIdx.x == 0) publish_routing(a, R);
    n_routed = R.n;
  }
  const uint16_t *xs = a.use_norm ? a.ws.xn : a.x;
  // Items of 64 rows while they fit the grid; 32-row items when they would
  // leave some blocks two 64-row items and others none (the routing, the
  // same in every block, makes the choice the same everywhere).
  const int groups = (Imax + 63) / 64, sh_groups = a.Is > 0 ? (a.Is + 63) / 64 : 0;
  const int n_items = sh_groups + n_routed * groups;
  if (n_items <= (int)gridDim.x) {
    for (int item = blockIdx.x; item < n_items; item += gridDim.x) gateup_item<4>(a, R, s_red, xs, item, groups, sh_groups);
  } else {
    const int groups2 = (Imax + 31) / 32, sh_groups2 = a.Is > 0 ? (a.Is + 31) / 32 : 0;
    const int n_items2 = sh_groups2 + n_routed * groups2;
    for (int item = blockIdx.x; item < n_items2; item += gridDim.x)
      gateup_item<2>(a, R, s_red, xs, item, groups2, sh_groups2);
  }
}

// One piece (two 128-K super-steps of each K half) of one entry's down
// weights and h, as one lane loads it.
template <int G>
struct DnPiece {
  uint4 q[2], hv[G][2][4];
  uint32_t sp[2];
  float sd, w[G];  // the entry's FP32 tensor scale and this lane's token weight per token group
};

// Down and combine: block = 8 output rows; the 8 waves take the entries
// (selected experts, then the shared expert) in turn, each over the full K,
// with the loads of the next units in flight.
//   The 16x16 MFMA tile is split in two along K: A row m holds weight row
//   m & 7 over K half m >> 3, B column n holds token 8g + (n & 7) of token
//   group g over K half n >> 3, so the C entries with m >> 3 == n >> 3 are
//   the two half-K products of (row, token) and the rest are discarded;
//   lane l and lane l ^ 40 hold the two halves.  G token groups (1 for up
//   to 8 tokens, 2 for up to 16) share each dequantised A fragment.  8-row
//   blocks put H/8 blocks on the GPU, each owning its rows outright (no
//   cross-block combine).
template <int G>
__global__ __launch_bounds__(kMmWaves *kWave) void k_down_mm(DecodeArgs a) {
  // A ring of RING pieces: every unit's loads are issued RING - 1 units
  // ahead of its math (a wave's entries at the full batch-8 shape, about
  // four, are then all in flight at once).
  constexpr int RING = G == 1 ? 4 : 2;
  __shared__ float s_red[kMmWaves][G][4][kWave];
  const int H = a.H, B = a.B;
  const int K = (a.E > 0) ? a.I : a.Is;  // Is == I when both exist
  const int C = K / 32, C2 = (C + 1) / 2, NP = (C2 + 7) / 8;  // chunks per K half; 8-chunk pieces
  const int Imax = a.I > a.Is ? a.I : a.Is;
  const int tid = threadIdx.x, lane = tid & (kWave - 1), wave = tid / kWave;
  const int m = lane & 15, p = lane >> 4, r8 = m & 7, kh = m >> 3;
  const int row0 = blockIdx.x * 8;
  const int n = row0 + r8;
  const int64_t mbytes = nvfp4_matrix_bytes(H, K);
  float tot[G][4];
#pragma unroll
  for (int g = 0; g < G; ++g) tot[g][0] = tot[g][1] = tot[g][2] = tot[g][3] = 0.f;
  // The entry arrays hold max_routed slots: the first 64 of this wave's
  // slots are read together with the count.
  int e_l = -1;
  uint32_t m_l = 0u;
  if (wave + lane * kMmWaves < a.max_routed) {
    e_l = a.ws.entry_expert[wave + lane * kMmWaves];
    m_l = a.ws.entry_mask[wave + lane * kMmWaves];
  }
  const int n_routed = (a.E > 0) ? *a.ws.n_routed : 0;
  const int n_entries = n_routed + (a.Is > 0 ? 1 : 0);
  const int mine = wave < n_entries ? (n_entries - wave + kMmWaves - 1) / kMmWaves : 0;
  const __amdgpu_buffer_rsrc_t hr = buf_rsrc(a.ws.h, (int64_t)(a.max_routed + 1) * B * Imax * 2);
  const __amdgpu_buffer_rsrc_t ewr = buf_rsrc(a.ws.entry_w, (int64_t)a.max_routed * kMaxBatch * 4);

  for (int i0 = 0; i0 < mine; i0 += kWave) {
    // lane i holds the expert (-1: shared) and token mask of this wave's
    // entry i0 + i
    {
      const int j = wave + (i0 + lane) * kMmWaves;
      if (i0 > 0 && j < n_routed) {
        e_l = a.ws.entry_expert[j];
        m_l = a.ws.entry_mask[j];
      }
      if (j >= n_routed) {
        e_l = -1;
        m_l = (1u << B) - 1u;
      }
    }
    const int cnt = min(mine - i0, kWave), nu = cnt * NP;
    // Units u >= nu in the ring's first pass load the last unit again (no
    // load of that pass depends on a branch) and are not multiplied.
    auto load = [&](int u, DnPiece<G> &L) __attribute__((always_inline)) {
      const int uu = u < nu ? u : nu - 1;
      const int ii = uu / NP, pc = uu - ii * NP;
      const int e = __builtin_amdgcn_readlane(e_l, ii);
      const uint32_t msk = (uint32_t)__builtin_amdgcn_readlane((int)m_l, ii);
      const int j = wave + (i0 + ii) * kMmWaves;
      const uint8_t *Wd = e >= 0 ? a.w_down + e * mbytes : a.sh_down;
      const __amdgpu_buffer_rsrc_t wr = buf_rsrc(Wd, mbytes);
      const int slot = e >= 0 ? j : a.max_routed;
      L.sd = *(e >= 0 ? a.w_scale + 3 * e + 2 : a.sh_scale + 2);
      const int t = lane & 15;  // C column of this lane after the MFMAs: token 8g + (t & 7)
#pragma unroll
      for (int g = 0; g < G; ++g) {
        const int tc = 8 * g + (t & 7);
        const bool wt = tc < B && ((msk >> tc) & 1u);
        const float ew = buf_load4f(ewr, (uint32_t)(j * kMaxBatch + tc) * 4u);
        L.w[g] = wt ? (e >= 0 ? ew : 1.0f) : 0.f;
      }
#pragma unroll
      for (int v = 0; v < 2; ++v) {
        const int cc = (pc * 2 + v) * 4 + p;  // chunk within this lane's K half
        const int c = kh * C2 + cc;
        const bool cok = cc < C2 && c < C;
        L.q[v] = buf_load16(wr, buf_off(cok, (uint32_t)(n * (K / 2) + c * 16)));
        L.sp[v] = buf_load2(wr, buf_off(cok, (uint32_t)(H * K / 2 + ((n >> 3) * (K / 32) + c) * 16 + (n & 7) * 2)));
#pragma unroll
        for (int g = 0; g < G; ++g) {
          const int tb = 8 * g + r8;  // B column m: token 8g + (m & 7)
          const bool tok = tb < B && ((msk >> tb) & 1u);
          const uint32_t hrow = (uint32_t)((slot * B + tb) * Imax) * 2u;
#pragma unroll
          for (int s = 0; s < 4; ++s)
            L.hv[g][v][s] = buf_load16(hr, buf_off(cok && tok, hrow + (uint32_t)(c * 32 + s * 8) * 2u));
        }
      }
    };
    f32x4 acc[G];
#pragma unroll
    for (int g = 0; g < G; ++g) acc[g] = f32x4{0.f, 0.f, 0.f, 0.f};
    auto step = [&](int u, const DnPiece<G> &L) __attribute__((always_inline)) {
      const int pc = u - (u / NP) * NP;
#pragma unroll
      for (int v = 0; v < 2; ++v)
#pragma unroll
        for (int s = 0; s < 4; ++s) {
          const float sc = e4m3_to_f32((L.sp[v] >> (8 * (s >> 1))) & 0xffu);
          const bf16x8 af = dq8(word_of(L.q[v], s), sc);
#pragma unroll
          for (int g = 0; g < G; ++g)
            acc[g] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                af, __builtin_bit_cast(bf16x8, u32x4{L.hv[g][v][s].x, L.hv[g][v][s].y, L.hv[g][v][s].z, L.hv[g][v][s].w}),
                acc[g], 0, 0, 0);
        }
      if (pc == NP - 1) {
        // entry done: lanes l < 32 with l & 8 == 0 add the other K half
        // (lane l ^ 40) and hold rows (l/16)*4 + i of token 8g + (l & 7)
#pragma unroll
        for (int g = 0; g < G; ++g) {
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const float full = acc[g][i] + xor_lane<8>(xor_lane<32>(acc[g][i]));
            tot[g][i] += L.w[g] * round_bf16(full * L.sd);
          }
          acc[g] = f32x4{0.f, 0.f, 0.f, 0.f};
        }
      }
    };
    // The first RING units are loaded unconditionally (the math of the
    // first pass then waits for exactly its own unit); later loads only for
    // units that exist.
    DnPiece<G> P[RING];
#pragma unroll
    for (int q = 0; q < RING; ++q) load(q, P[q]);
    for (int u0 = 0; u0 < nu; u0 += RING) {
#pragma unroll
      for (int q = 0; q < RING; ++q) {
        if (u0 + q < nu) step(u0 + q, P[q]);
        if (u0 + q + RING < nu) load(u0 + q + RING, P[q]);
      }
    }
  }
#pragma unroll
  for (int g = 0; g < G; ++g)
#pragma unroll
    for (int i = 0; i < 4; ++i) s_red[wave][g][i][lane] = tot[g][i];
  __syncthreads();
  // thread g * 32 + l (l < 32, l & 8 == 0): rows (l/16)*4 + i of token 8g + (l & 7)
  const int g = tid >> 5, l = tid & 31, t = 8 * g + (l & 7);
  if (g < G && (l & 8) == 0 && t < B) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      float v = 0.f;
#pragma unroll
      for (int w = 0; w < kMmWaves; ++w) v += s_red[w][g][i][l];
      const int64_t o = (int64_t)t * H + row0 + (l >> 4) * 4 + i;
      float r = round_bf16(v);
      if (a.residual) r = bf16_to_f32(a.x[o]) + r;
      a.y[o] = (uint16_t)f32_to_bf16(r);
    }
  }
}

// ---------------------------------------------------------------------------
// k_down: 4 output rows per block, every expert, weighted combine
// ---------------------------------------------------------------------------

constexpr int kMaxDownSlots = 64;  // entries reduced per pass (lane groups beyond idle)

template <int WT, int MAXT, int DW>
__global__ __launch_bounds__(DW *kWave) void k_down(DecodeArgs a) {
  const int H = a.H, B = a.B;
  const int K = (a.E > 0) ? a.I : a.Is;  // Is == I when both exist
  const int LPR = lanes_per_row(K), C = K / 32;
  const int lane = threadIdx.x & (kWave - 1), lg = lane % LPR;
  const int gi = threadIdx.x / LPR;  // lane group = entry slot of a pass
  const int slots_all = DW * (kWave / LPR);
  const int slots = slots_all < kMaxDownSlots ? slots_all : kMaxDownSlots;
  const int r0 = blockIdx.x * kRows;
  const int n_routed = (a.E > 0) ? *a.ws.n_routed : 0;
  const int n_entries = n_routed + (a.Is > 0 ? 1 : 0);
  const int Imax = a.I > a.Is ? a.I : a.Is;

  __shared__ float s_part[kMaxDownSlots][kRows][MAXT];
  float total = 0.f;  // thread (row, token) = (tid / MAXT, tid % MAXT), tid < 4*MAXT

  for (int pass = 0; pass * slots < n_entries; ++pass) {
    for (int i = threadIdx.x; i < slots * kRows * MAXT; i += blockDim.x) (&s_part[0][0][0])[i] = 0.f;
    __syncthreads();
    const int j = (gi < slots) ? pass * slots + gi : n_entries;
    uint32_t mask = 0;
    const uint8_t *Wd = nullptr;
    float Sd = 1.f;
    int hslot = 0;
    const float *wt = nullptr;
    if (j < n_routed) {
      const int e = a.ws.entry_expert[j];
      mask = a.ws.entry_mask[j];
      const int64_t mb = (WT == 1) ? nvfp4_matrix_bytes(H, K) : (int64_t)H * K * 2;
      Wd = a.w_down + e * mb;
      if (WT == 1) Sd = a.w_scale[3 * e + 2];
      hslot = j;
      wt = a.ws.entry_w + j * kMaxBatch;
    } else if (j == n_routed && j < n_entries) {
      mask = (1u << B) - 1u;
      Wd = a.sh_down;
      if (WT == 1) Sd = a.sh_scale[2];
      hslot = a.max_routed;
    }
    float acc[MAXT][kRows];
#pragma unroll
    for (int t = 0; t < MAXT; ++t)
#pragma unroll
      for (int r = 0; r < kRows; ++r) acc[t][r] = 0.f;
    if (mask) {
      for (int c = lg; c < C; c += LPR) {
        ChunkRaw cr;
        load_rows<WT>(Wd, H, K, r0, c, cr);
        ChunkBF cb;
        convert_rows<WT>(cr, cb);
        dot_tokens<WT, MAXT>(cb, a.ws.h + (int64_t)hslot * B * Imax, Imax, c, mask, B, acc);
      }
    }
    StaticFor<0, MAXT>::run([&](auto tc) __attribute__((always_inline)) {
      constexpr int t = decltype(tc)::value;
      if (t < B) {
        int row;
        float y2 = 0.f;
        const float ys = fold4(acc[t][0], acc[t][1], acc[t][2], acc[t][3], LPR, row, &y2);
        if (lg < (LPR == 2 ? 2 : kRows) && ((mask >> t) & 1u)) {
          const float w = wt ? wt[t] : 1.0f;
          s_part[gi][row][t] = w * round_bf16(ys * Sd);
          if (LPR == 2) s_part[gi][row + 1][t] = w * round_bf16(y2 * Sd);
        }
      }
    });
    __syncthreads();
    if (threadIdx.x < kRows * MAXT) {
      const int r = threadIdx.x / MAXT, t = threadIdx.x % MAXT;
      for (int s = 0; s < slots; ++s) total += s_part[s][r][t];
    }
    __syncthreads();
  }
  if (threadIdx.x < kRows * MAXT) {
    const int r = threadIdx.x / MAXT, t = threadIdx.x % MAXT;
    if (t < B) {
      const int64_t o = (int64_t)t * H + r0 + r;
      float v = round_bf16(total);
      if (a.residual) v = bf16_to_f32(a.x[o]) + v;
      a.y[o] = (uint16_t)f32_to_bf16(v);
    }
  }
}

// ---------------------------------------------------------------------------
// k_layer_b1: one token with routed experts, the whole layer in one kernel.
//   Blocks [0, rt_blocks): router rows.  Each block normalises the token in
//   LDS (every block computes the same bits) and publishes its rows'
//   logits as tagged words.
//   Blocks [rt_blocks, rt_blocks + gu_blocks): gate/up units.  Each block
//   normalises the token into LDS itself; blocks with routed units take
//   the routing (below) and publish h as tagged words.
//   The rest: down blocks of 8 output rows each (two 4-row halves of 2
//   waves), the weighted combine in LDS in a fixed expert order.
// Hand-overs (the logits to every routed gate/up block and down block, h
// to every down block) go through memory once per XCD: the first consumer
// block on an XCD (its agent-scope exchange of the layer's tag into the
// XCD's ticket returns something else) copies the tagged words into that
// XCD's stage, polling each word until it carries the tag, and raises the
// XCD's flag to the tag; the XCD's other consumers poll the flag and read
// the stage from the XCD's L2.  Producers never wait and have lower block
// indices than their consumers, which the hardware dispatches in order;
// every wait is bounded.
// ---------------------------------------------------------------------------

// Poll rounds (each ends in a short sleep) before a wait on another block
// of the same kernel gives up; reached only if that block never wrote.  A
// wait that gives up sets its bit in the workspace's status word (zeroed
// by every call), so the caller can tell such a call's outputs from good
// ones.
constexpr int kWaitSpin = 1 << 20;

__device__ __forceinline__ void report_giveup(const DecodeArgs &a, uint32_t bit) {
  __hip_atomic_fetch_or(a.ws.status, bit, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

constexpr int kDnHalf = 2 * kWave;  // threads per 4-row half of a down block

__device__ __forceinline__ int xcc_id() {
  return __builtin_amdgcn_s_getreg((3 << 11) | 20) & (kXcdSlots - 1);  // HW_REG_XCC_ID[3:0]
}

__device__ __forceinline__ uint32_t *sync_line(const DecodeArgs &a, int which, int xcc) {
  return a.ws.sync_lines + ((int64_t)which * kXcdSlots + xcc) * 64;
}

// True in exactly one block per XCD and layer call: the first to raise the
// ticket to the tag (tags grow within a call: a block that arrives after a
// later layer's leader is not a leader).
__device__ __forceinline__ bool take_ticket(const DecodeArgs &a, int which, int xcc) {
  return __hip_atomic_fetch_max(sync_line(a, which, xcc), a.tag, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) <
         a.tag;
}

// Leader: once its stores to the stage have reached the L2, the flag,
// raised to the tag and never lowered (a later layer may have raised it).
__device__ __forceinline__ void raise_flag(const DecodeArgs &a, int which, int xcc) {
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  __syncthreads();
  if (threadIdx.x == 0)
    __hip_atomic_fetch_max(sync_line(a, which, xcc), a.tag, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Others (thread 0): until the XCD's flag reaches the tag.  The flag is
// read with volatile loads (issued sc0 sc1), which miss this CU's cache;
// plain or sc0 reloads can keep returning a stale line from it (measured:
// no update in 200,000 polls).  Measured on MI355X: a flag raised by
// another block of the same XCD is seen about 0.4 us after the store.  The
// stage is then read once, after the flag, so this CU's cache holds no
// earlier copy of it (the kernel starts with the CU caches invalidated).
__device__ __forceinline__ void wait_flag(const DecodeArgs &a, int which, int xcc, uint32_t giveup_bit) {
  if (threadIdx.x == 0) {
    const volatile uint32_t *flag = sync_line(a, which, xcc);
    bool seen = false;
    for (int it = 0; it < kWaitSpin && !seen; ++it) {
      seen = *flag >= a.tag;
      if (!seen) __builtin_amdgcn_s_sleep(1);
    }
    if (!seen) report_giveup(a, giveup_bit);
  }
}

// Leader: the values of n tagged words into dst[0..n), each polled until
// it carries the tag; a thread keeps kCopy words in flight and re-reads
// all its missing ones in each round.  False if some word of this thread
// never arrived.
__device__ inline bool copy_tagged(const uint64_t *src, uint32_t *dst, int n, uint32_t tag) {
  constexpr int kCopy = 8;
  const int tid = threadIdx.x, nt = blockDim.x;
  bool all = true;
  for (int i0 = 0; i0 < n; i0 += kCopy * nt) {
    uint64_t v[kCopy];
#pragma unroll
    for (int k = 0; k < kCopy; ++k) {
      const int i = i0 + k * nt + tid;
      v[k] = i < n ? load_tagged(src + i) : (uint64_t)tag << 32;
    }
    bool done = false;
    for (int it = 0; it < kWaitSpin; ++it) {
      done = true;
#pragma unroll
      for (int k = 0; k < kCopy; ++k) done = done && (uint32_t)(v[k] >> 32) == tag;
      if (done) break;
      __builtin_amdgcn_s_sleep(1);
#pragma unroll
      for (int k = 0; k < kCopy; ++k)
        if ((uint32_t)(v[k] >> 32) != tag) v[k] = load_tagged(src + i0 + k * nt + tid);
    }
    all = all && done;
#pragma unroll
    for (int k = 0; k < kCopy; ++k) {
      const int i = i0 + k * nt + tid;
      if (i < n) dst[i] = (uint32_t)v[k];
    }
  }
  return all;
}

// The last block of k_router with `route` (batches of 2..8 tokens, one
// wave per token): the routing of the batch from the tagged logits the
// other blocks publish, polled into LDS (B * E floats, at most 32 KiB, in
// the activation stage this block does not use); the list and the top-k
// outputs are published for the expert kernels.
__device__ void route_block(const DecodeArgs &a, uint4 *lds) {
  __shared__ Routing R;
  __shared__ uint32_t s_mark[kMaxExperts];
  float *s_l = reinterpret_cast<float *>(lds);
  if (!copy_tagged(a.ws.sync_l, reinterpret_cast<uint32_t *>(s_l), a.B * a.E, a.tag))
    report_giveup(a, kStatusRouteWait);
  __syncthreads();
  build_routing(a, s_l, R, s_mark, (int)(blockDim.x / kWave));
  publish_routing(a, R);
}

// The token's routing from the logits the router blocks published, by way
// of this XCD's copy.  s_lead: a shared word for the ticket.  Ends with a
// barrier.  (Every consumer block polling the E words itself measured
// 0.2 us slower per layer: about 450 blocks re-reading the same 2 KB.)
__device__ inline void take_routing(const DecodeArgs &a, int xcc, Routing &R, uint32_t *s_mark, int &s_lead) {
  if (threadIdx.x == 0) s_lead = take_ticket(a, kLineLTicket, xcc);
  __syncthreads();
  float *stage = a.ws.xcd_l + (int64_t)xcc * a.ws.stage_l;
  if (s_lead) {
    if (!copy_tagged(a.ws.sync_l, reinterpret_cast<uint32_t *>(stage), a.E, a.tag))
      report_giveup(a, kStatusLogitWait);
    raise_flag(a, kLineLFlag, xcc);
  } else {
    wait_flag(a, kLineLFlag, xcc, kStatusLogitWait);
  }
  __syncthreads();
  build_routing(a, stage, R, s_mark, kGateupWaves);
}

// The token into LDS (s_x: H/8 pieces of 16 bytes) with the pre-norm when
// the layer has one: xn = BF16(x * inv * gain), inv = 1/sqrt(mean(x^2) +
// eps) from an FP64 sum of squares (exact per term), reduced in the same
// order in every block.  x0, g0: this thread's first pieces of x and of
// the gain, already loaded.  Ends with a barrier.
__device__ inline void stage_token(const DecodeArgs &a, uint4 *s_x, double *s_red, uint4 x0, uint4 g0) {
  const int H = a.H, n8 = H / 8;
  const int tid = threadIdx.x, lane = tid & (kWave - 1), wave = tid / kWave, nw = blockDim.x / kWave;
  const uint4 *xr = reinterpret_cast<const uint4 *>(a.x);
  const uint4 *gr = reinterpret_cast<const uint4 *>(a.norm_gain);
  double ss = 0.0;
  for (int i = tid; i < n8; i += blockDim.x) {
    const uint4 v = i == tid ? x0 : xr[i];
    s_x[i] = v;
    if (a.use_norm) {
      const uint32_t q[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const double lo = bf16_to_f32(q[j] & 0xffffu), hi = bf16_to_f32(q[j] >> 16);
        ss = fma(lo, lo, fma(hi, hi, ss));
      }
    }
  }
  if (!a.use_norm) {
    __syncthreads();
    return;
  }
  ss = group_sum_f64(ss, kWave);
  if (lane == 0) s_red[wave] = ss;
  __syncthreads();
  double tot = 0.0;
  for (int w = 0; w < nw; ++w) tot += s_red[w];
  const double inv = 1.0 / sqrt(tot / (double)H + (double)a.eps);
  const float inv_f = (float)inv;
  for (int i = tid; i < n8; i += blockDim.x) {
    const uint4 gv = i == tid ? g0 : gr[i];
    s_x[i] = norm_piece_bf16(s_x[i], gv, inv_f, inv);
  }
  __syncthreads();
}

// This thread's first pieces of x and of the gain.
__device__ __forceinline__ void first_pieces(const DecodeArgs &a, uint4 &x0, uint4 &g0) {
  const int tc = min((int)threadIdx.x, a.H / 8 - 1);  // clamped: unconditional loads
  x0 = reinterpret_cast<const uint4 *>(a.x)[tc];
  g0 = a.use_norm ? reinterpret_cast<const uint4 *>(a.norm_gain)[tc] : make_uint4(0, 0, 0, 0);
}

// Router rows of block rb: one row per lane group of LPR lanes (lane j of
// a group takes the row's 16-byte pieces j, j + LPR, ...), dotted with the
// token in LDS; the logit l = W_r xn + b (FP32) is published.  WAIT (the
// persistent step): token_wait() runs after the rows are requested and
// before the token is read, which waits for the previous layer's output;
// otherwise the token is requested first.
template <bool WAIT, typename TokenWait>
__device__ inline void router_block_b1(const DecodeArgs &a, int rb, uint4 *s_x, double *s_red,
                                       TokenWait token_wait) {
  const int H = a.H, E = a.E, n8 = H / 8;
  const int LPR = lanes_per_row(H);
  const int tid = threadIdx.x, lane = tid & (kWave - 1), wave = tid / kWave, lg = lane % LPR;
  const int row = (rb * kRouterWaves + wave) * (kWave / LPR) + lane / LPR;
  const uint4 *wr = reinterpret_cast<const uint4 *>(a.router_w + (int64_t)(row < E ? row : 0) * H);
  // Loads in the order they are needed (they complete in issue order): the
  // token and the gain (cache hits: the norm starts as soon as they land),
  // then the row's first four pieces and the bias, which come from memory
  // while the norm runs.
  // (indices clamped into the buffers: every load is unconditional, so the
  // waits before the norm cover the token and the gain only)
  const int tc = tid < n8 ? tid : n8 - 1;
  uint4 x0 = make_uint4(0, 0, 0, 0), g0 = make_uint4(0, 0, 0, 0);
  if (!WAIT) x0 = reinterpret_cast<const uint4 *>(a.x)[tc];
  if (a.use_norm) g0 = reinterpret_cast<const uint4 *>(a.norm_gain)[tc];
  uint4 w0[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) w0[i] = wr[min(lg + i * LPR, n8 - 1)];
#pragma unroll
  for (int i = 0; i < 4; ++i)
    if (!(row < E && lg + i * LPR < n8)) w0[i] = make_uint4(0, 0, 0, 0);
  float bias = a.router_b ? a.router_b[row < E ? row : E - 1] : 0.f;
  if (row >= E) bias = 0.f;
  if (WAIT) {
    token_wait();
    x0 = reinterpret_cast<const uint4 *>(a.x)[tc];
  }
  stage_token(a, s_x, s_red, x0, g0);
  if (row >= E) return;
  float acc = 0.f;
  for (int j0 = lg; j0 < n8; j0 += 4 * LPR) {
    uint4 w[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int j = j0 + i * LPR;
      if (j0 == lg) w[i] = w0[i];
      else w[i] = j < n8 ? wr[j] : make_uint4(0, 0, 0, 0);
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int j = j0 + i * LPR;
      if (j < n8) {
        const uint4 v = s_x[j];
        acc = dot2_bf16(w[i].x, v.x, acc);
        acc = dot2_bf16(w[i].y, v.y, acc);
        acc = dot2_bf16(w[i].z, v.z, acc);
        acc = dot2_bf16(w[i].w, v.w, acc);
      }
    }
  }
  const float v = group_sum(acc, LPR);
  if (lg == 0) publish_tagged(a.ws.sync_l + row, __float_as_uint(v + bias), a.tag);
}

// PERSIST (the persistent step): the residual input of this thread's row
// is xres (the row this block produced in the previous layer, or x in the
// first), and the output row goes to xres and, unless `last`, out as tagged
// words for the next layer's blocks; the last layer writes y.
template <int WT, bool PERSIST = false>
__device__ __forceinline__ void down_block_b1(const DecodeArgs &a, int dbid, int xcc, Routing &R, uint32_t *s_mark,
                                              float (&s_part)[2][kMaxDownSlots][kRows], int &s_llead,
                                              int &s_hlead, float *xres = nullptr, bool last = true) {
  const int H = a.H, K = a.I;  // experts present: Is is I or 0
  const int LPR = lanes_per_row(K), C = K / 32;
  const int tid = threadIdx.x, lane = tid & (kWave - 1), lg = lane % LPR;
  const int half = tid / kDnHalf, ht = tid % kDnHalf;
  const int gi = ht / LPR;  // entry slot of a pass
  const int slots_all = kDnHalf / LPR;
  const int slots = slots_all < kMaxDownSlots ? slots_all : kMaxDownSlots;
  const int r0 = dbid * (2 * kRows) + half * kRows;
  const int Imax = a.I > a.Is ? a.I : a.Is;
  if (tid == 0) s_hlead = take_ticket(a, kLineHTicket, xcc);
  take_routing(a, xcc, R, s_mark, s_llead);  // ends with a barrier
  const bool lead = s_hlead != 0;
  const int n_routed = R.n;
  const int n_entries = n_routed + (a.Is > 0 ? 1 : 0);
  uint16_t *stage = a.ws.xcd_h + (int64_t)xcc * a.ws.stage_elems;
  float total = 0.f;  // threads ht < 4: row r0 + ht

  for (int pass = 0; pass * slots < n_entries; ++pass) {
    for (int i = ht; i < slots * kRows; i += kDnHalf) (&s_part[half][0][0])[i] = 0.f;
    const int j = (gi < slots) ? pass * slots + gi : n_entries;
    const uint8_t *Wd = nullptr;
    float Sd = 1.f, w = 0.f;
    int hslot = 0;
    if (j < n_routed) {
      const int e = R.expert[j];
      const int64_t mb = (WT == 1) ? nvfp4_matrix_bytes(H, K) : (int64_t)H * K * 2;
      Wd = a.w_down + e * mb;
      if (WT == 1) Sd = a.w_scale[3 * e + 2];
      hslot = j;
      for (int r = 0; r < a.k; ++r)
        if (R.sel[0][r] == e) w = R.w[0][r];
    } else if (j == n_routed && j < n_entries) {
      Wd = a.sh_down;
      if (WT == 1) Sd = a.sh_scale[2];
      hslot = a.max_routed;
      w = 1.f;
    }
    // this lane's first weight chunk, loaded before the wait
    ChunkRaw cr;
    if (Wd) load_rows<WT>(Wd, H, K, r0, lg, cr);
    if (pass == 0) {
      // One token: the routed entries are slots 0..k-1 and the shared
      // expert slot k (= max_routed), so the entries' h words are the first
      // n_entries * Imax / 2 words.
      if (lead) {
        if (!copy_tagged(a.ws.sync_h, reinterpret_cast<uint32_t *>(stage), n_entries * (Imax / 2), a.tag))
          report_giveup(a, kStatusHWait);
        raise_flag(a, kLineHFlag, xcc);
      } else {
        wait_flag(a, kLineHFlag, xcc, kStatusHWait);
      }
    }
    __syncthreads();
    float acc[kRows] = {0.f, 0.f, 0.f, 0.f};
    if (Wd) {
      const int64_t hbase = (int64_t)hslot * Imax;  // the entry's h in the stage
      for (int c = lg; c < C; c += LPR) {
        if (c != lg) load_rows<WT>(Wd, H, K, r0, c, cr);
        uint32_t x[16];
        load16(stage + hbase + c * 32, x);
        ChunkBF cb;
        convert_rows<WT>(cr, cb);
        dot_rows<WT>(cb, x, acc);
      }
    }
    int row;
    float y2 = 0.f;
    const float ys = fold4(acc[0], acc[1], acc[2], acc[3], LPR, row, &y2);
    if (lg < (LPR == 2 ? 2 : kRows) && Wd) {
      s_part[half][gi][row] = w * round_bf16(ys * Sd);
      if (LPR == 2) s_part[half][gi][row + 1] = w * round_bf16(y2 * Sd);
    }
    __syncthreads();
    if (ht < kRows)
      for (int s2 = 0; s2 < slots; ++s2) total += s_part[half][s2][ht];
    __syncthreads();
  }
  if constexpr (PERSIST) {
    // every lane computes (lanes ht < 4 hold the rows), so that the pair
    // exchange below reads active lanes
    const int64_t o = r0 + (ht & (kRows - 1));
    const uint32_t yb = f32_to_bf16(*xres + round_bf16(total));
    const uint32_t other = xor_lane<1>(yb);
    if (ht < kRows) {
      *xres = bf16_to_f32(yb);
      if (last) a.y[o] = (uint16_t)yb;
      else if ((ht & 1) == 0) publish_tagged(a.ws.sync_y + o / 2, yb | (other << 16), a.tag);
    }
  } else if (ht < kRows) {
    const int64_t o = r0 + ht;
    float v = round_bf16(total);
    if (a.residual) v = bf16_to_f32(a.x[o]) + v;
    a.y[o] = (uint16_t)f32_to_bf16(v);
  }
}

template <int WT>
__global__ __launch_bounds__(kGateupWaves *kWave) void k_layer_b1(DecodeArgs a, int rt_blocks, int gu_blocks) {
  static_assert(kGateupWaves * kWave == 2 * kDnHalf, "a down block is two 4-row halves");
  static_assert(kRouterThreads == kGateupWaves * kWave, "router blocks have the same size");
  extern __shared__ uint4 s_x[];  // [H / 8] the token (router and gate/up blocks)
  __shared__ Routing R;
  __shared__ uint32_t s_mark[1];  // one token: the routing needs no marks
  __shared__ float s_part[2][kMaxDownSlots][kRows];
  __shared__ double s_red[kGateupWaves];
  __shared__ int s_llead, s_hlead;
  const int b = blockIdx.x;
  if (b < rt_blocks) {
    router_block_b1<false>(a, b, s_x, s_red, [] {});
    return;
  }
  const int xcc = xcc_id();
  if (b < rt_blocks + gu_blocks) {
    const int bid = b - rt_blocks;
    const int groups = kGateupWaves * (kWave / lanes_per_row(a.H));
    uint4 x0, g0;
    first_pieces(a, x0, g0);
    stage_token(a, s_x, s_red, x0, g0);
    if (bid * groups < a.max_routed * (a.I / kRows) || bid == 0) take_routing(a, xcc, R, s_mark, s_llead);
    gateup_block<WT, 1, true>(a, bid, R, reinterpret_cast<const uint16_t *>(s_x));
    // the top-k outputs, after this block's share of h (the down blocks
    // derive the routing themselves and read no entry list)
    if (bid == 0 && threadIdx.x < (unsigned)a.k) {
      a.out_idx[threadIdx.x] = R.sel[0][threadIdx.x];
      a.out_w[threadIdx.x] = R.w[0][threadIdx.x];
    }
  } else {
    down_block_b1<WT>(a, b - rt_blocks - gu_blocks, xcc, R, s_mark, s_part, s_llead, s_hlead);
  }
}

// ---------------------------------------------------------------------------
// k_step_b1: the persistent one-token step, consecutive MoE layers of one
// shape in one launch ("Day-0 Support for Flint on vLLM", section
// "Optimizations": the low-latency path loads each kernel's weights while
// the previous one still runs).  Every block keeps its k_layer_b1 role in
// every layer.  Between layers the output, not a kernel boundary, is
// handed over: the down blocks publish their rows as tagged words, and the
// router and gate/up blocks of the next layer take them through their
// XCD's stage like the logits and h.  So a router block has its next
// layer's rows in flight while it waits for that layer's input, and no
// launch separates the layers.  The down blocks keep their rows of the
// residual stream in registers.  Every block must be resident at once (the
// host checks the occupancy); each layer has its own stage set, so no block
// reads a stage address twice in a launch; tickets and flags only grow, so
// a block that is one layer behind cannot undo a later layer's hand-over.
// ---------------------------------------------------------------------------

// The previous layer's output (tagged with word_tag) into this XCD's copy
// for this layer, by one leader per XCD; everyone else waits for the flag.
// Ends with a barrier.
__device__ inline void take_token(const DecodeArgs &a, int xcc, uint16_t *stage, uint32_t word_tag, int &s_lead) {
  if (threadIdx.x == 0) s_lead = take_ticket(a, kLineYTicket, xcc);
  __syncthreads();
  if (s_lead) {
    if (!copy_tagged(a.ws.sync_y, reinterpret_cast<uint32_t *>(stage), a.H / 2, word_tag))
      report_giveup(a, kStatusYWait);
    raise_flag(a, kLineYFlag, xcc);
  } else {
    wait_flag(a, kLineYFlag, xcc, kStatusYWait);
  }
  __syncthreads();
}

// Layer l's arguments: the first layer's, with layer l's weights, tag and
// stage set.
__device__ __forceinline__ DecodeArgs layer_args(const PersistArgs &p, int l) {
  DecodeArgs a = p.a;
  const PersistLayer &W = p.L[l];
  a.router_w = W.router_w;
  a.router_b = W.router_b;
  a.w_gate = W.w_gate;
  a.w_up = W.w_up;
  a.w_down = W.w_down;
  a.w_scale = W.w_scale;
  a.sh_gate = W.sh_gate;
  a.sh_up = W.sh_up;
  a.sh_down = W.sh_down;
  a.sh_scale = W.sh_scale;
  a.norm_gain = W.norm_gain;
  a.tag = p.a.tag + (uint32_t)l;
  uint8_t *slot = p.stages + (int64_t)l * p.slot_bytes;
  a.ws.xcd_l = reinterpret_cast<float *>(slot);
  a.ws.xcd_h = reinterpret_cast<uint16_t *>(slot + p.off_h);
  return a;
}

__device__ __forceinline__ uint16_t *token_stage(const PersistArgs &p, int l, int xcc) {
  return reinterpret_cast<uint16_t *>(p.stages + (int64_t)l * p.slot_bytes + p.off_y) + (int64_t)xcc * p.a.H;
}

// Blocks [0, gu_blocks): gate/up; the rest: down blocks of 8 rows, of
// which the first rt_blocks also compute k_layer_b1's router block rows
// (the same function, so the same bits) at the start of every layer, while
// they would otherwise wait for the routing.  Fewer blocks than k_layer_b1
// (480 at the full shape), so that all are resident at two per CU.
template <int WT>
__global__ __launch_bounds__(kGateupWaves *kWave) void k_step_b1(PersistArgs p, int rt_blocks, int gu_blocks) {
  extern __shared__ uint4 s_x[];  // [H / 8] the token (router rows and gate/up blocks)
  __shared__ Routing R;
  __shared__ uint32_t s_mark[1];
  __shared__ float s_part[2][kMaxDownSlots][kRows];
  __shared__ double s_red[kGateupWaves];
  __shared__ int s_llead, s_hlead, s_ylead;
  const int b = blockIdx.x;
  const int xcc = xcc_id();
  const int n = p.n_layers;
  if (b < gu_blocks) {
    for (int l = 0; l < n; ++l) {
      DecodeArgs a = layer_args(p, l);
      const int groups = kGateupWaves * (kWave / lanes_per_row(a.H));
      if (l > 0) {
        uint16_t *ystage = token_stage(p, l, xcc);
        take_token(a, xcc, ystage, a.tag - 1, s_ylead);
        a.x = ystage;
      }
      uint4 x0, g0;
      first_pieces(a, x0, g0);
      stage_token(a, s_x, s_red, x0, g0);
      if (b * groups < a.max_routed * (a.I / kRows) || b == 0) take_routing(a, xcc, R, s_mark, s_llead);
      gateup_block<WT, 1, true>(a, b, R, reinterpret_cast<const uint16_t *>(s_x));
      __syncthreads();  // LDS is rewritten by the next layer
    }
  } else {
    const int dbid = b - gu_blocks;
    // this thread's row of the residual stream (threads ht < 4 of each
    // half hold it), from x for the first layer
    const int ht = threadIdx.x % kDnHalf, half = threadIdx.x / kDnHalf;
    float xres = bf16_to_f32(p.a.x[dbid * (2 * kRows) + half * kRows + (ht & (kRows - 1))]);
    for (int l = 0; l < n; ++l) {
      DecodeArgs a = layer_args(p, l);
      if (dbid < rt_blocks) {
        if (l > 0) {
          DecodeArgs ar = a;
          uint16_t *ystage = token_stage(p, l, xcc);
          ar.x = ystage;  // read once the hand-over has filled it
          router_block_b1<true>(ar, dbid, s_x, s_red, [&] { take_token(ar, xcc, ystage, ar.tag - 1, s_ylead); });
        } else {
          router_block_b1<false>(a, dbid, s_x, s_red, [] {});
        }
      }
      down_block_b1<WT, true>(a, dbid, xcc, R, s_mark, s_part, s_llead, s_hlead, &xres, l == n - 1);
      __syncthreads();
    }
  }
}

static int rt_blocks_of(const DecodeArgs &a) {
  const int rows_per_block = kRouterWaves * (kWave / lanes_per_row(a.H));
  return (a.E + rows_per_block - 1) / rows_per_block;
}
static int gu_blocks_of(const DecodeArgs &a) {
  const int groups = kGateupWaves * (kWave / lanes_per_row(a.H));
  const int units = a.max_routed * (a.I / kRows) + a.Is / kRows;
  return (units + groups - 1) / groups;
}

hipError_t persist_fits(const DecodeArgs &a, bool *fits) {
  int dev = 0, cus = 0, per_cu = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e == hipSuccess) e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
  if (e != hipSuccess) return e;
  e = a.wtype == 1 ? hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, k_step_b1<1>, kGateupWaves * kWave,
                                                                 (size_t)a.H * 2)
                   : hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, k_step_b1<0>, kGateupWaves * kWave,
                                                                 (size_t)a.H * 2);
  if (e != hipSuccess) return e;
  const int64_t grid = gu_blocks_of(a) + a.H / (2 * kRows);
  *fits = (int64_t)per_cu * cus >= grid && rt_blocks_of(a) <= a.H / (2 * kRows);
  return hipSuccess;
}

hipError_t launch_step_b1(const PersistArgs &p, hipStream_t stream) {
  const DecodeArgs &a = p.a;
  const int rt = rt_blocks_of(a), gu = gu_blocks_of(a);
  const int grid = gu + a.H / (2 * kRows);
  if (a.wtype == 1)
    hipLaunchKernelGGL(k_step_b1<1>, dim3(grid), dim3(kGateupWaves * kWave), (size_t)a.H * 2, stream, p, rt, gu);
  else
    hipLaunchKernelGGL(k_step_b1<0>, dim3(grid), dim3(kGateupWaves * kWave), (size_t)a.H * 2, stream, p, rt, gu);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Dense projection on one NVFP4 matrix for 1..8 tokens: the small-batch
// dense GEMV the pages pair with the MoE kernel ("Day-0 Support for Flint
// on vLLM", section "Optimizations": same packed NVFP4 weights, for the
// projections outside the MoE blocks):
//   y[t][n] = BF16(S * sum_k W[n][k] x[t][k]),  FP32 accumulation.
// ---------------------------------------------------------------------------

// One token (k_gemv): the block stages x in LDS once; each lane group of
// LPR lanes walks 4-row units (grid-stride), the next unit's weights in
// flight while the current one is multiplied (FP4 converted to BF16 in
// registers, v_dot2 with FP32 accumulation, block scales in FP32).
// acc[r] += W[r0 + r][chunk] . x[chunk] for one NVFP4 chunk, converting
// and multiplying one 8-element dword at a time (a small working set).
__device__ __forceinline__ void dot_rows_fp4(const ChunkRaw &cr, const uint32_t (&x)[16], float (&acc)[kRows]) {
#pragma unroll
  for (int r = 0; r < kRows; ++r) {
    const uint4 q = cr.q[r][0];
    float p0 = dot8_fp4_bf16(q.x, x[0], x[1], x[2], x[3], 0.f);
    p0 = dot8_fp4_bf16(q.y, x[4], x[5], x[6], x[7], p0);
    float p1 = dot8_fp4_bf16(q.z, x[8], x[9], x[10], x[11], 0.f);
    p1 = dot8_fp4_bf16(q.w, x[12], x[13], x[14], x[15], p1);
    acc[r] = fmaf(e4m3_to_f32(cr.scale[r] & 0xffu), p0, fmaf(e4m3_to_f32(cr.scale[r] >> 8), p1, acc[r]));
  }
}

constexpr int kGemvBlocksPerCu = 8;
constexpr int kGemvCus = 256;  // MI355X compute units: the grid is capped at 8 blocks per CU

__global__ __launch_bounds__(kGemvThreads) void k_gemv(GemvArgs g) {
  extern __shared__ uint4 s_gx[];  // x [K / 8] pieces of 16 bytes
  const int K = g.K, LPR = lanes_per_row(K), C = K / 32;
  const int groups = kGemvThreads / LPR;
  const int lane = threadIdx.x & (kWave - 1), lg = lane % LPR;
  for (int i = threadIdx.x; i < K / 8; i += kGemvThreads) s_gx[i] = reinterpret_cast<const uint4 *>(g.x)[i];
  const int64_t units = g.N / kRows, ustride = (int64_t)gridDim.x * groups;
  int64_t u = (int64_t)blockIdx.x * groups + threadIdx.x / LPR;
  const uint16_t *xs = reinterpret_cast<const uint16_t *>(s_gx);
  const float S = *g.scale;
  // one chunk per lane and unit when C <= LPR (every tiled K up to 2048),
  // else the lane walks its chunks inside the unit
  ChunkRaw nxt;
  if (u < units) load_rows<1>(g.w, g.N, K, (int)(u * kRows), lg, nxt);
  __syncthreads();
  // All lanes of a group take the same units, and the folds exchange
  // values only inside a group, so groups may leave the loop at different
  // times.
  for (; u < units; u += ustride) {
    float acc[kRows] = {0.f, 0.f, 0.f, 0.f};
    ChunkRaw cur = nxt;
    const int64_t un = u + ustride;
    for (int c = lg; c < C; c += LPR) {
      if (c != lg) load_rows<1>(g.w, g.N, K, (int)(u * kRows), c, cur);
      else if (un < units) load_rows<1>(g.w, g.N, K, (int)(un * kRows), lg, nxt);
      uint32_t x[16];
      load16(xs + c * 32, x);
      dot_rows_fp4(cur, x, acc);
    }
    int row;
    float y2 = 0.f;
    const float ys = fold4(acc[0], acc[1], acc[2], acc[3], LPR, row, &y2);
    if (lg < (LPR == 2 ? 2 : kRows)) {
      uint16_t *yr = g.y + u * kRows + row;
      yr[0] = (uint16_t)f32_to_bf16(ys * S);
      if (LPR == 2) yr[1] = (uint16_t)f32_to_bf16(y2 * S);
    }
  }
}

// 2..8 tokens (k_gemv_mm): on the matrix cores, as the batch expert kernels
// do: block = 64 weight rows (four 16-row A tiles), the tokens the 16
// columns of v_mfma_f32_16x16x32_bf16 (zero past the batch), each weight
// element dequantised once; the 8 waves split K and their partial sums meet
// in LDS.  Operand layout as in k_gateup_mm.
// The batch's x is staged in LDS when it fits the 32 KiB the K-partial
// sums use afterwards (B * K <= 16384): the token operands are then read
// from LDS right before their MFMAs and take no registers across the loads.
constexpr int kGemvMmStage = kMmWaves * 16 * kWave * 4;

template <bool STAGED>
__global__ __launch_bounds__(kMmWaves *kWave) void k_gemv_mm(GemvArgs g) {
  __shared__ float s_red[kMmWaves][16][kWave];
  const int K = g.K, B = g.B, C = K / 32, N = g.N;
  const int tid = threadIdx.x, lane = tid & (kWave - 1), wave = tid / kWave;
  const int r16 = lane & 15, p = lane >> 4;
  const int row0 = blockIdx.x * kMmRows;
  const uint16_t *xs = g.x;
  if (STAGED) {
    uint4 *st = reinterpret_cast<uint4 *>(&s_red[0][0][0]);
    for (int i = tid; i < B * K / 8; i += kMmWaves * kWave) st[i] = reinterpret_cast<const uint4 *>(g.x)[i];
    xs = reinterpret_cast<const uint16_t *>(st);
    __syncthreads();
  }
  f32x4 acc[4];
#pragma unroll
  for (int rg = 0; rg < 4; ++rg) acc[rg] = f32x4{0.f, 0.f, 0.f, 0.f};
  const int SS = (C + 3) / 4;
  // Two 128-K super-steps per pass, all their weight loads issued first.
  for (int ss0 = wave; ss0 < SS; ss0 += 2 * kMmWaves) {
    uint4 q[2][4], xv[2][4];
    uint32_t sc[2][4];
    bool tok[2];
    int cc[2];
#pragma unroll
    for (int v = 0; v < 2; ++v) {
      const int ss = ss0 + v * kMmWaves;
      const int c = ss * 4 + p;
      const bool cok = ss < SS && c < C;
      tok[v] = cok && r16 < B;
      cc[v] = c;
#pragma unroll
      for (int rg = 0; rg < 4; ++rg) {
        const int n = row0 + rg * 16 + r16;
        const bool ok = cok && n < N;
        q[v][rg] = ok ? *reinterpret_cast<const uint4 *>(g.w + (int64_t)n * (K / 2) + c * 16) : make_uint4(0, 0, 0, 0);
        sc[v][rg] = ok ? scale_pair(g.w, N, K, n, c) : 0u;
      }
      if (!STAGED) {
#pragma unroll
        for (int s = 0; s < 4; ++s)
          xv[v][s] = tok[v] ? *reinterpret_cast<const uint4 *>(xs + (int64_t)r16 * K + c * 32 + s * 8)
                            : make_uint4(0, 0, 0, 0);
      }
    }
#pragma unroll
    for (int v = 0; v < 2; ++v)
#pragma unroll
      for (int s = 0; s < 4; ++s) {
        const uint4 xq = STAGED ? (tok[v] ? *reinterpret_cast<const uint4 *>(xs + r16 * K + cc[v] * 32 + s * 8)
                                          : make_uint4(0, 0, 0, 0))
                                : xv[v][s];
        const bf16x8 bx = __builtin_bit_cast(bf16x8, u32x4{xq.x, xq.y, xq.z, xq.w});
#pragma unroll
        for (int rg = 0; rg < 4; ++rg) {
          const float sw = e4m3_to_f32((sc[v][rg] >> (8 * (s >> 1))) & 0xffu);
          acc[rg] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(dq8(word_of(q[v][rg], s), sw), bx, acc[rg], 0, 0, 0);
        }
      }
  }
  if (STAGED) __syncthreads();  // every wave is done with the staged x
#pragma unroll
  for (int rg = 0; rg < 4; ++rg)
#pragma unroll
    for (int i = 0; i < 4; ++i) s_red[wave][rg * 4 + i][lane] = acc[rg][i];
  __syncthreads();
  // 1024 (row group, value, lane) sums over the 8 waves, two per thread
  const float S = *g.scale;
#pragma unroll
  for (int k2 = 0; k2 < 2; ++k2) {
    const int idx = tid + k2 * kMmWaves * kWave;
    const int rg = idx >> 8, i = (idx >> 6) & 3, l = idx & 63;
    float v = 0.f;
#pragma unroll
    for (int w = 0; w < kMmWaves; ++w) v += s_red[w][rg * 4 + i][l];
    const int t = l & 15, n = row0 + rg * 16 + (l >> 4) * 4 + i;
    if (t < B && n < N) g.y[(int64_t)t * N + n] = (uint16_t)f32_to_bf16(v * S);
  }
}

hipError_t launch_gemv(const GemvArgs &g, hipStream_t stream) {
  if (g.B > 1) {
    const dim3 grid((g.N + kMmRows - 1) / kMmRows), block(kMmWaves * kWave);
    if ((int64_t)g.B * g.K * 2 <= kGemvMmStage) hipLaunchKernelGGL(k_gemv_mm<true>, grid, block, 0, stream, g);
    else hipLaunchKernelGGL(k_gemv_mm<false>, grid, block, 0, stream, g);
    return hipGetLastError();
  }
  const int groups = kGemvThreads / lanes_per_row(g.K);
  const int64_t units = g.N / kRows;
  const int64_t want = (units + groups - 1) / groups, cap = (int64_t)kGemvCus * kGemvBlocksPerCu;
  const int grid = (int)(want < cap ? want : cap);
  hipLaunchKernelGGL(k_gemv, dim3(grid), dim3(kGemvThreads), (size_t)g.K * 2, stream, g);
  return hipGetLastError();
}

__global__ __launch_bounds__(256) void k_sync_clear(uint32_t *p, int64_t n) {
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += (int64_t)gridDim.x * blockDim.x)
    __hip_atomic_store(p + i, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// ---------------------------------------------------------------------------
// Host launcher
// ---------------------------------------------------------------------------

// Launch with optional start/stop events attached to the dispatch itself
// (they time the kernel's execution, as a kernel trace does).
template <typename... Args>
static hipError_t launch(void (*kernel)(Args...), dim3 grid, dim3 block, size_t lds, hipStream_t stream,
                         hipEvent_t start, hipEvent_t stop, Args... args) {
  if (start && stop)
    hipExtLaunchKernelGGL(kernel, grid, block, (uint32_t)lds, stream, start, stop, 0u, args...);
  else
    hipLaunchKernelGGL(kernel, grid, block, lds, stream, args...);
  return hipGetLastError();
}

// Blocks of k_gateup_mm: at most one per compute unit (8 waves of over 200
// registers each fill one), each taking work items in turn.
constexpr int kMmGateupBlocks = 256;

template <int WT, int MAXT>
static hipError_t launch_experts(const DecodeArgs &a, hipStream_t stream, hipEvent_t const *ev) {
  hipError_t e;
  if (WT == 1 && MAXT > 1) {
    const int Imax = a.I > a.Is ? a.I : a.Is;
    const int groups = (Imax + kMmRows - 1) / kMmRows;
    const int items = a.max_routed * groups + (a.Is + kMmRows - 1) / kMmRows;
    const int grid = items < kMmGateupBlocks ? items : kMmGateupBlocks;
    if ((e = launch(k_gateup_mm, dim3(grid), dim3(kMmWaves * kWave), 0, stream,
                    ev ? ev[2] : nullptr, ev ? ev[3] : nullptr, a)) != hipSuccess)
      return e;
    if (a.B > 8)
      return launch(k_down_mm<2>, dim3(a.H / 8), dim3(kMmWaves * kWave), 0, stream, ev ? ev[4] : nullptr,
                    ev ? ev[5] : nullptr, a);
    return launch(k_down_mm<1>, dim3(a.H / 8), dim3(kMmWaves * kWave), 0, stream, ev ? ev[4] : nullptr,
                  ev ? ev[5] : nullptr, a);
  }
  {
    const int groups = kGateupWaves * (kWave / lanes_per_row(a.H));
    const int units = a.max_routed * (a.I / kRows) + a.Is / kRows;
    const int grid = (units + groups - 1) / groups;
    if ((e = launch(k_gateup<WT, MAXT>, dim3(grid), dim3(kGateupWaves * kWave), 0, stream, ev ? ev[2] : nullptr,
                    ev ? ev[3] : nullptr, a)) != hipSuccess)
      return e;
  }
  constexpr int DW = MAXT <= 2 ? 2 : MAXT <= 4 ? 4 : 8;
  return launch(k_down<WT, MAXT, DW>, dim3(a.H / kRows), dim3(DW * kWave), 0, stream, ev ? ev[4] : nullptr,
                ev ? ev[5] : nullptr, a);
}

// One token with routed experts: the whole layer in one kernel (its events
// are the gate/up pair; the router and down pairs are recorded empty).
template <int WT>
static hipError_t launch_layer_b1(const DecodeArgs &a, hipStream_t stream, hipEvent_t const *ev) {
  hipError_t e;
  const int LPR = lanes_per_row(a.H);
  const int rows_per_block = kRouterWaves * (kWave / LPR);
  const int rt = (a.E + rows_per_block - 1) / rows_per_block;
  const int groups = kGateupWaves * (kWave / LPR);
  const int units = a.max_routed * (a.I / kRows) + a.Is / kRows;
  const int gu = (units + groups - 1) / groups;
  const int grid = rt + gu + a.H / (2 * kRows);
  if (ev) {
    if ((e = hipEventRecord(ev[0], stream)) != hipSuccess) return e;
    if ((e = hipEventRecord(ev[1], stream)) != hipSuccess) return e;
  }
  if ((e = launch(k_layer_b1<WT>, dim3(grid), dim3(kGateupWaves * kWave), (size_t)a.H * 2, stream,
                  ev ? ev[2] : nullptr, ev ? ev[3] : nullptr, a, rt, gu)) != hipSuccess)
    return e;
  if (ev) {
    if ((e = hipEventRecord(ev[4], stream)) != hipSuccess) return e;
    return hipEventRecord(ev[5], stream);
  }
  return hipSuccess;
}

hipError_t launch_sync_clear(uint32_t *region, int64_t words, hipStream_t stream) {
  const int64_t blocks64 = (words + 255) / 256;
  const int blocks = (int)(blocks64 < 64 ? (blocks64 > 0 ? blocks64 : 1) : 64);
  hipLaunchKernelGGL(k_sync_clear, dim3(blocks), dim3(256), 0, stream, region, words);
  return hipGetLastError();
}

hipError_t launch_router_tokens(const DecodeArgs &a, hipStream_t stream) {
  const int rows_per_block = kRouterWaves * (kWave / lanes_per_row(a.H));
  return launch(k_router<kRouterWaves, 1>, dim3((a.E + rows_per_block - 1) / rows_per_block, a.B), dim3(kRouterThreads),
                0, stream, nullptr, nullptr, a, 0, 0);
}

hipError_t launch_decode(const DecodeArgs &a, hipStream_t stream, hipEvent_t const *ev) {
  // ev: NULL, or 6 events: start/stop of the router GEMV kernel, of the
  // gate/up kernel and of the down kernel (attached to the dispatches; for
  // measurement, eager launches only).
  hipError_t e;
  if (a.B == 1 && a.E > 0) return a.wtype == 1 ? launch_layer_b1<1>(a, stream, ev) : launch_layer_b1<0>(a, stream, ev);
  // NVFP4 batches with routed experts: three kernels.  The router has one
  // row of blocks per token; each block normalises its token itself (the
  // first block of a row also stores its xn) and stores plain logits; the
  // gate/up blocks derive the routing from them.
  if (a.wtype == 1 && a.B > 1 && a.E > 0) {
    const int rows_per_block = kRouterWaves * (kWave / lanes_per_row(a.H));
    if ((e = launch(k_router<kRouterWaves, 1>, dim3((a.E + rows_per_block - 1) / rows_per_block, a.B),
                    dim3(kRouterThreads), 0, stream, ev ? ev[0] : nullptr, ev ? ev[1] : nullptr, a, 0, 0)) !=
        hipSuccess)
      return e;
    switch (a.B <= 2 ? 2 : a.B <= 4 ? 4 : 8) {
      case 2: return launch_experts<1, 2>(a, stream, ev);
      case 4: return launch_experts<1, 4>(a, stream, ev);
      default: return launch_experts<1, 8>(a, stream, ev);
    }
  }
  // Other batches of several tokens normalise once in k_norm; a single
  // token normalises inside the router blocks (one launch fewer).
  const int xn_ready = (a.use_norm && a.B > 1) ? 1 : 0;
  if (xn_ready) {
    if ((e = launch(k_norm, dim3(a.B), dim3(kNormThreads), 0, stream, nullptr, nullptr, a)) != hipSuccess) return e;
  }
  if (a.E > 0) {
    // batches with routed experts: 8-wave blocks, the last of them derives
    // the routing from the others' logits
    const int rows_per_block = kRouteWaves * (kWave / lanes_per_row(a.H));
    const int grid = (a.E + rows_per_block - 1) / rows_per_block + 1;
    if ((e = launch(k_router<kRouteWaves, kMaxBatchBf16>, dim3(grid), dim3(kRouteWaves * kWave), 0, stream, ev ? ev[0] : nullptr,
                    ev ? ev[1] : nullptr, a, xn_ready, 1)) != hipSuccess)
      return e;
  } else if (a.use_norm && !xn_ready) {
    // a dense layer of one token: the pre-norm only
    if ((e = launch(k_router<kRouterWaves, 1>, dim3(1), dim3(kRouterThreads), 0, stream, ev ? ev[0] : nullptr,
                    ev ? ev[1] : nullptr, a, xn_ready, 0)) != hipSuccess)
      return e;
  }
  const int mt = a.B <= 1 ? 1 : a.B <= 2 ? 2 : a.B <= 4 ? 4 : 8;
  if (a.wtype == 1) {
    switch (mt) {
      case 1: return launch_experts<1, 1>(a, stream, ev);
      case 2: return launch_experts<1, 2>(a, stream, ev);
      case 4: return launch_experts<1, 4>(a, stream, ev);
      default: return launch_experts<1, 8>(a, stream, ev);
    }
  }
  switch (mt) {
    case 1: return launch_experts<0, 1>(a, stream, ev);
    case 2: return launch_experts<0, 2>(a, stream, ev);
    case 4: return launch_experts<0, 4>(a, stream, ev);
    default: return launch_experts<0, 8>(a, stream, ev);
  }
}

}  // namespace moe
