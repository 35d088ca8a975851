// Small-batch (1..8 tokens) decode path of the sigmoid-routed W4A16 MoE
// layer: three kernels per layer.
//
//   k_router_topk  pre-norm (optional), router GEMV (BF16 weights, FP32
//                  accumulation), then -- in the last workgroup to finish --
//                  sigmoid top-k, renormalisation and the list of distinct
//                  selected experts with their token masks and weights.
//   k_gateup       for every (selected or shared expert, 8-row group):
//                  gate and up GEMVs on NVFP4 (or BF16) weights decoded in
//                  registers, BF16 rounding of g and u, h = BF16(SiLU(g) u).
//   k_down         for every 8-row group of the output: the down GEMV of
//                  every selected expert and the shared expert, BF16
//                  rounding per expert, weighted FP32 combine, BF16 output
//                  (plus the residual when asked).
//
// What is computed follows "Day-0 Support for Flint on vLLM" (sections
// "Model architecture" and "Optimizations"): 256 experts, sigmoid top-6
// plus a shared expert; only the selected experts' weights are read;
// weight-only FP4 with BF16 activations; the reference's rounding points.
#include "common.h"

namespace moe {

constexpr int kBlock = 256;
constexpr int kWavesPerBlock = kBlock / kWave;

// ---------------------------------------------------------------------------
// Router: logits, then top-k and the expert work list in the last block.
// ---------------------------------------------------------------------------

// Better candidate: larger logit, then lower expert index.
__device__ inline bool cand_better(float va, int ia, float vb, int ib) {
  return va > vb || (va == vb && ia < ib);
}

__global__ __launch_bounds__(kBlock) void k_router_topk(DecodeArgs a) {
  extern __shared__ uint16_t s_x[];  // [B][H] BF16: x or its pre-norm
  __shared__ uint32_t s_mark[kMaxExperts];
  __shared__ int32_t s_sel[kMaxBatch][kMaxTopK];
  __shared__ float s_selw[kMaxBatch][kMaxTopK];
  __shared__ float s_red[kWavesPerBlock][kMaxBatch];
  __shared__ float s_inv[kMaxBatch];
  __shared__ int s_last;

  const int H = a.H, E = a.E, B = a.B;
  const int tid = threadIdx.x, lane = tid & (kWave - 1), wave = tid / kWave;

  // Stage x (or BF16(RMSNorm(x) * gain)) in LDS.
  if (a.use_norm) {
    float ss[kMaxBatch];
#pragma unroll
    for (int t = 0; t < kMaxBatch; ++t) ss[t] = 0.f;
    for (int t = 0; t < B; ++t)
      for (int i = tid; i < H; i += kBlock) {
        float v = bf16_to_f32(a.x[(int64_t)t * H + i]);
        ss[t] += v * v;
      }
    for (int t = 0; t < B; ++t) {
      float v = group_sum(ss[t], kWave);
      if (lane == 0) s_red[wave][t] = v;
    }
    __syncthreads();
    if (tid < B) {
      float v = 0.f;
      for (int w = 0; w < kWavesPerBlock; ++w) v += s_red[w][tid];
      s_inv[tid] = 1.0f / sqrtf(v / (float)H + a.eps);
    }
    __syncthreads();
    for (int t = 0; t < B; ++t)
      for (int i = tid; i < H; i += kBlock) {
        float v = bf16_to_f32(a.x[(int64_t)t * H + i]) * s_inv[t] * bf16_to_f32(a.norm_gain[i]);
        uint16_t r = (uint16_t)f32_to_bf16(v);
        s_x[t * H + i] = r;
        if (blockIdx.x == 0) a.ws.xn[(int64_t)t * H + i] = r;
      }
  } else {
    for (int i = tid; i < B * H; i += kBlock) s_x[i] = a.x[i];
  }
  __syncthreads();
  if (E == 0) return;  // dense layer: only the pre-norm was wanted

  // One expert row per lane group; a lane owns 32-element chunks.
  const int LPR = lanes_per_row(H), C = H / 32;
  const int groups = kBlock / LPR;
  const int row = blockIdx.x * groups + tid / LPR;
  const int lg = tid % LPR;
  if (row < E) {
    float acc[kMaxBatch];
#pragma unroll
    for (int t = 0; t < kMaxBatch; ++t) acc[t] = 0.f;
    const uint4 *wrow = reinterpret_cast<const uint4 *>(a.router_w + (int64_t)row * H);
    for (int c = lg; c < C; c += LPR) {
      uint4 w[4];
#pragma unroll
      for (int q = 0; q < 4; ++q) w[q] = wrow[c * 4 + q];
      for (int t = 0; t < B; ++t) {
        const uint4 *xr = reinterpret_cast<const uint4 *>(s_x + t * H) + c * 4;
        float s = acc[t];
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          uint4 xv = xr[q];
          s = dot2_bf16(w[q].x, xv.x, s);
          s = dot2_bf16(w[q].y, xv.y, s);
          s = dot2_bf16(w[q].z, xv.z, s);
          s = dot2_bf16(w[q].w, xv.w, s);
        }
        acc[t] = s;
      }
    }
    const float bias = a.router_b ? a.router_b[row] : 0.f;
    for (int t = 0; t < B; ++t) {
      float v = group_sum(acc[t], LPR);
      if (lg == 0) a.ws.logits[t * E + row] = v + bias;
    }
  } else {
    // Rows past E: the shuffles above are group-local, nothing to do.
  }

  // Completion count: the last block to finish selects the experts.
  __syncthreads();
  if (tid == 0) {
    __threadfence();
    unsigned prev = atomicAdd(a.ws.counter, 1u);
    s_last = (prev == gridDim.x - 1);
  }
  __syncthreads();
  if (!s_last) return;
  __threadfence();

  for (int e = tid; e < E; e += kBlock) s_mark[e] = 0u;
  __syncthreads();

  // Top-k per token, one wave per token.
  for (int t = wave; t < B; t += kWavesPerBlock) {
    const float *lt = a.ws.logits + t * E;
    float v[kMaxExperts / kWave];
    const int per = (E + kWave - 1) / kWave;
#pragma unroll
    for (int j = 0; j < kMaxExperts / kWave; ++j) {
      int e = lane + j * kWave;
      float lv = (j < per && e < E) ? lt[e] : -INFINITY;
      v[j] = (lv != lv) ? -INFINITY : lv;  // NaN never wins over a number
    }
    uint32_t taken = 0;  // bit j: candidate j of this lane already selected
    float selv[kMaxTopK];
    int seli[kMaxTopK];
    for (int r = 0; r < a.k; ++r) {
      float bv = -INFINITY;
      int bi = 0x7fffffff;
#pragma unroll
      for (int j = 0; j < kMaxExperts / kWave; ++j) {
        int e = lane + j * kWave;
        if (j < per && e < E && !((taken >> j) & 1u) && cand_better(v[j], e, bv, bi)) {
          bv = v[j];
          bi = e;
        }
      }
      for (int o = kWave / 2; o > 0; o >>= 1) {
        float ov = __shfl_xor(bv, o, kWave);
        int oi = __shfl_xor(bi, o, kWave);
        if (cand_better(ov, oi, bv, bi)) {
          bv = ov;
          bi = oi;
        }
      }
      if ((bi & (kWave - 1)) == lane) taken |= 1u << (bi / kWave);
      selv[r] = bv;
      seli[r] = bi;
    }
    if (lane == 0) {
      float s[kMaxTopK], sum = 0.f;
      for (int r = 0; r < a.k; ++r) {
        // The logit of a selected expert: re-read it (the reduction kept
        // -inf for NaN, which only matters for NaN input).
        float l = lt[seli[r]];
        s[r] = 1.0f / (1.0f + expf(-l));
        sum += s[r];
      }
      for (int r = 0; r < a.k; ++r) {
        float w = s[r] / sum;
        s_sel[t][r] = seli[r];
        s_selw[t][r] = w;
        a.out_idx[t * a.k + r] = seli[r];
        a.out_w[t * a.k + r] = w;
        atomicOr(&s_mark[seli[r]], 1u << t);
      }
      (void)selv;
    }
  }
  __syncthreads();

  // Distinct experts in ascending order with token masks and weights.
  if (wave == 0) {
    int count = 0;
    for (int base = 0; base < E; base += kWave) {
      int e = base + lane;
      uint32_t m = (e < E) ? s_mark[e] : 0u;
      unsigned long long ball = __ballot(m != 0u);
      int pre = __popcll(ball & ((1ull << lane) - 1ull));
      if (m) {
        int slot = count + pre;
        a.ws.entry_expert[slot] = e;
        a.ws.entry_mask[slot] = m;
        for (int t = 0; t < kMaxBatch; ++t) {
          float w = 0.f;
          if (t < B)
            for (int r = 0; r < a.k; ++r)
              if (s_sel[t][r] == e) w = s_selw[t][r];
          a.ws.entry_w[slot * kMaxBatch + t] = w;
        }
      }
      count += __popcll(ball);
    }
    if (lane == 0) {
      *a.ws.n_routed = count;
      __hip_atomic_store(a.ws.counter, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
  }
}

// ---------------------------------------------------------------------------
// Expert GEMV building blocks
// ---------------------------------------------------------------------------

// One lane's share of 8 rows x one 32-element chunk of an NVFP4 matrix:
// acc[r] += sum over the chunk of W[row0 + r][.] * x[.], before the tensor
// scale.  nib: 8 nibble loads (one per row), sc: the chunk's scale tile.
__device__ inline void nvfp4_chunk8(const uint4 (&nib)[8], const uint4 &sc, const uint4 (&xv)[4],
                                    float (&acc)[8]) {
  const uint32_t scw[4] = {sc.x, sc.y, sc.z, sc.w};
  const uint32_t xw[16] = {xv[0].x, xv[0].y, xv[0].z, xv[0].w, xv[1].x, xv[1].y, xv[1].z, xv[1].w,
                           xv[2].x, xv[2].y, xv[2].z, xv[2].w, xv[3].x, xv[3].y, xv[3].z, xv[3].w};
#pragma unroll
  for (int r = 0; r < 8; ++r) {
    const uint32_t nw[4] = {nib[r].x, nib[r].y, nib[r].z, nib[r].w};
    float p0 = 0.f, p1 = 0.f;
    p0 = dot8_fp4_bf16(nw[0], xw[0], xw[1], xw[2], xw[3], p0);
    p0 = dot8_fp4_bf16(nw[1], xw[4], xw[5], xw[6], xw[7], p0);
    p1 = dot8_fp4_bf16(nw[2], xw[8], xw[9], xw[10], xw[11], p1);
    p1 = dot8_fp4_bf16(nw[3], xw[12], xw[13], xw[14], xw[15], p1);
    // scale bytes of row r: 2r (block 2c) and 2r+1 (block 2c+1)
    uint32_t sword = scw[r >> 1] >> ((r & 1) * 16);
    float s0 = e4m3_to_f32(sword & 0xffu), s1 = e4m3_to_f32((sword >> 8) & 0xffu);
    acc[r] = fmaf(s0, p0, fmaf(s1, p1, acc[r]));
  }
}

__device__ inline void load_chunk8_nvfp4(const uint8_t *m, int64_t N, int64_t K, int rg, int c,
                                         uint4 (&nib)[8], uint4 &sc) {
  const int64_t rowb = K / 2;
  const uint8_t *p = m + (int64_t)(rg * 8) * rowb + (int64_t)c * 16;
#pragma unroll
  for (int r = 0; r < 8; ++r) nib[r] = *reinterpret_cast<const uint4 *>(p + r * rowb);
  sc = *reinterpret_cast<const uint4 *>(m + N * K / 2 + ((int64_t)rg * (K / 32) + c) * 16);
}

__device__ inline void load_x_chunk(const uint16_t *xrow, int c, uint4 (&xv)[4]) {
  const uint4 *p = reinterpret_cast<const uint4 *>(xrow) + c * 4;
#pragma unroll
  for (int q = 0; q < 4; ++q) xv[q] = p[q];
}

// BF16 weights: acc[r] += W[row0 + r][32c .. 32c+31] . x chunk, 8 rows.
__device__ inline void bf16_chunk8(const uint16_t *m, int64_t K, int rg, int c, const uint4 (&xv)[4],
                                   float (&acc)[8]) {
  const uint32_t xw[16] = {xv[0].x, xv[0].y, xv[0].z, xv[0].w, xv[1].x, xv[1].y, xv[1].z, xv[1].w,
                           xv[2].x, xv[2].y, xv[2].z, xv[2].w, xv[3].x, xv[3].y, xv[3].z, xv[3].w};
#pragma unroll
  for (int r = 0; r < 8; ++r) {
    const uint4 *p = reinterpret_cast<const uint4 *>(m + (int64_t)(rg * 8 + r) * K) + c * 4;
    float s = acc[r];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      uint4 w = p[q];
      s = dot2_bf16(w.x, xw[q * 4 + 0], s);
      s = dot2_bf16(w.y, xw[q * 4 + 1], s);
      s = dot2_bf16(w.z, xw[q * 4 + 2], s);
      s = dot2_bf16(w.w, xw[q * 4 + 3], s);
    }
    acc[r] = s;
  }
}

// Value of register-array element i for lane-dependent i without dynamic
// register indexing.
__device__ inline float pick8(const float (&v)[8], int i) {
  float r = 0.f;
#pragma unroll
  for (int q = 0; q < 8; ++q) r = (i == q) ? v[q] : r;
  return r;
}

// ---------------------------------------------------------------------------
// Gate/up + SiLU*up
// ---------------------------------------------------------------------------

template <int WT>
__global__ __launch_bounds__(kBlock) void k_gateup(DecodeArgs a) {
  const int H = a.H, I = a.I, B = a.B;
  const int LPR = lanes_per_row(H), C = H / 32;
  const int groups_per_block = kBlock / LPR;
  const int u = blockIdx.x * groups_per_block + threadIdx.x / LPR;
  const int lg = threadIdx.x % LPR;
  const int routed_units = a.max_routed * (I / 8);

  int slot, rg, N;
  uint32_t mask;
  const uint8_t *Wg, *Wu;
  float Sg = 1.f, Su = 1.f;
  if (u < routed_units) {
    slot = u / (I / 8);
    rg = u % (I / 8);
    if (slot >= *a.ws.n_routed) return;
    const int e = a.ws.entry_expert[slot];
    mask = a.ws.entry_mask[slot];
    N = I;
    const int64_t mb = (WT == 1) ? nvfp4_matrix_bytes(I, H) : (int64_t)I * H * 2;
    Wg = a.w_gate + e * mb;
    Wu = a.w_up + e * mb;
    if (WT == 1) {
      Sg = a.w_scale[3 * e + 0];
      Su = a.w_scale[3 * e + 1];
    }
  } else {
    rg = u - routed_units;
    if (rg >= a.Is / 8) return;
    slot = a.max_routed;
    mask = (1u << B) - 1u;
    N = a.Is;
    Wg = a.sh_gate;
    Wu = a.sh_up;
    if (WT == 1) {
      Sg = a.sh_scale[0];
      Su = a.sh_scale[1];
    }
  }
  const uint16_t *xs = a.use_norm ? a.ws.xn : a.x;
  const int Imax = a.I > a.Is ? a.I : a.Is;

  if (WT == 1 && C <= LPR) {
    // One chunk per lane: load the weights once, reuse them for each token.
    uint4 ng[8], nu[8], sg, su;
    load_chunk8_nvfp4(Wg, N, H, rg, lg, ng, sg);
    load_chunk8_nvfp4(Wu, N, H, rg, lg, nu, su);
    for (int t = 0; t < B; ++t) {
      if (!((mask >> t) & 1u)) continue;
      uint4 xv[4];
      load_x_chunk(xs + (int64_t)t * H, lg, xv);
      float ag[8] = {0, 0, 0, 0, 0, 0, 0, 0}, au[8] = {0, 0, 0, 0, 0, 0, 0, 0};
      nvfp4_chunk8(ng, sg, xv, ag);
      nvfp4_chunk8(nu, su, xv, au);
#pragma unroll
      for (int r = 0; r < 8; ++r) {
        ag[r] = group_sum(ag[r], LPR);
        au[r] = group_sum(au[r], LPR);
      }
      // Every lane holds all 8 sums; lanes of the group split the rows
      // (a group can have fewer than 8 lanes).
      for (int r = lg; r < 8; r += LPR) {
        float g = round_bf16(pick8(ag, r) * Sg);
        float uu = round_bf16(pick8(au, r) * Su);
        float h = g / (1.0f + expf(-g)) * uu;
        a.ws.h[((int64_t)slot * B + t) * Imax + rg * 8 + r] = (uint16_t)f32_to_bf16(h);
      }
    }
  } else {
    for (int t = 0; t < B; ++t) {
      if (!((mask >> t) & 1u)) continue;
      float ag[8] = {0, 0, 0, 0, 0, 0, 0, 0}, au[8] = {0, 0, 0, 0, 0, 0, 0, 0};
      for (int c = lg; c < C; c += LPR) {
        uint4 xv[4];
        load_x_chunk(xs + (int64_t)t * H, c, xv);
        if (WT == 1) {
          uint4 ng[8], nu[8], sg, su;
          load_chunk8_nvfp4(Wg, N, H, rg, c, ng, sg);
          load_chunk8_nvfp4(Wu, N, H, rg, c, nu, su);
          nvfp4_chunk8(ng, sg, xv, ag);
          nvfp4_chunk8(nu, su, xv, au);
        } else {
          bf16_chunk8(reinterpret_cast<const uint16_t *>(Wg), H, rg, c, xv, ag);
          bf16_chunk8(reinterpret_cast<const uint16_t *>(Wu), H, rg, c, xv, au);
        }
      }
#pragma unroll
      for (int r = 0; r < 8; ++r) {
        ag[r] = group_sum(ag[r], LPR);
        au[r] = group_sum(au[r], LPR);
      }
      // Every lane holds all 8 sums; lanes of the group split the rows
      // (a group can have fewer than 8 lanes).
      for (int r = lg; r < 8; r += LPR) {
        float g = round_bf16(pick8(ag, r) * Sg);
        float uu = round_bf16(pick8(au, r) * Su);
        float h = g / (1.0f + expf(-g)) * uu;
        a.ws.h[((int64_t)slot * B + t) * Imax + rg * 8 + r] = (uint16_t)f32_to_bf16(h);
      }
    }
  }
}

// ---------------------------------------------------------------------------
// Down GEMV + weighted combine (+ residual)
// ---------------------------------------------------------------------------

constexpr int kMaxSlots = 32;  // expert slots reduced per pass of k_down

template <int WT>
__global__ __launch_bounds__(kBlock) void k_down(DecodeArgs a) {
  const int H = a.H, B = a.B;
  const int K = (a.E > 0) ? a.I : a.Is;  // Is == I when both exist
  const int LPR = lanes_per_row(K), C = K / 32;
  const int slots = (kBlock / LPR) < kMaxSlots ? (kBlock / LPR) : kMaxSlots;
  const int slot_id = threadIdx.x / LPR, lg = threadIdx.x % LPR;
  const int rg = blockIdx.x;
  const int n_routed = (a.E > 0) ? *a.ws.n_routed : 0;
  const int n_entries = n_routed + (a.Is > 0 ? 1 : 0);
  const int Imax = a.I > a.Is ? a.I : a.Is;

  __shared__ float s_part[kMaxSlots][kMaxBatch][8];
  float total = 0.f;  // owned by thread (t, r) = (tid / 8, tid % 8)

  for (int base = 0; base < n_entries; base += slots) {
    const int j = (slot_id < slots) ? base + slot_id : n_entries;
    float contrib[kMaxBatch][8];
#pragma unroll
    for (int t = 0; t < kMaxBatch; ++t)
#pragma unroll
      for (int r = 0; r < 8; ++r) contrib[t][r] = 0.f;
    if (j < n_entries) {
      const uint8_t *Wd;
      float Sd = 1.f;
      uint32_t mask;
      int hslot;
      const float *wt = nullptr;
      if (j < n_routed) {
        const int e = a.ws.entry_expert[j];
        mask = a.ws.entry_mask[j];
        const int64_t mb = (WT == 1) ? nvfp4_matrix_bytes(H, K) : (int64_t)H * K * 2;
        Wd = a.w_down + e * mb;
        if (WT == 1) Sd = a.w_scale[3 * e + 2];
        hslot = j;
        wt = a.ws.entry_w + j * kMaxBatch;
      } else {
        mask = (1u << B) - 1u;
        Wd = a.sh_down;
        if (WT == 1) Sd = a.sh_scale[2];
        hslot = a.max_routed;
      }
      for (int t = 0; t < B; ++t) {
        if (!((mask >> t) & 1u)) continue;
        float acc[8] = {0, 0, 0, 0, 0, 0, 0, 0};
        for (int c = lg; c < C; c += LPR) {
          uint4 hv[4];
          load_x_chunk(a.ws.h + ((int64_t)hslot * B + t) * Imax, c, hv);
          if (WT == 1) {
            uint4 nb[8], sc;
            load_chunk8_nvfp4(Wd, H, K, rg, c, nb, sc);
            nvfp4_chunk8(nb, sc, hv, acc);
          } else {
            bf16_chunk8(reinterpret_cast<const uint16_t *>(Wd), K, rg, c, hv, acc);
          }
        }
        const float w = wt ? wt[t] : 1.0f;
#pragma unroll
        for (int r = 0; r < 8; ++r) contrib[t][r] = w * round_bf16(group_sum(acc[r], LPR) * Sd);
      }
    }
    if (lg == 0 && slot_id < slots) {
#pragma unroll
      for (int t = 0; t < kMaxBatch; ++t)
#pragma unroll
        for (int r = 0; r < 8; ++r) s_part[slot_id][t][r] = contrib[t][r];
    }
    __syncthreads();
    if (threadIdx.x < B * 8) {
      const int t = threadIdx.x / 8, r = threadIdx.x % 8;
      for (int s = 0; s < slots; ++s) total += s_part[s][t][r];
    }
    __syncthreads();
  }
  if (threadIdx.x < B * 8) {
    const int t = threadIdx.x / 8, r = threadIdx.x % 8;
    const int64_t o = (int64_t)t * H + rg * 8 + r;
    float v = round_bf16(total);
    if (a.residual) v = bf16_to_f32(a.x[o]) + v;
    a.y[o] = (uint16_t)f32_to_bf16(v);
  }
}

// ---------------------------------------------------------------------------
// Host launcher
// ---------------------------------------------------------------------------

hipError_t launch_decode(const DecodeArgs &a, hipStream_t stream) {
  if (a.E > 0 || a.use_norm) {
    const int LPR = lanes_per_row(a.H);
    const int rows_per_block = kBlock / LPR;
    const int grid = a.E > 0 ? (a.E + rows_per_block - 1) / rows_per_block : 1;
    const size_t lds = (size_t)a.B * a.H * 2;
    hipLaunchKernelGGL(k_router_topk, dim3(grid), dim3(kBlock), lds, stream, a);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  {
    const int LPR = lanes_per_row(a.H);
    const int groups = kBlock / LPR;
    const int units = a.max_routed * (a.I / 8) + a.Is / 8;
    const int grid = (units + groups - 1) / groups;
    if (a.wtype == 1)
      hipLaunchKernelGGL(k_gateup<1>, dim3(grid), dim3(kBlock), 0, stream, a);
    else
      hipLaunchKernelGGL(k_gateup<0>, dim3(grid), dim3(kBlock), 0, stream, a);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  {
    const int grid = a.H / 8;
    if (a.wtype == 1)
      hipLaunchKernelGGL(k_down<1>, dim3(grid), dim3(kBlock), 0, stream, a);
    else
      hipLaunchKernelGGL(k_down<0>, dim3(grid), dim3(kBlock), 0, stream, a);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

}  // namespace moe
