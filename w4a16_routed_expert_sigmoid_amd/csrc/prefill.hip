// Prefill of the sigmoid-routed W4A16 MoE layer over T tokens: the same
// per-token computation as the decode path, organised for the matrix cores.
// "Day-0 Support for Flint on vLLM", section "Optimizations": the MoE kernel
// also gives the largest prefill gain (8,192-token prefill measured).
//
//   k_pf_norm     (pre-norm layers) xn = BF16(RMSNorm(x) * gain), one wave per token
//   k_pf_router   logits = xn W_r^T + b: GEMM on v_mfma_f32_32x32x16_bf16
//                 (its first block also clears the expert counts and cursors)
//   k_pf_topk     sigmoid top-k per token (one wave each), renormalised
//                 weights, per-expert token counts (LDS histogram per block)
//   k_pf_place    expert offsets (every block scans the counts; block 0
//                 writes them and the tile list: every expert's rows in tiles
//                 of 128, then the shared expert's tiles), and each (token, k)
//                 pair's row in its expert's segment
//   k_pf_gemm_fp4<0>, <1>  (NVFP4 weights) grouped GEMMs over the tiles:
//                 gathered xn rows x the expert's gate and up matrices,
//                 epilogue h = BF16(SiLU(BF16(g)) BF16(u)); then h rows x the
//                 down matrix, epilogue y = BF16(acc * S_down) (below)
//   k_pf_gateup, k_pf_down  the same two GEMMs for BF16 weights
//   k_pf_combine  out = BF16(sum_j w_j y_row(t,j) + y_shared(t)) (+ residual)
//
// Row space of the grouped GEMMs: rows [0, P) are the P = T*k (token,
// expert) pairs sorted by expert; rows [P, P + T) are the shared expert's
// (token order).  h and y are stored per row.
#include <string.h>

#include "common.h"
#include "mm_rows.h"

namespace moe {

typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr int PBM = kPrefillTileRows;  // tile rows (tokens)
constexpr int PBN = 128;  // tile columns
constexpr int PBK = 32;   // K per stage (two 16-element NVFP4 blocks)
constexpr int PLD = PBK + 8;  // LDS row stride in BF16 elements (padding)
constexpr int PThreads = 256;

// ---------------------------------------------------------------------------
// Shared GEMM machinery: 4 waves as 2x2, each wave 64x64 of the 128x128 tile
// as 2x2 blocks of 32x32 (v_mfma_f32_32x32x16_bf16).  Lane layouts (checked
// on the GPU): A lane l holds row l%32, k (l/32)*8..+8; B lane l holds column
// l%32, k (l/32)*8..+8; C lane l, value i is row (i/4)*8 + (l/32)*4 + i%4,
// column l%32.
// ---------------------------------------------------------------------------



// 16 FP4 elements (8 bytes, element 2i in the low nibble of byte i) times
// the block scale s -> 16 BF16 (exact: E2M1 x E4M3 has <= 6 significant bits).
__device__ __forceinline__ void dequant16(uint32_t w0, uint32_t w1, float s, uint32_t (&o)[8]) {
  const uint32_t w[2] = {w0, w1};
#pragma unroll
  for (int d = 0; d < 2; ++d) {
#pragma unroll
    for (int b = 0; b < 4; ++b) {
      f32x2 v;
      switch (b) {
        case 0: v = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w[d], 1.0f, 0); break;
        case 1: v = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w[d], 1.0f, 1); break;
        case 2: v = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w[d], 1.0f, 2); break;
        default: v = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w[d], 1.0f, 3); break;
      }
      o[d * 4 + b] = f32_to_bf16(v.x * s) | (f32_to_bf16(v.y * s) << 16);
    }
  }
}

// B row of one stage into LDS: 16 K-elements starting at k (k % 16 == 0) of
// row n of matrix m (rows x K), as BF16.  Rows past the matrix are zero.
template <int BT>
__device__ __forceinline__ void stage_b(const uint8_t *m, int rows, int K, int n, int k, uint16_t *dst) {
  uint4 o0, o1;
  if (m == nullptr || n >= rows) {
    o0 = o1 = make_uint4(0, 0, 0, 0);
  } else if (BT == 1) {
    const uint2 nib = *reinterpret_cast<const uint2 *>(m + (int64_t)n * (K / 2) + k / 2);
    const uint8_t sb = m[(int64_t)rows * (K / 2) + ((int64_t)(n >> 3) * (K / 32) + k / 32) * 16 + (n & 7) * 2 +
                         ((k / 16) & 1)];
    uint32_t o[8];
    dequant16(nib.x, nib.y, e4m3_to_f32(sb), o);
    o0 = make_uint4(o[0], o[1], o[2], o[3]);
    o1 = make_uint4(o[4], o[5], o[6], o[7]);
  } else {
    const uint4 *p = reinterpret_cast<const uint4 *>(reinterpret_cast<const uint16_t *>(m) + (int64_t)n * K + k);
    o0 = p[0];
    o1 = p[1];
  }
  reinterpret_cast<uint4 *>(dst)[0] = o0;
  reinterpret_cast<uint4 *>(dst)[1] = o1;
}

__device__ __forceinline__ void stage_a(const uint16_t *row, int k, uint16_t *dst) {
  uint4 o0, o1;
  if (row == nullptr) {
    o0 = o1 = make_uint4(0, 0, 0, 0);
  } else {
    const uint4 *p = reinterpret_cast<const uint4 *>(row + k);
    o0 = p[0];
    o1 = p[1];
  }
  reinterpret_cast<uint4 *>(dst)[0] = o0;
  reinterpret_cast<uint4 *>(dst)[1] = o1;
}

// One stage of MFMAs from LDS: acc[mb][nb] += A[wm*64+mb*32..][.] x B[wn*64+nb*32..][.]^T
__device__ __forceinline__ void mfma_stage(const uint16_t *sA, const uint16_t *sB, f32x16 (&acc)[2][2]) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int wm = wave >> 1, wn = wave & 1;
#pragma unroll
  for (int ks = 0; ks < PBK / 16; ++ks) {
    bf16x8 a[2], b[2];
#pragma unroll
    for (int mb = 0; mb < 2; ++mb)
      a[mb] = *reinterpret_cast<const bf16x8 *>(sA + (wm * 64 + mb * 32 + (lane & 31)) * PLD + ks * 16 + (lane >> 5) * 8);
#pragma unroll
    for (int nb = 0; nb < 2; ++nb)
      b[nb] = *reinterpret_cast<const bf16x8 *>(sB + (wn * 64 + nb * 32 + (lane & 31)) * PLD + ks * 16 + (lane >> 5) * 8);
#pragma unroll
    for (int mb = 0; mb < 2; ++mb)
#pragma unroll
      for (int nb = 0; nb < 2; ++nb) acc[mb][nb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[mb], b[nb], acc[mb][nb], 0, 0, 0);
  }
}

// Row / column of value i of acc[mb][nb] within the 128x128 tile.
__device__ __forceinline__ int acc_row(int mb, int i) {
  const int lane = threadIdx.x & 63, wm = (threadIdx.x >> 6) >> 1;
  return wm * 64 + mb * 32 + (i / 4) * 8 + (lane >> 5) * 4 + (i % 4);
}
__device__ __forceinline__ int acc_col(int nb) {
  const int lane = threadIdx.x & 63, wn = (threadIdx.x >> 6) & 1;
  return wn * 64 + nb * 32 + (lane & 31);
}



// ---------------------------------------------------------------------------
// Small kernels
// ---------------------------------------------------------------------------


__global__ __launch_bounds__(PThreads) void k_pf_norm(PrefillArgs a) {
  const int lane = threadIdx.x & 63;
  const int t = blockIdx.x * (PThreads / 64) + (threadIdx.x >> 6);
  if (t >= a.T) return;
  const uint16_t *xr = a.x + (int64_t)t * a.H;
  double ss = 0.0;  // squares of BF16 values are exact in FP64
  if (a.H <= 64 * 8 * 8) {
    // up to 8 pieces per lane: the token and the gain loaded once, all in
    // flight together, the token kept in registers for the second pass
    // (pieces past H read as zeros and are not stored)
    constexpr int NP = 8;
    uint4 xv[NP], gv[NP];
#pragma unroll
    for (int j = 0; j < NP; ++j) {
      const int i = lane * 8 + j * 64 * 8;
      const int ic = i < a.H ? i : 0;
      xv[j] = *reinterpret_cast<const uint4 *>(xr + ic);
      gv[j] = *reinterpret_cast<const uint4 *>(a.norm_gain + ic);
      if (i >= a.H) xv[j] = make_uint4(0, 0, 0, 0);
    }
#pragma unroll
    for (int j = 0; j < NP; ++j) {
      const uint32_t w[4] = {xv[j].x, xv[j].y, xv[j].z, xv[j].w};
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const double lo = bf16_to_f32(w[q] & 0xffffu), hi = bf16_to_f32(w[q] >> 16);
        ss = fma(lo, lo, fma(hi, hi, ss));
      }
    }
    ss = group_sum_f64(ss, 64);
    const double inv = 1.0 / sqrt(ss / (double)a.H + (double)a.eps);
    const float inv_f = (float)inv;
#pragma unroll
    for (int j = 0; j < NP; ++j) {
      const int i = lane * 8 + j * 64 * 8;
      if (i < a.H) *reinterpret_cast<uint4 *>(a.xn + (int64_t)t * a.H + i) = norm_piece_bf16(xv[j], gv[j], inv_f, inv);
    }
    return;
  }
  for (int i = lane * 8; i < a.H; i += 64 * 8) {
    const uint4 v = *reinterpret_cast<const uint4 *>(xr + i);
    const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const double lo = bf16_to_f32(w[q] & 0xffffu), hi = bf16_to_f32(w[q] >> 16);
      ss = fma(lo, lo, fma(hi, hi, ss));
    }
  }
  ss = group_sum_f64(ss, 64);
  const double inv = 1.0 / sqrt(ss / (double)a.H + (double)a.eps);
  const float inv_f = (float)inv;
  for (int i = lane * 8; i < a.H; i += 64 * 8) {
    const uint4 v = *reinterpret_cast<const uint4 *>(xr + i);
    const uint4 g = *reinterpret_cast<const uint4 *>(a.norm_gain + i);
    *reinterpret_cast<uint4 *>(a.xn + (int64_t)t * a.H + i) = norm_piece_bf16(v, g, inv_f, inv);
  }
}

// Orderable 32-bit key of a logit (NaN as -inf; 0 = taken).
__device__ __forceinline__ uint32_t pf_key(float l) {
  if (l != l) l = -INFINITY;
  l += 0.0f;  // -0 -> +0: equal logits tie by index
  const uint32_t u = __float_as_uint(l);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// The logit of a key (NaN came in as -inf).
__device__ __forceinline__ float pf_key_logit(uint32_t u) {
  return __uint_as_float((u & 0x80000000u) ? (u & 0x7fffffffu) : ~u);
}

constexpr int kPfTokensPerWave = 2;
constexpr int kPfTopkWaves = 16;

// Top-k of each token (one wave per token at a time), weights, counts.  J:
// logits per lane (E <= 64 J); lane l holds experts l*J .. l*J+J-1, so the
// lowest expert index holding a key is in the lowest lane holding it.  Each
// round every lane notes the first slot of its own max and its keys and max
// without that slot, beside the wave max; one ballot then names the lowest
// lane holding the max, which drops its slot (ties to the lower index).
template <int J, int W>
__global__ __launch_bounds__(W *kWave) void k_pf_topk(PrefillArgs a) {
  __shared__ uint32_t s_hist[kMaxExperts];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  for (int e = threadIdx.x; e < a.E; e += W * kWave) s_hist[e] = 0u;
  __syncthreads();
  const int t0 = (blockIdx.x * W + wave) * kPfTokensPerWave;
  const __amdgpu_buffer_rsrc_t lr = buf_rsrc(a.logits, a.rsplit > 1 ? (int64_t)a.rsplit * a.T * a.E * 4 : 0);
  for (int tt = 0; tt < kPfTokensPerWave; ++tt) {
    const int t = t0 + tt;
    if (t >= a.T) break;
    uint32_t key[J];
    if (a.rsplit == 1) {
      const float *lt = a.logits + (int64_t)t * a.E;
#pragma unroll
      for (int j = 0; j < J; ++j) {
        const int e = lane * J + j;
        key[j] = (e < a.E) ? pf_key(lt[e]) : 0u;
      }
    } else {
      // the router's K splits (a split call has under 128 router tiles,
      // T E < 2^19, so its partial logits span under 16 MiB), summed in
      // split order; the partials
      // of four logits are loaded at once (splits past a.rsplit read zeros,
      // and adding +0 changes no sum that pf_key sees)
      const uint32_t lbase = (uint32_t)(t * a.E) * 4u, zstride = (uint32_t)(a.T * a.E) * 4u;
#pragma unroll
      for (int j0 = 0; j0 < J; j0 += 4) {
        float part[4][kRouterMaxSplit];
        const int e0 = lane * J + j0;
        if ((a.E & 3) == 0) {
          // E % 4 == 0: the four logits are one 16-byte piece of each split
#pragma unroll
          for (int z = 0; z < kRouterMaxSplit; ++z) {
            const uint4 v = buf_load16(lr, buf_off(e0 < a.E && z < a.rsplit, lbase + z * zstride + (uint32_t)e0 * 4u));
            part[0][z] = __uint_as_float(v.x);
            part[1][z] = __uint_as_float(v.y);
            part[2][z] = __uint_as_float(v.z);
            part[3][z] = __uint_as_float(v.w);
          }
        } else {
#pragma unroll
          for (int j = 0; j < 4; ++j)
#pragma unroll
            for (int z = 0; z < kRouterMaxSplit; ++z)
              part[j][z] =
                  buf_load4f(lr, buf_off(e0 + j < a.E && z < a.rsplit, lbase + z * zstride + (uint32_t)(e0 + j) * 4u));
        }
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const int e = lane * J + j0 + j;
          float l = part[j][0];
#pragma unroll
          for (int z = 1; z < kRouterMaxSplit; ++z) l += part[j][z];
          key[j0 + j] = (e < a.E) ? pf_key(l) : 0u;
        }
      }
    }
    uint32_t lmax = key[0];
#pragma unroll
    for (int j = 1; j < J; ++j) lmax = max(lmax, key[j]);
    int my_e = 0;
    float my_l = 0.f;
    for (int r = 0; r < a.k; ++r) {
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
      const int e = L * J + __builtin_amdgcn_readlane(jm, L);
      const bool mine = lane == L;
#pragma unroll
      for (int j = 0; j < J; ++j) key[j] = mine ? keyx[j] : key[j];
      lmax = mine ? lx : lmax;
      if (lane == r) {
        my_e = e;
        my_l = pf_key_logit(m);
      }
    }
    // the same arithmetic as the decode path: sigmoid from the hardware
    // base-2 exponential and reciprocal, the sum over lanes 0..7 (0 past k)
    // in a fixed butterfly order, one correctly rounded division
    const float s = (lane < a.k) ? __builtin_amdgcn_rcpf(1.0f + __builtin_amdgcn_exp2f(-my_l * 1.44269504088896341f))
                                 : 0.f;
    float sum = s + xor_lane<1>(s);
    sum += xor_lane<2>(sum);
    sum += xor_lane<4>(sum);
    if (lane < a.k) {
      a.out_idx[(int64_t)t * a.k + lane] = my_e;
      a.out_w[(int64_t)t * a.k + lane] = s / sum;
      atomicAdd(&s_hist[my_e], 1u);
    }
  }
  __syncthreads();
  for (int e = threadIdx.x; e < a.E; e += W * kWave)
    if (s_hist[e]) atomicAdd(&a.counts[e], (int)s_hist[e]);
}

// Expert offsets, the tile list and every pair's row.  Each block scans the
// expert counts in LDS (thread i owns experts 4i .. 4i+3; one scan over the
// 256 thread sums for rows and one for 128-row tiles); block 0 writes the
// offsets and the tile list.  Then the block's (token, k) pairs, PThreads * 2
// at a time: ranks within the block from an LDS histogram, one atomic per
// expert on a cursor that starts at zero, row = offset + cursor + rank.
constexpr int kPlaceExp = kMaxExperts / PThreads;  // experts per thread in the scan
static_assert(kMaxExperts % PThreads == 0, "the scan splits the experts evenly");
constexpr int kPlaceMaxBlocks = 1024;

__global__ __launch_bounds__(PThreads) void k_pf_place(PrefillArgs a) {
  __shared__ int s_rows[PThreads], s_tl[PThreads];
  __shared__ int s_off[kMaxExperts];
  __shared__ uint32_t s_cnt[kMaxExperts];
  __shared__ int s_base[kMaxExperts];
  const int tid = threadIdx.x;
  const int TR = a.tile_rows;
  int c[kPlaceExp], rows = 0, tl = 0;
#pragma unroll
  for (int j = 0; j < kPlaceExp; ++j) {
    const int e = tid * kPlaceExp + j;
    c[j] = e < a.E ? a.counts[e] : 0;
    rows += c[j];
    tl += (c[j] + TR - 1) / TR;
  }
  s_rows[tid] = rows;
  s_tl[tid] = tl;
  __syncthreads();
  for (int o = 1; o < PThreads; o <<= 1) {
    const int vr = tid >= o ? s_rows[tid - o] : 0, vt = tid >= o ? s_tl[tid - o] : 0;
    __syncthreads();
    s_rows[tid] += vr;
    s_tl[tid] += vt;
    __syncthreads();
  }
  int off = s_rows[tid] - rows, toff = s_tl[tid] - tl;
#pragma unroll
  for (int j = 0; j < kPlaceExp; ++j) {
    const int e = tid * kPlaceExp + j;
    s_off[e] = off;
    if (blockIdx.x == 0 && e < a.E) {
      a.offsets[e] = off;
      const int nt = (c[j] + TR - 1) / TR;
      for (int i = 0; i < nt; ++i) a.tiles[toff + i] = PfTile{off + i * TR, min(TR, c[j] - i * TR), e};
    }
    off += c[j];
    toff += (c[j] + TR - 1) / TR;
  }
  if (blockIdx.x == 0) {
    const int routed_tiles = s_tl[PThreads - 1];
    const int shared_tiles = a.Is > 0 ? (a.T + TR - 1) / TR : 0;
    for (int i = tid; i < shared_tiles; i += PThreads)
      a.tiles[routed_tiles + i] = PfTile{a.P + i * TR, min(TR, a.T - i * TR), -1};
    if (tid == 0) {
      a.offsets[a.E] = s_rows[PThreads - 1];
      *a.n_tiles = routed_tiles + shared_tiles;
    }
  }
  __syncthreads();

  constexpr int kPairsPerThread = 2;
  const int64_t P = (int64_t)a.T * a.k;
  for (int64_t b0 = (int64_t)blockIdx.x * PThreads * kPairsPerThread; b0 < P;
       b0 += (int64_t)gridDim.x * PThreads * kPairsPerThread) {
    for (int e = tid; e < a.E; e += PThreads) s_cnt[e] = 0u;
    __syncthreads();
    const int64_t q0 = b0 + (int64_t)tid * kPairsPerThread;
    int rank[kPairsPerThread], ex[kPairsPerThread];
#pragma unroll
    for (int i = 0; i < kPairsPerThread; ++i) {
      ex[i] = -1;
      if (q0 + i < P) {
        ex[i] = a.out_idx[q0 + i];
        rank[i] = (int)atomicAdd(&s_cnt[ex[i]], 1u);
      }
    }
    __syncthreads();
    for (int e = tid; e < a.E; e += PThreads)
      s_base[e] = s_cnt[e] ? s_off[e] + atomicAdd(&a.cursors[e], (int)s_cnt[e]) : 0;
    __syncthreads();
#pragma unroll
    for (int i = 0; i < kPairsPerThread; ++i) {
      if (ex[i] < 0) continue;
      const int pos = s_base[ex[i]] + rank[i];
      a.sorted_tok[pos] = (int)((q0 + i) / a.k);
      a.pair_pos[q0 + i] = pos;
    }
    __syncthreads();
  }
}

// ---------------------------------------------------------------------------
// GEMM kernels
// ---------------------------------------------------------------------------

// Router logits: rows = tokens, columns = experts, B = BF16 router weights.
// 64 x 64 tiles (enough blocks to fill the GPU at E = 256); each of the 4
// waves owns a 32 x 32 quarter; 128-K stages through LDS, the next stage's
// loads in flight during the current stage's MFMAs.
constexpr int RBM = 64, RBN = 64, RBK = 128, RLD = RBK + 8;
constexpr int RPART = RBK / 4, RV = RPART / 8;  // K elements and 16-byte loads per thread and stage

__global__ __launch_bounds__(PThreads) void k_pf_router(PrefillArgs a) {
  __shared__ __attribute__((aligned(16))) uint16_t sA[2][RBM * RLD];
  __shared__ __attribute__((aligned(16))) uint16_t sB[2][RBN * RLD];
  const int m0 = blockIdx.x * RBM, n0 = blockIdx.y * RBN;
  const uint16_t *xs = a.use_norm ? a.xn : a.x;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  // the expert counts the top-k kernel accumulates, and the cursors the
  // placement kernel advances, start at zero
  if (blockIdx.x == 0 && blockIdx.y == 0 && blockIdx.z == 0)
    for (int i = tid; i < a.E + 1; i += PThreads) {
      a.counts[i] = 0;
      a.cursors[i] = 0;
    }
  const int r = tid >> 2, part = tid & 3;  // loads: row r, K elements part*RPART .. +RPART of the stage
  const uint16_t *arow = (m0 + r < a.T) ? xs + (int64_t)(m0 + r) * a.H : nullptr;
  const uint16_t *brow = (n0 + r < a.E) ? a.router_w + (int64_t)(n0 + r) * a.H : nullptr;
  uint4 av[RV], bv[RV];
  auto load = [&](int k0) {
#pragma unroll
    for (int i = 0; i < RV; ++i) {
      av[i] = arow ? reinterpret_cast<const uint4 *>(arow + k0 + part * RPART)[i] : make_uint4(0, 0, 0, 0);
      bv[i] = brow ? reinterpret_cast<const uint4 *>(brow + k0 + part * RPART)[i] : make_uint4(0, 0, 0, 0);
    }
  };
  auto store = [&](int buf) {
#pragma unroll
    for (int i = 0; i < RV; ++i) {
      reinterpret_cast<uint4 *>(&sA[buf][r * RLD + part * RPART])[i] = av[i];
      reinterpret_cast<uint4 *>(&sB[buf][r * RLD + part * RPART])[i] = bv[i];
    }
  };
  const int wm = wave >> 1, wn = wave & 1;
  f32x16 acc = {};
  // this block's stages [s0, s1) of the a.rsplit splits of the depth
  // (H % 32 == 0; a ragged last stage reads zeros past H)
  const int S_all = (a.H + RBK - 1) / RBK, per = (S_all + a.rsplit - 1) / a.rsplit;
  const int s0 = blockIdx.z * per, S = min(S_all, s0 + per) - s0;
  auto load_k = [&](int k0) {
    // H % 32 == 0 and RPART is 16 or 32: a thread's part is wholly in or out
    if (k0 + part * RPART < a.H) {
      load(k0);
    } else {
#pragma unroll
      for (int i = 0; i < RV; ++i) av[i] = bv[i] = make_uint4(0, 0, 0, 0);
    }
  };
  load_k(s0 * RBK);
  store(0);
  for (int st = 0; st < S; ++st) {
    if (st + 1 < S) load_k((s0 + st + 1) * RBK);
    __syncthreads();
    const uint16_t *A = &sA[st & 1][(wm * 32 + (lane & 31)) * RLD + (lane >> 5) * 8];
    const uint16_t *Bm = &sB[st & 1][(wn * 32 + (lane & 31)) * RLD + (lane >> 5) * 8];
#pragma unroll
    for (int ks = 0; ks < RBK / 16; ++ks)
      acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(*reinterpret_cast<const bf16x8 *>(A + ks * 16),
                                                    *reinterpret_cast<const bf16x8 *>(Bm + ks * 16), acc, 0, 0, 0);
    if (st + 1 < S) store((st + 1) & 1);
  }
  const int n = n0 + wn * 32 + (lane & 31);
  if (n >= a.E) return;
  // split z writes partial array z; the first carries the bias
  const float bias = (a.router_b && blockIdx.z == 0) ? a.router_b[n] : 0.f;
  float *out = a.logits + (int64_t)blockIdx.z * a.T * a.E;
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    const int m = m0 + wm * 32 + (i / 4) * 8 + (lane >> 5) * 4 + (i % 4);
    if (m < a.T) out[(int64_t)m * a.E + n] = acc[i] + bias;
  }
}

// Gate/up of one tile: the 128 columns are [gate n0..n0+31, up n0..n0+31,
// gate n0+32..n0+63, up n0+32..n0+63], so each lane holds g and u of the same
// (row, column) in acc[mb][0] and acc[mb][1].
template <int BT>
__global__ __launch_bounds__(PThreads) void k_pf_gateup(PrefillArgs a) {
  __shared__ __attribute__((aligned(16))) uint16_t sA[PBM * PLD];
  __shared__ __attribute__((aligned(16))) uint16_t sB[PBN * PLD];
  if ((int)blockIdx.x >= *a.n_tiles) return;
  const PfTile tile = a.tiles[blockIdx.x];
  const bool shared = tile.e < 0;
  const int N = shared ? a.Is : a.I;
  const int n0 = blockIdx.y * 64;
  if (n0 >= N) return;
  const uint16_t *xs = a.use_norm ? a.xn : a.x;
  const int64_t mb_bytes = (BT == 1) ? nvfp4_matrix_bytes(a.I, a.H) : (int64_t)a.I * a.H * 2;
  const uint8_t *Wg = shared ? a.sh_gate : a.w_gate + tile.e * mb_bytes;
  const uint8_t *Wu = shared ? a.sh_up : a.w_up + tile.e * mb_bytes;
  const float Sg = BT == 1 ? (shared ? a.sh_scale[0] : a.w_scale[3 * tile.e]) : 1.f;
  const float Su = BT == 1 ? (shared ? a.sh_scale[1] : a.w_scale[3 * tile.e + 1]) : 1.f;

  const int r = threadIdx.x >> 1, half = threadIdx.x & 1;
  const uint16_t *arow = nullptr;
  if (r < tile.cnt) {
    const int p = tile.p0 + r;
    const int tok = shared ? p - a.P : a.sorted_tok[p];
    arow = xs + (int64_t)tok * a.H;
  }
  // B row r of the tile: column c = r -> matrix (gate/up) and row of it
  const int wn = r >> 6, nb = (r >> 5) & 1, c = r & 31;
  const uint8_t *Bm = nb ? Wu : Wg;
  const int brow = n0 + wn * 32 + c;

  f32x16 acc[2][2] = {};
  for (int k0 = 0; k0 < a.H; k0 += PBK) {
    stage_a(arow, k0 + half * 16, sA + r * PLD + half * 16);
    stage_b<BT>(Bm, N, a.H, brow, k0 + half * 16, sB + r * PLD + half * 16);
    __syncthreads();
    mfma_stage(sA, sB, acc);
    __syncthreads();
  }
  const int Imax = a.I > a.Is ? a.I : a.Is;
#pragma unroll
  for (int mb = 0; mb < 2; ++mb) {
    const int n = n0 + (threadIdx.x >> 6 & 1) * 32 + ((threadIdx.x & 63) & 31);
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int row = acc_row(mb, i);
      if (row < tile.cnt && n < N) {
        const float g = round_bf16(acc[mb][0][i] * Sg);
        const float u = round_bf16(acc[mb][1][i] * Su);
        const float h = silu_mul(g, u);
        a.h_rows[(int64_t)(tile.p0 + row) * Imax + n] = (uint16_t)f32_to_bf16(h);
      }
    }
  }
}

// Down of one tile: h rows x the expert's down matrix -> y rows.
template <int BT>
__global__ __launch_bounds__(PThreads) void k_pf_down(PrefillArgs a) {
  __shared__ __attribute__((aligned(16))) uint16_t sA[PBM * PLD];
  __shared__ __attribute__((aligned(16))) uint16_t sB[PBN * PLD];
  if ((int)blockIdx.x >= *a.n_tiles) return;
  const PfTile tile = a.tiles[blockIdx.x];
  const bool shared = tile.e < 0;
  const int K = shared ? a.Is : a.I;
  const int n0 = blockIdx.y * PBN;
  const int Imax = a.I > a.Is ? a.I : a.Is;
  const int64_t mb_bytes = (BT == 1) ? nvfp4_matrix_bytes(a.H, a.I) : (int64_t)a.H * a.I * 2;
  const uint8_t *Wd = shared ? a.sh_down : a.w_down + tile.e * mb_bytes;
  const float Sd = BT == 1 ? (shared ? a.sh_scale[2] : a.w_scale[3 * tile.e + 2]) : 1.f;

  const int r = threadIdx.x >> 1, half = threadIdx.x & 1;
  const uint16_t *arow = (r < tile.cnt) ? a.h_rows + (int64_t)(tile.p0 + r) * Imax : nullptr;
  f32x16 acc[2][2] = {};
  for (int k0 = 0; k0 < K; k0 += PBK) {
    stage_a(arow, k0 + half * 16, sA + r * PLD + half * 16);
    stage_b<BT>(Wd, a.H, K, n0 + r, k0 + half * 16, sB + r * PLD + half * 16);
    __syncthreads();
    mfma_stage(sA, sB, acc);
    __syncthreads();
  }
#pragma unroll
  for (int mb = 0; mb < 2; ++mb)
#pragma unroll
    for (int nb = 0; nb < 2; ++nb) {
      const int n = n0 + acc_col(nb);
      if (n >= a.H) continue;
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int row = acc_row(mb, i);
        if (row < tile.cnt)
          a.y_rows[(int64_t)(tile.p0 + row) * a.H + n] = (uint16_t)f32_to_bf16(acc[mb][nb][i] * Sd);
      }
    }
}

// ---------------------------------------------------------------------------
// NVFP4 grouped GEMM (gate/up and down).  A block of 8 waves (two per
// SIMD, so one wave's dequantisation overlaps the other's MFMAs) computes
// 128 rows of one tile against 512 weight rows; each wave owns 64 weight
// rows (two 32-row MFMA column blocks) across all 128 tile rows (four
// 32-row blocks): 4 x 2 accumulator tiles of 32x32 FP32.
//   A (activation rows): global -> registers -> LDS, 128 K per stage,
//     double-buffered, one barrier per stage; the next stage's loads are
//     in flight during the current stage's MFMAs.
//   B (weights): global -> registers directly (one stage ahead),
//     dequantised in registers.  Within a 128-K stage, lane half
//     h = lane/32 holds K elements [h*64, h*64 + 64) of its weight row
//     (32 contiguous bytes), and MFMA step s uses elements h*64 + s*8 .. +8;
//     the A fragments are read from LDS at the same K positions, so every K
//     element meets its partner.
//   A 32-row block of the tile that lies wholly past the tile's rows is
//     skipped (no MFMA issued for it).
//   The results leave through LDS as whole 16-byte row pieces.
// ---------------------------------------------------------------------------

constexpr int GWaves = 8;
constexpr int GThreads = GWaves * kWave;
constexpr int GBM = kPrefillTileRows;   // 128 tile rows
constexpr int GBK = 128;                // K per stage
constexpr int GLDA = GBK + 8;           // LDS row stride, BF16 elements (272 B)
constexpr int GBN = GWaves * 64;        // weight rows per block
constexpr int GChunk = 8;               // consecutive work items per XCD chunk
constexpr int kPfMidWaves = 4;          // waves per block on 32-row tiles (256 weight rows)

// Raw NVFP4 data of one lane for one stage and one weight row: 64 FP4
// (8 dwords) and the 4 block scales (two 16-bit scale pairs).
struct BRaw {
  uint4 q0, q1;
  uint32_t s0, s1;
};

// The lane's two 32-element chunks (c0 + 2h, c0 + 2h + 1) of weight row n
// of a K-column matrix: nibbles from the row, the scale pair of each chunk
// from the scale tile (n/8, chunk).  Chunks past K (and rows that do not
// exist, ok == false) read as zero.
__device__ __forceinline__ void load_b_stage(const uint8_t *nib_row, const uint8_t *scale_base, int n, int K,
                                             int k0, int h, bool ok, BRaw &r) {
  r.q0 = r.q1 = make_uint4(0, 0, 0, 0);
  r.s0 = r.s1 = 0;
  if (!ok) return;
  const int c = (k0 >> 5) + 2 * h;
  const int C = K >> 5;
  const int64_t st = ((int64_t)(n >> 3) * C) * 16 + (n & 7) * 2;
  if (c < C) {
    r.q0 = *reinterpret_cast<const uint4 *>(nib_row + c * 16);
    r.s0 = *reinterpret_cast<const uint16_t *>(scale_base + st + (int64_t)c * 16);
  }
  if (c + 1 < C) {
    r.q1 = *reinterpret_cast<const uint4 *>(nib_row + (c + 1) * 16);
    r.s1 = *reinterpret_cast<const uint16_t *>(scale_base + st + (int64_t)(c + 1) * 16);
  }
}

// One wave's MFMAs for one stage: 8 K-steps x AMB 32-row blocks x 2 weight
// blocks.  AMB is a compile-time count so the step loop is straight-line
// code.  Software-pipelined: the weights of step s + 1 are dequantised and
// its A fragments read from LDS before the MFMAs of step s are issued, so
// the vector work of one step overlaps the matrix work of the previous.
template <int AMB>
__device__ __forceinline__ void gemm_stage(const uint16_t *sA, const BRaw (&b)[2], f32x16 (&acc)[4][2]) {
  const int lane = threadIdx.x & 63, h = lane >> 5, l32 = lane & 31;
  float sc[2][4];
#pragma unroll
  for (int nb = 0; nb < 2; ++nb) {
    sc[nb][0] = e4m3_to_f32(b[nb].s0 & 0xffu);
    sc[nb][1] = e4m3_to_f32(b[nb].s0 >> 8);
    sc[nb][2] = e4m3_to_f32(b[nb].s1 & 0xffu);
    sc[nb][3] = e4m3_to_f32(b[nb].s1 >> 8);
  }
  auto dq_step = [&](int s, int nb) {
    const uint4 &q = s < 4 ? b[nb].q0 : b[nb].q1;
    const uint32_t w = (s & 3) == 0 ? q.x : (s & 3) == 1 ? q.y : (s & 3) == 2 ? q.z : q.w;
    return dq8(w, sc[nb][s >> 1]);
  };
  const uint16_t *arow = sA + l32 * GLDA + h * 64;
  bf16x8 af[2][AMB], bf[2][2];
#pragma unroll
  for (int mb = 0; mb < AMB; ++mb) af[0][mb] = *reinterpret_cast<const bf16x8 *>(arow + mb * 32 * GLDA);
  bf[0][0] = dq_step(0, 0);
  bf[0][1] = dq_step(0, 1);
#pragma unroll
  for (int s = 0; s < 8; ++s) {
    if (s + 1 < 8) {
#pragma unroll
      for (int mb = 0; mb < AMB; ++mb)
        af[(s + 1) & 1][mb] = *reinterpret_cast<const bf16x8 *>(arow + mb * 32 * GLDA + (s + 1) * 8);
      bf[(s + 1) & 1][0] = dq_step(s + 1, 0);
      bf[(s + 1) & 1][1] = dq_step(s + 1, 1);
    }
#pragma unroll
    for (int mb = 0; mb < AMB; ++mb) {
      acc[mb][0] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[s & 1][mb], bf[s & 1][0], acc[mb][0], 0, 0, 0);
      acc[mb][1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[s & 1][mb], bf[s & 1][1], acc[mb][1], 0, 0, 0);
    }
  }
}

// K loop of one block: A stages through LDS (double-buffered), B stages
// through registers (one stage ahead).  AMAX: 32-row blocks the tile rows
// can fill (4, or 1 for 32-row tiles); thread (ar, ap) loads NV 16-byte
// pieces of tile row ar per stage.
template <int AMB, int AMAX, int NV>
__device__ __forceinline__ void gemm_mainloop(uint16_t (*sA)[AMAX * 32 * GLDA], const uint16_t *arow, int ar, int ap,
                                              const uint8_t *const (&nib)[2], const uint8_t *const (&scl)[2],
                                              const int (&nrow)[2], const bool (&bok)[2], int K,
                                              f32x16 (&acc)[4][2]) {
  const int h = (threadIdx.x & 63) >> 5;
  const int S = (K + GBK - 1) / GBK;
  uint4 av[NV];
  auto load_a = [&](int k0) {
#pragma unroll
    for (int i = 0; i < NV; ++i) av[i] = make_uint4(0, 0, 0, 0);
    if (arow && k0 + ap * NV * 8 < K) {
      const uint4 *p = reinterpret_cast<const uint4 *>(arow + k0 + ap * NV * 8);
#pragma unroll
      for (int i = 0; i < NV; ++i) av[i] = p[i];
    }
  };
  auto store_a = [&](int buf) {
    uint4 *d = reinterpret_cast<uint4 *>(&sA[buf][ar * GLDA + ap * NV * 8]);
#pragma unroll
    for (int i = 0; i < NV; ++i) d[i] = av[i];
  };
  BRaw bcur[2], bnext[2];
  load_a(0);
#pragma unroll
  for (int j = 0; j < 2; ++j) load_b_stage(nib[j], scl[j], nrow[j], K, 0, h, bok[j], bnext[j]);
  store_a(0);
  for (int st = 0; st < S; ++st) {
#pragma unroll
    for (int j = 0; j < 2; ++j) bcur[j] = bnext[j];
    if (st + 1 < S) {
      load_a((st + 1) * GBK);
#pragma unroll
      for (int j = 0; j < 2; ++j) load_b_stage(nib[j], scl[j], nrow[j], K, (st + 1) * GBK, h, bok[j], bnext[j]);
    }
    __syncthreads();
    gemm_stage<AMB>(sA[st & 1], bcur, acc);
    if (st + 1 < S) store_a((st + 1) & 1);
  }
}

// K loop of a 32-row tile (one 32-row block).  Same stages as
// gemm_mainloop, but every load is a branch-free buffer load (a lane or
// stage with nothing to load reads zeros past the range's end) and the two
// weight buffers take turns (b0 current while b1 fills, then the reverse)
// instead of being copied: no exec-mask branches or register moves in the
// loop, which matters where one weight fragment feeds a single 32-row block
// and the loop's VALU work is mostly dequantisation.
//   a_off: byte offset of this thread's A piece in its row (kBufNone for
//     rows past the tile); nib_off / scl_off: byte offsets of the lane's
//     first chunk and its scale pair at K = 0 (kBufNone for rows past N).
template <int NV>
__device__ __forceinline__ void gemm_mainloop_32(uint16_t (*sA)[32 * GLDA], __amdgpu_buffer_rsrc_t ar_rsrc,
                                                 uint32_t a_off, int ar, int ap, const __amdgpu_buffer_rsrc_t (&br)[2],
                                                 const uint32_t (&nib_off)[2], const uint32_t (&scl_off)[2], int K,
                                                 f32x16 (&acc)[4][2]) {
  const int h = (threadIdx.x & 63) >> 5;
  const int S = (K + GBK - 1) / GBK, C = K >> 5;
  uint4 av[NV];
  BRaw b0[2], b1[2];
  auto load_a = [&](int st) {
    const int k0 = st * GBK;
    const bool ok = st < S && k0 + ap * NV * 8 < K;
#pragma unroll
    for (int i = 0; i < NV; ++i) av[i] = buf_load16(ar_rsrc, buf_off(ok, a_off + (uint32_t)k0 * 2 + i * 16));
  };
  auto store_a = [&](int buf) {
    uint4 *d = reinterpret_cast<uint4 *>(&sA[buf][ar * GLDA + ap * NV * 8]);
#pragma unroll
    for (int i = 0; i < NV; ++i) d[i] = av[i];
  };
  auto load_b = [&](int st, BRaw (&r)[2]) {
    const int k0 = st * GBK, c = (k0 >> 5) + 2 * h;
    const bool ok0 = st < S && c < C, ok1 = st < S && c + 1 < C;
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const uint32_t nb = nib_off[j] + (uint32_t)k0 / 2, sb = scl_off[j] + (uint32_t)k0 / 2;
      r[j].q0 = buf_load16(br[j], buf_off(ok0, nb));
      r[j].q1 = buf_load16(br[j], buf_off(ok1, nb + 16));
      r[j].s0 = buf_load2(br[j], buf_off(ok0, sb));
      r[j].s1 = buf_load2(br[j], buf_off(ok1, sb + 16));
    }
  };
  // stage st: the operands of st + 1 go out, stage st computes, and the A
  // rows of st + 1 move to LDS
  auto step = [&](int st, const BRaw (&cur)[2], BRaw (&fill)[2]) {
    load_a(st + 1);
    load_b(st + 1, fill);
    __syncthreads();
    gemm_stage<1>(sA[st & 1], cur, acc);
    store_a((st + 1) & 1);
  };
  load_a(0);
  load_b(0, b0);
  store_a(0);
  for (int st = 0; st < S; st += 2) {
    step(st, b0, b1);
    if (st + 1 >= S) break;
    step(st + 1, b1, b0);
  }
}

// The (tile, n-block) item of grid slot `slot`: items are spread over the 8
// XCDs in chunks of GChunk consecutive items (neighbouring items share A
// rows or the expert's weights in that XCD's L2).
__device__ __forceinline__ int gemm_item(int slot) {
  const int xcd = slot & 7, q = slot >> 3;
  return ((q / GChunk) * 8 + xcd) * GChunk + (q % GChunk);
}

// MODE 0: gate/up (K = H) -> h rows; MODE 1: down (K = I or Is) -> y rows.
// WAVES waves per block, 64 weight rows each.  AMAX = 1: tiles of at most
// 32 rows (calls of 49..1024 tokens): a quarter of the A stage and the
// accumulators, so that three blocks of 4 waves share a compute unit (at
// most 168 registers) and hide each other's load waits; the small blocks
// also give the few experts of such calls more items to spread over.
template <int MODE, int AMAX, int WAVES>
__global__ __launch_bounds__(WAVES * kWave, AMAX == 1 ? 12 / WAVES : 8 / WAVES) void k_pf_gemm_fp4(PrefillArgs a,
                                                                                                  int nblk) {
  constexpr int NT = WAVES * kWave;  // threads
  constexpr int BN = WAVES * 64;     // weight rows per block
  constexpr int NV = AMAX * 32 * GBK / (8 * NT);  // A: 16-byte pieces per thread and stage
  static_assert(NV >= 1 && NV * 8 * NT == AMAX * 32 * GBK, "the threads cover the A stage");
  __shared__ __attribute__((aligned(16))) uint16_t sA[2][AMAX * 32 * GLDA];
  const int w = gemm_item(blockIdx.x);
  if (w >= *a.n_tiles * nblk) return;
  const PfTile tile = a.tiles[w / nblk];
  const int nb_i = w % nblk;
  const bool shared = tile.e < 0;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, h = lane >> 5, l32 = lane & 31;
  const int Imax = a.I > a.Is ? a.I : a.Is;
  const int Iw = shared ? a.Is : a.I;
  const int K = MODE == 0 ? a.H : Iw;
  const int N = MODE == 0 ? Iw : a.H;
  const int64_t mat_bytes = nvfp4_matrix_bytes(MODE == 0 ? a.I : a.H, MODE == 0 ? a.H : a.I);

  // A rows: thread (ar, ap) loads AMAX * 8 K-elements of tile row ar per stage.
  constexpr int PARTS = NT / (AMAX * 32);  // threads per tile row in the A loads
  const int ar = tid / PARTS, ap = tid % PARTS;
  const uint16_t *arow = nullptr;
  if (ar < tile.cnt) {
    const int p = tile.p0 + ar;
    if (MODE == 0) {
      const uint16_t *xs = a.use_norm ? a.xn : a.x;
      arow = xs + (int64_t)(shared ? p - a.P : a.sorted_tok[p]) * a.H;
    } else {
      arow = a.h_rows + (int64_t)p * Imax;
    }
  }
  // This lane's two weight rows.  Gate/up: a wave's first 32 weight rows
  // are gate rows and its next 32 the up rows of the same 32 output columns.
  const uint8_t *mats[2];
  int nrow[2];
  float tscale[2];
  if (MODE == 0) {
    const int hc = nb_i * (BN / 2) + wave * 32 + l32;
    mats[0] = shared ? a.sh_gate : a.w_gate + tile.e * mat_bytes;
    mats[1] = shared ? a.sh_up : a.w_up + tile.e * mat_bytes;
    nrow[0] = nrow[1] = hc;
    tscale[0] = shared ? a.sh_scale[0] : a.w_scale[3 * tile.e];
    tscale[1] = shared ? a.sh_scale[1] : a.w_scale[3 * tile.e + 1];
  } else {
    mats[0] = mats[1] = shared ? a.sh_down : a.w_down + tile.e * mat_bytes;
    nrow[0] = nb_i * BN + wave * 64 + l32;
    nrow[1] = nrow[0] + 32;
    tscale[0] = tscale[1] = shared ? a.sh_scale[2] : a.w_scale[3 * tile.e + 2];
  }
  const uint8_t *nib[2], *scl[2];
  bool bok[2];
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    bok[j] = nrow[j] < N;
    nib[j] = mats[j] + (int64_t)nrow[j] * (K / 2);
    scl[j] = mats[j] + (int64_t)N * (K / 2);
  }
  const int active_mb = (tile.cnt + 31) >> 5;
  f32x16 acc[4][2] = {};
  const uint8_t *const nibc[2] = {nib[0], nib[1]}, *const sclc[2] = {scl[0], scl[1]};
  if constexpr (AMAX == 1) {
    // 32-row tiles: the operands as buffer ranges and offsets when both fit
    // below 2 GiB (any shape of the model's size; larger ones take the
    // pointer loop)
    const uint16_t *abase = MODE == 0 ? (a.use_norm ? a.xn : a.x) : a.h_rows;
    const int64_t arow_elems = MODE == 0 ? a.H : Imax;
    const int64_t abytes = (MODE == 0 ? (int64_t)a.T : (int64_t)(a.P + a.T)) * arow_elems * 2;
    const int64_t wbytes = nvfp4_matrix_bytes(N, K);
    if (abytes < (int64_t)kBufNone && wbytes < (int64_t)kBufNone) {
      uint32_t a_off = kBufNone;
      if (ar < tile.cnt) {
        const int p = tile.p0 + ar;
        const int64_t row = MODE == 0 ? (shared ? p - a.P : a.sorted_tok[p]) : p;
        a_off = (uint32_t)(row * arow_elems * 2) + (uint32_t)(ap * NV * 16);
      }
      const __amdgpu_buffer_rsrc_t br[2] = {buf_rsrc(mats[0], wbytes), buf_rsrc(mats[1], wbytes)};
      uint32_t nib_off[2], scl_off[2];
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        nib_off[j] = bok[j] ? (uint32_t)(nrow[j] * (K / 2) + 32 * h) : kBufNone;
        scl_off[j] = bok[j] ? (uint32_t)((int64_t)N * (K / 2) + (int64_t)(nrow[j] >> 3) * (K >> 5) * 16 +
                                         (nrow[j] & 7) * 2 + 32 * h)
                            : kBufNone;
      }
      gemm_mainloop_32<NV>(sA, buf_rsrc(abase, abytes), a_off, ar, ap, br, nib_off, scl_off, K, acc);
    } else {
      gemm_mainloop<1, AMAX, NV>(sA, arow, ar, ap, nibc, sclc, nrow, bok, K, acc);
    }
  } else {
    switch (active_mb) {
      case 4: gemm_mainloop<4, AMAX, NV>(sA, arow, ar, ap, nibc, sclc, nrow, bok, K, acc); break;
      case 3: gemm_mainloop<3, AMAX, NV>(sA, arow, ar, ap, nibc, sclc, nrow, bok, K, acc); break;
      case 2: gemm_mainloop<2, AMAX, NV>(sA, arow, ar, ap, nibc, sclc, nrow, bok, K, acc); break;
      default: gemm_mainloop<1, AMAX, NV>(sA, arow, ar, ap, nibc, sclc, nrow, bok, K, acc); break;
    }
  }

  // Epilogue.  Value i of acc[mb][j] is tile row mb*32 + (i/4)*8 + h*4 + i%4
  // and weight row nrow[j].  The BF16 results of RPP rows at a time go to
  // LDS (the A buffers, free now) and leave as whole 16-byte row pieces.
  constexpr int OC = MODE == 0 ? BN / 2 : BN;  // output columns of the block
  constexpr int OS = OC + 8;                   // staging row stride (elements)
  // rows per pass: as many whole 8-row groups as the A buffers hold, dividing the tile rows
  constexpr int RPP_FIT = (int)sizeof(sA) / (OS * 2) / 8 * 8;
  constexpr int RPP = RPP_FIT >= AMAX * 32 ? AMAX * 32 : RPP_FIT >= 64 ? 64 : RPP_FIT >= 32 ? 32 : 16;
  static_assert(RPP * OS * 2 <= (int)sizeof(sA), "a staging pass fits the A buffers");
  static_assert(RPP % 8 == 0 && (AMAX * 32) % RPP == 0, "passes split the rows at 8-row groups");
  uint16_t *const stg = &sA[0][0];
  const int col0 = nb_i * OC;
  uint16_t *out = MODE == 0 ? a.h_rows : a.y_rows;
  const int64_t ostride = MODE == 0 ? Imax : a.H;
  constexpr int CPR = OC / 8;  // 16-byte pieces per row
#pragma unroll
  for (int pass = 0; pass < AMAX * 32 / RPP; ++pass) {
    if (pass * RPP >= tile.cnt) break;
    __syncthreads();  // the A buffers (or the previous pass) are free
#pragma unroll
    for (int mb = 0; mb < AMAX; ++mb) {
      if (mb >= active_mb) continue;
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        // the 8-row group of value i lies wholly in one pass (RPP is a multiple of 8)
        if ((mb * 32 + (i >> 2) * 8) / RPP != pass) continue;
        const int r = mb * 32 - pass * RPP + (i >> 2) * 8 + h * 4 + (i & 3);
        if (MODE == 0) {
          const float g = round_bf16(acc[mb][0][i] * tscale[0]);
          const float u = round_bf16(acc[mb][1][i] * tscale[1]);
          stg[r * OS + wave * 32 + l32] = (uint16_t)f32_to_bf16(silu_mul(g, u));
        } else {
          stg[r * OS + wave * 64 + l32] = (uint16_t)f32_to_bf16(acc[mb][0][i] * tscale[0]);
          stg[r * OS + wave * 64 + 32 + l32] = (uint16_t)f32_to_bf16(acc[mb][1][i] * tscale[1]);
        }
      }
    }
    __syncthreads();
    const int rows = min(RPP, tile.cnt - pass * RPP);
    for (int qi = tid; qi < rows * CPR; qi += NT) {
      const int r = qi / CPR, c8 = qi % CPR;
      const int col = col0 + c8 * 8;
      if (col >= N) continue;
      const uint4 v = *reinterpret_cast<const uint4 *>(stg + r * OS + c8 * 8);
      uint4 *dst = reinterpret_cast<uint4 *>(out + (int64_t)(tile.p0 + pass * RPP + r) * ostride + col);
      if (MODE == 1) {
        // y rows are read once, by the combine kernel: stream them past the L2
        __builtin_nontemporal_store(v.x, &dst->x);
        __builtin_nontemporal_store(v.y, &dst->y);
        __builtin_nontemporal_store(v.z, &dst->z);
        __builtin_nontemporal_store(v.w, &dst->w);
      } else {
        *dst = v;
      }
    }
  }
}

constexpr int64_t kPfSmallBlocks = 512;  // two rounds of one block per compute unit

// ---------------------------------------------------------------------------
// Small-tile prefill (NVFP4, up to kPrefillSmallMaxTokens tokens): tiles of
// at most 16 rows, so that an expert's few rows do not fill a 128-row tile
// with padding and one block does not stream a quarter of an expert's
// weights alone.  Each (tile, row group) item runs on one block as in the
// small-batch decode kernels: the tile's rows are the 16 token columns of
// v_mfma_f32_16x16x32_bf16 tiles, K is split over the 8 waves.
// ---------------------------------------------------------------------------

// Gate/up: item (tile, 64 h columns); h rows as the large-tile kernel
// writes them.
__global__ __launch_bounds__(kMmWaves *kWave) void k_pf_small_gateup(PrefillArgs a) {
  __shared__ float s_red[kMmWaves][32][kWave];
  const int n_tiles = *a.n_tiles;
  const int Imax = a.I > a.Is ? a.I : a.Is;
  const int groups = (Imax + 63) / 64;
  const int64_t mb = nvfp4_matrix_bytes(a.I, a.H);
  const uint16_t *xs = a.use_norm ? a.xn : a.x;
  const int col = threadIdx.x & 15;
  for (int item = blockIdx.x; item < n_tiles * groups; item += gridDim.x) {
    const PfTile tile = a.tiles[item / groups];
    const int row0 = (item % groups) * 64;
    const bool shared = tile.e < 0;
    const int N = shared ? a.Is : a.I;
    if (row0 >= N) continue;  // block-uniform
    const uint8_t *Wg = shared ? a.sh_gate : a.w_gate + tile.e * mb;
    const uint8_t *Wu = shared ? a.sh_up : a.w_up + tile.e * mb;
    const float Sg = shared ? a.sh_scale[0] : a.w_scale[3 * tile.e + 0];
    const float Su = shared ? a.sh_scale[1] : a.w_scale[3 * tile.e + 1];
    int xrow = -1;  // this lane's token row
    if (col < tile.cnt) xrow = shared ? tile.p0 + col - a.P : a.sorted_tok[tile.p0 + col];
    mm_rows<4, true>(a.H, xs, a.T, a.H, xrow, Wg, Wu, Sg, Su, N, row0, (1u << tile.cnt) - 1u, s_red,
                     [&](int t, int n, uint32_t v) { a.h_rows[(int64_t)(tile.p0 + t) * Imax + n] = (uint16_t)v; });
  }
}

// Down: item (tile, 128 output columns); y rows as the large-tile kernel
// writes them, for the combine.
__global__ __launch_bounds__(kMmWaves *kWave) void k_pf_small_down(PrefillArgs a) {
  __shared__ float s_red[kMmWaves][32][kWave];
  const int n_tiles = *a.n_tiles;
  const int Imax = a.I > a.Is ? a.I : a.Is;
  const int groups = (a.H + 127) / 128;
  const int64_t mb = nvfp4_matrix_bytes(a.H, a.I);
  const int col = threadIdx.x & 15;
  for (int item = blockIdx.x; item < n_tiles * groups; item += gridDim.x) {
    const PfTile tile = a.tiles[item / groups];
    const int row0 = (item % groups) * 128;
    const bool shared = tile.e < 0;
    const int K = shared ? a.Is : a.I;
    const uint8_t *Wd = shared ? a.sh_down : a.w_down + tile.e * mb;
    const float Sd = shared ? a.sh_scale[2] : a.w_scale[3 * tile.e + 2];
    const int hrow = col < tile.cnt ? tile.p0 + col : -1;
    mm_rows<8, false>(K, a.h_rows, a.P + a.T, Imax, hrow, Wd, Wd, Sd, Sd, a.H, row0, (1u << tile.cnt) - 1u, s_red,
                      [&](int t, int n, uint32_t v) { a.y_rows[(int64_t)(tile.p0 + t) * a.H + n] = (uint16_t)v; });
  }
}

// out[t] = BF16(sum_j w_j y_row(t, j) + y_shared(t)) (+ residual); 8 columns
// per thread, one block per token.
__global__ __launch_bounds__(PThreads) void k_pf_combine(PrefillArgs a) {
  const int t = blockIdx.x;
  // the token's pair rows and weights first, then every row's piece in
  // flight together (selections past k read the first row and add nothing)
  // (a layer without routed experts has no pairs: row 0 stands in)
  int prow[kMaxTopK];
  float pw[kMaxTopK];
#pragma unroll
  for (int j = 0; j < kMaxTopK; ++j) prow[j] = 0, pw[j] = 0.f;
  if (a.k > 0) {
#pragma unroll
    for (int j = 0; j < kMaxTopK; ++j) {
      const int jj = j < a.k ? j : 0;
      prow[j] = a.pair_pos[(int64_t)t * a.k + jj];
      pw[j] = a.out_w[(int64_t)t * a.k + jj];
    }
  }
  for (int c = threadIdx.x * 8; c < a.H; c += PThreads * 8) {
    float acc[8] = {0, 0, 0, 0, 0, 0, 0, 0};
    uint4 yv[kMaxTopK];
#pragma unroll
    for (int j = 0; j < kMaxTopK; ++j) yv[j] = *reinterpret_cast<const uint4 *>(a.y_rows + (int64_t)prow[j] * a.H + c);
#pragma unroll
    for (int j = 0; j < kMaxTopK; ++j) {
      if (j >= a.k) break;
      const float w = pw[j];
      const uint32_t q[4] = {yv[j].x, yv[j].y, yv[j].z, yv[j].w};
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        acc[2 * i] = fmaf(w, bf16_to_f32(q[i] & 0xffffu), acc[2 * i]);
        acc[2 * i + 1] = fmaf(w, bf16_to_f32(q[i] >> 16), acc[2 * i + 1]);
      }
    }
    if (a.Is > 0) {
      const uint4 v = *reinterpret_cast<const uint4 *>(a.y_rows + (int64_t)(a.P + t) * a.H + c);
      const uint32_t q[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        acc[2 * i] += bf16_to_f32(q[i] & 0xffffu);
        acc[2 * i + 1] += bf16_to_f32(q[i] >> 16);
      }
    }
    uint32_t o[4];
    // the layer input only when it is added back
    const uint4 xv = a.residual ? *reinterpret_cast<const uint4 *>(a.x + (int64_t)t * a.H + c) : make_uint4(0, 0, 0, 0);
    const uint32_t xq[4] = {xv.x, xv.y, xv.z, xv.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      float lo = round_bf16(acc[2 * i]), hi = round_bf16(acc[2 * i + 1]);
      if (a.residual) {
        lo += bf16_to_f32(xq[i] & 0xffffu);
        hi += bf16_to_f32(xq[i] >> 16);
      }
      o[i] = f32_to_bf16(lo) | (f32_to_bf16(hi) << 16);
    }
    *reinterpret_cast<uint4 *>(a.y + (int64_t)t * a.H + c) = make_uint4(o[0], o[1], o[2], o[3]);
  }
}

// ---------------------------------------------------------------------------
// Host launcher
// ---------------------------------------------------------------------------

template <int BT>
static hipError_t launch_prefill_t(const PrefillArgs &args, hipStream_t s) {
  hipError_t e;
#define MOE_CK_LAUNCH() \
  if ((e = hipGetLastError()) != hipSuccess) return e
  // Small-tile calls with routed experts run the decode path's router (one
  // row of blocks per token, the pre-norm in each block): its 64 blocks per
  // token spread the router weights over the GPU, where the GEMM router's
  // 64 x 64 tiles would put them on E/64 blocks.  It writes one [T][E]
  // array of logits.
  const bool token_router =
      BT == 1 && args.tile_rows == kPrefillSmallRows && args.E > 0 && args.H <= kRouterTokenMaxHidden;
  PrefillArgs a = args;
  if (token_router) a.rsplit = 1;
  if (a.use_norm && !token_router) {
    hipLaunchKernelGGL(k_pf_norm, dim3((a.T + 3) / 4), dim3(PThreads), 0, s, a);
    MOE_CK_LAUNCH();
  }
  if (a.E > 0) {
    if (token_router) {
      DecodeArgs d;
      memset(&d, 0, sizeof(d));
      d.H = a.H;
      d.E = a.E;
      d.B = a.T;
      d.use_norm = a.use_norm;
      d.eps = a.eps;
      d.x = a.x;
      d.router_w = a.router_w;
      d.router_b = a.router_b;
      d.norm_gain = a.norm_gain;
      d.ws.xn = a.xn;
      d.ws.logits = a.logits;
      // the expert counts the top-k kernel accumulates, and the cursors the
      // placement kernel advances, start at zero
      d.zero0 = a.counts;
      d.zero1 = a.cursors;
      d.zero_n = a.E + 1;
      if ((e = launch_router_tokens(d, s)) != hipSuccess) return e;
    } else {
      hipLaunchKernelGGL(k_pf_router, dim3((a.T + RBM - 1) / RBM, (a.E + RBN - 1) / RBN, a.rsplit), dim3(PThreads), 0, s,
                         a);
      MOE_CK_LAUNCH();
    }
    const int waves = (a.T + kPfTokensPerWave - 1) / kPfTokensPerWave;
    // calls of up to 2048 tokens: blocks of 4 waves spread them over more
    // compute units
    if (a.T <= 2048) {
      const dim3 tg((waves + 3) / 4), tb(4 * kWave);
      if (a.E <= 4 * kWave) hipLaunchKernelGGL((k_pf_topk<4, 4>), tg, tb, 0, s, a);
      else hipLaunchKernelGGL((k_pf_topk<kMaxExperts / kWave, 4>), tg, tb, 0, s, a);
    } else {
      const dim3 tg((waves + kPfTopkWaves - 1) / kPfTopkWaves), tb(kPfTopkWaves * kWave);
      if (a.E <= 4 * kWave) hipLaunchKernelGGL((k_pf_topk<4, kPfTopkWaves>), tg, tb, 0, s, a);
      else hipLaunchKernelGGL((k_pf_topk<kMaxExperts / kWave, kPfTopkWaves>), tg, tb, 0, s, a);
    }
    MOE_CK_LAUNCH();
  }
  {
    // one block at least: it writes the tile list (the shared expert's tiles
    // even without routed experts)
    const int64_t pairs = (int64_t)a.T * a.k;
    const int64_t want = (pairs + 2 * PThreads - 1) / (2 * PThreads);
    const int blocks = (int)(want < 1 ? 1 : want > kPlaceMaxBlocks ? kPlaceMaxBlocks : want);
    hipLaunchKernelGGL(k_pf_place, dim3(blocks), dim3(PThreads), 0, s, a);
    MOE_CK_LAUNCH();
  }
  const int nmax = a.I > a.Is ? a.I : a.Is;
  if (BT == 1 && a.tile_rows == kPrefillSmallRows) {
    // blocks: every item of the largest tile count, at most kPfSmallBlocks
    const int64_t gu = (int64_t)a.max_tiles * ((nmax + 63) / 64), dn = (int64_t)a.max_tiles * ((a.H + 127) / 128);
    hipLaunchKernelGGL(k_pf_small_gateup, dim3((unsigned)(gu < kPfSmallBlocks ? gu : kPfSmallBlocks)),
                       dim3(kMmWaves * kWave), 0, s, a);
    MOE_CK_LAUNCH();
    hipLaunchKernelGGL(k_pf_small_down, dim3((unsigned)(dn < kPfSmallBlocks ? dn : kPfSmallBlocks)),
                       dim3(kMmWaves * kWave), 0, s, a);
    MOE_CK_LAUNCH();
  } else if (BT == 1) {
    // grid: every (tile, n-block) item, rounded up to whole XCD chunks
    const int bn = a.tile_rows <= 32 ? kPfMidWaves * 64 : GBN;  // weight rows per block
    const int nb_gu = (nmax + bn / 2 - 1) / (bn / 2), nb_dn = (a.H + bn - 1) / bn;
    const int64_t round = 8 * GChunk;
    const int64_t g_gu = ((int64_t)a.max_tiles * nb_gu + round - 1) / round * round;
    const int64_t g_dn = ((int64_t)a.max_tiles * nb_dn + round - 1) / round * round;
    if (a.tile_rows <= 32) {
      hipLaunchKernelGGL((k_pf_gemm_fp4<0, 1, kPfMidWaves>), dim3((unsigned)g_gu), dim3(kPfMidWaves * kWave), 0, s,
                         a, nb_gu);
      MOE_CK_LAUNCH();
      hipLaunchKernelGGL((k_pf_gemm_fp4<1, 1, kPfMidWaves>), dim3((unsigned)g_dn), dim3(kPfMidWaves * kWave), 0, s,
                         a, nb_dn);
      MOE_CK_LAUNCH();
    } else {
      hipLaunchKernelGGL((k_pf_gemm_fp4<0, 4, GWaves>), dim3((unsigned)g_gu), dim3(GThreads), 0, s, a, nb_gu);
      MOE_CK_LAUNCH();
      hipLaunchKernelGGL((k_pf_gemm_fp4<1, 4, GWaves>), dim3((unsigned)g_dn), dim3(GThreads), 0, s, a, nb_dn);
      MOE_CK_LAUNCH();
    }
  } else {
    hipLaunchKernelGGL(k_pf_gateup<BT>, dim3(a.max_tiles, (nmax + 63) / 64), dim3(PThreads), 0, s, a);
    MOE_CK_LAUNCH();
    hipLaunchKernelGGL(k_pf_down<BT>, dim3(a.max_tiles, (a.H + PBN - 1) / PBN), dim3(PThreads), 0, s, a);
    MOE_CK_LAUNCH();
  }
  hipLaunchKernelGGL(k_pf_combine, dim3(a.T), dim3(PThreads), 0, s, a);
  MOE_CK_LAUNCH();
#undef MOE_CK_LAUNCH
  return hipSuccess;
}

hipError_t launch_prefill(const PrefillArgs &a, hipStream_t s) {
  return a.wtype == 1 ? launch_prefill_t<1>(a, s) : launch_prefill_t<0>(a, s);
}

}  // namespace moe
