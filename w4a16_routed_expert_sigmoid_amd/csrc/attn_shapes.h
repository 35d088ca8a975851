// Shape arithmetic of the decode attention, in plain C++ with no HIP
// dependency (the kernels include it through attn.h, the host-only
// validation unit directly): tile and group limits, the split of a
// token's context into chunks, and the MFMA lane order of the KV-cache
// tiles.  Every function is constexpr, so device code can call it too.
#pragma once

#include <stddef.h>
#include <stdint.h>

#include "shapes.h"

namespace moe {

// Decode attention: head_dim 128, tiles of 32 positions, one MFMA column
// per query head of a GQA group (at most 16), blocks of 8 waves.
constexpr int kAttnD = 128;
constexpr int kAttnTile = 32;
constexpr int kAttnMaxGroup = 16;
constexpr int kAttnWaves = 8;
constexpr int kAttnMaxBatch = 256;
constexpr int kAttnTargetBlocks = 256;  // one block per CU of the chip
constexpr int64_t kAttnMaxPos = (int64_t)1 << 40;  // positions 0 .. 2^40 - 1
constexpr int32_t kAttnMaxSlots = 1 << 24;         // cache positions per token row

// KV-cache tiles: 32 positions of one (token row, KV head), 4096 BF16 keys
// then, in the value cache, 4096 BF16 values, each stored in the lane order
// of the matrix-core operands that read them, so that every 16-byte lane
// load of the decode kernel is part of one contiguous 1 KiB wave load.
// Position offset o (0..31) in its tile, dimension d (0..127):
//   keys:   operand (half tt, k-step s) of the score product; lane 16 g + r
//           holds position 8 (r / 4) + 4 tt + r % 4, dims 8 (4 s + g) .. + 8
//   values: operand dt of the value product; lane 16 g + r holds dim
//           16 dt + r, positions 8 g .. 8 g + 7
constexpr int kAttnTileElems = kAttnTile * kAttnD;
constexpr int attn_k_index(int o, int d) {
  return ((((o >> 2) & 1) * 4 + (d >> 5)) * 64 + ((d >> 3) & 3) * 16 + (((o >> 3) << 2) | (o & 3))) * 8 + (d & 7);
}
constexpr int attn_v_index(int o, int d) { return ((d >> 4) * 64 + (o >> 3) * 16 + (d & 15)) * 8 + (o & 7); }

// FP32 partial of one (token, KV head, chunk): the G heads' 128 weighted
// value sums, then their running maxima and sums, padded to 16 bytes.
constexpr int64_t attn_part_floats(int64_t G) { return G * kAttnD + (2 * G + 3) / 4 * 4; }

// Split of one token's attended tiles into chunks, one block per chunk.
struct AttnPlan {
  int64_t span, tiles;  // most positions / 32-position tiles a token attends
  int32_t chunks, tpc;  // chunks per (token, KV head), tiles per chunk
};

// span: the most positions one token attends (window, context bound).
// Full-context tiles start at position 0; a window starts anywhere, so it
// can straddle one more tile.  One chunk when the tiles fit three per wave,
// else about one block per CU over the batch's (token, KV head) pairs, at
// least one tile per wave.
constexpr AttnPlan attn_plan(int64_t span, bool windowed, int64_t batch, int64_t n_kv) {
  const int64_t tiles = windowed ? (span + kAttnTile - 2) / kAttnTile + 1 : (span + kAttnTile - 1) / kAttnTile;
  int64_t chunks = 1, tpc = tiles;
  if (tiles > 3 * kAttnWaves) {
    const int64_t pairs = batch * n_kv;
    int64_t want = (kAttnTargetBlocks + pairs - 1) / pairs;
    tpc = (tiles + want - 1) / want;
    if (tpc < kAttnWaves) tpc = kAttnWaves;
    chunks = (tiles + tpc - 1) / tpc;
  }
  return AttnPlan{span, tiles, (int32_t)chunks, (int32_t)tpc};
}

}  // namespace moe
