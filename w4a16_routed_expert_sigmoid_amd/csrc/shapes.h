// Shape arithmetic of the library, in plain C++ with no HIP dependency:
// sizes of the NVFP4 runtime layout, the tiling limits the kernels
// accept, and the constants the workspace layouts are built from.  The
// kernels include it through common.h; the host-only validation unit
// (validate.cpp) includes it directly, so that unit also builds without
// the HIP runtime.  Every function is constexpr, which makes it callable
// from device code as well.
#pragma once

#include <stddef.h>
#include <stdint.h>

namespace moe {

constexpr int kWave = 64;
constexpr int kMaxBatch = 8;   // decode path: up to eight tokens
constexpr int kMaxTopK = 8;
constexpr int kXcdSlots = 16;  // XCC_ID is a 4-bit field
constexpr int kMaxExperts = 1024;
constexpr int kPrefillTileRows = 128;       // rows of one prefill GEMM tile
constexpr int32_t kMaxPrefillTokens = 1 << 22;
constexpr size_t kWsAlign = 256;            // workspace pieces start on 256-byte lines

// Lines of the decode sync region: per XCD, the logit ticket and flag, the
// h ticket and flag, and the layer-output ticket and flag of the persistent
// step (256 bytes each, word 0 used).
enum {
  kLineLTicket = 0,
  kLineLFlag = 1,
  kLineHTicket = 2,
  kLineHFlag = 3,
  kLineYTicket = 4,
  kLineYFlag = 5,
  kSyncLines = 6
};

// Layers of one persistent step launch (their weight pointers travel as
// kernel arguments).
constexpr int kPersistMaxLayers = 24;

// Bits of the status word: a bounded wait on another block of the same
// kernel ran out of polls (the values it waited for never arrived); an
// attention token's position was out of range (its output rows are zero).
enum { kStatusLogitWait = 1, kStatusHWait = 2, kStatusRouteWait = 4, kStatusBadPos = 8, kStatusYWait = 16 };

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

constexpr int64_t nvfp4_nibble_bytes(int64_t n, int64_t k) { return n * k / 2; }
constexpr int64_t nvfp4_matrix_bytes(int64_t n, int64_t k) { return n * k / 2 + n * k / 16; }

// Lanes that share one row: all 64 when a row has >= 64 chunks (each lane
// then walks chunks lane, lane+64, ...), else the chunk count, which must
// be a power of two.
constexpr int lanes_per_row(int k) { return k / 32 >= kWave ? kWave : k / 32; }

// A reduction dimension the GEMV kernels tile: at least two 32-element
// chunks, and either a power of two of them or at least one per lane.
constexpr bool k_tileable(int64_t k) {
  return k >= 64 && k % 32 == 0 && (k / 32 >= kWave || ((k / 32) & (k / 32 - 1)) == 0);
}

// Prefill: one GEMM tile of up to 128 rows of one expert's segment.
struct PfTile {
  int p0, cnt, e;  // first row, rows (<= 128), expert (-1: the shared expert)
};

// Upper bound of the 128-row tiles of a prefill call: the routed rows in
// whole tiles plus one ragged tile per non-empty expert, and the shared
// expert's rows.
constexpr int64_t prefill_max_tiles(int64_t T, int64_t k, int64_t E, bool shared) {
  return (E > 0 ? (T * k + kPrefillTileRows - 1) / kPrefillTileRows + (E < T * k ? E : T * k) : 0) +
         (shared ? (T + kPrefillTileRows - 1) / kPrefillTileRows : 0);
}

}  // namespace moe
