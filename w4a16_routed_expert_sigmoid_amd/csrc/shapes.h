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
constexpr int kMaxBatch = 16;     // decode path: up to 16 tokens (NVFP4 weights)
constexpr int kMaxBatchBf16 = 8;  // decode path with BF16 weights, and the dense projection
constexpr int kMaxRouteStage = 16384;  // floats of a batch gate/up block's routing stage: B * E logits + E marks
constexpr int kMaxTopK = 8;
constexpr int kXcdSlots = 16;  // XCC_ID is a 4-bit field
constexpr int kMaxExperts = 1024;
constexpr int kPrefillTileRows = 128;       // rows of one prefill GEMM tile
constexpr int kPrefillSmallRows = 16;       // rows of a small-tile prefill tile (up to kPrefillSmallMaxTokens tokens)
constexpr int kPrefillSmallMaxTokens = 48;
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

// Prefill: one GEMM tile of up to 128 (or 16) rows of one expert's segment.
struct PfTile {
  int p0, cnt, e;  // first row, rows (<= the tile height), expert (-1: the shared expert)
};

// Upper bound of the tiles of `rows` rows of a prefill call: the routed
// rows in whole tiles plus one ragged tile per non-empty expert, and the
// shared expert's rows.
constexpr int64_t prefill_max_tiles(int64_t T, int64_t k, int64_t E, bool shared, int64_t rows = kPrefillTileRows) {
  return (E > 0 ? (T * k + rows - 1) / rows + (E < T * k ? E : T * k) : 0) + (shared ? (T + rows - 1) / rows : 0);
}

// Rows per prefill tile: NVFP4 calls of up to kPrefillSmallMaxTokens tokens
// take 16-row tiles (each expert's few rows as the 16 token columns of the
// decode kernels' matrix-core tiles); NVFP4 calls of up to
// kPrefillMidMaxTokens tokens kPrefillMidRows-row tiles on the grouped GEMM
// (an expert with many rows spreads over several blocks instead of one long
// item); the rest 128-row tiles.
constexpr int kPrefillMidRows = 32;
constexpr int kPrefillMidMaxTokens = 1024;
constexpr int prefill_tile_rows(int64_t T, int wtype) {
  return (wtype == 1 && T <= kPrefillSmallMaxTokens)  ? kPrefillSmallRows
         : (wtype == 1 && T <= kPrefillMidMaxTokens) ? kPrefillMidRows
                                                     : kPrefillTileRows;
}

// K splits of the prefill router GEMM (64 x 64 tiles, 128-K stages): calls
// with fewer than kRouterMinBlocks tiles split the depth (at most
// kRouterMaxSplit ways) so that about that many blocks run, each split
// writing its own partial logits (the top-k sums them in split order).
// Every split holds at least one stage.
constexpr int kRouterMinBlocks = 128;
constexpr int kRouterMaxSplit = 8;
constexpr int prefill_router_split(int64_t T, int64_t E, int64_t H) {
  const int64_t base = ((T + 63) / 64) * ((E + 63) / 64);
  const int64_t stages = (H + 127) / 128;
  if (E <= 0 || base >= kRouterMinBlocks) return 1;
  int64_t split = (kRouterMinBlocks + base - 1) / base;
  if (split > kRouterMaxSplit) split = kRouterMaxSplit;
  if (split > stages) split = stages;
  const int64_t per = (stages + split - 1) / split;
  return (int)((stages + per - 1) / per);
}

// Rows of [E] logits the prefill workspace reserves: at least
// prefill_router_split(T, E, H) * T, and non-decreasing in T (a workspace
// sized for T tokens serves every smaller call).
constexpr int64_t prefill_router_logit_rows(int64_t T, int64_t E, int64_t H) {
  const int64_t stages = (H + 127) / 128;
  const int64_t cap = T + 64 * kRouterMinBlocks / (E > 0 ? (E + 63) / 64 : 1) + 64;
  const int64_t most = T * (stages < kRouterMaxSplit ? stages : kRouterMaxSplit);
  return most < cap ? most : cap;
}

}  // namespace moe
