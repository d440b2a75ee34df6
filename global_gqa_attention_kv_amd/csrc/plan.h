// plan.h -- how an attention call is spread over workgroups, and how large a
// workspace it needs.  Plain C++ (no HIP): the dispatch in api.cpp calls it
// with the shape of the current device, and the host tests build it with
// g++ and drive it with any device shape.  Not part of the public ABI.
#pragma once

#include <stddef.h>
#include <stdint.h>

#include "gqa_attn.h"

namespace gqa {

constexpr int kHq = GQA_NUM_Q_HEADS;      // 32 query heads
constexpr int kHkv = GQA_NUM_KV_HEADS;    // 2 KV heads
constexpr int kGroup = kHq / kHkv;        // 16 query heads per KV head
constexpr int kD = GQA_HEAD_DIM;          // 128
constexpr int kW = GQA_WINDOW;            // 2048-slot ring
constexpr int kMaxBatch = GQA_MAX_BATCH;
constexpr int kTokenElems = kHkv * kD;    // 256 bf16 per token per cache

// Compute units and XCDs (dies with an L2 of their own) of the device a
// call runs on.  A full MI355X has 256 CUs in 8 XCDs.
struct DeviceShape {
  int cus;
  int xcds;
};
constexpr DeviceShape kDefaultShape = {256, 8};

// ---------------------------------------------------------------- decode
constexpr int kDecTile = 64;               // keys per tile
// Global-layer decode workgroups resident per CU (80 KB of LDS each).
constexpr int kGlobalWGsPerCU = 2;
// Local layers at small batch: the 16 heads of a KV head split over 4
// workgroups (head groups) that read the same tile.
constexpr int kLocalSmallHeads = 8;
constexpr int kLocalSmallMaxBatch = 2;
// Most key splits of one decode or block call (a merge loads them all at
// once).
constexpr int kMaxSplits = 256;

// Device-resident scratch of the entry point that allocates nothing
// (gqa_attn_decode_noalloc): room for the decode partials of every batch
// size and context on a 256-CU device (the largest, batch 1 or 2 at 131072
// keys, needs 4.3 MB).
constexpr size_t kNoAllocScratchBytes = GQA_NOALLOC_SCRATCH_BYTES;
static_assert(kNoAllocScratchBytes % 256 == 0, "scratch alignment");

// A decode workgroup serves all 16 query heads (or one head group) of one
// (sequence, KV head) over a split of tiles_per_split tiles.
struct DecodePlan {
  int splits;           // S: key splits per (sequence, KV head)
  int tiles_per_split;  // tiles of kDecTile keys per split
  int heads_per_wg;     // 16, or kLocalSmallHeads (head groups share a tile)
};
DecodePlan plan_decode(int kind, int B, int64_t max_keys,
                       const DeviceShape& dev);
// Partial sums [B][2][head groups][splits][heads x 130] floats.
size_t decode_ws_bytes(int B, const DecodePlan& plan);

// ---------------------------------------------------------------- block
constexpr int kBlkTile = 64;               // keys per tile
constexpr int kBlkQpw = 16;                // query tokens per workgroup
constexpr int kBlkQpwSmall = 8;            // local layers with key splits
constexpr int kBlkMaxSplits = 128;         // key splits of a block call

struct BlockPlan {
  int qpw;          // query tokens per workgroup (x 16 heads = rows)
  int qgroups;      // ceil(n / qpw)
  int splits;       // key splits (1 = no partials)
  int grid;         // workgroups launched
  int walks;        // work items each workgroup takes in turn (no splits)
  size_t klin_bytes;   // local: pre-rotated keys
  size_t part_bytes;   // split partials
};
// always_split: key splits (one or more, partials and merge) whatever the
// shape, with 8-token workgroups on local layers, as verification and
// drafted blocks over fp8 caches take.
BlockPlan plan_block(int kind, int B, int n, int64_t max_keys,
                     const DeviceShape& dev, bool always_split = false);
size_t block_ws_bytes(const BlockPlan& plan);

}  // namespace gqa
