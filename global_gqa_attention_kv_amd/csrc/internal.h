// internal.h -- definitions shared by the host dispatch and the HIP kernels
// of libgqa_attn.so.  Not part of the public ABI.
#pragma once

#include <hip/hip_runtime.h>
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

// ---------------------------------------------------------------- append
struct AppendParams {
  const uint16_t* k_new;   // [B][n][2][128]
  const uint16_t* v_new;
  uint16_t* k;             // cache base
  uint16_t* v;
  int64_t seq_stride;      // elements
  int64_t capacity;
  int32_t n;               // tokens per sequence in k_new
  int32_t first;           // first token index written (local: max(0, n-2048))
  int32_t local;
  int32_t pad_;
  int64_t pos0[kMaxBatch];
};
hipError_t launch_kv_append(const AppendParams& p, int B, int count,
                            hipStream_t s);

// ---------------------------------------------------------------- decode
constexpr int kDecTile = 64;               // keys per tile
// Global-layer decode: waves per workgroup (each takes 16 keys of every
// tile for all 16 query heads), K and V tile slots in its LDS ring (16 KB
// each; K tiles are loaded one tile further ahead than V tiles), and how
// many such workgroups fit one CU (80 KB of LDS each).  Four waves, two
// workgroups per CU measured fastest: eight waves (two heads each), or three
// or four workgroups per CU with one slot each, lose more VALU efficiency
// than they gain.
constexpr int kGlobalWaves = 4;
constexpr int kGlobalKRing = 3;
constexpr int kGlobalVRing = 2;
constexpr int kGlobalWGsPerCU = 2;
// Local-layer decode (latency-bound, one tile per workgroup): 8 waves of 2
// heads put more waves behind each tile than 4 waves of 4 heads.
constexpr int kLocalWaves = 8;
// Local layers at small batch: the 16 heads of a KV head split over 4
// workgroups of 2 waves (2 heads each), which read the same tile (L2 hits
// after the first) and each do a quarter of the products.
constexpr int kLocalSmallHeads = 4;
constexpr int kLocalSmallWaves = 2;
constexpr int kLocalSmallMaxBatch = 2;
// Most key splits of one decode call (the merge kernel loads them all at once).
constexpr int kMaxSplits = 256;

// A workgroup serves all 16 query heads of one (sequence, KV head) over a
// split of tiles_per_split tiles; a second kernel merges the splits.
struct DecodePlan {
  int splits;           // S: key splits per (sequence, KV head)
  int tiles_per_split;  // tiles of kDecTile keys per split
  int heads_per_wg;     // 16, or kLocalSmallHeads (head groups share a tile)
};
DecodePlan plan_decode(int kind, int B, int64_t max_keys);
size_t decode_ws_bytes(int B, const DecodePlan& plan);

struct DecodeParams {
  const uint16_t* k;       // cache base (sequence 0, slot 0, head 0)
  uint16_t* k_mut;         // same cache, written when k_new is given
  const uint16_t* v;
  uint16_t* v_mut;
  const uint16_t* k_new;   // [B][1][2][128] new token, or null
  const uint16_t* v_new;
  const uint32_t* q;       // [B][32][64] bf16 pairs
  float* part;             // partial sums, see decode.hip
  float* out;              // [B][32][128]
  int64_t seq_stride;      // elements
  float scale_log2;        // softmax scale * log2(e)
  int32_t splits;
  int32_t tiles_per_split;
  int32_t units;           // B * 2 * splits
  float rope_rev[kD / 2];  // local: theta^(-c/64) / (2 pi), revolutions per position
  const int64_t* pos_dev;  // device positions [B] (read instead of pos), or null
  int64_t max_pos;         // with pos_dev: positions above it are not attended
  int64_t pos[kMaxBatch];
};
hipError_t launch_decode(const DecodeParams& p, const DecodePlan& plan,
                         bool local, int B, hipStream_t s);

// ---------------------------------------------------------------- block
// A block of n query tokens per sequence at positions pos0 .. pos0+n-1 whose
// K/V (k_blk, v_blk) are not in the cache yet: chunked prefill (n up to a
// few thousand, bf16 output), speculative verification (n <= 16, fp32
// output, keys split across workgroups) and a drafted block whose tokens
// are predicted together (as verification, without the causal order inside
// the block).
constexpr int kBlkTile = 64;               // keys per tile
constexpr int kCUs = 256;                  // compute units of an MI355X
constexpr int kBlkQpw = 16;                // query tokens per workgroup
constexpr int kMaxPrefill = GQA_MAX_CONTEXT;

struct BlockPlan {
  int qpw;          // query tokens per workgroup (x 16 heads = rows)
  int qgroups;      // ceil(n / qpw)
  int splits;       // key splits (1 = no partials)
  size_t klin_bytes;   // local: pre-rotated keys
  size_t part_bytes;   // split partials
};
BlockPlan plan_block(int kind, int B, int n, int64_t max_keys);
size_t block_ws_bytes(const BlockPlan& plan);

struct BlockParams {
  const uint16_t* q;        // [B][n][32][128]
  const uint16_t* k_blk;    // [B][n][2][128]
  const uint16_t* v_blk;
  const uint16_t* k_cache;  // layer cache base
  const uint16_t* v_cache;
  uint16_t* k_lin;          // local: rotated keys [B][klin_rows][2][128]
  float* part;              // split partials
  void* out;                // [B][n][32][128], bf16 or fp32
  int64_t seq_stride;       // cache elements per sequence
  int64_t klin_rows;        // rows of k_lin per sequence
  int32_t n;
  int32_t qgroups;
  int32_t splits;
  int32_t batch;            // B
  int32_t together;         // 1: every query sees the whole block (global)
  float scale_log2;
  float rope_rev[kD / 2];
  int64_t pos0[kMaxBatch];
};
hipError_t launch_block(const BlockParams& p, const BlockPlan& plan,
                        bool local, bool out_f32, int B, hipStream_t s);

}  // namespace gqa
