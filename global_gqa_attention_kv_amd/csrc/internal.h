// internal.h -- definitions shared by the host dispatch and the HIP kernels
// of libgqa_attn.so.  Not part of the public ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "gqa_attn.h"
#include "plan.h"

namespace gqa {

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

// Append to an fp8 cache: the new bf16 tokens are quantised to E4M3 with one
// scale per (token, KV head) (kv_append.hip).
struct AppendFp8Params {
  const uint16_t* k_new;   // [B][n][2][128] bf16
  const uint16_t* v_new;
  uint8_t* k;              // code cache base
  uint8_t* v;
  float* k_scale;          // scales [B][2][capacity]
  float* v_scale;
  int64_t seq_stride;      // bytes between sequences of the codes
  int64_t scale_stride;    // floats between sequences of the scales
  int64_t capacity;
  int32_t n;
  int32_t first;
  int32_t local;
  int32_t pad_;
  int64_t pos0[kMaxBatch];
};
hipError_t launch_kv_append_fp8(const AppendFp8Params& p, int B, int count,
                                hipStream_t s);

// The first rows[b] slots of each sequence's fp8 cache as bf16 (code x
// scale, rounded once to bf16), into a copy the bf16 block kernels read:
// the prior a prefill chunk over an fp8 cache attends to (kv_append.hip).
struct DequantParams {
  const uint8_t* k8;       // codes, sequence b at byte b * seq_stride
  const uint8_t* v8;
  const float* k_scale;    // scales [B][2][capacity]
  const float* v_scale;
  uint16_t* k_out;         // bf16 copy, sequence b at element b * out_stride
  uint16_t* v_out;
  int64_t seq_stride;
  int64_t scale_stride;
  int64_t capacity;
  int64_t out_stride;
  int64_t rows[kMaxBatch];
};
hipError_t launch_dequant_cache(const DequantParams& p, int B,
                                int64_t max_rows, hipStream_t s);

// ---------------------------------------------------------------- decode
// Global-layer decode: waves per workgroup (each takes 16 keys of every
// tile for all 16 query heads) and K and V tile slots in its LDS ring (16 KB
// each; K tiles are loaded one tile further ahead than V tiles); two such
// workgroups fit one CU (kGlobalWGsPerCU, 80 KB of LDS each).  Four waves,
// two workgroups per CU measured fastest: eight waves (two heads each), or
// three or four workgroups per CU with one slot each, lose more VALU
// efficiency than they gain.
constexpr int kGlobalWaves = 4;
constexpr int kGlobalKRing = 3;
constexpr int kGlobalVRing = 2;
// Local-layer decode (latency-bound, one tile per workgroup): 8 waves of 2
// heads put more waves behind each tile than 4 waves of 4 heads.
constexpr int kLocalWaves = 8;
// Local layers at small batch: the 16 heads of a KV head split over two
// workgroups of kLocalSmallHeads = 8 heads in 4 waves, which read the same
// tile (L2 hits after the first) and each do half of the products (measured
// at batch 1 against four workgroups of 4 heads in 2 waves: 52-layer step at
// 131072 keys 818 -> 799 us; one workgroup of 16 heads was slower still).
constexpr int kLocalSmallWaves = 4;

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
  int32_t xcds;            // XCDs of the device (workgroup placement)
  float rope_rev[kD / 2];  // local: theta^(-c/64) / (2 pi), revolutions per position
  const int64_t* pos_dev;  // device positions [B] (read instead of pos), or null
  int64_t max_pos;         // with pos_dev: positions above it are not attended
  // fp8 caches (E4M3 codes plus one fp32 scale per token and KV head)
  const uint8_t* k8;       // codes, sequence b at byte b * seq_stride
  const uint8_t* v8;
  const float* k_scale;    // scales [B][2][capacity]
  const float* v_scale;
  int64_t scale_stride;    // floats between sequences of the scales
  int64_t capacity;        // slots per sequence (KV-head stride of the scales)
  int64_t pos[kMaxBatch];
};
hipError_t launch_decode(const DecodeParams& p, const DecodePlan& plan,
                         bool local, bool fp8, int B, hipStream_t s);

// Device address of the current device's copy of the no-allocation scratch
// (kNoAllocScratchBytes), looked up on the first call on each device; null
// when there is no device or the lookup fails.
void* noalloc_scratch();

// ---------------------------------------------------------------- block
// A block of n query tokens per sequence at positions pos0 .. pos0+n-1 whose
// K/V (k_blk, v_blk) are not in the cache yet: chunked prefill (n up to a
// few thousand, bf16 output), speculative verification (n <= 16, fp32
// output, keys split across workgroups) and a drafted block whose tokens
// are predicted together (as verification, without the causal order inside
// the block).
constexpr int kMaxPrefill = GQA_MAX_CONTEXT;

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
  int32_t qpw;              // query tokens per workgroup (the plan's)
  float scale_log2;
  float rope_rev[kD / 2];
  // fp8 caches (key-split calls): E4M3 codes (sequence b at byte
  // b * seq_stride) and one fp32 scale per (token, KV head) [B][2][capacity]
  const uint8_t* k8;
  const uint8_t* v8;
  const float* k_scale;
  const float* v_scale;
  int64_t scale_stride;     // floats between sequences of the scales
  int64_t capacity;         // slots per sequence (KV-head stride of the scales)
  int64_t pos0[kMaxBatch];
};
// fp8: the cache is read through k8 / v8 and the scales; the plan must come
// from plan_block(..., always_split = true).
hipError_t launch_block(const BlockParams& p, const BlockPlan& plan,
                        bool local, bool out_f32, int B, hipStream_t s,
                        bool fp8 = false);

}  // namespace gqa
