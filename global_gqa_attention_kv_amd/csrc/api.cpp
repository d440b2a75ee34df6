// api.cpp -- the extern "C" entry points of libgqa_attn.so (see
// include/gqa_attn.h).  Each call validates on the host, fills a kernel
// parameter block and enqueues on the caller's stream.
#include <math.h>
#include <string.h>

#include "internal.h"
#include "validate.h"

namespace gqa {

namespace {
// Global-layer decode: as many split-kernel workgroups as fit the 256 CUs at
// once, so the launch runs as one full round (a partial second round would
// leave part of the device idle at the end).
constexpr int kDecodeTargetWGs = 256 * kGlobalWGsPerCU;
static_assert(kDecodeTargetWGs / 2 <= kMaxSplits, "merge kernel capacity");
size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }
}  // namespace

DecodePlan plan_decode(int kind, int B, int64_t max_keys) {
  const int64_t tiles = (max_keys + kDecTile - 1) / kDecTile;
  DecodePlan p;
  p.heads_per_wg = kGroup;
  if (kind == GQA_LOCAL) {
    if (B <= kLocalSmallMaxBatch) p.heads_per_wg = kLocalSmallHeads;
    // the window is 32 tiles: one tile per workgroup up to batch 4 (256
    // workgroups), then longer splits so a launch stays near 256
    p.tiles_per_split = B >= 8 ? B / 4 : 1;
    if (p.tiles_per_split > (int)tiles) p.tiles_per_split = (int)tiles;
    if (p.tiles_per_split < 1) p.tiles_per_split = 1;
    p.splits = (int)((tiles + p.tiles_per_split - 1) / p.tiles_per_split);
    if (p.splits < 1) p.splits = 1;
    return p;
  }
  int64_t want = kDecodeTargetWGs / (2 * B);
  if (want < 1) want = 1;
  int64_t per = (tiles + want - 1) / want;
  if (per < 1) per = 1;
  p.tiles_per_split = (int)per;
  p.splits = (int)((tiles + per - 1) / per);
  if (p.splits < 1) p.splits = 1;
  return p;
}

// Workspace: the partial sums [B][2][head groups][splits][heads x 130]
// floats (m[heads], l[heads], o[heads][128] per split).
size_t decode_ws_bytes(int B, const DecodePlan& plan) {
  return align256((size_t)B * kHkv * plan.splits * kGroup * (kD + 2) *
                  sizeof(float));
}

// Block operations.  Workgroups take 16 query tokens of one KV head; the
// key range is split across workgroups (down to one 64-key tile each) only
// when the query groups alone cannot fill the device with kBlockTargetWGs
// workgroups: always for verification (<= 16 tokens), for short prefills.
namespace {
constexpr int kBlockTargetWGs = 256;
}

BlockPlan plan_block(int kind, int B, int n, int64_t max_keys) {
  BlockPlan p;
  p.qpw = kBlkQpw;
  p.qgroups = (n + p.qpw - 1) / p.qpw;
  // keys one workgroup may see: its window (local) or everything before it
  const int64_t wg_keys =
      kind == GQA_LOCAL ? (int64_t)kW - 1 + p.qpw : max_keys;
  const int64_t tiles = (wg_keys + kBlkTile - 1) / kBlkTile;
  const int64_t groups = (int64_t)p.qgroups * kHkv * B;
  int64_t splits = 1;
  if (groups < kBlockTargetWGs)
    splits = (kBlockTargetWGs + groups - 1) / groups;
  // down to one tile per workgroup (measured on the local verify: one tile
  // per workgroup beat two now that split partials are bf16 rows)
  if (splits > tiles) splits = tiles;
  if (splits < 1) splits = 1;
  p.splits = (int)splits;
  // local layers without key splits read pre-rotated keys from the
  // workspace; split calls rotate each tile in LDS
  p.klin_bytes = kind == GQA_LOCAL && p.splits == 1
                     ? align256((size_t)B * ((size_t)kW + n) * kTokenElems * 2)
                     : 0;
  p.part_bytes = p.splits > 1
                     ? align256((size_t)B * kHkv * p.qgroups * p.splits *
                                p.qpw * kGroup * 68 * sizeof(float))
                     : 0;
  return p;
}

// Rotated keys (local layers), then partial sums (split keys).
size_t block_ws_bytes(const BlockPlan& plan) {
  const size_t n = plan.klin_bytes + plan.part_bytes;
  return n ? n : 256;
}

}  // namespace gqa

using namespace gqa;

extern "C" {

int gqa_abi_version(void) { return GQA_ABI_VERSION; }

const char* gqa_status_string(int status) {
  switch (status) {
    case GQA_OK: return "ok";
    case GQA_ERR_INVALID_ARG: return "invalid argument";
    case GQA_ERR_POS_RANGE: return "position out of range";
    case GQA_ERR_MISALIGNED: return "pointer or stride not 16-byte aligned";
    case GQA_ERR_WS_TOO_SMALL: return "workspace too small";
    case GQA_ERR_UNSUPPORTED: return "layer outside the compiled shape";
    case GQA_ERR_HIP: return "HIP launch failed";
    default: return "unknown status";
  }
}

size_t gqa_workspace_bytes(int op, int kind, int B, int n, int64_t max_ctx) {
  if (B < 1 || B > GQA_MAX_BATCH || n < 1 || max_ctx < 1) return 0;
  if (kind != GQA_LOCAL && kind != GQA_GLOBAL) return 0;
  if (kind == GQA_GLOBAL && max_ctx > GQA_MAX_CONTEXT) return 0;
  switch (op) {
    case GQA_OP_DECODE: {
      const int64_t keys = visible_keys(kind, max_ctx - 1);
      return decode_ws_bytes(B, plan_decode(kind, B, keys));
    }
    case GQA_OP_DRAFT:
      if (kind != GQA_GLOBAL) return 0;
      [[fallthrough]];
    case GQA_OP_VERIFY:
    case GQA_OP_PREFILL: {
      const bool verify = op != GQA_OP_PREFILL;
      if (n > (verify ? GQA_MAX_VERIFY : GQA_MAX_CONTEXT)) return 0;
      const int64_t keys = visible_keys(kind, max_ctx - 1);
      return block_ws_bytes(plan_block(kind, B, n, keys));
    }
    default:
      return 0;
  }
}

int gqa_kv_append(const gqa_layer* layer, const void* k_new, const void* v_new,
                  const int64_t* pos0, int B, int n, void* stream) {
  int rc = check_append(layer, k_new, v_new, pos0, B, n);
  if (rc != GQA_OK) return rc;
  AppendParams p;
  memset(&p, 0, sizeof p);
  p.k_new = static_cast<const uint16_t*>(k_new);
  p.v_new = static_cast<const uint16_t*>(v_new);
  p.k = static_cast<uint16_t*>(layer->k);
  p.v = static_cast<uint16_t*>(layer->v);
  p.seq_stride = layer->seq_stride;
  p.capacity = layer->capacity;
  p.n = n;
  p.local = layer->kind == GQA_LOCAL;
  p.first = (p.local && n > kW) ? n - kW : 0;
  for (int b = 0; b < B; ++b) p.pos0[b] = pos0[b];
  const int count = n - p.first;
  hipError_t e = launch_kv_append(p, B, count, (hipStream_t)stream);
  return e == hipSuccess ? GQA_OK : GQA_ERR_HIP;
}

static int decode_impl(const gqa_layer* layer, const void* q,
                       const void* k_new, const void* v_new,
                       const int64_t* pos, int B, float* out, void* ws,
                       size_t ws_bytes, void* stream,
                       const int64_t* pos_dev = nullptr,
                       int64_t max_pos = 0) {
  int64_t max_keys = 0;
  int rc;
  if (pos_dev) {
    // the kernels read the positions; the host checks the bound they are
    // held to, exactly as it checks a position
    if ((uintptr_t)pos_dev & 7u) return GQA_ERR_MISALIGNED;
    int64_t bound[kMaxBatch];
    if (B < 1 || B > GQA_MAX_BATCH) return GQA_ERR_INVALID_ARG;
    for (int b = 0; b < B; ++b) bound[b] = max_pos;
    rc = check_decode(layer, q, bound, B, out, &max_keys);
  } else {
    rc = check_decode(layer, q, pos, B, out, &max_keys);
  }
  if (rc != GQA_OK) return rc;
  if (k_new || v_new) {
    if (!k_new || !v_new) return GQA_ERR_INVALID_ARG;
    if (((uintptr_t)k_new & 15u) || ((uintptr_t)v_new & 15u))
      return GQA_ERR_MISALIGNED;
  }
  const DecodePlan plan = plan_decode(layer->kind, B, max_keys);
  if (plan.splits > kMaxSplits) return GQA_ERR_UNSUPPORTED;
  const size_t need = decode_ws_bytes(B, plan);
  if (!ws) return GQA_ERR_INVALID_ARG;
  if (((uintptr_t)ws & 255u) != 0) return GQA_ERR_MISALIGNED;
  if (ws_bytes < need) return GQA_ERR_WS_TOO_SMALL;
  DecodeParams p;
  memset(&p, 0, sizeof p);
  p.k = static_cast<const uint16_t*>(layer->k);
  p.k_mut = static_cast<uint16_t*>(layer->k);
  p.v = static_cast<const uint16_t*>(layer->v);
  p.v_mut = static_cast<uint16_t*>(layer->v);
  p.k_new = static_cast<const uint16_t*>(k_new);
  p.v_new = static_cast<const uint16_t*>(v_new);
  p.q = static_cast<const uint32_t*>(q);
  p.part = static_cast<float*>(ws);
  p.out = out;
  p.seq_stride = layer->seq_stride;
  p.scale_log2 = (float)(1.0 / sqrt((double)kD) * 1.4426950408889634);
  p.splits = plan.splits;
  p.tiles_per_split = plan.tiles_per_split;
  p.units = B * kHkv * plan.splits;
  const bool local = layer->kind == GQA_LOCAL;
  if (local) {
    // revolutions per position of frequency c: theta^(-c/64) / (2 pi),
    // evaluated in double and rounded once.
    for (int c = 0; c < kD / 2; ++c)
      p.rope_rev[c] = (float)(pow(layer->rope_theta, -(double)c / (kD / 2)) /
                              (2.0 * 3.14159265358979323846));
  }
  p.pos_dev = pos_dev;
  p.max_pos = max_pos;
  for (int b = 0; b < B; ++b) p.pos[b] = pos_dev ? max_pos : pos[b];
  hipError_t e = launch_decode(p, plan, local, B, (hipStream_t)stream);
  return e == hipSuccess ? GQA_OK : GQA_ERR_HIP;
}

int gqa_attn_decode(const gqa_layer* layer, const void* q, const int64_t* pos,
                    int B, float* out, void* ws, size_t ws_bytes,
                    void* stream) {
  return decode_impl(layer, q, nullptr, nullptr, pos, B, out, ws, ws_bytes,
                     stream);
}

int gqa_attn_decode_append(const gqa_layer* layer, const void* q,
                           const void* k_new, const void* v_new,
                           const int64_t* pos, int B, float* out, void* ws,
                           size_t ws_bytes, void* stream) {
  if (!k_new || !v_new) return GQA_ERR_INVALID_ARG;
  return decode_impl(layer, q, k_new, v_new, pos, B, out, ws, ws_bytes,
                     stream);
}

int gqa_attn_decode_dev(const gqa_layer* layer, const void* q,
                        const void* k_new, const void* v_new,
                        const int64_t* pos_dev, int64_t max_pos, int B,
                        float* out, void* ws, size_t ws_bytes, void* stream) {
  if (!pos_dev) return GQA_ERR_INVALID_ARG;
  return decode_impl(layer, q, k_new, v_new, nullptr, B, out, ws, ws_bytes,
                     stream, pos_dev, max_pos);
}

static int block_impl(const gqa_layer* layer, const void* q,
                      const void* k_blk, const void* v_blk,
                      const int64_t* pos0, int B, int n, void* out, void* ws,
                      size_t ws_bytes, bool verify, bool together,
                      void* stream) {
  int64_t max_keys = 0;
  int rc = check_block(layer, q, k_blk, v_blk, pos0, B, n, out, verify,
                       &max_keys);
  if (rc != GQA_OK) return rc;
  if (together && layer->kind != GQA_GLOBAL) return GQA_ERR_UNSUPPORTED;
  const BlockPlan plan = plan_block(layer->kind, B, n, max_keys);
  if (!ws) return GQA_ERR_INVALID_ARG;
  if (((uintptr_t)ws & 255u) != 0) return GQA_ERR_MISALIGNED;
  if (ws_bytes < block_ws_bytes(plan)) return GQA_ERR_WS_TOO_SMALL;
  BlockParams p;
  memset(&p, 0, sizeof p);
  p.q = static_cast<const uint16_t*>(q);
  p.k_blk = static_cast<const uint16_t*>(k_blk);
  p.v_blk = static_cast<const uint16_t*>(v_blk);
  p.k_cache = static_cast<const uint16_t*>(layer->k);
  p.v_cache = static_cast<const uint16_t*>(layer->v);
  char* const scratch = static_cast<char*>(ws);
  p.k_lin = plan.klin_bytes ? reinterpret_cast<uint16_t*>(scratch) : nullptr;
  p.part = plan.part_bytes
               ? reinterpret_cast<float*>(scratch + plan.klin_bytes)
               : nullptr;
  p.out = out;
  p.seq_stride = layer->seq_stride;
  p.klin_rows = (int64_t)kW + n;
  p.n = n;
  p.qgroups = plan.qgroups;
  p.splits = plan.splits;
  p.batch = B;
  p.together = together ? 1 : 0;
  p.scale_log2 = (float)(1.0 / sqrt((double)kD) * 1.4426950408889634);
  const bool local = layer->kind == GQA_LOCAL;
  if (local) {
    for (int c = 0; c < kD / 2; ++c)
      p.rope_rev[c] = (float)(pow(layer->rope_theta, -(double)c / (kD / 2)) /
                              (2.0 * 3.14159265358979323846));
  }
  for (int b = 0; b < B; ++b) p.pos0[b] = pos0[b];
  hipError_t e = launch_block(p, plan, local, verify, B, (hipStream_t)stream);
  return e == hipSuccess ? GQA_OK : GQA_ERR_HIP;
}

int gqa_attn_verify(const gqa_layer* layer, const void* q, const void* k_blk,
                    const void* v_blk, const int64_t* pos0, int B, int n,
                    float* out, void* ws, size_t ws_bytes, void* stream) {
  return block_impl(layer, q, k_blk, v_blk, pos0, B, n, out, ws, ws_bytes,
                    true, false, stream);
}

int gqa_attn_draft_block(const gqa_layer* layer, const void* q,
                         const void* k_blk, const void* v_blk,
                         const int64_t* pos0, int B, int n, float* out,
                         void* ws, size_t ws_bytes, void* stream) {
  return block_impl(layer, q, k_blk, v_blk, pos0, B, n, out, ws, ws_bytes,
                    true, true, stream);
}

int gqa_attn_prefill(const gqa_layer* layer, const void* q,
                     const void* k_chunk, const void* v_chunk,
                     const int64_t* pos0, int B, int n, void* out, void* ws,
                     size_t ws_bytes, void* stream) {
  return block_impl(layer, q, k_chunk, v_chunk, pos0, B, n, out, ws,
                    ws_bytes, false, false, stream);
}

}  // extern "C"
