// api.cpp -- the extern "C" entry points of libgqa_attn.so (see
// include/gqa_attn.h).  Each call validates on the host, fills a kernel
// parameter block and enqueues on the caller's stream.
#include <math.h>
#include <string.h>

#include <atomic>

#include "internal.h"
#include "validate.h"

namespace gqa {

// Compute units and XCDs of the device current on the calling thread, read
// from the runtime once per device and remembered (the planners size the
// launches for them).  Without a device (host-only use) the shape of a full
// MI355X is assumed.
DeviceShape current_device_shape() {
  constexpr int kMaxDevices = 64;
  static std::atomic<int> cache[kMaxDevices];  // cus << 8 | xcds, 0 = unread
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices)
    return kDefaultShape;
  const int c = cache[dev].load(std::memory_order_relaxed);
  if (c > 0) return DeviceShape{c >> 8, c & 255};
  int cus = 0, xcds = 0;
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount,
                            dev) != hipSuccess ||
      cus <= 0 || cus >= (1 << 22))
    return kDefaultShape;
  if (hipDeviceGetAttribute(&xcds, hipDeviceAttributeNumberOfXccs, dev) !=
          hipSuccess ||
      xcds <= 0 || xcds > 255)
    xcds = 1;
  cache[dev].store(cus << 8 | xcds, std::memory_order_relaxed);
  return DeviceShape{cus, xcds};
}

}  // namespace gqa

namespace gqa {

// Workspace of a prefill chunk over an fp8 cache: the bf16 prefill's own
// workspace, then a bf16 copy of the prior (K then V, copy_rows tokens per
// sequence: the positions before the chunk on global layers, the ring on
// local layers).
struct PrefillFp8Ws {
  BlockPlan plan;
  size_t block_bytes;   // the bf16 prefill's workspace
  size_t copy_off;      // byte offset of the K copy
  int64_t copy_rows;
  size_t total;
};
static PrefillFp8Ws prefill_fp8_ws(int kind, int B, int n, int64_t max_keys,
                                   int64_t max_ctx, const DeviceShape& dev) {
  PrefillFp8Ws w;
  w.plan = plan_block(kind, B, n, max_keys, dev);
  w.block_bytes = block_ws_bytes(w.plan);
  w.copy_off = (w.block_bytes + 255) & ~(size_t)255;
  w.copy_rows = kind == GQA_LOCAL ? kW : (max_ctx > 1 ? max_ctx - 1 : 1);
  w.total = w.copy_off + 2 * (size_t)B * w.copy_rows * kTokenElems * 2;
  return w;
}

}  // namespace gqa

using namespace gqa;

extern "C" {

int gqa_abi_version(void) { return GQA_ABI_VERSION; }

int gqa_layer_kind(int layer) {
  if (layer < 0 || layer >= GQA_NUM_LAYERS) return GQA_ERR_INVALID_ARG;
  return layer % 4 == 3 ? GQA_GLOBAL : GQA_LOCAL;
}

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
      return decode_ws_bytes(
          B, plan_decode(kind, B, keys, current_device_shape()));
    }
    case GQA_OP_DRAFT:
      if (kind != GQA_GLOBAL) return 0;
      [[fallthrough]];
    case GQA_OP_VERIFY:
    case GQA_OP_PREFILL: {
      const bool verify = op != GQA_OP_PREFILL;
      if (n > (verify ? GQA_MAX_VERIFY : GQA_MAX_CONTEXT)) return 0;
      const int64_t keys = visible_keys(kind, max_ctx - 1);
      const DeviceShape dev = current_device_shape();
      const size_t need = block_ws_bytes(plan_block(kind, B, n, keys, dev));
      if (!verify) return need;
      // one verify workspace serves both cache formats (fp8 calls always
      // split their keys)
      const size_t need8 =
          block_ws_bytes(plan_block(kind, B, n, keys, dev, true));
      return need > need8 ? need : need8;
    }
    case GQA_OP_PREFILL_FP8: {
      if (n > GQA_MAX_CONTEXT) return 0;
      const int64_t keys = visible_keys(kind, max_ctx - 1);
      return prefill_fp8_ws(kind, B, n, keys, max_ctx,
                            current_device_shape()).total;
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

// Decode on a bf16 cache (layer) or an fp8 cache (layer8, with layer null;
// no fused append, host positions only).
static int decode_impl(const gqa_layer* layer, const void* q,
                       const void* k_new, const void* v_new,
                       const int64_t* pos, int B, float* out, void* ws,
                       size_t ws_bytes, void* stream,
                       const int64_t* pos_dev = nullptr,
                       int64_t max_pos = 0, bool noalloc = false,
                       const gqa_layer_fp8* layer8 = nullptr) {
  int64_t max_keys = 0;
  int rc;
  if (layer8) {
    rc = check_decode_fp8(layer8, q, pos, B, out, &max_keys);
  } else if (pos_dev) {
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
  const int32_t kind = layer8 ? layer8->kind : layer->kind;
  const double theta = layer8 ? layer8->rope_theta : layer->rope_theta;
  const DeviceShape dev = current_device_shape();
  const DecodePlan plan = plan_decode(kind, B, max_keys, dev);
  if (plan.splits > kMaxSplits) return GQA_ERR_UNSUPPORTED;
  const size_t need = decode_ws_bytes(B, plan);
  if (noalloc) {
    // the partials go to the device-resident scratch
    if (need > kNoAllocScratchBytes) return GQA_ERR_WS_TOO_SMALL;
    ws = noalloc_scratch();
    ws_bytes = kNoAllocScratchBytes;
    if (!ws) return GQA_ERR_HIP;
  }
  if (!ws) return GQA_ERR_INVALID_ARG;
  if (((uintptr_t)ws & 255u) != 0) return GQA_ERR_MISALIGNED;
  if (ws_bytes < need) return GQA_ERR_WS_TOO_SMALL;
  DecodeParams p;
  memset(&p, 0, sizeof p);
  if (layer8) {
    p.k8 = static_cast<const uint8_t*>(layer8->k);
    p.v8 = static_cast<const uint8_t*>(layer8->v);
    p.k_scale = layer8->k_scale;
    p.v_scale = layer8->v_scale;
    p.seq_stride = layer8->seq_stride;
    p.scale_stride = layer8->scale_stride;
    p.capacity = layer8->capacity;
  } else {
    p.k = static_cast<const uint16_t*>(layer->k);
    p.k_mut = static_cast<uint16_t*>(layer->k);
    p.v = static_cast<const uint16_t*>(layer->v);
    p.v_mut = static_cast<uint16_t*>(layer->v);
    p.k_new = static_cast<const uint16_t*>(k_new);
    p.v_new = static_cast<const uint16_t*>(v_new);
    p.seq_stride = layer->seq_stride;
    p.capacity = layer->capacity;
  }
  p.q = static_cast<const uint32_t*>(q);
  p.part = static_cast<float*>(ws);
  p.out = out;
  p.scale_log2 = (float)(1.0 / sqrt((double)kD) * 1.4426950408889634);
  p.splits = plan.splits;
  p.tiles_per_split = plan.tiles_per_split;
  p.units = B * kHkv * plan.splits;
  p.xcds = dev.xcds;
  const bool local = kind == GQA_LOCAL;
  if (local) {
    // revolutions per position of frequency c: theta^(-c/64) / (2 pi),
    // evaluated in double and rounded once.
    for (int c = 0; c < kD / 2; ++c)
      p.rope_rev[c] = (float)(pow(theta, -(double)c / (kD / 2)) /
                              (2.0 * 3.14159265358979323846));
  }
  p.pos_dev = pos_dev;
  p.max_pos = max_pos;
  for (int b = 0; b < B; ++b) p.pos[b] = pos_dev ? max_pos : pos[b];
  hipError_t e = launch_decode(p, plan, local, layer8 != nullptr, B,
                               (hipStream_t)stream);
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

int gqa_kv_append_fp8(const gqa_layer_fp8* layer, const void* k_new,
                      const void* v_new, const int64_t* pos0, int B, int n,
                      void* stream) {
  int rc = check_append_fp8(layer, k_new, v_new, pos0, B, n);
  if (rc != GQA_OK) return rc;
  AppendFp8Params p;
  memset(&p, 0, sizeof p);
  p.k_new = static_cast<const uint16_t*>(k_new);
  p.v_new = static_cast<const uint16_t*>(v_new);
  p.k = static_cast<uint8_t*>(layer->k);
  p.v = static_cast<uint8_t*>(layer->v);
  p.k_scale = layer->k_scale;
  p.v_scale = layer->v_scale;
  p.seq_stride = layer->seq_stride;
  p.scale_stride = layer->scale_stride;
  p.capacity = layer->capacity;
  p.n = n;
  p.local = layer->kind == GQA_LOCAL;
  p.first = (p.local && n > kW) ? n - kW : 0;
  for (int b = 0; b < B; ++b) p.pos0[b] = pos0[b];
  hipError_t e = launch_kv_append_fp8(p, B, n - p.first, (hipStream_t)stream);
  return e == hipSuccess ? GQA_OK : GQA_ERR_HIP;
}

int gqa_attn_decode_fp8(const gqa_layer_fp8* layer, const void* q,
                        const int64_t* pos, int B, float* out, void* ws,
                        size_t ws_bytes, void* stream) {
  return decode_impl(nullptr, q, nullptr, nullptr, pos, B, out, ws, ws_bytes,
                     stream, nullptr, 0, false, layer);
}

int gqa_attn_decode_noalloc(const gqa_layer* layer, const void* q,
                            const void* k_new, const void* v_new,
                            const int64_t* pos, int B, float* out,
                            void* stream) {
  return decode_impl(layer, q, k_new, v_new, pos, B, out, nullptr, 0, stream,
                     nullptr, 0, true);
}

// A validated block call on a bf16 cache with its plan.
static int block_launch(const gqa_layer* layer, const void* q,
                        const void* k_blk, const void* v_blk,
                        const int64_t* pos0, int B, int n, void* out,
                        void* ws, size_t ws_bytes, bool verify, bool together,
                        const BlockPlan& plan, void* stream) {
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
  p.qpw = plan.qpw;
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
  const BlockPlan plan =
      plan_block(layer->kind, B, n, max_keys, current_device_shape());
  return block_launch(layer, q, k_blk, v_blk, pos0, B, n, out, ws, ws_bytes,
                      verify, together, plan, stream);
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

// Verification or a drafted block over an fp8 cache.
static int block_impl_fp8(const gqa_layer_fp8* layer, const void* q,
                          const void* k_blk, const void* v_blk,
                          const int64_t* pos0, int B, int n, void* out,
                          void* ws, size_t ws_bytes, bool together,
                          void* stream) {
  int64_t max_keys = 0;
  int rc = check_block_fp8(layer, q, k_blk, v_blk, pos0, B, n, out, true,
                           &max_keys);
  if (rc != GQA_OK) return rc;
  if (together && layer->kind != GQA_GLOBAL) return GQA_ERR_UNSUPPORTED;
  const BlockPlan plan =
      plan_block(layer->kind, B, n, max_keys, current_device_shape(), true);
  if (!ws) return GQA_ERR_INVALID_ARG;
  if (((uintptr_t)ws & 255u) != 0) return GQA_ERR_MISALIGNED;
  if (ws_bytes < block_ws_bytes(plan)) return GQA_ERR_WS_TOO_SMALL;
  BlockParams p;
  memset(&p, 0, sizeof p);
  p.q = static_cast<const uint16_t*>(q);
  p.k_blk = static_cast<const uint16_t*>(k_blk);
  p.v_blk = static_cast<const uint16_t*>(v_blk);
  p.k8 = static_cast<const uint8_t*>(layer->k);
  p.v8 = static_cast<const uint8_t*>(layer->v);
  p.k_scale = layer->k_scale;
  p.v_scale = layer->v_scale;
  p.scale_stride = layer->scale_stride;
  p.capacity = layer->capacity;
  p.part = reinterpret_cast<float*>(ws);
  p.out = out;
  p.seq_stride = layer->seq_stride;  // bytes of codes per sequence
  p.n = n;
  p.qgroups = plan.qgroups;
  p.qpw = plan.qpw;
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
  hipError_t e =
      launch_block(p, plan, local, true, B, (hipStream_t)stream, true);
  return e == hipSuccess ? GQA_OK : GQA_ERR_HIP;
}

int gqa_attn_verify_fp8(const gqa_layer_fp8* layer, const void* q,
                        const void* k_blk, const void* v_blk,
                        const int64_t* pos0, int B, int n, float* out,
                        void* ws, size_t ws_bytes, void* stream) {
  return block_impl_fp8(layer, q, k_blk, v_blk, pos0, B, n, out, ws, ws_bytes,
                        false, stream);
}

int gqa_attn_draft_block_fp8(const gqa_layer_fp8* layer, const void* q,
                             const void* k_blk, const void* v_blk,
                             const int64_t* pos0, int B, int n, float* out,
                             void* ws, size_t ws_bytes, void* stream) {
  return block_impl_fp8(layer, q, k_blk, v_blk, pos0, B, n, out, ws, ws_bytes,
                        true, stream);
}

int gqa_attn_prefill_fp8(const gqa_layer_fp8* layer, const void* q,
                         const void* k_chunk, const void* v_chunk,
                         const int64_t* pos0, int B, int n, void* out,
                         void* ws, size_t ws_bytes, void* stream) {
  int64_t max_keys = 0;
  int rc = check_block_fp8(layer, q, k_chunk, v_chunk, pos0, B, n, out, false,
                           &max_keys);
  if (rc != GQA_OK) return rc;
  const bool local = layer->kind == GQA_LOCAL;
  int64_t max_pos0 = 0;
  for (int b = 0; b < B; ++b) max_pos0 = pos0[b] > max_pos0 ? pos0[b] : max_pos0;
  const PrefillFp8Ws lay = prefill_fp8_ws(layer->kind, B, n, max_keys,
                                          max_pos0 + n, current_device_shape());
  if (!ws) return GQA_ERR_INVALID_ARG;
  if (((uintptr_t)ws & 255u) != 0) return GQA_ERR_MISALIGNED;
  if (ws_bytes < lay.total) return GQA_ERR_WS_TOO_SMALL;
  char* const scratch = static_cast<char*>(ws);
  // the prior of every sequence as bf16: global layers its positions
  // 0 .. pos0 - 1 (slot = position), local layers the ring's slots that hold
  // positions before pos0
  DequantParams d;
  memset(&d, 0, sizeof d);
  d.k8 = static_cast<const uint8_t*>(layer->k);
  d.v8 = static_cast<const uint8_t*>(layer->v);
  d.k_scale = layer->k_scale;
  d.v_scale = layer->v_scale;
  d.seq_stride = layer->seq_stride;
  d.scale_stride = layer->scale_stride;
  d.capacity = layer->capacity;
  d.k_out = reinterpret_cast<uint16_t*>(scratch + lay.copy_off);
  d.v_out = d.k_out + (size_t)B * lay.copy_rows * kTokenElems;
  d.out_stride = lay.copy_rows * kTokenElems;
  int64_t max_rows = 0;
  for (int b = 0; b < B; ++b) {
    d.rows[b] = local ? (pos0[b] < kW ? pos0[b] : kW) : pos0[b];
    if (d.rows[b] > max_rows) max_rows = d.rows[b];
  }
  hipError_t e = launch_dequant_cache(d, B, max_rows, (hipStream_t)stream);
  if (e != hipSuccess) return GQA_ERR_HIP;
  // the bf16 prefill over the copy, which holds the prior exactly where a
  // bf16 cache of capacity copy_rows would
  gqa_layer view;
  memset(&view, 0, sizeof view);
  view.kind = layer->kind;
  view.window = layer->window;
  view.capacity = lay.copy_rows;
  view.rope_theta = layer->rope_theta;
  view.k = d.k_out;
  view.v = d.v_out;
  view.seq_stride = d.out_stride;
  return block_launch(&view, q, k_chunk, v_chunk, pos0, B, n, out, ws,
                      lay.block_bytes, false, false, lay.plan, stream);
}

int gqa_attn_prefill(const gqa_layer* layer, const void* q,
                     const void* k_chunk, const void* v_chunk,
                     const int64_t* pos0, int B, int n, void* out, void* ws,
                     size_t ws_bytes, void* stream) {
  return block_impl(layer, q, k_chunk, v_chunk, pos0, B, n, out, ws,
                    ws_bytes, false, false, stream);
}

}  // extern "C"
