// validate.cpp -- host-side argument checks of the C ABI.  Every entry point
// runs these before it enqueues anything; a failure returns a GQA_ERR_* code
// and leaves the stream untouched.  Order of precedence: INVALID_ARG (null
// pointers, batch or token counts), UNSUPPORTED (a layer outside the compiled
// shape), MISALIGNED, POS_RANGE.
#include "validate.h"

#include <math.h>

namespace gqa {

namespace {
// Positions stay below 2^31 - 4096, so the kernels' 32-bit key-range
// arithmetic (a block's last key + 1, a tile's first key + 64) cannot wrap.
constexpr int64_t kMaxPos = GQA_MAX_POSITION;
bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }
}  // namespace

int64_t visible_keys(int kind, int64_t pos) {
  return kind == GQA_LOCAL ? (pos + 1 < GQA_WINDOW ? pos + 1 : GQA_WINDOW)
                           : pos + 1;
}

// The compiled shape: local layers a 2048-slot ring with RoPE, global layers
// a linear cache of at most 131072 slots without RoPE.
static int check_shape(int32_t kind, int32_t window, int64_t capacity,
                       double rope_theta) {
  if (kind == GQA_LOCAL) {
    if (window != GQA_WINDOW || capacity != GQA_WINDOW ||
        !(rope_theta > 0.0) || !isfinite(rope_theta))
      return GQA_ERR_UNSUPPORTED;
  } else if (kind == GQA_GLOBAL) {
    if (window != 0 || rope_theta != 0.0 || capacity < 1 ||
        capacity > GQA_MAX_CONTEXT)
      return GQA_ERR_UNSUPPORTED;
  } else {
    return GQA_ERR_UNSUPPORTED;
  }
  return GQA_OK;
}

// Positions of one decode step (pos[b]), or of blocks of n tokens starting
// at pos[b]; *max_keys: the most keys any query sees.
static int check_positions(int32_t kind, int64_t capacity, const int64_t* pos,
                           int B, int n, int64_t* max_keys) {
  int64_t mk = 0;
  for (int b = 0; b < B; ++b) {
    if (pos[b] < 0 || pos[b] + n - 1 > kMaxPos) return GQA_ERR_POS_RANGE;
    if (kind == GQA_GLOBAL && pos[b] + n > capacity) return GQA_ERR_POS_RANGE;
    const int64_t k = visible_keys(kind, pos[b] + n - 1);
    if (k > mk) mk = k;
  }
  if (max_keys) *max_keys = mk;
  return GQA_OK;
}

int check_layer(const gqa_layer* L) {
  if (!L || !L->k || !L->v) return GQA_ERR_INVALID_ARG;
  int rc = check_shape(L->kind, L->window, L->capacity, L->rope_theta);
  if (rc != GQA_OK) return rc;
  const int64_t token = (int64_t)GQA_NUM_KV_HEADS * GQA_HEAD_DIM;
  if (L->seq_stride < L->capacity * token) return GQA_ERR_INVALID_ARG;
  if (L->seq_stride % 8 != 0 || !aligned16(L->k) || !aligned16(L->v))
    return GQA_ERR_MISALIGNED;
  return GQA_OK;
}

int check_layer_fp8(const gqa_layer_fp8* L) {
  if (!L || !L->k || !L->v || !L->k_scale || !L->v_scale)
    return GQA_ERR_INVALID_ARG;
  int rc = check_shape(L->kind, L->window, L->capacity, L->rope_theta);
  if (rc != GQA_OK) return rc;
  const int64_t token = (int64_t)GQA_NUM_KV_HEADS * GQA_HEAD_DIM;  // bytes
  if (L->seq_stride < L->capacity * token ||
      L->scale_stride < L->capacity * GQA_NUM_KV_HEADS)
    return GQA_ERR_INVALID_ARG;
  if (L->seq_stride % 16 != 0 || !aligned16(L->k) || !aligned16(L->v) || !aligned16(L->k_scale) ||
      !aligned16(L->v_scale))
    return GQA_ERR_MISALIGNED;
  return GQA_OK;
}

int check_append_fp8(const gqa_layer_fp8* L, const void* k_new,
                     const void* v_new, const int64_t* pos0, int B, int n) {
  if (!k_new || !v_new || !pos0 || B < 1 || B > GQA_MAX_BATCH || n < 1)
    return GQA_ERR_INVALID_ARG;
  int rc = check_layer_fp8(L);
  if (rc != GQA_OK) return rc;
  if (!aligned16(k_new) || !aligned16(v_new)) return GQA_ERR_MISALIGNED;
  return check_positions(L->kind, L->capacity, pos0, B, n, nullptr);
}

int check_decode_fp8(const gqa_layer_fp8* L, const void* q, const int64_t* pos,
                     int B, const float* out, int64_t* max_keys) {
  if (!q || !pos || !out || B < 1 || B > GQA_MAX_BATCH)
    return GQA_ERR_INVALID_ARG;
  int rc = check_layer_fp8(L);
  if (rc != GQA_OK) return rc;
  if (!aligned16(q) || !aligned16(out)) return GQA_ERR_MISALIGNED;
  return check_positions(L->kind, L->capacity, pos, B, 1, max_keys);
}

int check_append(const gqa_layer* L, const void* k_new, const void* v_new,
                 const int64_t* pos0, int B, int n) {
  if (!k_new || !v_new || !pos0 || B < 1 || B > GQA_MAX_BATCH || n < 1)
    return GQA_ERR_INVALID_ARG;
  int rc = check_layer(L);
  if (rc != GQA_OK) return rc;
  if (!aligned16(k_new) || !aligned16(v_new)) return GQA_ERR_MISALIGNED;
  for (int b = 0; b < B; ++b) {
    if (pos0[b] < 0 || pos0[b] + n - 1 > kMaxPos) return GQA_ERR_POS_RANGE;
    if (L->kind == GQA_GLOBAL && pos0[b] + n > L->capacity)
      return GQA_ERR_POS_RANGE;
  }
  return GQA_OK;
}

int check_decode(const gqa_layer* L, const void* q, const int64_t* pos, int B,
                 const float* out, int64_t* max_keys) {
  if (!q || !pos || !out || B < 1 || B > GQA_MAX_BATCH)
    return GQA_ERR_INVALID_ARG;
  int rc = check_layer(L);
  if (rc != GQA_OK) return rc;
  if (!aligned16(q) || !aligned16(out)) return GQA_ERR_MISALIGNED;
  int64_t mk = 0;
  for (int b = 0; b < B; ++b) {
    if (pos[b] < 0 || pos[b] > kMaxPos) return GQA_ERR_POS_RANGE;
    if (L->kind == GQA_GLOBAL && pos[b] >= L->capacity)
      return GQA_ERR_POS_RANGE;
    const int64_t k = visible_keys(L->kind, pos[b]);
    if (k > mk) mk = k;
  }
  *max_keys = mk;
  return GQA_OK;
}

int check_block(const gqa_layer* L, const void* q, const void* k_blk,
                const void* v_blk, const int64_t* pos0, int B, int n,
                const void* out, bool verify, int64_t* max_keys) {
  if (!q || !k_blk || !v_blk || !pos0 || !out || B < 1 || B > GQA_MAX_BATCH ||
      n < 1 || n > (verify ? GQA_MAX_VERIFY : GQA_MAX_CONTEXT))
    return GQA_ERR_INVALID_ARG;
  int rc = check_layer(L);
  if (rc != GQA_OK) return rc;
  if (!aligned16(q) || !aligned16(k_blk) || !aligned16(v_blk) ||
      !aligned16(out))
    return GQA_ERR_MISALIGNED;
  int64_t mk = 0;
  for (int b = 0; b < B; ++b) {
    if (pos0[b] < 0 || pos0[b] + n - 1 > kMaxPos) return GQA_ERR_POS_RANGE;
    if (L->kind == GQA_GLOBAL && pos0[b] + n > L->capacity)
      return GQA_ERR_POS_RANGE;
    const int64_t k = visible_keys(L->kind, pos0[b] + n - 1);
    if (k > mk) mk = k;
  }
  *max_keys = mk;
  return GQA_OK;
}

int check_block_fp8(const gqa_layer_fp8* L, const void* q, const void* k_blk,
                    const void* v_blk, const int64_t* pos0, int B, int n,
                    const void* out, bool verify, int64_t* max_keys) {
  if (!q || !k_blk || !v_blk || !pos0 || !out || B < 1 || B > GQA_MAX_BATCH ||
      n < 1 || n > (verify ? GQA_MAX_VERIFY : GQA_MAX_CONTEXT))
    return GQA_ERR_INVALID_ARG;
  int rc = check_layer_fp8(L);
  if (rc != GQA_OK) return rc;
  if (!aligned16(q) || !aligned16(k_blk) || !aligned16(v_blk) ||
      !aligned16(out))
    return GQA_ERR_MISALIGNED;
  return check_positions(L->kind, L->capacity, pos0, B, n, max_keys);
}

}  // namespace gqa
