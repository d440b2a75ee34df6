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

int check_layer(const gqa_layer* L) {
  if (!L || !L->k || !L->v) return GQA_ERR_INVALID_ARG;
  if (L->kind == GQA_LOCAL) {
    if (L->window != GQA_WINDOW || L->capacity != GQA_WINDOW ||
        !(L->rope_theta > 0.0) || !isfinite(L->rope_theta))
      return GQA_ERR_UNSUPPORTED;
  } else if (L->kind == GQA_GLOBAL) {
    if (L->window != 0 || L->rope_theta != 0.0 || L->capacity < 1 ||
        L->capacity > GQA_MAX_CONTEXT)
      return GQA_ERR_UNSUPPORTED;
  } else {
    return GQA_ERR_UNSUPPORTED;
  }
  const int64_t token = (int64_t)GQA_NUM_KV_HEADS * GQA_HEAD_DIM;
  if (L->seq_stride < L->capacity * token) return GQA_ERR_INVALID_ARG;
  if (L->seq_stride % 8 != 0 || !aligned16(L->k) || !aligned16(L->v))
    return GQA_ERR_MISALIGNED;
  return GQA_OK;
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

}  // namespace gqa
