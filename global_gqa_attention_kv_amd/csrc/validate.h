// validate.h -- host-side argument checks of the C ABI (plain C++, no HIP).
#pragma once

#include <stddef.h>
#include <stdint.h>

#include "gqa_attn.h"

namespace gqa {

// Visible keys of a query at `pos` on a layer of `kind`.
int64_t visible_keys(int kind, int64_t pos);

int check_layer(const gqa_layer* L);
int check_append(const gqa_layer* L, const void* k_new, const void* v_new,
                 const int64_t* pos0, int B, int n);
// On success *max_keys is the largest visible-key count over the batch.
int check_decode(const gqa_layer* L, const void* q, const int64_t* pos, int B,
                 const float* out, int64_t* max_keys);

// The same for layers whose cache is fp8 codes plus scales.
int check_layer_fp8(const gqa_layer_fp8* L);
int check_append_fp8(const gqa_layer_fp8* L, const void* k_new,
                     const void* v_new, const int64_t* pos0, int B, int n);
int check_decode_fp8(const gqa_layer_fp8* L, const void* q, const int64_t* pos,
                     int B, const float* out, int64_t* max_keys);

// Verification (verify = true, n <= 16) or prefill of a block of n tokens.
// On success *max_keys is the largest key count any query of the call sees.
int check_block(const gqa_layer* L, const void* q, const void* k_blk,
                const void* v_blk, const int64_t* pos0, int B, int n,
                const void* out, bool verify, int64_t* max_keys);
// The same over an fp8 cache.
int check_block_fp8(const gqa_layer_fp8* L, const void* q, const void* k_blk,
                    const void* v_blk, const int64_t* pos0, int B, int n,
                    const void* out, bool verify, int64_t* max_keys);

}  // namespace gqa
