// kv_append.hip -- bit-exact scatter of new K/V tokens into a layer cache.
//
// Global layers keep every position (slot = position); local layers keep a
// ring of 2048 slots (slot = position mod 2048) and reuse stale slots
// cyclically, as the runtimewire.com page "Tomas Koutsky explains how Meta
// fits Muse Glimmer into 24 GB" ("Narrow cache") requires of an engine that
// wants the sliding-window saving.  One token of one cache is 2 heads x 128
// bf16 = 512 B; a wave copies K (lanes 0-31) and V (lanes 32-63) of one token
// with 16-byte loads and stores.
#include "device_common.h"
#include "internal.h"

namespace gqa {

__global__ __launch_bounds__(64) void kv_append_kernel(const AppendParams p) {
  const int lane = threadIdx.x;
  const int b = blockIdx.y;
  const int t = p.first + blockIdx.x;
  const int64_t pos = p.pos0[b] + t;
  const int64_t slot = p.local ? (pos & (kW - 1)) : pos;
  const bool is_v = lane >= 32;
  const int chunk = lane & 31;  // 16-byte chunk of the 512-byte token
  const uint16_t* src = (is_v ? p.v_new : p.k_new) +
                        ((int64_t)b * p.n + t) * kTokenElems + chunk * 8;
  uint16_t* dst = (is_v ? p.v : p.k) + (int64_t)b * p.seq_stride +
                  slot * kTokenElems + chunk * 8;
  *reinterpret_cast<uint4*>(dst) = *reinterpret_cast<const uint4*>(src);
}

hipError_t launch_kv_append(const AppendParams& p, int B, int count,
                            hipStream_t s) {
  hipLaunchKernelGGL(kv_append_kernel, dim3(count, B), dim3(64), 0, s, p);
  return hipGetLastError();
}

// Append to an fp8 cache.  A cache quantised to fewer bits per entry is one
// of the factors the runtimewire.com page ("Narrow cache") names for the
// memory a cache really takes; the format is read as OCP FP8 E4M3 with one
// fp32 scale per (token, KV head) for K and for V: s = amax / 448, code =
// E4M3 round-to-nearest-even of clamp(x / s, -448, 448) (both divisions
// rounded to nearest in fp32), amax = 0 giving s = 0 and zero codes.  One
// wave per token: lanes 0-31 take K, 32-63 V, 16 lanes per KV head with 8
// values (16 bytes of bf16) each; the head's largest magnitude is reduced
// over its 16 lanes.
__global__ __launch_bounds__(64) void kv_append_fp8_kernel(
    const AppendFp8Params p) {
  const int lane = threadIdx.x;
  const int b = blockIdx.y;
  const int t = p.first + blockIdx.x;
  const int64_t pos = p.pos0[b] + t;
  const int64_t slot = p.local ? (pos & (kW - 1)) : pos;
  const bool is_v = lane >= 32;
  const int g = (lane >> 4) & 1;  // KV head
  const int j = lane & 15;        // values 8 j .. 8 j + 7 of the head
  const uint16_t* src = (is_v ? p.v_new : p.k_new) +
                        ((int64_t)b * p.n + t) * kTokenElems + g * kD + j * 8;
  const uint4 raw = *reinterpret_cast<const uint4*>(src);
  const uint32_t w[4] = {raw.x, raw.y, raw.z, raw.w};
  float x[8];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    x[2 * i] = __builtin_bit_cast(float, w[i] << 16);
    x[2 * i + 1] = __builtin_bit_cast(float, w[i] & 0xFFFF0000u);
  }
  float amax = 0.0f;
#pragma unroll
  for (int i = 0; i < 8; ++i) amax = fmaxf(amax, fabsf(x[i]));
  amax = row_max(amax);
  const float scale = __fdiv_rn(amax, 448.0f);
  uint32_t c0 = 0, c1 = 0;
  if (amax > 0.0f) {
    float y[8];
#pragma unroll
    for (int i = 0; i < 8; ++i)
      y[i] = fminf(fmaxf(__fdiv_rn(x[i], scale), -448.0f), 448.0f);
    // two codes per conversion, first value in the lower byte
    c0 = __builtin_amdgcn_cvt_pk_fp8_f32(y[0], y[1], 0, false);
    c0 = __builtin_amdgcn_cvt_pk_fp8_f32(y[2], y[3], c0, true);
    c1 = __builtin_amdgcn_cvt_pk_fp8_f32(y[4], y[5], 0, false);
    c1 = __builtin_amdgcn_cvt_pk_fp8_f32(y[6], y[7], c1, true);
  }
  uint8_t* dst = (is_v ? p.v : p.k) + (int64_t)b * p.seq_stride +
                 slot * (kHkv * kD) + g * kD + j * 8;
  *reinterpret_cast<uint2*>(dst) = make_uint2(c0, c1);
  if (j == 0)
    (is_v ? p.v_scale : p.k_scale)[(int64_t)b * p.scale_stride +
                                   g * p.capacity + slot] = scale;
}

hipError_t launch_kv_append_fp8(const AppendFp8Params& p, int B, int count,
                                hipStream_t s) {
  hipLaunchKernelGGL(kv_append_fp8_kernel, dim3(count, B), dim3(64), 0, s, p);
  return hipGetLastError();
}

}  // namespace gqa
