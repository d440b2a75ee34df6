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

// fp8 cache -> bf16 copy for a prefill chunk over an fp8 cache: 32 threads
// per slot, thread c of K (c < 16) or V takes the 16 codes 16 (c % 8) .. of
// KV head c / 8.  Each code becomes its exact bf16 value, is multiplied by
// its row's scale in fp32 and rounded once to bf16 (the operand rounding the
// bf16 kernels apply to every key they rotate or scale).
__global__ __launch_bounds__(256) void dequant_cache_kernel(
    const DequantParams p) {
  const int b = blockIdx.y;
  const int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const int64_t slot = idx >> 5;
  if (slot >= p.rows[b]) return;
  const int part = (int)(idx & 31);
  const bool is_v = part >= 16;
  const int c = part & 15, g = c >> 3;
  const uint8_t* src = (is_v ? p.v8 : p.k8) + (int64_t)b * p.seq_stride +
                       slot * kTokenElems + c * 16;
  const float sc = (is_v ? p.v_scale : p.k_scale)[(int64_t)b * p.scale_stride +
                                                 g * p.capacity + slot];
  const uint4 raw = *reinterpret_cast<const uint4*>(src);
  const uint32_t w[4] = {raw.x, raw.y, raw.z, raw.w};
  uint32_t o[8];
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    const uint32_t lo = __builtin_bit_cast(
        uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w[e], 1.0f, false));
    const uint32_t hi = __builtin_bit_cast(
        uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w[e], 1.0f, true));
    o[2 * e] = pack_bf16(bf16_lo(lo) * sc, bf16_hi(lo) * sc);
    o[2 * e + 1] = pack_bf16(bf16_lo(hi) * sc, bf16_hi(hi) * sc);
  }
  uint4* dst = reinterpret_cast<uint4*>(
      (is_v ? p.v_out : p.k_out) + (int64_t)b * p.out_stride +
      slot * kTokenElems + c * 16);
  dst[0] = make_uint4(o[0], o[1], o[2], o[3]);
  dst[1] = make_uint4(o[4], o[5], o[6], o[7]);
}

hipError_t launch_dequant_cache(const DequantParams& p, int B,
                                int64_t max_rows, hipStream_t s) {
  if (max_rows <= 0) return hipSuccess;
  hipLaunchKernelGGL(dequant_cache_kernel,
                     dim3((unsigned)((max_rows * 32 + 255) / 256), B),
                     dim3(256), 0, s, p);
  return hipGetLastError();
}

}  // namespace gqa
