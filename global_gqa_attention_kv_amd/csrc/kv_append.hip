// kv_append.hip -- bit-exact scatter of new K/V tokens into a layer cache.
//
// Global layers keep every position (slot = position); local layers keep a
// ring of 2048 slots (slot = position mod 2048) and reuse stale slots
// cyclically, as the runtimewire.com page "Tomas Koutsky explains how Meta
// fits Muse Glimmer into 24 GB" ("Narrow cache") requires of an engine that
// wants the sliding-window saving.  One token of one cache is 2 heads x 128
// bf16 = 512 B; a wave copies K (lanes 0-31) and V (lanes 32-63) of one token
// with 16-byte loads and stores.
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

}  // namespace gqa
