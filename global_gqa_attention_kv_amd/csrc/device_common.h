// device_common.h -- small device helpers for the gfx950 kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

namespace gqa {

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));

// a.lo*b.lo + a.hi*b.hi + c with bf16 pairs packed in 32-bit words
// (v_dot2_f32_bf16: products exact in fp32, fp32 accumulation).
__device__ __forceinline__ float dot2_bf16(uint32_t a, uint32_t b, float c) {
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, a),
                                         __builtin_bit_cast(bf16x2_t, b), c,
                                         false);
}

// acc += dot2(word broadcast from lane LANE of this lane's 16-lane row of q,
// k).  The DPP row_newbcast operand lets 16 distinct wave-uniform words live
// in one VGPR (replicated in the four rows) instead of SGPRs.  Hazard: none
// of q, k, acc may have been written by either of the two VALU instructions
// before this one (the compiler cannot see that the asm is a DPP op).  The
// callers interleave independent accumulators, so a product's accumulator
// was last written four products earlier; the first product of each
// accumulator (FIRST), whose accumulator was just initialised, carries its
// own two wait states.  A host test checks the generated code.
// The sixteen products of one 16-byte K chunk against four query heads, as
// one asm block: for pair p = 0..3 of chunk C (k word k[p], query word q[p])
// and head h, a[h] += dot2(q[p] broadcast from lane h LPH + (4C + p) / PPL of
// the row, k[p]).  The compiler puts a wait state between consecutive asm
// blocks (it cannot see what they hold), so fewer, larger blocks issue fewer
// of them.  Inside the block a product's accumulator was written four
// products earlier; FIRST adds two wait states for accumulators that were
// just initialised.
#define GQA_DOT1(A, Q, K, L)                                            \
  "v_dot2c_f32_bf16_dpp %" #A ", %" #Q ", %" #K " row_newbcast:%" #L \
  " row_mask:0xf bank_mask:0xf\n\t"
#define GQA_DOT16                                                       \
  GQA_DOT1(0, 4, 8, 12) GQA_DOT1(1, 4, 8, 13) GQA_DOT1(2, 4, 8, 14)   \
  GQA_DOT1(3, 4, 8, 15) GQA_DOT1(0, 5, 9, 16) GQA_DOT1(1, 5, 9, 17)   \
  GQA_DOT1(2, 5, 9, 18) GQA_DOT1(3, 5, 9, 19) GQA_DOT1(0, 6, 10, 20)  \
  GQA_DOT1(1, 6, 10, 21) GQA_DOT1(2, 6, 10, 22) GQA_DOT1(3, 6, 10, 23) \
  GQA_DOT1(0, 7, 11, 24) GQA_DOT1(1, 7, 11, 25) GQA_DOT1(2, 7, 11, 26) \
  GQA_DOT1(3, 7, 11, 27)
#define GQA_LANE(P, H) "i"((H) * LPH + (4 * C + (P)) / PPL)
#define GQA_DOT16_OPERANDS                                              \
  : "+v"(a[0]), "+v"(a[1]), "+v"(a[2]), "+v"(a[3])                      \
  : "v"(q[0]), "v"(q[1]), "v"(q[2]), "v"(q[3]), "v"(k[0]), "v"(k[1]),  \
    "v"(k[2]), "v"(k[3]), GQA_LANE(0, 0), GQA_LANE(0, 1), GQA_LANE(0, 2), \
    GQA_LANE(0, 3), GQA_LANE(1, 0), GQA_LANE(1, 1), GQA_LANE(1, 2),      \
    GQA_LANE(1, 3), GQA_LANE(2, 0), GQA_LANE(2, 1), GQA_LANE(2, 2),      \
    GQA_LANE(2, 3), GQA_LANE(3, 0), GQA_LANE(3, 1), GQA_LANE(3, 2),      \
    GQA_LANE(3, 3)
template <int LPH, int PPL, int C, bool FIRST>
__device__ __forceinline__ void dot2_bf16_bcast16(const uint32_t (&q)[4],
                                                  const uint32_t (&k)[4],
                                                  float (&a)[4]) {
  if constexpr (FIRST)
    asm("s_nop 1\n\t" GQA_DOT16 GQA_DOT16_OPERANDS);
  else
    asm(GQA_DOT16 GQA_DOT16_OPERANDS);
}
#undef GQA_DOT16_OPERANDS
#undef GQA_LANE
#undef GQA_DOT16
#undef GQA_DOT1

template <int LANE, bool FIRST = false>
__device__ __forceinline__ float dot2_bf16_bcast(uint32_t q, uint32_t k,
                                                 float acc) {
  if constexpr (FIRST)
    asm("s_nop 1\n\t"
        "v_dot2c_f32_bf16_dpp %0, %1, %2 row_newbcast:%3 row_mask:0xf "
        "bank_mask:0xf"
        : "+v"(acc)
        : "v"(q), "v"(k), "i"(LANE));
  else
    asm("v_dot2c_f32_bf16_dpp %0, %1, %2 row_newbcast:%3 row_mask:0xf "
        "bank_mask:0xf"
        : "+v"(acc)
        : "v"(q), "v"(k), "i"(LANE));
  return acc;
}

// The result of a DPP product is not ready for a plain VALU read two wait
// states later (measured: the last product of a chain was lost when its
// accumulator was summed that soon).  A chain of products updates each
// accumulator four instructions apart, which holds; after the chain's last
// product, this puts five wait states before any other use of the four
// accumulators.  The operands tie the wait to them, so the compiler cannot
// move their readers above it.  A host test checks the generated code.
__device__ __forceinline__ void dpp_settle(float& a, float& b, float& c,
                                           float& d) {
  asm volatile("s_nop 4" : "+v"(a), "+v"(b), "+v"(c), "+v"(d));
}

// Calls f(I) for I = 0 .. N-1 with I a compile-time constant.
template <int I, int N, typename F>
__device__ __forceinline__ void static_for(F&& f) {
  if constexpr (I < N) {
    f(std::integral_constant<int, I>{});
    static_for<I + 1, N>(f);
  }
}

__device__ __forceinline__ float bf16_lo(uint32_t w) {
  return __builtin_bit_cast(float, w << 16);
}
__device__ __forceinline__ float bf16_hi(uint32_t w) {
  return __builtin_bit_cast(float, w & 0xFFFF0000u);
}

// Two floats -> packed bf16 pair, round to nearest even.
__device__ __forceinline__ uint32_t pack_bf16(float lo, float hi) {
  bf16x2_t r = {(__bf16)lo, (__bf16)hi};
  return __builtin_bit_cast(uint32_t, r);
}

__device__ __forceinline__ uint16_t to_bf16(float x) {
  return __builtin_bit_cast(uint16_t, (__bf16)x);
}

__device__ __forceinline__ float fast_exp2(float x) {
  return __builtin_amdgcn_exp2f(x);
}

// sin and cos of 2*pi*r for |r| <= 0.5 (v_sin_f32 / v_cos_f32 take their
// argument in revolutions).
__device__ __forceinline__ void sincos_rev(float r, float* s, float* c) {
  *s = __builtin_amdgcn_sinf(r);
  *c = __builtin_amdgcn_cosf(r);
}

// Cross-lane reductions with no LDS round trip (a ds_bpermute costs an LDS
// latency per step): DPP moves inside each 16-lane row -- quad swaps, the
// half-row mirror (lane i <-> 7 - i of each 8), the row mirror (i <-> 15 - i)
// and the rotation by 8 (i <-> i ^ 8) -- and gfx950's v_permlane16_swap /
// v_permlane32_swap across rows, which hand both lanes of a pair (l, l ^ 16
// or l, l ^ 32) the pair's two values in the same order.  Each step combines
// two lanes of equal coverage with a commutative operation, so every lane
// of the reduced group ends with the same bits.
template <int CTRL>
__device__ __forceinline__ float dpp_mov(float x) {
  return __builtin_bit_cast(
      float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, x), CTRL, 0xF,
                                      0xF, false));
}
// The swaps are written in assembly: this compiler's builtins for them hand
// back one of the two results twice when both are combined (an add of the
// pair came out as one register added to itself).  Two wait states separate
// the last VALU write of an operand from the swap.
// every lane l gets the values of lanes l & ~16 and l | 16
__device__ __forceinline__ void xchg16(uint32_t& lo, uint32_t& hi) {
  asm volatile("s_nop 1\n\tv_permlane16_swap_b32 %0, %1" : "+v"(lo), "+v"(hi));
}
// every lane l gets the values of lanes l & ~32 and l | 32
__device__ __forceinline__ void xchg32(uint32_t& lo, uint32_t& hi) {
  asm volatile("s_nop 1\n\tv_permlane32_swap_b32 %0, %1" : "+v"(lo), "+v"(hi));
}
template <int STRIDE>
__device__ __forceinline__ float xmax(float x) {
  uint32_t a = __builtin_bit_cast(uint32_t, x), b = a;
  if constexpr (STRIDE == 16) xchg16(a, b); else xchg32(a, b);
  return fmaxf(__builtin_bit_cast(float, a), __builtin_bit_cast(float, b));
}
template <int STRIDE>
__device__ __forceinline__ float xsum(float x) {
  uint32_t a = __builtin_bit_cast(uint32_t, x), b = a;
  if constexpr (STRIDE == 16) xchg16(a, b); else xchg32(a, b);
  return __builtin_bit_cast(float, a) + __builtin_bit_cast(float, b);
}
// over the 16 lanes of each row
__device__ __forceinline__ float row_max(float x) {
  x = fmaxf(x, dpp_mov<0xB1>(x));   // quad_perm [1, 0, 3, 2]
  x = fmaxf(x, dpp_mov<0x4E>(x));   // quad_perm [2, 3, 0, 1]
  x = fmaxf(x, dpp_mov<0x141>(x));  // row_half_mirror
  return fmaxf(x, dpp_mov<0x140>(x));  // row_mirror
}
__device__ __forceinline__ float row_sum(float x) {
  x += dpp_mov<0xB1>(x);
  x += dpp_mov<0x4E>(x);
  x += dpp_mov<0x141>(x);
  return x + dpp_mov<0x140>(x);
}
// over lanes l, l ^ 16, l ^ 32, l ^ 48
__device__ __forceinline__ float rows_sum(float x) {
  return xsum<32>(xsum<16>(x));
}
// over lanes l, l ^ 8, l ^ 16, ..., l ^ 56 (same l % 8)
__device__ __forceinline__ float stride8_sum(float x) {
  return rows_sum(x + dpp_mov<0x128>(x));  // row_ror:8
}
// over the 64 lanes
__device__ __forceinline__ float wave_max(float x) {
  return xmax<32>(xmax<16>(row_max(x)));
}
__device__ __forceinline__ float wave_sum(float x) {
  return rows_sum(row_sum(x));
}

}  // namespace gqa
