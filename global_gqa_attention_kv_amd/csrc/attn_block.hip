// attn_block.hip -- attention for a block of query tokens on bf16 MFMA:
// chunked prefill and speculative verification.
//
// What is computed: n query tokens per sequence at positions p0 .. p0+n-1,
// whose K/V arrive with the call and are not yet in the cache.  Query i sees
// the cached keys before p0 plus the block's own keys up to i (causal inside
// the block); on a local layer only the 2048 positions i-2047 .. i, with
// RoPE on queries and keys; on a global layer every position 0 .. i, no
// RoPE.  Pages: "Tomas Koutsky explains how Meta fits Muse Glimmer into 24
// GB" (runtimewire.com), "Long context still costs compute" (global layers
// run full attention over the prompt, in memory-efficient kernels that never
// store the score matrix; the causal mask carries order); "Deep dive into
// Muse Glimmer" (shishifenxi.com) section 04 and "Meta open-sources the 30B
// Muse Glimmer" (kongchang.com), "Trick 3: D-Flash" (a 16-token drafted
// block verified by the main model in one pass, causal within the block).
//
// Design (gfx950, v_mfma_f32_32x32x16_bf16, fp32 accumulation):
//  * Rows are (query, head) pairs: a workgroup takes QPW query tokens x the
//    16 query heads of one KV head, so every K/V tile staged in LDS serves
//    16 x QPW rows (GQA reuse); each wave owns 32 rows = 2 tokens x 16 heads.
//  * Scores are formed transposed, S^T = K Q^T, so each lane ends up owning
//    one row and 16 keys of every 32-key block: the row maximum is 31 in-lane
//    max operations plus one exchange with the partner lane 32 away, and the
//    probabilities, rounded to bf16, are directly the B operand of the P.V
//    product (O^T = V^T P^T) -- P never goes through LDS.  The contraction's
//    key order inside each 16-key step follows the score layout; V^T is read
//    in that same order.
//  * K tiles sit in LDS row-major (rows padded to 272 B); V tiles are
//    transposed on their way into LDS (rows of 64 keys padded to 136 B, the
//    8-byte units XOR-swizzled by dim/8 against write conflicts) so a lane
//    reads 4 consecutive keys of one dimension with one 8-byte load.
//  * Online softmax in the log2 domain with a lazy maximum (rescale only when
//    a score exceeds the running maximum by more than 2^8); masks are applied
//    only on tiles that cross the causal diagonal or the window edge.
//  * Local layers: a pre-pass rotates the window's cached keys and the
//    block's keys into the workspace once; queries are rotated when loaded.
//    Both use offsets relative to p0 (<R_i q, R_j k> is unchanged by a common
//    shift), keeping the fp32 angle arithmetic small.
//  * Verification splits each sequence's key range across workgroups and
//    merges the partial (m, l, o) rows in a second kernel.
#include <type_traits>

#include "device_common.h"
#include "internal.h"

namespace gqa {

namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));

constexpr float kTauB = 8.0f;
constexpr int kKRow = 272;                  // bytes per key row of a K tile
constexpr int kVRow = 136;                  // bytes per dim row of a V^T tile
constexpr int kKsB = kBlkTile * kKRow;      // 17408
constexpr int kVtB = kD * kVRow;            // 17408
constexpr int kPartRow = 132;               // floats: o[128], m, l, pad

__device__ __forceinline__ uint32_t word(const uint4& v, int e) {
  return e == 0 ? v.x : e == 1 ? v.y : e == 2 ? v.z : v.w;
}

__device__ __forceinline__ int64_t ring_prior(int64_t pos0) {
  return pos0 < kW ? pos0 : kW;
}

// Local layers: write the RoPE-rotated keys of positions p0 - W' .. p0+n-1
// (W' = min(p0, 2048) cached positions before the block) into k_lin, rotated
// by their offset from p0.  One wave per key row (2 heads x 128 dims).
__global__ __launch_bounds__(64) void rope_keys_kernel(const BlockParams p) {
  const int b = blockIdx.y;
  const int r = blockIdx.x;
  const int64_t pos0 = p.pos0[b];
  const int64_t wprior = ring_prior(pos0);
  if (r >= wprior + p.n) return;
  const int64_t j = pos0 - wprior + r;  // key position
  const uint16_t* src =
      j < pos0 ? p.k_cache + (int64_t)b * p.seq_stride +
                     (j & (kW - 1)) * kTokenElems
               : p.k_blk + ((int64_t)b * p.n + (j - pos0)) * kTokenElems;
  const int lane = threadIdx.x;
  const int head = lane >> 5, c = lane & 31;  // dims 2c, 2c+1 and +64
  const uint32_t* s32 = reinterpret_cast<const uint32_t*>(src + head * kD);
  uint32_t x = s32[c], y = s32[c + 32];
  rope_pair(x, y, (float)(j - pos0), p.rope_rev[2 * c], p.rope_rev[2 * c + 1]);
  uint32_t* d32 = reinterpret_cast<uint32_t*>(
      p.k_lin + ((int64_t)b * p.klin_rows + r) * kTokenElems + head * kD);
  d32[c] = x;
  d32[c + 32] = y;
}

// QPW = 8: 256 threads, at least two waves per SIMD (two workgroups per CU);
// QPW = 16: 512 threads, one workgroup per CU.
template <int QPW, bool LOCAL, bool SPLIT, bool OUT_F32>
__global__ __launch_bounds__(QPW * 32, 2) void block_attn_kernel(
    const BlockParams p) {
  constexpr int WAVES = QPW / 2;
  constexpr int NT = WAVES * 64;
  constexpr int ROWS = QPW * kGroup;
  constexpr int KLOADS = kBlkTile * 16 / NT;         // 16-B K chunks/thread
  __shared__ __attribute__((aligned(16))) uint8_t smem[kKsB + kVtB];
  uint8_t* Ks = smem;
  uint8_t* Vt = smem + kKsB;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int hi5 = lane >> 5;
  const int row = lane & 31;

  // workgroup -> (sequence, KV head, query group, key split); query groups
  // with the longest key ranges are dispatched first
  int bid = blockIdx.x;
  const int split = bid % p.splits;
  bid /= p.splits;
  const int qg = p.qgroups - 1 - bid % p.qgroups;
  bid /= p.qgroups;
  const int g = bid % kHkv;
  const int b = bid / kHkv;

  // positions fit in 32 bits (validated on the host)
  const int pos0 = (int)p.pos0[b];
  const int q_first = qg * QPW;
  const int q_last = min(p.n - 1, q_first + QPW - 1);
  const int i_first = pos0 + q_first, i_last = pos0 + q_last;
  const int k_lo = LOCAL ? max(0, i_first - (kW - 1)) : 0;
  const int k_hi = i_last + 1;
  const int tiles_all = (k_hi - k_lo + kBlkTile - 1) / kBlkTile;
  const int tps = (tiles_all + p.splits - 1) / p.splits;
  const int t_begin = split * tps;
  const int ntiles = max(0, min(tiles_all, t_begin + tps) - t_begin);

  // this lane's row: token qi of the block, query head `head`
  const int qi = q_first + 2 * w + (row >> 4);
  const bool row_valid = qi <= q_last;
  const int qic = min(qi, q_last);
  const int head = g * kGroup + (row & 15);
  const int qpos = pos0 + qic;
  const int klin0 = pos0 - (int)ring_prior(pos0);  // position of k_lin row 0

  // ---- Q^T operand: 8 k-steps of 16 dims, this lane's 8 dims of each
  bf16x8_t qreg[8];
  {
    const uint16_t* qrow =
        p.q + (((int64_t)b * p.n + qic) * kHq + head) * kD + 8 * hi5;
    uint4 raw[8];
#pragma unroll
    for (int k = 0; k < 8; ++k)
      raw[k] = *reinterpret_cast<const uint4*>(qrow + 16 * k);
    if (LOCAL) {
      const float delta = (float)qic;
#pragma unroll
      for (int k = 0; k < 4; ++k)
        rope_rotate(raw[k], raw[k + 4], delta, p.rope_rev + 16 * k + 8 * hi5);
    }
#pragma unroll
    for (int k = 0; k < 8; ++k) qreg[k] = __builtin_bit_cast(bf16x8_t, raw[k]);
  }

  const uint16_t* kc_base = p.k_cache + (int64_t)b * p.seq_stride + g * kD;
  const uint16_t* vc_base = p.v_cache + (int64_t)b * p.seq_stride + g * kD;
  const uint16_t* kb_base = p.k_blk + (int64_t)b * p.n * kTokenElems + g * kD;
  const uint16_t* vb_base = p.v_blk + (int64_t)b * p.n * kTokenElems + g * kD;
  const uint16_t* kl_base =
      p.k_lin + (int64_t)b * p.klin_rows * kTokenElems + g * kD;

  auto k_src = [&](int j) -> const uint16_t* {
    if (LOCAL) return kl_base + (j - klin0) * kTokenElems;
    return j < pos0 ? kc_base + j * kTokenElems
                    : kb_base + (j - pos0) * kTokenElems;
  };
  auto v_src = [&](int j) -> const uint16_t* {
    if (j >= pos0) return vb_base + (j - pos0) * kTokenElems;
    return vc_base + (LOCAL ? (j & (kW - 1)) : j) * kTokenElems;
  };

  // V staging unit: KPU consecutive keys x 8 dims (one 16-byte chunk of
  // each key); NT units cover the 64-key tile.
  constexpr int KPU = kBlkTile * 16 / NT;  // 4 (256 threads) or 2 (512)
  // native vectors (not the uint4 struct) so the registers are never copied
  // through private memory
  u32x4_t kreg[KLOADS];
  uint4 vreg[KPU];
  auto load_tile = [&](int t) {
    const int kb = k_lo + (t_begin + t) * kBlkTile;
    static_for<0, KLOADS>([&](auto I) {
      const int u = tid + I * NT;
      const int key = u >> 4, c = u & 15;
      const int j = min(kb + key, k_hi - 1);
      kreg[I] = *reinterpret_cast<const u32x4_t*>(k_src(j) + c * 8);
    });
    const int kq = tid >> 4, c = tid & 15;
    static_for<0, KPU>([&](auto R) {
      const int j = min(kb + KPU * kq + R, k_hi - 1);
      vreg[R] = *reinterpret_cast<const uint4*>(v_src(j) + c * 8);
    });
  };
  auto store_tile = [&]() {
    static_for<0, KLOADS>([&](auto I) {
      const int u = tid + I * NT;
      const int key = u >> 4, c = u & 15;
      *reinterpret_cast<u32x4_t*>(Ks + key * kKRow + c * 16) = kreg[I];
    });
    // V^T rows are stored with the 8-byte (4-key) units XOR-swizzled by
    // (dim / 8): without it the 16 lanes of a write group, which hold dims
    // 8c + e for c = 0..15, would hit only 4 bank groups.
    const int kq = tid >> 4, c = tid & 15;
    static_for<0, 4>([&](auto E) {
      // dims 8c+2e and 8c+2e+1 of keys KPU*kq .. KPU*kq+KPU-1
      const int unit = (KPU * kq) >> 2;          // 8-byte unit of the keys
      const int sub = (KPU * kq) & 3;            // key offset inside it
      uint8_t* even =
          Vt + (8 * c + 2 * E) * kVRow + ((unit ^ c) << 3) + 2 * sub;
      uint8_t* odd = even + kVRow;
      if constexpr (KPU == 4) {
        const uint32_t w0 = word(vreg[0], E), w1 = word(vreg[1], E);
        const uint32_t w2 = word(vreg[2], E), w3 = word(vreg[3], E);
        *reinterpret_cast<uint2*>(even) =
            make_uint2(interleave_lo(w0, w1), interleave_lo(w2, w3));
        *reinterpret_cast<uint2*>(odd) =
            make_uint2(interleave_hi(w0, w1), interleave_hi(w2, w3));
      } else {
        const uint32_t w0 = word(vreg[0], E), w1 = word(vreg[1], E);
        *reinterpret_cast<uint32_t*>(even) = interleave_lo(w0, w1);
        *reinterpret_cast<uint32_t*>(odd) = interleave_hi(w0, w1);
      }
    });
  };

  f32x16_t O[4];
#pragma unroll
  for (int d = 0; d < 4; ++d)
#pragma unroll
    for (int i = 0; i < 16; ++i) O[d][i] = 0.0f;
  float m_run = -INFINITY, l_run = 0.0f;

  if (ntiles > 0) load_tile(0);
  for (int t = 0; t < ntiles; ++t) {
    store_tile();
    __syncthreads();
    if (t + 1 < ntiles) load_tile(t + 1);

    // ---- S^T = K Q^T for two 32-key blocks
    f32x16_t S[2];
#pragma unroll
    for (int be = 0; be < 2; ++be) {
#pragma unroll
      for (int i = 0; i < 16; ++i) S[be][i] = 0.0f;
#pragma unroll
      for (int k = 0; k < 8; ++k) {
        const bf16x8_t a = *reinterpret_cast<const bf16x8_t*>(
            Ks + (32 * be + row) * kKRow + (2 * k + hi5) * 16);
        S[be] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, qreg[k], S[be], 0,
                                                        0, 0);
      }
    }

    // ---- softmax update for this lane's row.  The maximum is taken on raw
    // scores (the scale is positive) and the scale is folded into the
    // exponent: p = 2^(s * scale_log2 - m).
    const int kb = k_lo + (t_begin + t) * kBlkTile;
    const bool edge = (kb + kBlkTile - 1 > i_first) ||
                      (LOCAL && kb <= i_last - kW);
    if (edge) {
      // key kb + off + 4 hi5 is visible iff off <= rel and (local)
      // off > rel - W
      const int rel = qpos - kb - 4 * hi5;
#pragma unroll
      for (int be = 0; be < 2; ++be)
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const int off = 32 * be + 8 * (i >> 2) + (i & 3);
          const bool ok = off <= rel && (!LOCAL || off > rel - kW);
          S[be][i] = ok ? S[be][i] : -INFINITY;
        }
    }
    float mt = -INFINITY;
#pragma unroll
    for (int be = 0; be < 2; ++be)
#pragma unroll
      for (int i = 0; i < 16; ++i) mt = fmaxf(mt, S[be][i]);
    mt = fmaxf(mt, __shfl_xor(mt, 32, 64)) * p.scale_log2;
    if (__any(mt > m_run + kTauB)) {
      const float mn = fmaxf(m_run, mt);
      const float alpha = mn == m_run ? 1.0f : fast_exp2(m_run - mn);
      m_run = mn;
      l_run *= alpha;
#pragma unroll
      for (int d = 0; d < 4; ++d)
#pragma unroll
        for (int i = 0; i < 16; ++i) O[d][i] *= alpha;
    }
    // a row that has seen no visible key yet keeps m = -inf; any finite
    // base then turns its -inf scores into zero weights
    const float mb = m_run == -INFINITY ? 0.0f : m_run;
    bf16x8_t P[4];  // 16-key contraction steps: (block be, half tt)
#pragma unroll
    for (int be = 0; be < 2; ++be)
#pragma unroll
      for (int tt = 0; tt < 2; ++tt) {
        uint32_t w4[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const float p0 =
              fast_exp2(fmaf(S[be][8 * tt + 2 * j], p.scale_log2, -mb));
          const float p1 =
              fast_exp2(fmaf(S[be][8 * tt + 2 * j + 1], p.scale_log2, -mb));
          w4[j] = pack_bf16(p0, p1);
          // the denominator sums exactly the bf16 weights P.V uses
          l_run = dot2_bf16(w4[j], 0x3F803F80u, l_run);
        }
        P[2 * be + tt] = __builtin_bit_cast(
            bf16x8_t, make_uint4(w4[0], w4[1], w4[2], w4[3]));
      }

    // ---- O^T += V^T P^T over four 16-key steps, four 32-dim blocks
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      // keys 16c + 4 hi5 + 0..3 and + 8..11: 8-byte units u0 and u0 + 2
      const int u0 = 4 * c + hi5;
#pragma unroll
      for (int d = 0; d < 4; ++d) {
        const int dim = 32 * d + row, sw = dim >> 3;
        const uint8_t* vr = Vt + dim * kVRow;
        const uint2 lo = *reinterpret_cast<const uint2*>(vr + ((u0 ^ sw) << 3));
        const uint2 hi =
            *reinterpret_cast<const uint2*>(vr + (((u0 + 2) ^ sw) << 3));
        const uint4 a4 = make_uint4(lo.x, lo.y, hi.x, hi.y);
        O[d] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
            __builtin_bit_cast(bf16x8_t, a4), P[c], O[d], 0, 0, 0);
      }
    }
    __syncthreads();
  }

  // ---- epilogue: this lane holds row `row`, dims 32d + 8(i>>2) + 4 hi5 + i&3
  const float l_tot = l_run + __shfl_xor(l_run, 32, 64);
  if constexpr (SPLIT) {
    const int prow = (2 * w + (row >> 4)) * kGroup + (row & 15);
    float* base = p.part +
                  ((((size_t)(b * kHkv + g) * p.qgroups + qg) * p.splits +
                    split) * ROWS + prow) * kPartRow;
#pragma unroll
    for (int d = 0; d < 4; ++d)
#pragma unroll
      for (int ib = 0; ib < 4; ++ib)
        *reinterpret_cast<float4*>(base + 32 * d + 8 * ib + 4 * hi5) =
            make_float4(O[d][4 * ib], O[d][4 * ib + 1], O[d][4 * ib + 2],
                        O[d][4 * ib + 3]);
    if (hi5 == 0) {
      base[kD] = m_run;
      base[kD + 1] = l_tot;
    }
  } else {
    if (!row_valid) return;
    const float inv = 1.0f / l_tot;
    const size_t obase = (((size_t)b * p.n + qi) * kHq + head) * kD;
#pragma unroll
    for (int d = 0; d < 4; ++d)
#pragma unroll
      for (int ib = 0; ib < 4; ++ib) {
        const int dim = 32 * d + 8 * ib + 4 * hi5;
        const float x0 = O[d][4 * ib] * inv, x1 = O[d][4 * ib + 1] * inv;
        const float x2 = O[d][4 * ib + 2] * inv, x3 = O[d][4 * ib + 3] * inv;
        if constexpr (OUT_F32) {
          *reinterpret_cast<float4*>(static_cast<float*>(p.out) + obase + dim) =
              make_float4(x0, x1, x2, x3);
        } else {
          *reinterpret_cast<uint2*>(static_cast<uint16_t*>(p.out) + obase +
                                    dim) =
              make_uint2(pack_bf16(x0, x1), pack_bf16(x2, x3));
        }
      }
  }
}

// Merge the key splits of one (sequence, token, query head, quarter of the
// head dimension): 8 float4 columns x 32 split lanes per workgroup.
template <int QPW, bool OUT_F32>
__global__ __launch_bounds__(256) void block_merge_kernel(const BlockParams p) {
  constexpr int ROWS = QPW * kGroup;
  const int dq = blockIdx.x & 3;
  int rest = blockIdx.x >> 2;
  const int h = rest % kHq;
  rest /= kHq;
  const int qi = rest % p.n;
  const int b = rest / p.n;
  const int g = h / kGroup;
  const int qg = qi / QPW;
  const int prow = (qi - qg * QPW) * kGroup + (h % kGroup);
  const float* base =
      p.part + (((size_t)(b * kHkv + g) * p.qgroups + qg) * p.splits * ROWS +
                prow) * kPartRow;
  const size_t sstride = (size_t)ROWS * kPartRow;
  const int tid = threadIdx.x;
  const int c4 = tid & 7, sl = tid >> 3;
  const int d = dq * 32 + c4 * 4;
  float M = -INFINITY, L = 0.0f;
  float4 O = make_float4(0.0f, 0.0f, 0.0f, 0.0f);
  constexpr int kBatch = 4;
  for (int s0 = sl; s0 < p.splits; s0 += 32 * kBatch) {
    float ms[kBatch], ls[kBatch];
    float4 os[kBatch];
#pragma unroll
    for (int i = 0; i < kBatch; ++i) {
      const int s = s0 + 32 * i;
      const float* ps = base + (size_t)min(s, p.splits - 1) * sstride;
      ms[i] = s < p.splits ? ps[kD] : -INFINITY;
      ls[i] = ps[kD + 1];
      os[i] = *reinterpret_cast<const float4*>(ps + d);
    }
#pragma unroll
    for (int i = 0; i < kBatch; ++i) {
      if (ms[i] == -INFINITY) continue;
      const float mn = fmaxf(M, ms[i]);
      const float a = fast_exp2(M - mn), c = fast_exp2(ms[i] - mn);
      L = L * a + ls[i] * c;
      O.x = O.x * a + os[i].x * c;
      O.y = O.y * a + os[i].y * c;
      O.z = O.z * a + os[i].z * c;
      O.w = O.w * a + os[i].w * c;
      M = mn;
    }
  }
  __shared__ float red[32][8][6];
  red[sl][c4][0] = M;
  red[sl][c4][1] = L;
  red[sl][c4][2] = O.x;
  red[sl][c4][3] = O.y;
  red[sl][c4][4] = O.z;
  red[sl][c4][5] = O.w;
  __syncthreads();
  if (sl != 0) return;
  float Mt = -INFINITY;
  for (int i = 0; i < 32; ++i) Mt = fmaxf(Mt, red[i][c4][0]);
  float Lt = 0.0f, x = 0.0f, y = 0.0f, z = 0.0f, ww = 0.0f;
  for (int i = 0; i < 32; ++i) {
    if (red[i][c4][0] == -INFINITY) continue;
    const float c = fast_exp2(red[i][c4][0] - Mt);
    Lt += red[i][c4][1] * c;
    x += red[i][c4][2] * c;
    y += red[i][c4][3] * c;
    z += red[i][c4][4] * c;
    ww += red[i][c4][5] * c;
  }
  const float inv = 1.0f / Lt;
  const size_t o = (((size_t)b * p.n + qi) * kHq + h) * kD + d;
  if constexpr (OUT_F32) {
    *reinterpret_cast<float4*>(static_cast<float*>(p.out) + o) =
        make_float4(x * inv, y * inv, z * inv, ww * inv);
  } else {
    *reinterpret_cast<uint2*>(static_cast<uint16_t*>(p.out) + o) =
        make_uint2(pack_bf16(x * inv, y * inv), pack_bf16(z * inv, ww * inv));
  }
}

template <int QPW, bool LOCAL, bool OUT_F32>
hipError_t launch_main(const BlockParams& p, int B, hipStream_t s) {
  const dim3 grid(p.splits * p.qgroups * kHkv * B);
  const dim3 block(QPW * 32);
  if (p.splits > 1) {
    hipLaunchKernelGGL((block_attn_kernel<QPW, LOCAL, true, OUT_F32>), grid,
                       block, 0, s, p);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL((block_merge_kernel<QPW, OUT_F32>),
                       dim3(B * p.n * kHq * 4), dim3(256), 0, s, p);
  } else {
    hipLaunchKernelGGL((block_attn_kernel<QPW, LOCAL, false, OUT_F32>), grid,
                       block, 0, s, p);
  }
  return hipGetLastError();
}

}  // namespace

hipError_t launch_block(const BlockParams& p, const BlockPlan& plan,
                        bool local, bool out_f32, int B, hipStream_t s) {
  if (local) {
    hipLaunchKernelGGL(rope_keys_kernel, dim3((unsigned)p.klin_rows, B),
                       dim3(64), 0, s, p);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  if (plan.qpw == 16) {
    if (local)
      return out_f32 ? launch_main<16, true, true>(p, B, s)
                     : launch_main<16, true, false>(p, B, s);
    return out_f32 ? launch_main<16, false, true>(p, B, s)
                   : launch_main<16, false, false>(p, B, s);
  }
  if (local)
    return out_f32 ? launch_main<8, true, true>(p, B, s)
                   : launch_main<8, true, false>(p, B, s);
  return out_f32 ? launch_main<8, false, true>(p, B, s)
                 : launch_main<8, false, false>(p, B, s);
}

}  // namespace gqa
