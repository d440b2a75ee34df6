// decode.hip -- split-K flash-decode for one query token per sequence.
//
// What is computed (pages "Deep dive into Muse Glimmer", shishifenxi.com,
// section 01, and "Tomas Koutsky explains how Meta fits Muse Glimmer into
// 24 GB", runtimewire.com, "Narrow cache" / "Long context still costs
// compute"): for each sequence b and query head h, softmax(q.k_j / sqrt(128))
// weighted sum of v_j over the visible keys of KV head h/16 -- all positions
// 0..p on a global layer, positions p-2047..p through the 2048-slot ring with
// RoPE on a local layer.
//
// Design (gfx950, VALU; decode is a streaming read of the cache):
//  * A workgroup owns one (sequence, KV head, key split) and serves query
//    heads of that KV head out of the same tiles, so each cached K/V byte is
//    fetched from HBM once per workgroup that needs it.
//  * Keys stream through LDS in tiles of 64.  K rows sit with an XOR swizzle
//    of their 16-byte chunks so a lane can read a whole row without bank
//    conflicts.
//  * Q.K: lane = key; the query words are wave-uniform, held 16 to a VGPR
//    and broadcast with DPP row_newbcast into v_dot2c_f32_bf16 (bf16
//    products exact, fp32 accumulation).
//  * Online softmax in the log2 domain with a lazy maximum: the running
//    maximum is only raised (and the accumulators rescaled) when some score
//    exceeds it by more than 2^8, which keeps every exponent <= 2^8 while
//    skipping nearly all cross-lane reductions.  The denominator sums exactly
//    the bf16 weights the P.V product uses.
//  * P.V: P goes to wave-private LDS as bf16 key pairs; each lane
//    accumulates 8 dimensions of its wave's heads over a quarter of the
//    tile's key pairs with the packed-pair dot; the quarters are summed at
//    the end.
//  * Each workgroup writes (m, l, o) for its split; the splits are merged
//    with the log-sum-exp rule.
//  * Optionally the call appends the query's own K/V: the kernel reads that
//    key from the new-token buffers and one workgroup stores it to its slot,
//    saving a separate append launch per layer.
//
// Two kernels:
//  * decode_wide_kernel (global layers, long caches): all 16 heads per
//    workgroup (4 per wave), direct-to-LDS tile loads into a two-slot ring,
//    V read back transposed (see the kernel); a second kernel merges.
//  * decode_kernel (local layers, 2048-key windows, latency-bound): 4 heads
//    per workgroup (one per wave), one or two tiles per workgroup; tiles are
//    staged through VGPRs so each key is rotated by its offset to the query
//    (j - i) on its way into LDS -- <R_i q, R_j k> = <q, R_{j-i} k>, so the
//    query stays unrotated and the angles stay small (|j - i| < 2048; fp32
//    angle error ~1e-4 rad) -- and V is re-packed into (key 2i, key 2i+1)
//    pairs.  The four head groups of a tile are placed on one XCD so they
//    share its L2, and the last workgroup of each (sequence, KV head, head
//    group), found with a device-scope counter in the workspace, merges the
//    splits in the same launch.  The partials travel with device-scope
//    (write-through) stores and loads, so no workgroup has to write back its
//    whole L2.
#include "device_common.h"
#include "internal.h"

namespace gqa {

namespace {

typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
constexpr float kTau = 8.0f;  // lazy-rescale threshold in log2 units
constexpr int kKsBytes = kDecTile * 256;        // 64 rows x 256 B
constexpr int kVsBytes = (kDecTile / 2) * 512;  // 32 key pairs x 128 words

__device__ __forceinline__ int64_t slot_of(int64_t position, bool local) {
  return local ? (position & (kW - 1)) : position;
}

template <bool LOCAL, int HW, bool FUSED>
__global__ __launch_bounds__(kDecThreads) void decode_kernel(
    const DecodeParams p) {
  constexpr int HG = 4 / HW;              // head groups per KV head
  constexpr int HPW = 4 * HW;             // query heads per workgroup
  constexpr int PF = HPW * (kD + 2);      // floats of one partial
  constexpr int kPsWave = (kDecTile / 2) * HW * 4;
  __shared__ __attribute__((aligned(16)))
  uint8_t smem[kKsBytes + kVsBytes + 4 * kPsWave];
  __shared__ int s_ticket;
  uint8_t* Ks = smem;
  uint8_t* Vs = smem + kKsBytes;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  uint8_t* Ps = smem + kKsBytes + kVsBytes + w * kPsWave;

  // workgroup -> (unit, head group).  Consecutive workgroup ids go to
  // different XCDs round-robin, so the HG workgroups of one unit are placed
  // 8 ids apart: same XCD, same L2, dispatched together.
  int unit, hg;
  if (HG == 1) {
    unit = blockIdx.x;
    hg = 0;
  } else {
    const int r = blockIdx.x % (8 * HG);
    unit = (blockIdx.x / (8 * HG)) * 8 + (r & 7);
    hg = r >> 3;
  }
  if (unit >= p.units) return;  // padding of the XCD-aware grid
  const int split = unit % p.splits;
  const int bg = unit / p.splits;  // b * 2 + g
  const int g = bg % kHkv;
  const int b = bg / kHkv;

  const int64_t pos = p.pos[b];
  const int64_t j_first = LOCAL ? (pos > kW - 1 ? pos - (kW - 1) : 0) : 0;
  const int nkeys = (int)(pos - j_first + 1);
  const int span = p.tiles_per_split * kDecTile;
  const int k_begin = split * span;
  const int k_end = min(nkeys, k_begin + span);
  const bool has_keys = k_begin < nkeys;
  const int new_key = nkeys - 1;          // key index of the query's own token
  const bool use_new = p.k_new != nullptr;
  float* const part_base = p.part + (size_t)(bg * HG + hg) * p.splits * PF;
  float* const part = part_base + (size_t)split * PF;

  // The call appends the query's own token: one workgroup writes it to its
  // slot, which no other workgroup reads in this launch (they take that key
  // from k_new / v_new).
  if (use_new && g == 0 && hg == 0 && has_keys && new_key / span == split &&
      tid < 64) {
    const bool is_v = tid >= 32;
    const int chunk = tid & 31;
    const uint16_t* src = (is_v ? p.v_new : p.k_new) +
                          (int64_t)b * kTokenElems + chunk * 8;
    uint16_t* dst = (is_v ? p.v_mut : p.k_mut) + (int64_t)b * p.seq_stride +
                    slot_of(pos, LOCAL) * kTokenElems + chunk * 8;
    *reinterpret_cast<uint4*>(dst) = *reinterpret_cast<const uint4*>(src);
  }

  if (has_keys) {
    const int ntiles = (k_end - k_begin + kDecTile - 1) / kDecTile;
    const uint16_t* Kb = p.k + (int64_t)b * p.seq_stride + g * kD;
    const uint16_t* Vb = p.v + (int64_t)b * p.seq_stride + g * kD;
    const uint16_t* Kn = p.k_new + (int64_t)b * kTokenElems + g * kD;
    const uint16_t* Vn = p.v_new + (int64_t)b * kTokenElems + g * kD;
    const int head0 = g * kGroup + hg * HPW + w * HW;  // this wave's heads
    // The wave's HW query rows (64 bf16 pairs each) held as wave-uniform
    // words for the DPP broadcast: within every 16-lane row, lane n keeps
    // pairs (n % LPH) * PPL .. + PPL - 1 of head n / LPH in qv[0 .. PPL).
    constexpr int LPH = 16 / HW;       // lanes per head
    constexpr int PPL = 4 * HW;        // pairs per lane = VGPRs used
    uint32_t qv[PPL];
    {
      const int n = lane & 15;
      const uint32_t* src = p.q +
                            ((int64_t)b * kHq + head0 + n / LPH) * (kD / 2) +
                            (n % LPH) * PPL;
#pragma unroll
      for (int v = 0; v < PPL; v += 4) {
        const uint4 w4 = *reinterpret_cast<const uint4*>(src + v);
        qv[v] = w4.x;
        qv[v + 1] = w4.y;
        qv[v + 2] = w4.z;
        qv[v + 3] = w4.w;
      }
    }

    uint4 kreg[2][2];  // [unit][dims 8c..8c+7 | 8c+64..8c+71]
    uint4 vreg[2][2];  // [unit][key 2r | key 2r+1]

    auto key_row = [&](const uint16_t* base, const uint16_t* fresh, int key) {
      return (use_new && key == new_key)
                 ? fresh
                 : base + slot_of(j_first + key, LOCAL) * kTokenElems;
    };
    auto load_tile = [&](int t) {
      const int kb = k_begin + t * kDecTile;
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        const int u = tid + i * kDecThreads;
        const int row = u >> 3, cp = u & 7;
        const int key = min(kb + row, k_end - 1);
        const uint16_t* src = key_row(Kb, Kn, key) + cp * 8;
        kreg[i][0] = *reinterpret_cast<const uint4*>(src);
        kreg[i][1] = *reinterpret_cast<const uint4*>(src + 64);
      }
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        const int u = tid + i * kDecThreads;
        const int rp = u >> 4, c = u & 15;
        const int ka = min(kb + 2 * rp, k_end - 1);
        const int kc = min(kb + 2 * rp + 1, k_end - 1);
        vreg[i][0] =
            *reinterpret_cast<const uint4*>(key_row(Vb, Vn, ka) + c * 8);
        vreg[i][1] =
            *reinterpret_cast<const uint4*>(key_row(Vb, Vn, kc) + c * 8);
      }
    };

    auto store_tile = [&](int t) {
      const int kb = k_begin + t * kDecTile;
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        const int u = tid + i * kDecThreads;
        const int row = u >> 3, cp = u & 7;
        uint4 lo = kreg[i][0], hi = kreg[i][1];
        if (LOCAL) {
          const int key = min(kb + row, k_end - 1);
          rope_rotate(lo, hi, (float)(j_first + key - pos),
                      p.rope_rev + cp * 8);
        }
        *reinterpret_cast<uint4*>(Ks + row * 256 + ((cp ^ (row & 15)) << 4)) =
            lo;
        *reinterpret_cast<uint4*>(Ks + row * 256 +
                                  (((cp + 8) ^ (row & 15)) << 4)) = hi;
      }
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        const int u = tid + i * kDecThreads;
        const int rp = u >> 4, c = u & 15;
        const uint4 a = vreg[i][0], e = vreg[i][1];
        uint4 o0, o1;
        o0.x = interleave_lo(a.x, e.x);
        o0.y = interleave_hi(a.x, e.x);
        o0.z = interleave_lo(a.y, e.y);
        o0.w = interleave_hi(a.y, e.y);
        o1.x = interleave_lo(a.z, e.z);
        o1.y = interleave_hi(a.z, e.z);
        o1.z = interleave_lo(a.w, e.w);
        o1.w = interleave_hi(a.w, e.w);
        *reinterpret_cast<uint4*>(Vs + rp * 512 + c * 32) = o0;
        *reinterpret_cast<uint4*>(Vs + rp * 512 + c * 32 + 16) = o1;
      }
    };

    float m[HW], lsum[HW], o[HW][8];
#pragma unroll
    for (int hl = 0; hl < HW; ++hl) {
      m[hl] = -INFINITY;
      lsum[hl] = 0.0f;
#pragma unroll
      for (int e = 0; e < 8; ++e) o[hl][e] = 0.0f;
    }
    const int dg = lane & 15, kg = lane >> 4;

    load_tile(0);
    for (int t = 0; t < ntiles; ++t) {
      store_tile(t);
      __syncthreads();
      if (t + 1 < ntiles) load_tile(t + 1);

      // ---- scores: lane = key of this tile, HW heads per wave; the query
      // word of (head hl, pair p) is broadcast from lane hl*LPH + p/PPL.
      // The lane's K row is read from LDS in 4 batches of 64 B, one batch
      // ahead of the products; consecutive products alternate between
      // heads so no product waits on the previous one's accumulator.
      // A DPP instruction must not read (in any operand) a VGPR written by
      // either of the two VALU instructions before it: every head keeps
      // NACC partial sums, so consecutive products always update different
      // accumulators, four instructions apart.
      constexpr int NACC = 4 / HW;
      float acc[HW][NACC];
#pragma unroll
      for (int hl = 0; hl < HW; ++hl)
#pragma unroll
        for (int a = 0; a < NACC; ++a) acc[hl][a] = 0.0f;
      const uint8_t* krow = Ks + lane * 256;
      u32x4_t kbuf[2][4];
      auto read_batch = [&](auto Bt, u32x4_t(&dst)[4]) {
        static_for<0, 4>([&](auto J) {
          constexpr int C = 4 * Bt + J;
          dst[J] = *reinterpret_cast<const u32x4_t*>(
              krow + ((C ^ (lane & 15)) << 4));
        });
      };
      read_batch(std::integral_constant<int, 0>{}, kbuf[0]);
      static_for<0, 4>([&](auto Bt) {
        if constexpr (Bt + 1 < 4)
          read_batch(std::integral_constant<int, Bt + 1>{},
                     kbuf[(Bt + 1) & 1]);
        static_for<0, 4>([&](auto J) {
          constexpr int C = 4 * Bt + J;
          static_for<0, 4>([&](auto I) {
            constexpr int pr = 4 * C + I;
            static_for<0, HW>([&](auto HL) {
              constexpr int ii = I, bb = Bt & 1, jj = J, hh = HL;
              acc[hh][ii % NACC] =
                  dot2_bf16_bcast<HL * LPH + pr / PPL, (C == 0 && ii < NACC)>(
                      qv[pr % PPL], kbuf[bb][jj][ii], acc[hh][ii % NACC]);
            });
          });
        });
      });
      const bool valid = k_begin + t * kDecTile + lane < k_end;
      float s2[HW];
      bool need = false;
#pragma unroll
      for (int hl = 0; hl < HW; ++hl) {
        float a = acc[hl][0];
#pragma unroll
        for (int k = 1; k < NACC; ++k) a += acc[hl][k];
        s2[hl] = valid ? a * p.scale_log2 : -INFINITY;
        need |= s2[hl] > m[hl] + kTau;
      }
      if (__any(need)) {  // wave-uniform: raise the running maximum
#pragma unroll
        for (int hl = 0; hl < HW; ++hl) {
          const float mn = fmaxf(m[hl], wave_max(s2[hl]));
          const float alpha = fast_exp2(m[hl] - mn);
          m[hl] = mn;
          lsum[hl] *= alpha;
#pragma unroll
          for (int e = 0; e < 8; ++e) o[hl][e] *= alpha;
        }
      }
      uint16_t* P16 = reinterpret_cast<uint16_t*>(Ps);
#pragma unroll
      for (int hl = 0; hl < HW; ++hl) {
        // the denominator sums exactly the bf16 weights the P.V product
        // uses, so the weights of every output sum to one
        const uint16_t pb = to_bf16(fast_exp2(s2[hl] - m[hl]));
        lsum[hl] += __builtin_bit_cast(float, (uint32_t)pb << 16);
        P16[(lane >> 1) * (2 * HW) + hl * 2 + (lane & 1)] = pb;
      }
      __builtin_amdgcn_s_waitcnt(0xc07f);  // lgkmcnt(0): P visible to the wave
      __builtin_amdgcn_wave_barrier();

      // ---- P.V: lane = (8 dims, key-pair group)
#pragma unroll
      for (int i = 0; i < kDecTile / 8; ++i) {
        const int kp = kg + 4 * i;
        uint32_t pw[HW];
        if constexpr (HW == 4) {
          const uint4 pp = *reinterpret_cast<const uint4*>(Ps + kp * 16);
          pw[0] = pp.x;
          pw[1] = pp.y;
          pw[2] = pp.z;
          pw[3] = pp.w;
        } else {
#pragma unroll
          for (int hl = 0; hl < HW; ++hl)
            pw[hl] = *reinterpret_cast<const uint32_t*>(Ps + (kp * HW + hl) * 4);
        }
        const uint4 va =
            *reinterpret_cast<const uint4*>(Vs + kp * 512 + dg * 32);
        const uint4 vb =
            *reinterpret_cast<const uint4*>(Vs + kp * 512 + dg * 32 + 16);
        const uint32_t vw[8] = {va.x, va.y, va.z, va.w,
                                vb.x, vb.y, vb.z, vb.w};
#pragma unroll
        for (int hl = 0; hl < HW; ++hl)
#pragma unroll
          for (int e = 0; e < 8; ++e)
            o[hl][e] = dot2_bf16(pw[hl], vw[e], o[hl][e]);
      }
      __syncthreads();
    }

    // ---- reduce over the 4 key-pair groups and the 64 key lanes, write
#pragma unroll
    for (int hl = 0; hl < HW; ++hl) {
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        o[hl][e] += __shfl_xor(o[hl][e], 16, 64);
        o[hl][e] += __shfl_xor(o[hl][e], 32, 64);
      }
      lsum[hl] = wave_sum(lsum[hl]);
    }
    if (kg == 0) {
#pragma unroll
      for (int hl = 0; hl < HW; ++hl) {
        float* dst = part + 2 * HPW + (w * HW + hl) * kD + dg * 8;
        if constexpr (FUSED) {
#pragma unroll
          for (int e = 0; e < 8; ++e) store_dev(dst + e, o[hl][e]);
        } else {
          float4* d4 = reinterpret_cast<float4*>(dst);
          d4[0] = make_float4(o[hl][0], o[hl][1], o[hl][2], o[hl][3]);
          d4[1] = make_float4(o[hl][4], o[hl][5], o[hl][6], o[hl][7]);
        }
      }
    }
    if (lane == 0) {
#pragma unroll
      for (int hl = 0; hl < HW; ++hl) {
        if constexpr (FUSED) {
          store_dev(part + w * HW + hl, m[hl]);
          store_dev(part + HPW + w * HW + hl, lsum[hl]);
        } else {
          part[w * HW + hl] = m[hl];
          part[HPW + w * HW + hl] = lsum[hl];
        }
      }
    }
  } else {
    // a split past this sequence's keys contributes nothing
    for (int i = tid; i < PF; i += kDecThreads) {
      const float x = i < HPW ? -INFINITY : 0.0f;
      if constexpr (FUSED)
        store_dev(part + i, x);
      else
        part[i] = x;
    }
  }

  if constexpr (FUSED) {
  // ---- the last workgroup of this (sequence, KV head, head group) merges.
  // The partial went out with device-scope stores; once they have completed
  // the counter is bumped (device scope), and the workgroup that takes the
  // last ticket reads every partial with device-scope loads.
  wait_vmem();
  __syncthreads();
  if (tid == 0)
    s_ticket = __hip_atomic_fetch_add(&p.counters[bg * HG + hg], 1,
                                      __ATOMIC_RELAXED,
                                      __HIP_MEMORY_SCOPE_AGENT);
  __syncthreads();
  if (s_ticket != p.splits - 1) return;

  static_assert(HPW * kD / 4 == 128, "fused merge covers 4 heads");
  const int f = tid & 127;            // float4 of the 4 x 128 outputs
  const int half = tid >> 7;          // splits s = half, half + 2, ...
  const int hl = f >> 5, d4 = f & 31;
  float M = -INFINITY, L = 0.0f;
  float4 O = make_float4(0.0f, 0.0f, 0.0f, 0.0f);
  constexpr int kBatch = 16;  // up to 32 splits: every load in one batch
  for (int s0 = half; s0 < p.splits; s0 += 2 * kBatch) {
    float ms[kBatch], ls[kBatch];
    float4 os[kBatch];
#pragma unroll
    for (int i = 0; i < kBatch; ++i) {
      const int s = s0 + 2 * i;
      const float* ps = part_base + (size_t)min(s, p.splits - 1) * PF;
      const float* po = ps + 2 * HPW + hl * kD + d4 * 4;
      ms[i] = s < p.splits ? load_dev(ps + hl) : -INFINITY;
      ls[i] = load_dev(ps + HPW + hl);
      os[i] = make_float4(load_dev(po), load_dev(po + 1), load_dev(po + 2),
                          load_dev(po + 3));
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
  // combine the two halves through LDS
  float* red = reinterpret_cast<float*>(smem);
  if (half == 1) {
    red[f * 6 + 0] = M;
    red[f * 6 + 1] = L;
    red[f * 6 + 2] = O.x;
    red[f * 6 + 3] = O.y;
    red[f * 6 + 4] = O.z;
    red[f * 6 + 5] = O.w;
  }
  __syncthreads();
  if (half == 0) {
    const float M2 = red[f * 6 + 0];
    const float mn = fmaxf(M, M2);
    const float a = M == -INFINITY ? 0.0f : fast_exp2(M - mn);
    const float c = M2 == -INFINITY ? 0.0f : fast_exp2(M2 - mn);
    const float Lt = L * a + red[f * 6 + 1] * c;
    const float inv = 1.0f / Lt;
    float4 r;
    r.x = (O.x * a + red[f * 6 + 2] * c) * inv;
    r.y = (O.y * a + red[f * 6 + 3] * c) * inv;
    r.z = (O.z * a + red[f * 6 + 4] * c) * inv;
    r.w = (O.w * a + red[f * 6 + 5] * c) * inv;
    const int h = g * kGroup + hg * HPW + hl;
    *reinterpret_cast<float4*>(p.out + ((size_t)b * kHq + h) * kD + d4 * 4) = r;
    if (tid == 0)  // ready for the next call
      __hip_atomic_store(&p.counters[bg * HG + hg], 0, __ATOMIC_RELAXED,
                         __HIP_MEMORY_SCOPE_AGENT);
  }
  }  // FUSED
}

// ---------------------------------------------------------------------------
// Wide shape (global layers): a workgroup serves all 16 query heads of its KV
// head (4 per wave) over a long key split; two workgroups share a CU.  The
// tiles go straight from HBM into a two-slot LDS ring with direct-to-LDS
// loads (global_load_lds_dwordx4: the 16 bytes of lane l land at the wave's
// LDS base + 16 l, never passing through VGPRs), marked non-temporal since
// the cache is streamed once per step; tile t + 1 is in flight while tile t
// is consumed.
//  * K rows keep the narrow shape's layout: 16-byte chunk c of key row r sits
//    at chunk slot c ^ (r & 15) (the lane that fills slot s fetches chunk
//    s ^ (r & 15)), so lane = key reads its whole row conflict-free.
//  * V rows stay in key order with chunk c at slot c ^ 2(r & 7).  The P.V
//    operands are read with ds_read_b64_tr_b16, which gives each lane four
//    consecutive keys of one dimension: two key-interleaved bf16 pairs, the
//    operand v_dot2_f32_bf16 wants, with no VALU re-packing.  The XOR puts
//    the eight keys read by each 32-lane half on different banks.
//  * P.V lanes: lane 16 g + j owns dimensions j, j + 16, ..., j + 112 of its
//    wave's 4 heads and keys 16 q + 4 g .. + 3 of each 16-key quarter q; the
//    four groups g are summed at the end.
//  * The tile loop is unrolled twice so every LDS address is a per-lane
//    register plus a constant.
constexpr int kTileBytes = kDecTile * 256;    // one 64-key tile of K or V
constexpr int kSlotBytes = 2 * kTileBytes;    // K tile, then V tile

typedef short v4i16_t __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) u32x4_t lds_u32x4_t;
typedef __attribute__((address_space(3))) v4i16_t lds_v4i16_t;

// Direct-to-LDS load of 16 bytes per lane from a per-lane address: lane l's
// bytes land at LDS byte address lds + 16 l (lds wave-uniform).  Written as
// inline assembly so the compiler does not hold every later LDS read behind
// it: the caller waits for completion (s_waitcnt vmcnt) and publishes the
// data with a barrier.  M0 carries the LDS address; it is saved and
// restored, and one wait state separates its write from the load.
__device__ __forceinline__ void dma16(const uint16_t* src, uint32_t lds) {
  uint32_t saved;
  asm volatile(
      "s_mov_b32 %0, m0\n\t"
      "s_mov_b32 m0, %2\n\t"
      "s_nop 0\n\t"
      "global_load_lds_dwordx4 %1, off nt\n\t"
      "s_mov_b32 m0, %0"
      : "=&s"(saved)
      : "v"(src), "s"(lds)
      : "memory");
}
// The same from a wave-uniform base plus a 32-bit per-lane byte offset.
__device__ __forceinline__ void dma16(const uint16_t* base, uint32_t off,
                                      uint32_t lds) {
  uint32_t saved;
  asm volatile(
      "s_mov_b32 %0, m0\n\t"
      "s_mov_b32 m0, %3\n\t"
      "s_nop 0\n\t"
      "global_load_lds_dwordx4 %1, %2 nt\n\t"
      "s_mov_b32 m0, %0"
      : "=&s"(saved)
      : "v"(off), "s"(base), "s"(lds)
      : "memory");
}
// s_waitcnt vmcnt(N): at most N of this wave's vector memory operations
// (here: ring loads) still outstanding.
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  asm volatile("s_waitcnt vmcnt(%0)" ::"i"(N) : "memory");
}

// WAVES waves share the 16 query heads (16 / WAVES each); RING tile slots.
template <int WAVES, int RING>
__global__ __launch_bounds__(64 * WAVES, 1) void decode_wide_kernel(
    const DecodeParams p) {
  constexpr int NT = 64 * WAVES;
  constexpr int HW = kGroup / WAVES;  // query heads per wave
  constexpr int LPH = 16 / HW;        // lanes per head in the q broadcast rows
  constexpr int PPL = 4 * HW;         // q pairs per lane
  constexpr int PF = kGroup * (kD + 2);
  constexpr int RPW = kDecTile / WAVES;   // tile rows each wave loads
  constexpr int LPT = RPW / 4;            // loads per K (or V) tile per wave
  constexpr int PSW = (kDecTile / 2) * HW * 4;  // P bytes per wave
  static_assert(HW == 2 || HW == 4, "P reads assume 2 or 4 heads per wave");
  __shared__ __attribute__((aligned(16)))
  uint8_t smem[RING * kSlotBytes + WAVES * PSW];
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  uint8_t* Ps = smem + RING * kSlotBytes + w * PSW;

  const int unit = blockIdx.x;
  if (unit >= p.units) return;
  const int split = unit % p.splits;
  const int bg = unit / p.splits;  // b * 2 + g
  const int g = bg % kHkv;
  const int b = bg / kHkv;

  const int64_t pos = p.pos[b];
  const int nkeys = (int)(pos + 1);
  const int span = p.tiles_per_split * kDecTile;
  const int k_begin = split * span;
  const int k_end = min(nkeys, k_begin + span);
  const bool has_keys = k_begin < nkeys;
  const int new_key = nkeys - 1;
  const bool use_new = p.k_new != nullptr;
  float* const part = p.part + ((size_t)bg * p.splits + split) * PF;

  // the call appends the query's own token (see decode_kernel)
  if (use_new && g == 0 && has_keys && new_key / span == split && tid < 64) {
    const bool is_v = tid >= 32;
    const int chunk = tid & 31;
    const uint16_t* src = (is_v ? p.v_new : p.k_new) +
                          (int64_t)b * kTokenElems + chunk * 8;
    uint16_t* dst = (is_v ? p.v_mut : p.k_mut) + (int64_t)b * p.seq_stride +
                    pos * kTokenElems + chunk * 8;
    *reinterpret_cast<uint4*>(dst) = *reinterpret_cast<const uint4*>(src);
  }

  if (!has_keys) {
    for (int i = tid; i < PF; i += NT) part[i] = i < kGroup ? -INFINITY : 0.0f;
    return;
  }

  const int ntiles = (k_end - k_begin + kDecTile - 1) / kDecTile;
  const uint16_t* Kb = p.k + (int64_t)b * p.seq_stride + g * kD;
  const uint16_t* Vb = p.v + (int64_t)b * p.seq_stride + g * kD;
  const uint16_t* Kn = p.k_new + (int64_t)b * kTokenElems + g * kD;
  const uint16_t* Vn = p.v_new + (int64_t)b * kTokenElems + g * kD;
  const int head0 = g * kGroup + w * HW;

  // q words for the DPP broadcast, as in decode_kernel
  uint32_t qv[PPL];
  {
    const int n = lane & 15;
    const uint32_t* src = p.q +
                          ((int64_t)b * kHq + head0 + n / LPH) * (kD / 2) +
                          (n % LPH) * PPL;
#pragma unroll
    for (int v = 0; v < PPL; v += 4) {
      const uint4 w4 = *reinterpret_cast<const uint4*>(src + v);
      qv[v] = w4.x;
      qv[v + 1] = w4.y;
      qv[v + 2] = w4.z;
      qv[v + 3] = w4.w;
    }
  }
  // The waits in the tile loop count only the ring loads, so the q loads
  // complete here.  Passing q through an (empty) asm also tells the
  // compiler the loads are done: it cannot see the waits inside asm and
  // would otherwise repeat a full vmcnt wait before every use in the loop.
  wait_vmcnt<0>();
#pragma unroll
  for (int v = 0; v < PPL; ++v) asm volatile("" : "+v"(qv[v]));

  // Tile t -> slot t % RING.  Wave w fills rows RPW w .. RPW (w+1) - 1 of
  // the K and V tiles, four rows (1 KB) per load: lane l takes row
  // RPW w + 4i + l/16 and chunk slot l % 16.
  const int rsub = lane >> 4, cs = lane & 15;
  uint32_t kdma[LPT], vdma[LPT];  // byte offsets from the tile's first key
#pragma unroll
  for (int i = 0; i < LPT; ++i) {
    const int row = RPW * w + 4 * i + rsub;
    kdma[i] = row * (kTokenElems * 2) + ((cs ^ (row & 15)) << 4);
    vdma[i] = row * (kTokenElems * 2) + ((cs ^ (2 * (row & 7))) << 4);
  }
  const uint32_t lds_base = (uint32_t)(uintptr_t)smem;
  auto issue_tile = [&](int t, auto SLOT) {
    const int kb = k_begin + t * kDecTile;
    const uint32_t kl = __builtin_amdgcn_readfirstlane(
        lds_base + SLOT * kSlotBytes + w * RPW * 256);
    if (kb + kDecTile <= k_end && (!use_new || new_key >= kb + kDecTile)) {
      // a full tile of cached keys
      const uint16_t* kt = Kb + (int64_t)kb * kTokenElems;
      const uint16_t* vt = Vb + (int64_t)kb * kTokenElems;
#pragma unroll
      for (int i = 0; i < LPT; ++i) {
        dma16(kt, kdma[i], kl + i * 1024);
        dma16(vt, vdma[i], kl + kTileBytes + i * 1024);
      }
    } else {
      // the split's last tile: keys past its end repeat the last key (they
      // are masked), and the query's own key comes from k_new / v_new
#pragma unroll
      for (int i = 0; i < LPT; ++i) {
        const int row = RPW * w + 4 * i + rsub;
        const int key = min(kb + row, k_end - 1);
        const bool fresh = use_new && key == new_key;
        const uint16_t* krow = fresh ? Kn : Kb + (int64_t)key * kTokenElems;
        const uint16_t* vrow = fresh ? Vn : Vb + (int64_t)key * kTokenElems;
        dma16(krow + ((cs ^ (row & 15)) << 3), kl + i * 1024);
        dma16(vrow + ((cs ^ (2 * (row & 7))) << 3),
              kl + kTileBytes + i * 1024);
      }
    }
  };

  float m[HW], lsum[HW], o[HW][8];
#pragma unroll
  for (int hl = 0; hl < HW; ++hl) {
    m[hl] = -INFINITY;
    lsum[hl] = 0.0f;
#pragma unroll
    for (int e = 0; e < 8; ++e) o[hl][e] = 0.0f;
  }

  // LDS read offsets: the K row of key = lane, and the P.V transposes (the
  // 16-lane group kg reads keys 16q + 4kg + (j >> 2), dims 16e + 4(j & 3)).
  const int kg = lane >> 4, jl = lane & 15, ja = jl & 3, je = jl >> 2;
  uint32_t krd[16], vrd[8];
#pragma unroll
  for (int c = 0; c < 16; ++c) krd[c] = lds_base + lane * 256 + ((c ^ jl) << 4);
#pragma unroll
  for (int e = 0; e < 8; ++e)
    vrd[e] = lds_base + kTileBytes + (4 * kg + je) * 256 +
             32 * (e ^ ((4 * kg + je) & 7)) +
             8 * ja;
  // P words of key pairs 8q + 2kg and 8q + 2kg + 1
  const uint32_t prd = (uint32_t)(uintptr_t)Ps + 2 * kg * HW * 4;

  auto consume = [&](int t, auto SLOT) {
    constexpr uint32_t so = SLOT * kSlotBytes;
    // ---- scores (lane = key), exactly as in decode_kernel
    constexpr int NACC = 4 / HW;
    float acc[HW][NACC];
#pragma unroll
    for (int hl = 0; hl < HW; ++hl)
#pragma unroll
      for (int a = 0; a < NACC; ++a) acc[hl][a] = 0.0f;
    u32x4_t kbuf[2][4];
    auto read_batch = [&](auto Bt, u32x4_t(&dst)[4]) {
      static_for<0, 4>([&](auto J) {
        dst[J] = *reinterpret_cast<const lds_u32x4_t*>(krd[4 * Bt + J] + so);
      });
    };
    read_batch(std::integral_constant<int, 0>{}, kbuf[0]);
    static_for<0, 4>([&](auto Bt) {
      if constexpr (Bt + 1 < 4)
        read_batch(std::integral_constant<int, Bt + 1>{}, kbuf[(Bt + 1) & 1]);
      static_for<0, 4>([&](auto J) {
        constexpr int C = 4 * Bt + J;
        static_for<0, 4>([&](auto I) {
          constexpr int pr = 4 * C + I;
          static_for<0, HW>([&](auto HL) {
            constexpr int ii = I, bb = Bt & 1, jj = J, hh = HL;
            acc[hh][ii % NACC] =
                dot2_bf16_bcast<HL * LPH + pr / PPL, (C == 0 && ii < NACC)>(
                    qv[pr % PPL], kbuf[bb][jj][ii], acc[hh][ii % NACC]);
          });
        });
      });
    });
    const bool valid = k_begin + t * kDecTile + lane < k_end;
    float s2[HW];
    bool need = false;
#pragma unroll
    for (int hl = 0; hl < HW; ++hl) {
      float a = acc[hl][0];
#pragma unroll
      for (int k = 1; k < NACC; ++k) a += acc[hl][k];
      s2[hl] = valid ? a * p.scale_log2 : -INFINITY;
      need |= s2[hl] > m[hl] + kTau;
    }
    if (__any(need)) {
#pragma unroll
      for (int hl = 0; hl < HW; ++hl) {
        const float mn = fmaxf(m[hl], wave_max(s2[hl]));
        const float alpha = fast_exp2(m[hl] - mn);
        m[hl] = mn;
        lsum[hl] *= alpha;
#pragma unroll
        for (int e = 0; e < 8; ++e) o[hl][e] *= alpha;
      }
    }
    uint16_t* P16 = reinterpret_cast<uint16_t*>(Ps);
#pragma unroll
    for (int hl = 0; hl < HW; ++hl) {
      const uint16_t pb = to_bf16(fast_exp2(s2[hl] - m[hl]));
      lsum[hl] += __builtin_bit_cast(float, (uint32_t)pb << 16);
      P16[(lane >> 1) * (2 * HW) + hl * 2 + (lane & 1)] = pb;
    }
    __builtin_amdgcn_s_waitcnt(0xc07f);  // lgkmcnt(0): P visible to the wave
    __builtin_amdgcn_wave_barrier();

    // ---- P.V over the four 16-key quarters of the tile
    static_for<0, 4>([&](auto Q) {
      uint32_t pa[HW], pc[HW];  // pairs 8Q + 2kg and 8Q + 2kg + 1
      if constexpr (HW == 4) {
        const u32x4_t x = *reinterpret_cast<const lds_u32x4_t*>(prd + Q * 128);
        const u32x4_t y =
            *reinterpret_cast<const lds_u32x4_t*>(prd + Q * 128 + 16);
        static_for<0, 4>([&](auto H) {
          constexpr int h = H;
          pa[h] = x[h];
          pc[h] = y[h];
        });
      } else {
        const u32x4_t x = *reinterpret_cast<const lds_u32x4_t*>(prd + Q * 64);
        pa[0] = x[0];
        pa[1] = x[1];
        pc[0] = x[2];
        pc[1] = x[3];
      }
      static_for<0, 8>([&](auto E) {
        const v4i16_t r = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            reinterpret_cast<lds_v4i16_t*>(vrd[E] + so + Q * 16 * 256));
        const uint2 vw = __builtin_bit_cast(uint2, r);
#pragma unroll
        for (int hl = 0; hl < HW; ++hl) {
          o[hl][E] = dot2_bf16(pa[hl], vw.x, o[hl][E]);
          o[hl][E] = dot2_bf16(pc[hl], vw.y, o[hl][E]);
        }
      });
    });
  };

  static_for<0, RING - 1>([&](auto T) {
    if (T < ntiles) issue_tile(T, T);
  });
  for (int t0 = 0; t0 < ntiles; t0 += RING) {
    static_for<0, RING>([&](auto S) {
      const int t = t0 + S;
      if (t < ntiles) {
        // tile t has landed (this wave's rows) once only the later tiles'
        // loads are outstanding; the barrier publishes every wave's rows
        // and frees the slot consumed in the previous step
        const int later = min(RING - 2, ntiles - 1 - t);
        static_for<0, RING - 1>([&](auto L) {
          if (later == L) wait_vmcnt<L * 2 * LPT>();
        });
        __syncthreads();
        if (t + RING - 1 < ntiles)
          issue_tile(t + RING - 1,
                     std::integral_constant<int, (S + RING - 1) % RING>{});
        consume(t, S);
      }
    });
  }

  // ---- reduce over the four key groups and the 64 key lanes, write
#pragma unroll
  for (int hl = 0; hl < HW; ++hl) {
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      o[hl][e] += __shfl_xor(o[hl][e], 16, 64);
      o[hl][e] += __shfl_xor(o[hl][e], 32, 64);
    }
    lsum[hl] = wave_sum(lsum[hl]);
  }
  if (kg == 0) {
#pragma unroll
    for (int hl = 0; hl < HW; ++hl) {
      float* dst = part + 2 * kGroup + (w * HW + hl) * kD + jl;
#pragma unroll
      for (int e = 0; e < 8; ++e) dst[16 * e] = o[hl][e];
    }
  }
  if (lane == 0) {
#pragma unroll
    for (int hl = 0; hl < HW; ++hl) {
      part[w * HW + hl] = m[hl];
      part[kGroup + w * HW + hl] = lsum[hl];
    }
  }
}

// Merge the split partials of one (sequence, query head, quarter of the
// head dimension): with M the largest split maximum,
// o = sum 2^(m_s - M) o_s / sum 2^(m_s - M) l_s.  256 threads = 8 float4
// columns x 32 split lanes, so all loads of a column are in flight at once.
__global__ __launch_bounds__(256) void decode_merge_kernel(
    const DecodeParams p, int heads_per_wg) {
  const int dq = blockIdx.x & 3;
  const int h = (blockIdx.x >> 2) % kHq;
  const int b = (blockIdx.x >> 2) / kHq;
  const int g = h / kGroup, hh = h % kGroup;
  const int hpw = heads_per_wg, hg = hh / hpw, hl = hh % hpw;
  const int hgroups = kGroup / hpw;
  const int pf = hpw * (kD + 2);
  const float* base =
      p.part + (size_t)((b * kHkv + g) * hgroups + hg) * p.splits * pf;
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
      const float* ps = base + (size_t)min(s, p.splits - 1) * pf;
      ms[i] = s < p.splits ? ps[hl] : -INFINITY;
      ls[i] = ps[hpw + hl];
      os[i] = *reinterpret_cast<const float4*>(ps + 2 * hpw + hl * kD + d);
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
  if (sl == 0) {
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
    *reinterpret_cast<float4*>(p.out + ((size_t)b * kHq + h) * kD + d) =
        make_float4(x * inv, y * inv, z * inv, ww * inv);
  }
}

}  // namespace

hipError_t launch_decode(const DecodeParams& p, const DecodePlan& plan,
                         bool local, int B, hipStream_t s) {
  const dim3 block(kDecThreads);
  if (plan.narrow) {
    const int grid = (p.units + 7) / 8 * 8 * plan.head_groups;
    if (local)
      hipLaunchKernelGGL((decode_kernel<true, 1, true>), dim3(grid), block, 0,
                         s, p);
    else
      hipLaunchKernelGGL((decode_kernel<false, 1, true>), dim3(grid), block,
                         0, s, p);
    return hipGetLastError();
  }
  if (local) return hipErrorInvalidValue;  // local layers use the narrow shape
  hipLaunchKernelGGL((decode_wide_kernel<kWideWaves, kWideRing>), dim3(p.units),
                     dim3(64 * kWideWaves), 0, s, p);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(decode_merge_kernel, dim3(B * kHq * 4), dim3(256), 0, s,
                     p, plan.heads_per_wg);
  return hipGetLastError();
}

}  // namespace gqa
