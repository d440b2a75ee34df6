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
//  * A workgroup owns one (sequence, KV head, key split) and serves all 16
//    query heads of that KV head out of the same tiles, so each cached K/V
//    byte is fetched from HBM once.  Global layers: 4 waves, two workgroups
//    per CU, long splits; each wave takes the 16 keys of every tile whose
//    rows it loads itself, for all 16 heads, so the waves never wait for one
//    another inside the tile loop and merge their sums once at the end.
//    Local layers (a 2048-key window, so latency rather than bandwidth): 8
//    waves of 2 heads over the whole tile, one 64-key tile per workgroup up
//    to batch 4.
//  * Tiles of 64 keys go straight from HBM into LDS rings with direct-to-LDS
//    loads (global_load_lds_dwordx4: lane l's 16 bytes land at the wave's LDS
//    base + 16 l, never passing through VGPRs), marked non-temporal since the
//    cache is streamed once per step.  K and V tiles have rings of their own;
//    on global layers K tiles are loaded two tiles ahead and V tiles one
//    (three K slots, two V slots: 80 KB, two workgroups per CU).
//  * Q.K: lane = key (global layers: lane 16 r + j = key j of the wave's 16,
//    heads 4 r .. 4 r + 3); the query words are uniform across each 16-lane
//    row, held 16 to a VGPR and broadcast with DPP row_newbcast into
//    v_dot2c_f32_bf16 (bf16 products exact, fp32 accumulation).  K rows sit in LDS with 16-byte
//    chunk c of row r at chunk slot c ^ (r & 15), so a lane reads its whole
//    row without bank conflicts.
//  * Local layers rotate each landed K tile in LDS by its keys' offsets to
//    the query (j - i): <R_i q, R_j k> = <q, R_{j-i} k>, so the query stays
//    unrotated and the angles stay small (|j - i| < 2048; fp32 angle error
//    ~1e-4 rad).  The angles' sines and cosines are taken while the tile is
//    still in flight.
//  * Online softmax in the log2 domain with a lazy maximum: the running
//    maximum is only raised (and the accumulators rescaled) when some score
//    exceeds it by more than 2^8, which keeps every exponent <= 2^8 while
//    skipping nearly all cross-lane reductions.  The denominator sums exactly
//    the bf16 weights the P.V product uses.
//  * P.V: each 16-lane row of a wave takes the 16 keys whose scores it holds;
//    the bf16 weights of a key pair are packed into one lane and broadcast to
//    the row with DPP row_newbcast (P never goes through LDS).  V rows stay in
//    key order (chunk c at slot c ^ 2(r & 7)) and are read with
//    ds_read_b64_tr_b16, which gives each lane four consecutive keys of one
//    dimension: two key-interleaved bf16 pairs, the operand v_dot2_f32_bf16
//    wants, with no VALU re-packing.
//  * Each workgroup writes (m, l, o) for its split; a second kernel merges
//    the splits with the log-sum-exp rule.
//  * Optionally the call appends the query's own K/V: the kernel reads that
//    key from the new-token buffers and one workgroup stores it to its slot,
//    saving a separate append launch per layer.
#include "device_common.h"
#include "internal.h"

namespace gqa {

namespace {

typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
constexpr float kTau = 8.0f;  // lazy-rescale threshold in log2 units
__device__ __forceinline__ int64_t slot_of(int64_t position, bool local) {
  return local ? (position & (kW - 1)) : position;
}

// The tile loop is unrolled over the period of the slot pattern so every LDS
// address is a per-lane register plus a constant.  P.V lanes: lane 16 g + j
// owns dimensions j, j + 16, ..., j + 112 of its wave's heads and keys
// 16 g .. 16 g + 15; the four rows g are summed at the end.
constexpr int kTileBytes = kDecTile * 256;    // one 64-key tile of K or V

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
// Direct-to-LDS load of 4 bytes per lane (lane l's word lands at lds + 4 l).
__device__ __forceinline__ void dma4(const float* src, uint32_t lds) {
  uint32_t saved;
  asm volatile(
      "s_mov_b32 %0, m0\n\t"
      "s_mov_b32 m0, %2\n\t"
      "s_nop 0\n\t"
      "global_load_lds_dword %1, off\n\t"
      "s_mov_b32 m0, %0"
      : "=&s"(saved)
      : "v"(src), "s"(lds)
      : "memory");
}

// Two E4M3 codes (the lower or upper half of w, first code in the lower
// byte) as a bf16 pair, exactly (scale 1).
template <bool HI>
__device__ __forceinline__ uint32_t cvt_fp8x2_bf16(uint32_t w) {
  return __builtin_bit_cast(
      uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.0f, HI));
}

// s_waitcnt vmcnt(N): at most N of this wave's vector memory operations
// (here: ring loads) still outstanding.
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  asm volatile("s_waitcnt vmcnt(%0)" ::"i"(N) : "memory");
}

// A workgroup of WAVES waves serves HPW of the 16 query heads (HPW / WAVES
// per wave; 16 / HPW workgroups share each tile); KR slots for K tiles and
// VR for V tiles (K tiles are needed first in a step, so they may be loaded
// one tile further ahead).  LOCAL: the keys are the window
// max(0, pos - 2047) .. pos read through the ring, and each landed K tile is
// rotated in LDS by its keys' offsets to the query before the products.
// KSPLIT: the waves split every tile's keys instead of the heads -- wave w
// takes the 16 keys whose rows it loads itself, for all 16 heads (row r of
// the wave: heads 4 r .. 4 r + 3) -- so no wave reads another's rows and
// the tile loop needs no barrier; the four waves' sums are combined once at
// the end.
//
// F8: the cache holds E4M3 codes plus one fp32 scale per (token, KV head).
// The rings then hold code tiles (64 rows of 128 bytes) and each row's scale;
// once its rows have landed, each wave dequantises them (code x scale, to
// bf16) into a bf16 staging tile laid out as the bf16 rings are, and the
// products read the staging tile.
template <int WAVES, int HPW, int KR, int VR, bool LOCAL, bool KSPLIT = false,
          bool F8 = false>
__global__ __launch_bounds__(64 * WAVES, 1) void decode_split_kernel(
    const DecodeParams p) {
  constexpr int NT = 64 * WAVES;
  constexpr int HW = HPW / WAVES;     // query heads per wave
  constexpr int HG = kGroup / HPW;    // workgroups sharing a tile (head groups)
  constexpr int LPH = 16 / HW;        // lanes per head in the q broadcast rows
  constexpr int PPL = 4 * HW;         // q pairs per lane
  constexpr int PF = HPW * (kD + 2);
  constexpr int RPW = kDecTile / WAVES;   // tile rows each wave loads
  constexpr int LPT = RPW / 4;            // loads per K (or V) tile per wave
  static_assert(HW == 2 || HW == 4, "two or four heads per wave");
  static_assert(KR == VR || KR == VR + 1, "K at most one tile further ahead");
  static_assert(!KSPLIT || (!LOCAL && WAVES == 4 && HPW == kGroup && KR > 1),
                "key split: global layers, four waves of 16 keys, all heads");
  // F8 LDS: code rings (8 KB a tile), per-wave scale slots (64 words each),
  // then the bf16 staging tiles of K and V
  constexpr int kCodeTile = kDecTile * kD;                 // 8 KB
  constexpr int kScaleSlot = WAVES * 256;                  // bytes per slot
  constexpr int kF8Bytes = (KR + VR) * (kCodeTile + kScaleSlot) +
                           2 * kTileBytes;
  constexpr int kSmem = F8 ? kF8Bytes : (KR + VR) * kTileBytes;
  static_assert(!F8 || RPW % 8 == 0, "whole 1 KB code loads per wave");
  __shared__ __attribute__((aligned(16))) uint8_t smem[kSmem];
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);

  // workgroup -> (unit, head group).  Consecutive workgroup ids go to the
  // device's XCDs round-robin, so the HG workgroups of one unit are placed
  // X = p.xcds ids apart: same XCD, same L2, dispatched together.  (The map
  // is one-to-one for any X; only the L2 sharing depends on it.)
  int unit = blockIdx.x, hg = 0;
  if constexpr (HG > 1) {
    const int X = p.xcds;
    const int r = blockIdx.x % (X * HG);
    unit = (blockIdx.x / (X * HG)) * X + r % X;
    hg = r / X;
  } else {
    // When the (sequence, KV head) pairs divide evenly over the XCDs, all
    // splits of one pair run on one XCD (ids X apart), where the merge
    // kernel's workgroups for that pair run too, reading the partials from
    // that XCD's L2.
    const int X = p.xcds, S = p.splits, BG = p.units / S;
    if (X > 1 && BG % X == 0) {
      const int xcd = blockIdx.x % X, s = blockIdx.x / X;
      unit = (xcd + X * (s / S)) * S + s % S;
    }
  }
  if (unit >= p.units) return;  // padding of the XCD-aware grid
  const int split = unit % p.splits;
  const int bg = unit / p.splits;  // b * 2 + g
  const int g = bg % kHkv;
  const int b = bg / kHkv;

  // positions come with the call, or from device memory (checked against
  // the bound the host validated; a position outside it is not attended)
  int64_t pos = p.pos[b];
  bool pos_ok = true;
  if (p.pos_dev) {
    pos = p.pos_dev[b];
    pos_ok = pos >= 0 && pos <= p.max_pos;
    if (!pos_ok) pos = 0;
  }
  // key index k is position j_first + k
  const int64_t j_first = LOCAL ? (pos > kW - 1 ? pos - (kW - 1) : 0) : 0;
  const int nkeys = (int)(pos - j_first + 1);
  const int span = p.tiles_per_split * kDecTile;
  const int k_begin = split * span;
  const int k_end = min(nkeys, k_begin + span);
  const bool has_keys = k_begin < nkeys;
  const int new_key = nkeys - 1;
  const bool use_new = p.k_new != nullptr;
  float* const part =
      p.part + (((size_t)bg * HG + hg) * p.splits + split) * PF;

  if (!pos_ok) {  // NaN partials make the merged output NaN; no append
    for (int i = tid; i < PF; i += NT) part[i] = __builtin_nanf("");
    return;
  }

  // The call appends the query's own token: one workgroup writes it to its
  // slot, which no other workgroup reads in this launch (they take that key
  // from k_new / v_new).
  if (!F8 && use_new && g == 0 && hg == 0 && has_keys &&
      new_key / span == split && tid < 64) {
    const bool is_v = tid >= 32;
    const int chunk = tid & 31;
    const uint16_t* src = (is_v ? p.v_new : p.k_new) +
                          (int64_t)b * kTokenElems + chunk * 8;
    uint16_t* dst = (is_v ? p.v_mut : p.k_mut) + (int64_t)b * p.seq_stride +
                    slot_of(pos, LOCAL) * kTokenElems + chunk * 8;
    *reinterpret_cast<uint4*>(dst) = *reinterpret_cast<const uint4*>(src);
  }

  if (!has_keys) {
    for (int i = tid; i < PF; i += NT) part[i] = i < HPW ? -INFINITY : 0.0f;
    return;
  }

  const int ntiles = (k_end - k_begin + kDecTile - 1) / kDecTile;
  const uint16_t* Kb = p.k + (int64_t)b * p.seq_stride + g * kD;
  const uint16_t* Vb = p.v + (int64_t)b * p.seq_stride + g * kD;
  // F8: codes (seq_stride in bytes) and scales of this (sequence, KV head)
  const uint8_t* K8b = p.k8 + (int64_t)b * p.seq_stride + g * kD;
  const uint8_t* V8b = p.v8 + (int64_t)b * p.seq_stride + g * kD;
  const float* KSb = p.k_scale + (int64_t)b * p.scale_stride + g * p.capacity;
  const float* VSb = p.v_scale + (int64_t)b * p.scale_stride + g * p.capacity;
  const uint16_t* Kn = p.k_new + (int64_t)b * kTokenElems + g * kD;
  const uint16_t* Vn = p.v_new + (int64_t)b * kTokenElems + g * kD;
  // first head of this lane's row: the wave's heads, or (KSPLIT) row r's
  const int hrow = KSPLIT ? (lane >> 4) * HW : w * HW;  // within the group
  const int head0 = g * kGroup + hg * HPW + hrow;

  // The wave's HW query rows (64 bf16 pairs each) held as wave-uniform words
  // for the DPP broadcast: within every 16-lane row, lane n keeps pairs
  // (n % LPH) * PPL .. + PPL - 1 of head n / LPH in qv[0 .. PPL).
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

  // Tile t -> K slot t % KR, V slot t % VR.  Wave w fills rows
  // RPW w .. RPW (w+1) - 1 of the K and V tiles, four rows (1 KB) per load:
  // lane l takes row RPW w + 4i + l/16 and chunk slot l % 16.
  const int rsub = lane >> 4, cs = lane & 15;
  uint32_t kdma[LPT], vdma[LPT];  // byte offsets from the tile's first key
#pragma unroll
  for (int i = 0; i < LPT; ++i) {
    const int row = RPW * w + 4 * i + rsub;
    kdma[i] = row * (kTokenElems * 2) + ((cs ^ (row & 15)) << 4);
    vdma[i] = row * (kTokenElems * 2) + ((cs ^ (2 * (row & 7))) << 4);
  }
  // K slot k at lds_base + k * kTileBytes, V slot v at vbase + v * kTileBytes
  const uint32_t lds_base = (uint32_t)(uintptr_t)smem;
  const uint32_t vbase = lds_base + KR * kTileBytes;
  // Wave w's rows of tile t of K (IS_V false) or V into LDS at lds.  A full
  // tile of cached keys in consecutive slots loads from one wave-uniform
  // base; the split's last tile repeats its last key past the end (masked)
  // and takes the query's own key from k_new / v_new.
  auto issue = [&](int t, auto IS_V, uint32_t lds) {
    const uint16_t* base = IS_V ? Vb : Kb;
    const uint16_t* fresh_row = IS_V ? Vn : Kn;
    const int kb = k_begin + t * kDecTile;
    const int64_t slot0 = slot_of(j_first + kb, LOCAL);
    lds = __builtin_amdgcn_readfirstlane(lds + w * RPW * 256);
    if (kb + kDecTile <= k_end && (!use_new || new_key >= kb + kDecTile) &&
        (!LOCAL || slot0 + kDecTile <= kW)) {
      const uint16_t* tb = base + slot0 * kTokenElems;
#pragma unroll
      for (int i = 0; i < LPT; ++i)
        dma16(tb, IS_V ? vdma[i] : kdma[i], lds + i * 1024);
    } else {
#pragma unroll
      for (int i = 0; i < LPT; ++i) {
        const int row = RPW * w + 4 * i + rsub;
        const int key = min(kb + row, k_end - 1);
        const bool fresh = use_new && key == new_key;
        const int64_t slot = slot_of(j_first + key, LOCAL);
        const uint16_t* src = fresh ? fresh_row : base + slot * kTokenElems;
        const int c = IS_V ? cs ^ (2 * (row & 7)) : cs ^ (row & 15);
        dma16(src + (c << 3), lds + i * 1024);
      }
    }
  };
  auto issue_k = [&](int t, auto KS) {
    issue(t, std::false_type{}, lds_base + KS * kTileBytes);
  };
  auto issue_v = [&](int t, auto VS) {
    issue(t, std::true_type{}, vbase + VS * kTileBytes);
  };

  // F8: code slots of K then V, their scale slots (wave w's 256 bytes each),
  // then the bf16 staging tiles.  Lane l of wave w loads code chunk l % 8 of
  // row RPW w + 8 i + l / 8 (a row is 128 codes of one KV head) and the scale
  // of row RPW w + l % RPW.
  constexpr int LPT8 = RPW / 8;                 // 1 KB code loads per tile
  const uint32_t k8base = lds_base;
  const uint32_t v8base = k8base + KR * kCodeTile;
  const uint32_t ksbase = v8base + VR * kCodeTile;
  const uint32_t vsbase = ksbase + KR * kScaleSlot;
  const uint32_t stk = vsbase + VR * kScaleSlot;  // staging K, bf16
  const uint32_t stv = stk + kTileBytes;          // staging V, bf16
  const int crow = lane >> 3, cch = lane & 7;
  const int srow = RPW * w + lane % RPW;
  auto issue8 = [&](int t, auto IS_V, uint32_t lds, uint32_t slds) {
    const uint8_t* base = IS_V ? V8b : K8b;
    const float* sb = IS_V ? VSb : KSb;
    const int kb = k_begin + t * kDecTile;
    const int64_t slot0 = slot_of(j_first + kb, LOCAL);
    lds = __builtin_amdgcn_readfirstlane(lds + w * RPW * kD);
    slds = __builtin_amdgcn_readfirstlane(slds + w * 256);
    if (kb + kDecTile <= k_end && (!LOCAL || slot0 + kDecTile <= kW)) {
      const uint8_t* tb = base + slot0 * (kHkv * kD);
#pragma unroll
      for (int i = 0; i < LPT8; ++i)
        dma16(reinterpret_cast<const uint16_t*>(tb),
              (uint32_t)((RPW * w + 8 * i + crow) * (kHkv * kD) + cch * 16),
              lds + i * 1024);
      dma4(sb + slot0 + srow, slds);
    } else {
#pragma unroll
      for (int i = 0; i < LPT8; ++i) {
        const int key = min(kb + RPW * w + 8 * i + crow, k_end - 1);
        const int64_t slot = slot_of(j_first + key, LOCAL);
        dma16(reinterpret_cast<const uint16_t*>(base + slot * (kHkv * kD) +
                                                cch * 16),
              lds + i * 1024);
      }
      dma4(sb + slot_of(j_first + min(kb + srow, k_end - 1), LOCAL), slds);
    }
  };
  auto issue8_k = [&](int t, auto KS) {
    issue8(t, std::false_type{}, k8base + KS * kCodeTile,
           ksbase + KS * kScaleSlot);
  };
  auto issue8_v = [&](int t, auto VS) {
    issue8(t, std::true_type{}, v8base + VS * kCodeTile,
           vsbase + VS * kScaleSlot);
  };
  // loads one tile issue puts in flight per wave (the ring waits count them)
  constexpr int LPI = F8 ? LPT8 + 1 : LPT;
  // Wave w turns its own rows of the landed code tiles into bf16 codes in
  // the staging tiles (exact: every E4M3 value is a bf16 value), in the
  // swizzled layouts the products read; the scales are applied to the
  // scores (K) and the weights (V).
  auto dequant = [&](auto KS, auto VS) {
    static_for<0, LPT8>([&](auto I) {
      const int row = RPW * w + 8 * I + crow;
      static_for<0, 2>([&](auto IV) {
        const uint32_t src = (IV ? v8base + VS * kCodeTile
                                 : k8base + KS * kCodeTile) +
                             row * kD + cch * 16;
        const u32x4_t c = *reinterpret_cast<const lds_u32x4_t*>(src);
        u32x4_t lo, hi;
#pragma unroll
        for (int e = 0; e < 2; ++e) {
          lo[2 * e] = cvt_fp8x2_bf16<false>(c[e]);
          lo[2 * e + 1] = cvt_fp8x2_bf16<true>(c[e]);
          hi[2 * e] = cvt_fp8x2_bf16<false>(c[e + 2]);
          hi[2 * e + 1] = cvt_fp8x2_bf16<true>(c[e + 2]);
        }
        const int swz = IV ? 2 * (row & 7) : (row & 15);
        const uint32_t dst = (IV ? stv : stk) + row * 256;
        *reinterpret_cast<lds_u32x4_t*>(dst + (((2 * cch) ^ swz) << 4)) = lo;
        *reinterpret_cast<lds_u32x4_t*>(dst + (((2 * cch + 1) ^ swz) << 4)) =
            hi;
      });
    });
  };
  // scale of key k of the landed tile in K slot KS (V slot VS)
  auto kscale = [&](int k, auto KS) {
    return *reinterpret_cast<const __attribute__((address_space(3))) float*>(
        ksbase + KS * kScaleSlot + (k / RPW) * 256 + 4 * (k % RPW));
  };
  auto vscale = [&](int k, auto VS) {
    return *reinterpret_cast<const __attribute__((address_space(3))) float*>(
        vsbase + VS * kScaleSlot + (k / RPW) * 256 + 4 * (k % RPW));
  };
  // the K tile the products (and the local rotation) read
  auto ktile = [&](auto KS) -> uint32_t {
    return F8 ? stk : lds_base + KS * kTileBytes;
  };

  float m[HW], lsum[HW], o[HW][8];
#pragma unroll
  for (int hl = 0; hl < HW; ++hl) {
    // KSPLIT: a wave may see no valid key in its first tiles; a finite
    // floor keeps 2^(s - m) at 0 there instead of 2^(-inf + inf)
    m[hl] = KSPLIT ? -1e30f : -INFINITY;
    lsum[hl] = 0.0f;
    // each accumulator gets a register of its own (a shared zero would be
    // copied in right before the first DPP product that reads it)
#pragma unroll
    for (int e = 0; e < 8; ++e) asm volatile("v_mov_b32 %0, 0" : "=v"(o[hl][e]));
  }

  // LDS read offsets: the K row of key = lane (KSPLIT: 16 w + lane % 16),
  // and the P.V transposes: row kg of the wave (lanes 16 kg ..) reads keys
  // 16 kg + 4 q + (j >> 2) (KSPLIT: 16 w + 4 q + (j >> 2) in every row), dims
  // 16 e + 4 (j & 3) for key quad q of its row; for odd q the swizzle puts
  // dims 16 e at the offset of dims 16 (e ^ 4) of q = 0.
  const int kg = lane >> 4, jl = lane & 15, ja = jl & 3, je = jl >> 2;
  uint32_t krd[16], vrd[8];
  // KSPLIT: key 16 w + jl in the products, V rows 16 w .. of every row
  const int krow = KSPLIT ? 16 * w + jl : lane;
  const int vgrp = KSPLIT ? w : kg;
  const uint32_t kread = F8 ? stk : lds_base, vread = F8 ? stv : vbase;
#pragma unroll
  for (int c = 0; c < 16; ++c) krd[c] = kread + krow * 256 + ((c ^ jl) << 4);
#pragma unroll
  for (int e = 0; e < 8; ++e)
    vrd[e] = vread + (16 * vgrp + je) * 256 + 32 * (e ^ je) + 8 * ja;

  auto consume = [&](int t, auto KS, auto VS) {
    constexpr uint32_t so = F8 ? 0 : KS * kTileBytes;
    constexpr uint32_t vso = F8 ? 0 : VS * kTileBytes;
    // F8: the scales of this lane's key (the one whose scores it holds)
    float ksc = 1.0f, vsc = 1.0f;
    if constexpr (F8) {
      ksc = kscale(krow, KS) * p.scale_log2;
      vsc = vscale(krow, VS);
    }
    // ---- scores: lane = key of this tile (KSPLIT: key krow); the query
    // word of (head hl, pair pr) is broadcast from lane hl * LPH + pr / PPL
    // of the lane's row.  The lane's K row
    // is read from LDS in 4 batches of 64 B, one batch ahead of the
    // products; consecutive products alternate between accumulators, so a
    // product's accumulator was last written four instructions earlier (a
    // DPP instruction must not read a VGPR written by either of the two
    // VALU instructions before it).
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
        constexpr int bb = Bt & 1, jj = J;
        if constexpr (HW == 4) {
          // pairs 4C .. 4C + 3 for the four heads in one asm block
          const uint32_t qw[4] = {qv[(4 * C) % PPL], qv[(4 * C + 1) % PPL],
                                  qv[(4 * C + 2) % PPL],
                                  qv[(4 * C + 3) % PPL]};
          const uint32_t kw[4] = {kbuf[bb][jj][0], kbuf[bb][jj][1],
                                  kbuf[bb][jj][2], kbuf[bb][jj][3]};
          float a4[4] = {acc[0][0], acc[1][0], acc[2][0], acc[3][0]};
          dot2_bf16_bcast16<LPH, PPL, C, C == 0>(qw, kw, a4);
          acc[0][0] = a4[0], acc[1][0] = a4[1], acc[2][0] = a4[2],
          acc[3][0] = a4[3];
        } else {
          static_for<0, 4>([&](auto I) {
            constexpr int pr = 4 * C + I;
            static_for<0, HW>([&](auto HL) {
              constexpr int ii = I, hh = HL;
              acc[hh][ii % NACC] =
                  dot2_bf16_bcast<HL * LPH + pr / PPL, (C == 0 && ii < NACC)>(
                      qv[pr % PPL], kbuf[bb][jj][ii], acc[hh][ii % NACC]);
            });
          });
        }
      });
    });
    static_assert(HW * NACC == 4, "four score accumulators per wave");
    // V^T operands of key quad QQ of the row (see P.V below); the first
    // quad's are read before the softmax, each next quad's one quad ahead
    uint2 vw[2][8];
    auto read_quad = [&](auto QQ, uint2(&dst)[8]) {
      static_for<0, 8>([&](auto E) {
        constexpr int e = (QQ & 1) ? (E ^ 4) : E;
        const v4i16_t r = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            reinterpret_cast<lds_v4i16_t*>(vrd[e] + vso + QQ * 1024));
        dst[E] = __builtin_bit_cast(uint2, r);
      });
    };
    read_quad(std::integral_constant<int, 0>{}, vw[0]);
    dpp_settle(acc[0][0], acc[(1 / NACC) % HW][1 % NACC],
               acc[(2 / NACC) % HW][2 % NACC], acc[(3 / NACC) % HW][3 % NACC]);
    const bool valid = k_begin + t * kDecTile + krow < k_end;
    float s2[HW];
    bool need = false;
#pragma unroll
    for (int hl = 0; hl < HW; ++hl) {
      float a = acc[hl][0];
#pragma unroll
      for (int k = 1; k < NACC; ++k) a += acc[hl][k];
      s2[hl] = valid ? a * (F8 ? ksc : p.scale_log2) : -INFINITY;
      need |= s2[hl] > m[hl] + kTau;
    }
    if (__any(need)) {
#pragma unroll
      for (int hl = 0; hl < HW; ++hl) {
        const float mn =
            fmaxf(m[hl], KSPLIT ? row_max(s2[hl]) : wave_max(s2[hl]));
        const float alpha = fast_exp2(m[hl] - mn);
        m[hl] = mn;
        lsum[hl] *= alpha;
#pragma unroll
        for (int e = 0; e < 8; ++e) o[hl][e] *= alpha;
      }
    }
    // ---- P.V.  Lane 16 r + j takes the 16 keys of its own row r and
    // dimensions j, j + 16, ..., j + 112.  The bf16 weights of key pair i of
    // the row (keys 2i, 2i + 1) are packed into lane 2i and broadcast to the
    // row with DPP row_newbcast, so P never goes through LDS.
    uint32_t pk[HW];
#pragma unroll
    for (int hl = 0; hl < HW; ++hl) {
      uint32_t pb;
      if constexpr (F8) {
        // the weight times the key's V scale goes into P.V; the
        // denominator sums the weights themselves
        const float pw = fast_exp2(s2[hl] - m[hl]);
        lsum[hl] += pw;
        pb = to_bf16(pw * vsc);
      } else {
        pb = to_bf16(fast_exp2(s2[hl] - m[hl]));
        lsum[hl] += __builtin_bit_cast(float, pb << 16);
      }
      // lanes 2i take lane 2i + 1's weight (quad_perm [1, 1, 3, 3])
      const uint32_t nb = __builtin_amdgcn_mov_dpp((int)pb, 0xF5, 0xF, 0xF, false);
      pk[hl] = pb | (nb << 16);
    }
    // two wait states between the last VALU write of a weight pair and the
    // DPP products that read it
    if constexpr (HW == 4)
      asm volatile("s_nop 1" : "+v"(pk[0]), "+v"(pk[1]), "+v"(pk[2]), "+v"(pk[3]));
    else
      asm volatile("s_nop 1" : "+v"(pk[0]), "+v"(pk[1]));
    static_for<0, 4>([&](auto QQ) {  // keys 4 QQ .. 4 QQ + 3 of the row
      if constexpr (QQ + 1 < 4)
        read_quad(std::integral_constant<int, QQ + 1>{}, vw[(QQ + 1) & 1]);
      constexpr int cb = QQ & 1;
      // keys (4 QQ, 4 QQ + 1) for every accumulator, then (4 QQ + 2, + 3):
      // a product's accumulator was last written HW * 8 products earlier
      static_for<0, 8>([&](auto E) {
        static_for<0, HW>([&](auto HL) {
          o[HL][E] =
              dot2_bf16_bcast<4 * QQ, false>(pk[HL], vw[cb][E].x, o[HL][E]);
        });
      });
      static_for<0, 8>([&](auto E) {
        static_for<0, HW>([&](auto HL) {
          o[HL][E] =
              dot2_bf16_bcast<4 * QQ + 2, false>(pk[HL], vw[cb][E].y, o[HL][E]);
        });
      });
    });
    // the last four products' results settle before any plain read
    constexpr int L0 = HW * 8 - 4;
    dpp_settle(o[L0 % HW][L0 / HW], o[(L0 + 1) % HW][(L0 + 1) / HW],
               o[(L0 + 2) % HW][(L0 + 2) / HW], o[(L0 + 3) % HW][(L0 + 3) / HW]);
  };

  // LOCAL: thread i rotates items i, i + NT, ... of the K tile, item u =
  // (key row u / 8, dims 8 (u % 8) .. + 7 against dims 64 + 8 (u % 8) ..).
  // The angles' sines and cosines are taken before the tile is waited for,
  // so they overlap the load.
  constexpr int RIT = LOCAL ? kDecTile * 8 / NT : 0;  // items per thread
  float rc[RIT > 0 ? RIT : 1][8], rs[RIT > 0 ? RIT : 1][8];
  auto rope_angles = [&](int t) {
#pragma unroll
    for (int i = 0; i < RIT; ++i) {
      const int u = tid + i * NT, row = u >> 3, cp = u & 7;
      const int key = min(k_begin + t * kDecTile + row, k_end - 1);
      const float delta = (float)(j_first + key - pos);
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        float r = delta * p.rope_rev[cp * 8 + e];
        r -= rintf(r);
        sincos_rev(r, &rs[i][e], &rc[i][e]);
      }
    }
  };
  auto rope_tile = [&](auto SLOT) {
#pragma unroll
    for (int i = 0; i < RIT; ++i) {
      const int u = tid + i * NT, row = u >> 3, cp = u & 7;
      lds_u32x4_t* lo = reinterpret_cast<lds_u32x4_t*>(
          ktile(SLOT) + row * 256 + ((cp ^ (row & 15)) << 4));
      lds_u32x4_t* hi = reinterpret_cast<lds_u32x4_t*>(
          ktile(SLOT) + row * 256 + (((cp + 8) ^ (row & 15)) << 4));
      u32x4_t a = *lo, c = *hi;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const float x0 = bf16_lo(a[e]), x1 = bf16_hi(a[e]);
        const float y0 = bf16_lo(c[e]), y1 = bf16_hi(c[e]);
        const float c0 = rc[i][2 * e], s0 = rs[i][2 * e];
        const float c1 = rc[i][2 * e + 1], s1 = rs[i][2 * e + 1];
        a[e] = pack_bf16(x0 * c0 - y0 * s0, x1 * c1 - y1 * s1);
        c[e] = pack_bf16(y0 * c0 + x0 * s0, y1 * c1 + x1 * s1);
      }
      *lo = a;
      *hi = c;
    }
  };

  constexpr auto C0 = std::integral_constant<int, 0>{};
  // after a wave's dequantisation: its LDS writes are complete before any
  // read of the staging tiles (KSPLIT: the wave reads only its own rows)
  auto dequant_done = [&]() {
    if constexpr (KSPLIT)
      asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
    else
      __syncthreads();
  };
  if constexpr (KR == 1) {
    // one tile per workgroup (the planner guarantees it): load, wait, use
    if (ntiles > 0) {
      if constexpr (F8) {
        issue8_k(0, C0);
        issue8_v(0, C0);
      } else {
        issue_k(0, C0);
        issue_v(0, C0);
      }
      if constexpr (LOCAL) rope_angles(0);
      wait_vmcnt<0>();
      __syncthreads();
      if constexpr (F8) {
        dequant(C0, C0);
        dequant_done();
      }
      if constexpr (LOCAL) {
        rope_tile(C0);
        __syncthreads();
      }
      consume(0, C0, C0);
    }
  } else {
    // Step s (after its barrier) loads V of tile s + VR - 1, then K of tile
    // s + KR - 1, into the slots tile s - 1 used; the prologue issues what
    // steps -(KR - 1) .. -1 would have.
    constexpr int DK = KR - 1, DV = VR - 1;
    constexpr int PER = KR == VR ? KR : KR * VR;  // slot pattern period
    auto load_k = [&](int t, auto KS) {
      if constexpr (F8) issue8_k(t, KS); else issue_k(t, KS);
    };
    auto load_v = [&](int t, auto VS) {
      if constexpr (F8) issue8_v(t, VS); else issue_v(t, VS);
    };
    static_for<0, DK>([&](auto I) {
      constexpr int s0 = I - DK;
      if constexpr (s0 + DV >= 0) {
        if (s0 + DV < ntiles)
          load_v(s0 + DV, std::integral_constant<int, (s0 + DV) % VR>{});
      }
      if (s0 + DK < ntiles)
        load_k(s0 + DK, std::integral_constant<int, (s0 + DK) % KR>{});
    });
    for (int t0 = 0; t0 < ntiles; t0 += PER) {
      static_for<0, PER>([&](auto S) {
        const int t = t0 + S;
        if (t < ntiles) {
          if constexpr (LOCAL) rope_angles(t);
          // tile t has landed (this wave's rows) once at most the K tile
          // issued after V of tile t is outstanding; the barrier publishes
          // every wave's rows and frees the slots of tile t - 1
          if (DK > DV && t + 1 < ntiles)
            wait_vmcnt<LPI>();
          else
            wait_vmcnt<0>();
          if constexpr (!KSPLIT) __syncthreads();
          if (t + DV < ntiles)
            load_v(t + DV, std::integral_constant<int, (S + DV) % VR>{});
          if (t + DK < ntiles)
            load_k(t + DK, std::integral_constant<int, (S + DK) % KR>{});
          if constexpr (F8) {
            dequant(std::integral_constant<int, S % KR>{},
                    std::integral_constant<int, S % VR>{});
            dequant_done();
          }
          if constexpr (LOCAL) {
            rope_tile(std::integral_constant<int, S % KR>{});
            __syncthreads();
          }
          consume(t, std::integral_constant<int, S % KR>{},
                  std::integral_constant<int, S % VR>{});
        }
      });
    }
  }

  if constexpr (KSPLIT) {
    // ---- each wave holds (m, l, o) of all 16 heads over its own keys (row
    // r: heads 4 r ..; the row's 16 lanes split l over keys and o over
    // dims).  Once every wave is done with the ring, they meet in LDS and
    // are merged with the log-sum-exp rule: with M the largest of the four
    // maxima, l = sum 2^(m_w - M) l_w, o = sum 2^(m_w - M) o_w.
#pragma unroll
    for (int hl = 0; hl < HW; ++hl) lsum[hl] = row_sum(lsum[hl]);
    float* const cm = reinterpret_cast<float*>(smem);   // [4 waves][16]
    float* const cl = cm + WAVES * HPW;                  // [4][16]
    float* const co = cl + WAVES * HPW;                  // [4][16][128]
    __syncthreads();
#pragma unroll
    for (int hl = 0; hl < HW; ++hl) {
      const int h = hrow + hl;
      if (jl == 0) {
        cm[w * HPW + h] = m[hl];
        cl[w * HPW + h] = lsum[hl];
      }
      float* dst = co + (w * HPW + h) * kD + jl;
#pragma unroll
      for (int e = 0; e < 8; ++e) dst[16 * e] = o[hl][e];
    }
    __syncthreads();
    // thread: head tid / 16, dims 8 (tid % 16) .. + 7
    const int h = tid >> 4, d0 = (tid & 15) * 8;
    float M = cm[h];
#pragma unroll
    for (int v = 1; v < WAVES; ++v) M = fmaxf(M, cm[v * HPW + h]);
    float L = 0.0f, O[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) O[e] = 0.0f;
#pragma unroll
    for (int v = 0; v < WAVES; ++v) {
      const float c = fast_exp2(cm[v * HPW + h] - M);
      L += c * cl[v * HPW + h];
      const float* src = co + (v * HPW + h) * kD + d0;
#pragma unroll
      for (int e = 0; e < 8; ++e) O[e] += c * src[e];
    }
    float* dst = part + 2 * HPW + h * kD + d0;
#pragma unroll
    for (int e = 0; e < 8; ++e) dst[e] = O[e];
    if ((tid & 15) == 0) {
      part[h] = M;
      part[HPW + h] = L;
    }
    return;
  }

  // ---- reduce over the four key groups and the 64 key lanes, write
#pragma unroll
  for (int hl = 0; hl < HW; ++hl) {
#pragma unroll
    for (int e = 0; e < 8; ++e) o[hl][e] = rows_sum(o[hl][e]);
    lsum[hl] = wave_sum(lsum[hl]);
  }
  if (kg == 0) {
#pragma unroll
    for (int hl = 0; hl < HW; ++hl) {
      float* dst = part + 2 * HPW + (w * HW + hl) * kD + jl;
#pragma unroll
      for (int e = 0; e < 8; ++e) dst[16 * e] = o[hl][e];
    }
  }
  if (lane == 0) {
#pragma unroll
    for (int hl = 0; hl < HW; ++hl) {
      part[w * HW + hl] = m[hl];
      part[HPW + w * HW + hl] = lsum[hl];
    }
  }
}

// Merge the split partials of one (sequence, query head, quarter of the
// head dimension): with M the largest split maximum,
// o = sum 2^(m_s - M) o_s / sum 2^(m_s - M) l_s.  256 threads = 32 split
// lanes x 8 float4 columns (thread = 8 lane + column); lane j takes splits
// j, j + 32, ... with every load of the call in flight at once.  M is found
// first (wave maximum, then across the four waves), so the weighted sums
// need no rescaling and the split lanes combine by plain addition.
__global__ __launch_bounds__(256) void decode_merge_kernel(
    const DecodeParams p, int hpw) {
  int dq = blockIdx.x & 3;
  int h = (blockIdx.x >> 2) % kHq;
  int b = (blockIdx.x >> 2) / kHq;
  {
    // the split kernel's XCD grouping (one (sequence, KV head) pair per
    // XCD): this workgroup's pair is the one whose splits ran on its XCD
    const int X = p.xcds, BG = (int)gridDim.x / (kGroup * 4);
    if (hpw == kGroup && X > 1 && BG % X == 0) {
      const int xcd = blockIdx.x % X, s = blockIdx.x / X;
      const int bg = xcd + X * (s / (kGroup * 4)), r = s % (kGroup * 4);
      b = bg / kHkv;
      h = (bg % kHkv) * kGroup + r / 4;
      dq = r % 4;
    }
  }
  const int g = h / kGroup, hh = h % kGroup;
  const int hg = hh / hpw, hl = hh % hpw;  // head group, head within it
  const int pf = hpw * (kD + 2);
  const float* base =
      p.part + ((size_t)(b * kHkv + g) * (kGroup / hpw) + hg) * p.splits * pf;
  const int tid = threadIdx.x;
  const int c4 = tid & 7, sl = tid >> 3, w = tid >> 6;
  const int d = dq * 32 + c4 * 4;
  __shared__ float wmax[4];
  __shared__ float4 wsum[4][8];
  __shared__ float wl[4][8];
  // every split's loads at once (the planner keeps splits <= kMaxSplits)
  constexpr int kPer = kMaxSplits / 32;
  float ms[kPer], ls[kPer];
  float4 os[kPer];
  const int nper = (p.splits + 31) / 32;  // batches holding a split
#pragma unroll
  for (int i = 0; i < kPer; ++i) {
    ms[i] = -INFINITY;
    ls[i] = 0.0f;
    os[i] = make_float4(0.0f, 0.0f, 0.0f, 0.0f);
    if (i >= nper) continue;
    const int s = sl + 32 * i;
    const float* ps = base + (size_t)min(s, p.splits - 1) * pf;
    ms[i] = s < p.splits ? ps[hl] : -INFINITY;
    ls[i] = ps[hpw + hl];
    os[i] = *reinterpret_cast<const float4*>(ps + 2 * hpw + hl * kD + d);
  }
  float mx = -INFINITY;
#pragma unroll
  for (int i = 0; i < kPer; ++i) mx = fmaxf(mx, ms[i]);
  mx = wave_max(mx);
  if ((tid & 63) == 0) wmax[w] = mx;
  __syncthreads();
  const float M = fmaxf(fmaxf(wmax[0], wmax[1]), fmaxf(wmax[2], wmax[3]));
  // splits without keys (m = -inf) and padding lanes get weight 0
  float L = 0.0f;
  float4 O = make_float4(0.0f, 0.0f, 0.0f, 0.0f);
#pragma unroll
  for (int i = 0; i < kPer; ++i) {
    const float c = fast_exp2(ms[i] - M);
    L += ls[i] * c;
    O.x += os[i].x * c;
    O.y += os[i].y * c;
    O.z += os[i].z * c;
    O.w += os[i].w * c;
  }
  // sum over the 32 split lanes: the 8 lanes of a wave that share a column
  // are 8 apart, then the four waves
  L = stride8_sum(L);
  O.x = stride8_sum(O.x);
  O.y = stride8_sum(O.y);
  O.z = stride8_sum(O.z);
  O.w = stride8_sum(O.w);
  if ((tid & 63) < 8) {
    wsum[w][c4] = O;
    wl[w][c4] = L;
  }
  __syncthreads();
  if (tid < 8) {
    float Lt = 0.0f;
    float4 r = make_float4(0.0f, 0.0f, 0.0f, 0.0f);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      Lt += wl[j][c4];
      r.x += wsum[j][c4].x;
      r.y += wsum[j][c4].y;
      r.z += wsum[j][c4].z;
      r.w += wsum[j][c4].w;
    }
    const float inv = 1.0f / Lt;
    *reinterpret_cast<float4*>(p.out + ((size_t)b * kHq + h) * kD + d) =
        make_float4(r.x * inv, r.y * inv, r.z * inv, r.w * inv);
  }
}


template <bool F8>
hipError_t launch_split(const DecodeParams& p, const DecodePlan& plan,
                        bool local, hipStream_t s) {
  if (local && plan.heads_per_wg == kLocalSmallHeads) {
    // small batches: HG workgroups (head groups) share each tile
    constexpr int HG = kGroup / kLocalSmallHeads;
    const int grid = (p.units + p.xcds - 1) / p.xcds * p.xcds * HG;
    if (p.tiles_per_split != 1) return hipErrorInvalidValue;
    hipLaunchKernelGGL((decode_split_kernel<kLocalSmallWaves, kLocalSmallHeads,
                                            1, 1, true, false, F8>),
                       dim3(grid), dim3(64 * kLocalSmallWaves), 0, s, p);
  } else if (local) {
    hipLaunchKernelGGL(
        (decode_split_kernel<kLocalWaves, kGroup, 2, 2, true, false, F8>),
        dim3(p.units), dim3(64 * kLocalWaves), 0, s, p);
  } else {
    hipLaunchKernelGGL(
        (decode_split_kernel<kGlobalWaves, kGroup, kGlobalKRing,
                             kGlobalVRing, false, true, F8>),
        dim3(p.units), dim3(64 * kGlobalWaves), 0, s, p);
  }
  return hipGetLastError();
}

}  // namespace

hipError_t launch_decode(const DecodeParams& p, const DecodePlan& plan,
                         bool local, bool fp8, int B, hipStream_t s) {
  hipError_t e = fp8 ? launch_split<true>(p, plan, local, s)
                     : launch_split<false>(p, plan, local, s);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(decode_merge_kernel, dim3(B * kHq * 4), dim3(256), 0, s,
                     p, plan.heads_per_wg);
  return hipGetLastError();
}

}  // namespace gqa
