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
// A block can also be taken as predicted together, as a block-diffusion
// drafter does (shishifenxi.com section 04): then every query of the block
// sees the whole block (global layers only, where a query's position
// matters only through the keys it sees).
//
// Design (gfx950, v_mfma_f32_32x32x16_bf16, fp32 accumulation):
//  * Rows are (query, head) pairs: a workgroup takes 16 query tokens x the
//    16 query heads of one KV head (256 rows, 8 waves of 32 rows = 2 tokens
//    x 16 heads), so every K/V tile staged in LDS serves 256 rows (GQA
//    reuse).  8 waves (two per SIMD) and 224 VGPRs each: one workgroup per
//    CU.  Local layers with key splits (verification) take 8 tokens per
//    workgroup (4 waves, 128 rows): there each workgroup holds one or two
//    tiles and its chain of loads and products is latency, which half the
//    rows shorten.
//  * Scores are formed transposed, S^T = K Q^T, so each lane ends up owning
//    one row and 16 keys of every 32-key block: the row maximum is 31 in-lane
//    max operations plus one exchange with the partner lane 32 away, and the
//    probabilities, rounded to bf16, are directly the B operand of the P.V
//    product (O^T = V^T P^T) -- P never goes through LDS.
//  * Tiles of 64 keys stream into a four-slot LDS ring with direct-to-LDS
//    loads (no VGPR staging).  Rows of 256 bytes (one key), 16-byte chunks
//    XOR-swizzled per row; the V^T operand is read with ds_read_b64_tr_b16.
//  * Online softmax in the log2 domain with a lazy maximum (rescale only when
//    a score exceeds the running maximum by more than 2^8); masks are applied
//    only on tiles that cross the causal diagonal or the window edge.
//  * Local layers: a pre-pass rotates the window's cached keys and the
//    block's keys into the workspace once; queries are rotated when loaded.
//    Both use offsets relative to p0 (<R_i q, R_j k> is unchanged by a common
//    shift), keeping the fp32 angle arithmetic small.
//  * Verification splits each sequence's key range across workgroups (down
//    to one tile each) and merges the partial rows in a second kernel; a
//    partial row is the split's output divided by its own denominator, as
//    fp16 scaled by a power of two that puts the row's largest magnitude in
//    [2^14, 2^15), plus the maximum, the denominator and the inverse scale in
//    fp32 (fp16's 11-bit significand keeps this intermediate rounding an
//    eighth of a bf16 rounding at the same 2 bytes per element).
#include <type_traits>

#include "device_common.h"
#include "internal.h"

namespace gqa {

namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));

constexpr float kTauB = 8.0f;
constexpr int kTileB = kBlkTile * 256;      // one 64-key tile of K or V
constexpr int kSlotB = 2 * kTileB;          // K tile, then V tile
constexpr int kRing = 4;                    // tile slots in LDS (128 KB)
// Partial row of a key split, in 4-byte words: words 0..63 the row's output
// over the split normalised by its own denominator, times 2^(15 - e) where
// 2^(e - 1) <= max |o / l| < 2^e, as 128 fp16; word 64 the maximum m, word
// 65 the denominator l, word 66 the inverse scale 2^(e - 15) (fp32), word 67
// padding.
constexpr int kPartRow = 68;
// the exponent e is clamped so both scales stay normal fp32 numbers (rows
// below 2^-100 keep their absolute error far under any bf16 rounding)
constexpr int kPartExpMin = -100;
// fp8 caches (verification and drafted blocks, key splits only): code tiles
// (64 rows of one KV head's 128 E4M3 codes for K, then for V) and their
// rows' scales stream into a ring of kRing slots; each wave turns its own
// rows of a landed tile into bf16 codes in one of two staging slots laid out
// as the bf16 ring slots are, so the products run unchanged on them, and
// the scores take the K scales and the weights the V scales.  The block's
// own tokens (bf16, not in the cache) sit in LDS for the whole call.
constexpr int kCodeTileB = kBlkTile * kD;               // 8 KB of codes
constexpr int kCodeSlotB = 2 * kCodeTileB;              // K codes, V codes
constexpr int kScaleSlotB = 2 * kBlkTile * 4;           // 64 K, 64 V scales
constexpr int kF8Codes = 2 * kSlotB;                    // after the staging
constexpr int kF8BlkRows = GQA_MAX_VERIFY;
// LDS of the fp8 variant with `waves` waves: staging, code ring, then the
// scale ring (per slot, for K then V, each wave's 64 scale words: lane l
// the scale of its row l % (64 / waves)), the staging scales, the block's
// rows and (local layers) the query RoPE table.
struct F8Lds {
  int raw, raw_slot, st_sc, blk, rtab, size;
};
constexpr F8Lds f8_lds(int waves, int qpw, bool local) {
  F8Lds l{};
  l.raw_slot = 2 * waves * 256;
  l.raw = kF8Codes + kRing * kCodeSlotB;
  l.st_sc = l.raw + kRing * l.raw_slot;
  l.blk = l.st_sc + 2 * kScaleSlotB;
  l.rtab = l.blk + 2 * kF8BlkRows * 256;
  l.size = l.rtab + (local ? qpw * 32 * 16 : 0);
  return l;
}
static_assert(f8_lds(kBlkQpw / 2, kBlkQpw, false).size <= 160 * 1024 &&
                  f8_lds(kBlkQpwSmall / 2, kBlkQpwSmall, true).size <=
                      160 * 1024,
              "fp8 block kernel LDS");

__device__ __forceinline__ uint32_t pack_f16(float lo, float hi) {
  typedef _Float16 f16x2_t __attribute__((ext_vector_type(2)));
  f16x2_t r = {(_Float16)lo, (_Float16)hi};
  return __builtin_bit_cast(uint32_t, r);
}
__device__ __forceinline__ float f16_lo(uint32_t w) {
  return (float)__builtin_bit_cast(_Float16, (uint16_t)(w & 0xFFFFu));
}
__device__ __forceinline__ float f16_hi(uint32_t w) {
  return (float)__builtin_bit_cast(_Float16, (uint16_t)(w >> 16));
}

typedef short v4i16_t __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) bf16x8_t lds_bf16x8_t;
typedef __attribute__((address_space(3))) v4i16_t lds_v4i16_t;
typedef __attribute__((address_space(3))) u32x4_t lds_u32x4_t;

// Direct-to-LDS load of 16 bytes per lane: lane l's bytes land at LDS byte
// address lds + 16 l (lds wave-uniform).  Inline assembly, so the compiler
// does not hold every later LDS read behind it; the caller waits
// (s_waitcnt vmcnt) and publishes with a barrier.  M0 carries the LDS
// address; it is saved and restored, with one wait state before the load.
__device__ __forceinline__ void dma16(const uint16_t* src, uint32_t lds) {
  uint32_t saved;
  asm volatile(
      "s_mov_b32 %0, m0\n\t"
      "s_mov_b32 m0, %2\n\t"
      "s_nop 0\n\t"
      "global_load_lds_dwordx4 %1, off\n\t"
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
      "global_load_lds_dwordx4 %1, %2\n\t"
      "s_mov_b32 m0, %0"
      : "=&s"(saved)
      : "v"(off), "s"(base), "s"(lds)
      : "memory");
}
// Direct-to-LDS load of 4 bytes per active lane (lane l's word lands at
// lds + 4 l); lanes outside the exec mask load nothing.
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
// byte) as a bf16 pair, exactly (every E4M3 value is a bf16 value).
template <bool HI>
__device__ __forceinline__ uint32_t cvt_fp8x2_bf16(uint32_t w) {
  return __builtin_bit_cast(
      uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.0f, HI));
}
__device__ __forceinline__ void wait_vmcnt0() {
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
}
// s_waitcnt vmcnt(N): at most N of this wave's vector memory operations
// (here: tile loads) still outstanding.
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  asm volatile("s_waitcnt vmcnt(%0)" ::"i"(N) : "memory");
}

__device__ __forceinline__ int64_t ring_prior(int64_t pos0) {
  return pos0 < kW ? pos0 : kW;
}

// Local layers: write the RoPE-rotated keys of positions p0 - W' .. p0+n-1
// (W' = min(p0, 2048) cached positions before the block) into k_lin, rotated
// by their offset from p0.  16 lanes per key row: lane c takes dimensions
// 4c .. 4c + 3 against 64 + 4c .. of both KV heads, so each angle's sine and
// cosine serve both heads; 16 rows per 256-thread workgroup.
constexpr int kRopeRowsPerWG = 16;
__global__ __launch_bounds__(256) void rope_keys_kernel(const BlockParams p) {
  const int b = blockIdx.y;
  const int r = blockIdx.x * kRopeRowsPerWG + (threadIdx.x >> 4);
  const int c = threadIdx.x & 15;
  const int64_t pos0 = p.pos0[b];
  const int64_t wprior = ring_prior(pos0);
  if (r >= wprior + p.n) return;
  const int64_t j = pos0 - wprior + r;  // key position
  const uint16_t* src =
      j < pos0 ? p.k_cache + (int64_t)b * p.seq_stride +
                     (j & (kW - 1)) * kTokenElems
               : p.k_blk + ((int64_t)b * p.n + (j - pos0)) * kTokenElems;
  uint16_t* dst = p.k_lin + ((int64_t)b * p.klin_rows + r) * kTokenElems;
  const float delta = (float)(j - pos0);
  // angles of frequencies 4c .. 4c + 3 (dims 4c + i pair with 64 + 4c + i)
  float sn[4], cs[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    float t = delta * p.rope_rev[4 * c + i];
    t -= rintf(t);
    sincos_rev(t, &sn[i], &cs[i]);
  }
#pragma unroll
  for (int h = 0; h < kHkv; ++h) {
    const uint2 xw = *reinterpret_cast<const uint2*>(src + h * kD + 4 * c);
    const uint2 yw =
        *reinterpret_cast<const uint2*>(src + h * kD + kD / 2 + 4 * c);
    const float x[4] = {bf16_lo(xw.x), bf16_hi(xw.x), bf16_lo(xw.y),
                        bf16_hi(xw.y)};
    const float y[4] = {bf16_lo(yw.x), bf16_hi(yw.x), bf16_lo(yw.y),
                        bf16_hi(yw.y)};
    float a[4], e[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      a[i] = x[i] * cs[i] - y[i] * sn[i];
      e[i] = y[i] * cs[i] + x[i] * sn[i];
    }
    *reinterpret_cast<uint2*>(dst + h * kD + 4 * c) =
        make_uint2(pack_bf16(a[0], a[1]), pack_bf16(a[2], a[3]));
    *reinterpret_cast<uint2*>(dst + h * kD + kD / 2 + 4 * c) =
        make_uint2(pack_bf16(e[0], e[1]), pack_bf16(e[2], e[3]));
  }
}

// Largest of 16 scores as a tree of three-input maxima (depth 3, where a
// running maximum would chain 16 dependent instructions).
__device__ __forceinline__ float max16(const f32x16_t& v) {
  float m[5];
#pragma unroll
  for (int i = 0; i < 5; ++i)
    m[i] = fmaxf(fmaxf(v[3 * i], v[3 * i + 1]), v[3 * i + 2]);
  return fmaxf(fmaxf(fmaxf(m[0], m[1]), m[2]),
               fmaxf(fmaxf(m[3], m[4]), v[15]));
}

// Tile t goes to ring slot t % 4, loaded three tiles ahead (direct-to-LDS,
// so tile t + 3 is in flight while tile t is consumed).  K chunk c of row r
// sits at chunk
// slot c ^ (r & 15), so the 32 lanes reading one chunk of 32 consecutive
// keys hit distinct banks; V chunk c at slot c ^ X(r & 3), X = {0, 4, 10,
// 14}: the four keys of a 16-lane group of ds_read_b64_tr_b16, and the 64
// bytes of each key read by a 32-lane half, land on distinct banks.
template <int QPW, bool LOCAL, bool SPLIT, bool OUT_F32, bool F8 = false>
__global__ __launch_bounds__(QPW * 32, 1) void block_attn_kernel(
    const BlockParams p) {
  static_assert(!F8 || SPLIT, "fp8 caches: key-split calls only");
  constexpr F8Lds L8 = f8_lds(QPW / 2, QPW, LOCAL);
  constexpr int WAVES = QPW / 2;  // waves of 32 rows (2 tokens x 16 heads)
  constexpr int RING = kRing;
  constexpr int ROWS = QPW * kGroup;
  constexpr int RPW = kBlkTile / WAVES;   // tile rows each wave loads
  constexpr int LPT = RPW / 4;            // 1-KB loads per K or V tile per wave
  __shared__ __attribute__((aligned(16))) uint8_t
      smem[F8 ? L8.size : RING * kSlotB];
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int hi5 = lane >> 5;
  const int row = lane & 31;

  // Work items are (sequence, KV head, query group, key split); with key
  // splits a workgroup takes one item.  Without them (prefill) the grid is
  // at most one workgroup per CU and each workgroup walks several items in
  // snake order (w, 2G - 1 - w, 2G + w, ...), pairing a long key range with
  // a short one, so no second dispatch round starts cold.  Items with the
  // longest key ranges come first.
  const int items = p.splits * p.qgroups * kHkv * p.batch;
  const int G = gridDim.x;
  const int walks = SPLIT ? 1 : (items + G - 1) / G;
  for (int j = 0; j < walks; ++j) {
  const int item = SPLIT ? (int)blockIdx.x
                   : (j & 1) ? (j + 1) * G - 1 - (int)blockIdx.x
                             : j * G + (int)blockIdx.x;
  if (item >= items) break;  // uniform across the workgroup
  if (j > 0) __syncthreads();  // the previous item's waves are done with LDS
  int bid = item;
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
  // Last key position each query of the group sees: its own (causal inside
  // the block), or the block's last one when the block's tokens are
  // predicted together (no order inside the block; layers without RoPE).
  const int blk_last = pos0 + p.n - 1;
  const int see_first = p.together ? blk_last : i_first;
  const int k_lo = LOCAL ? max(0, i_first - (kW - 1)) : 0;
  const int k_hi = (p.together ? blk_last : i_last) + 1;
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
  const int qsee = p.together ? blk_last : qpos;
  const int klin0 = pos0 - (int)ring_prior(pos0);  // position of k_lin row 0

  // Local layers: the sines and cosines of the workgroup's 16 tokens x 64
  // frequencies, taken once (each thread one token and two frequencies) into
  // the last ring slot, which no tile uses before the first step's barrier;
  // the 16 lanes of a token (one per head) then read them instead of each
  // evaluating its own.  Entry 32 t + j holds (sin, cos) of frequencies 2j
  // and 2j + 1 at token q_first + t.
  float4* const rtab = reinterpret_cast<float4*>(
      smem + (F8 ? L8.rtab : (RING - 1) * kSlotB));
  if constexpr (LOCAL) {
    static_assert(WAVES * 64 == QPW * 32, "one table entry per thread");
    const int t = tid >> 5, j = tid & 31;
    const float tok = (float)min(q_first + t, q_last);
    float r0 = tok * p.rope_rev[2 * j], r1 = tok * p.rope_rev[2 * j + 1];
    r0 -= rintf(r0);
    r1 -= rintf(r1);
    float4 e;
    sincos_rev(r0, &e.x, &e.y);
    sincos_rev(r1, &e.z, &e.w);
    rtab[tid] = e;
    __syncthreads();
  }

  // ---- Q^T operand: 8 k-steps of 16 dims, this lane's 8 dims of each
  bf16x8_t qreg[8];
  {
    const uint16_t* qrow =
        p.q + (((int64_t)b * p.n + qic) * kHq + head) * kD + 8 * hi5;
    uint4 raw[8];
#pragma unroll
    for (int k = 0; k < 8; ++k)
      raw[k] = *reinterpret_cast<const uint4*>(qrow + 16 * k);
    // q is rotated (local layers) and multiplied by scale * log2(e) in fp32,
    // then rounded to bf16 once: the products then come out in log2 units
    // and the softmax needs no per-score multiply
    const float c = p.scale_log2;
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      uint32_t* lo = reinterpret_cast<uint32_t*>(&raw[k]);
      uint32_t* hi = reinterpret_cast<uint32_t*>(&raw[k + 4]);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        float x0 = bf16_lo(lo[e]), x1 = bf16_hi(lo[e]);
        float y0 = bf16_lo(hi[e]), y1 = bf16_hi(hi[e]);
        if (LOCAL) {
          // frequencies 16k + 8 hi5 + 2e and + 1 at this row's token
          const float4 sc = rtab[32 * (qic - q_first) + 8 * k + 4 * hi5 + e];
          const float s0 = sc.x, c0 = sc.y, s1 = sc.z, c1 = sc.w;
          const float a0 = x0 * c0 - y0 * s0, a1 = x1 * c1 - y1 * s1;
          const float b0 = y0 * c0 + x0 * s0, b1 = y1 * c1 + x1 * s1;
          x0 = a0, x1 = a1, y0 = b0, y1 = b1;
        }
        lo[e] = pack_bf16(x0 * c, x1 * c);
        hi[e] = pack_bf16(y0 * c, y1 * c);
      }
    }
#pragma unroll
    for (int k = 0; k < 8; ++k) qreg[k] = __builtin_bit_cast(bf16x8_t, raw[k]);
  }
  // The ring waits below count only the tile loads, so the q loads complete
  // here; passing q through an (empty) asm tells the compiler they are done
  // (it cannot see waits inside asm and would otherwise wait again before
  // every use in the loop).
  wait_vmcnt0();
#pragma unroll
  for (int k = 0; k < 8; ++k) asm volatile("" : "+v"(qreg[k]));

  const uint16_t* kc_base = p.k_cache + (int64_t)b * p.seq_stride + g * kD;
  const uint16_t* vc_base = p.v_cache + (int64_t)b * p.seq_stride + g * kD;
  const uint16_t* kb_base = p.k_blk + (int64_t)b * p.n * kTokenElems + g * kD;
  const uint16_t* vb_base = p.v_blk + (int64_t)b * p.n * kTokenElems + g * kD;
  const uint16_t* kl_base =
      p.k_lin + (int64_t)b * p.klin_rows * kTokenElems + g * kD;

  // Local layers read their keys rotated: from the pre-rotated copy in the
  // workspace (KLIN, prefill: a key serves many workgroups), or raw from the
  // ring and the block, rotated in LDS once a tile lands (ROTK, split
  // verification: each key serves one workgroup).
  constexpr bool ROTK = LOCAL && SPLIT;
  constexpr bool KLIN = LOCAL && !SPLIT;
  auto k_src = [&](int j) -> const uint16_t* {
    if (KLIN) return kl_base + (j - klin0) * kTokenElems;
    if (j >= pos0) return kb_base + (j - pos0) * kTokenElems;
    return kc_base + (LOCAL ? (j & (kW - 1)) : j) * kTokenElems;
  };
  auto v_src = [&](int j) -> const uint16_t* {
    if (j >= pos0) return vb_base + (j - pos0) * kTokenElems;
    return vc_base + (LOCAL ? (j & (kW - 1)) : j) * kTokenElems;
  };

  // Wave w fills tile rows RPW w .. RPW (w+1) - 1, four rows (1 KB) per
  // load: lane l takes row RPW w + 4i + l/16 and chunk slot l % 16.  Keys
  // past the range repeat its last key (masked).
  const uint32_t lds_base = (uint32_t)(uintptr_t)smem;
  const int rsub = lane >> 4, cs = lane & 15;
  auto vswz = [](int r) { return 4 * (r & 3) + 2 * ((r >> 1) & 1); };
  // byte offsets of this lane's chunks from the tile's first key row
  uint32_t kdma[LPT], vdma[LPT];
#pragma unroll
  for (int i = 0; i < LPT; ++i) {
    const int r = RPW * w + 4 * i + rsub;
    kdma[i] = r * (kTokenElems * 2) + ((cs ^ (r & 15)) << 4);
    vdma[i] = r * (kTokenElems * 2) + ((cs ^ vswz(r)) << 4);
  }
  auto issue_tile = [&](int t, auto SLOT) {
    const int kb = k_lo + (t_begin + t) * kBlkTile;
    const uint32_t kl = __builtin_amdgcn_readfirstlane(
        lds_base + SLOT * kSlotB + w * RPW * 256);
    // A full tile whose rows are consecutive in one buffer loads from a
    // wave-uniform base; otherwise (range end, cache/block boundary, ring
    // wrap) each row is located on its own.
    const bool full = kb + kBlkTile <= k_hi;
    const bool in_cache = kb + kBlkTile <= pos0, in_blk = kb >= pos0;
    const int ring = LOCAL ? (kb & (kW - 1)) : kb;
    const uint16_t* kt =
        !full ? nullptr
        : KLIN ? kl_base + (kb - klin0) * kTokenElems
        : in_cache ? (!LOCAL || ring + kBlkTile <= kW
                          ? kc_base + ring * kTokenElems : nullptr)
        : in_blk ? kb_base + (kb - pos0) * kTokenElems : nullptr;
    const uint16_t* vt =
        !full ? nullptr
        : in_cache ? (!LOCAL || ring + kBlkTile <= kW
                          ? vc_base + ring * kTokenElems : nullptr)
        : in_blk ? vb_base + (kb - pos0) * kTokenElems : nullptr;
    if (kt) {
#pragma unroll
      for (int i = 0; i < LPT; ++i) dma16(kt, kdma[i], kl + i * 1024);
    } else {
#pragma unroll
      for (int i = 0; i < LPT; ++i) {
        const int r = RPW * w + 4 * i + rsub;
        dma16(k_src(min(kb + r, k_hi - 1)) + ((cs ^ (r & 15)) << 3),
              kl + i * 1024);
      }
    }
    if (vt) {
#pragma unroll
      for (int i = 0; i < LPT; ++i)
        dma16(vt, vdma[i], kl + kTileB + i * 1024);
    } else {
#pragma unroll
      for (int i = 0; i < LPT; ++i) {
        const int r = RPW * w + 4 * i + rsub;
        dma16(v_src(min(kb + r, k_hi - 1)) + ((cs ^ vswz(r)) << 3),
              kl + kTileB + i * 1024);
      }
    }
  };

  // ---- fp8 caches.  Codes: sequence b at byte b * seq_stride, rows of
  // 2 x 128 codes; scales [B][2][capacity].  Wave w loads code rows
  // RPW w .. RPW (w+1) - 1 of tile t into ring slot t % RING (lane l: row
  // RPW w + 8i + l / 8, codes 16 (l % 8) .. + 15) and the rows' K and V
  // scales (lane l: row RPW w + l % RPW; every lane loads, as a
  // direct-to-LDS load places lane l's word at its base + 4 l).  Rows at
  // block positions (not cached yet)
  // read the slot they map to and are replaced from the block's rows when
  // dequantised; rows past the range repeat its last key (masked).
  constexpr int LPT8 = RPW / 8;         // 1-KB code loads per K (V) tile
  constexpr int LPI8 = 2 * LPT8 + 2;    // loads of one tile per wave
  const uint8_t* k8_base = p.k8 + (int64_t)b * p.seq_stride + g * kD;
  const uint8_t* v8_base = p.v8 + (int64_t)b * p.seq_stride + g * kD;
  const float* ks_base =
      p.k_scale + (int64_t)b * p.scale_stride + (int64_t)g * p.capacity;
  const float* vs_base =
      p.v_scale + (int64_t)b * p.scale_stride + (int64_t)g * p.capacity;
  const int crow = lane >> 3, cch = lane & 7;
  auto slot8 = [](int j) { return LOCAL ? (j & (kW - 1)) : j; };
  auto issue_tile8 = [&](int t, auto SLOT) {
    const int kb = k_lo + (t_begin + t) * kBlkTile;
    const uint32_t cb = __builtin_amdgcn_readfirstlane(
        lds_base + kF8Codes + SLOT * kCodeSlotB + RPW * w * kD);
#pragma unroll
    for (int i = 0; i < LPT8; ++i) {
      const int j = min(kb + RPW * w + 8 * i + crow, k_hi - 1);
      const int64_t off = (int64_t)slot8(j) * kTokenElems + cch * 16;
      dma16(reinterpret_cast<const uint16_t*>(k8_base + off), cb + i * 1024);
      dma16(reinterpret_cast<const uint16_t*>(v8_base + off),
            cb + kCodeTileB + i * 1024);
    }
    const uint32_t sb = __builtin_amdgcn_readfirstlane(
        lds_base + L8.raw + SLOT * L8.raw_slot + w * 256);
    const int j = min(kb + RPW * w + lane % RPW, k_hi - 1);
    dma4(ks_base + slot8(j), sb);
    dma4(vs_base + slot8(j), sb + WAVES * 256);
  };
  // Wave w's own rows of the landed tile in ring slot SLOT -> bf16 codes in
  // staging slot ST (exact), in the swizzled layouts the products read; a
  // row at a block position takes the block's bf16 row instead.  Lane l of
  // a row writes dims 16 (l % 8) .. + 15; lane 0 of the row its K and V
  // scales (1 for block rows) to the staging scales.
  auto dequant8 = [&](int t, auto SLOT, auto ST) {
    const int kb = k_lo + (t_begin + t) * kBlkTile;
    static_for<0, LPT8>([&](auto I) {
      const int r = RPW * w + 8 * I + crow;
      const int j = min(kb + r, k_hi - 1);
      const bool blk = j >= pos0;
      static_for<0, 2>([&](auto IV) {
        u32x4_t lo, hi;
        if (blk) {
          const uint32_t src = lds_base + L8.blk +
                               (IV * kF8BlkRows + (j - pos0)) * 256 + cch * 32;
          lo = *reinterpret_cast<const lds_u32x4_t*>(src);
          hi = *reinterpret_cast<const lds_u32x4_t*>(src + 16);
        } else {
          const u32x4_t c = *reinterpret_cast<const lds_u32x4_t*>(
              lds_base + kF8Codes + SLOT * kCodeSlotB + IV * kCodeTileB +
              r * kD + cch * 16);
#pragma unroll
          for (int e = 0; e < 2; ++e) {
            lo[2 * e] = cvt_fp8x2_bf16<false>(c[e]);
            lo[2 * e + 1] = cvt_fp8x2_bf16<true>(c[e]);
            hi[2 * e] = cvt_fp8x2_bf16<false>(c[e + 2]);
            hi[2 * e + 1] = cvt_fp8x2_bf16<true>(c[e + 2]);
          }
        }
        const int swz = IV ? vswz(r) : (r & 15);
        const uint32_t dst = lds_base + ST * kSlotB + IV * kTileB + r * 256;
        *reinterpret_cast<lds_u32x4_t*>(dst + (((2 * cch) ^ swz) << 4)) = lo;
        *reinterpret_cast<lds_u32x4_t*>(dst + (((2 * cch + 1) ^ swz) << 4)) =
            hi;
      });
      if (cch == 0) {
        // this row's scale words: wave w's lane r - RPW w
        const float* raw = reinterpret_cast<const float*>(
            smem + L8.raw + SLOT * L8.raw_slot + w * 256 + 4 * (r - RPW * w));
        float* st = reinterpret_cast<float*>(smem + L8.st_sc + ST * kScaleSlotB);
        st[r] = blk ? 1.0f : raw[0];
        st[kBlkTile + r] = blk ? 1.0f : raw[WAVES * 64];
      }
    });
  };
  // Local layers: each wave rotates its own rows of the staging K tile by
  // their keys' offsets from p0 (item i: row RPW w + 8i + l / 8, dims
  // 8 (l % 8) .. + 7 against 64 + 8 (l % 8) ..); the angles are taken while
  // the tile is in flight.
  float rc8[LPT8][8], rs8[LPT8][8];
  auto rope_angles8 = [&](int t) {
    const int kb = k_lo + (t_begin + t) * kBlkTile;
#pragma unroll
    for (int i = 0; i < LPT8; ++i) {
      const int j = min(kb + RPW * w + 8 * i + crow, k_hi - 1);
      const float delta = (float)(j - pos0);
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        float rr = delta * p.rope_rev[cch * 8 + e];
        rr -= rintf(rr);
        sincos_rev(rr, &rs8[i][e], &rc8[i][e]);
      }
    }
  };
  auto rope_own = [&](auto ST) {
#pragma unroll
    for (int i = 0; i < LPT8; ++i) {
      const int r = RPW * w + 8 * i + crow;
      const uint32_t rb = lds_base + ST * kSlotB + r * 256;
      lds_u32x4_t* lo =
          reinterpret_cast<lds_u32x4_t*>(rb + ((cch ^ (r & 15)) << 4));
      lds_u32x4_t* hi =
          reinterpret_cast<lds_u32x4_t*>(rb + (((cch + 8) ^ (r & 15)) << 4));
      u32x4_t a = *lo, c = *hi;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const float x0 = bf16_lo(a[e]), x1 = bf16_hi(a[e]);
        const float y0 = bf16_lo(c[e]), y1 = bf16_hi(c[e]);
        const float c0 = rc8[i][2 * e], s0 = rs8[i][2 * e];
        const float c1 = rc8[i][2 * e + 1], s1 = rs8[i][2 * e + 1];
        a[e] = pack_bf16(x0 * c0 - y0 * s0, x1 * c1 - y1 * s1);
        c[e] = pack_bf16(y0 * c0 + x0 * s0, y1 * c1 + x1 * s1);
      }
      *lo = a;
      *hi = c;
    }
  };

  // LDS read addresses.  K operand of k-step k: key 32be + row, chunk
  // 2k + hi5 (+ 8192 B for be = 1).  V^T operand of dim block d: the
  // 16-lane group G (keys + 4(G >> 1), dims + 16(G & 1)) transposes keys
  // 16c + 4(G >> 1) + e, e = (lane & 15) >> 2, at dims 32d + 16(G & 1) +
  // 4((lane & 15) & 3); keys + 8 are 2048 B further.
  uint32_t krd[8], vrd[4];
#pragma unroll
  for (int k = 0; k < 8; ++k)
    krd[k] = lds_base + row * 256 + (((2 * k + hi5) ^ (row & 15)) << 4);
  {
    const int G = lane >> 4, jl = lane & 15, ja = jl & 3, je = jl >> 2;
#pragma unroll
    for (int d = 0; d < 4; ++d)
      vrd[d] = lds_base + kTileB + (4 * (G >> 1) + je) * 256 +
               (((4 * d + 2 * (G & 1) + (ja >> 1)) ^ vswz(je)) << 4) +
               8 * (ja & 1);
  }

  f32x16_t O[4];
#pragma unroll
  for (int d = 0; d < 4; ++d)
#pragma unroll
    for (int i = 0; i < 16; ++i) O[d][i] = 0.0f;
  float m_run = -INFINITY, l_run = 0.0f;
  f32x16_t negmb;  // -(score base) of this lane's row, in all 16 entries
#pragma unroll
  for (int i = 0; i < 16; ++i) negmb[i] = 0.0f;

  auto consume = [&](int t, auto SLOT) {
    constexpr uint32_t so = SLOT * kSlotB;
    // ---- S^T = K Q^T for two 32-key blocks.  The K operands of block 0 are
    // all requested before its first product and those of block 1 while
    // block 0 multiplies, so no product waits on a fresh LDS read.
    // The accumulators start at -mb (mb: the row's running maximum, 0 while
    // it has none; the first product of each block adds onto the constant
    // vector negmb), so they end up holding s - mb in log2 units.
    const float mb = -negmb[0];
    // fp8: the products start from zero and take their keys' K scales below
    f32x16_t acc0;
#pragma unroll
    for (int i = 0; i < 16; ++i) acc0[i] = F8 ? 0.0f : negmb[i];
    f32x16_t S[2];
    bf16x8_t ka[2][8];
#pragma unroll
    for (int k = 0; k < 8; ++k)
      ka[0][k] = *reinterpret_cast<const lds_bf16x8_t*>(krd[k] + so);
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      S[0] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
          ka[0][k], qreg[k], k == 0 ? acc0 : S[0], 0, 0, 0);
      ka[1][k] = *reinterpret_cast<const lds_bf16x8_t*>(krd[k] + so + 8192);
    }
#pragma unroll
    for (int k = 0; k < 8; ++k)
      S[1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
          ka[1][k], qreg[k], k == 0 ? acc0 : S[1], 0, 0, 0);
    // The V^T operands of the first 16-key step of P.V are requested
    // meanwhile (they do not depend on the softmax).
    constexpr uint32_t vo = so;  // vrd[] already points into the V tile
    v4i16_t vt[2][4][2];  // [step parity][dim block][keys +0..3 | +8..11]
    auto read_vt = [&](int c, v4i16_t(&dst)[4][2]) {
#pragma unroll
      for (int d = 0; d < 4; ++d) {
        dst[d][0] = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            reinterpret_cast<lds_v4i16_t*>(vrd[d] + vo + c * 4096));
        dst[d][1] = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            reinterpret_cast<lds_v4i16_t*>(vrd[d] + vo + c * 4096 + 2048));
      }
    };
    read_vt(0, vt[0]);
    // issue order: 8 reads, then (product, read) x 8, then the 8 block-1
    // products interleaved with the 8 V^T reads
    __builtin_amdgcn_sched_group_barrier(0x100, 8, 0);
    static_for<0, 8>([&](auto) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
    });
    static_for<0, 8>([&](auto) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
    });

    // fp8: score s = product x (its key's K scale) - mb; the lane's keys of
    // block be, entry 4 qd + e, are 32 be + 8 qd + 4 hi5 + e
    const uint32_t scb = lds_base + L8.st_sc + SLOT * kScaleSlotB + 16 * hi5;
    if constexpr (F8) {
#pragma unroll
      for (int be = 0; be < 2; ++be)
#pragma unroll
        for (int qd = 0; qd < 4; ++qd) {
          const u32x4_t k4 = *reinterpret_cast<const lds_u32x4_t*>(
              scb + 4 * (32 * be + 8 * qd));
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            // the element goes through a scalar: a bit cast taken directly
            // on a vector element reads element 0 with this compiler
            const uint32_t kw = k4[e];
            S[be][4 * qd + e] =
                fmaf(S[be][4 * qd + e], __builtin_bit_cast(float, kw), -mb);
          }
        }
    }
    // ---- softmax update for this lane's row.  The maximum is taken on raw
    // scores, already scaled to log2 units and shifted by -mb: p = 2^(S).
    const int kb = k_lo + (t_begin + t) * kBlkTile;
    const bool edge = (kb + kBlkTile - 1 > see_first) ||
                      (LOCAL && kb <= i_last - kW);
    if (edge) {
      // key kb + off + 4 hi5 is visible iff off <= rel and (local)
      // off > rel - W
      const int rel = qsee - kb - 4 * hi5;
#pragma unroll
      for (int be = 0; be < 2; ++be)
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const int off = 32 * be + 8 * (i >> 2) + (i & 3);
          const bool ok = off <= rel && (!LOCAL || off > rel - kW);
          S[be][i] = ok ? S[be][i] : -INFINITY;
        }
    }
    // This lane's largest score (its 16 keys of each block), log2 units.
    // A row's two lanes (32 apart) decide together exactly as on the row
    // maximum would (x -> x + mb is monotonic), so the exchange with the
    // partner lane is only taken on the rare rescaling path.
    const float ml = fmaxf(max16(S[0]), max16(S[1])) + mb;
    if (__any(ml > m_run + kTauB)) {
      const float mt = xmax<32>(ml);  // tile max of the row
      const float mn = fmaxf(m_run, mt);
      const float alpha = mn == m_run ? 1.0f : fast_exp2(m_run - mn);
      m_run = mn;
      l_run *= alpha;
#pragma unroll
      for (int d = 0; d < 4; ++d)
#pragma unroll
        for (int i = 0; i < 16; ++i) O[d][i] *= alpha;
      // re-base this tile's scores (and the next tiles') on the new maximum;
      // a row that has seen no visible key yet keeps m = -inf and base 0,
      // which turns its -inf scores into zero weights
      const float nb = mn == -INFINITY ? 0.0f : mn;
      const float shift = mb - nb;
#pragma unroll
      for (int be = 0; be < 2; ++be)
#pragma unroll
        for (int i = 0; i < 16; ++i) S[be][i] += shift;
#pragma unroll
      for (int i = 0; i < 16; ++i) negmb[i] = -nb;
    }
    bf16x8_t P[4];  // 16-key contraction steps: (block be, half tt)
    // the denominator sums exactly the bf16 weights P.V uses, in four
    // independent partial sums (a single running sum would chain sixteen
    // dependent instructions)
    float lp[4] = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
    for (int be = 0; be < 2; ++be)
#pragma unroll
      for (int tt = 0; tt < 2; ++tt) {
        uint32_t w4[4], pv[4];
        // fp8: the V scales of keys 32 be + 8 (2 tt + h) + 4 hi5 + 0..3
        u32x4_t v4[2];
        if constexpr (F8) {
#pragma unroll
          for (int h = 0; h < 2; ++h)
            v4[h] = *reinterpret_cast<const lds_u32x4_t*>(
                scb + 4 * (kBlkTile + 32 * be + 8 * (2 * tt + h)));
        }
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const float p0 = fast_exp2(S[be][8 * tt + 2 * j]);
          const float p1 = fast_exp2(S[be][8 * tt + 2 * j + 1]);
          w4[j] = pack_bf16(p0, p1);
          lp[j] = dot2_bf16(w4[j], 0x3F803F80u, lp[j]);
          if constexpr (F8) {
            // the weight times its key's V scale, rounded once
            const uint32_t v0 = v4[j >> 1][2 * (j & 1)];
            const uint32_t v1 = v4[j >> 1][2 * (j & 1) + 1];
            pv[j] = pack_bf16(p0 * __builtin_bit_cast(float, v0),
                              p1 * __builtin_bit_cast(float, v1));
          } else {
            pv[j] = w4[j];
          }
        }
        P[2 * be + tt] = __builtin_bit_cast(
            bf16x8_t, make_uint4(pv[0], pv[1], pv[2], pv[3]));
      }
    l_run += (lp[0] + lp[1]) + (lp[2] + lp[3]);

    // ---- O^T += V^T P^T over four 16-key steps, four 32-dim blocks; the
    // operands of step c + 1 are read while step c multiplies
    static_for<0, 4>([&](auto C) {
      constexpr int c = C;
      if constexpr (c + 1 < 4) read_vt(c + 1, vt[(c + 1) & 1]);
#pragma unroll
      for (int d = 0; d < 4; ++d) {
        // keys 16c + 4 hi5 + 0..3, then + 8..11, at this lane's dimension
        const uint2 l2 = __builtin_bit_cast(uint2, vt[c & 1][d][0]);
        const uint2 h2 = __builtin_bit_cast(uint2, vt[c & 1][d][1]);
        const bf16x8_t a4 = __builtin_bit_cast(
            bf16x8_t, make_uint4(l2.x, l2.y, h2.x, h2.y));
        O[d] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a4, P[c], O[d], 0, 0,
                                                       0);
      }
    });
    static_for<0, 3>([&](auto) {
      static_for<0, 4>([&](auto) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 1);
        __builtin_amdgcn_sched_group_barrier(0x100, 2, 1);
      });
    });
    __builtin_amdgcn_sched_group_barrier(0x008, 4, 1);
  };

  // ROTK: thread i rotates items i, i + NT, ... of a landed K tile, item
  // u = (key row u / 8, dims 8 (u % 8) .. + 7 against dims 64 + 8 (u % 8)
  // ..), by the key's offset from p0 (the queries carry theirs); the sines
  // and cosines are taken before the tile is waited for, so they overlap
  // its load.
  constexpr int NT = WAVES * 64;
  constexpr int RIT = kBlkTile * 8 / NT;  // items per thread
  static_assert(RIT * NT == kBlkTile * 8, "whole items per thread");
  float rc[RIT][8], rs[RIT][8];
  auto rope_angles = [&](int t) {
    const int kb = k_lo + (t_begin + t) * kBlkTile;
#pragma unroll
    for (int it = 0; it < RIT; ++it) {
      const int u = tid + it * NT;
      const int j = min(kb + (u >> 3), k_hi - 1);
      const float delta = (float)(j - pos0);
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        float r = delta * p.rope_rev[(u & 7) * 8 + e];
        r -= rintf(r);
        sincos_rev(r, &rs[it][e], &rc[it][e]);
      }
    }
  };
  auto rope_tile = [&](auto SLOT) {
#pragma unroll
    for (int it = 0; it < RIT; ++it) {
      const int u = tid + it * NT;
      const int r = u >> 3, cp = u & 7;
      lds_u32x4_t* lo = reinterpret_cast<lds_u32x4_t*>(
          lds_base + SLOT * kSlotB + r * 256 + ((cp ^ (r & 15)) << 4));
      lds_u32x4_t* hi = reinterpret_cast<lds_u32x4_t*>(
          lds_base + SLOT * kSlotB + r * 256 + (((cp + 8) ^ (r & 15)) << 4));
      u32x4_t a = *lo, c = *hi;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const float x0 = bf16_lo(a[e]), x1 = bf16_hi(a[e]);
        const float y0 = bf16_lo(c[e]), y1 = bf16_hi(c[e]);
        const float c0 = rc[it][2 * e], s0 = rs[it][2 * e];
        const float c1 = rc[it][2 * e + 1], s1 = rs[it][2 * e + 1];
        a[e] = pack_bf16(x0 * c0 - y0 * s0, x1 * c1 - y1 * s1);
        c[e] = pack_bf16(y0 * c0 + x0 * s0, y1 * c1 + x1 * s1);
      }
      *lo = a;
      *hi = c;
    }
  };

  if constexpr (F8) {
    // the block's bf16 K and V rows of this KV head (rows n .. 15 repeat
    // the last), 8 KB, then the first code tiles; the block rows are
    // waited for and published before any wave dequantises
    static_for<0, 8 / WAVES>([&](auto I) {
      const int u = (I * WAVES + w) * 64 + lane;  // 16-byte chunk of the 8 KB
      const int rr = u >> 4, ch = u & 15;         // K rows 0..15, V 16..31
      const int tok = min(rr & 15, p.n - 1);
      const uint16_t* src = ((rr >> 4) ? p.v_blk : p.k_blk) +
                            ((int64_t)b * p.n + tok) * kTokenElems + g * kD +
                            ch * 8;
      dma16(src, lds_base + L8.blk + (I * WAVES + w) * 1024);
    });
    static_for<0, RING - 1>([&](auto T) {
      if (T < ntiles) issue_tile8(T, T);
    });
    {
      const int issued = min(RING - 1, ntiles);
      static_for<0, RING>([&](auto L) {
        if (issued == L) wait_vmcnt<L * LPI8>();
      });
    }
    __syncthreads();
    // tile t: codes in ring slot t % RING, bf16 in staging slot t % 2.  The
    // barrier after the dequantisation publishes the staging slot; every
    // wave has then finished the tile before (the other staging slot's
    // previous user, t - 2, was consumed before the last barrier) and the
    // code slot of t - 1, which the next tile's loads reuse.
    for (int t0 = 0; t0 < ntiles; t0 += RING) {
      static_for<0, RING>([&](auto S) {
        const int t = t0 + S;
        constexpr auto ST = std::integral_constant<int, S % 2>{};
        if (t < ntiles) {
          if constexpr (LOCAL) rope_angles8(t);
          const int later = min(RING - 2, ntiles - 1 - t);
          static_for<0, RING - 1>([&](auto L) {
            if (later == L) wait_vmcnt<L * LPI8>();
          });
          dequant8(t, S, ST);
          if constexpr (LOCAL) rope_own(ST);
          __syncthreads();
          if (t + RING - 1 < ntiles)
            issue_tile8(t + RING - 1,
                        std::integral_constant<int, (S + RING - 1) % RING>{});
          consume(t, ST);
        }
      });
    }
  } else {
  // tile t -> slot t % RING, loaded RING - 1 tiles ahead; the loop is
  // unrolled RING times so every slot offset is a constant
  static_for<0, RING - 1>([&](auto T) {
    if (T < ntiles) issue_tile(T, T);
  });
  for (int t0 = 0; t0 < ntiles; t0 += RING) {
    static_for<0, RING>([&](auto S) {
      const int t = t0 + S;
      if (t < ntiles) {
        if constexpr (ROTK) rope_angles(t);
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
        if constexpr (ROTK) {
          rope_tile(S);
          __syncthreads();
        }
        consume(t, S);
      }
    });
  }
  }  // bf16 cache

  // ---- epilogue: this lane holds row `row`, dims 32d + 8(i>>2) + 4 hi5 + i&3
  const float l_tot = xsum<32>(l_run);
  if constexpr (SPLIT) {
    const int prow = (2 * w + (row >> 4)) * kGroup + (row & 15);
    float* base = p.part +
                  ((((size_t)(b * kHkv + g) * p.qgroups + qg) * p.splits +
                    split) * ROWS + prow) * kPartRow;
    // a row with no visible key in this split (l = 0) stores zeros
    const float inv = l_tot > 0.0f ? 1.0f / l_tot : 0.0f;
    // the row's largest |o| (64 dimensions here, 64 in the lane 32 away)
    float amax = 0.0f;
#pragma unroll
    for (int d = 0; d < 4; ++d)
#pragma unroll
      for (int i = 0; i < 16; ++i) amax = fmaxf(amax, fabsf(O[d][i]));
    int e;
    (void)frexpf(xmax<32>(amax) * inv, &e);
    e = max(e, kPartExpMin);
    const float sc = inv * ldexpf(1.0f, 15 - e);
    uint32_t* ob = reinterpret_cast<uint32_t*>(base);
#pragma unroll
    for (int d = 0; d < 4; ++d)
#pragma unroll
      for (int ib = 0; ib < 4; ++ib)
        *reinterpret_cast<uint2*>(ob + (32 * d + 8 * ib + 4 * hi5) / 2) =
            make_uint2(pack_f16(O[d][4 * ib] * sc, O[d][4 * ib + 1] * sc),
                       pack_f16(O[d][4 * ib + 2] * sc,
                                O[d][4 * ib + 3] * sc));
    if (hi5 == 0)
      *reinterpret_cast<float4*>(base + kD / 2) =
          make_float4(m_run, l_tot, ldexpf(1.0f, e - 15), 0.0f);
  } else if (row_valid) {
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
  }  // work items
}

// Merge the key splits of one (sequence, token, query head), one wave,
// lane 8 sl + c: split lane sl takes splits sl, sl + 8, ... (every split's
// loads in flight at once), column c dimensions 16c .. 16c + 15.  The
// largest split maximum M is found first, so the weighted sums need no
// rescaling; with the stored o'_s = o_s / l_s (held as o'_s / r_s in fp16,
// r_s the row's inverse scale),
// o = sum 2^(m_s - M) l_s o'_s / sum 2^(m_s - M) l_s.  The maximum and the
// sums are reduced over the eight split lanes of a column (lanes c, c + 8,
// ..., c + 56) in registers, with no LDS and no barrier.
constexpr int kWaveMergeSplitsB = kBlkMaxSplits;
template <bool OUT_F32>
__global__ __launch_bounds__(64) void block_merge_kernel(
    const BlockParams p) {
  const int ROWS = p.qpw * kGroup;
  int rest = blockIdx.x;
  const int h = rest % kHq;
  rest /= kHq;
  const int qi = rest % p.n;
  const int b = rest / p.n;
  const int g = h / kGroup;
  const int qg = qi / p.qpw;
  const int prow = (qi - qg * p.qpw) * kGroup + (h % kGroup);
  const float* base =
      p.part + (((size_t)(b * kHkv + g) * p.qgroups + qg) * p.splits * ROWS +
                prow) * kPartRow;
  const size_t sstride = (size_t)ROWS * kPartRow;
  const int lane = threadIdx.x;
  const int c = lane & 7, sl = lane >> 3;
  constexpr int kPer = kWaveMergeSplitsB / 8;
  float4 st[kPer];    // m, l, inverse scale
  uint4 os[kPer][2];  // dims 16c .. 16c + 15 as scaled fp16
  const int nper = (p.splits + 7) / 8;  // batches holding a split
#pragma unroll
  for (int i = 0; i < kPer; ++i) {
    st[i] = make_float4(-INFINITY, 0.0f, 0.0f, 0.0f);
    os[i][0] = os[i][1] = make_uint4(0, 0, 0, 0);
    if (i >= nper) continue;
    const float* ps =
        base + (size_t)min(sl + 8 * i, p.splits - 1) * sstride;
    st[i] = *reinterpret_cast<const float4*>(ps + kD / 2);
    os[i][0] = *reinterpret_cast<const uint4*>(ps + 8 * c);
    os[i][1] = *reinterpret_cast<const uint4*>(ps + 8 * c + 4);
  }
  // lanes past the last split (they loaded the last split again) weigh 0;
  // masked only now, so no batch's loads wait for an earlier batch's
  float ms[kPer];
  float M = -INFINITY;
#pragma unroll
  for (int i = 0; i < kPer; ++i) {
    ms[i] = sl + 8 * i < p.splits ? st[i].x : -INFINITY;
    M = fmaxf(M, ms[i]);
  }
  M = fmaxf(M, dpp_mov<0x128>(M));  // row_ror:8, the other split lane of the row
  M = xmax<32>(xmax<16>(M));
  // splits without visible keys (m = -inf) and padding lanes weigh 0
  float L = 0.0f, O[16];
#pragma unroll
  for (int j = 0; j < 16; ++j) O[j] = 0.0f;
#pragma unroll
  for (int i = 0; i < kPer; ++i) {
    const float cw = fast_exp2(ms[i] - M) * st[i].y;
    L += cw;
    const float cwr = cw * st[i].z;
    const uint32_t* wv = reinterpret_cast<const uint32_t*>(&os[i][0]);
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      O[2 * j] += f16_lo(wv[j]) * cwr;
      O[2 * j + 1] += f16_hi(wv[j]) * cwr;
    }
  }
  L = stride8_sum(L);
#pragma unroll
  for (int j = 0; j < 16; ++j) O[j] = stride8_sum(O[j]);
  if (sl != 0) return;
  const float inv = 1.0f / L;
  const size_t o = (((size_t)b * p.n + qi) * kHq + h) * kD + 16 * c;
  if constexpr (OUT_F32) {
    float4* dst = reinterpret_cast<float4*>(static_cast<float*>(p.out) + o);
#pragma unroll
    for (int j = 0; j < 4; ++j)
      dst[j] = make_float4(O[4 * j] * inv, O[4 * j + 1] * inv,
                           O[4 * j + 2] * inv, O[4 * j + 3] * inv);
  } else {
    uint4* dst = reinterpret_cast<uint4*>(static_cast<uint16_t*>(p.out) + o);
#pragma unroll
    for (int j = 0; j < 2; ++j)
      dst[j] = make_uint4(pack_bf16(O[8 * j] * inv, O[8 * j + 1] * inv),
                          pack_bf16(O[8 * j + 2] * inv, O[8 * j + 3] * inv),
                          pack_bf16(O[8 * j + 4] * inv, O[8 * j + 5] * inv),
                          pack_bf16(O[8 * j + 6] * inv, O[8 * j + 7] * inv));
  }
}

template <bool LOCAL, bool OUT_F32>
hipError_t launch_main(const BlockParams& p, const BlockPlan& plan, int B,
                       hipStream_t s) {
  // without key splits: at most one workgroup per CU, each walking its
  // items (the kernel derives the walk from the grid)
  const dim3 grid(plan.grid);
  if (p.splits > 1) {
    bool small = false;
    if constexpr (LOCAL) small = plan.qpw == kBlkQpwSmall;
    if constexpr (LOCAL) {
      if (small)
        hipLaunchKernelGGL(
            (block_attn_kernel<kBlkQpwSmall, true, true, OUT_F32>), grid,
            dim3(kBlkQpwSmall * 32), 0, s, p);
    }
    if (!small)
      hipLaunchKernelGGL((block_attn_kernel<kBlkQpw, LOCAL, true, OUT_F32>),
                         grid, dim3(kBlkQpw * 32), 0, s, p);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL((block_merge_kernel<OUT_F32>), dim3(B * p.n * kHq),
                       dim3(64), 0, s, p);
  } else {
    hipLaunchKernelGGL((block_attn_kernel<kBlkQpw, LOCAL, false, OUT_F32>),
                       grid, dim3(kBlkQpw * 32), 0, s, p);
  }
  return hipGetLastError();
}

}  // namespace

// fp8 caches (verification and drafted blocks): the key-split kernels for
// any split count, then the merge.  Local layers take 8-token workgroups,
// global layers 16.
static hipError_t launch_block_fp8(const BlockParams& p, const BlockPlan& plan,
                                   bool local, int B, hipStream_t s) {
  if (plan.walks != 1 || plan.klin_bytes != 0 || p.part == nullptr ||
      p.n > kF8BlkRows || p.splits > kBlkMaxSplits ||
      plan.grid != p.splits * p.qgroups * kHkv * B || p.qpw != plan.qpw ||
      plan.qpw != (local ? kBlkQpwSmall : kBlkQpw))
    return hipErrorInvalidValue;
  const dim3 grid(plan.grid);
  if (local)
    hipLaunchKernelGGL(
        (block_attn_kernel<kBlkQpwSmall, true, true, true, true>), grid,
        dim3(kBlkQpwSmall * 32), 0, s, p);
  else
    hipLaunchKernelGGL((block_attn_kernel<kBlkQpw, false, true, true, true>),
                       grid, dim3(kBlkQpw * 32), 0, s, p);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL((block_merge_kernel<true>), dim3(B * p.n * kHq), dim3(64),
                     0, s, p);
  return hipGetLastError();
}

hipError_t launch_block(const BlockParams& p, const BlockPlan& plan,
                        bool local, bool out_f32, int B, hipStream_t s,
                        bool fp8) {
  if (fp8) {
    if (!out_f32) return hipErrorInvalidValue;
    return launch_block_fp8(p, plan, local, B, s);
  }
  // 8-token workgroups only for local layers with key splits
  const bool small = local && p.splits > 1 && plan.qpw == kBlkQpwSmall;
  if ((plan.qpw != kBlkQpw && !small) || p.qpw != plan.qpw ||
      p.splits > kBlkMaxSplits || plan.grid < 1 ||
      (p.splits > 1 && plan.grid != p.splits * p.qgroups * kHkv * B))
    return hipErrorInvalidValue;
  if (local) {
    if (p.splits == 1) {  // keys rotated once into the workspace
      hipLaunchKernelGGL(rope_keys_kernel,
                         dim3((unsigned)((p.klin_rows + kRopeRowsPerWG - 1) /
                                         kRopeRowsPerWG),
                              B),
                         dim3(256), 0, s, p);
      hipError_t e = hipGetLastError();
      if (e != hipSuccess) return e;
    }
    return out_f32 ? launch_main<true, true>(p, plan, B, s)
                   : launch_main<true, false>(p, plan, B, s);
  }
  return out_f32 ? launch_main<false, true>(p, plan, B, s)
                 : launch_main<false, false>(p, plan, B, s);
}

}  // namespace gqa
