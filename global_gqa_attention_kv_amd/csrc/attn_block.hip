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
//    CU.
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
//    bf16, plus the maximum and the denominator in fp32.
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
constexpr int kWaves = kBlkQpw / 2;         // 8 waves of 32 rows
// Partial row of a key split, in 4-byte words: words 0..63 the row's output
// over the split normalised by its own denominator (o / l) as 128 bf16,
// word 64 the maximum m, word 65 the denominator l (fp32), 2 words padding.
constexpr int kPartRow = 68;

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

// Tile t goes to ring slot t % 4, loaded three tiles ahead (direct-to-LDS,
// so tile t + 3 is in flight while tile t is consumed).  K chunk c of row r
// sits at chunk
// slot c ^ (r & 15), so the 32 lanes reading one chunk of 32 consecutive
// keys hit distinct banks; V chunk c at slot c ^ X(r & 3), X = {0, 4, 10,
// 14}: the four keys of a 16-lane group of ds_read_b64_tr_b16, and the 64
// bytes of each key read by a 32-lane half, land on distinct banks.
template <bool LOCAL, bool SPLIT, bool OUT_F32>
__global__ __launch_bounds__(kWaves * 64, 1) void block_attn_kernel(
    const BlockParams p) {
  constexpr int QPW = kBlkQpw;
  constexpr int WAVES = kWaves;
  constexpr int RING = kRing;
  constexpr int ROWS = QPW * kGroup;
  constexpr int RPW = kBlkTile / WAVES;   // tile rows each wave loads
  constexpr int LPT = RPW / 4;            // 1-KB loads per K or V tile per wave
  __shared__ __attribute__((aligned(16))) uint8_t smem[RING * kSlotB];
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
  float4* const rtab = reinterpret_cast<float4*>(smem + (RING - 1) * kSlotB);
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
    f32x16_t S[2];
    bf16x8_t ka[2][8];
#pragma unroll
    for (int k = 0; k < 8; ++k)
      ka[0][k] = *reinterpret_cast<const lds_bf16x8_t*>(krd[k] + so);
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      S[0] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
          ka[0][k], qreg[k], k == 0 ? negmb : S[0], 0, 0, 0);
      ka[1][k] = *reinterpret_cast<const lds_bf16x8_t*>(krd[k] + so + 8192);
    }
#pragma unroll
    for (int k = 0; k < 8; ++k)
      S[1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
          ka[1][k], qreg[k], k == 0 ? negmb : S[1], 0, 0, 0);
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
    float mt = -INFINITY;
#pragma unroll
    for (int be = 0; be < 2; ++be)
#pragma unroll
      for (int i = 0; i < 16; ++i) mt = fmaxf(mt, S[be][i]);
    mt = fmaxf(mt, __shfl_xor(mt, 32, 64)) + mb;  // tile max, log2 units
    if (__any(mt > m_run + kTauB)) {
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
#pragma unroll
    for (int be = 0; be < 2; ++be)
#pragma unroll
      for (int tt = 0; tt < 2; ++tt) {
        uint32_t w4[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const float p0 = fast_exp2(S[be][8 * tt + 2 * j]);
          const float p1 = fast_exp2(S[be][8 * tt + 2 * j + 1]);
          w4[j] = pack_bf16(p0, p1);
          // the denominator sums exactly the bf16 weights P.V uses
          l_run = dot2_bf16(w4[j], 0x3F803F80u, l_run);
        }
        P[2 * be + tt] = __builtin_bit_cast(
            bf16x8_t, make_uint4(w4[0], w4[1], w4[2], w4[3]));
      }

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

  // ROTK: thread i rotates item i of a landed K tile, item u = (key row
  // u / 8, dims 8 (u % 8) .. + 7 against dims 64 + 8 (u % 8) ..), by the
  // key's offset from p0 (the queries carry theirs); the sines and cosines
  // are taken before the tile is waited for, so they overlap its load.
  static_assert(!ROTK || WAVES * 64 == kBlkTile * 8, "one item per thread");
  float rc[8], rs[8];
  auto rope_angles = [&](int t) {
    const int kb = k_lo + (t_begin + t) * kBlkTile;
    const int j = min(kb + (tid >> 3), k_hi - 1);
    const float delta = (float)(j - pos0);
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      float r = delta * p.rope_rev[(tid & 7) * 8 + e];
      r -= rintf(r);
      sincos_rev(r, &rs[e], &rc[e]);
    }
  };
  auto rope_tile = [&](auto SLOT) {
    const int r = tid >> 3, cp = tid & 7;
    lds_u32x4_t* lo = reinterpret_cast<lds_u32x4_t*>(
        lds_base + SLOT * kSlotB + r * 256 + ((cp ^ (r & 15)) << 4));
    lds_u32x4_t* hi = reinterpret_cast<lds_u32x4_t*>(
        lds_base + SLOT * kSlotB + r * 256 + (((cp + 8) ^ (r & 15)) << 4));
    u32x4_t a = *lo, c = *hi;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const float x0 = bf16_lo(a[e]), x1 = bf16_hi(a[e]);
      const float y0 = bf16_lo(c[e]), y1 = bf16_hi(c[e]);
      const float c0 = rc[2 * e], s0 = rs[2 * e];
      const float c1 = rc[2 * e + 1], s1 = rs[2 * e + 1];
      a[e] = pack_bf16(x0 * c0 - y0 * s0, x1 * c1 - y1 * s1);
      c[e] = pack_bf16(y0 * c0 + x0 * s0, y1 * c1 + x1 * s1);
    }
    *lo = a;
    *hi = c;
  };

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

  // ---- epilogue: this lane holds row `row`, dims 32d + 8(i>>2) + 4 hi5 + i&3
  const float l_tot = l_run + __shfl_xor(l_run, 32, 64);
  if constexpr (SPLIT) {
    const int prow = (2 * w + (row >> 4)) * kGroup + (row & 15);
    float* base = p.part +
                  ((((size_t)(b * kHkv + g) * p.qgroups + qg) * p.splits +
                    split) * ROWS + prow) * kPartRow;
    // a row with no visible key in this split (l = 0) stores zeros
    const float inv = l_tot > 0.0f ? 1.0f / l_tot : 0.0f;
    uint32_t* ob = reinterpret_cast<uint32_t*>(base);
#pragma unroll
    for (int d = 0; d < 4; ++d)
#pragma unroll
      for (int ib = 0; ib < 4; ++ib)
        *reinterpret_cast<uint2*>(ob + (32 * d + 8 * ib + 4 * hi5) / 2) =
            make_uint2(pack_bf16(O[d][4 * ib] * inv, O[d][4 * ib + 1] * inv),
                       pack_bf16(O[d][4 * ib + 2] * inv,
                                 O[d][4 * ib + 3] * inv));
    if (hi5 == 0) {
      base[kD / 2] = m_run;
      base[kD / 2 + 1] = l_tot;
    }
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

// Merge the key splits of one (sequence, token, query head): 32 split lanes
// x 8 columns of 16 dimensions per workgroup (thread = 8 lane + column), so
// the split rows are read whole, every split's loads in flight at once.  The
// largest split maximum M is found first, so the weighted sums need no
// rescaling and the split lanes combine by plain addition; with the stored
// o'_s = o_s / l_s, o = sum 2^(m_s - M) l_s o'_s / sum 2^(m_s - M) l_s.
template <bool OUT_F32>
__global__ __launch_bounds__(256) void block_merge_kernel(const BlockParams p) {
  constexpr int ROWS = kBlkQpw * kGroup;
  int rest = blockIdx.x;
  const int h = rest % kHq;
  rest /= kHq;
  const int qi = rest % p.n;
  const int b = rest / p.n;
  const int g = h / kGroup;
  const int qg = qi / kBlkQpw;
  const int prow = (qi - qg * kBlkQpw) * kGroup + (h % kGroup);
  const float* base =
      p.part + (((size_t)(b * kHkv + g) * p.qgroups + qg) * p.splits * ROWS +
                prow) * kPartRow;
  constexpr size_t sstride = (size_t)ROWS * kPartRow;
  const int tid = threadIdx.x;
  const int c = tid & 7, sl = tid >> 3, w = tid >> 6;
  __shared__ float wmax[4];
  __shared__ float wsum[4][8][17];
  constexpr int kPer = kMaxSplits / 32;  // the planner keeps splits <= 256
  float ms[kPer], ls[kPer];
  uint4 os[kPer][2];  // dims 16c .. 16c + 15 as bf16
  const int nper = (p.splits + 31) / 32;  // batches holding a split
#pragma unroll
  for (int i = 0; i < kPer; ++i) {
    ms[i] = -INFINITY;
    ls[i] = 0.0f;
    os[i][0] = os[i][1] = make_uint4(0, 0, 0, 0);
    if (i >= nper) continue;
    const int s = sl + 32 * i;
    const float* ps = base + (size_t)min(s, p.splits - 1) * sstride;
    ms[i] = s < p.splits ? ps[kD / 2] : -INFINITY;
    ls[i] = ps[kD / 2 + 1];
    os[i][0] = *reinterpret_cast<const uint4*>(ps + 8 * c);
    os[i][1] = *reinterpret_cast<const uint4*>(ps + 8 * c + 4);
  }
  float mx = -INFINITY;
#pragma unroll
  for (int i = 0; i < kPer; ++i) mx = fmaxf(mx, ms[i]);
  mx = wave_max(mx);
  if ((tid & 63) == 0) wmax[w] = mx;
  __syncthreads();
  const float M = fmaxf(fmaxf(wmax[0], wmax[1]), fmaxf(wmax[2], wmax[3]));
  // splits without visible keys (m = -inf) and padding lanes weigh 0
  float L = 0.0f, O[16];
#pragma unroll
  for (int j = 0; j < 16; ++j) O[j] = 0.0f;
#pragma unroll
  for (int i = 0; i < kPer; ++i) {
    const float cw = fast_exp2(ms[i] - M) * ls[i];
    L += cw;
    const uint32_t* wv = reinterpret_cast<const uint32_t*>(&os[i][0]);
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      O[2 * j] += bf16_lo(wv[j]) * cw;
      O[2 * j + 1] += bf16_hi(wv[j]) * cw;
    }
  }
  // the 8 split lanes of a wave that share a column are 8 apart
#pragma unroll
  for (int o = 8; o <= 32; o <<= 1) {
    L += __shfl_xor(L, o, 64);
#pragma unroll
    for (int j = 0; j < 16; ++j) O[j] += __shfl_xor(O[j], o, 64);
  }
  if ((tid & 63) < 8) {
#pragma unroll
    for (int j = 0; j < 16; ++j) wsum[w][c][j] = O[j];
    wsum[w][c][16] = L;
  }
  __syncthreads();
  if (tid >= 8) return;
  float r[17];
#pragma unroll
  for (int j = 0; j < 17; ++j)
    r[j] = wsum[0][c][j] + wsum[1][c][j] + wsum[2][c][j] + wsum[3][c][j];
  const float inv = 1.0f / r[16];
  const size_t o = (((size_t)b * p.n + qi) * kHq + h) * kD + 16 * c;
  if constexpr (OUT_F32) {
    float4* dst = reinterpret_cast<float4*>(static_cast<float*>(p.out) + o);
#pragma unroll
    for (int j = 0; j < 4; ++j)
      dst[j] = make_float4(r[4 * j] * inv, r[4 * j + 1] * inv,
                           r[4 * j + 2] * inv, r[4 * j + 3] * inv);
  } else {
    uint4* dst = reinterpret_cast<uint4*>(static_cast<uint16_t*>(p.out) + o);
#pragma unroll
    for (int j = 0; j < 2; ++j)
      dst[j] = make_uint4(pack_bf16(r[8 * j] * inv, r[8 * j + 1] * inv),
                          pack_bf16(r[8 * j + 2] * inv, r[8 * j + 3] * inv),
                          pack_bf16(r[8 * j + 4] * inv, r[8 * j + 5] * inv),
                          pack_bf16(r[8 * j + 6] * inv, r[8 * j + 7] * inv));
  }
}

template <bool LOCAL, bool OUT_F32>
hipError_t launch_main(const BlockParams& p, int B, hipStream_t s) {
  const int items = p.splits * p.qgroups * kHkv * B;
  // without key splits: at most one workgroup per CU, each walking its items
  const int walks = p.splits > 1 ? 1 : (items + kCUs - 1) / kCUs;
  const dim3 grid((items + walks - 1) / walks);
  const dim3 block(kWaves * 64);
  if (p.splits > 1) {
    hipLaunchKernelGGL((block_attn_kernel<LOCAL, true, OUT_F32>), grid, block,
                       0, s, p);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL((block_merge_kernel<OUT_F32>),
                       dim3(B * p.n * kHq), dim3(256), 0, s, p);
  } else {
    hipLaunchKernelGGL((block_attn_kernel<LOCAL, false, OUT_F32>), grid, block,
                       0, s, p);
  }
  return hipGetLastError();
}

}  // namespace

hipError_t launch_block(const BlockParams& p, const BlockPlan& plan,
                        bool local, bool out_f32, int B, hipStream_t s) {
  if (plan.qpw != kBlkQpw || p.splits > kMaxSplits) return hipErrorInvalidValue;
  if (local) {
    if (p.splits == 1) {  // keys rotated once into the workspace
      hipLaunchKernelGGL(rope_keys_kernel, dim3((unsigned)p.klin_rows, B),
                         dim3(64), 0, s, p);
      hipError_t e = hipGetLastError();
      if (e != hipSuccess) return e;
    }
    return out_f32 ? launch_main<true, true>(p, B, s)
                   : launch_main<true, false>(p, B, s);
  }
  return out_f32 ? launch_main<false, true>(p, B, s)
                 : launch_main<false, false>(p, B, s);
}

}  // namespace gqa
