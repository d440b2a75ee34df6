/*
 * gqa_attn.h -- C ABI of libgqa_attn.so: grouped-query attention with a
 * hybrid local / global KV cache on AMD MI355X (gfx950).
 *
 * The model shape is compiled in: 32 query heads share 2 KV heads of
 * dimension 128; query head h reads KV head h / 16.  Layers repeat three
 * local layers and one global layer.
 *   - Local layer: RoPE (base rope_theta) on queries and keys; each query at
 *     position i attends to positions max(0, i-2047) .. i.  Its cache is a
 *     ring of 2048 slots, slot = position mod 2048.
 *   - Global layer: no RoPE; each query at position i attends to positions
 *     0 .. i.  Its cache is linear, slot = position, up to 131072 slots.
 * Sources: "Deep dive into Muse Glimmer" (shishifenxi.com) section 01 (52
 * layers, 32 query / 2 KV heads, dim 128, 3 local then 1 global, nearby 2048
 * tokens, about 1024 B of KV per token per layer); "Tomas Koutsky explains
 * how Meta fits Muse Glimmer into 24 GB" (runtimewire.com), "Narrow cache"
 * (131,072-token context, sliding-window entries reused cyclically) and "Long
 * context still costs compute" (global layers omit RoPE).
 *
 * Conventions for every entry point
 *   - All tensors are device pointers, bf16 unless stated, dense row-major,
 *     16-byte aligned.  Positions are HOST arrays of int64, one per sequence.
 *   - Every call is asynchronous on `stream` (a hipStream_t; NULL = the null
 *     stream).  The library never allocates, frees or synchronises.  Its only
 *     global state is a per-device record of the device's compute-unit and
 *     XCD counts (read once, used to size launches) and the device-resident
 *     scratch of gqa_attn_decode_noalloc; every other entry point is safe to
 *     call from several threads on different streams.
 *   - Arguments are validated on the host before anything is launched; a
 *     non-zero return means nothing was enqueued (except GQA_ERR_HIP, which
 *     reports a failed launch).  Faults inside a kernel surface at the
 *     caller's next synchronisation.  No C++ exception crosses the ABI.
 *   - Batch size B is 1 .. GQA_MAX_BATCH.
 *   - Workspaces: every attention call takes a caller-owned scratch buffer
 *     `ws` (256-byte aligned) of at least gqa_workspace_bytes(op, ...) bytes
 *     for its partial results.  It needs no initialisation and carries
 *     nothing from one call to the next, so one workspace, sized for the
 *     largest request, serves every operation and layer kind issued in order
 *     on one stream.  Calls that may overlap in time need separate
 *     workspaces.
 */
#ifndef GQA_ATTN_H
#define GQA_ATTN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define GQA_ABI_VERSION 1

#define GQA_NUM_Q_HEADS 32
#define GQA_NUM_KV_HEADS 2
#define GQA_HEAD_DIM 128
#define GQA_WINDOW 2048
#define GQA_MAX_CONTEXT 131072
#define GQA_MAX_BATCH 64
#define GQA_MAX_VERIFY 16
#define GQA_NUM_LAYERS 52
/* Largest position any token may have (local layers; global layers are
 * bounded by their capacity): 2^31 - 4097, so the kernels' 32-bit key-range
 * arithmetic never wraps. */
#define GQA_MAX_POSITION 2147479551
/* Device-resident scratch of gqa_attn_decode_noalloc, per GPU (8 MiB). */
#define GQA_NOALLOC_SCRATCH_BYTES 8388608

/* Layer kinds. */
#define GQA_LOCAL 0
#define GQA_GLOBAL 1

/* Operations, for gqa_workspace_bytes. */
#define GQA_OP_DECODE 0
#define GQA_OP_VERIFY 1
#define GQA_OP_PREFILL 2
#define GQA_OP_DRAFT 3
#define GQA_OP_PREFILL_FP8 4  /* gqa_attn_prefill_fp8 */

/* Status codes. */
#define GQA_OK 0
#define GQA_ERR_INVALID_ARG (-1)  /* null pointer, B or n out of range      */
#define GQA_ERR_POS_RANGE (-2)    /* position < 0, past a global cache, or
                                     above GQA_MAX_POSITION                 */
#define GQA_ERR_MISALIGNED (-3)   /* a pointer or stride not 16-B aligned    */
#define GQA_ERR_WS_TOO_SMALL (-4) /* workspace smaller than required        */
#define GQA_ERR_UNSUPPORTED (-5)  /* layer descriptor outside compiled shape */
#define GQA_ERR_HIP (-6)          /* a kernel launch failed                  */

/* One attention layer's cache, owned by the caller.
 *   kind       GQA_LOCAL or GQA_GLOBAL
 *   window     GQA_WINDOW for local layers, 0 for global layers
 *   capacity   slots per sequence: GQA_WINDOW (local) or 1..GQA_MAX_CONTEXT
 *              (global)
 *   rope_theta RoPE base for local layers (> 0), 0 for global layers
 *   k, v       device bf16 caches [B][capacity][2][128]; sequence b starts at
 *              element b * seq_stride
 *   seq_stride elements between sequences, >= capacity * 256, multiple of 8 */
typedef struct gqa_layer {
  int32_t kind;
  int32_t window;
  int64_t capacity;
  double rope_theta;
  void* k;
  void* v;
  int64_t seq_stride;
} gqa_layer;

/* Kind of layer `layer` (0-based) of the 52-layer stack: GQA_GLOBAL when
 * layer % 4 == 3, GQA_LOCAL otherwise -- three local layers, then one
 * global layer, 13 times (39 local + 13 global).  Returns
 * GQA_ERR_INVALID_ARG for an index outside 0 .. GQA_NUM_LAYERS-1.  The
 * caller describes layer l's cache with this kind (local: window
 * GQA_WINDOW, capacity GQA_WINDOW, RoPE; global: window 0, linear cache,
 * no RoPE).
 * Pages: shishifenxi.com section 01 (52 layers, a repeating cycle of three
 * sliding-window layers followed by one full-attention layer);
 * runtimewire.com "Narrow cache" (every fourth layer is global: 39
 * sliding-window layers and 13 full layers). */
int gqa_layer_kind(int layer);

/* Append n tokens per sequence to a layer's cache (bit-exact copy).
 * k_new, v_new: [B][n][2][128] bf16; token t of sequence b has position
 * pos0[b] + t.  Global layers write slot = position (pos0[b] + n must not
 * exceed capacity).  Local layers write slot = position mod 2048 and, when
 * n > 2048, only the last 2048 tokens (the earlier ones would be overwritten
 * anyway), so no two writes of one call collide.  n >= 1.
 * Pages: runtimewire.com "Narrow cache" (cyclic reuse of sliding-window
 * entries; about 1024 B per token per layer, shishifenxi.com section 01). */
int gqa_kv_append(const gqa_layer* layer, const void* k_new, const void* v_new,
                  const int64_t* pos0, int B, int n, void* stream);

/* One decode step: one query token per sequence at position pos[b], whose
 * own K/V is already in the cache.  q: [B][32][128] bf16; out: [B][32][128]
 * fp32.  Global layers attend to positions 0..pos[b] (pos[b] < capacity);
 * local layers to max(0, pos[b]-2047)..pos[b] through the ring, with RoPE.
 * Scale 1/sqrt(128).  The key range is split across workgroups (split-K)
 * whose partial softmax sums are merged on the device.
 * Workspace: gqa_workspace_bytes(GQA_OP_DECODE, kind, B, 1, max pos + 1)
 * bytes (see the workspace rules above).
 * Pages: shishifenxi.com section 01 (each new token reads the cached keys
 * and values); runtimewire.com "Narrow cache" and "Long context still costs
 * compute". */
int gqa_attn_decode(const gqa_layer* layer, const void* q, const int64_t* pos,
                    int B, float* out, void* ws, size_t ws_bytes,
                    void* stream);

/* gqa_kv_append(layer, k_new, v_new, pos, B, 1) followed by
 * gqa_attn_decode(layer, q, pos, ...), in one launch: the new token's K/V
 * (k_new, v_new: [B][1][2][128] bf16) is stored to its slot and used as the
 * last key of the attention.  Same workspace rules as gqa_attn_decode. */
int gqa_attn_decode_append(const gqa_layer* layer, const void* q,
                           const void* k_new, const void* v_new,
                           const int64_t* pos, int B, float* out, void* ws,
                           size_t ws_bytes, void* stream);

/* Decode with DEVICE-resident positions, for a step captured once in a HIP
 * graph and replayed while the sequences advance (the caller updates
 * pos_dev between replays, e.g. with an add kernel inside the graph).
 * pos_dev: device int64 [B], read by the kernels when they run; max_pos:
 * a host bound on every pos_dev[b], validated like a position (global:
 * max_pos < capacity) -- it plans the key splits and sizes the workspace
 * (gqa_workspace_bytes(GQA_OP_DECODE, kind, B, 1, max_pos + 1)).  k_new,
 * v_new: both null (attend only, as gqa_attn_decode) or both given (append
 * and attend, as gqa_attn_decode_append).  A device position outside
 * [0, max_pos] is not attended: that sequence's output rows are NaN and
 * nothing of it is appended.  Other arguments, layouts and the workspace
 * rules as gqa_attn_decode.  Pages: shishifenxi.com section 01 (each new
 * token reads the cached keys and values); runtimewire.com "Narrow cache"
 * (a serving engine reuses one cache layout across steps). */
int gqa_attn_decode_dev(const gqa_layer* layer, const void* q,
                        const void* k_new, const void* v_new,
                        const int64_t* pos_dev, int64_t max_pos, int B,
                        float* out, void* ws, size_t ws_bytes, void* stream);

/* gqa_attn_decode / gqa_attn_decode_append without a workspace, for callers
 * that cannot allocate device memory: code under HIP graph capture, tight
 * serving loops, harnesses that forbid allocation.  k_new, v_new: both null
 * (attend only, as gqa_attn_decode) or both given (append the token, then
 * attend, as gqa_attn_decode_append); other arguments and layouts as
 * gqa_attn_decode, same kernels and results.  The split partials go to a
 * device-resident scratch array of GQA_NOALLOC_SCRATCH_BYTES that the
 * library holds on each GPU it runs on until the process ends; the call
 * allocates nothing.  A call whose partials need more returns
 * GQA_ERR_WS_TOO_SMALL (on a 256-CU MI355X none does: every batch size and
 * context needs at most 4.3 MB).  Every call on one GPU shares that GPU's
 * scratch: calls that may overlap in time on one GPU (different streams,
 * threads) race; calls issued in order on one stream do not.  The first call
 * on each device looks up the scratch's address (no allocation); make that
 * first call outside a graph capture.  GQA_ERR_HIP: the lookup failed. */
int gqa_attn_decode_noalloc(const gqa_layer* layer, const void* q,
                            const void* k_new, const void* v_new,
                            const int64_t* pos, int B, float* out,
                            void* stream);

/* Speculative verification of a drafted block of n (1..GQA_MAX_VERIFY)
 * tokens per sequence at positions pos0[b] .. pos0[b]+n-1, in one pass.
 * q: [B][n][32][128] bf16; k_blk, v_blk: [B][n][2][128] bf16, the block's
 * own K/V, NOT yet in the cache (the cache holds every position < pos0[b]);
 * out: [B][n][32][128] fp32.  Token r attends to the cached positions before
 * pos0[b] in its range (global: all of them; local: those >= pos0[b]+r-2047,
 * through the ring, with RoPE) and to block tokens 0..r (causal inside the
 * block).  The call does not touch the cache: append the accepted prefix
 * afterwards with gqa_kv_append, so rejected drafts never overwrite ring
 * entries that are still inside the window.  Global layers need
 * pos0[b] + n <= capacity.  ws must hold
 * gqa_workspace_bytes(GQA_OP_VERIFY, kind, B, n, max pos0 + n) bytes.
 * Pages: shishifenxi.com section 04 (a block of 16 drafted tokens verified
 * by the main model at once); kongchang.com "Meta open-sources the 30B Muse
 * Glimmer", "Trick 3: D-Flash" (parallel verification under the causal
 * mask). */
int gqa_attn_verify(const gqa_layer* layer, const void* q, const void* k_blk,
                    const void* v_blk, const int64_t* pos0, int B, int n,
                    float* out, void* ws, size_t ws_bytes, void* stream);

/* Attention of a drafted block whose n (1..GQA_MAX_VERIFY) tokens at
 * positions pos0[b] .. pos0[b]+n-1 are predicted together, as in one step of
 * a block-diffusion drafter: every token of the block attends to the cached
 * positions 0 .. pos0[b]-1 and to ALL n block tokens (no causal order inside
 * the block).  Global layers only (GQA_GLOBAL: no RoPE, no window); a local
 * layer returns GQA_ERR_UNSUPPORTED.  Arguments, layouts (q [B][n][32][128]
 * bf16, k_blk / v_blk [B][n][2][128] bf16 not in the cache, out
 * [B][n][32][128] fp32), ownership and errors as gqa_attn_verify; ws must
 * hold gqa_workspace_bytes(GQA_OP_DRAFT, GQA_GLOBAL, B, n, max pos0 + n)
 * bytes.  The cache is not touched.
 * Pages: shishifenxi.com section 04 (the drafter predicts a 16-token block
 * in parallel by block diffusion instead of token by token, and the target's
 * hidden features from five of its layers enter every drafter layer's keys
 * and values -- here: the cached context). */
int gqa_attn_draft_block(const gqa_layer* layer, const void* q,
                         const void* k_blk, const void* v_blk,
                         const int64_t* pos0, int B, int n, float* out,
                         void* ws, size_t ws_bytes, void* stream);

/* Chunked prefill: n (1..GQA_MAX_CONTEXT) prompt tokens per sequence at
 * positions pos0[b] .. pos0[b]+n-1.  Same visibility rules and arguments as
 * gqa_attn_verify (the chunk's K/V are passed in and not appended; the
 * cache holds the positions before pos0[b]), but out is bf16 [B][n][32][128],
 * rounded to nearest even from fp32.  ws must hold
 * gqa_workspace_bytes(GQA_OP_PREFILL, kind, B, n, max pos0 + n) bytes.
 * Append the chunk with gqa_kv_append afterwards.
 * Pages: runtimewire.com "Long context still costs compute" (global layers
 * run full attention during prompt processing with memory-efficient kernels
 * that never store the attention matrix; the cost stays quadratic). */
int gqa_attn_prefill(const gqa_layer* layer, const void* q,
                     const void* k_chunk, const void* v_chunk,
                     const int64_t* pos0, int B, int n, void* out, void* ws,
                     size_t ws_bytes, void* stream);

/* ---------------------------------------------------------- fp8 caches
 * A layer's cache may instead hold 8-bit codes: OCP FP8 E4M3 (sign, 4-bit
 * exponent with bias 7, 3-bit mantissa, largest finite value 448) plus one
 * fp32 scale per (token, KV head), separately for K and for V -- 528 bytes
 * per token per layer instead of 1024.  A head's 128 values x are stored as
 * s = amax / 448 (amax: their largest magnitude) and
 * code = round-to-nearest-even(clamp(x / s, -448, 448)), both divisions
 * rounded to nearest in fp32; amax = 0 stores s = 0 and zero codes.
 * Attention reads the values code * s.
 * Pages: runtimewire.com "Narrow cache" (cache quantisation is among the
 * factors that change how much memory the cache really takes; the pages
 * give no format -- this one is the library's reading).
 *
 * One attention layer's fp8 cache, owned by the caller.
 *   kind, window, capacity, rope_theta  as in gqa_layer
 *   k, v          device uint8 codes [B][capacity][2][128]; sequence b starts
 *                 at byte b * seq_stride
 *   k_scale, v_scale  device fp32 scales [B][2][capacity]; sequence b starts
 *                 at element b * scale_stride, KV head g at + g * capacity
 *   seq_stride    bytes between sequences, >= capacity * 256, multiple of 16
 *   scale_stride  floats between sequences, >= 2 * capacity
 * All four buffers 16-byte aligned. */
typedef struct gqa_layer_fp8 {
  int32_t kind;
  int32_t window;
  int64_t capacity;
  double rope_theta;
  void* k;
  void* v;
  float* k_scale;
  float* v_scale;
  int64_t seq_stride;
  int64_t scale_stride;
} gqa_layer_fp8;

/* gqa_kv_append for an fp8 cache: quantises n new bf16 tokens per sequence
 * (k_new, v_new: [B][n][2][128] bf16) as above and writes their codes and
 * scales to the slots gqa_kv_append would use (global: position; local:
 * position mod 2048, only the last 2048 tokens of a block).  Bit-exact:
 * the codes and scales are fully determined by the bf16 inputs.  Errors as
 * gqa_kv_append. */
int gqa_kv_append_fp8(const gqa_layer_fp8* layer, const void* k_new,
                      const void* v_new, const int64_t* pos0, int B, int n,
                      void* stream);

/* gqa_attn_decode over an fp8 cache: one query token per sequence at
 * pos[b] (its own K/V already appended), attending to the dequantised keys
 * and values (global: positions 0..pos[b]; local: pos[b]-2047..pos[b]
 * through the ring, with RoPE).  q [B][32][128] bf16, out [B][32][128]
 * fp32; workspace and errors as gqa_attn_decode
 * (gqa_workspace_bytes(GQA_OP_DECODE, kind, B, 1, max pos + 1)). */
int gqa_attn_decode_fp8(const gqa_layer_fp8* layer, const void* q,
                        const int64_t* pos, int B, float* out, void* ws,
                        size_t ws_bytes, void* stream);

/* gqa_attn_verify over an fp8 cache: n (1..GQA_MAX_VERIFY) drafted tokens
 * per sequence at positions pos0[b] .. pos0[b]+n-1, causal inside the
 * block, attending to the cached tokens as their dequantised values
 * (code * scale) and to the block's own tokens at their bf16 values (k_blk,
 * v_blk [B][n][2][128] bf16: not in the cache yet, so not quantised; append
 * the accepted ones with gqa_kv_append_fp8 afterwards).  q [B][n][32][128]
 * bf16, out [B][n][32][128] fp32; workspace
 * gqa_workspace_bytes(GQA_OP_VERIFY, kind, B, n, max pos0 + n) (one verify
 * workspace serves both cache formats); errors as gqa_attn_verify.
 * Pages: shishifenxi.com "Deep dive into Muse Glimmer" section 04 (the main
 * model checks a drafted block in one pass) and runtimewire.com "Narrow
 * cache" (cache quantisation). */
int gqa_attn_verify_fp8(const gqa_layer_fp8* layer, const void* q,
                        const void* k_blk, const void* v_blk,
                        const int64_t* pos0, int B, int n, float* out,
                        void* ws, size_t ws_bytes, void* stream);

/* gqa_attn_draft_block over an fp8 cache (global layers): every query of
 * the block sees the dequantised cache before the block and the whole
 * block at its bf16 values.  Arguments, workspace
 * (gqa_workspace_bytes(GQA_OP_DRAFT, ...)) and errors as
 * gqa_attn_draft_block. */
int gqa_attn_draft_block_fp8(const gqa_layer_fp8* layer, const void* q,
                             const void* k_blk, const void* v_blk,
                             const int64_t* pos0, int B, int n, float* out,
                             void* ws, size_t ws_bytes, void* stream);

/* gqa_attn_prefill over an fp8 cache: a chunk of n (1..GQA_MAX_CONTEXT)
 * prompt tokens per sequence at pos0[b] .. pos0[b]+n-1, attending causally
 * (local layers: banded over 2048 positions, with RoPE) to the cached
 * tokens as their dequantised values and to the chunk's own tokens at their
 * bf16 values (k_chunk, v_chunk [B][n][2][128] bf16, not in the cache yet;
 * append them with gqa_kv_append_fp8 afterwards).  q [B][n][32][128] bf16,
 * out [B][n][32][128] bf16.  The call first writes a bf16 copy of the
 * cached prior into the workspace (code * scale rounded once to bf16, 1 KiB
 * per token: every position before the chunk on a global layer, the
 * 2048-slot ring on a local one) and runs the bf16 prefill on it; ws must
 * hold gqa_workspace_bytes(GQA_OP_PREFILL_FP8, kind, B, n, max pos0 + n)
 * bytes; errors as gqa_attn_prefill.
 * Pages: runtimewire.com "Long context still costs compute" and "Narrow
 * cache". */
int gqa_attn_prefill_fp8(const gqa_layer_fp8* layer, const void* q,
                         const void* k_chunk, const void* v_chunk,
                         const int64_t* pos0, int B, int n, void* out,
                         void* ws, size_t ws_bytes, void* stream);

/* Workspace bytes an operation needs for any call on a layer of `kind` with
 * batch B, n tokens per sequence and context (keys visible to the last
 * query) at most max_ctx.  Returns 0 for invalid arguments. */
size_t gqa_workspace_bytes(int op, int kind, int B, int n, int64_t max_ctx);

/* A static description of a status code. */
const char* gqa_status_string(int status);

/* GQA_ABI_VERSION of the loaded library. */
int gqa_abi_version(void);

#ifdef __cplusplus
}
#endif
#endif
