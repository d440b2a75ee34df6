// plan.cpp -- work plans of the attention calls (see plan.h).
#include "plan.h"

namespace gqa {

namespace {
size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }
int cus_of(const DeviceShape& dev) { return dev.cus > 0 ? dev.cus : 1; }
}  // namespace

DecodePlan plan_decode(int kind, int B, int64_t max_keys,
                       const DeviceShape& dev) {
  const int cus = cus_of(dev);
  const int64_t tiles = (max_keys + kDecTile - 1) / kDecTile;
  DecodePlan p;
  p.heads_per_wg = kGroup;
  int64_t per;
  if (kind == GQA_LOCAL) {
    if (B <= kLocalSmallMaxBatch) p.heads_per_wg = kLocalSmallHeads;
    // the window is 32 tiles: one tile per workgroup while the launch holds
    // at most one workgroup per CU (batch 4 on 256 CUs), then longer splits
    // so it stays near one per CU
    per = (int64_t)B * kHkv * (kW / kDecTile) / cus;
  } else {
    // as many workgroups as fit the device at once, so the launch runs as
    // one full round (a partial second round would leave part of the
    // device idle at the end)
    int64_t want = (int64_t)cus * kGlobalWGsPerCU / (kHkv * B);
    if (want < 1) want = 1;
    per = (tiles + want - 1) / want;
  }
  if (per > tiles) per = tiles;
  if (per < 1) per = 1;
  // no more splits than the merge takes
  if ((tiles + per - 1) / per > kMaxSplits) per = (tiles + kMaxSplits - 1) /
                                                  kMaxSplits;
  p.tiles_per_split = (int)per;
  p.splits = (int)((tiles + per - 1) / per);
  if (p.splits < 1) p.splits = 1;
  return p;
}

size_t decode_ws_bytes(int B, const DecodePlan& plan) {
  return align256((size_t)B * kHkv * plan.splits * kGroup * (kD + 2) *
                  sizeof(float));
}

// Block operations.  Workgroups take 16 query tokens of one KV head; the key
// range is split across workgroups (down to one 64-key tile each) only when
// the query groups alone cannot give every CU a workgroup: always for
// verification (<= 16 tokens), for short prefills.  Without splits at most
// one workgroup per CU is launched, each walking several work items.  Local
// layers whose keys are split take 8 tokens per workgroup (4 waves) as long
// as the groups of 8 still leave CUs over: each workgroup then holds one or
// two tiles, its chain of query load, tile rotation, products and partial
// rows is latency, and half the rows shorten it.
BlockPlan plan_block(int kind, int B, int n, int64_t max_keys,
                     const DeviceShape& dev, bool always_split) {
  const int cus = cus_of(dev);
  BlockPlan p;
  auto shape = [&](int qpw) {
    p.qpw = qpw;
    p.qgroups = (n + qpw - 1) / qpw;
    // keys one workgroup may see: its window (local) or everything before it
    const int64_t wg_keys =
        kind == GQA_LOCAL ? (int64_t)kW - 1 + qpw : max_keys;
    const int64_t tiles = (wg_keys + kBlkTile - 1) / kBlkTile;
    const int64_t groups = (int64_t)p.qgroups * kHkv * B;
    int64_t splits = 1;
    if (groups < cus) splits = (cus + groups - 1) / groups;
    // down to one tile per workgroup (measured on the local verify: one
    // tile per workgroup beat two now that split partials are 2-byte rows)
    if (splits > tiles) splits = tiles;
    if (splits > kBlkMaxSplits) splits = kBlkMaxSplits;
    if (splits < 1) splits = 1;
    p.splits = (int)splits;
    return groups;
  };
  int64_t groups = shape(kBlkQpw);
  if (kind == GQA_LOCAL && (p.splits > 1 || always_split)) {
    groups = shape(kBlkQpwSmall);
    // groups of 8 fill the CUs (split calls over fp8 caches keep them)
    if (p.splits == 1 && !always_split) groups = shape(kBlkQpw);
  }
  const bool split = p.splits > 1 || always_split;
  const int64_t items = (int64_t)p.splits * groups;
  p.walks = split ? 1 : (int)((items + cus - 1) / cus);
  p.grid = (int)((items + p.walks - 1) / p.walks);
  // local layers without key splits read pre-rotated keys from the
  // workspace; split calls rotate each tile in LDS
  p.klin_bytes = kind == GQA_LOCAL && !split
                     ? align256((size_t)B * ((size_t)kW + n) * kTokenElems * 2)
                     : 0;
  p.part_bytes = split
                     ? align256((size_t)B * kHkv * p.qgroups * p.splits *
                                p.qpw * kGroup * 68 * sizeof(float))
                     : 0;
  return p;
}

// Rotated keys (local layers), then partial sums (split keys).
size_t block_ws_bytes(const BlockPlan& plan) {
  const size_t n = plan.klin_bytes + plan.part_bytes;
  return n ? n : 256;
}

}  // namespace gqa
