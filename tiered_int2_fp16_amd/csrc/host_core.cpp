// Host-side geometry of a window-tiered KV pool (pure C++17).
#include "host_core.h"

#include <algorithm>
#include <cmath>

namespace kvtier {

static bool bad(std::string* err, const std::string& m) {
  if (err) *err = m;
  return false;
}

bool geometry_init(const kv_pool_config& c, Geometry* g, std::string* err) {
  if (c.batch < 1 || c.layers < 1) return bad(err, "batch and layers must be >= 1");
  if (c.kv_heads < 1 || c.q_heads < 1 || c.q_heads % c.kv_heads)
    return bad(err, "q_heads must be a positive multiple of kv_heads");
  const int grp = c.q_heads / c.kv_heads;
  if (grp != 1 && grp != 2 && grp != 4 && grp != 7 && grp != 8)
    return bad(err, "GQA group size (q_heads / kv_heads) must be 1, 2, 4, 7 or 8");
  if (c.head_dim != 64 && c.head_dim != 128) return bad(err, "head_dim must be 64 or 128");
  if (c.window < kTile || c.window > 256 || c.window % kTile)
    return bad(err, "window must be a multiple of 32 in [32, 256]");
  if (c.max_windows < 1 || c.max_windows > kMaxWindows)
    return bad(err, "max_windows must be in [1, 4096]");
  // the newest (partial) window must stay bf16: appends write into it
  if (c.n_recent < 1) return bad(err, "n_recent must be >= 1");
  if (c.max_windows * (c.window / kTile) > kMaxTiles)
    return bad(err, "max_windows * window / 32 must be <= 8192 (tiles per segment)");
  if (c.bf16_slots < 1 || c.bf16_slots > kMaxBf16Slots)
    return bad(err, "bf16_slots must be in [1, 16383]");
  if (c.ledger_slots < 0 || c.ledger_slots > kMaxLedgerSlots)
    return bad(err, "ledger_slots must be in [0, 32767]");
  if (c.ledger_bits != 0 && c.ledger_bits != 2 && c.ledger_bits != 4 && c.ledger_bits != 8)
    return bad(err, "ledger_bits must be 0 (= 2), 2, 4 or 8");
  const double segs = double(c.batch) * c.layers;
  if (segs > 1e7) return bad(err, "too many segments");

  Geometry r;
  r.cfg = c;
  r.cfg.ledger_bits = c.ledger_bits == 0 ? 2 : c.ledger_bits;
  r.group = grp;
  r.segments = c.batch * c.layers;
  const size_t wd = size_t(c.window) * c.head_dim;
  r.bf16_block = 2 * wd * 2;
  r.entry = size_t(r.cfg.ledger_bits + 1) * wd / 4;
  const size_t per_seg_heads = size_t(c.kv_heads);
  r.size[KV_REGION_BF16] = size_t(r.segments) * c.bf16_slots * per_seg_heads * r.bf16_block;
  r.size[KV_REGION_LEDGER] = size_t(r.segments) * c.ledger_slots * per_seg_heads * r.entry;
  r.size[KV_REGION_PAGES] = size_t(r.segments) * c.max_windows * 4;
  r.size[KV_REGION_SCORES] = size_t(r.segments) * c.max_windows * 4;
  r.size[KV_REGION_TOKENS] = size_t(r.segments) * 4;
  // work region, in int32 units
  size_t w = 0;
  // per layer, list 0: demotions, 1: promotions (a layer's moves can be
  // planned ahead of another layer's data kernels)
  r.work_items = w;    w += size_t(c.layers) * 2 * size_t(c.batch) * c.max_windows * 4;
  r.work_counts = w;   w += size_t(c.layers) * 2 * size_t(c.batch);
  r.size[KV_REGION_WORK] = w * 4;
  r.size[KV_REGION_ERR] = 4;
  size_t off = 0;
  for (int i = 0; i < KV_REGION_COUNT; ++i) {
    r.off[i] = off;
    off = align256(off + r.size[i]);
  }
  r.total = off;
  *g = r;
  return true;
}

int attn_splits(const Geometry& g, int compute_units) {
  const kv_pool_config& c = g.cfg;
  const int pairs = c.batch * c.kv_heads;
  // two workgroups per compute unit over the whole launch
  int s = (2 * std::max(compute_units, 1) + pairs - 1) / pairs;
  const int tiles = c.max_windows * (c.window / kTile);
  s = std::max(1, std::min(s, 64));
  s = std::min(s, std::max(1, tiles));
  return s;
}

AttnWorkspace attn_workspace(const Geometry& g, int splits) {
  const kv_pool_config& c = g.cfg;
  AttnWorkspace w;
  const size_t pairs = size_t(c.batch) * c.kv_heads;
  const size_t qrows = size_t(c.batch) * c.q_heads;
  size_t off = 0;
  w.partials = off;  off += align256(pairs * splits * g.group * c.head_dim * 4);
  w.ml = off;        off += align256(qrows * splits * 8);
  w.tile_mass = off; off += align256(qrows * size_t(c.max_windows) * (c.window / kTile) * 8);
  w.app_mass = off;  off += align256(qrows * 8);
  w.app_info = off;  off += align256(size_t(c.batch) * 8 * 4);
  w.total = off;
  return w;
}

void tier_counts(int n, int n_recent, double budget_frac, double hi_frac, int ledger_bits, int* n_hi,
                 int* n_lo) {
  volatile double a = hi_frac * double(n);   // volatile: no contraction across steps
  int hi = std::min(n, std::max(n_recent, int(std::floor(a))));
  volatile double b = budget_frac * double(n);
  volatile double c = b - double(hi);
  volatile double d = c * 16.0;
  volatile double e = d / double(ledger_bits + 1);
  int lo = std::max(0, std::min(n - hi, int(std::floor(e))));
  *n_hi = hi;
  *n_lo = lo;
}

}  // namespace kvtier
