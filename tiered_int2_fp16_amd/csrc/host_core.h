// Host-side geometry of a window-tiered KV pool: validation, arena regions,
// workspace sizing.  Pure C++17 (no HIP), so it builds and tests on any host.
#pragma once

#include <cstddef>
#include <cstdint>
#include <string>

#include "kvtier.h"

namespace kvtier {

constexpr int kTile = 32;            // tokens per attention tile = ledger group length
constexpr int kMaxWindows = 4096;    // page-table entries per segment (LDS bound)
constexpr int kMaxTiles = 8192;      // 32-token tiles per segment (LDS bound)
constexpr int kMaxBf16Slots = 16383; // 14-bit slot field
constexpr int kMaxLedgerSlots = 32767;  // 15-bit slot field
constexpr int kAttnThreads = 256;    // 4 wave64 per attention workgroup
constexpr int kAttnWaves = kAttnThreads / 64;

struct Geometry {
  kv_pool_config cfg{};       // ledger_bits normalised: 2, 4 or 8
  int group = 0;              // q heads per kv head
  int segments = 0;           // layers * batch
  size_t bf16_block = 0;      // bytes of one (slot, kv head) bf16 block: K+V
  size_t entry = 0;           // bytes of one (slot, kv head) ledger entry: (b+1)*W*D/4
  size_t off[KV_REGION_COUNT]{};
  size_t size[KV_REGION_COUNT]{};
  size_t total = 0;
  // KV_REGION_WORK sub-layout (int32 offsets into the region)
  size_t work_items = 0;      // int4 [layers][2][batch][max_windows]: window, src, dst, flag
                              // (list 0 demotions, list 1 promotions)
  size_t work_counts = 0;     // int  [layers][2][batch]
};

// Validate `cfg` and fill `g`.  On failure returns false with a message.
bool geometry_init(const kv_pool_config& cfg, Geometry* g, std::string* err);

// Attention split-K factor: workgroups per (sequence, kv head).
int attn_splits(const Geometry& g, int compute_units);

// Byte offsets of the attention workspace regions (each 256-byte aligned).
struct AttnWorkspace {
  size_t partials = 0;   // float [batch][kv_heads][splits][group][D]: unnormalised outputs
  size_t ml = 0;         // float2 [batch][q_heads][splits]: running max, sum of each workgroup
  size_t tile_mass = 0;  // float2 [batch][max_windows*W/32][q_heads]: raw tile mass, its max
  size_t app_mass = 0;   // float2 [batch][q_heads]: the same for an appended token
  size_t app_info = 0;   // int [batch][8]: append decision of the step
  size_t total = 0;
};
AttnWorkspace attn_workspace(const Geometry& g, int splits);

// Tier counts of a segment with n windows and a ledger of ledger_bits-bit
// codes (the router's formula; double precision, evaluated in the documented
// order).
void tier_counts(int n, int n_recent, double budget_frac, double hi_frac, int ledger_bits, int* n_hi,
                 int* n_lo);

inline size_t align256(size_t x) { return (x + 255) & ~size_t(255); }

}  // namespace kvtier
