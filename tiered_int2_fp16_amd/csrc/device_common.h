// Device view of a pool and helpers shared by the gfx950 kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "kvtier.h"

namespace kvtier {

// Page-table entry: bits 0-1 tier, bit 2 has-ledger, bits 3-16 bf16 slot,
// bits 17-31 ledger slot.
enum : int { TIER_E = 0, TIER_Q = 1, TIER_F = 2 };

__host__ __device__ inline int pe_tier(uint32_t e) { return int(e & 3u); }
__host__ __device__ inline bool pe_has_ledger(uint32_t e) { return (e >> 2) & 1u; }
__host__ __device__ inline int pe_bslot(uint32_t e) { return int((e >> 3) & 0x3FFFu); }
__host__ __device__ inline int pe_lslot(uint32_t e) { return int(e >> 17); }
__host__ __device__ inline uint32_t pe_make(int tier, bool has_ledger, int bslot, int lslot) {
  return uint32_t(tier) | (uint32_t(has_ledger) << 2) | (uint32_t(bslot & 0x3FFF) << 3) |
         (uint32_t(lslot) << 17);
}

// Everything a kernel needs to address the pool's arena.
struct PoolView {
  uint16_t* bf16;     // bf16 window slots
  uint8_t* ledger;    // ledger entries ((lbits+1)*W*D/4 bytes each)
  uint32_t* pages;    // [segment][max_windows]
  float* scores;      // [segment][max_windows]
  int32_t* tokens;    // [segment]
  int32_t* work;      // work region (int32 units)
  int32_t* err;       // device error word
  int B, L, Hq, Hkv, D, W, maxw, R, nb, nl, G;
  int lbits;          // ledger code width: 2, 4 or 8
  int work_items, work_counts;  // int32 offsets into work
  int cus;            // compute units of the pool's device (launch sizing)

  __device__ uint16_t* block(int seg, int slot, int kvh) const {
    return bf16 + ((size_t(seg) * nb + slot) * Hkv + kvh) * size_t(2 * W * D);
  }
  __device__ uint8_t* entry(int seg, int slot, int kvh) const {
    return ledger + ((size_t(seg) * nl + slot) * Hkv + kvh) * (size_t(lbits + 1) * W * D / 4);
  }
};

__device__ inline void set_err(int32_t* err, int bits) {
  __hip_atomic_fetch_or(err, bits, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

__device__ inline float bf16_to_f32(uint16_t h) { return __uint_as_float(uint32_t(h) << 16); }

// float -> bf16 bits, round to nearest even (finite inputs).
__device__ inline uint16_t f32_to_bf16_rne(float x) {
  uint32_t u = __float_as_uint(x);
  return uint16_t((u + 0x7FFFu + ((u >> 16) & 1u)) >> 16);
}

__device__ inline int windows_of(int tokens, int W) { return (tokens + W - 1) / W; }

}  // namespace kvtier
