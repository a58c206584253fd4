// Tiered decode attention with per-window mass for gfx950 (matrix cores).
//
// QEvict technical summary ("Methodologie: QEvict", "Kernmechanismen",
// "Implementatie"): bf16 windows and ledger windows (INT2 in the summary's
// experiments; 4 or 8 bits per pool here) both take part in attention,
// evicted windows do not; grouped-query attention; the attention each window
// receives is what the cumulative score adds up.  Unlike the summary's
// FlashAttention-2 path, which dequantises and rebuilds caches before attention
// ("Resultaten", efficiency), ledger tiles are decoded in registers inside this
// kernel: HBM carries b + 1 bits per b-bit value (codes plus fp16 scale and
// min per 32 values), never a rebuilt bf16 copy.  "INT2" below names the
// ledger tier at any of its widths.
//
// Work split: grid (splits, kv heads, sequences), 4 wave64 per workgroup.  The
// live 32-token tiles of a (sequence, kv head) are listed per tier (bf16,
// INT2) and each tier's list is cut evenly over all waves of all splits, so
// every wave - and so every SIMD and CU - gets its share of the bytes (mostly
// bf16) and of the decode work (mostly INT2).  A wave requests its first INT2
// tiles, requests its first bf16 tile once the first INT2 tile is in, decodes
// its INT2 tiles while the bf16 data arrives, then streams its bf16 tiles;
// both loops are double-buffered in registers.  It keeps an online softmax
// (running max, sum, output) for the G query heads of its kv head; every
// tile's raw mass is recorded with the running max it was taken at.  A second
// kernel combines the partials of each (sequence, kv head) into the output and
// normalises the window masses (the order of tokens does not matter:
// A.V = A_P.V_P, LogQuant summary, "Positie-agnostische optimalisatie").
// Splitting the combine off keeps every workgroup of the first kernel free of
// device-wide fences and atomics; the kernel boundary orders the two.
//
// One tile = 16x16x32 MFMAs with the token/dim placement of layout.h:
//  bf16: S = K.q^T (bf16 inputs, exact products) then O^T += V^T.P^T with P
//        split into bf16 high and low parts (2^-17 relative error).
//  ledger (b-bit codes, b = 2, 4, 8; INT2 in the QEvict summary's
//        experiments): a code c becomes the fp16 value 1 + c/2^b, exactly
//        (two register operations per pair of codes).  With per-channel K
//        scale s and min m,
//          q.k = sum_d (1 + c/2^b)(2^b s q) + sum_d q (m - 2^b s);
//        2^b s q is exact in fp32 and goes to the MFMA as fp16 high + low
//        parts, the second sum (constant over the tile's tokens) is taken in
//        fp32 - an fp16 rounding of either would shift a whole tile's logits
//        at once.  Each lane forms its own B operand from the tile's scales,
//        which reach it through the wave's LDS buffer.  With per-token V
//        scale s' and min m',
//          sum_t p v = sum_t (1 + c/2^b)(2^b p s') + sum_t (m' - 2^b s')(2^b p) / 2^b:
//        one MFMA per 16 channels for the codes, four for the min term.
//
// A decode step may append a token: it is attended straight from k_new/v_new
// and stored in the newest window by the combine kernel, which also rewrites
// the page table entry and token count - after every attention workgroup has
// read them.
#include <hip/hip_ext.h>
#include <math.h>

#include <type_traits>

#include "host_core.h"
#include "launch.h"
#include "layout.h"

namespace kvtier {

namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int kGMax = 8;     // query heads per kv head supported
constexpr int kMaxSplits = 64;
constexpr int kMassWindows = 16;   // windows per mass block of the combine kernel, at most

__device__ inline int uniform(int x) { return __builtin_amdgcn_readfirstlane(x); }

// 2^x with the hardware instruction (results below 2^-126 flush to zero, which
// is below anything a probability here can contribute)
__device__ inline float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// x combined with the same lane of the other 16-lane rows / 32-lane halves
// (the lanes holding other tokens of the same head)
__device__ inline float max_rows(float x) {
  auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  x = fmaxf(__uint_as_float(a[0]), __uint_as_float(a[1]));
  auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(b[0]), __uint_as_float(b[1]));
}
__device__ inline float sum_rows(float x) {
  auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  x = __uint_as_float(a[0]) + __uint_as_float(a[1]);
  auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(b[0]) + __uint_as_float(b[1]);
}

// x summed over the column groups of a 16-lane row: lanes n, n + 16/NREP, ..
// (DPP row rotations by 4 and 8 lanes, or by 8 alone)
template <int NREP>
__device__ inline float sum_groups_t(float x) {
  if constexpr (NREP == 4)
    x += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x124, 0xF, 0xF, false));  // row_ror:4
  if constexpr (NREP >= 2)
    x += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x128, 0xF, 0xF, false));  // row_ror:8
  return x;
}

// Materialise uniform values (kernel arguments) in SGPRs at this point.
template <typename T>
__device__ inline void in_sgpr(const T& x) {
  asm volatile("" ::"s"(x));
}
template <typename... T>
__device__ inline void in_sgprs(const T&... x) {
  (in_sgpr(x), ...);
}

__device__ inline f32x4 mfma_bf16(bf16x8 a, bf16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}
__device__ inline f32x4 mfma_f16(f16x8 a, f16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
}

// Inclusive prefix sum over the 64 lanes of a wave (DPP row shifts within
// 16-lane rows, then row broadcasts across them).
__device__ inline int wave_incl_scan(int x) {
  x += __builtin_amdgcn_update_dpp(0, x, 0x111, 0xF, 0xF, false);  // row_shr:1
  x += __builtin_amdgcn_update_dpp(0, x, 0x112, 0xF, 0xF, false);  // row_shr:2
  x += __builtin_amdgcn_update_dpp(0, x, 0x114, 0xF, 0xF, false);  // row_shr:4
  x += __builtin_amdgcn_update_dpp(0, x, 0x118, 0xF, 0xF, false);  // row_shr:8
  x += __builtin_amdgcn_update_dpp(0, x, 0x142, 0xA, 0xF, false);  // row_bcast:15 -> rows 1, 3
  x += __builtin_amdgcn_update_dpp(0, x, 0x143, 0xC, 0xF, false);  // row_bcast:31 -> rows 2, 3
  return x;
}

// Buffer resource over `bytes` bytes at `base` (raw, unswizzled).  Lanes whose
// offset is out of range read zeros and touch no memory; bytes == 0 makes a
// whole load a no-op.
__device__ inline __amdgpu_buffer_rsrc_t tile_rsrc(const void* base, int bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, bytes, 0x00020000);
}
__device__ inline uint4 load16(__amdgpu_buffer_rsrc_t r, int off) {
  return __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0));
}
// Wait for every outstanding vector memory operation (s_waitcnt vmcnt(0),
// other counters left alone).
__device__ inline void drain_loads() { __builtin_amdgcn_s_waitcnt(0x0F70); }
__device__ inline uint32_t load4(__amdgpu_buffer_rsrc_t r, int off) {
  return uint32_t(__builtin_amdgcn_raw_buffer_load_b32(r, off, 0, 0));
}
// A buffer offset, or (when !valid) one past any resource here: that lane
// reads zeros and touches no memory.
__device__ inline int boff(bool valid, int off) { return valid ? off : int(0x80000000u); }
__device__ inline float2 as_f2(uint2 u) { return make_float2(__uint_as_float(u.x), __uint_as_float(u.y)); }
__device__ inline uint2 load8(__amdgpu_buffer_rsrc_t r, int off) {
  return __builtin_bit_cast(uint2, __builtin_amdgcn_raw_buffer_load_b64(r, off, 0, 0));
}

// (m & y) | (~m & c): one v_bfi_b32 when m and c sit in VGPRs the optimiser
// cannot see into (see opaque()).  Written as plain operations, not inline
// assembly: the compiler then knows the instruction's VGPR write and inserts
// the wait states a matrix-core read of the result needs.
__device__ inline uint32_t bit_select(uint32_t m, uint32_t y, uint32_t c) { return (m & y) | (~m & c); }
// x in a VGPR, its value hidden from constant folding (no instruction is
// emitted): two constants of a bit select stay register operands of one
// instruction instead of being folded into two literal operations.
__device__ inline uint32_t opaque(uint32_t x) {
  asm volatile("" : "+v"(x));
  return x;
}

// Eight INT2 codes of one operand chunk -> fp16 (1 + c/4).  Word X holds the
// fields of chunks 2w (SEL 0) and 2w+1 (SEL 1); register j takes the fields
// j + 4*SEL (low half) and j + 4*SEL + 8 (high half), 16 bits apart: one shift
// puts both at mantissa bits 8-9 and a bit select adds the exponent of 1.0.
// `mask` = 0x03000300 and `one` = 0x3C003C00 come in registers.
template <int SEL>
__device__ inline f16x8 decode_codes(uint32_t X, uint32_t mask, uint32_t one) {
  uint32_t r[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int sh = 2 * (j + 4 * SEL);
    const uint32_t y = sh <= 8 ? (X << (8 - sh)) : (X >> (sh - 8));
    r[j] = bit_select(mask, y, one);
  }
  return __builtin_bit_cast(f16x8, make_uint4(r[0], r[1], r[2], r[3]));
}

// Eight 4-bit codes of one chunk (word X, field f = element 2(f%4) + f/4)
// -> fp16 (1 + c/16): register j takes fields j and j + 4, 16 bits apart; one
// shift puts both at mantissa bits 6-9, a bit select adds the exponent of 1.0.
// `mask` = 0x03C003C0 and `one` = 0x3C003C00 come in registers.
__device__ inline f16x8 decode_codes4(uint32_t X, uint32_t mask, uint32_t one) {
  uint32_t r[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int sh = 4 * j;
    const uint32_t y = sh <= 6 ? (X << (6 - sh)) : (X >> (sh - 6));
    r[j] = bit_select(mask, y, one);
  }
  return __builtin_bit_cast(f16x8, make_uint4(r[0], r[1], r[2], r[3]));
}

// Eight 8-bit codes of one chunk (bytes 0-3 of X0, then of X1, in element
// order) -> fp16 (1 + c/256): a byte permute spreads elements 2j, 2j+1 over
// the low bytes of the two halves, a shift-or places them at mantissa bits
// 2-9 under the exponent of 1.0.
__device__ inline f16x8 decode_codes8(uint32_t X0, uint32_t X1) {
  uint32_t r[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const uint32_t t = __builtin_amdgcn_perm(0u, (j >> 1) ? X1 : X0, (j & 1) ? 0x0C030C02u : 0x0C010C00u);
    r[j] = (t << 2) | 0x3C003C00u;
  }
  return __builtin_bit_cast(f16x8, make_uint4(r[0], r[1], r[2], r[3]));
}

// The fp16 values 1 + c/2^BITS of the eight codes of chunk c of a part
// (`w`: the lane's code words of that part).
template <int BITS, int CW>
__device__ inline f16x8 decode_chunk(const uint32_t (&w)[CW], int c, uint32_t mask, uint32_t one) {
  if constexpr (BITS == 2)
    return (c & 1) ? decode_codes<1>(w[c >> 1], mask, one) : decode_codes<0>(w[c >> 1], mask, one);
  else if constexpr (BITS == 4)
    return decode_codes4(w[c], mask, one);
  else
    return decode_codes8(w[2 * c], w[2 * c + 1]);
}

__device__ inline bf16x8 as_bf16x8(uint4 u) { return __builtin_bit_cast(bf16x8, u); }

// Tile table entry: slot (15 bits) | window (12 bits) << 15 | tile (3 bits) << 27
__device__ inline uint32_t te_make(int slot, int w, int k) {
  return uint32_t(slot) | (uint32_t(w) << 15) | (uint32_t(k) << 27);
}
__device__ inline int te_slot(uint32_t e) { return int(e & 0x7FFFu); }
__device__ inline int te_win(uint32_t e) { return int((e >> 15) & 0xFFFu); }
__device__ inline int te_tile(uint32_t e) { return int(e >> 27); }

// per-wave running softmax state and accumulators
template <int NB>
struct WaveState {
  float m_run, l_run;
  f32x4 o[NB];   // O^T block nb: lane (g, n) holds column n, channels 16nb + 4g + i
  f32x4 ob;      // 2^b x ledger V min term: lane (0, n) holds column n, channel group i
};

// Online softmax over one tile of 8 scores per lane, z = s * scale + shift
// (scale > 0; a score of -inf is a masked token).  The reference max m_run is
// raised lazily: only when some head's tile max exceeds it by more than kTau
// do all heads move to their new max and the accumulators rescale (not at all
// on the wave's first tile, when they are still zero).  Until then a tile's
// values are taken against the older reference, so p <= 2^kTau.  Returns
// p[e] = 2^LG exp2(z[e] - m_run) and the tile sum of exp2(z - m_run).
// (2^b p <= 2^(b+3) keeps 2^b p s' in fp16 range for |s'| < 65504 / 2^(b+3))
constexpr float kTau = 3.f;

template <int NB, int LG>
__device__ inline void softmax_tile(WaveState<NB>& st, const float (&s)[8], float scale, float shift,
                                    float (&p)[8], float* rs_out) {
  float sm = s[0];
#pragma unroll
  for (int e = 1; e < 8; ++e) sm = fmaxf(sm, s[e]);
  const float tm = fmaf(max_rows(sm), scale, shift);
  if (__builtin_amdgcn_ballot_w64(tm > st.m_run + kTau)) {
    const float mn = fmaxf(st.m_run, tm);
    if (st.m_run != -INFINITY) {   // the same on every lane: all heads start and move together
      const float alpha = fast_exp2(st.m_run - mn);
#pragma unroll
      for (int nb = 0; nb < NB; ++nb) st.o[nb] *= alpha;
      st.ob *= alpha;
      st.l_run *= alpha;
    }
    st.m_run = mn;
  }
  const float off = shift - st.m_run + float(LG);
  float rs = 0.f;
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    p[e] = fast_exp2(fmaf(s[e], scale, off));
    rs += p[e];
  }
  rs = sum_rows(rs) * (1.f / float(1 << LG));
  st.l_run += rs;
  *rs_out = rs;
}

}  // namespace

// The first six arguments (the layer's page table and token counts, the page
// table's row length, the query and its head counts) come preloaded in SGPRs
// (the library is built with kernarg preloading), so the first loads - page
// table, token count, query - need no kernel-argument load.
template <int D, int GP, int BITS>
__global__ __launch_bounds__(256, 2) void attn_kernel(const uint32_t* __restrict__ pages_layer,
                                                      const int32_t* __restrict__ tokens_layer, int maxw_arg,
                                                      const uint16_t* __restrict__ q_arg, int hq_arg, int g_arg,
                                                      PoolView pv, AttnArgs a) {
  constexpr int KK = D / 32;   // 32-dim slices of the QK product
  constexpr int NB = D / 16;   // 16-channel blocks of the PV product (= code chunks per part)
  constexpr int CW = BITS * D / 64;   // 32-bit code words per lane per part
  constexpr int SCW = D / 32;        // 32-bit words per lane of a tile's scale block
  constexpr float kCodeScale = float(1 << BITS);   // 2^b
  constexpr int kList = 64;    // tile entries a wave lists at a time
  constexpr int kMixedList = 8;   // INT2 tiles from which a wave takes both tiers in one loop
  extern __shared__ uint32_t s_dyn[];    // plan (page entries, tile prefixes), slot bitmap
  __shared__ float s_wm[kAttnWaves][kGMax], s_wl[kAttnWaves][kGMax];
  __shared__ float s_wo[kAttnWaves][kGMax][D];
  __shared__ float s_wb[kAttnWaves][kGMax][4];
  __shared__ __attribute__((aligned(16))) uint8_t s_scb[kAttnWaves][8 * D];  // ledger tile scales
  __shared__ float2 s_rec[kAttnWaves][kList][kGMax];                           // their raw masses
  __shared__ int s_gt[kMaxWindows / 64];                                       // tiles per 64 windows

  const int split = blockIdx.x, kvh = blockIdx.y, b = blockIdx.z;
  const int tid = threadIdx.x, lane = tid & 63, wid = uniform(tid >> 6);
  const int g = lane >> 4, hn = lane & 15;   // lane = (column block g, column hn)
  // The 16 MFMA columns carry the query heads replicated: column hn holds head
  // hh = hn % GP of column group jc = hn / GP (GP = 4 when G <= 4, else 8).
  // bf16 tiles and INT2 logits give every group the same values; in an INT2
  // tile's V product group jc carries the scales of one 32-channel group, so
  // a single B operand serves RG channel groups (NPASS operands per tile).
  constexpr int RG = (D / 32) < (16 / GP) ? (D / 32) : (16 / GP);
  constexpr int NPASS = (D / 32) / RG;
  constexpr int NREP = 16 / GP;                            // column groups
  constexpr int NKK = (D / 32) > NREP ? (D / 32) / NREP : 1;   // tile-constant slices per lane
  const int hh = hn % GP, jc = hn / GP;
  const int W = pv.W, maxw = pv.maxw, TPW = W / 32, G = pv.G;
  const int seg = a.layer * pv.B + b;
  const int S = a.splits;

  // ------------------------------------- first: page table and token count
  // issued before anything that needs the kernel arguments in memory; the
  // first 1024 entries of the table (entries past the row read 0)
  uint32_t e_first[4];
  {
    const auto prs = tile_rsrc(pages_layer + size_t(b) * maxw_arg, maxw_arg * 4);
#pragma unroll
    for (int j = 0; j < 4; ++j) e_first[j] = load4(prs, (256 * j + tid) * 4);
  }
  // (a vector load, so it goes out now rather than after the argument loads)
  const uint32_t len_raw = load4(tile_rsrc(tokens_layer, (b + 1) * 4), b * 4);

  // ------------------------------------------------------------ the query
  // also from preloaded arguments: it does not depend on the plan.  Lane
  // (g, hn) holds channels 32kk + 8g .. 32kk + 8g + 7 of head hh: the B
  // operand of the QK products.  Buffer loads without a branch (lanes of heads
  // past G read zeros), so the plan's wait for the page table is exact.
  constexpr float kLog2e = 1.4426950408889634f;
  const float qscale = kLog2e / sqrtf(float(D));
  bf16x8 qb[KK];    // q (bf16)
  {
    const auto rq = tile_rsrc(q_arg + (size_t(b) * hq_arg + size_t(kvh) * g_arg) * D, g_arg * D * 2);
#pragma unroll
    for (int kk = 0; kk < KK; ++kk)
      qb[kk] = as_bf16x8(load16(rq, boff(hh < g_arg, (hh * D + 32 * kk + 8 * g) * 2)));
  }
  __builtin_amdgcn_sched_barrier(0);   // the page table, token count and query loads stay in this order
  // Every other kernel argument the kernel reads, fetched in one batch while
  // those loads are in flight.  Left to itself the compiler requests some
  // before the page table (so the first HBM load waits for an argument round
  // trip) and the plan's only after the page table arrives (a second one).
  in_sgprs(pv.bf16, pv.ledger, pv.pages, pv.err, a.k_new, a.v_new, a.mass, a.partials, a.ml, a.tile_mass,
           a.app_mass, a.app_info);
  in_sgprs(pv.B, pv.Hq, pv.Hkv, pv.W, pv.maxw, pv.nb, pv.nl, pv.G, a.layer, a.splits, a.plan_words, a.acc_scores);

  // ------------------------------------------------ tile plan (workgroup)
  // The page table goes to LDS once per workgroup: thread t takes windows
  // t, t + 256, ...; their entries are loaded before the token count is known.
  // s_ex[w] holds the live tiles before window w within its 64-window group
  // (bf16 tiles in the low 16 bits, INT2 tiles in the high 16 bits) and
  // s_gt[r] the total of group r.  After a barrier every thread writes the
  // tile entries of its windows into s_tiles - all live bf16 tiles in window
  // order, then all INT2 tiles - and after a second barrier each wave reads
  // its share of that array as its tile lists.  (Having each wave search the
  // table for its own tiles took about a microsecond of issue per wave.)
  uint32_t* s_pe = s_dyn;                                        // [roundup(maxw, 256)]
  int* s_ex = reinterpret_cast<int*>(s_dyn + a.plan_words);      // [roundup(maxw, 256)]
  uint32_t* s_tiles = s_dyn + 2 * a.plan_words;                  // [maxw * W / 32]
  uint32_t* s_used = s_tiles + maxw * TPW;                       // bf16 slot bitmap (append)
  const int len_old = uniform(int(len_raw));
  const uint32_t* gp = pv.pages + size_t(seg) * maxw;
  const int n_old = windows_of(len_old, W);
  auto tiles_of = [&](uint32_t e, int w) -> int {
    if (w >= n_old) return 0;
    const int t = pe_tier(e);
    const int vt = (min(W, len_old - w * W) + 31) / 32;
    return t == TIER_F ? vt : (t == TIER_Q ? (vt << 16) : 0);
  };
  int ex_first[4];   // the first 1024 windows' prefixes, kept for the scatter below
  {
    const int JR = a.plan_words / 256;
    auto stage = [&](const uint32_t (&e4)[4], int j0, int (&ex4)[4]) {
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        ex4[j] = 0;
        if ((j0 == 0 && j == 0) || j0 + j < JR) {   // JR >= 1: the first group always stages
          const int w = 256 * (j0 + j) + tid;
          const int c = tiles_of(e4[j], w);
          const int incl = wave_incl_scan(c);
          s_pe[w] = e4[j];
          s_ex[w] = incl - c;
          ex4[j] = incl - c;
          if (lane == 63) s_gt[w >> 6] = incl;
        }
      }
    };
    stage(e_first, 0, ex_first);
    if (JR > 4) {   // a table of more than 1024 windows
      const auto pt = tile_rsrc(gp, maxw * 4);   // lanes past the table read 0
      for (int j0 = 4; j0 < JR; j0 += 4) {
        uint32_t e4[4];
        int ex4[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) e4[j] = load4(pt, (256 * (j0 + j) + tid) * 4);
        stage(e4, j0, ex4);
      }
      // Nothing of this path is left pending: otherwise the compiler's wait
      // analysis keeps these loads in flight on every path and waits for all
      // loads (the query included) before reusing their registers.
      drain_loads();
    }
  }
  __syncthreads();
  const int NG = (n_old + 63) / 64;   // 64-window groups (<= 64)
  int gbase;                           // lane r: live tiles before group r
  int tot;
  {
    const int t = lane < NG ? s_gt[lane] : 0;
    const int incl = wave_incl_scan(t);
    gbase = incl - t;
    tot = __builtin_amdgcn_readlane(incl, 63);
  }
  const int NF = tot & 0xFFFF, NQ = tot >> 16;
  {
    // thread t places the tiles of windows t, t + 256, ...: window 256j + t
    // lies in group 4j + wid (the same for the whole wave).  The first 1024
    // windows' entries and prefixes are still in registers from the staging.
    const int JR = a.plan_words / 256;
    for (int j = 0; j < JR; ++j) {
      const int grp = 4 * j + wid;
      if (grp >= NG) break;
      const int gb = __builtin_amdgcn_readlane(gbase, grp);
      const int w = 256 * j + tid;
      if (w < n_old) {
        uint32_t e;
        int ex;
        if (j < 4) {
          e = j == 0 ? e_first[0] : (j == 1 ? e_first[1] : (j == 2 ? e_first[2] : e_first[3]));
          ex = j == 0 ? ex_first[0] : (j == 1 ? ex_first[1] : (j == 2 ? ex_first[2] : ex_first[3]));
        } else {
          e = s_pe[w];
          ex = s_ex[w];
        }
        const int t = pe_tier(e);
        if (t == TIER_F || t == TIER_Q) {
          const int sh = t == TIER_F ? 0 : 16;
          const int ti = ((gb >> sh) & 0xFFFF) + ((ex >> sh) & 0xFFFF) + (t == TIER_F ? 0 : NF);
          const int vt = (min(W, len_old - w * W) + 31) / 32;
          const int sl = t == TIER_F ? pe_bslot(e) : pe_lslot(e);
          for (int k = 0; k < vt; ++k) s_tiles[ti + k] = te_make(sl, w, k);
        }
      }
    }
  }
  __syncthreads();
  // Every wave takes an even share of the bf16 tiles and, separately, of the
  // INT2 tiles, so HBM bytes (mostly bf16) and decode work (mostly INT2) are
  // spread alike over all waves - and so over all SIMDs and CUs.
  const int nwaves = S * kAttnWaves, widx = split * kAttnWaves + wid;
  const int q_beg = widx * NQ / nwaves, q_end = (widx + 1) * NQ / nwaves;
  // INT2 shares of k or k + 1 tiles: when the bf16 tiles fit on the waves
  // with k, only those take them (evenly), so no wave holds both an extra
  // INT2 tile and a bf16 tile.  Waves with k + 1 before wave x:
  // floor(x NQ / nwaves) - k x.
  int f_beg, f_end;
  {
    const int k = NQ / nwaves, n_lo = (k + 1) * nwaves - NQ;
    if (NQ % nwaves != 0 && NF <= n_lo) {
      const int r = widx - (q_beg - k * widx);   // rank among the k-tile waves
      const bool lo = q_end - q_beg == k;
      f_beg = r * NF / n_lo;
      f_end = lo ? (r + 1) * NF / n_lo : f_beg;
    } else {
      f_beg = widx * NF / nwaves;
      f_end = (widx + 1) * NF / nwaves;
    }
  }
  // the wave's current chunk of each list (at most kList tiles of a tier)
  const uint32_t* listf = s_tiles + f_beg;
  const uint32_t* listq = s_tiles + NF + q_beg;

  // ------------------------------------------------- the append decision
  // Taken by wave 0 of split 0 of each (sequence, kv head); the combine kernel
  // stores the token and rewrites the page table after every workgroup read it.
  int app_ok = 0, app_slot = 0, app_row = 0, app_new = 0, app_err = 0;
  if (a.k_new != nullptr && split == 0 && wid == 0) {
    if (len_old % W != 0) {
      const uint32_t e = s_pe[n_old - 1];
      app_ok = pe_tier(e) == TIER_F;
      app_slot = pe_bslot(e);
      app_row = len_old % W;
      if (!app_ok) app_err = KV_ERR_APPEND_STATE;
    } else {
      // a new window opens: the lowest bf16 slot no live bf16 window holds
      const int words = (pv.nb + 31) / 32;
      for (int i = lane; i < words; i += 64) s_used[i] = 0u;
      __builtin_amdgcn_wave_barrier();
      for (int w = lane; w < n_old; w += 64) {
        const uint32_t e = s_pe[w];
        if (pe_tier(e) == TIER_F && pe_bslot(e) < pv.nb)
          atomicOr(&s_used[pe_bslot(e) >> 5], 1u << (pe_bslot(e) & 31));
      }
      __builtin_amdgcn_wave_barrier();
      int slot = 0x7FFFFFFF;
      for (int i = lane; i < words; i += 64) {
        const uint32_t x = ~s_used[i];
        if (x) {
          const int j = i * 32 + __builtin_ctz(x);
          if (j < pv.nb) slot = min(slot, j);
        }
      }
#pragma unroll
      for (int off = 32; off > 0; off >>= 1) slot = min(slot, __shfl_xor(slot, off, 64));
      const bool cap = n_old < maxw;
      app_ok = cap && slot != 0x7FFFFFFF;
      app_slot = app_ok ? slot : 0;
      app_new = 1;
      if (!app_ok) app_err = cap ? KV_ERR_NO_BF16_SLOT : KV_ERR_CAPACITY;
    }
  }
  // (the decision and any error bits are stored at the end of the kernel: a
  // store here would count among the loads in flight - loads and stores share
  // one counter - and make the first tile wait for all of them)

  WaveState<NB> st;
  st.m_run = -INFINITY;
  st.l_run = 0.f;
#pragma unroll
  for (int nb = 0; nb < NB; ++nb) st.o[nb] = f32x4{0.f, 0.f, 0.f, 0.f};
  st.ob = f32x4{0.f, 0.f, 0.f, 0.f};
  // raw tile masses of this kv head's query heads: row h holds tile w*TPW + k
  // raw tile masses: row (tile w*TPW + k), column query head
  float2* tmass = a.tile_mass + size_t(b) * maxw * TPW * pv.Hq + size_t(kvh) * G;
  // tile masses feed the window masses and the fused score update
  const bool want_mass = a.mass != nullptr || a.acc_scores != 0;
  const bool rec_mass = want_mass && g == 0 && hn < G;
  float2(*rec)[kGMax] = s_rec[wid];
  // the raw masses of a listed chunk of nt tiles go out after the chunk: no
  // global store inside the tile loops, where it would hold up the next
  // tile's loads
  auto flush_masses = [&](int nt, const uint32_t* list, bool from_top = false) {
    if (!want_mass) return;
    __builtin_amdgcn_wave_barrier();
    // heads fastest: the G records of a tile (adjacent in memory) go out from
    // adjacent lanes, one contiguous piece per tile
    for (int idx = lane; idx < nt * G; idx += 64) {
      const int t = idx / G, h = idx - t * G;
      const uint32_t e = list[t];
      tmass[(size_t(te_win(e)) * TPW + te_tile(e)) * pv.Hq + h] = rec[from_top ? kList - 1 - t : t][h];
    }
    __builtin_amdgcn_wave_barrier();
  };

  // ------------------------------------------------------------ tile loops
  // Issue order: the first two INT2 tiles, then the first bf16 tile, then the
  // INT2 tiles are decoded while the (larger) bf16 data is still arriving;
  // the bf16 tiles come last.  Loads go through a buffer resource spanning one
  // tile; a prefetch past the last tile gets an empty resource and reads zeros
  // without touching memory, so no load sits behind a branch and every tile
  // waits only for its own loads.
  constexpr int kTileBytes = 64 * D * 2;
  struct FB {
    uint4 k[NB];
    uint4 v[NB];
  };
  auto load_f = [&](FB& fb, int i, int nt) {
    const uint32_t e = uniform(int(listf[max(0, min(i, nt - 1))]));
    const uint16_t* base = pv.block(seg, te_slot(e), kvh) + size_t(te_tile(e)) * 64 * D;
    const auto rs = tile_rsrc(base, i < nt ? kTileBytes : 0);
#pragma unroll
    for (int c = 0; c < NB; ++c) fb.k[c] = load16(rs, (c * 64 + lane) * 16);
#pragma unroll
    for (int c = 0; c < NB; ++c) fb.v[c] = load16(rs, 32 * D * 2 + (c * 64 + lane) * 16);
  };
  auto compute_f = [&](FB& fb, int t) {   // record row t
    const uint32_t e = uniform(int(listf[t]));
    const int w = te_win(e), k = te_tile(e);
    const int valid = min(32, len_old - w * W - 32 * k);
    f32x4 s0 = {0.f, 0.f, 0.f, 0.f}, s1 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int kk = 0; kk < KK; ++kk) {
      s0 = mfma_bf16(as_bf16x8(fb.k[kk]), qb[kk], s0);
      s1 = mfma_bf16(as_bf16x8(fb.k[KK + kk]), qb[kk], s1);
    }
    float z[8], p[8], rs;
#pragma unroll
    for (int i4 = 0; i4 < 4; ++i4) {
      z[i4] = (8 * g + i4 < valid) ? s0[i4] : -INFINITY;
      z[4 + i4] = (8 * g + 4 + i4 < valid) ? s1[i4] : -INFINITY;
    }
    softmax_tile<NB, 0>(st, z, qscale, 0.f, p, &rs);
    if (valid < 32) {   // stale values past the last token: zero them (0 * NaN)
#pragma unroll
      for (int c = 0; c < NB; ++c) {
        uint32_t w4[4] = {fb.v[c].x, fb.v[c].y, fb.v[c].z, fb.v[c].w};
#pragma unroll
        for (int e2 = 0; e2 < 4; ++e2) {
          if (8 * g + 2 * e2 >= valid) w4[e2] &= 0xFFFF0000u;
          if (8 * g + 2 * e2 + 1 >= valid) w4[e2] &= 0x0000FFFFu;
        }
        fb.v[c] = make_uint4(w4[0], w4[1], w4[2], w4[3]);
      }
    }
    bf16x8 ph, pl;
#pragma unroll
    for (int e2 = 0; e2 < 8; ++e2) {
      ph[e2] = (__bf16)p[e2];
      pl[e2] = (__bf16)(p[e2] - float(ph[e2]));
    }
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) {
      st.o[nb] = mfma_bf16(as_bf16x8(fb.v[nb]), ph, st.o[nb]);
      st.o[nb] = mfma_bf16(as_bf16x8(fb.v[nb]), pl, st.o[nb]);
    }
    if (rec_mass) rec[t][hn] = make_float2(rs, st.m_run);
  };

  // decode constants (mask of a code pair's fields, exponent of 1.0), held in
  // VGPRs for the bit selects
  const uint32_t kMaskR = opaque(BITS == 2 ? 0x03000300u : 0x03C003C0u), kOneR = opaque(0x3C003C00u);
  const float kNegOne = __int_as_float(uniform(int(opaque(0xBF800000u))));   // -1.0f in an SGPR
  // 2^b q in fp16 (4q for INT2) and this lane's slices of the tile constant
  // (q4[jc + i * NREP], zero past KK); formed once the wave's first tile loads
  // are out, so the wait for the query never holds them back
  f16x8 q4[KK];
  f16x8 q4s[NKK];
  auto make_q4 = [&]() {
#pragma unroll
    for (int kk = 0; kk < KK; ++kk)
#pragma unroll
      for (int e = 0; e < 8; ++e) q4[kk][e] = (_Float16)(kCodeScale * float(qb[kk][e]));
#pragma unroll
    for (int i = 0; i < NKK; ++i) {
      q4s[i] = f16x8{0, 0, 0, 0, 0, 0, 0, 0};
#pragma unroll
      for (int kk = 0; kk < KK; ++kk)
        if (jc + i * NREP == kk) q4s[i] = q4[kk];
    }
  };
  const layout::LedgerTile LT(D, BITS);
  struct QB {
    uint32_t kc[CW], vc[CW], sc[SCW];
  };
  // a lane's NW consecutive words of an area (16-byte loads, or one 8-byte load)
  auto load_words = [&](__amdgpu_buffer_rsrc_t rs, int off, auto& w) {
    constexpr int NW = sizeof(w) / sizeof(uint32_t);
    if constexpr (NW % 4 == 0) {
#pragma unroll
      for (int i = 0; i < NW / 4; ++i) {
        const uint4 u = load16(rs, off + lane * NW * 4 + 16 * i);
        w[4 * i] = u.x;
        w[4 * i + 1] = u.y;
        w[4 * i + 2] = u.z;
        w[4 * i + 3] = u.w;
      }
    } else {
      const uint2 u = load8(rs, off + lane * 8);
      w[0] = u.x;
      w[1] = u.y;
    }
  };
  auto load_q = [&](QB& qq, int i, int nt) {
    const uint32_t e = uniform(int(listq[max(0, min(i, nt - 1))]));
    const uint8_t* t = pv.entry(seg, te_slot(e), kvh) + size_t(te_tile(e)) * LT.bytes;
    const auto rs = tile_rsrc(t, i < nt ? LT.bytes : 0);
    load_words(rs, LT.kc, qq.kc);
    load_words(rs, LT.vc, qq.vc);
    load_words(rs, LT.ks, qq.sc);
  };
  uint8_t* scb = s_scb[wid];
  auto compute_q = [&](QB& qq, int t, int rt) {   // record row rt
    // the tile's scale block (Ks | Km | Vs | Vm) into this wave's LDS buffer.
    // Lanes read each other's words: wavefront-scope fences order the previous
    // tile's reads before this store and this store before the reads below
    // (the compiler may not move LDS accesses across them; they emit no
    // instruction, since the LDS completes one wave's operations in order).
    __builtin_amdgcn_fence(__ATOMIC_ACQ_REL, "wavefront");
    __builtin_amdgcn_wave_barrier();
    if constexpr (SCW == 4)
      reinterpret_cast<uint4*>(scb)[lane] = make_uint4(qq.sc[0], qq.sc[1], qq.sc[2], qq.sc[3]);
    else
      reinterpret_cast<uint2*>(scb)[lane] = make_uint2(qq.sc[0], qq.sc[1]);
    __builtin_amdgcn_fence(__ATOMIC_ACQ_REL, "wavefront");
    __builtin_amdgcn_wave_barrier();
    const f16x8* ks = reinterpret_cast<const f16x8*>(scb);              // [D]
    const f16x8* km = reinterpret_cast<const f16x8*>(scb + 2 * D);      // [D]
    const f16x8* vs = reinterpret_cast<const f16x8*>(scb + 4 * D);      // [D/32][32]
    const f16x8* vm = reinterpret_cast<const f16x8*>(scb + 6 * D);
    // Each lane forms its own B operand: 2^b s q as an fp16 product plus its
    // exact fp16 residual (fma TwoProduct).  The tile constant
    // sum_d q (m - 2^b s) = sum 2^b q m / 2^b - sum 2^b q s (fp16 pairs, fp32
    // sums) is split over the column groups (group jc takes slices jc,
    // jc + NREP, ..) and completed across groups and lane rows.
    f32x4 s0 = {0.f, 0.f, 0.f, 0.f}, s1 = {0.f, 0.f, 0.f, 0.f};
    float cm = 0.f, cs = 0.f;
#pragma unroll
    for (int i = 0; i < NKK; ++i) {
      const int kk = min(jc + i * NREP, KK - 1);   // q4s is zero past the last slice
      const f16x8 m8 = km[4 * kk + g], s8 = ks[4 * kk + g];
#pragma unroll
      for (int e2 = 0; e2 < 4; ++e2) {
        const f16x2 qq2 = {q4s[i][2 * e2], q4s[i][2 * e2 + 1]};
        cm = __builtin_amdgcn_fdot2(qq2, f16x2{m8[2 * e2], m8[2 * e2 + 1]}, cm, false);
        cs = __builtin_amdgcn_fdot2(qq2, f16x2{s8[2 * e2], s8[2 * e2 + 1]}, cs, false);
      }
    }
    // A wave raises its priority for the QK and PV sections (code decode and
    // MFMA), so the SIMD's two waves take turns: one there while the other
    // runs its softmax (attention 1.5 % faster at 32K; on the bf16 tiles it
    // made no measurable difference and is not used).
    __builtin_amdgcn_s_setprio(1);
#pragma unroll
    for (int kk = 0; kk < KK; ++kk) {
      const f16x8 s8 = ks[4 * kk + g];
      const f16x8 qh = q4[kk] * s8;
      const f16x8 ql = __builtin_elementwise_fma(q4[kk], s8, -qh);
      const int c0 = kk, c1 = KK + kk;                               // chunks of blk 0 / 1
      const f16x8 a0 = decode_chunk<BITS>(qq.kc, c0, kMaskR, kOneR);
      const f16x8 a1 = decode_chunk<BITS>(qq.kc, c1, kMaskR, kOneR);
      s0 = mfma_f16(a0, qh, s0);
      s0 = mfma_f16(a0, ql, s0);
      s1 = mfma_f16(a1, qh, s1);
      s1 = mfma_f16(a1, ql, s1);
    }
    __builtin_amdgcn_s_setprio(0);
    // the MFMA result lanes (g, hn) hold head hh, as the B operand lanes do
    const float bias0 = sum_rows(sum_groups_t<NREP>(fmaf(cm, 1.f / kCodeScale, -cs)));
    const float z[8] = {s0[0], s0[1], s0[2], s0[3], s1[0], s1[1], s1[2], s1[3]};
    float p[8], rs;
    softmax_tile<NB, BITS>(st, z, qscale, bias0 * qscale, p, &rs);   // p = 2^b x probability
    // 2^b p as fp16 high + low parts, then 2^b p s' = high*s' + (exact
    // residual of that product + low*s'), all in packed fp16
    // (the residual x - p4 is exact in fp32; taken as a fused multiply-add
    // by -1 held in a register, it is one mixed-precision FMA that reads its
    // fp16 half of p4's packed register, instead of a conversion back to fp32
    // and a subtraction; the empty asm keeps the compiler from converting p
    // to fp16 a second time for those reads)
    f16x8 p4, p4l;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const f16x2 h2 = __builtin_bit_cast(
          f16x2, opaque(__builtin_bit_cast(uint32_t, f16x2{(_Float16)p[2 * r], (_Float16)p[2 * r + 1]})));
      p4[2 * r] = h2[0];
      p4[2 * r + 1] = h2[1];
      p4l[2 * r] = (_Float16)__builtin_fmaf(float(h2[0]), kNegOne, p[2 * r]);
      p4l[2 * r + 1] = (_Float16)__builtin_fmaf(float(h2[1]), kNegOne, p[2 * r + 1]);
    }
    // v = (m' - 2^b s') + (1 + c/2^b) 2^b s'.  The min term, 2^b times over:
    // sum_t 2^b p m' + sum_t 2^b p (-2^b s'), straight from the fp16 scales
    // (-2^b s' is exact; exact products; row = 32-channel group jr, rows >=
    // D/32 repeat and are not read).
    __builtin_amdgcn_s_setprio(1);
    {
      const int jr = hn & (D / 32 - 1);
      const f16x8 vm8 = vm[4 * jr + g], vn8 = vs[4 * jr + g] * (_Float16)(-kCodeScale);
      st.ob = mfma_f16(vm8, p4, st.ob);
      st.ob = mfma_f16(vm8, p4l, st.ob);
      st.ob = mfma_f16(vn8, p4, st.ob);
      st.ob = mfma_f16(vn8, p4l, st.ob);
    }
    // one B operand per pass: column group jc takes channel group
    // ps * RG + jc (the other groups' columns of st.o[nb] are not read)
#pragma unroll
    for (int ps = 0; ps < NPASS; ++ps) {
      const f16x8 sv = vs[4 * (ps * RG + jc % RG) + g];
      const f16x8 ph = p4 * sv;
      const f16x8 pl = __builtin_elementwise_fma(p4l, sv, __builtin_elementwise_fma(p4, sv, -ph));
#pragma unroll
      for (int nb = 2 * ps * RG; nb < 2 * (ps + 1) * RG; ++nb) {
        const f16x8 av = decode_chunk<BITS>(qq.vc, nb, kMaskR, kOneR);
        st.o[nb] = mfma_f16(av, ph, st.o[nb]);
        st.o[nb] = mfma_f16(av, pl, st.o[nb]);
      }
    }
    __builtin_amdgcn_s_setprio(0);
    if (rec_mass) rec[rt][hn] = make_float2(rs, st.m_run);
  };

  // The wave's first bf16 tile, in flight while INT2 tiles are decoded - but
  // not beside two 8-bit tiles, whose code words leave no room for it.
  constexpr bool kEarlyF = BITS != 8;
  FB FA;
  // ---------------------------------------------------------- INT2 tiles
  // two tiles in flight; a buffer is refilled as soon as its tile is consumed
  // (sched_barrier keeps the loads ahead of the next tile's math).  Instanced
  // with and without the early bf16 load so that the compiler counts the
  // loads in flight exactly on both paths.
  auto int2_tiles = [&](auto early_f) {
    int cb = q_beg, nt = max(0, min(q_end, cb + kList) - cb);
    QB A, Bq;
    load_q(A, 0, nt);
    load_q(Bq, 1, nt);
    __builtin_amdgcn_sched_barrier(0);
    make_q4();
    int i0 = 0;
    if constexpr (decltype(early_f)::value) {
      // The bf16 tile is requested once the first INT2 tile is in: all waves'
      // INT2 data is then served ahead of the (larger) bf16 data, which
      // arrives while INT2 tiles are decoded.  The first two tiles sit outside
      // the loop, where the compiler can count the loads in flight exactly
      // (every load here is unconditional); the loop's own count would make
      // its first wait include the bf16 tile.
      if (nt > 0) compute_q(A, 0, 0);
      load_q(A, 2, nt);
      __builtin_amdgcn_sched_barrier(0);
      load_f(FA, 0, min(f_end, f_beg + kList) - f_beg);
      __builtin_amdgcn_sched_barrier(0);
      if (nt > 1) compute_q(Bq, 1, 1);
      load_q(Bq, 3, nt);
      __builtin_amdgcn_sched_barrier(0);
      i0 = 2;
    }
    __builtin_amdgcn_sched_barrier(0);
    while (nt > 0) {
      for (int i = i0; i < nt; i += 2) {
        compute_q(A, i, i);
        if (i + 1 >= nt) break;
        load_q(A, i + 2, nt);
        __builtin_amdgcn_sched_barrier(0);
        compute_q(Bq, i + 1, i + 1);
        load_q(Bq, i + 3, nt);   // (empty past the end: one path back to the loop head)
        __builtin_amdgcn_sched_barrier(0);
      }
      drain_loads();   // the last (empty) prefetch: nothing pending into the next chunk
      flush_masses(nt, listq);
      cb += kList;
      nt = max(0, min(q_end, cb + kList) - cb);
      i0 = 0;
      if (nt > 0) {
        listq = s_tiles + NF + cb;
        load_q(A, 0, nt);
        load_q(Bq, 1, nt);
        __builtin_amdgcn_sched_barrier(0);
      }
    }
  };
  // Both tiers in one loop: a wave with a long INT2 list and some bf16 tiles
  // takes one bf16 tile after every K INT2 tiles, so that the bf16 bytes
  // stream in while INT2 tiles are decoded (an INT2 tile costs far more
  // instructions per byte than a bf16 tile); the bf16 tiles left over run in
  // the bf16 loop after it.  A wave's loads complete in the order they were
  // issued, so an INT2 tile requested behind a bf16 tile's 16 KB waits for
  // all of it: K = 8 was measured fastest at the 128K loop (against 4, 6, 12
  // and 16), K = 4 at the Mistral step, whose shares hold fewer INT2 tiles
  // per bf16 tile.  Two
  // INT2 tiles and one bf16 tile are in flight; every load is unconditional
  // (empty resources past the ends), so each tile waits only for its own
  // loads.  INT2 tiles record their masses from the top rows of the record
  // block, bf16 tiles from the bottom (both lists fit one chunk).
  int f_done = 0;   // bf16 tiles of the first chunk taken in the mixed loop
  auto mixed_tiles = [&](auto group) {
    constexpr int K = decltype(group)::value;   // INT2 tiles per bf16 tile
    const int nq = q_end - q_beg, nf = f_end - f_beg;
    QB A, Bq;
    load_q(A, 0, nq);
    __builtin_amdgcn_sched_barrier(0);
    load_q(Bq, 1, nq);
    __builtin_amdgcn_sched_barrier(0);
    load_f(FA, 0, nf);
    __builtin_amdgcn_sched_barrier(0);
    make_q4();
    // whole groups of K (the tiles past the end load nothing and are not
    // computed): the loop has no early exit, so every path into its head has
    // the same loads in flight in the same order
    int jf = 0;
    auto slot = [&](QB& qq, int i, int k) {
      if (k == 0 || i + k < nq) compute_q(qq, i + k, kList - 1 - k - i);
      load_q(qq, i + k + 2, nq);
      __builtin_amdgcn_sched_barrier(0);
    };
    for (int i = 0; i < nq; i += K) {
      slot(A, i, 0);
      slot(Bq, i, 1);
      slot(A, i, 2);
      slot(Bq, i, 3);
      if constexpr (K == 8) {
        slot(A, i, 4);
        slot(Bq, i, 5);
        slot(A, i, 6);
        slot(Bq, i, 7);
      }
      if (jf < nf) compute_f(FA, jf);
      ++jf;
      load_f(FA, jf, nf);   // (empty past the end)
      __builtin_amdgcn_sched_barrier(0);
    }
    drain_loads();   // FA (the next bf16 tile, if any) is in; nothing else pending
    flush_masses(nq, listq, true);
    f_done = min(jf, nf);
  };
  // A short share - at most three INT2 tiles and one bf16 tile, as at 32K
  // context: all of its INT2 tiles are requested right after the plan, its
  // bf16 tile once the first INT2 tile is in.  The INT2 decode sets the
  // critical path here: requested together, the bf16 bytes delayed the INT2
  // data by about a microsecond, while requested after the first INT2 tile
  // they arrive during the decode of the others.  Each tile waits only for
  // its own loads.
  // (4-bit code words are larger: two INT2-tier tiles there)
  constexpr int kShortQ = BITS == 2 ? 3 : 2;
  auto short_tiles = [&]() {
    const int nq = q_end - q_beg, nf = f_end - f_beg;
    QB A, Bq, C;
    load_q(A, 0, nq);
    load_q(Bq, 1, nq);
    if constexpr (kShortQ > 2) load_q(C, 2, nq);
    __builtin_amdgcn_sched_barrier(0);
    make_q4();
    if (nq > 0) compute_q(A, 0, 0);
    load_f(FA, 0, nf);
    __builtin_amdgcn_sched_barrier(0);
    if (nq > 1) compute_q(Bq, 1, 1);
    if constexpr (kShortQ > 2)
      if (nq > 2) compute_q(C, 2, 2);
    flush_masses(nq, listq);
    if (nf > 0) compute_f(FA, 0);
    flush_masses(nf, listf);
  };
  // (head groups of more than four need the registers of their wider B
  // operands: they keep the tiers apart)
  bool mixed = false, short_share = false;
  if constexpr (BITS == 2 || D == 64) {
    short_share = q_end - q_beg <= kShortQ && f_end - f_beg <= 1;
    if (short_share) short_tiles();
  }
  if constexpr (GP == 4 && BITS == 2) {
    const int nq_all = q_end - q_beg, nf_all = f_end - f_beg;
    mixed = !short_share && nq_all >= kMixedList && nq_all + nf_all <= kList;
    // one bf16 tile per eight INT2 tiles for INT2-heavy shares (the 128K loop,
    // about five INT2 tiles per bf16 tile), per four otherwise (the Mistral
    // step, about three: attention 48.3 -> 45.6 us by kernel trace)
    if (mixed) {
      if (nq_all > 4 * nf_all)
        mixed_tiles(std::integral_constant<int, 8>{});
      else
        mixed_tiles(std::integral_constant<int, 4>{});
    }
  }
  if (!mixed && !short_share) {
    if (f_beg < f_end && kEarlyF)
      int2_tiles(std::true_type{});
    else
      int2_tiles(std::false_type{});
  }

  // ---------------------------------------------------------- bf16 tiles
  for (int cb = short_share ? f_end : f_beg; cb < f_end; cb += kList) {
    const int ce = min(f_end, cb + kList), nt = ce - cb;
    const int i0 = cb == f_beg ? f_done : 0;   // FA holds tile i0 after the mixed loop
    listf = s_tiles + cb;
    if (cb != f_beg || !kEarlyF) load_f(FA, 0, nt);   // (else requested among the INT2 tiles)
    FB Bf;
    load_f(Bf, i0 + 1, nt);
    __builtin_amdgcn_sched_barrier(0);
    for (int i = i0; i < nt; i += 2) {
      compute_f(FA, i);
      if (i + 1 >= nt) break;
      load_f(FA, i + 2, nt);
      __builtin_amdgcn_sched_barrier(0);
      compute_f(Bf, i + 1);
      load_f(Bf, i + 3, nt);   // (empty past the end: one path back to the loop head)
      __builtin_amdgcn_sched_barrier(0);
    }
    drain_loads();
    flush_masses(nt, listf);
  }

  // ------------------------------------------- the appended token (VALU)
  // Taken after the tiles (the online softmax does not depend on the order of
  // tokens): a block ahead of the tile loops made every wave wait for its
  // query loads before requesting any tile.  (A wave-uniform branch.)
  if (uniform(app_ok)) {
    const uint16_t* kn = a.k_new + (size_t(b) * pv.Hkv + kvh) * D;
    const uint16_t* vn = a.v_new + (size_t(b) * pv.Hkv + kvh) * D;
    // the query again from memory (the one wave that takes this block): left
    // in qb, its conversions were hoisted ahead of the tile loads
    const auto rq = tile_rsrc(q_arg + (size_t(b) * hq_arg + size_t(kvh) * g_arg) * D, g_arg * D * 2);
    // the lane's byte offset into the query, formed here from an opaque copy
    // of the lane index: an offset shared with the first query load would be
    // kept across the tile loops, where registers run out (it was spilled)
    const int ln = int(opaque(uint32_t(lane)));
    const int hq2 = (ln & 15) % GP, g2 = ln >> 4;
    float zp = 0.f;
#pragma unroll
    for (int kk = 0; kk < KK; ++kk) {
      const bf16x8 kv = as_bf16x8(*reinterpret_cast<const uint4*>(kn + 32 * kk + 8 * g2));
      const bf16x8 qa = as_bf16x8(load16(rq, boff(hq2 < g_arg, (hq2 * D + 32 * kk + 8 * g2) * 2)));
#pragma unroll
      for (int e = 0; e < 8; ++e) zp = fmaf(float(qa[e]), float(kv[e]), zp);
    }
    zp = sum_rows(zp);
    // the token counts once: only lane group 0 carries it into the softmax;
    // its probability then reaches the other groups' output channels
    float z[8], p[8], rs;
    z[0] = g == 0 ? zp : -INFINITY;
#pragma unroll
    for (int e = 1; e < 8; ++e) z[e] = -INFINITY;
    softmax_tile<NB, 0>(st, z, qscale, 0.f, p, &rs);
    const float p0 = __shfl(p[0], hn, 64);
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) {
      const uint2 u = *reinterpret_cast<const uint2*>(vn + 16 * nb + 4 * g);
      st.o[nb][0] = fmaf(p0, __uint_as_float(u.x << 16), st.o[nb][0]);
      st.o[nb][1] = fmaf(p0, __uint_as_float(u.x & 0xFFFF0000u), st.o[nb][1]);
      st.o[nb][2] = fmaf(p0, __uint_as_float(u.y << 16), st.o[nb][2]);
      st.o[nb][3] = fmaf(p0, __uint_as_float(u.y & 0xFFFF0000u), st.o[nb][3]);
    }
    if (rec_mass) a.app_mass[size_t(b) * pv.Hq + size_t(kvh) * G + hn] = make_float2(rs, st.m_run);
  }
  // the step's append decision for the combine kernel, and its error bits
  if (split == 0 && wid == 0 && kvh == 0 && lane == 0) {
    int32_t* info = a.app_info + 8 * b;
    info[0] = app_ok;
    info[1] = app_slot;
    info[2] = app_row;
    info[3] = app_new;
    info[4] = len_old;
    if (app_err) set_err(pv.err, app_err);
  }

  // -------------------------------------------- combine the 4 waves in LDS
  // channels of block nb come from the column group that carried their
  // channel group's scales (any group for the min term, m and l)
  if (hh < G) {
#pragma unroll
    for (int nb = 0; nb < NB; ++nb)
      if (jc == (nb / 2) % RG) {
#pragma unroll
        for (int i4 = 0; i4 < 4; ++i4) s_wo[wid][hh][16 * nb + 4 * g + i4] = st.o[nb][i4];
      }
  }
  if (hn < G) {
    if (g == 0) {
      s_wm[wid][hn] = st.m_run;
      s_wl[wid][hn] = st.l_run;
#pragma unroll
      for (int i4 = 0; i4 < 4; ++i4) s_wb[wid][hn][i4] = st.ob[i4];
    }
  }
  __syncthreads();
  // partial of this workgroup: o [G][D]; (max, sum) of each head to ml
  float* part = a.partials + ((size_t(b) * pv.Hkv + kvh) * S + split) * G * D;
  for (int idx = tid; idx < G * D; idx += 256) {
    const int h = idx / D, d = idx - h * D;
    float M = -INFINITY;
#pragma unroll
    for (int v = 0; v < kAttnWaves; ++v) M = fmaxf(M, s_wm[v][h]);
    float acc = 0.f;
#pragma unroll
    for (int v = 0; v < kAttnWaves; ++v) {
      const float sc = s_wm[v][h] == -INFINITY ? 0.f : fast_exp2(s_wm[v][h] - M);
      acc += sc * fmaf(1.f / kCodeScale, s_wb[v][h][d >> 5], s_wo[v][h][d]);   // s_wb: 2^b x the min term
    }
    part[idx] = acc;
  }
  if (tid < G) {
    float M = -INFINITY;
#pragma unroll
    for (int v = 0; v < kAttnWaves; ++v) M = fmaxf(M, s_wm[v][tid]);
    float L = 0.f;
#pragma unroll
    for (int v = 0; v < kAttnWaves; ++v)
      L += s_wm[v][tid] == -INFINITY ? 0.f : fast_exp2(s_wm[v][tid] - M) * s_wl[v][tid];
    a.ml[(size_t(b) * pv.Hq + size_t(kvh) * G + tid) * S + split] = make_float2(M, L);
  }
}

// --------------------------------------------------------------------------
// Combine.  Blocks x < Hkv * (D / 32) produce 32 output channels of every
// query head of kv head x / (D / 32) (the first block of a kv head also stores
// an appended token's K/V); blocks beyond normalise the window masses of 32
// windows for every query head, optionally adding them to the cumulative
// scores.  Every block issues all of its loads before its first barrier.

// x combined over the 32 lanes of its half-wave: DPP within each 16-lane row
// (xor 1, xor 2, half-row mirror, row mirror), then the row pair.
template <typename Op>
__device__ inline float half_reduce(float x, Op op) {
  x = op(x, __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0xB1, 0xF, 0xF, false)));
  x = op(x, __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x4E, 0xF, 0xF, false)));
  x = op(x, __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x141, 0xF, 0xF, false)));
  x = op(x, __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x140, 0xF, 0xF, false)));
  auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return op(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
// Max and normaliser of one query head over the splits: lane c of a 32-lane
// half-wave takes splits c and c + 32 (raw m, l pairs of the workgroups).
// (The output blocks use it: 4 - 8 rows of 32 lanes reduce their heads at once.)
__device__ inline float2 head_mz(float m0, float l0, float m1, float l1) {
  const float M = half_reduce(fmaxf(m0, m1), [](float u, float v) { return fmaxf(u, v); });
  float z = 0.f;
  if (m0 != -INFINITY) z = l0 * fast_exp2(m0 - M);
  if (m1 != -INFINITY) z = fmaf(l1, fast_exp2(m1 - M), z);
  z = half_reduce(z, [](float u, float v) { return u + v; });
  return make_float2(M, z);
}
// x combined over the 8 lanes of its group (DPP xor 1, xor 2, half-row mirror)
template <typename Op>
__device__ inline float oct_reduce(float x, Op op) {
  x = op(x, __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0xB1, 0xF, 0xF, false)));
  x = op(x, __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x4E, 0xF, 0xF, false)));
  return op(x, __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x141, 0xF, 0xF, false)));
}



// SL: channels of one output block (32, or the whole head when the splits
// are few: a thread then reduces at most kMaxSplits / 4 = 16 splits of its
// item, which covers them).
template <int D, int SL>
__global__ __launch_bounds__(256) void combine_kernel(PoolView pv, AttnArgs a, int acc_scores, int mass_lg) {
  constexpr int kSlice = SL, NO = D / kSlice;
  __shared__ float s_m[kMaxSplits * kGMax];
  __shared__ float s_hm[kGMax], s_hz[kGMax];
  __shared__ float4 s_acc[256];
  __shared__ int s_win[kMassWindows];
  extern __shared__ float s_dynf[];   // mass blocks: M, 1/Z [Hq], masses [mw][Hq], appended [Hq]
  const int b = blockIdx.y, x = blockIdx.x, tid = threadIdx.x;
  // Every kernel argument that either kind of block reads is fetched in one
  // batch here: left to itself, the compiler requests a branch's arguments
  // only once the branch is taken, a dependent round trip each.
  uint16_t* const bf16_p = pv.bf16;
  uint32_t* const pages_p = pv.pages;
  float* const scores_p = pv.scores;
  int32_t* const tokens_p = pv.tokens;
  const float* const part_p = a.partials;
  const float2* const ml_p = a.ml;
  float* const out_p = a.out;
  const uint16_t* const kn_p = a.k_new;
  const uint16_t* const vn_p = a.v_new;
  const int32_t* const info_p = a.app_info;
  const float2* const tm_p = a.tile_mass;
  const float2* const am_p = a.app_mass;
  float* const mass_p = a.mass;
  const int G = pv.G, Hkv = pv.Hkv, Hq = pv.Hq, S = a.splits, W = pv.W, maxw = pv.maxw, nb = pv.nb;
  const int layer = a.layer, B = pv.B;
  in_sgprs(bf16_p, pages_p, scores_p, tokens_p, part_p, ml_p, out_p, kn_p, vn_p, info_p, tm_p, am_p, mass_p);
  in_sgprs(G, Hkv, Hq, S, W, maxw, nb, layer, B, acc_scores);
  const int TPW = W / 32, seg = layer * B + b;
  const int32_t* info = info_p + 8 * b;
  // the step's append decision (app, slot, row, new window, tokens before),
  // read as vector loads among each block's other loads
  const auto rinfo = tile_rsrc(info, 5 * 4);

  if (x < Hkv * NO) {
    // -------------------------------------------------------- output slice
    const int kvh = x / NO, sl = x % NO;
    const auto rp = tile_rsrc(part_p + (size_t(b) * Hkv + kvh) * S * G * D, S * G * D * 4);
    const auto rml = tile_rsrc(ml_p + (size_t(b) * Hq + size_t(kvh) * G) * S, G * S * 8);
    const int items = G * (kSlice / 4);   // (head, 4 channels)
    const int groups = 256 / items;       // split groups, >= 4
    const int it = tid % items, grp = tid / items;
    const int h = it / (kSlice / 4);
    const int d = sl * kSlice + 4 * (it % (kSlice / 4));
    const bool act = grp < groups;
    constexpr int kPer = kMaxSplits / 4;
    float4 v4[kPer];
#pragma unroll
    for (int j = 0; j < kPer; ++j) {
      const int sp = grp + j * groups;
      const uint4 u = load16(rp, boff(act && sp < S, ((sp * G + h) * D + d) * 4));
      v4[j] = make_float4(__uint_as_float(u.x), __uint_as_float(u.y), __uint_as_float(u.z), __uint_as_float(u.w));
    }
    const int c32 = tid & 31, r8 = tid >> 5;   // (split lane, row of 32 threads)
    // row r8 (< G) reduces head r8: splits c32 and c32 + 32
    const bool v0 = r8 < G && c32 < S, v1 = r8 < G && c32 + 32 < S;
    const float2 u0 = as_f2(load8(rml, boff(v0, (r8 * S + c32) * 8)));
    const float2 u1 = as_f2(load8(rml, boff(v1, (r8 * S + c32 + 32) * 8)));
    const uint4 inf4 = load16(rinfo, 0);   // needed only at the end
    const uint32_t i4 = load4(rinfo, 16);
    const float m0 = v0 ? u0.x : -INFINITY, l0 = u0.y, m1 = v1 ? u1.x : -INFINITY, l1 = u1.y;
    if (v0) s_m[c32 * G + r8] = m0;
    if (v1) s_m[(c32 + 32) * G + r8] = m1;
    const float2 mz = head_mz(m0, l0, m1, l1);
    if (r8 < G && c32 == 0) {
      s_hm[r8] = mz.x;
      s_hz[r8] = mz.y;
    }
    __syncthreads();
    const float M = s_hm[h];
    float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
    for (int j = 0; j < kPer; ++j) {
      const int sp = grp + j * groups;
      if (act && sp < S) {
        const float ms = s_m[sp * G + h];
        const float sc = ms == -INFINITY ? 0.f : fast_exp2(ms - M);
        acc.x = fmaf(sc, v4[j].x, acc.x);
        acc.y = fmaf(sc, v4[j].y, acc.y);
        acc.z = fmaf(sc, v4[j].z, acc.z);
        acc.w = fmaf(sc, v4[j].w, acc.w);
      }
    }
    if (act) s_acc[tid] = acc;
    // the append decision is read here, ahead of the output store: the memory
    // counter is in order, so a read of it after the store would wait for the
    // store's completion
    const int app = uniform(int(inf4.x)), slot = uniform(int(inf4.y)), row = uniform(int(inf4.z));
    const int newwin = uniform(int(inf4.w)), len_old = uniform(int(i4));
    __syncthreads();
    if (tid < items) {
      float4 t4 = s_acc[tid];
      for (int q2 = 1; q2 < groups; ++q2) {
        const float4 u = s_acc[q2 * items + tid];
        t4.x += u.x; t4.y += u.y; t4.z += u.z; t4.w += u.w;
      }
      const float Z = s_hz[h], iz = Z > 0.f ? 1.f / Z : 0.f;
      *reinterpret_cast<float4*>(out_p + (size_t(b) * Hq + size_t(kvh) * G + h) * D + d) =
          make_float4(t4.x * iz, t4.y * iz, t4.z * iz, t4.w * iz);
    }
    if (app && sl == 0) {
      // the appended token joins its window (no kernel of this step reads it)
      const int len = len_old + 1;
      const int n_old = windows_of(len_old, W);
      uint16_t* dst = bf16_p + ((size_t(seg) * nb + slot) * Hkv + kvh) * size_t(2 * W * D);
      for (int dd = tid; dd < D; dd += 256) {
        // both values loaded before either store (a load after a store would
        // wait for the store's completion)
        const uint16_t kv = kn_p[(size_t(b) * Hkv + kvh) * D + dd];
        const uint16_t vv = vn_p[(size_t(b) * Hkv + kvh) * D + dd];
        dst[layout::bf16_window_k(row, dd, D)] = kv;
        dst[layout::bf16_window_v(row, dd, D)] = vv;
      }
      if (kvh == 0 && tid == 0) {
        if (newwin) pages_p[size_t(seg) * maxw + n_old] = pe_make(TIER_F, false, slot, 0);
        tokens_p[seg] = len;
      }
    }
    return;
  }

  // ---------------------------------------------------------- window masses
  if (!mass_p && !acc_scores) return;
  const int mw = 1 << mass_lg;   // windows per mass block: 8 or 16
  const int w0 = (x - Hkv * NO) * mw;
  if (w0 >= maxw) return;
  float* s_M = s_dynf;             // [Hq]
  float* s_Zh = s_dynf + Hq;       // [Hq] 1 / normaliser
  float* s_mv = s_dynf + 2 * Hq;   // [mw][Hq]
  float2* s_app = reinterpret_cast<float2*>(s_dynf + (2 + mw) * Hq);   // [Hq]
  // thread pairs (head h, window wl), heads fastest: pair p = tid + 256 i has
  // h = p % Hq, wl = p / Hq, and the records of one tile of all heads are
  // contiguous
  constexpr int kPairs = 4, kTiles = 8;   // pairs per batch; tiles per window at most
  const int npairs = Hq * mw;
  const int bpairs = min(kPairs, (npairs + 255) / 256);   // pairs of a thread in one batch
  const auto rtm = tile_rsrc(tm_p + size_t(b) * maxw * TPW * Hq, maxw * TPW * Hq * 8);
  const auto rml = tile_rsrc(ml_p + size_t(b) * Hq * S, Hq * S * 8);
  const auto rpg = tile_rsrc(pages_p + size_t(seg) * maxw, maxw * 4);
  const auto rsc = tile_rsrc(scores_p + size_t(seg) * maxw, maxw * 4);
  auto tile_masses = [&](int p0, float2 (&t)[kPairs][kTiles]) {
#pragma unroll
    for (int i = 0; i < kPairs; ++i) {
      if (i >= bpairs) break;   // uniform: no load instruction for pairs the block does not have
      const int pi = p0 + tid + 256 * i, h = pi % Hq, w = w0 + pi / Hq;
#pragma unroll
      for (int k = 0; k < kTiles; ++k) {
        if (k >= TPW) break;    // uniform: only the tiles a window has
        t[i][k] = as_f2(load8(rtm, boff(pi < npairs && w < maxw, ((w * TPW + k) * Hq + h) * 8)));
      }
    }
  };
  // One round of loads, all in flight together: the append info, the tile
  // masses, the page entries and scores of the block's windows, the appended
  // token's records and the (m, l) pairs of the per-head reductions.  Nothing
  // waits for the append info: entries past the window count are loaded too
  // and ignored.
  const uint4 inf4 = load16(rinfo, 0);
  const uint32_t i4 = load4(rinfo, 16);
  float2 t1[kPairs][kTiles];
  tile_masses(0, t1);
  const int wt = w0 + tid;   // thread tid < mw: its window's page entry and score
  const bool tw = tid < mw && wt < maxw;
  const uint32_t pe = load4(rpg, boff(tw, wt * 4));
  const float s_old = __uint_as_float(load4(rsc, boff(acc_scores && tw, wt * 4)));
  const auto rap = tile_rsrc(am_p + size_t(b) * Hq, Hq * 8);
  const float2 appm = as_f2(load8(rap, boff(tid < Hq, tid * 8)));
  // max and 1 / normaliser of every query head over the splits: 8 lanes per
  // head, lane c8 taking splits c8, c8 + 8, ... (S <= 64), 32 heads a pass
  {
    const int c8 = tid & 7, hr = tid >> 3;
    for (int h0 = 0; h0 < Hq; h0 += 32) {
      const int h = h0 + hr;
      float2 v[kMaxSplits / 8];
#pragma unroll
      for (int j = 0; j < kMaxSplits / 8; ++j) {
        const int sp = c8 + 8 * j;
        const bool ok = h < Hq && sp < S;
        v[j] = as_f2(load8(rml, boff(ok, (h * S + sp) * 8)));
        if (!ok) v[j].x = -INFINITY;
      }
      float m = v[0].x;
#pragma unroll
      for (int j = 1; j < kMaxSplits / 8; ++j) m = fmaxf(m, v[j].x);
      m = oct_reduce(m, [](float u, float w) { return fmaxf(u, w); });
      float z = 0.f;
#pragma unroll
      for (int j = 0; j < kMaxSplits / 8; ++j)
        if (v[j].x != -INFINITY) z = fmaf(v[j].y, fast_exp2(v[j].x - m), z);
      z = oct_reduce(z, [](float u, float w) { return u + w; });
      if (c8 == 0 && h < Hq) {
        s_M[h] = m;
        s_Zh[h] = z > 0.f ? 1.f / z : 0.f;   // reciprocal of the normaliser
      }
    }
  }
  const int app = uniform(int(inf4.x)), len_old = uniform(int(i4));
  const int len = len_old + (app ? 1 : 0);
  const int n_old = windows_of(len_old, W), n_win = windows_of(len, W);
  const bool tin = tid < mw && wt < n_win;
  if (app) {
    if (tid < Hq) s_app[tid] = appm;
    for (int h = tid + 256; h < Hq; h += 256) s_app[h] = as_f2(load8(rap, h * 8));
  }
  // liveness and valid tiles of the block's windows
  if (tid < mw) {
    bool live = false;
    int vt = 0;
    if (tin) {
      if (wt < n_old) {
        live = pe_tier(pe) != TIER_E;
        vt = (min(W, len_old - wt * W) + 31) / 32;
      } else {
        live = true;   // the window the appended token opened
      }
    }
    s_win[tid] = live ? vt + 1 : 0;   // 0: not live; else 1 + valid tiles
  }
  __syncthreads();
  const int vwin = app ? len_old / W : -1;
  auto masses = [&](int p0, const float2 (&t)[kPairs][kTiles]) {
#pragma unroll
    for (int i = 0; i < kPairs; ++i) {
      const int pi = p0 + tid + 256 * i, h = pi % Hq, wl = pi / Hq;
      if (pi >= npairs) break;
      const int lw = s_win[wl];
      const int vt = lw - 1;
      const float M = s_M[h];
      float acc = 0.f;
#pragma unroll
      for (int k = 0; k < kTiles; ++k) {
        if (k >= TPW) break;
        if (k < vt) acc += t[i][k].x * fast_exp2(t[i][k].y - M);
      }
      if (w0 + wl == vwin) acc += s_app[h].x * fast_exp2(s_app[h].y - M);
      s_mv[wl * Hq + h] = lw ? acc * s_Zh[h] : 0.f;
    }
  };
  masses(0, t1);
  for (int p0 = 256 * kPairs; p0 < npairs; p0 += 256 * kPairs) {
    float2 t2[kPairs][kTiles];
    tile_masses(p0, t2);
    masses(p0, t2);
  }
  // the old score is taken into its register here, ahead of the mass stores:
  // the memory counter is in order, so waiting for it after the stores would
  // wait for their completion (an empty asm statement that reads the register)
  asm volatile("" ::"v"(s_old));
  __syncthreads();
  // masses out in window order (the block's mw consecutive windows per head)
  if (mass_p) {
    for (int idx = tid; idx < npairs; idx += 256) {
      const int h = idx >> mass_lg, ww = idx & (mw - 1);
      if (w0 + ww < n_win) mass_p[(size_t(b) * Hq + h) * maxw + w0 + ww] = s_mv[ww * Hq + h];
    }
  }
  if (acc_scores && tin && s_win[tid]) {
    float ssum = 0.f;
    for (int h = 0; h < Hq; ++h) ssum += s_mv[tid * Hq + h];   // heads in order
    scores_p[size_t(seg) * maxw + wt] = s_old + ssum;
  }
}

template <int D, int GP, int BITS>
static hipError_t launch_attn_kernel(const PoolView& pv, const AttnArgs& a, size_t shm, hipStream_t s) {
  const uint32_t* pl = pv.pages + size_t(a.layer) * pv.B * pv.maxw;
  const int32_t* tl = pv.tokens + size_t(a.layer) * pv.B;
  if (a.ev_start || a.ev_stop) {
    hipExtLaunchKernelGGL((attn_kernel<D, GP, BITS>), dim3(a.splits, pv.Hkv, pv.B), dim3(256), uint32_t(shm), s,
                          a.ev_start, a.ev_stop, 0u, pl, tl, pv.maxw, a.q, pv.Hq, pv.G, pv, a);
  } else {
    hipLaunchKernelGGL((attn_kernel<D, GP, BITS>), dim3(a.splits, pv.Hkv, pv.B), dim3(256), shm, s, pl, tl, pv.maxw,
                       a.q, pv.Hq, pv.G, pv, a);
  }
  return hipGetLastError();
}

template <int D>
static hipError_t launch_attn_t(const PoolView& pv, const AttnArgs& a, hipStream_t s) {
  const size_t shm = (2 * size_t(a.plan_words) + size_t(pv.maxw) * (pv.W / 32) + (pv.nb + 31) / 32) * 4;
  hipError_t e;
  if (pv.lbits == 2)
    e = pv.G <= 4 ? launch_attn_kernel<D, 4, 2>(pv, a, shm, s) : launch_attn_kernel<D, 8, 2>(pv, a, shm, s);
  else if (pv.lbits == 4)
    e = pv.G <= 4 ? launch_attn_kernel<D, 4, 4>(pv, a, shm, s) : launch_attn_kernel<D, 8, 4>(pv, a, shm, s);
  else
    e = pv.G <= 4 ? launch_attn_kernel<D, 4, 8>(pv, a, shm, s) : launch_attn_kernel<D, 8, 8>(pv, a, shm, s);
  if (e != hipSuccess) return e;
  // Mass blocks of 16 windows; of 8 when that makes at most 64 blocks in all
  // (a short launch, where more blocks with half the pairs each end sooner:
  // 32K step 18.2 -> 17.8 us; with more blocks the redundant per-block head
  // reductions cost more than they save).
  const int mb16 = (pv.maxw + kMassWindows - 1) / kMassWindows;
  const int mass_lg = pv.B * mb16 <= 64 ? 3 : 4;
  const int mw = 1 << mass_lg;
  const int mass_blocks = (a.mass || a.acc_scores) ? (pv.maxw + mw - 1) / mw : 0;
  // Output blocks: one per kv head when there are at most 8 splits (the
  // Mistral-7B step, 2 splits: the combine 8.5 -> 6.1 us; at 16 splits the
  // Qwen2.5-7B step gained nothing), else one per 32-channel slice, so a
  // thread's share of a many-split reduction stays short.
  const size_t cshm = size_t(4 + mw) * pv.Hq * 4;
  if (a.splits <= 8)
    hipLaunchKernelGGL((combine_kernel<D, D>), dim3(pv.Hkv + mass_blocks, pv.B), dim3(256), cshm, s, pv, a,
                       a.acc_scores, mass_lg);
  else
    hipLaunchKernelGGL((combine_kernel<D, 32>), dim3(pv.Hkv * (D / 32) + mass_blocks, pv.B), dim3(256), cshm, s,
                       pv, a, a.acc_scores, mass_lg);
  return hipGetLastError();
}

hipError_t launch_attn(const PoolView& pv, const AttnArgs& a, hipStream_t s) {
  if (pv.G > kGMax) return hipErrorInvalidValue;
  if (pv.D == 64) return launch_attn_t<64>(pv, a, s);
  if (pv.D == 128) return launch_attn_t<128>(pv, a, s);
  return hipErrorInvalidValue;
}

}  // namespace kvtier
