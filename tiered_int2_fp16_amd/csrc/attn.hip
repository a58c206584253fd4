// Tiered decode attention with per-window mass for gfx950 (matrix cores).
//
// QEvict technical summary ("Methodologie: QEvict", "Kernmechanismen",
// "Implementatie"): bf16 windows and INT2 windows both take part in attention,
// evicted windows do not; grouped-query attention; the attention each window
// receives is what the cumulative score adds up.  Unlike the summary's
// FlashAttention-2 path, which dequantises and rebuilds caches before attention
// ("Resultaten", efficiency), INT2 tiles are decoded in registers inside this
// kernel: HBM carries 3 bits per INT2 value, never a rebuilt bf16 copy.
//
// Work split: grid (splits, kv heads, sequences), 4 wave64 per workgroup.  The
// live 32-token tiles of a (sequence, kv head) are listed bf16 first, then
// INT2, weighted 16 (bf16, 16 KB) and kWq (INT2, 3 KB) and the weight range is
// cut evenly over all waves of all splits.  A wave streams its bf16 tiles and
// then its INT2 tiles, each loop double-buffered in registers, and keeps an
// online softmax (running max, sum, output) for the G query heads of its kv
// head; every tile's raw mass is recorded with the running max it was taken
// at.  A second kernel combines the partials of each (sequence, kv head) into
// the output and normalises the window masses (the order of tokens does not
// matter: A.V = A_P.V_P, LogQuant summary, "Positie-agnostische optimalisatie").
// Splitting the combine off keeps every workgroup of the first kernel free of
// device-wide fences and atomics; the kernel boundary orders the two.
//
// One tile = 16x16x32 MFMAs with the token/dim placement of layout.h:
//  bf16: S = K.q^T (bf16 inputs, exact products) then O^T += V^T.P^T with P
//        split into bf16 high and low parts (2^-17 relative error).
//  INT2: a code c becomes the fp16 value 1 + c/4 (two bit operations per pair
//        of codes).  With per-channel K scale s and min m,
//          q.k = sum_d (1 + c/4)(4 s q) + sum_d q (m - 4 s);
//        4 s q is exact in fp32 and goes to the MFMA as fp16 high + low parts,
//        the second sum (constant over the tile's tokens) is taken in fp32 -
//        an fp16 rounding of either would shift a whole tile's logits at once.
//        Both are computed once per (head, channel) in a compact lane layout
//        and handed to the MFMA layout through the wave's LDS buffer.  With
//        per-token V scale s' and min m',
//          sum_t p v = sum_t (1 + c/4)(4 p s') + sum_t (m'/4 - s')(4 p):
//        one MFMA per 16 channels for the codes, one for the min term.  The
//        tile's scales reach the lanes that need them through the same LDS
//        buffer.
//
// A decode step may append a token: it is attended straight from k_new/v_new
// and stored in the newest window by the combine kernel, which also rewrites
// the page table entry and token count - after every attention workgroup has
// read them.
#include <hip/hip_ext.h>
#include <math.h>

#include "host_core.h"
#include "launch.h"
#include "layout.h"

namespace kvtier {

namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int kGMax = 8;     // query heads per kv head supported
constexpr int kWq = 5;       // weight of an INT2 tile (a bf16 tile weighs 16)
constexpr int kMaxSplits = 64;
constexpr int kMassWindows = 64;   // windows per mass block of the combine kernel

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

__device__ inline f32x4 mfma_bf16(bf16x8 a, bf16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}
__device__ inline f32x4 mfma_f16(f16x8 a, f16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
}

// Exclusive scan of one int per thread over a 256-thread block.
__device__ inline int block_excl_scan(int v, int* tmp, int* total) {
  const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
  int x = v;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const int y = __shfl_up(x, off, 64);
    if (lane >= off) x += y;
  }
  if (lane == 63) tmp[wid] = x;
  __syncthreads();
  int base = 0;
  for (int i = 0; i < wid; ++i) base += tmp[i];
  *total = tmp[0] + tmp[1] + tmp[2] + tmp[3];
  __syncthreads();
  return base + x - v;
}

// Eight INT2 codes of one operand chunk -> fp16 (1 + c/4).  Word X holds the
// fields of chunks 2w (SEL 0) and 2w+1 (SEL 1); register j takes the fields
// j + 4*SEL (low half) and j + 4*SEL + 8 (high half), 16 bits apart.
template <int SEL>
__device__ inline f16x8 decode_codes(uint32_t X) {
  uint32_t r[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int sh = 2 * (j + 4 * SEL);
    const uint32_t y = sh <= 8 ? (X << (8 - sh)) : (X >> (sh - 8));
    r[j] = (y & 0x03000300u) | 0x3C003C00u;
  }
  return __builtin_bit_cast(f16x8, make_uint4(r[0], r[1], r[2], r[3]));
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
  f32x4 o[NB];   // O^T block nb: lane (g, n) holds head n, channels 16nb + 4g + i
  f32x4 ob;      // INT2 V min term: lane (0, n) holds head n, channel group i
};

template <int NB>
__device__ inline void softmax_tile(WaveState<NB>& st, const float (&z)[8], float (&p)[8], float* rs_out) {
  float tm = z[0];
#pragma unroll
  for (int e = 1; e < 8; ++e) tm = fmaxf(tm, z[e]);
  tm = max_rows(tm);
  const float mn = fmaxf(st.m_run, tm);
  const float alpha = fast_exp2(st.m_run - mn);
  float rs = 0.f;
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    p[e] = fast_exp2(z[e] - mn);
    rs += p[e];
  }
  rs = sum_rows(rs);
  st.l_run = st.l_run * alpha + rs;
  st.m_run = mn;
  if (__builtin_amdgcn_ballot_w64(alpha != 1.f)) {
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) st.o[nb] *= alpha;
    st.ob *= alpha;
  }
  *rs_out = rs;
}

}  // namespace

template <int D>
__global__ __launch_bounds__(256, 2) void attn_kernel(PoolView pv, AttnArgs a) {
  constexpr int KK = D / 32;   // 32-dim slices of the QK product
  constexpr int NB = D / 16;   // 16-channel blocks of the PV product (= code chunks per part)
  constexpr int CW = D / 32;   // 32-bit code words per lane per part
  constexpr int kList = 64;    // tile entries a wave lists at a time
  constexpr int kQGroup = 4;   // INT2 tiles loaded together
  extern __shared__ uint32_t s_used[];   // [(nb + 31) / 32] bf16 slot bitmap (append only)
  __shared__ float s_wm[kAttnWaves][kGMax], s_wl[kAttnWaves][kGMax];
  __shared__ float s_wo[kAttnWaves][kGMax][D];
  __shared__ float s_wb[kAttnWaves][kGMax][4];
  __shared__ __attribute__((aligned(16))) uint8_t s_scb[kAttnWaves][8 * D];  // INT2 tile scales
  __shared__ __attribute__((aligned(16))) _Float16 s_bq[kAttnWaves][2][kGMax * D];  // 4sq hi, lo
  __shared__ float s_cst[kAttnWaves][kGMax];                                   // tile constants
  __shared__ uint32_t s_list[kAttnWaves][kList];                               // a wave's tiles

  const int split = blockIdx.x, kvh = blockIdx.y, b = blockIdx.z;
  const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
  const int g = lane >> 4, hn = lane & 15;   // lane = (column block g, head hn)
  const int W = pv.W, maxw = pv.maxw, TPW = W / 32, G = pv.G;
  const int seg = a.layer * pv.B + b;
  const int S = a.splits;

  // ------------------------------------------------------------ the query
  // issued first: it does not depend on the plan
  constexpr float kLog2e = 1.4426950408889634f;
  const float qscale = kLog2e / sqrtf(float(D));
  bf16x8 qb[KK];    // q (bf16) for the bf16 tiles
  constexpr int kRounds = (kGMax * (D / 8) + 63) / 64;
  f16x8 qc[kRounds];  // 4*q in the compact (head, 8-channel chunk) layout
  {
    const uint16_t* qp = a.q + (size_t(b) * pv.Hq + size_t(kvh) * G + hn) * D + 8 * g;
#pragma unroll
    for (int kk = 0; kk < KK; ++kk) {
      uint4 u = make_uint4(0, 0, 0, 0);
      if (hn < G) u = *reinterpret_cast<const uint4*>(qp + 32 * kk);
      qb[kk] = as_bf16x8(u);
    }
#pragma unroll
    for (int r = 0; r < kRounds; ++r) {
      const int it = 64 * r + lane, h = it / (D / 8), c8 = it % (D / 8);
      uint4 u = make_uint4(0, 0, 0, 0);
      if (h < G) u = *reinterpret_cast<const uint4*>(a.q + (size_t(b) * pv.Hq + size_t(kvh) * G + h) * D + 8 * c8);
      const uint32_t w4[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        qc[r][2 * e] = (_Float16)(4.f * __uint_as_float(w4[e] << 16));
        qc[r][2 * e + 1] = (_Float16)(4.f * __uint_as_float(w4[e] & 0xFFFF0000u));
      }
    }
  }

  // ------------------------------------------------ wave-local tile plan
  // Every wave reads the page table and prefix-sums the live tiles itself
  // (bf16 tiles in the low 16 bits, INT2 tiles in the high 16 bits): no
  // workgroup barrier before the first tile load.
  const int len_old = pv.tokens[seg];
  const int n_old = windows_of(len_old, W);
  const uint32_t* gp = pv.pages + size_t(seg) * maxw;
  const int per = (n_old + 63) / 64;
  const int wl0 = min(n_old, lane * per), wl1 = min(n_old, wl0 + per);
  int cnt = 0;
  for (int w = wl0; w < wl1; ++w) {
    const int t = pe_tier(gp[w]);
    const int vt = (min(W, len_old - w * W) + 31) / 32;
    cnt += t == TIER_F ? vt : (t == TIER_Q ? (vt << 16) : 0);
  }
  int incl = cnt;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const int y = __shfl_up(incl, off, 64);
    if (lane >= off) incl += y;
  }
  const int tot = uniform(__shfl(incl, 63, 64));
  const int NF = tot & 0xFFFF, NQ = tot >> 16;
  const int excl = incl - cnt;
  const long U = 16L * NF + long(kWq) * NQ;
  const long nwaves = long(S) * kAttnWaves;
  const long widx = long(split) * kAttnWaves + wid;
  const long u0 = widx * U / nwaves, u1 = (widx + 1) * U / nwaves;
  auto cdiv = [](long x, long y) { return x <= 0 ? 0L : (x + y - 1) / y; };
  const int f_beg = int(min(long(NF), cdiv(u0, 16))), f_end = int(min(long(NF), cdiv(u1, 16)));
  const int q_beg = int(min(long(NQ), cdiv(u0 - 16L * NF, kWq)));
  const int q_end = int(min(long(NQ), cdiv(u1 - 16L * NF, kWq)));
  uint32_t* list = s_list[wid];
  // lanes write the entries of tiles [lo, hi) of tier `tier` that sit in their windows
  auto build_list = [&](int tier, int lo, int hi) {
    int ti = tier == TIER_F ? (excl & 0xFFFF) : (excl >> 16);
    for (int w = wl0; w < wl1 && ti < hi; ++w) {
      const uint32_t e = gp[w];
      if (pe_tier(e) != tier) continue;
      const int vt = (min(W, len_old - w * W) + 31) / 32;
      const int sl = tier == TIER_F ? pe_bslot(e) : pe_lslot(e);
      for (int k = 0; k < vt; ++k, ++ti)
        if (ti >= lo && ti < hi) list[ti - lo] = te_make(sl, w, k);
    }
  };

  // ------------------------------------------------- the append decision
  // Taken by wave 0 of split 0 of each (sequence, kv head); the combine kernel
  // stores the token and rewrites the page table after every workgroup read it.
  int app_ok = 0, app_slot = 0, app_row = 0, app_new = 0;
  if (a.k_new != nullptr && split == 0 && wid == 0) {
    if (len_old % W != 0) {
      const uint32_t e = gp[n_old - 1];
      app_ok = pe_tier(e) == TIER_F;
      app_slot = pe_bslot(e);
      app_row = len_old % W;
      if (!app_ok && kvh == 0 && lane == 0) set_err(pv.err, KV_ERR_APPEND_STATE);
    } else {
      // a new window opens: the lowest bf16 slot no live bf16 window holds
      const int words = (pv.nb + 31) / 32;
      for (int i = lane; i < words; i += 64) s_used[i] = 0u;
      for (int w = lane; w < n_old; w += 64) {
        const uint32_t e = gp[w];
        if (pe_tier(e) == TIER_F && pe_bslot(e) < pv.nb)
          atomicOr(&s_used[pe_bslot(e) >> 5], 1u << (pe_bslot(e) & 31));
      }
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
      if (!app_ok && kvh == 0 && lane == 0) set_err(pv.err, cap ? KV_ERR_NO_BF16_SLOT : KV_ERR_CAPACITY);
    }
    if (kvh == 0 && lane == 0) {
      int32_t* info = a.app_info + 8 * b;
      info[0] = app_ok;
      info[1] = app_slot;
      info[2] = app_row;
      info[3] = app_new;
      info[4] = len_old;
    }
  }
  if (a.k_new == nullptr && split == 0 && kvh == 0 && tid == 0) {
    int32_t* info = a.app_info + 8 * b;
    info[0] = 0;
    info[4] = len_old;
  }

  WaveState<NB> st;
  st.m_run = -INFINITY;
  st.l_run = 0.f;
#pragma unroll
  for (int nb = 0; nb < NB; ++nb) st.o[nb] = f32x4{0.f, 0.f, 0.f, 0.f};
  st.ob = f32x4{0.f, 0.f, 0.f, 0.f};
  float2* tmass = reinterpret_cast<float2*>(a.tile_mass) +
                  (size_t(b) * pv.Hkv + kvh) * (size_t(maxw) * TPW + 1) * G;
  const bool rec_mass = a.mass != nullptr && g == 0 && hn < G;

  // ------------------------------------------- the appended token (VALU)
  if (app_ok) {
    const uint16_t* kn = a.k_new + (size_t(b) * pv.Hkv + kvh) * D;
    const uint16_t* vn = a.v_new + (size_t(b) * pv.Hkv + kvh) * D;
    float zp = 0.f;
#pragma unroll
    for (int kk = 0; kk < KK; ++kk) {
      const bf16x8 kv = as_bf16x8(*reinterpret_cast<const uint4*>(kn + 32 * kk + 8 * g));
#pragma unroll
      for (int e = 0; e < 8; ++e) zp = fmaf(float(qb[kk][e]), float(kv[e]), zp);
    }
    zp = sum_rows(zp);
    // the token counts once: only lane group 0 carries it into the softmax;
    // its probability then reaches the other groups' output channels
    float z[8], p[8], rs;
    z[0] = g == 0 ? zp * qscale : -INFINITY;
#pragma unroll
    for (int e = 1; e < 8; ++e) z[e] = -INFINITY;
    softmax_tile<NB>(st, z, p, &rs);
    const float p0 = __shfl(p[0], hn, 64);
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) {
      const uint2 u = *reinterpret_cast<const uint2*>(vn + 16 * nb + 4 * g);
      st.o[nb][0] = fmaf(p0, __uint_as_float(u.x << 16), st.o[nb][0]);
      st.o[nb][1] = fmaf(p0, __uint_as_float(u.x & 0xFFFF0000u), st.o[nb][1]);
      st.o[nb][2] = fmaf(p0, __uint_as_float(u.y << 16), st.o[nb][2]);
      st.o[nb][3] = fmaf(p0, __uint_as_float(u.y & 0xFFFF0000u), st.o[nb][3]);
    }
    if (rec_mass) tmass[size_t(maxw) * TPW * G + hn] = make_float2(rs, st.m_run);
  }

  // ---------------------------------------------------------- bf16 tiles
  {
    struct FB {
      uint4 k[NB];
      uint4 v[NB];
    };
    auto load_f = [&](FB& fb, uint32_t e) {
      const uint16_t* base = pv.block(seg, te_slot(e), kvh) + size_t(te_tile(e)) * 64 * D;
      const uint4* kp = reinterpret_cast<const uint4*>(base);
      const uint4* vp = reinterpret_cast<const uint4*>(base + 32 * D);
#pragma unroll
      for (int c = 0; c < NB; ++c) fb.k[c] = kp[c * 64 + lane];
#pragma unroll
      for (int c = 0; c < NB; ++c) fb.v[c] = vp[c * 64 + lane];
    };
    auto compute_f = [&](FB& fb, uint32_t e) {
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
        z[i4] = (8 * g + i4 < valid) ? s0[i4] * qscale : -INFINITY;
        z[4 + i4] = (8 * g + 4 + i4 < valid) ? s1[i4] * qscale : -INFINITY;
      }
      softmax_tile<NB>(st, z, p, &rs);
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
      if (rec_mass) tmass[(size_t(w) * TPW + k) * G + hn] = make_float2(rs, st.m_run);
    };
    for (int cb = f_beg; cb < f_end; cb += kList) {
      const int ce = min(f_end, cb + kList), nt = ce - cb;
      build_list(TIER_F, cb, ce);
      FB A, Bf;
      int i = 0;
      load_f(A, uniform(int(list[0])));
      while (i < nt) {
        if (i + 1 < nt) load_f(Bf, uniform(int(list[i + 1])));
        compute_f(A, uniform(int(list[i])));
        if (++i >= nt) break;
        if (i + 1 < nt) load_f(A, uniform(int(list[i + 1])));
        compute_f(Bf, uniform(int(list[i])));
        ++i;
      }
    }
  }

  // ---------------------------------------------------------- INT2 tiles
  {
    const layout::LedgerTile LT(D);
    struct QB {
      uint32_t kc[CW], vc[CW], sc[CW];
    };
    auto load_words = [&](const uint8_t* p, uint32_t (&w)[CW]) {
      if constexpr (CW == 4) {
        const uint4 u = reinterpret_cast<const uint4*>(p)[lane];
        w[0] = u.x;
        w[1] = u.y;
        w[2] = u.z;
        w[3] = u.w;
      } else {
        const uint2 u = reinterpret_cast<const uint2*>(p)[lane];
        w[0] = u.x;
        w[1] = u.y;
      }
    };
    auto load_q = [&](QB& qq, uint32_t e) {
      const uint8_t* t = pv.entry(seg, te_slot(e), kvh) + size_t(te_tile(e)) * LT.bytes;
      load_words(t + LT.kc, qq.kc);
      load_words(t + LT.vc, qq.vc);
      load_words(t + LT.ks, qq.sc);
    };
    uint8_t* scb = s_scb[wid];
    f16x8* bh = reinterpret_cast<f16x8*>(s_bq[wid][0]);
    f16x8* bl = reinterpret_cast<f16x8*>(s_bq[wid][1]);
    float* cst = s_cst[wid];
    auto compute_q = [&](QB& qq, uint32_t e) {
      const int w = te_win(e), k = te_tile(e);
      // the tile's scale block (Ks | Km | Vs | Vm) into this wave's LDS buffer
      if constexpr (CW == 4)
        reinterpret_cast<uint4*>(scb)[lane] = make_uint4(qq.sc[0], qq.sc[1], qq.sc[2], qq.sc[3]);
      else
        reinterpret_cast<uint2*>(scb)[lane] = make_uint2(qq.sc[0], qq.sc[1]);
      const f16x8* ks = reinterpret_cast<const f16x8*>(scb);              // [D]
      const f16x8* km = reinterpret_cast<const f16x8*>(scb + 2 * D);      // [D]
      const f16x8* vs = reinterpret_cast<const f16x8*>(scb + 4 * D);      // [D/32][32]
      const f16x8* vm = reinterpret_cast<const f16x8*>(scb + 6 * D);
      // 4 s q split into fp16 high + low parts, and the tile constant
      // sum_d q (m - 4 s) in fp32, once per (head, dim) in a compact lane
      // layout: item (h, c8) = head h, channels 8*c8..8*c8+7.
#pragma unroll
      for (int r = 0; r < kRounds; ++r) {
        const int it = 64 * r + lane, h = it / (D / 8), c8 = it % (D / 8);
        if (h < G) {
          const f16x8 s8 = ks[c8], m8 = km[c8];
          // 4 s q: fp16 product plus its exact fp16 residual (fma TwoProduct)
          const f16x8 hi8 = qc[r] * s8;
          const f16x8 lo8 = __builtin_elementwise_fma(qc[r], s8, -hi8);
          float cp = 0.f;
#pragma unroll
          for (int e2 = 0; e2 < 8; ++e2)
            cp = fmaf(float(qc[r][e2]), fmaf(float(m8[e2]), 0.25f, -float(s8[e2])), cp);
          bh[h * (D / 8) + c8] = hi8;
          bl[h * (D / 8) + c8] = lo8;
#pragma unroll
          for (int off = 1; off < D / 8; off <<= 1) cp += __shfl_xor(cp, off, 64);
          if (c8 == 0) cst[h] = cp;
        }
      }
      const int hh = hn < G ? hn : G - 1;
      f32x4 s0 = {0.f, 0.f, 0.f, 0.f}, s1 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int kk = 0; kk < KK; ++kk) {
        const f16x8 qh = bh[hh * (D / 8) + 4 * kk + g];
        const f16x8 ql = bl[hh * (D / 8) + 4 * kk + g];
        const int c0 = kk, c1 = KK + kk;                               // chunks of blk 0 / 1
        const f16x8 a0 = (c0 & 1) ? decode_codes<1>(qq.kc[c0 >> 1]) : decode_codes<0>(qq.kc[c0 >> 1]);
        const f16x8 a1 = (c1 & 1) ? decode_codes<1>(qq.kc[c1 >> 1]) : decode_codes<0>(qq.kc[c1 >> 1]);
        s0 = mfma_f16(a0, qh, s0);
        s0 = mfma_f16(a0, ql, s0);
        s1 = mfma_f16(a1, qh, s1);
        s1 = mfma_f16(a1, ql, s1);
      }
      const float bias0 = cst[hh];
      float z[8], p[8], rs;
#pragma unroll
      for (int i4 = 0; i4 < 4; ++i4) {
        z[i4] = (s0[i4] + bias0) * qscale;
        z[4 + i4] = (s1[i4] + bias0) * qscale;
      }
      softmax_tile<NB>(st, z, p, &rs);
      // 4p as fp16 high + low parts, then 4 p s' = high*s' + (exact residual
      // of that product + low*s'), all in packed fp16
      f16x8 p4, p4l;
#pragma unroll
      for (int e2 = 0; e2 < 8; ++e2) {
        const float x = 4.f * p[e2];
        p4[e2] = (_Float16)x;
        p4l[e2] = (_Float16)(x - float(p4[e2]));
      }
      const int jr = hn & (D / 32 - 1);   // min-term row = 32-channel group (rows >= D/32 unused)
      const f16x8 mv = (vm[4 * jr + g] + vs[4 * jr + g] * (_Float16)1.5f) * (_Float16)0.25f;
      st.ob = mfma_f16(mv, p4, st.ob);
      const f16x8 ctr = {(_Float16)1.375f, (_Float16)1.375f, (_Float16)1.375f, (_Float16)1.375f,
                         (_Float16)1.375f, (_Float16)1.375f, (_Float16)1.375f, (_Float16)1.375f};
#pragma unroll
      for (int jd = 0; jd < D / 32; ++jd) {
        const f16x8 sv = vs[4 * jd + g];
        const f16x8 ph = p4 * sv;
        const f16x8 pl = __builtin_elementwise_fma(p4l, sv, __builtin_elementwise_fma(p4, sv, -ph));
#pragma unroll
        for (int h2 = 0; h2 < 2; ++h2) {
          const int nb = 2 * jd + h2;
          const f16x8 av = ((nb & 1) ? decode_codes<1>(qq.vc[nb >> 1]) : decode_codes<0>(qq.vc[nb >> 1])) - ctr;
          st.o[nb] = mfma_f16(av, ph, st.o[nb]);
          st.o[nb] = mfma_f16(av, pl, st.o[nb]);
        }
      }
      if (rec_mass) tmass[(size_t(w) * TPW + k) * G + hn] = make_float2(rs, st.m_run);
    };
    for (int cb = q_beg; cb < q_end; cb += kList) {
      const int ce = min(q_end, cb + kList), nt = ce - cb;
      build_list(TIER_Q, cb, ce);
      // groups of kQGroup tiles: a whole group's loads are in flight together,
      // and the next group's loads are issued before this group is computed
      QB A[kQGroup], Bq[kQGroup];
      auto load_group = [&](QB (&grp)[kQGroup], int i0) {
#pragma unroll
        for (int j = 0; j < kQGroup; ++j)
          if (i0 + j < nt) load_q(grp[j], uniform(int(list[i0 + j])));
      };
      auto compute_group = [&](QB (&grp)[kQGroup], int i0) {
#pragma unroll
        for (int j = 0; j < kQGroup; ++j)
          if (i0 + j < nt) compute_q(grp[j], uniform(int(list[i0 + j])));
      };
      int i = 0;
      load_group(A, 0);
      while (i < nt) {
        if (i + kQGroup < nt) load_group(Bq, i + kQGroup);
        compute_group(A, i);
        i += kQGroup;
        if (i >= nt) break;
        if (i + kQGroup < nt) load_group(A, i + kQGroup);
        compute_group(Bq, i);
        i += kQGroup;
      }
    }
  }

  // -------------------------------------------- combine the 4 waves in LDS
  if (hn < G) {
#pragma unroll
    for (int nb = 0; nb < NB; ++nb)
#pragma unroll
      for (int i4 = 0; i4 < 4; ++i4) s_wo[wid][hn][16 * nb + 4 * g + i4] = st.o[nb][i4];
    if (g == 0) {
      s_wm[wid][hn] = st.m_run;
      s_wl[wid][hn] = st.l_run;
#pragma unroll
      for (int i4 = 0; i4 < 4; ++i4) s_wb[wid][hn][i4] = st.ob[i4];
    }
  }
  __syncthreads();
  // partial of this workgroup: o [G][D], then max [G], then sum [G]
  const int P = (G * (D + 2) + 3) & ~3;
  float* part = a.partials + ((size_t(b) * pv.Hkv + kvh) * S + split) * P;
  for (int idx = tid; idx < G * (D + 2); idx += 256) {
    const int h = idx < G * D ? idx / D : (idx - G * D) % G;
    float M = -INFINITY;
#pragma unroll
    for (int v = 0; v < kAttnWaves; ++v) M = fmaxf(M, s_wm[v][h]);
    float acc = 0.f;
    if (idx >= G * D && idx < G * D + G) {
      acc = M;
    } else {
#pragma unroll
      for (int v = 0; v < kAttnWaves; ++v) {
        const float sc = s_wm[v][h] == -INFINITY ? 0.f : fast_exp2(s_wm[v][h] - M);
        if (idx >= G * D) {
          acc += sc * s_wl[v][h];
        } else {
          const int d = idx % D;
          acc += sc * (s_wo[v][h][d] + s_wb[v][h][d >> 5]);
        }
      }
    }
    part[idx] = acc;
  }
}

// --------------------------------------------------------------------------
// Combine: blocks x < Hkv produce the output of kv head x of sequence y (and
// store an appended token's K/V); blocks x >= Hkv normalise the window masses
// of 256 windows for every query head, optionally adding them to the
// cumulative scores.
template <int D>
__global__ __launch_bounds__(256) void combine_kernel(PoolView pv, AttnArgs a, int acc_scores) {
  __shared__ float s_scale[kMaxSplits * kGMax];
  __shared__ float4 s_acc[256];
  __shared__ float s_pm[256], s_pz[256];
  extern __shared__ float s_mz[];            // mass blocks: max, normaliser [Hq], masses [64][Hq]
  const int b = blockIdx.y, x = blockIdx.x, tid = threadIdx.x;
  const int G = pv.G, Hkv = pv.Hkv, Hq = pv.Hq, S = a.splits, W = pv.W, maxw = pv.maxw;
  const int TPW = W / 32, seg = a.layer * pv.B + b;
  const int P = (G * (D + 2) + 3) & ~3;
  const int32_t* info = a.app_info + 8 * b;
  const int app = info[0], slot = info[1], row = info[2], newwin = info[3], len_old = info[4];
  const int len = len_old + (app ? 1 : 0);
  const int n_old = windows_of(len_old, W), n_win = windows_of(len, W);

  if (x < Hkv) {
    const int kvh = x;
    const float* parts = a.partials + (size_t(b) * Hkv + kvh) * S * P;
    float* s_lsum = reinterpret_cast<float*>(s_acc);
    for (int i = tid; i < S * G; i += 256) {
      s_scale[i] = parts[size_t(i / G) * P + G * D + i % G];
      s_lsum[i] = parts[size_t(i / G) * P + G * D + G + i % G];
    }
    __syncthreads();
    if (tid < G) {
      float M = -INFINITY, Z = 0.f;
      for (int sp = 0; sp < S; ++sp) M = fmaxf(M, s_scale[sp * G + tid]);
      for (int sp = 0; sp < S; ++sp) {
        const float ms = s_scale[sp * G + tid];
        const float sc = ms == -INFINITY ? 0.f : exp2f(ms - M);
        s_scale[sp * G + tid] = sc;
        Z += sc * s_lsum[sp * G + tid];
      }
      s_pz[tid] = Z;
    }
    __syncthreads();
    __syncthreads();
    const int items = G * D / 4, groups = 256 / items;
    const int it = tid % items, grp = tid / items;
    float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
    if (grp < groups) {
      const int h = (4 * it) / D;
      const float4* po = reinterpret_cast<const float4*>(parts) + it;
      // all of this thread's partial outputs in flight at once, 16 at a time
      for (int sp0 = grp; sp0 < S; sp0 += 16 * groups) {
        float4 v4[16];
#pragma unroll
        for (int j = 0; j < 16; ++j) {
          const int sp = sp0 + j * groups;
          v4[j] = sp < S ? po[size_t(sp) * (P / 4)] : make_float4(0.f, 0.f, 0.f, 0.f);
        }
#pragma unroll
        for (int j = 0; j < 16; ++j) {
          const int sp = sp0 + j * groups;
          const float sc = sp < S ? s_scale[sp * G + h] : 0.f;
          acc.x = fmaf(sc, v4[j].x, acc.x);
          acc.y = fmaf(sc, v4[j].y, acc.y);
          acc.z = fmaf(sc, v4[j].z, acc.z);
          acc.w = fmaf(sc, v4[j].w, acc.w);
        }
      }
      s_acc[grp * items + it] = acc;
    }
    __syncthreads();
    if (tid < items) {
      float4 t4 = s_acc[tid];
      for (int q2 = 1; q2 < groups; ++q2) {
        const float4 u = s_acc[q2 * items + tid];
        t4.x += u.x; t4.y += u.y; t4.z += u.z; t4.w += u.w;
      }
      const int h = (4 * tid) / D, d = (4 * tid) % D;
      const float Z = s_pz[h], iz = Z > 0.f ? 1.f / Z : 0.f;
      *reinterpret_cast<float4*>(a.out + (size_t(b) * Hq + size_t(kvh) * G + h) * D + d) =
          make_float4(t4.x * iz, t4.y * iz, t4.z * iz, t4.w * iz);
    }
    if (app) {
      // the appended token joins its window (no kernel of this step reads it)
      uint16_t* dst = pv.block(seg, slot, kvh);
      for (int d = tid; d < D; d += 256) {
        dst[layout::bf16_window_k(row, d, D)] = a.k_new[(size_t(b) * Hkv + kvh) * D + d];
        dst[layout::bf16_window_v(row, d, D)] = a.v_new[(size_t(b) * Hkv + kvh) * D + d];
      }
      if (kvh == 0 && tid == 0) {
        if (newwin) pv.pages[size_t(seg) * maxw + n_old] = pe_make(TIER_F, false, slot, 0);
        pv.tokens[seg] = len;
      }
    }
    return;
  }

  // ---------------------------------------------------------- window masses
  // 64 windows per block; thread (window wl, head lane hq) takes heads hq, hq+4, ...
  if (!a.mass && !acc_scores) return;
  const int w0 = (x - Hkv) * kMassWindows;
  if (w0 >= n_win) return;
  float* s_M = s_mz;             // [Hq]
  float* s_Zh = s_mz + Hq;       // [Hq]
  float* s_mv = s_mz + 2 * Hq;   // [kMassWindows][Hq]
  // per-head max and normaliser over all splits: threads (h, c) scan splits c, c + C, ...
  const int hs = min(Hq, 256), C = max(1, 256 / Hq);
  for (int h0 = 0; h0 < Hq; h0 += 256) {
    const int h = h0 + tid % hs, c = tid / hs;
    float M = -INFINITY, Z = 0.f;
    if (h < Hq && c < C) {
      const int kvh = h / G, hl = h % G;
      const float* parts = a.partials + (size_t(b) * Hkv + kvh) * S * P + G * D;
#pragma unroll 8
      for (int sp = c; sp < S; sp += C) {
        const float ms = parts[size_t(sp) * P + hl], ls = parts[size_t(sp) * P + G + hl];
        if (ms != -INFINITY) {
          const float mn = fmaxf(M, ms);
          Z = Z * exp2f(M - mn) + ls * exp2f(ms - mn);
          M = mn;
        }
      }
    }
    s_pm[tid] = M;
    s_pz[tid] = Z;
    __syncthreads();
    if (tid < min(Hq - h0, 256)) {
      float Mh = -INFINITY, Zh = 0.f;
      for (int cc = 0; cc < C; ++cc) {
        const float ms = s_pm[cc * hs + tid], zs = s_pz[cc * hs + tid];
        if (ms == -INFINITY) continue;
        const float mn = fmaxf(Mh, ms);
        Zh = Zh * exp2f(Mh - mn) + zs * exp2f(ms - mn);
        Mh = mn;
      }
      s_M[h0 + tid] = Mh;
      s_Zh[h0 + tid] = Zh;
    }
    __syncthreads();
  }
  const int wl = tid % kMassWindows, hq = tid / kMassWindows;
  const int w = w0 + wl;
  const bool in = w < n_win;
  bool live = false;
  int vt = 0;
  if (in) {
    if (w < n_old) {
      live = pe_tier(pv.pages[size_t(seg) * maxw + w]) != TIER_E;
      vt = (min(W, len_old - w * W) + 31) / 32;
    } else {
      live = true;   // the window the appended token opened
    }
  }
  const bool vwin = app && w == len_old / W;
  // tile masses of 4 heads (all their tiles) in flight at once
  constexpr int HL = 256 / kMassWindows;   // head lanes per window
  const float2* tm0 = reinterpret_cast<const float2*>(a.tile_mass);
  for (int h0 = hq; h0 < Hq; h0 += 4 * HL) {
    float2 t[4][8];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int h = h0 + j * HL;
      const int kvh = h / G, hl = h % G;
      const float2* tm = tm0 + (size_t(b) * Hkv + kvh) * (size_t(maxw) * TPW + 1) * G;
      const bool on = in && live && h < Hq;
#pragma unroll
      for (int k = 0; k < 8; ++k)
        t[j][k] = (on && k < vt) ? tm[(size_t(w) * TPW + k) * G + hl] : make_float2(0.f, 0.f);
    }
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int h = h0 + j * HL;
      if (h >= Hq) break;
      float mv = 0.f;
      if (in && live) {
        const float M = s_M[h], Z = s_Zh[h];
        float acc = 0.f;
#pragma unroll
        for (int k = 0; k < 8; ++k)
          if (k < vt) acc += t[j][k].x * exp2f(t[j][k].y - M);
        if (vwin) {
          const int kvh = h / G, hl = h % G;
          const float2 tv = tm0[(size_t(b) * Hkv + kvh) * (size_t(maxw) * TPW + 1) * G +
                                size_t(maxw) * TPW * G + hl];
          acc += tv.x * exp2f(tv.y - M);
        }
        mv = Z > 0.f ? acc / Z : 0.f;
      }
      if (in && a.mass) a.mass[(size_t(b) * Hq + h) * maxw + w] = mv;
      s_mv[wl * Hq + h] = mv;
    }
  }
  __syncthreads();
  if (acc_scores && hq == 0 && in && live) {
    float ssum = 0.f;
    for (int h = 0; h < Hq; ++h) ssum += s_mv[wl * Hq + h];   // heads in order
    pv.scores[size_t(seg) * maxw + w] += ssum;
  }
}

template <int D>
static hipError_t launch_attn_t(const PoolView& pv, const AttnArgs& a, hipStream_t s) {
  const size_t shm = size_t((pv.nb + 31) / 32) * 4;
  if (a.ev_start || a.ev_stop) {
    hipExtLaunchKernelGGL((attn_kernel<D>), dim3(a.splits, pv.Hkv, pv.B), dim3(256), uint32_t(shm), s,
                          a.ev_start, a.ev_stop, 0u, pv, a);
  } else {
    hipLaunchKernelGGL((attn_kernel<D>), dim3(a.splits, pv.Hkv, pv.B), dim3(256), shm, s, pv, a);
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int mass_blocks = (a.mass || a.acc_scores) ? (pv.maxw + kMassWindows - 1) / kMassWindows : 0;
  hipLaunchKernelGGL((combine_kernel<D>), dim3(pv.Hkv + mass_blocks, pv.B), dim3(256),
                     size_t(2 + kMassWindows) * pv.Hq * 4, s, pv, a, a.acc_scores);
  return hipGetLastError();
}

hipError_t launch_attn(const PoolView& pv, const AttnArgs& a, hipStream_t s) {
  if (pv.G > kGMax) return hipErrorInvalidValue;
  if (pv.D == 64) return launch_attn_t<64>(pv, a, s);
  if (pv.D == 128) return launch_attn_t<128>(pv, a, s);
  return hipErrorInvalidValue;
}

}  // namespace kvtier
