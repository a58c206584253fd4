// Tiered decode attention with per-window mass for gfx950.
//
// QEvict technical summary ("Methodologie: QEvict", "Kernmechanismen",
// "Implementatie"): bf16 windows and INT2 windows both take part in attention,
// evicted windows do not; grouped-query attention; the attention each window
// receives is what the cumulative score adds up.  Unlike the summary's
// FlashAttention-2 path, which dequantises and rebuilds caches before attention
// ("Resultaten", efficiency), INT2 tiles are dequantised in registers inside
// this kernel: HBM carries 3 bits per INT2 value, never a rebuilt bf16 copy.
//
// Work split: grid (splits, kv heads, sequences), 4 wave64 per workgroup.  The
// live tiles (32 tokens of one window) of a (sequence, kv head) are weighted by
// their bytes (bf16 tile 16 KB, INT2 tile 3 KB) and the weight range is cut
// evenly over all waves of all splits.  Each wave keeps an online softmax
// (running max, sum, output) for the G query heads of its kv head and records
// every tile's raw mass with the running max it was taken at; the last
// workgroup of a (sequence, kv head) combines the partials into the output and
// the normalised window masses (tokens may be taken in any order:
// A.V = A_P.V_P, LogQuant summary, "Positie-agnostische optimalisatie").
//
// A decode step may append a token: it is attended straight from k_new/v_new
// and stored in the newest window afterwards; the page table and token count
// are rewritten by the last workgroup of the sequence, after every workgroup of
// that sequence has read them.
#include <hip/hip_ext.h>
#include <math.h>

#include "host_core.h"
#include "launch.h"

namespace kvtier {

namespace {

__device__ inline int uniform(int x) { return __builtin_amdgcn_readfirstlane(x); }

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

__device__ inline void unpack_bf16x8(const uint4 u, float (&f)[8]) {
  const uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    f[2 * i] = __uint_as_float(w[i] << 16);
    f[2 * i + 1] = __uint_as_float(w[i] & 0xFFFF0000u);
  }
}

__device__ inline void unpack_f16x8(const uint4 u, float (&f)[8]) {
  const uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    f[2 * i] = float(__builtin_bit_cast(_Float16, uint16_t(w[i] & 0xFFFFu)));
    f[2 * i + 1] = float(__builtin_bit_cast(_Float16, uint16_t(w[i] >> 16)));
  }
}

__device__ inline float half_at(const uint8_t* p, int idx) {
  return float(__builtin_bit_cast(_Float16, reinterpret_cast<const uint16_t*>(p)[idx]));
}

}  // namespace

template <int D, int G>
__global__ __launch_bounds__(256) void attn_kernel(PoolView pv, AttnArgs a) {
  constexpr int LPR = D / 8;      // lanes per token row (8 values each)
  constexpr int RS = 64 / LPR;    // token rows per wave step
  constexpr int STEPS = kTile / RS;
  extern __shared__ int smem_i[];
  __shared__ int s_tmp[4];
  __shared__ int s_app[4];        // append ok, slot, row, new window
  __shared__ float s_wm[kAttnWaves][G], s_wl[kAttnWaves][G];
  __shared__ float s_wo[kAttnWaves][G][D];
  __shared__ int s_last;

  const int split = blockIdx.x, kvh = blockIdx.y, b = blockIdx.z;
  const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
  const int r = lane / LPR, c = lane % LPR;
  const int W = pv.W, maxw = pv.maxw, TPW = W / kTile;
  const int seg = a.layer * pv.B + b;
  const int S = a.splits;
  int* s_pref = smem_i;                                              // [maxw + 2]
  uint32_t* s_info = reinterpret_cast<uint32_t*>(smem_i + maxw + 2);  // [maxw + 1]
  uint32_t* s_used = s_info + maxw + 1;                               // [(nb + 31) / 32]

  // ---------------------------------------------------------------- state
  const int len_old = pv.tokens[seg];
  const int n_old = windows_of(len_old, W);
  const uint32_t* gp = pv.pages + size_t(seg) * maxw;
  for (int w = tid; w < n_old; w += 256) s_info[w] = gp[w];
  const bool want_append = a.k_new != nullptr;
  if (tid == 0) s_app[0] = 0;
  __syncthreads();
  if (want_append) {
    if (len_old % W != 0) {
      if (tid == 0) {
        const uint32_t e = s_info[n_old - 1];
        s_app[0] = pe_tier(e) == TIER_F;
        s_app[1] = pe_bslot(e);
        s_app[2] = len_old % W;
        s_app[3] = 0;
        if (!s_app[0] && split == 0 && kvh == 0) set_err(pv.err, KV_ERR_APPEND_STATE);
      }
    } else {
      // a new window opens: the lowest bf16 slot no live bf16 window holds
      const int words = (pv.nb + 31) / 32;
      for (int i = tid; i < words; i += 256) s_used[i] = 0u;
      __syncthreads();
      for (int w = tid; w < n_old; w += 256) {
        const uint32_t e = s_info[w];
        if (pe_tier(e) == TIER_F && pe_bslot(e) < pv.nb)
          atomicOr(&s_used[pe_bslot(e) >> 5], 1u << (pe_bslot(e) & 31));
      }
      __syncthreads();
      if (tid == 0) {
        int slot = -1;
        for (int i = 0; i < words && slot < 0; ++i) {
          const uint32_t x = ~s_used[i];
          if (x) {
            const int j = i * 32 + __builtin_ctz(x);
            if (j < pv.nb) slot = j;
            break;
          }
        }
        const bool cap = n_old < maxw;
        s_app[0] = cap && slot >= 0;
        s_app[1] = slot;
        s_app[2] = 0;
        s_app[3] = 1;
        if (!s_app[0] && split == 0 && kvh == 0)
          set_err(pv.err, cap ? KV_ERR_NO_BF16_SLOT : KV_ERR_CAPACITY);
        if (s_app[0]) s_info[n_old] = pe_make(TIER_F, false, slot, 0);
      }
    }
  }
  __syncthreads();
  const bool appending = s_app[0] != 0;
  const int len = len_old + (appending ? 1 : 0);
  const int n = windows_of(len, W);

  // --------------------------------------- byte-weighted tile partition
  {
    const int per = (n + 255) / 256;
    const int w0 = tid * per, w1 = min(n, w0 + per);
    int sum = 0;
    for (int w = w0; w < w1; ++w) {
      const int t = pe_tier(s_info[w]);
      const int vt = (min(W, len - w * W) + kTile - 1) / kTile;
      sum += t == TIER_F ? 16 * vt : (t == TIER_Q ? 3 * vt : 0);
    }
    int total;
    int run = block_excl_scan(sum, s_tmp, &total);
    for (int w = w0; w < w1; ++w) {
      s_pref[w] = run;
      const int t = pe_tier(s_info[w]);
      const int vt = (min(W, len - w * W) + kTile - 1) / kTile;
      run += t == TIER_F ? 16 * vt : (t == TIER_Q ? 3 * vt : 0);
    }
    if (tid == 0) s_pref[n] = total;
  }
  __syncthreads();
  const int U = s_pref[n];
  const long nwaves = long(S) * kAttnWaves;
  const long widx = long(split) * kAttnWaves + wid;
  const int u0 = int(widx * U / nwaves), u1 = int((widx + 1) * U / nwaves);

  // ------------------------------------------------------------ the query
  constexpr float kLog2e = 1.4426950408889634f;
  const float qscale = kLog2e / sqrtf(float(D));
  float qf[G][8];
  {
    const uint16_t* qp = a.q + (size_t(b) * pv.Hq + size_t(kvh) * G) * D + 8 * c;
#pragma unroll
    for (int h = 0; h < G; ++h) {
      float f[8];
      unpack_bf16x8(*reinterpret_cast<const uint4*>(qp + size_t(h) * D), f);
#pragma unroll
      for (int e = 0; e < 8; ++e) qf[h][e] = f[e] * qscale;
    }
  }
  const uint16_t* knew = a.k_new ? a.k_new + (size_t(b) * pv.Hkv + kvh) * D : nullptr;
  const uint16_t* vnew = a.v_new ? a.v_new + (size_t(b) * pv.Hkv + kvh) * D : nullptr;

  float m_run[G], l_run[G], o[G][8];
#pragma unroll
  for (int h = 0; h < G; ++h) {
    m_run[h] = -INFINITY;
    l_run[h] = 0.f;
#pragma unroll
    for (int e = 0; e < 8; ++e) o[h][e] = 0.f;
  }
  const EntryLayout L(W, D);
  float2* tmass = reinterpret_cast<float2*>(a.tile_mass) +
                  (size_t(b) * pv.Hkv + kvh) * size_t(maxw) * TPW * G;

  // first window whose weight range ends past u0
  int wlo = 0, whi = n;
  while (wlo < whi) {
    const int mid = (wlo + whi) >> 1;
    if (s_pref[mid + 1] > u0) whi = mid; else wlo = mid + 1;
  }
  for (int w = uniform(wlo); w < n && s_pref[w] < u1; ++w) {
    const uint32_t e = uniform(int(s_info[w]));
    const int tier = pe_tier(e);
    if (tier == TIER_E) continue;
    const int valid = min(W, len - w * W);
    const int vt = (valid + kTile - 1) / kTile;
    const int tw = tier == TIER_F ? 16 : 3;
    const int pw = uniform(s_pref[w]);
    for (int k = 0; k < vt; ++k) {
      const int st = pw + k * tw;
      if (st < u0) continue;
      if (st >= u1) break;
      float z[STEPS][G];
      float p[STEPS][G];
      if (tier == TIER_F) {
        const uint16_t* Kp = pv.block(seg, pe_bslot(e), kvh);
#pragma unroll
        for (int i = 0; i < STEPS; ++i) {
          const int row = kTile * k + i * RS + r;
          const int pos = w * W + row;
          float part[G];
#pragma unroll
          for (int h = 0; h < G; ++h) part[h] = 0.f;
          if (pos < len) {
            const uint16_t* src = (appending && pos == len_old) ? knew : Kp + size_t(row) * D;
            float kv[8];
            unpack_bf16x8(*reinterpret_cast<const uint4*>(src + 8 * c), kv);
#pragma unroll
            for (int h = 0; h < G; ++h)
#pragma unroll
              for (int x = 0; x < 8; ++x) part[h] = fmaf(qf[h][x], kv[x], part[h]);
          }
#pragma unroll
          for (int h = 0; h < G; ++h) {
#pragma unroll
            for (int off = 1; off < LPR; off <<= 1) part[h] += __shfl_xor(part[h], off, 64);
            z[i][h] = pos < len ? part[h] : -INFINITY;
          }
        }
      } else {
        const uint8_t* E = pv.entry(seg, pe_lslot(e), kvh);
        float ks[8], km[8];
        unpack_f16x8(*reinterpret_cast<const uint4*>(E + L.ks + (size_t(k) * D + 8 * c) * 2), ks);
        unpack_f16x8(*reinterpret_cast<const uint4*>(E + L.km + (size_t(k) * D + 8 * c) * 2), km);
        float qs[G][8], qm[G];
#pragma unroll
        for (int h = 0; h < G; ++h) {
          qm[h] = 0.f;
#pragma unroll
          for (int x = 0; x < 8; ++x) {
            qs[h][x] = qf[h][x] * ks[x];
            qm[h] = fmaf(qf[h][x], km[x], qm[h]);
          }
        }
#pragma unroll
        for (int i = 0; i < STEPS; ++i) {
          const int row = kTile * k + i * RS + r;
          const uint32_t cw = *reinterpret_cast<const uint16_t*>(E + L.kc + size_t(row) * (D / 4) + 2 * c);
          float part[G];
#pragma unroll
          for (int h = 0; h < G; ++h) {
            part[h] = qm[h];
#pragma unroll
            for (int x = 0; x < 8; ++x) part[h] = fmaf(qs[h][x], float((cw >> (2 * x)) & 3u), part[h]);
#pragma unroll
            for (int off = 1; off < LPR; off <<= 1) part[h] += __shfl_xor(part[h], off, 64);
            z[i][h] = part[h];
          }
        }
      }
      // online softmax update with this tile
      float rsum[G];
#pragma unroll
      for (int h = 0; h < G; ++h) {
        float tm = z[0][h];
#pragma unroll
        for (int i = 1; i < STEPS; ++i) tm = fmaxf(tm, z[i][h]);
#pragma unroll
        for (int off = LPR; off < 64; off <<= 1) tm = fmaxf(tm, __shfl_xor(tm, off, 64));
        const float mn = fmaxf(m_run[h], tm);
        const float alpha = exp2f(m_run[h] - mn);
        float s = 0.f;
#pragma unroll
        for (int i = 0; i < STEPS; ++i) {
          p[i][h] = exp2f(z[i][h] - mn);
          s += p[i][h];
        }
#pragma unroll
        for (int off = LPR; off < 64; off <<= 1) s += __shfl_xor(s, off, 64);
        rsum[h] = s;
        l_run[h] = l_run[h] * alpha + s;
        m_run[h] = mn;
#pragma unroll
        for (int x = 0; x < 8; ++x) o[h][x] *= alpha;
      }
      if (tier == TIER_F) {
        const uint16_t* Vp = pv.block(seg, pe_bslot(e), kvh) + size_t(W) * D;
#pragma unroll
        for (int i = 0; i < STEPS; ++i) {
          const int row = kTile * k + i * RS + r;
          const int pos = w * W + row;
          if (pos < len) {
            const uint16_t* src = (appending && pos == len_old) ? vnew : Vp + size_t(row) * D;
            float vv[8];
            unpack_bf16x8(*reinterpret_cast<const uint4*>(src + 8 * c), vv);
#pragma unroll
            for (int h = 0; h < G; ++h)
#pragma unroll
              for (int x = 0; x < 8; ++x) o[h][x] = fmaf(p[i][h], vv[x], o[h][x]);
          }
        }
      } else {
        const uint8_t* E = pv.entry(seg, pe_lslot(e), kvh);
#pragma unroll
        for (int i = 0; i < STEPS; ++i) {
          const int row = kTile * k + i * RS + r;
          const uint32_t cw = *reinterpret_cast<const uint16_t*>(E + L.vc + size_t(row) * (D / 4) + 2 * c);
          const float vsc = half_at(E + L.vs, row * (D / 32) + c / 4);
          const float vmn = half_at(E + L.vm, row * (D / 32) + c / 4);
#pragma unroll
          for (int h = 0; h < G; ++h) {
            const float ps = p[i][h] * vsc, pm = p[i][h] * vmn;
#pragma unroll
            for (int x = 0; x < 8; ++x) o[h][x] = fmaf(ps, float((cw >> (2 * x)) & 3u), o[h][x] + pm);
          }
        }
      }
      if (a.mass && lane == 0) {
#pragma unroll
        for (int h = 0; h < G; ++h) tmass[(size_t(w) * TPW + k) * G + h] = make_float2(rsum[h], m_run[h]);
      }
    }
  }

  // -------------------------------------------- combine the 4 waves in LDS
#pragma unroll
  for (int h = 0; h < G; ++h)
#pragma unroll
    for (int x = 0; x < 8; ++x)
#pragma unroll
      for (int off = LPR; off < 64; off <<= 1) o[h][x] += __shfl_xor(o[h][x], off, 64);
  if (r == 0) {
#pragma unroll
    for (int h = 0; h < G; ++h)
#pragma unroll
      for (int x = 0; x < 8; ++x) s_wo[wid][h][8 * c + x] = o[h][x];
  }
  if (lane == 0) {
#pragma unroll
    for (int h = 0; h < G; ++h) {
      s_wm[wid][h] = m_run[h];
      s_wl[wid][h] = l_run[h];
    }
  }
  __syncthreads();
  const int P = G * (D + 2);
  float* part = a.partials + ((size_t(b) * pv.Hkv + kvh) * S + split) * P;
  for (int idx = tid; idx < P; idx += 256) {
    const int h = idx < 2 * G ? idx % G : (idx - 2 * G) / D;
    float M = -INFINITY;
#pragma unroll
    for (int v = 0; v < kAttnWaves; ++v) M = fmaxf(M, s_wm[v][h]);
    float acc = 0.f;
    if (idx < G) {
      acc = M;
    } else {
#pragma unroll
      for (int v = 0; v < kAttnWaves; ++v) {
        const float sc = s_wm[v][h] == -INFINITY ? 0.f : exp2f(s_wm[v][h] - M);
        acc += sc * (idx < 2 * G ? s_wl[v][h] : s_wo[v][h][(idx - 2 * G) % D]);
      }
    }
    part[idx] = acc;
  }

  // ------------------------------------ the last workgroup combines splits
  __threadfence();
  __syncthreads();
  int32_t* ctr = pv.work + pv.attn_counters + b * pv.Hkv + kvh;
  if (tid == 0) {
    const int prev = __hip_atomic_fetch_add(ctr, 1, __ATOMIC_ACQ_REL, __HIP_MEMORY_SCOPE_AGENT);
    s_last = prev == S - 1;
  }
  __syncthreads();
  if (!s_last) return;
  __threadfence();
  if (tid == 0) __hip_atomic_store(ctr, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);

  float* s_scale = &s_wo[0][0][0];          // [S][G], S * G <= 4 * G * D
  __shared__ float s_M[G], s_Z[G];
  const float* parts = a.partials + (size_t(b) * pv.Hkv + kvh) * S * P;
  if (tid < G) {
    float M = -INFINITY;
    for (int s = 0; s < S; ++s) M = fmaxf(M, parts[size_t(s) * P + tid]);
    float Z = 0.f;
    for (int s = 0; s < S; ++s) {
      const float ms = parts[size_t(s) * P + tid];
      const float sc = ms == -INFINITY ? 0.f : exp2f(ms - M);
      s_scale[s * G + tid] = sc;
      Z += sc * parts[size_t(s) * P + G + tid];
    }
    s_M[tid] = M;
    s_Z[tid] = Z;
  }
  __syncthreads();
  for (int idx = tid; idx < G * D; idx += 256) {
    const int h = idx / D, d = idx % D;
    float acc = 0.f;
    for (int s = 0; s < S; ++s) acc += s_scale[s * G + h] * parts[size_t(s) * P + 2 * G + h * D + d];
    const float Z = s_Z[h];
    a.out[(size_t(b) * pv.Hq + size_t(kvh) * G + h) * D + d] = Z > 0.f ? acc / Z : 0.f;
  }
  if (a.mass) {
    for (int h = 0; h < G; ++h) {
      const float M = s_M[h], Z = s_Z[h];
      float* mo = a.mass + (size_t(b) * pv.Hq + size_t(kvh) * G + h) * maxw;
      for (int w = tid; w < n; w += 256) {
        const uint32_t e = s_info[w];
        float acc = 0.f;
        if (pe_tier(e) != TIER_E) {
          const int vt = (min(W, len - w * W) + kTile - 1) / kTile;
          for (int k = 0; k < vt; ++k) {
            const float2 t = tmass[(size_t(w) * TPW + k) * G + h];
            acc += t.x * exp2f(t.y - M);
          }
        }
        mo[w] = Z > 0.f ? acc / Z : 0.f;
      }
    }
  }
  if (appending) {
    // store the appended token in its window (no workgroup reads that row)
    uint16_t* dst = pv.block(seg, s_app[1], kvh) + size_t(s_app[2]) * D;
    for (int d = tid; d < D; d += 256) {
      dst[d] = knew[d];
      dst[size_t(W) * D + d] = vnew[d];
    }
    __threadfence();
    __syncthreads();
    if (tid == 0) {
      int32_t* sc = pv.work + pv.seg_counters + b;
      const int prev = __hip_atomic_fetch_add(sc, 1, __ATOMIC_ACQ_REL, __HIP_MEMORY_SCOPE_AGENT);
      if (prev == pv.Hkv - 1) {
        __hip_atomic_store(sc, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        if (s_app[3]) pv.pages[size_t(seg) * maxw + n_old] = pe_make(TIER_F, false, s_app[1], 0);
        pv.tokens[seg] = len;
      }
    }
  }
}

template <int D, int G>
static hipError_t launch_attn_t(const PoolView& pv, const AttnArgs& a, hipStream_t s) {
  const size_t shm = size_t(pv.maxw + 2) * 4 + size_t(pv.maxw + 1) * 4 + size_t((pv.nb + 31) / 32) * 4;
  if (a.ev_start || a.ev_stop) {
    hipExtLaunchKernelGGL((attn_kernel<D, G>), dim3(a.splits, pv.Hkv, pv.B), dim3(256), uint32_t(shm), s,
                          a.ev_start, a.ev_stop, 0u, pv, a);
  } else {
    hipLaunchKernelGGL((attn_kernel<D, G>), dim3(a.splits, pv.Hkv, pv.B), dim3(256), shm, s, pv, a);
  }
  return hipGetLastError();
}

hipError_t launch_attn(const PoolView& pv, const AttnArgs& a, hipStream_t s) {
#define KV_CASE(DD, GG) \
  if (pv.D == DD && pv.G == GG) return launch_attn_t<DD, GG>(pv, a, s);
  KV_CASE(64, 1) KV_CASE(64, 2) KV_CASE(64, 4) KV_CASE(64, 7) KV_CASE(64, 8)
  KV_CASE(128, 1) KV_CASE(128, 2) KV_CASE(128, 4) KV_CASE(128, 7) KV_CASE(128, 8)
#undef KV_CASE
  return hipErrorInvalidValue;
}

}  // namespace kvtier
