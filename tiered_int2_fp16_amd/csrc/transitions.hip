// Window transitions for gfx950: prefill, demote (INT2 quantise into the
// write-once ledger), promote (dequantise back to bf16), canonical read-back.
//
// QEvict technical summary, "Kernmechanismen": a bf16 window whose importance
// drops is demoted to the quantised tier; a quantised window whose cumulative
// score rises is dequantised and promoted; a window is quantised only once, at
// its first demotion, and the ledger entry is reused by every later promotion
// and demotion so approximation error does not compound.
//
// Each transition is two launches: a plan kernel (one workgroup per sequence)
// validates the items in order, assigns the lowest free slot and rewrites the
// page table; a data kernel then moves the bytes of every planned item.
#include "launch.h"

namespace kvtier {

// ------------------------------------------------------------------ prefill
__global__ __launch_bounds__(256) void prefill_kernel(PoolView pv, int layer, const uint16_t* k,
                                                      const uint16_t* v, int T, const float* prior) {
  const int w = blockIdx.x, kvh = blockIdx.y, b = blockIdx.z;
  const int seg = layer * pv.B + b;
  const int D = pv.D, W = pv.W, n = windows_of(T, W);
  uint16_t* dk = pv.block(seg, w, kvh);
  uint16_t* dv = dk + size_t(W) * D;
  const size_t src = (size_t(b) * pv.Hkv + kvh) * size_t(T) * D;
  const int vec = D / 8;
  for (int idx = threadIdx.x; idx < W * vec; idx += blockDim.x) {
    const int t = idx / vec, c = idx % vec, pos = w * W + t;
    uint4 a = make_uint4(0, 0, 0, 0), bb = make_uint4(0, 0, 0, 0);
    if (pos < T) {
      a = *reinterpret_cast<const uint4*>(k + src + size_t(pos) * D + 8 * c);
      bb = *reinterpret_cast<const uint4*>(v + src + size_t(pos) * D + 8 * c);
    }
    *reinterpret_cast<uint4*>(dk + size_t(t) * D + 8 * c) = a;
    *reinterpret_cast<uint4*>(dv + size_t(t) * D + 8 * c) = bb;
  }
  if (kvh == 0 && threadIdx.x == 0) {
    pv.pages[size_t(seg) * pv.maxw + w] = pe_make(TIER_F, false, w, 0);
    pv.scores[size_t(seg) * pv.maxw + w] = prior ? prior[size_t(b) * n + w] : 0.f;
  }
  if (w == 0 && kvh == 0) {
    for (int x = n + threadIdx.x; x < pv.maxw; x += blockDim.x) {
      pv.pages[size_t(seg) * pv.maxw + x] = 0u;
      pv.scores[size_t(seg) * pv.maxw + x] = 0.f;
    }
    if (threadIdx.x == 0) pv.tokens[seg] = T;
  }
}

hipError_t launch_prefill(const PoolView& pv, int layer, const uint16_t* k, const uint16_t* v,
                          int tokens, const float* prior, hipStream_t s) {
  const int n = (tokens + pv.W - 1) / pv.W;
  hipLaunchKernelGGL(prefill_kernel, dim3(n, pv.Hkv, pv.B), dim3(256), 0, s, pv, layer, k, v, tokens,
                     prior);
  return hipGetLastError();
}

// -------------------------------------------------------------- the codec
// One group of 32 values: asymmetric min/max INT2.  Signed zeros are made +0,
// s = fp16((max - min) / 3), m = fp16(min); codes use the stored fp16 values:
// c = clamp(rint_even((x - m) / s), 0, 3), or 0 when s == 0.  float32 IEEE
// arithmetic throughout (correctly rounded divide, no contraction).
__device__ inline void quant_group(float (&x)[32], uint8_t (&c)[32], uint16_t* s_out, uint16_t* m_out) {
  float mn, mx;
#pragma unroll
  for (int i = 0; i < 32; ++i) x[i] = (x[i] == 0.f) ? 0.f : x[i];
  mn = x[0];
  mx = x[0];
#pragma unroll
  for (int i = 1; i < 32; ++i) {
    mn = fminf(mn, x[i]);
    mx = fmaxf(mx, x[i]);
  }
  const float d = mx - mn;
  const float s32 = __fdiv_rn(d, 3.0f);
  const _Float16 hs = (_Float16)s32;
  const _Float16 hm = (_Float16)mn;
  const float s = (float)hs, m = (float)hm;
#pragma unroll
  for (int i = 0; i < 32; ++i) {
    float q = 0.f;
    if (s != 0.f) {
      const float u = x[i] - m;
      q = fminf(fmaxf(rintf(__fdiv_rn(u, s)), 0.f), 3.f);
    }
    c[i] = uint8_t(q);
  }
  *s_out = __builtin_bit_cast(uint16_t, hs);
  *m_out = __builtin_bit_cast(uint16_t, hm);
}

// ------------------------------------------------------------------ demote
struct WorkItem {
  int w, src, dst, flag;  // flag 1: move bytes; 2: tier flip only; 0: invalid
};

__device__ inline int find_free(uint32_t* bits, int nbits) {
  for (int word = 0; word * 32 < nbits; ++word) {
    uint32_t x = ~bits[word];
    if (x) {
      const int j = word * 32 + __builtin_ctz(x);
      if (j >= nbits) return -1;
      bits[word] |= 1u << (j & 31);
      return j;
    }
  }
  return -1;
}

// promote == false: demote plan (ledger slots); true: promote plan (bf16 slots).
__global__ __launch_bounds__(256) void plan_kernel(PoolView pv, int layer, const int32_t* items, int stride,
                                                   const int32_t* counts, int promote) {
  extern __shared__ uint32_t smem[];
  const int b = blockIdx.x, seg = layer * pv.B + b;
  const int maxw = pv.maxw, W = pv.W;
  const int nslots = promote ? pv.nb : pv.nl;
  const int words = (nslots + 31) / 32;
  uint32_t* pages = smem;
  uint32_t* used = smem + maxw;
  const int len = pv.tokens[seg];
  const int n = windows_of(len, W);
  uint32_t* gp = pv.pages + size_t(seg) * maxw;
  for (int w = threadIdx.x; w < maxw; w += blockDim.x) pages[w] = gp[w];
  for (int i = threadIdx.x; i < words; i += blockDim.x) used[i] = 0u;
  __syncthreads();
  for (int w = threadIdx.x; w < maxw; w += blockDim.x) {
    const uint32_t e = pages[w];
    if (promote) {
      if (pe_tier(e) == TIER_F && w < n) {
        const int sl = pe_bslot(e);
        if (sl < nslots) atomicOr(&used[sl >> 5], 1u << (sl & 31));
      }
    } else if (pe_tier(e) != TIER_E && pe_has_ledger(e)) {
      const int sl = pe_lslot(e);
      if (sl < nslots) atomicOr(&used[sl >> 5], 1u << (sl & 31));
    }
  }
  __syncthreads();
  WorkItem* work = reinterpret_cast<WorkItem*>(pv.work + pv.work_items) + size_t(b) * maxw;
  if (threadIdx.x == 0) {
    int cnt = counts[b];
    int errs = 0;
    const int cap = stride < maxw ? stride : maxw;
    if (cnt < 0) cnt = 0;
    if (cnt > cap) {
      cnt = cap;
      errs |= KV_ERR_ITEM_RANGE;
    }
    for (int i = 0; i < cnt; ++i) {
      const int w = items[size_t(b) * stride + i];
      WorkItem it{w, -1, -1, 0};
      if (w < 0 || w >= n) {
        errs |= KV_ERR_ITEM_RANGE;
      } else {
        const uint32_t e = pages[w];
        if (!promote) {
          if (pe_tier(e) != TIER_F || (w + 1) * W > len) {
            errs |= KV_ERR_DEMOTE_STATE;
          } else if (pe_has_ledger(e)) {
            pages[w] = pe_make(TIER_Q, true, 0, pe_lslot(e));
            it.flag = 2;
          } else {
            const int j = find_free(used, nslots);
            if (j < 0) {
              errs |= KV_ERR_NO_LEDGER_SLOT;
            } else {
              pages[w] = pe_make(TIER_Q, true, 0, j);
              it = WorkItem{w, pe_bslot(e), j, 1};
            }
          }
        } else {
          if (pe_tier(e) != TIER_Q || !pe_has_ledger(e)) {
            errs |= KV_ERR_PROMOTE_STATE;
          } else {
            const int j = find_free(used, nslots);
            if (j < 0) {
              errs |= KV_ERR_NO_BF16_SLOT;
            } else {
              pages[w] = pe_make(TIER_F, true, j, pe_lslot(e));
              it = WorkItem{w, pe_lslot(e), j, 1};
            }
          }
        }
      }
      work[i] = it;
    }
    pv.work[pv.work_counts + b] = cnt;
    if (errs) set_err(pv.err, errs);
  }
  __syncthreads();
  for (int w = threadIdx.x; w < maxw; w += blockDim.x) gp[w] = pages[w];
}

__global__ __launch_bounds__(256) void quantize_kernel(PoolView pv, int layer, int cap) {
  __shared__ uint8_t codes[256 * 128];
  const int kvh = blockIdx.y, W = pv.W, D = pv.D;
  const EntryLayout L(W, D);
  const WorkItem* work = reinterpret_cast<const WorkItem*>(pv.work + pv.work_items);
  for (int k = blockIdx.x; k < pv.B * cap; k += gridDim.x) {
    const int b = k / cap, i = k % cap;
    if (i >= pv.work[pv.work_counts + b]) continue;
    const WorkItem it = work[size_t(b) * pv.maxw + i];
    if (it.flag != 1) continue;
    const int seg = layer * pv.B + b;
    const uint16_t* K = pv.block(seg, it.src, kvh);
    const uint16_t* V = K + size_t(W) * D;
    uint8_t* E = pv.entry(seg, it.dst, kvh);
    uint16_t* ks = reinterpret_cast<uint16_t*>(E + L.ks);
    uint16_t* km = reinterpret_cast<uint16_t*>(E + L.km);
    uint16_t* vs = reinterpret_cast<uint16_t*>(E + L.vs);
    uint16_t* vm = reinterpret_cast<uint16_t*>(E + L.vm);
    // K: one group per (32-token block j, channel d)
    for (int g = threadIdx.x; g < (W / 32) * D; g += blockDim.x) {
      const int j = g / D, d = g % D;
      float x[32];
      uint8_t c[32];
#pragma unroll
      for (int t = 0; t < 32; ++t) x[t] = bf16_to_f32(K[size_t(32 * j + t) * D + d]);
      quant_group(x, c, ks + j * D + d, km + j * D + d);
#pragma unroll
      for (int t = 0; t < 32; ++t) codes[(32 * j + t) * D + d] = c[t];
    }
    __syncthreads();
    for (int p = threadIdx.x; p < W * D / 16; p += blockDim.x) {
      uint32_t word = 0;
#pragma unroll
      for (int e = 0; e < 16; ++e) word |= uint32_t(codes[16 * p + e]) << (2 * e);
      reinterpret_cast<uint32_t*>(E + L.kc)[p] = word;
    }
    __syncthreads();
    // V: one group per (token t, 32-channel block jj)
    const int vg = D / 32;
    for (int g = threadIdx.x; g < W * vg; g += blockDim.x) {
      const int t = g / vg, jj = g % vg;
      float x[32];
      uint8_t c[32];
      const uint4* src = reinterpret_cast<const uint4*>(V + size_t(t) * D + 32 * jj);
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const uint4 u = src[q];
        const uint32_t ww[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          x[8 * q + 2 * r] = __uint_as_float(ww[r] << 16);
          x[8 * q + 2 * r + 1] = __uint_as_float(ww[r] & 0xFFFF0000u);
        }
      }
      quant_group(x, c, vs + t * vg + jj, vm + t * vg + jj);
#pragma unroll
      for (int e = 0; e < 32; ++e) codes[t * D + 32 * jj + e] = c[e];
    }
    __syncthreads();
    for (int p = threadIdx.x; p < W * D / 16; p += blockDim.x) {
      uint32_t word = 0;
#pragma unroll
      for (int e = 0; e < 16; ++e) word |= uint32_t(codes[16 * p + e]) << (2 * e);
      reinterpret_cast<uint32_t*>(E + L.vc)[p] = word;
    }
    __syncthreads();
  }
}

// Promote: bf16_rne(fmaf(c, s, m)) for every value of the window.
__global__ __launch_bounds__(256) void dequant_kernel(PoolView pv, int layer, int cap) {
  const int kvh = blockIdx.y, W = pv.W, D = pv.D;
  const EntryLayout L(W, D);
  const WorkItem* work = reinterpret_cast<const WorkItem*>(pv.work + pv.work_items);
  for (int k = blockIdx.x; k < pv.B * cap; k += gridDim.x) {
    const int b = k / cap, i = k % cap;
    if (i >= pv.work[pv.work_counts + b]) continue;
    const WorkItem it = work[size_t(b) * pv.maxw + i];
    if (it.flag != 1) continue;
    const int seg = layer * pv.B + b;
    const uint8_t* E = pv.entry(seg, it.src, kvh);
    uint16_t* K = pv.block(seg, it.dst, kvh);
    uint16_t* V = K + size_t(W) * D;
    const uint16_t* ks = reinterpret_cast<const uint16_t*>(E + L.ks);
    const uint16_t* km = reinterpret_cast<const uint16_t*>(E + L.km);
    const uint16_t* vs = reinterpret_cast<const uint16_t*>(E + L.vs);
    const uint16_t* vm = reinterpret_cast<const uint16_t*>(E + L.vm);
    // 8 consecutive values (16 B of bf16, one 16-bit code word) per thread step
    for (int idx = threadIdx.x; idx < W * D / 8; idx += blockDim.x) {
      const int t = idx / (D / 8), d0 = 8 * (idx % (D / 8));
      const uint32_t kw = reinterpret_cast<const uint16_t*>(E + L.kc)[idx];
      const uint32_t vw = reinterpret_cast<const uint16_t*>(E + L.vc)[idx];
      const float vsc = float(__builtin_bit_cast(_Float16, vs[t * (D / 32) + d0 / 32]));
      const float vmn = float(__builtin_bit_cast(_Float16, vm[t * (D / 32) + d0 / 32]));
      uint32_t ko[4], vo[4];
#pragma unroll
      for (int e = 0; e < 8; e += 2) {
        float kk[2], vv[2];
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          const int d = d0 + e + h;
          const float s = float(__builtin_bit_cast(_Float16, ks[(t / 32) * D + d]));
          const float m = float(__builtin_bit_cast(_Float16, km[(t / 32) * D + d]));
          kk[h] = __builtin_fmaf(float((kw >> (2 * (e + h))) & 3u), s, m);
          vv[h] = __builtin_fmaf(float((vw >> (2 * (e + h))) & 3u), vsc, vmn);
        }
        ko[e / 2] = uint32_t(f32_to_bf16_rne(kk[0])) | (uint32_t(f32_to_bf16_rne(kk[1])) << 16);
        vo[e / 2] = uint32_t(f32_to_bf16_rne(vv[0])) | (uint32_t(f32_to_bf16_rne(vv[1])) << 16);
      }
      *reinterpret_cast<uint4*>(K + size_t(t) * D + d0) = make_uint4(ko[0], ko[1], ko[2], ko[3]);
      *reinterpret_cast<uint4*>(V + size_t(t) * D + d0) = make_uint4(vo[0], vo[1], vo[2], vo[3]);
    }
  }
}

static hipError_t launch_transition(const PoolView& pv, int layer, const int32_t* items, int stride,
                                    const int32_t* counts, bool promote, hipStream_t s) {
  const int nslots = promote ? pv.nb : pv.nl;
  const size_t shm = size_t(pv.maxw) * 4 + size_t((nslots + 31) / 32) * 4;
  hipLaunchKernelGGL(plan_kernel, dim3(pv.B), dim3(256), shm, s, pv, layer, items, stride, counts,
                     int(promote));
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int cap = stride < pv.maxw ? stride : pv.maxw;
  if (cap <= 0) return hipSuccess;
  int grid = pv.B * cap;
  if (grid > 1024) grid = 1024;
  if (promote)
    hipLaunchKernelGGL(dequant_kernel, dim3(grid, pv.Hkv), dim3(256), 0, s, pv, layer, cap);
  else
    hipLaunchKernelGGL(quantize_kernel, dim3(grid, pv.Hkv), dim3(256), 0, s, pv, layer, cap);
  return hipGetLastError();
}

hipError_t launch_demote(const PoolView& pv, int layer, const int32_t* items, int stride,
                         const int32_t* counts, hipStream_t s) {
  return launch_transition(pv, layer, items, stride, counts, false, s);
}

hipError_t launch_promote(const PoolView& pv, int layer, const int32_t* items, int stride,
                          const int32_t* counts, hipStream_t s) {
  return launch_transition(pv, layer, items, stride, counts, true, s);
}

// ---------------------------------------------------------------- read-back
__global__ __launch_bounds__(256) void read_kernel(PoolView pv, int layer, int b, int w, int ledger,
                                                   uint8_t* dst) {
  const int seg = layer * pv.B + b;
  const uint32_t e = (w >= 0 && w < pv.maxw) ? pv.pages[size_t(seg) * pv.maxw + w] : 0u;
  const size_t per = ledger ? size_t(3 * pv.W * pv.D / 4) : size_t(4 * pv.W * pv.D);
  const bool ok = ledger ? (pe_tier(e) != TIER_E && pe_has_ledger(e)) : (pe_tier(e) == TIER_F);
  if (!ok && threadIdx.x == 0) set_err(pv.err, KV_ERR_READ_MISSING);
  for (int kvh = 0; kvh < pv.Hkv; ++kvh) {
    const uint8_t* src = ok ? (ledger ? pv.entry(seg, pe_lslot(e), kvh)
                                      : reinterpret_cast<const uint8_t*>(pv.block(seg, pe_bslot(e), kvh)))
                            : nullptr;
    for (size_t i = threadIdx.x; i < per / 16; i += blockDim.x) {
      uint4 x = make_uint4(0, 0, 0, 0);
      if (ok) x = reinterpret_cast<const uint4*>(src)[i];
      reinterpret_cast<uint4*>(dst + kvh * per)[i] = x;
    }
  }
}

hipError_t launch_read(const PoolView& pv, int layer, int b, int window, bool ledger, void* dst,
                       hipStream_t s) {
  hipLaunchKernelGGL(read_kernel, dim3(1), dim3(256), 0, s, pv, layer, b, window, int(ledger),
                     static_cast<uint8_t*>(dst));
  return hipGetLastError();
}

}  // namespace kvtier
