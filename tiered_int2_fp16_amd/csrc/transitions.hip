// Window transitions for gfx950: prefill, demote (b-bit quantise into the
// write-once ledger, b = 2, 4 or 8), promote (dequantise back to bf16),
// canonical read-back.
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
#include "layout.h"

namespace kvtier {

// ------------------------------------------------------------------ prefill
// One workgroup per (window, kv head, sequence): the window's tokens, read in
// the caller's [token][dim] order, are written in the tile layout of layout.h.
__global__ __launch_bounds__(256) void prefill_kernel(PoolView pv, int layer, const uint16_t* k,
                                                      const uint16_t* v, int T, const float* prior) {
  const int w = blockIdx.x, kvh = blockIdx.y, b = blockIdx.z;
  const int seg = layer * pv.B + b;
  const int D = pv.D, W = pv.W, n = windows_of(T, W);
  uint16_t* blk = pv.block(seg, w, kvh);
  const size_t src = (size_t(b) * pv.Hkv + kvh) * size_t(T) * D;
  const int per_tile = 4 * D;  // 16-byte chunks per part per tile
  for (int idx = threadIdx.x; idx < (W / 32) * 2 * per_tile; idx += blockDim.x) {
    const int tile = idx / (2 * per_tile), rem = idx % (2 * per_tile);
    const bool is_v = rem >= per_tile;
    const int c = is_v ? rem - per_tile : rem;
    const int cmb = c >> 6, lane = c & 63;
    uint32_t word[4];
#pragma unroll
    for (int e2 = 0; e2 < 4; ++e2) {
      uint32_t pair = 0;
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        int t, d;
        if (is_v) layout::v_chunk_elem(cmb, lane, 2 * e2 + h, &t, &d);
        else layout::k_chunk_elem(cmb, lane, 2 * e2 + h, D, &t, &d);
        const int pos = w * W + tile * 32 + t;
        const uint16_t x = pos < T ? (is_v ? v : k)[src + size_t(pos) * D + d] : uint16_t(0);
        pair |= uint32_t(x) << (16 * h);
      }
      word[e2] = pair;
    }
    *reinterpret_cast<uint4*>(blk + size_t(tile) * 64 * D + (is_v ? 32 * D : 0) + size_t(c) * 8) =
        make_uint4(word[0], word[1], word[2], word[3]);
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
// One group of 32 values: asymmetric min/max with L = 2^b - 1 levels.
// Signed zeros are made +0, s = fp16((max - min) / L), m = fp16(min); codes
// use the stored fp16 values: c = clamp(rint_even((x - m) / s), 0, L), or 0
// when s == 0.  float32 IEEE arithmetic throughout (correctly rounded divide,
// no contraction).
template <int BITS>
__device__ inline void quant_group(const float* xp, int xstride, uint8_t* cp, int cstride, uint16_t* s_out,
                                   uint16_t* m_out) {
  constexpr float kTop = float((1 << BITS) - 1);
  float x[32];
#pragma unroll
  for (int i = 0; i < 32; ++i) {
    const float v = xp[i * xstride];
    x[i] = (v == 0.f) ? 0.f : v;
  }
  float mn = x[0], mx = x[0];
#pragma unroll
  for (int i = 1; i < 32; ++i) {
    mn = fminf(mn, x[i]);
    mx = fmaxf(mx, x[i]);
  }
  const float d = mx - mn;
  const float s32 = __fdiv_rn(d, kTop);
  const _Float16 hs = (_Float16)s32;
  const _Float16 hm = (_Float16)mn;
  const float s = (float)hs, m = (float)hm;
  // rint(fl(u / s)) from u * rcp(s).  Only the ties k + 1/2 (k < L) decide
  // a code (the clamp absorbs the rest), and the two quotients differ by
  // under 2e-7 relative (rcp within one ulp, one rounding of the product),
  // so the codes agree unless a quotient r lies within 1e-5 * (1 + r) of
  // some k + 1/2: such values are redone with the exact division in a
  // separate, rolled loop (it runs rarely; kept out of line, its code is not
  // fetched with the common path).
  const float rcp = s == 0.f ? 0.f : __builtin_amdgcn_rcpf(s);
  uint32_t near = 0;
#pragma unroll
  for (int i = 0; i < 32; ++i) {
    const float r = (x[i] - m) * rcp;
    near |= uint32_t(s != 0.f && fabsf(r - floorf(r) - 0.5f) < 1e-5f * (1.f + fabsf(r))) << i;
    cp[i * cstride] = uint8_t(fminf(fmaxf(rintf(r), 0.f), kTop));
  }
  while (near) {
    const int i = __builtin_ctz(near);
    near &= near - 1;
    const float v = xp[i * xstride];
    const float u = ((v == 0.f) ? 0.f : v) - m;
    cp[i * cstride] = uint8_t(fminf(fmaxf(rintf(__fdiv_rn(u, s)), 0.f), kTop));
  }
  *s_out = __builtin_bit_cast(uint16_t, hs);
  *m_out = __builtin_bit_cast(uint16_t, hm);
}

// ------------------------------------------------------------------ demote
struct WorkItem {
  int w, src, dst, flag;  // flag 1: move bytes; 2: tier flip only; 0: invalid
};

// Lowest free slot at or after word *cursor (slots are taken in ascending
// order, so the words before the cursor are full); marks it used.
__device__ inline int take_free(uint32_t* bits, int nbits, int* cursor) {
  for (int word = *cursor; word * 32 < nbits; ++word) {
    const uint32_t x = ~bits[word];
    if (x) {
      const int j = word * 32 + __builtin_ctz(x);
      if (j >= nbits) return -1;
      bits[word] |= 1u << (j & 31);
      *cursor = word;
      return j;
    }
  }
  *cursor = (nbits + 31) / 32;
  return -1;
}

// promote == false: demote plan (ledger slots); true: promote plan (bf16 slots).
// One workgroup per sequence.  The page table, the occupied-slot bitmap and
// the item list are staged in LDS; items are then validated and given slots
// in list order (the lowest free slot each), and the page table is written
// back.
__global__ __launch_bounds__(256) void plan_kernel(PoolView pv, int layer, const int32_t* items, int stride,
                                                   const int32_t* counts, int promote) {
  extern __shared__ uint32_t smem[];
  const int b = blockIdx.x, seg = layer * pv.B + b, tid = threadIdx.x;
  const int maxw = pv.maxw, W = pv.W;
  const int nslots = promote ? pv.nb : pv.nl;
  const int words = (nslots + 31) / 32;
  const int cap = stride < maxw ? stride : maxw;
  uint32_t* pages = smem;                                         // [maxw]
  uint32_t* used = smem + maxw;                                   // [words]
  int32_t* item_w = reinterpret_cast<int32_t*>(used + words);    // [cap]
  const int len = pv.tokens[seg];
  const int n = windows_of(len, W);
  uint32_t* gp = pv.pages + size_t(seg) * maxw;
  int cnt = counts[b];
  int errs = 0;
  if (cnt < 0) cnt = 0;
  if (cnt > cap) {
    cnt = cap;
    errs |= KV_ERR_ITEM_RANGE;
  }
  for (int w = tid; w < maxw; w += blockDim.x) pages[w] = gp[w];
  for (int i = tid; i < words; i += blockDim.x) used[i] = 0u;
  for (int i = tid; i < cnt; i += blockDim.x) item_w[i] = items[size_t(b) * stride + i];
  __syncthreads();
  for (int w = tid; w < maxw; w += blockDim.x) {
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
  if (tid == 0) {
    int cursor = 0;
    for (int i = 0; i < cnt; ++i) {
      const int w = item_w[i];
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
            const int j = take_free(used, nslots, &cursor);
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
            const int j = take_free(used, nslots, &cursor);
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
  for (int w = tid; w < maxw; w += blockDim.x) gp[w] = pages[w];
}

// The data kernels walk units (item, kv head, 32-token tile) of sequence
// blockIdx.y; a workgroup takes units blockIdx.x, blockIdx.x + gridDim.x, ...
// up to the planned item count, so a launch sized for the largest possible
// list costs little when the list is short.

// Demote data kernel: quantise one tile of a bf16 window into its ledger
// entry.  K groups are the tile's channels (32 tokens each), V groups each
// token's 32-channel blocks.
// (D, the head dimension, and BITS, the code width, are template parameters:
// the chunk and field index arithmetic below then reduces to shifts and masks)
template <int D, int BITS>
__global__ __launch_bounds__(256) void quantize_kernel(PoolView pv, int layer) {
  __shared__ float xs[2][32][129];          // K, V of one tile, canonical [token][dim]
  __shared__ uint8_t cs[2][32][132];        // their codes (rows padded: no bank conflicts)
  const int b = blockIdx.y, tid = threadIdx.x, W = pv.W, TPW = W / 32;
  const int seg = layer * pv.B + b;
  const layout::LedgerTile LT(D, BITS);
  const WorkItem* work = reinterpret_cast<const WorkItem*>(pv.work + pv.work_items) + size_t(b) * pv.maxw;
  // the first unit's work item is read together with the count (the item
  // list always has room for it; it is used only if the count covers it)
  const WorkItem first = work[blockIdx.x / (pv.Hkv * TPW)];
  const int units = pv.work[pv.work_counts + b] * pv.Hkv * TPW;
  for (int u = blockIdx.x; u < units; u += gridDim.x) {
    const int i = u / (pv.Hkv * TPW), r = u % (pv.Hkv * TPW), kvh = r / TPW, tile = r % TPW;
    const WorkItem it = u == int(blockIdx.x) ? first : work[i];
    if (it.flag != 1) continue;
    const uint16_t* tb = pv.block(seg, it.src, kvh) + size_t(tile) * 64 * D;
    uint8_t* et = pv.entry(seg, it.dst, kvh) + size_t(tile) * LT.bytes;
    // the tile's 16-byte chunks, all requested first, into the canonical layout
    constexpr int kMaxChunks = 4;   // 8 * D / 256 for D <= 128
    uint4 qv[kMaxChunks];
#pragma unroll
    for (int j = 0; j < kMaxChunks; ++j) {
      const int c = tid + j * 256;
      if (c < 8 * D) qv[j] = reinterpret_cast<const uint4*>(tb)[c];
    }
#pragma unroll
    for (int j = 0; j < kMaxChunks; ++j) {
      const int c = tid + j * 256;
      if (c >= 8 * D) break;
      const int part = c / (4 * D), cc = c % (4 * D), cmb = cc >> 6, lane = cc & 63;
      const uint4 q = qv[j];
      const uint32_t w4[4] = {q.x, q.y, q.z, q.w};
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        int t, d;
        if (part) layout::v_chunk_elem(cmb, lane, e, &t, &d);
        else layout::k_chunk_elem(cmb, lane, e, D, &t, &d);
        xs[part][t][d] = __uint_as_float((e & 1) ? (w4[e >> 1] & 0xFFFF0000u) : (w4[e >> 1] << 16));
      }
    }
    __syncthreads();
    uint16_t* ks = reinterpret_cast<uint16_t*>(et + LT.ks);
    uint16_t* km = reinterpret_cast<uint16_t*>(et + LT.km);
    uint16_t* vs = reinterpret_cast<uint16_t*>(et + LT.vs);
    uint16_t* vm = reinterpret_cast<uint16_t*>(et + LT.vm);
    for (int g = tid; g < D + D; g += blockDim.x) {
      if (g < D)   // K group: channel g over the tile's 32 tokens
        quant_group<BITS>(&xs[0][0][g], 129, &cs[0][0][g], 132, ks + g, km + g);
      else {       // V group: token t, channels 32j..32j+31
        const int t = (g - D) / (D / 32), j = (g - D) % (D / 32);
        quant_group<BITS>(&xs[1][t][32 * j], 1, &cs[1][t][32 * j], 1, vs + j * 32 + t, vm + j * 32 + t);
      }
    }
    __syncthreads();
    // pack: one 32-bit code word per thread step (64 lanes x BITS*D/64 words
    // per part, 32/BITS fields per word)
    constexpr int CWB = BITS * D / 64;
    constexpr int words = 64 * CWB;
    for (int x = tid; x < 2 * words; x += blockDim.x) {
      const bool is_v = x >= words;
      const int q = is_v ? x - words : x;
      const int lane = q / CWB, w = q % CWB;
      uint32_t word = 0;
#pragma unroll
      for (int f = 0; f < 32 / BITS; ++f) {
        int cmb, e, t, d;
        layout::field_elem_b(BITS, w, f, &cmb, &e);
        if (is_v) layout::v_chunk_elem(cmb, lane, e, &t, &d);
        else layout::k_chunk_elem(cmb, lane, e, D, &t, &d);
        word |= uint32_t(cs[is_v][t][d]) << (BITS * f);
      }
      reinterpret_cast<uint32_t*>(et + (is_v ? LT.vc : LT.kc))[lane * CWB + w] = word;
    }
    __syncthreads();
  }
}

// Promote data kernel: bf16_rne(fmaf(c, s, m)) for every value of one tile.
// A ledger chunk (lane, cmb) and the bf16 chunk (cmb, lane) hold the same 8
// values, so each thread step turns one chunk's codes (one or two code words)
// into one 16-byte chunk; the tile's scale block is staged in LDS first.
template <int D, int BITS>
__global__ __launch_bounds__(256) void dequant_kernel(PoolView pv, int layer) {
  __shared__ uint4 s_sc[64];   // Ks | Km | Vs | Vm of one tile (8 D bytes, D <= 128)
  const int b = blockIdx.y, tid = threadIdx.x, W = pv.W, TPW = W / 32;
  const int seg = layer * pv.B + b;
  const layout::LedgerTile LT(D, BITS);
  constexpr uint32_t kMask = (1u << BITS) - 1u;
  const WorkItem* work = reinterpret_cast<const WorkItem*>(pv.work + pv.work_items) + size_t(b) * pv.maxw;
  // the first unit's work item is read together with the count (used only if
  // the count covers it)
  const WorkItem first = work[blockIdx.x / (pv.Hkv * TPW)];
  const int units = pv.work[pv.work_counts + b] * pv.Hkv * TPW;
  const _Float16* ks = reinterpret_cast<const _Float16*>(s_sc);
  const _Float16* km = ks + D;
  const _Float16* vs = ks + 2 * D;
  const _Float16* vm = ks + 3 * D;
  for (int u = blockIdx.x; u < units; u += gridDim.x) {
    const int i = u / (pv.Hkv * TPW), r = u % (pv.Hkv * TPW), kvh = r / TPW, tile = r % TPW;
    const WorkItem it = u == int(blockIdx.x) ? first : work[i];
    if (it.flag != 1) continue;
    const uint8_t* et = pv.entry(seg, it.src, kvh) + size_t(tile) * LT.bytes;
    uint16_t* tb = pv.block(seg, it.dst, kvh) + size_t(tile) * 64 * D;
    // every load of the tile before the barrier: the scale block and the
    // code word of each of this thread's chunks
    if (tid < D / 2) s_sc[tid] = reinterpret_cast<const uint4*>(et + LT.ks)[tid];
    constexpr int kMaxChunks = 4;   // 8 * D / 256 for D <= 128
    uint32_t words[kMaxChunks], words_hi[kMaxChunks];   // a chunk's code words (8 bits: two)
#pragma unroll
    for (int j = 0; j < kMaxChunks; ++j) {
      const int c = tid + j * 256;
      if (c < 8 * D) {
        const bool is_v = c >= 4 * D;
        const int cc = is_v ? c - 4 * D : c, cmb = cc >> 6, lane = cc & 63;
        int wb, bit;
        layout::code_pos(cmb, lane, 0, D, BITS, &wb, &bit);
        const uint32_t* cw = reinterpret_cast<const uint32_t*>(et + (is_v ? LT.vc : LT.kc) + wb);
        words[j] = cw[0];
        words_hi[j] = BITS == 8 ? cw[1] : 0u;
      }
    }
    __syncthreads();
#pragma unroll
    for (int j = 0; j < kMaxChunks; ++j) {
      const int c = tid + j * 256;
      if (c >= 8 * D) break;
      const bool is_v = c >= 4 * D;
      const int cc = is_v ? c - 4 * D : c, cmb = cc >> 6, lane = cc & 63;
      uint32_t out[4];
#pragma unroll
      for (int e2 = 0; e2 < 4; ++e2) {
        uint32_t pair = 0;
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          const int e = 2 * e2 + h;
          int wb, bit;
          layout::code_pos(cmb, lane, e, D, BITS, &wb, &bit);
          const uint32_t word = (BITS == 8 && e >= 4) ? words_hi[j] : words[j];
          const float code = float((word >> bit) & kMask);
          int t, d;
          float sc, mn;
          if (is_v) {
            layout::v_chunk_elem(cmb, lane, e, &t, &d);
            sc = float(vs[(d >> 5) * 32 + t]);
            mn = float(vm[(d >> 5) * 32 + t]);
          } else {
            layout::k_chunk_elem(cmb, lane, e, D, &t, &d);
            sc = float(ks[d]);
            mn = float(km[d]);
          }
          pair |= uint32_t(f32_to_bf16_rne(__builtin_fmaf(code, sc, mn))) << (16 * h);
        }
        out[e2] = pair;
      }
      reinterpret_cast<uint4*>(tb + (is_v ? 32 * D : 0))[cc] = make_uint4(out[0], out[1], out[2], out[3]);
    }
    __syncthreads();
  }
}

static hipError_t launch_transition(const PoolView& pv, int layer, const int32_t* items, int stride,
                                    const int32_t* counts, bool promote, hipStream_t s) {
  const int nslots = promote ? pv.nb : pv.nl;
  const int cap = stride < pv.maxw ? stride : pv.maxw;
  const size_t shm = (size_t(pv.maxw) + size_t((nslots + 31) / 32) + size_t(cap > 0 ? cap : 0)) * 4;
  hipLaunchKernelGGL(plan_kernel, dim3(pv.B), dim3(256), shm, s, pv, layer, items, stride, counts,
                     int(promote));
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  if (cap <= 0) return hipSuccess;
  // about 1024 workgroups in all, never more than the largest unit count
  const long max_units = long(cap) * pv.Hkv * (pv.W / 32);
  long gx = (1024 + pv.B - 1) / pv.B;
  if (gx > max_units) gx = max_units;
  if (gx < 1) gx = 1;
  const int wi = pv.lbits == 2 ? 0 : (pv.lbits == 4 ? 1 : 2);
  const int di = pv.D == 64 ? 0 : 1;
  typedef void (*Kern)(PoolView, int);
  static const Kern kDequant[2][3] = {{dequant_kernel<64, 2>, dequant_kernel<64, 4>, dequant_kernel<64, 8>},
                                      {dequant_kernel<128, 2>, dequant_kernel<128, 4>, dequant_kernel<128, 8>}};
  static const Kern kQuant[2][3] = {{quantize_kernel<64, 2>, quantize_kernel<64, 4>, quantize_kernel<64, 8>},
                                    {quantize_kernel<128, 2>, quantize_kernel<128, 4>, quantize_kernel<128, 8>}};
  hipLaunchKernelGGL(promote ? kDequant[di][wi] : kQuant[di][wi], dim3(unsigned(gx), pv.B), dim3(256), 0, s, pv,
                     layer);
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
// Canonical copies for inspection: bf16 K then V [kv_head][2][W][D]; ledger
// entries as Kc, Vc [W][D*b/8] (b-bit code of (t, d) in byte d*b/8, bits
// (d*b)%8 .. +b-1), Ks, Km fp16 [W/32][D], Vs, Vm fp16 [W][D/32].
__global__ __launch_bounds__(256) void read_kernel(PoolView pv, int layer, int b, int w, int ledger,
                                                   uint8_t* dst) {
  const int seg = layer * pv.B + b, W = pv.W, D = pv.D;
  const uint32_t e = (w >= 0 && w < pv.maxw) ? pv.pages[size_t(seg) * pv.maxw + w] : 0u;
  const bool ok = ledger ? (pe_tier(e) != TIER_E && pe_has_ledger(e)) : (pe_tier(e) == TIER_F);
  if (!ok && threadIdx.x == 0) set_err(pv.err, KV_ERR_READ_MISSING);
  const int BITS = pv.lbits, per = 8 / BITS, row = D * BITS / 8;   // codes per byte, bytes per row
  const layout::LedgerTile LT(D, BITS);
  for (int kvh = 0; kvh < pv.Hkv; ++kvh) {
    if (!ledger) {
      uint16_t* out = reinterpret_cast<uint16_t*>(dst) + size_t(kvh) * 2 * W * D;
      const uint16_t* blk = ok ? pv.block(seg, pe_bslot(e), kvh) : nullptr;
      for (int x = threadIdx.x; x < W * D; x += blockDim.x) {
        const int t = x / D, d = x % D;
        out[x] = ok ? blk[layout::bf16_window_k(t, d, D)] : uint16_t(0);
        out[W * D + x] = ok ? blk[layout::bf16_window_v(t, d, D)] : uint16_t(0);
      }
    } else {
      uint8_t* out = dst + size_t(kvh) * (size_t(BITS + 1) * W * D / 4);
      const uint8_t* E = ok ? pv.entry(seg, pe_lslot(e), kvh) : nullptr;
      uint8_t* kc = out;
      uint8_t* vc = out + W * row;
      uint16_t* ks = reinterpret_cast<uint16_t*>(out + 2 * W * row);
      uint16_t* km = ks + (W / 32) * D;
      uint16_t* vs = km + (W / 32) * D;
      uint16_t* vm = vs + W * (D / 32);
      const uint32_t mask = (1u << BITS) - 1u;
      for (int x = threadIdx.x; x < W * row; x += blockDim.x) {
        const int t = x / row, d0 = per * (x % row);
        uint32_t kb = 0, vb = 0;
        if (ok) {
          const uint8_t* et = E + size_t(t / 32) * LT.bytes;
          for (int q = 0; q < per; ++q) {
            int wb, bit;
            layout::k_code_pos(t % 32, d0 + q, D, BITS, &wb, &bit);
            kb |= ((*reinterpret_cast<const uint32_t*>(et + LT.kc + wb) >> bit) & mask) << (BITS * q);
            layout::v_code_pos(t % 32, d0 + q, D, BITS, &wb, &bit);
            vb |= ((*reinterpret_cast<const uint32_t*>(et + LT.vc + wb) >> bit) & mask) << (BITS * q);
          }
        }
        kc[x] = uint8_t(kb);
        vc[x] = uint8_t(vb);
      }
      for (int x = threadIdx.x; x < (W / 32) * D; x += blockDim.x) {
        const int tile = x / D, d = x % D;
        const uint8_t* et = ok ? E + size_t(tile) * LT.bytes : nullptr;
        ks[x] = ok ? reinterpret_cast<const uint16_t*>(et + LT.ks)[d] : uint16_t(0);
        km[x] = ok ? reinterpret_cast<const uint16_t*>(et + LT.km)[d] : uint16_t(0);
      }
      for (int x = threadIdx.x; x < W * (D / 32); x += blockDim.x) {
        const int t = x / (D / 32), j = x % (D / 32);
        const uint8_t* et = ok ? E + size_t(t / 32) * LT.bytes : nullptr;
        vs[x] = ok ? reinterpret_cast<const uint16_t*>(et + LT.vs)[j * 32 + t % 32] : uint16_t(0);
        vm[x] = ok ? reinterpret_cast<const uint16_t*>(et + LT.vm)[j * 32 + t % 32] : uint16_t(0);
      }
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
