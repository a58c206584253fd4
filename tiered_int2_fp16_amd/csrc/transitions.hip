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
// page table; a data kernel then moves the bytes of every planned item.  A
// routing event's demotions and promotions together take three: one plan
// launch for both lists, then the two data kernels (a caller may also plan
// a layer's moves ahead, on another stream, and launch its data kernels
// later).
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
// no contraction).  The sign of a zero x never changes x - m (m is never -0).
// The demote kernel decides each code by exact comparisons of x - m with
// half-way points (k + 1/2) s instead of dividing.

// ------------------------------------------------------------------ demote
struct WorkItem {
  int w, src, dst, flag;  // flag 1: move bytes; 2: tier flip only; 0: invalid
};

// A plan's item list: items int32 [batch][stride] of window indices, counts
// int32 [batch]; items == nullptr: no such list in this launch.
struct PlanList {
  const int32_t* items;
  const int32_t* counts;
  int stride;
};

// The demote plan (ledger slots), the promote plan (bf16 slots), or both in
// one launch, the demotions first: the promote plan then starts from the row
// the demote plan left, exactly as when the two are launched one after the
// other.  One workgroup per sequence.  The page-table row and the item lists
// are staged in LDS with one batch of loads; for each plan, the free-slot
// bitmap too.  A plan's outcome is that of taking its items one by one in
// list order, each valid item the lowest free slot, computed for all items
// at once:
//  - an item is checked against the row as the plan found it; a window
//    listed again after its first occurrence has the outcome of that
//    occurrence's state: after a success it has moved (a state error), after
//    a failure it fails the same way;
//  - the k-th item (in list order) that needs a slot takes the k-th free
//    slot in ascending order, and every such item from the free count on
//    finds none (no slot is freed during a plan).
// Each plan writes its work list (list 0: demotions, list 1: promotions, of
// this layer) and item count; the updated row is written back at the end.
__global__ __launch_bounds__(256) void plan_kernel(PoolView pv, int layer, PlanList dl, PlanList pl) {
  extern __shared__ uint32_t smem[];
  __shared__ int s_wsum[4];
  __shared__ int s_errs;
  const int b = blockIdx.x, seg = layer * pv.B + b, tid = threadIdx.x;
  const int lane = tid & 63, wv = tid >> 6;
  const int maxw = pv.maxw, W = pv.W;
  const int cap_d = dl.items ? min(dl.stride, maxw) : 0;
  const int cap_p = pl.items ? min(pl.stride, maxw) : 0;
  const int words_max = (max(dl.items ? pv.nl : 0, pl.items ? pv.nb : 0) + 31) / 32;
  uint32_t* pages = smem;                                             // [maxw]
  int32_t* first = reinterpret_cast<int32_t*>(pages + maxw);         // [maxw] first list position
  uint32_t* freew = reinterpret_cast<uint32_t*>(first + maxw);       // [words] free slots
  int32_t* fpc = reinterpret_cast<int32_t*>(freew + words_max);      // [words + 1] free slots before a word
  // [cap] each list's items: their windows, then each item's outcome packed
  // as window | flag << 12 | error kind << 14 | slot << 16 (flag 1: move
  // bytes, 2: tier flip only; error kind 1: window out of range, 2: state,
  // 3: no free slot)
  int32_t* item_d = fpc + words_max + 1;
  int32_t* item_p = item_d + cap_d;
  const int len = pv.tokens[seg];
  const int n = windows_of(len, W);
  const int cnt_d = dl.items ? dl.counts[b] : 0, cnt_p = pl.items ? pl.counts[b] : 0;
  uint32_t* gp = pv.pages + size_t(seg) * maxw;
  if (tid == 0) s_errs = 0;
  // the row and the item lists (their first cap entries: no wait for the
  // counts), eight entries of each per thread in flight at a time; buffer
  // loads read zeros past the ends without touching memory
  {
    const auto rp = __builtin_amdgcn_make_buffer_rsrc(gp, (short)0, maxw * 4, 0x00020000);
    const auto rd = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<int32_t*>(dl.items ? dl.items + size_t(b) * dl.stride : nullptr), (short)0, cap_d * 4,
        0x00020000);
    const auto rq = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<int32_t*>(pl.items ? pl.items + size_t(b) * pl.stride : nullptr), (short)0, cap_p * 4,
        0x00020000);
    for (int base = 0; base < maxw; base += 8 * 256) {   // (caps <= maxw)
      uint32_t rw[8], id8[8], ip8[8];
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        rw[j] = __builtin_amdgcn_raw_buffer_load_b32(rp, (base + 256 * j + tid) * 4, 0, 0);
        id8[j] = __builtin_amdgcn_raw_buffer_load_b32(rd, (base + 256 * j + tid) * 4, 0, 0);
        ip8[j] = __builtin_amdgcn_raw_buffer_load_b32(rq, (base + 256 * j + tid) * 4, 0, 0);
      }
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const int x = base + 256 * j + tid;
        if (x < maxw) pages[x] = rw[j];
        if (x < cap_d) item_d[x] = int32_t(id8[j]);
        if (x < cap_p) item_p[x] = int32_t(ip8[j]);
      }
    }
  }
  // one plan over the staged row
  auto plan = [&](int cnt, int32_t* item_w, int cap, bool promote) {
    const int nslots = promote ? pv.nb : pv.nl;
    const int words = (nslots + 31) / 32;
    if (cnt < 0) cnt = 0;
    if (cnt > cap) {
      cnt = cap;
      if (tid == 0) atomicOr(&s_errs, KV_ERR_ITEM_RANGE);
    }
    for (int i = tid; i < words; i += blockDim.x) {
      const int rest = nslots - 32 * i;
      freew[i] = rest >= 32 ? 0xFFFFFFFFu : ((1u << rest) - 1u);
    }
    for (int w = tid; w < maxw; w += blockDim.x) first[w] = 0x7FFFFFFF;
    __syncthreads();
    // occupied slots out of the free map; each window's first list position
    for (int w = tid; w < maxw; w += blockDim.x) {
      const uint32_t e = pages[w];
      int sl = -1;
      if (promote) {
        if (pe_tier(e) == TIER_F && w < n) sl = pe_bslot(e);
      } else if (pe_tier(e) != TIER_E && pe_has_ledger(e)) {
        sl = pe_lslot(e);
      }
      if (sl >= 0 && sl < nslots) atomicAnd(&freew[sl >> 5], ~(1u << (sl & 31)));
    }
    for (int i = tid; i < cnt; i += blockDim.x) {
      const int w = item_w[i];
      if (w >= 0 && w < n) atomicMin(&first[w], i);
    }
    __syncthreads();
    // free slots before each word: one wave, 64 words a pass
    if (wv == 0) {
      int run = 0;
      for (int w0 = 0; w0 < words; w0 += 64) {
        const int wd = w0 + lane;
        const int c = wd < words ? __popc(freew[wd]) : 0;
        int incl = c;
#pragma unroll
        for (int off = 1; off < 64; off <<= 1) {
          const int y = __shfl_up(incl, off, 64);
          if (lane >= off) incl += y;
        }
        if (wd < words) fpc[wd] = run + incl - c;
        run += __shfl(incl, 63, 64);
      }
      if (lane == 0) fpc[words] = run;
    }
    __syncthreads();
    const int nfree = fpc[words];
    // items in rounds of 256: validation against the row as found, rank
    // among the items that need a slot, slot
    int base = 0;
    for (int r0 = 0; r0 < cnt; r0 += 256) {
      const int i = r0 + tid;
      int need = 0, flag = 0, err = 0, slot = 0;
      if (i < cnt) {
        const int w = item_w[i];
        if (w < 0 || w >= n) {
          err = KV_ERR_ITEM_RANGE;
        } else if (first[w] == i) {
          const uint32_t e = pages[w];
          if (!promote) {
            if (pe_tier(e) != TIER_F || (w + 1) * W > len) err = KV_ERR_DEMOTE_STATE;
            else if (pe_has_ledger(e)) flag = 2;
            else need = 1;
          } else {
            if (pe_tier(e) != TIER_Q || !pe_has_ledger(e)) err = KV_ERR_PROMOTE_STATE;
            else need = 1;
          }
        }
      }
      const uint64_t bal = __ballot(need);
      if (lane == 0) s_wsum[wv] = __popcll(bal);
      __syncthreads();
      int rank = base + __popcll(bal & ((uint64_t(1) << lane) - 1));
      for (int v = 0; v < wv; ++v) rank += s_wsum[v];
      base += s_wsum[0] + s_wsum[1] + s_wsum[2] + s_wsum[3];
      __syncthreads();
      if (need) {
        if (rank < nfree) {
          // the word holding free slot number `rank`, then that slot within it
          int lo = 0, hi = words;
          while (hi - lo > 1) {
            const int mid = (lo + hi) >> 1;
            if (fpc[mid] <= rank) lo = mid;
            else hi = mid;
          }
          uint32_t x = freew[lo];
          for (int k = rank - fpc[lo]; k > 0; --k) x &= x - 1u;
          slot = 32 * lo + __builtin_ctz(x);
          flag = 1;
        } else {
          err = promote ? KV_ERR_NO_BF16_SLOT : KV_ERR_NO_LEDGER_SLOT;
        }
      }
      const int kind = err == KV_ERR_ITEM_RANGE ? 1 : (err == 0 ? 0 : (need ? 3 : 2));
      __syncthreads();   // (every thread has read its item's window above)
      if (i < cnt)
        item_w[i] = int32_t(uint32_t(kind == 1 ? 0 : item_w[i]) | (uint32_t(flag) << 12) |
                            (uint32_t(kind) << 14) | (uint32_t(slot) << 16));
    }
    __syncthreads();
    // the work list; first occurrences update the row, later ones take their
    // first occurrence's state
    const int list = promote ? 1 : 0;
    WorkItem* work =
        reinterpret_cast<WorkItem*>(pv.work + pv.work_items) + ((size_t(layer) * 2 + list) * pv.B + b) * maxw;
    const int err_state = promote ? KV_ERR_PROMOTE_STATE : KV_ERR_DEMOTE_STATE;
    const int err_slot = promote ? KV_ERR_NO_BF16_SLOT : KV_ERR_NO_LEDGER_SLOT;
    int errs = 0;
    for (int i = tid; i < cnt; i += blockDim.x) {
      const uint32_t o = uint32_t(item_w[i]);
      const int w = int(o & 0xFFFu), flag = int((o >> 12) & 3u), slot = int(o >> 16);
      int kind = int((o >> 14) & 3u);
      WorkItem it{w, -1, -1, 0};
      if (kind != 1 && first[w] != i) {
        // a later listing of the window: its first occurrence moved it (a
        // state error now), or failed, and this one fails the same way
        const uint32_t of = uint32_t(item_w[first[w]]);
        kind = ((of >> 12) & 3u) ? 2 : int((of >> 14) & 3u);
      } else if (flag) {
        const uint32_t e = pages[w];
        if (!promote) {
          if (flag == 2) {
            pages[w] = pe_make(TIER_Q, true, 0, pe_lslot(e));
            it.flag = 2;
          } else {
            pages[w] = pe_make(TIER_Q, true, 0, slot);
            it = WorkItem{w, pe_bslot(e), slot, 1};
          }
        } else {
          pages[w] = pe_make(TIER_F, true, slot, pe_lslot(e));
          it = WorkItem{w, pe_lslot(e), slot, 1};
        }
      }
      errs |= kind == 1 ? KV_ERR_ITEM_RANGE : (kind == 2 ? err_state : (kind == 3 ? err_slot : 0));
      work[i] = it;
    }
    if (errs) atomicOr(&s_errs, errs);
    if (tid == 0) pv.work[pv.work_counts + (size_t(layer) * 2 + list) * pv.B + b] = cnt;
    __syncthreads();   // the row's updates are in before anything reads it again
  };
  if (dl.items) plan(cnt_d, item_d, cap_d, false);
  if (pl.items) plan(cnt_p, item_p, cap_p, true);
  if (tid == 0 && s_errs) set_err(pv.err, s_errs);
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
// the chunk and field index arithmetic below then reduces to shifts, masks and
// constants)
//
// Per unit (one 32-token tile of one kv head), three phases and three
// barriers, one LDS buffer (so that four workgroups fit a CU at head_dim 128;
// two buffers for alternate units, one barrier fewer, held it to three):
//  0. every thread writes its 16-byte chunks of the tile (loaded into
//     registers while the previous unit was processed) to LDS with one store
//     each: K as [token][channel], V as [channel][token];
//  1. each group's min and max from two threads (16-bit pairs of LDS rows,
//     one exchange across the wave's halves), its fp16 scale and min, and
//     the parameters of its codes published in LDS;
//  2. one thread per pair of packed code words whose values share their
//     groups reads the words' values (16-byte LDS loads) and the groups'
//     parameters, decides the codes and assembles the words in registers.
// Each code word has one writer: no atomics.  A unit's results (scales, mins,
// code words) stay in registers until the next unit has been written to LDS;
// they are then stored, just before the loads of the unit after it are
// issued, so those loads never wait behind freshly issued stores.
template <int D, int BITS>
__global__ __launch_bounds__(256, D == 128 ? 4 : 3) void quantize_kernel(PoolView pv, int layer,
                                                                        const WorkItem* __restrict__ items,
                                                                        const int32_t* __restrict__ counts) {
  constexpr int KP = D + 8;    // K rows [token][channel] (bf16), padded
  constexpr int VP = 40;       // V rows [channel][token] (bf16), padded; 8 more per 32 rows
  constexpr int CWB = BITS * D / 64;          // code words per lane per part
  constexpr int NW = 64 * CWB;                // code words per part
  constexpr int PPT = NW >= 256 ? NW / 256 : 1;   // code-word pairs per thread (NW pairs in all)
  constexpr int NCH = 8 * D / 256;            // 16-byte chunks per thread (K and V)
  constexpr int NCW = BITS == 2 ? 2 : 1;      // chunks per code word
  constexpr float kTop = float((1 << BITS) - 1);
  __shared__ __attribute__((aligned(16))) uint16_t sk[32 * KP];
  __shared__ __attribute__((aligned(16))) uint16_t sv[D * VP + (D / 32) * 8];
  // group parameters (phase 1 to phase 2): K group of channel d at d, V group
  // (token t, block j) at D + 32 j + t.  INT2: (m, s) as a float pair, the
  // thresholds formed where they are used (halving the LDS reads of phase 2:
  // plan + quantise 51.4 -> 50.4 us median over six same-box runs each);
  // 4 and 8 bits: (m, 1/s, s, s/2)
  __shared__ float4 pp[2 * D];
  auto vrow = [](int d) { return d * VP + (d >> 5) * 8; };   // (a wave's two 32-row blocks hit other banks)
  const int b = blockIdx.y, tid = threadIdx.x, W = pv.W, TPW = W / 32;
  const bool has_group = 2 * D >= 256 || tid < 2 * D;   // phase 1 threads (whole waves)
  const int seg = layer * pv.B + b;
  const layout::LedgerTile LT(D, BITS);
  const WorkItem* work = items + size_t(b) * pv.maxw;   // (not written here: scalar loads)
  const int units = counts[b] * pv.Hkv * TPW;
  const int per_item = pv.Hkv * TPW;
  // the unit's item (flag 1: move bytes; flag 0 past the list)
  auto item_of = [&](int u) { return u < units ? work[u / per_item] : WorkItem{0, 0, 0, 0}; };
  // the unit's tile chunks; a unit that moves nothing loads nothing (empty
  // resource)
  auto fetch = [&](int u, const WorkItem& it, uint4 (&qv)[NCH]) {
    const int r = u % per_item, kvh = r / TPW, tile = r % TPW;
    const uint16_t* tb = pv.block(seg, it.flag == 1 ? it.src : 0, kvh) + size_t(tile) * 64 * D;
    const auto rs = __builtin_amdgcn_make_buffer_rsrc(const_cast<uint16_t*>(tb), (short)0,
                                                      it.flag == 1 ? 128 * D : 0, 0x00020000);
#pragma unroll
    for (int j = 0; j < NCH; ++j)
      qv[j] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(rs, (tid + 256 * j) * 16, 0, 0));
  };
  // pair i of this thread: its index x among the NW pairs (K pairs first)
  // and its two code words (lane, w).  K: (lane, w) and (lane, w + CWB/2),
  // the same channels in the two 16-token halves of the tile.  V, the same
  // tokens and 32-channel block: INT2 (lane, w) and (lane + 8, w) (lane bit
  // 3 clear), 4 bits (lane, w) and (lane, w + 1) (w even), 8 bits (lane, w)
  // and (lane, w + 2) (w bit 1 clear).
  auto pair_of = [&](int i, int (&lane)[2], int (&w)[2]) {
    const int x = tid + 256 * i;
    const int y = x >= NW / 2 ? x - NW / 2 : x;
    lane[0] = lane[1] = y & 63;
    if (x < NW / 2) {
      w[0] = y >> 6;
      w[1] = w[0] + CWB / 2;
    } else if (BITS == 2) {
      lane[0] = (y & 7) | ((y & 24) << 1);
      lane[1] = lane[0] + 8;
      w[0] = w[1] = y >> 5;
    } else if (BITS == 4) {
      w[0] = 2 * (y >> 6);
      w[1] = w[0] + 1;
    } else {
      const int j = y >> 6;
      w[0] = (j & 1) | ((j >> 1) << 2);
      w[1] = w[0] + 2;
    }
    return x;
  };
  // the previous unit's results: entry tile (null: none), this thread's
  // group (g, K or V) with its fp16 scale and min, and its code words
  uint8_t* pend_et = nullptr;
  int pend_g = 0;
  bool pend_v = false;
  uint16_t pend_s = 0, pend_m = 0;
  uint32_t pend_w[2 * PPT];
  auto flush = [&]() {
    if (!pend_et) return;   // (the same for the whole workgroup)
    if (has_group) {
      reinterpret_cast<uint16_t*>(pend_et + (pend_v ? LT.vs : LT.ks))[pend_g] = pend_s;
      reinterpret_cast<uint16_t*>(pend_et + (pend_v ? LT.vm : LT.km))[pend_g] = pend_m;
    }
#pragma unroll
    for (int i = 0; i < PPT; ++i) {
      int lane[2], w[2];
      const int x = pair_of(i, lane, w);
      if (NW < 256 && x >= NW) break;
      uint32_t* cw = reinterpret_cast<uint32_t*>(pend_et + (x >= NW / 2 ? LT.vc : LT.kc));
      cw[lane[0] * CWB + w[0]] = pend_w[2 * i];
      cw[lane[1] * CWB + w[1]] = pend_w[2 * i + 1];
    }
    pend_et = nullptr;
  };

  int u = blockIdx.x;
  WorkItem it = item_of(u);
  uint4 qv[NCH];
  fetch(u, it, qv);
  for (; u < units; u += gridDim.x) {
    const WorkItem itn = item_of(u + gridDim.x);
    const bool move = it.flag == 1;   // (the same for the whole workgroup)
    __syncthreads();   // every thread is done with the previous unit's LDS data
    const int r = u % per_item, kvh = r / TPW, tile = r % TPW;
    uint8_t* et = pv.entry(seg, it.dst, kvh) + size_t(tile) * LT.bytes;
    // 0. chunks to LDS: chunk c < 4 D is K chunk (cmb, lane) = (c / 64, c % 64),
    //    8 channels of one token; the rest V chunks, 8 tokens of one channel
    if (move) {
#pragma unroll
      for (int j = 0; j < NCH; ++j) {
        const int c = tid + 256 * j;
        int t, d;
        if (256 * j < 4 * D) {
          layout::k_chunk_elem(c >> 6, c & 63, 0, D, &t, &d);
          *reinterpret_cast<uint4*>(&sk[t * KP + d]) = qv[j];
        } else {
          layout::v_chunk_elem((c - 4 * D) >> 6, c & 63, 0, &t, &d);
          *reinterpret_cast<uint4*>(&sv[vrow(d) + t]) = qv[j];
        }
      }
    }
    flush();
    fetch(u + gridDim.x, itn, qv);   // the next unit's bytes, in flight during the rest of this one
    it = itn;
    if (!move) continue;
    __syncthreads();
    // 1. group parameters.  The first D threads take the K groups, the next D
    //    the V groups (whole waves each).  A thread reads 16 bf16 pairs: half
    //    of each of two groups (K: channels 2p, 2p + 1 over 16 tokens; V:
    //    tokens 2p', 2p' + 1 of a 32-channel block over 16 channels).  Lanes l
    //    and l ^ 32 hold the two halves; after one exchange lane l finishes
    //    the pair's first group and lane l ^ 32 its second.
    if (has_group) {
      const bool is_v = __builtin_amdgcn_readfirstlane(int(tid >= D)) != 0;   // (whole waves: scalar branches)
      const int idx = is_v ? tid - D : tid, l = idx & 63, h = l >> 5;
      const int p = (idx >> 6) * 32 + (l & 31);   // the pair, 0 .. D/2 - 1
      uint32_t x[16];
      int g;   // the group this thread finishes: K channel, or 32 j + token for V
      if (!is_v) {
        const uint32_t* src = reinterpret_cast<const uint32_t*>(sk + 16 * h * KP + 2 * p);
#pragma unroll
        for (int i = 0; i < 16; ++i) x[i] = src[i * (KP / 2)];
        g = 2 * p + h;
      } else {
        const int tp = p & 15, j = p >> 4;
        const uint32_t* src = reinterpret_cast<const uint32_t*>(sv + vrow(32 * j + 16 * h) + 2 * tp);
#pragma unroll
        for (int i = 0; i < 16; ++i) x[i] = src[i * (VP / 2)];
        g = 32 * j + 2 * tp + h;
      }
      float mn0 = INFINITY, mx0 = -INFINITY, mn1 = INFINITY, mx1 = -INFINITY;
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const float a = __uint_as_float(x[i] << 16), c = __uint_as_float(x[i] & 0xFFFF0000u);
        mn0 = fminf(mn0, a);
        mx0 = fmaxf(mx0, a);
        mn1 = fminf(mn1, c);
        mx1 = fmaxf(mx1, c);
      }
      // lane h = 0 keeps the first group and receives its partner's half of
      // it; lane h = 1 the second
      const float smn = __shfl_xor(h ? mn0 : mn1, 32, 64), smx = __shfl_xor(h ? mx0 : mx1, 32, 64);
      float mn = fminf(h ? mn1 : mn0, smn), mx = fmaxf(h ? mx1 : mx0, smx);
      mn = mn == 0.f ? 0.f : mn;   // -0 -> +0 (the extremes of the canonical values)
      mx = mx == 0.f ? 0.f : mx;
      const float s32 = __fdiv_rn(mx - mn, kTop);
      const _Float16 hs = (_Float16)s32;
      const _Float16 hm = (_Float16)mn;
      const float sc = (float)hs;
      // the parameters phase 2 reads (see there); s == 0 (all codes 0) is
      // published as m = 0 and infinite thresholds (INT2: s = inf)
      const bool zero = sc == 0.f;
      const float m = zero ? 0.f : (float)hm;
      if (BITS == 2) {
        reinterpret_cast<float2*>(pp)[is_v ? D + g : g] = make_float2(m, zero ? INFINITY : sc);
      } else {
        pp[is_v ? D + g : g] = zero ? make_float4(0.f, 0.f, INFINITY, INFINITY)
                                    : make_float4(m, __builtin_amdgcn_rcpf(sc), sc, 0.5f * sc);
      }
      pend_g = g;   // K: [channel]; V: [j][token]
      pend_v = is_v;
      pend_s = __builtin_bit_cast(uint16_t, hs);
      pend_m = __builtin_bit_cast(uint16_t, hm);
    }
    __syncthreads();
    // 2. code words, in pairs whose values share their groups (PPT pairs a
    //    thread); a wave's pairs are all K or all V.  Each chunk position of
    //    the pair reads its 8 groups' parameters once for both words.
    //    The code of x in a group (m, s) is decided exactly, without a
    //    division: with u = x - m (the oracle's float32 difference) and the
    //    half-way points t_k = (k + 1/2) s, which are exact in float32 (s is
    //    an fp16 value, k + 1/2 has at most 9 significant bits), u/s lies
    //    above, at or below k + 1/2 exactly when u lies above, at or below
    //    t_k, and its float32 rounding never crosses k + 1/2 (k + 1/2 = 1/2,
    //    where it may land on it from below, rounds to code 0 either way).
    //    Hence for INT2 c = [u > t_0] + [u >= t_1] + [u > t_2] (a tie at an
    //    odd k goes up, at an even k down: round half to even).  For 4 and 8
    //    bits the approximate code c' = rint(clamp(u rcp(s), 0, L)) is within
    //    one of the true one; the half-way points on either side of c' then
    //    decide it, a tie going to the even side, and the result is clamped.
#pragma unroll
    for (int i = 0; i < PPT; ++i) {
      int lane[2], w[2];
      const int x = pair_of(i, lane, w);
      if (NW < 256 && x >= NW) break;   // (head_dim 64, INT2: waves 2 and 3 have no pair)
      const bool is_v = __builtin_amdgcn_readfirstlane(int(x >= NW / 2)) != 0;   // (whole waves)
      uint32_t word[2] = {0u, 0u};
#pragma unroll
      for (int j = 0; j < NCW; ++j) {
        uint4 vals[2];
        int pb = 0;   // the parameter index of element 0 (elements e at pb + e)
#pragma unroll
        for (int k = 0; k < 2; ++k) {
          const int cmb = BITS == 2 ? 2 * w[k] + j : (BITS == 4 ? w[k] : w[k] >> 1);
          int t0, d0;
          if (!is_v) {
            layout::k_chunk_elem(cmb, lane[k], 0, D, &t0, &d0);   // 8 channels d0.. of token t0
            vals[k] = *reinterpret_cast<const uint4*>(&sk[t0 * KP + d0]);
            pb = d0;
          } else {
            layout::v_chunk_elem(cmb, lane[k], 0, &t0, &d0);      // 8 tokens t0.. of channel d0
            vals[k] = *reinterpret_cast<const uint4*>(&sv[vrow(d0) + t0]);
            pb = D + 32 * (d0 >> 5) + t0;
          }
        }
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          if (BITS == 8 && (e >> 2) != (w[0] & 1)) continue;   // the other half of the chunk
          float4 P;
          if (BITS == 2) {
            const float2 P2 = reinterpret_cast<const float2*>(pp)[pb + e];
            P = make_float4(P2.x, 0.5f * P2.y, 1.5f * P2.y, 2.5f * P2.y);
          } else {
            P = pp[pb + e];
          }
#pragma unroll
          for (int k = 0; k < 2; ++k) {
            const uint32_t hw = (&vals[k].x)[e >> 1];
            const float u = __uint_as_float((e & 1) ? (hw & 0xFFFF0000u) : (hw << 16)) - P.x;
            int wb, bit;
            const int cmb = BITS == 2 ? 2 * w[k] + j : (BITS == 4 ? w[k] : w[k] >> 1);
            layout::code_pos(cmb, lane[k], e, D, BITS, &wb, &bit);
            if (BITS == 2) {
              // With t0 < t1 < t2 (finite s > 0), u >= t1 implies u > t0
              // and u < t1 implies u <= t2: one comparison picks the half, a
              // second the code within it; the two bits go in as constants
              // at the field's position.  (s = 0 or inf: the thresholds are
              // all inf and a finite u gets 0 either way; u = +inf there
              // means the defining quotient u/s is inf/inf, which has no
              // code.)
              const bool up = u >= P.z;
              word[k] |= (up ? (2u << bit) : 0u) | (u > (up ? P.w : P.y) ? (1u << bit) : 0u);
            } else {
              uint32_t code;
              const float c = rintf(__builtin_amdgcn_fmed3f(u * P.y, 0.f, kTop));
              const int ci = int(c), odd = ci & 1;
              const float tlo = fmaf(c, P.z, -P.w);   // (c - 1/2) s
              const float thi = tlo + P.z;            // (c + 1/2) s
              // a tie moves an odd c to its even neighbour: compare with the
              // next float above tlo and below thi (both positive for odd c)
              const int cc = ci - int(u < __int_as_float(__float_as_int(tlo) + odd)) +
                             int(u > __int_as_float(__float_as_int(thi) - odd));
              code = uint32_t(cc < 0 ? 0 : (cc > int(kTop) ? int(kTop) : cc));
              word[k] |= code << bit;
            }
          }
        }
      }
      pend_w[2 * i] = word[0];
      pend_w[2 * i + 1] = word[1];
    }
    pend_et = et;
  }
  flush();
}

// Promote data kernel: bf16_rne(fmaf(c, s, m)) for every value of one tile.
// A ledger chunk (lane, cmb) and the bf16 chunk (cmb, lane) hold the same 8
// values, so each thread turns one chunk's codes (one or two code words) into
// one 16-byte chunk; the tile's scale block (Ks | Km | Vs | Vm, 8 D bytes) is
// staged in LDS.  A workgroup loads the code words and scale blocks of a
// batch of four units at once, then decodes and stores them one after the
// other.  The float32 results are never subnormal (c s + m is 0 or at least
// 2^-24 in magnitude: every term is a multiple of the fp16 quantum 2^-24),
// and the hardware's packed bf16 conversion rounds them to nearest even.
template <int D, int BITS>
__global__ __launch_bounds__(256) void dequant_kernel(PoolView pv, int layer, const WorkItem* __restrict__ items,
                                                     const int32_t* __restrict__ counts) {
  constexpr int NCH = 8 * D / 256;   // 16-byte chunks per thread (K chunks first, then V)
  constexpr int NWC = BITS == 8 ? 2 : 1;   // code words per chunk
  constexpr int NBU = 4;             // units whose loads go out together (a batch)
  __shared__ uint4 s_sc[NBU][D / 2];
  typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
  typedef float f32x2 __attribute__((ext_vector_type(2)));
  const int b = blockIdx.y, tid = threadIdx.x, W = pv.W, TPW = W / 32;
  const int seg = layer * pv.B + b;
  const layout::LedgerTile LT(D, BITS);
  constexpr uint32_t kMask = (1u << BITS) - 1u;
  const WorkItem* work = items + size_t(b) * pv.maxw;   // (not written here: scalar loads)
  const int units = counts[b] * pv.Hkv * TPW;
  const int per_item = pv.Hkv * TPW;
  // the unit's code words (NWC per chunk) and, for tid < D/2, 16-byte piece
  // tid of its scale block; a unit that moves nothing loads nothing
  auto fetch = [&](int u, const WorkItem& it, uint32_t (&cw)[NCH][NWC], uint4& scp) {
    const int r = u % per_item, kvh = r / TPW, tile = r % TPW;
    const uint8_t* et = pv.entry(seg, it.flag == 1 ? it.src : 0, kvh) + size_t(tile) * LT.bytes;
    const auto rs = __builtin_amdgcn_make_buffer_rsrc(const_cast<uint8_t*>(et), (short)0,
                                                      it.flag == 1 ? int(LT.bytes) : 0, 0x00020000);
#pragma unroll
    for (int j = 0; j < NCH; ++j) {
      const int c = tid + 256 * j;
      const bool is_v = 256 * j >= 4 * D;
      const int cc = is_v ? c - 4 * D : c;
      int wb, bit;
      layout::code_pos(cc >> 6, cc & 63, 0, D, BITS, &wb, &bit);
#pragma unroll
      for (int q = 0; q < NWC; ++q)
        cw[j][q] = __builtin_amdgcn_raw_buffer_load_b32(rs, int((is_v ? LT.vc : LT.kc) + wb + 4 * q), 0, 0);
    }
    // (threads from D/2 on load piece 0 again and do not use it)
    scp = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(
                                        rs, int(LT.ks + 16 * (tid < D / 2 ? tid : 0)), 0, 0));
  };
  // Batches of NBU units (u0, u0 + gridDim.x, ...): every load of a batch goes
  // out before its first store, so no wait for a unit's data also waits for
  // stores (a wave's memory counter is in order); each unit's 16 KB of bf16
  // is stored as soon as it is decoded.
  for (int u0 = blockIdx.x; u0 < units; u0 += NBU * gridDim.x) {
    WorkItem its[NBU];
    uint32_t cw[NBU][NCH][NWC];
    uint4 scp[NBU];
    // every item of the batch first (no branch: a unit past the list takes
    // the last item's entry with its flag cleared), then every load
#pragma unroll
    for (int k = 0; k < NBU; ++k) {
      const int u = u0 + k * gridDim.x;
      its[k] = work[min(u, units - 1) / per_item];
      if (u >= units) its[k].flag = 0;
    }
#pragma unroll
    for (int k = 0; k < NBU; ++k) fetch(u0 + k * gridDim.x, its[k], cw[k], scp[k]);
    if (u0 != blockIdx.x) __syncthreads();   // the previous batch's scale reads are done
    if (tid < D / 2) {
#pragma unroll
      for (int k = 0; k < NBU; ++k) s_sc[k][tid] = scp[k];
    }
    __syncthreads();
#pragma unroll
    for (int k = 0; k < NBU; ++k) {
      const WorkItem& it = its[k];
      if (it.flag != 1) continue;   // (the same for the whole workgroup)
      const int u = u0 + k * gridDim.x;
      const int r = u % per_item, kvh = r / TPW, tile = r % TPW;
      uint16_t* tb = pv.block(seg, it.dst, kvh) + size_t(tile) * 64 * D;
      const _Float16* ks = reinterpret_cast<const _Float16*>(s_sc[k]);
      const _Float16* km = ks + D;
      const _Float16* vs = ks + 2 * D;
      const _Float16* vm = ks + 3 * D;
#pragma unroll
      for (int j = 0; j < NCH; ++j) {
        const int c = tid + 256 * j;
        const bool is_v = 256 * j >= 4 * D;
        const int cc = is_v ? c - 4 * D : c, cmb = cc >> 6, lane = cc & 63;
        // the chunk's 8 scales and mins: K channels d0 .. d0 + 7, or V tokens
        // t0 .. t0 + 7 of channel block d0 / 32
        int t0, d0;
        if (is_v) layout::v_chunk_elem(cmb, lane, 0, &t0, &d0);
        else layout::k_chunk_elem(cmb, lane, 0, D, &t0, &d0);
        const int pb = is_v ? (d0 >> 5) * 32 + t0 : d0;
        const uint4 s8 = *reinterpret_cast<const uint4*>(is_v ? vs + pb : ks + pb);
        const uint4 m8 = *reinterpret_cast<const uint4*>(is_v ? vm + pb : km + pb);
        const uint32_t sw[4] = {s8.x, s8.y, s8.z, s8.w}, mw[4] = {m8.x, m8.y, m8.z, m8.w};
        uint32_t out[4];
#pragma unroll
        for (int e2 = 0; e2 < 4; ++e2) {
          f32x2 f;
#pragma unroll
          for (int h = 0; h < 2; ++h) {
            const int e = 2 * e2 + h;
            int wb, bit;
            layout::code_pos(cmb, lane, e, D, BITS, &wb, &bit);
            const uint32_t word = (BITS == 8 && e >= 4) ? cw[k][j][NWC - 1] : cw[k][j][0];
            const float code = float((word >> bit) & kMask);
            const float sc = float(__builtin_bit_cast(_Float16, uint16_t(sw[e2] >> (16 * h))));
            const float mn = float(__builtin_bit_cast(_Float16, uint16_t(mw[e2] >> (16 * h))));
            f[h] = __builtin_fmaf(code, sc, mn);
          }
          out[e2] = __builtin_bit_cast(uint32_t, __builtin_convertvector(f, bf16x2));
        }
        reinterpret_cast<uint4*>(tb + (is_v ? 32 * D : 0))[is_v ? c - 4 * D : c] =
            make_uint4(out[0], out[1], out[2], out[3]);
      }
    }
  }
}

// The data kernel of one planned list of `layer` (list 0: demotions, 1:
// promotions) of at most cap items per sequence.
static hipError_t launch_data(const PoolView& pv, int layer, int cap, bool promote, hipStream_t s) {
  // the quantise kernel: its occupancy in workgroups per compute unit (four
  // at head_dim 128, three at 64: one round, no tail of late workgroups); the
  // dequantise kernel: four, each taking its units in batches of four (at
  // the Mistral-7B step, 4096 units, one batch per workgroup; measured
  // against two units per batch at eight workgroups per CU, and four or eight
  // units per batch at four or eight per CU).  Never more than the largest
  // unit count.
  const long max_units = long(cap) * pv.Hkv * (pv.W / 32);
  long gx = ((promote ? 4L : (pv.D == 128 ? 4L : 3L)) * pv.cus + pv.B - 1) / pv.B;
  if (gx > max_units) gx = max_units;
  if (gx < 1) gx = 1;
  const int wi = pv.lbits == 2 ? 0 : (pv.lbits == 4 ? 1 : 2);
  const int di = pv.D == 64 ? 0 : 1;
  typedef void (*Kern)(PoolView, int, const WorkItem*, const int32_t*);
  static const Kern kDequant[2][3] = {{dequant_kernel<64, 2>, dequant_kernel<64, 4>, dequant_kernel<64, 8>},
                                      {dequant_kernel<128, 2>, dequant_kernel<128, 4>, dequant_kernel<128, 8>}};
  static const Kern kQuant[2][3] = {{quantize_kernel<64, 2>, quantize_kernel<64, 4>, quantize_kernel<64, 8>},
                                    {quantize_kernel<128, 2>, quantize_kernel<128, 4>, quantize_kernel<128, 8>}};
  const int list = promote ? 1 : 0;
  const WorkItem* items =
      reinterpret_cast<const WorkItem*>(pv.work + pv.work_items) + (size_t(layer) * 2 + list) * pv.B * pv.maxw;
  const int32_t* counts = pv.work + pv.work_counts + (size_t(layer) * 2 + list) * pv.B;
  hipLaunchKernelGGL(promote ? kDequant[di][wi] : kQuant[di][wi], dim3(unsigned(gx), pv.B), dim3(256), 0, s, pv,
                     layer, items, counts);
  return hipGetLastError();
}

// The plan of a layer's moves: one launch for both lists (either may be
// absent, items == nullptr).  When the two lists and the row would need more
// than 64 KB of LDS, the two plans launch one after the other.
hipError_t launch_plan(const PoolView& pv, int layer, const int32_t* d_items, int d_stride,
                       const int32_t* d_counts, const int32_t* p_items, int p_stride,
                       const int32_t* p_counts, hipStream_t s) {
  const int cap_d = d_items ? (d_stride < pv.maxw ? d_stride : pv.maxw) : 0;
  const int cap_p = p_items ? (p_stride < pv.maxw ? p_stride : pv.maxw) : 0;
  const int slots = max(d_items ? pv.nl : 0, p_items ? pv.nb : 0);
  const int words = (slots + 31) / 32;
  // plan LDS: row, first positions, free map and its word prefix, items
  const size_t shm = (2 * size_t(pv.maxw) + 2 * size_t(words) + 1 + size_t(cap_d) + size_t(cap_p)) * 4;
  if (d_items && p_items && shm > 64 * 1024) {
    // (each plan alone stays within 58 KB at the largest configuration)
    hipError_t e = launch_plan(pv, layer, d_items, d_stride, d_counts, nullptr, 0, nullptr, s);
    if (e != hipSuccess) return e;
    return launch_plan(pv, layer, nullptr, 0, nullptr, p_items, p_stride, p_counts, s);
  }
  hipLaunchKernelGGL(plan_kernel, dim3(pv.B), dim3(256), shm, s, pv, layer,
                     PlanList{d_items, d_counts, d_stride}, PlanList{p_items, p_counts, p_stride});
  return hipGetLastError();
}

// The data kernels of the lists planned for `layer`: the quantise kernel,
// then the dequantise kernel, which may write a promoted window into a bf16
// slot whose demoted window the quantise kernel reads (stream order).
// cap_d, cap_p: the lists' largest item counts (grid sizing only).
hipError_t launch_moves(const PoolView& pv, int layer, int cap_d, int cap_p, hipStream_t s) {
  hipError_t e;
  if (cap_d > 0 && (e = launch_data(pv, layer, cap_d, false, s)) != hipSuccess) return e;
  if (cap_p > 0 && (e = launch_data(pv, layer, cap_p, true, s)) != hipSuccess) return e;
  return hipSuccess;
}

hipError_t launch_transitions(const PoolView& pv, int layer, const int32_t* d_items, int d_stride,
                              const int32_t* d_counts, const int32_t* p_items, int p_stride,
                              const int32_t* p_counts, hipStream_t s) {
  hipError_t e = launch_plan(pv, layer, d_items, d_stride, d_counts, p_items, p_stride, p_counts, s);
  if (e != hipSuccess) return e;
  const int cap_d = d_items ? (d_stride < pv.maxw ? d_stride : pv.maxw) : 0;
  const int cap_p = p_items ? (p_stride < pv.maxw ? p_stride : pv.maxw) : 0;
  return launch_moves(pv, layer, cap_d, cap_p, s);
}

hipError_t launch_demote(const PoolView& pv, int layer, const int32_t* items, int stride,
                         const int32_t* counts, hipStream_t s) {
  return launch_transitions(pv, layer, items, stride, counts, nullptr, 0, nullptr, s);
}

hipError_t launch_promote(const PoolView& pv, int layer, const int32_t* items, int stride,
                          const int32_t* counts, hipStream_t s) {
  return launch_transitions(pv, layer, nullptr, 0, nullptr, items, stride, counts, s);
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
