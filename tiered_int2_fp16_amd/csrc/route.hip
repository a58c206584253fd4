// Cumulative scoring and the byte-budget router for gfx950.
//
// QEvict technical summary: window importance is the attention score
// accumulated over time ("Kernmechanismen", cumulative scoring); windows are
// routed among full precision, the recoverable low-bit tier and evicted within a fixed
// byte budget ("Methodologie: QEvict"; "Kernbijdragen" item 2); evicted
// windows are gone for good.
//
// Readings where the pages are silent: the R newest windows always stay bf16;
// tier counts come from the budget as
//   n_hi = min(n, max(R, floor(phi*n))),
//   n_lo = max(0, min(n - n_hi, floor((beta*n - n_hi)*16/(b+1))))
// in double precision in that order (16/(b+1) = bf16 bytes over the bytes of
// a window's b-bit ledger entry, 16/3 for INT2); ranking is score descending,
// then window index ascending.
#include "launch.h"

namespace kvtier {

// S[w] += sum over the layer's query heads of mass[h][w], for live windows.
__global__ __launch_bounds__(256) void score_kernel(PoolView pv, int layer, const float* mass) {
  const int b = blockIdx.y, seg = layer * pv.B + b;
  const int w = blockIdx.x * blockDim.x + threadIdx.x;
  const int n = windows_of(pv.tokens[seg], pv.W);
  if (w >= n) return;
  if (pe_tier(pv.pages[size_t(seg) * pv.maxw + w]) == TIER_E) return;
  // heads summed in order (the fused decode-step combine adds them the same way);
  // loads issued eight at a time
  float acc = 0.f;
  const float* m = mass + size_t(b) * pv.Hq * pv.maxw + w;
  int h = 0;
  for (; h + 8 <= pv.Hq; h += 8) {
    float v[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) v[j] = m[size_t(h + j) * pv.maxw];
#pragma unroll
    for (int j = 0; j < 8; ++j) acc += v[j];
  }
  for (; h < pv.Hq; ++h) acc += m[size_t(h) * pv.maxw];
  pv.scores[size_t(seg) * pv.maxw + w] += acc;
}

// Tier counts, IEEE double in the documented order, every operation rounded
// on its own.  HIP compiles with fp-contract=fast, which would fuse
// beta * n - n_hi into one fused multiply-add (the __d*_rn functions are the
// plain operators, contractible, in this toolchain): at n = 25, beta = 0.3
// and a 4-bit ledger that gives floor(7.999..) = 7 ledger windows where the
// formula gives 8.  Contraction is off for the operators below.
__device__ inline void device_tier_counts(int n, int R, int lbits, double beta, double phi, int* hi, int* lo) {
#pragma clang fp contract(off)
  const double a = phi * double(n);
  int h = int(floor(a));
  h = h > R ? h : R;
  h = h < n ? h : n;
  const double bn = beta * double(n);
  const double x = ((bn - double(h)) * 16.0) / double(lbits + 1);
  int l = int(floor(x));
  l = l < n - h ? l : n - h;
  l = l > 0 ? l : 0;
  *hi = h;
  *lo = l;
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

// Ranking key of an eligible window: the score's bits made order-preserving
// as an unsigned integer in the high word, ~w in the low word, so that
// key(x) > key(w) exactly when S[x] > S[w], or S[x] == S[w] and x < w.
// Ineligible windows get 0, below every eligible key.
__device__ inline uint64_t rank_key(float score, int w) {
  uint32_t b = __float_as_uint(score);
  if (b == 0x80000000u) b = 0u;   // -0 ties with +0, as the float compare has it
  const uint32_t o = (b & 0x80000000u) ? ~b : (b | 0x80000000u);
  return (uint64_t(o) << 32) | uint64_t(0xFFFFFFFFu - uint32_t(w));
}

// One workgroup per sequence: rank the eligible windows by counting, assign
// tiers, emit the transition lists in ascending window order, apply evictions.
// Rows with more rankable windows than this are ranked by a sort (the pair
// counts grow with the square of the row: 1021 windows took about 25 us on
// the one workgroup of a sequence).
constexpr int kSortFrom = 512;

// Key slots of the router's LDS: the row rounded up to 8, and to a power of
// two for the sort of long rows.
__host__ __device__ inline int key_slots(int maxw) {
  int n = 8;
  while (n < maxw) n <<= 1;
  return maxw > kSortFrom ? n : (maxw + 7) & ~7;
}

__global__ __launch_bounds__(1024) void route_kernel(PoolView pv, int layer, double beta, double phi,
                                                     int32_t* transitions, int32_t* counts) {
  extern __shared__ __attribute__((aligned(16))) uint32_t smem[];
  const int b = blockIdx.x, seg = layer * pv.B + b, tid = threadIdx.x;
  const int maxw = pv.maxw, kpad = key_slots(maxw);
  uint64_t* key = reinterpret_cast<uint64_t*>(smem);         // [kpad] rank_key, 0 if not eligible
  int* rank = reinterpret_cast<int*>(smem + 2 * kpad);       // [maxw]
  uint32_t* pages = smem + 2 * kpad + maxw;                  // [maxw]
  uint8_t* newt = reinterpret_cast<uint8_t*>(smem + 2 * kpad + 2 * maxw);  // [maxw]
  __shared__ int wave_tot[16][4];
  uint32_t* gp = pv.pages + size_t(seg) * maxw;
  const float* gs = pv.scores + size_t(seg) * maxw;
  // the token count, the page entries and the scores in one round of loads
  // (none of them waits for another; entries past the row read 0)
  const int len = pv.tokens[seg];
  constexpr int kPer = 4;   // windows per thread in the first round (1024 threads: 4096 windows)
  uint32_t e4[kPer];
  float s4[kPer];
  {
    const auto rp = __builtin_amdgcn_make_buffer_rsrc(gp, (short)0, maxw * 4, 0x00020000);
    const auto rsc = __builtin_amdgcn_make_buffer_rsrc(const_cast<float*>(gs), (short)0, maxw * 4, 0x00020000);
#pragma unroll
    for (int j = 0; j < kPer; ++j) {
      const int w = tid + int(blockDim.x) * j;
      e4[j] = __builtin_amdgcn_raw_buffer_load_b32(rp, w * 4, 0, 0);
      s4[j] = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(rsc, w * 4, 0, 0));
    }
  }
  const int n = windows_of(len, pv.W);
  const int fr = n - pv.R > 0 ? n - pv.R : 0;  // first recent window
  int n_hi, n_lo;
  device_tier_counts(n, pv.R, pv.lbits, beta, phi, &n_hi, &n_lo);
  int nf = n_hi - (n - fr);
  nf = nf > 0 ? nf : 0;
  const int fpad = (fr + 7) & ~7;
#pragma unroll
  for (int j = 0; j < kPer; ++j) {
    const int w = tid + int(blockDim.x) * j;
    if (w < fpad) key[w] = (w < fr && pe_tier(e4[j]) != TIER_E) ? rank_key(s4[j], w) : 0;
    if (w < n) {
      pages[w] = e4[j];
      rank[w] = 0;
    }
  }
  // (rows longer than kPer x 1024 windows: the rest, as before)
  for (int w = tid + kPer * int(blockDim.x); w < fpad; w += blockDim.x) {
    uint64_t k = 0;
    if (w < fr) {
      const uint32_t e = gp[w];
      if (pe_tier(e) != TIER_E) k = rank_key(gs[w], w);
    }
    key[w] = k;
  }
  for (int w = tid + kPer * int(blockDim.x); w < n; w += blockDim.x) {
    pages[w] = gp[w];
    rank[w] = 0;
  }
  __syncthreads();
  // rank[w] = number of x with key[x] > key[w].  Long rows: the keys are
  // sorted in LDS (bitonic, descending; keys are distinct but for the zeros
  // of windows that take no part, which sort last), and a key's position is
  // its rank.  Short rows: one unsigned compare per key pair; thread jobs (w,
  // part), each part counting one slice of x, eight keys per step.
  if (fr > kSortFrom) {
    int N = 8;
    while (N < fpad) N <<= 1;   // (N <= kpad)
    for (int w = fpad + tid; w < N; w += blockDim.x) key[w] = 0;
    __syncthreads();
    for (int k = 2; k <= N; k <<= 1) {
      for (int j = k >> 1; j > 0; j >>= 1) {
        for (int i = tid; i < N; i += blockDim.x) {
          const int ixj = i ^ j;
          if (ixj > i) {
            const uint64_t x = key[i], y = key[ixj];
            const bool desc = (i & k) == 0;
            if (desc ? x < y : x > y) {
              key[i] = y;
              key[ixj] = x;
            }
          }
        }
        __syncthreads();
      }
    }
    for (int p = tid; p < N; p += blockDim.x) {
      const uint64_t x = key[p];
      if (x) rank[int(0xFFFFFFFFu - uint32_t(x))] = p;
    }
  } else {
    const int parts = fr > 0 ? max(1, min(8, int(blockDim.x) / fr)) : 1;
    const int chunk = ((fpad / 8 + parts - 1) / parts) * 8;
    for (int job = tid; job < fr * parts; job += blockDim.x) {
      const int w = job % fr, part = job / fr;
      const uint64_t kw = key[w];
      if (kw == 0) continue;   // not eligible
      const int x0 = part * chunk, x1 = min(fpad, x0 + chunk);
      int cnt = 0;
      for (int x = x0; x < x1; x += 8) {
        uint64_t k8[8];
#pragma unroll
        for (int j = 0; j < 8; j += 2) {
          const ulonglong2 v = *reinterpret_cast<const ulonglong2*>(key + x + j);
          k8[j] = v.x;
          k8[j + 1] = v.y;
        }
#pragma unroll
        for (int j = 0; j < 8; ++j) cnt += k8[j] > kw;
      }
      if (cnt) atomicAdd(&rank[w], cnt);
    }
  }
  __syncthreads();
  for (int w = tid; w < n; w += blockDim.x) {
    const int t = pe_tier(pages[w]);
    int nt = t;
    if (t != TIER_E) {
      if (w >= fr) {
        nt = TIER_F;
      } else {
        const int r = rank[w];
        nt = r < nf ? TIER_F : (r < nf + n_lo ? TIER_Q : TIER_E);
      }
    }
    newt[w] = uint8_t(nt);
  }
  __syncthreads();
  // Ordered compaction: each thread owns a contiguous run of windows.
  const int per = (n + blockDim.x - 1) / blockDim.x;
  const int w0 = threadIdx.x * per, w1 = min(n, w0 + per);
  int c[4] = {0, 0, 0, 0};  // demote, promote, evict, first quantisation
  for (int w = w0; w < w1; ++w) {
    const int t = pe_tier(pages[w]), nt = newt[w];
    c[0] += (t == TIER_F && nt == TIER_Q);
    c[1] += (t == TIER_Q && nt == TIER_F);
    c[2] += (t != TIER_E && nt == TIER_E);
    c[3] += (t == TIER_F && nt == TIER_Q && !pe_has_ledger(pages[w]));
  }
  const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
  int pre[4];
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    const int x = wave_incl_scan(c[k]);
    pre[k] = x - c[k];
    if (lane == 63) wave_tot[wid][k] = x;
  }
  __syncthreads();
  const int nw = (blockDim.x + 63) / 64;
  if (threadIdx.x < 4) {
    int tot = 0;
    for (int i = 0; i < nw; ++i) tot += wave_tot[i][threadIdx.x];
    if (counts) counts[threadIdx.x * pv.B + b] = tot;
  }
#pragma unroll
  for (int k = 0; k < 4; ++k)
    for (int i = 0; i < wid; ++i) pre[k] += wave_tot[i][k];
  __syncthreads();
  if (transitions) {
    int32_t* dl = transitions + (size_t(0) * pv.B + b) * maxw;
    int32_t* pl = transitions + (size_t(1) * pv.B + b) * maxw;
    int32_t* el = transitions + (size_t(2) * pv.B + b) * maxw;
    for (int w = w0; w < w1; ++w) {
      const int t = pe_tier(pages[w]), nt = newt[w];
      if (t == TIER_F && nt == TIER_Q) dl[pre[0]++] = w;
      if (t == TIER_Q && nt == TIER_F) pl[pre[1]++] = w;
      if (t != TIER_E && nt == TIER_E) el[pre[2]++] = w;
    }
  }
  // evictions take effect now: both copies are released
  for (int w = threadIdx.x; w < n; w += blockDim.x)
    if (pe_tier(pages[w]) != TIER_E && newt[w] == TIER_E) gp[w] = 0u;
}

// Routing diagnostics of the QEvict summary ("Kernbijdragen", item 1): selection
// churn and Global LIR from the counts of a routing event, future missed mass
// from the window masses of a shadow cache that keeps every window in bf16.
// One block per sequence; diag float [batch][5] (see kv_route_diagnostics).
__global__ __launch_bounds__(256) void diag_kernel(PoolView pv, int layer, const int32_t* counts,
                                                   const float* shadow_mass, float* diag) {
  __shared__ float s_miss[4];
  __shared__ int s_live[4];
  const int b = blockIdx.x, seg = layer * pv.B + b, tid = threadIdx.x;
  const int lane = tid & 63, wid = tid >> 6;
  const uint32_t* pages = pv.pages + size_t(seg) * pv.maxw;
  // every load is independent of the token count and the page entries (the
  // window bound and the evicted test only select), so all go out at once
  const int tokens = pv.tokens[seg];
  int live = 0;
  float miss = 0.f;
  for (int w = tid; w < pv.maxw; w += 256) {
    const uint32_t e = pages[w];
    float acc = 0.f;
    if (shadow_mass) {
      const float* m = shadow_mass + size_t(b) * pv.Hq * pv.maxw + w;
#pragma unroll 8
      for (int h = 0; h < pv.Hq; ++h) acc += m[size_t(h) * pv.maxw];
    }
    const bool in = w < windows_of(tokens, pv.W);
    const bool ev = in && pe_tier(e) == TIER_E;
    live += (in && !ev) ? 1 : 0;
    if (ev) miss += acc;
  }
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) {
    live += __shfl_xor(live, off, 64);
    miss += __shfl_xor(miss, off, 64);
  }
  if (lane == 0) {
    s_live[wid] = live;
    s_miss[wid] = miss;
  }
  __syncthreads();
  if (tid != 0) return;
  const int live_now = s_live[0] + s_live[1] + s_live[2] + s_live[3];
  float* d = diag + size_t(b) * 5;
  if (counts) {
    const int dem = counts[b], pro = counts[pv.B + b], evi = counts[2 * pv.B + b];
    const int before = live_now + evi;
    d[0] = before > 0 ? __fdiv_rn(float(dem + pro + evi), float(before)) : 0.f;
    d[1] += float(pro);
    d[2] += float(dem);
    d[3] = d[2] > 0.f ? __fdiv_rn(d[1], d[2]) : 0.f;
  }
  if (shadow_mass) d[4] = ((s_miss[0] + s_miss[1]) + (s_miss[2] + s_miss[3])) / float(pv.Hq);
}

hipError_t launch_route_diagnostics(const PoolView& pv, int layer, const int32_t* counts,
                                    const float* shadow_mass, float* diag, hipStream_t s) {
  hipLaunchKernelGGL(diag_kernel, dim3(pv.B), dim3(256), 0, s, pv, layer, counts, shadow_mass, diag);
  return hipGetLastError();
}

hipError_t launch_score_route(const PoolView& pv, int layer, const float* mass, int do_route,
                              double beta, double phi, int32_t* transitions, int32_t* counts,
                              hipStream_t s) {
  if (mass) {
    hipLaunchKernelGGL(score_kernel, dim3((pv.maxw + 255) / 256, pv.B), dim3(256), 0, s, pv, layer,
                       mass);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  if (do_route) {
    const size_t shm = size_t(key_slots(pv.maxw)) * 8 + size_t(pv.maxw) * 9;
    hipLaunchKernelGGL(route_kernel, dim3(pv.B), dim3(1024), shm, s, pv, layer, beta, phi, transitions,
                       counts);
    return hipGetLastError();
  }
  return hipSuccess;
}

}  // namespace kvtier
