// Cumulative scoring and the byte-budget router for gfx950.
//
// QEvict technical summary: window importance is the attention score
// accumulated over time ("Kernmechanismen", cumulative scoring); windows are
// routed among full precision, recoverable INT2 and evicted within a fixed
// byte budget ("Methodologie: QEvict"; "Kernbijdragen" item 2); evicted
// windows are gone for good.
//
// Readings where the pages are silent: the R newest windows always stay bf16;
// tier counts come from the budget as
//   n_hi = min(n, max(R, floor(phi*n))),
//   n_lo = max(0, min(n - n_hi, floor((beta*n - n_hi)*16/3)))
// in double precision in that order (16/3 = bf16 bytes over INT2 bytes of a
// window); ranking is score descending, then window index ascending.
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

// Tier counts, IEEE double in the documented order (explicit roundings: no
// contraction into fused multiply-adds).
__device__ inline void device_tier_counts(int n, int R, double beta, double phi, int* hi, int* lo) {
  const double a = __dmul_rn(phi, double(n));
  int h = int(floor(a));
  h = h > R ? h : R;
  h = h < n ? h : n;
  const double x = __ddiv_rn(__dmul_rn(__dsub_rn(__dmul_rn(beta, double(n)), double(h)), 16.0), 3.0);
  int l = int(floor(x));
  l = l < n - h ? l : n - h;
  l = l > 0 ? l : 0;
  *hi = h;
  *lo = l;
}

// One workgroup per sequence: rank the eligible windows by counting, assign
// tiers, emit the transition lists in ascending window order, apply evictions.
__global__ __launch_bounds__(1024) void route_kernel(PoolView pv, int layer, double beta, double phi,
                                                     int32_t* transitions, int32_t* counts) {
  extern __shared__ uint32_t smem[];
  const int b = blockIdx.x, seg = layer * pv.B + b, tid = threadIdx.x;
  const int maxw = pv.maxw, kpad = (maxw + 7) & ~7;
  float* key = reinterpret_cast<float*>(smem);               // [kpad] score of eligible windows, else NaN
  int* rank = reinterpret_cast<int*>(smem + kpad);           // [maxw]
  uint32_t* pages = smem + kpad + maxw;                      // [maxw]
  uint8_t* newt = reinterpret_cast<uint8_t*>(smem + kpad + 2 * maxw);  // [maxw]
  __shared__ int wave_tot[16][4];
  const int len = pv.tokens[seg];
  const int n = windows_of(len, pv.W);
  const int fr = n - pv.R > 0 ? n - pv.R : 0;  // first recent window
  int n_hi, n_lo;
  device_tier_counts(n, pv.R, beta, phi, &n_hi, &n_lo);
  int nf = n_hi - (n - fr);
  nf = nf > 0 ? nf : 0;
  uint32_t* gp = pv.pages + size_t(seg) * maxw;
  const float* gs = pv.scores + size_t(seg) * maxw;
  const int fpad = (fr + 7) & ~7;
  for (int w = tid; w < fpad; w += blockDim.x) {
    float k = __builtin_nanf("");
    if (w < fr) {
      const uint32_t e = gp[w];
      if (pe_tier(e) != TIER_E) k = gs[w];
    }
    key[w] = k;
  }
  for (int w = tid; w < n; w += blockDim.x) {
    pages[w] = gp[w];
    rank[w] = 0;
  }
  __syncthreads();
  // rank[w] = number of eligible x with S[x] > S[w], or S[x] == S[w] and x < w
  // (NaN keys never compare).  Thread jobs (w, part): each part counts one
  // slice of x, eight keys per step.
  {
    const int parts = fr > 0 ? max(1, min(8, int(blockDim.x) / fr)) : 1;
    const int chunk = ((fpad / 8 + parts - 1) / parts) * 8;
    for (int job = tid; job < fr * parts; job += blockDim.x) {
      const int w = job % fr, part = job / fr;
      const float sw = key[w];
      if (sw != sw) continue;   // not eligible
      const int x0 = part * chunk, x1 = min(fpad, x0 + chunk);
      int cnt = 0;
      for (int x = x0; x < x1; x += 8) {
        const float4 a = *reinterpret_cast<const float4*>(key + x);
        const float4 c = *reinterpret_cast<const float4*>(key + x + 4);
        const float k8[8] = {a.x, a.y, a.z, a.w, c.x, c.y, c.z, c.w};
#pragma unroll
        for (int j = 0; j < 8; ++j) cnt += (k8[j] > sw) || (k8[j] == sw && x + j < w);
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
    int x = c[k];
    for (int off = 1; off < 64; off <<= 1) {
      const int y = __shfl_up(x, off, 64);
      if (lane >= off) x += y;
    }
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
    const size_t shm = size_t((pv.maxw + 7) & ~7) * 4 + size_t(pv.maxw) * 9;
    hipLaunchKernelGGL(route_kernel, dim3(pv.B), dim3(1024), shm, s, pv, layer, beta, phi, transitions,
                       counts);
    return hipGetLastError();
  }
  return hipSuccess;
}

}  // namespace kvtier
