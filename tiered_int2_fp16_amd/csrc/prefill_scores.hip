// Initial window scores from the prefill attention, for gfx950.
//
// The RDKV summary ("Technische Samenvatting: RDKV", 2.1) weighs a cached token
// by the attention it receives over all query positions, w_t = sum_tau
// a_{tau,t}, computed once after the prefill with the full cache (2.2, phase
// 1).  These weights seed QEvict's cumulative window scores ("Technische
// Samenvatting: QEvict", Kernmechanismen): S[w] = sum over query heads and over
// the window's tokens of w_t.  The prefill attention is causal; query head h
// reads kv head h / G.
//
// Three kernels, all dense 16x16x32 bf16 MFMA tiles (lane l holds 8
// consecutive values of operand row l%16 at column block l/16; a result lane
// holds rows 4*(l/16)+i of column l%16):
//   1. row pass: each wave takes 48 queries (three 16-row operand blocks held
//      in registers) and walks the keys 0..q in chunks of 32, each chunk's key
//      operands serving all three blocks.  Per lane it keeps a running (max,
//      sum) in the log2 domain, merged over the 16 lanes of a row at the end:
//      lse[q] = max + log2(sum);
//   2. column pass: each wave takes 48 keys and walks the queries T-1 down to
//      t in chunks of 32, adding exp2(s - lse[q]): w[t] per head (downwards,
//      so that the workgroups in flight read the same query chunks from L2);
//   3. window sums: S[w] = sum over heads (in order) and the window's tokens
//      (a fixed tree) of w.
// The four waves of a workgroup hold adjacent 48-row ranges and walk the same
// chunks, so each stage of two chunks is loaded once per workgroup into a
// double-buffered LDS tile (one barrier per stage) and read from there by
// every wave; the next stage is requested before the current stage's math.  Chunks wholly
// inside the causal region skip the mask; in the row pass they also leave the
// running max in place unless a score passes it by kSlack.
#include "launch.h"

namespace kvtier {

namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

__device__ inline __amdgpu_buffer_rsrc_t span_rsrc(const void* base, int bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, bytes, 0x00020000);
}
__device__ inline bf16x8 load_row8(__amdgpu_buffer_rsrc_t r, int off) {
  return __builtin_bit_cast(bf16x8, __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0));
}
__device__ inline f32x4 mfma_bf16(bf16x8 a, bf16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}
__device__ inline float exp2_hw(float x) { return __builtin_amdgcn_exp2f(x); }

// (max, sum) pairs in the log2 domain merged; an empty side (max -inf) adds nothing
__device__ inline void merge_ms(float& m, float& l, float mo, float lo) {
  const float M = fmaxf(m, mo);
  if (M == -INFINITY) return;
  l = (m == -INFINITY ? 0.f : l * exp2_hw(m - M)) + (mo == -INFINITY ? 0.f : lo * exp2_hw(mo - M));
  m = M;
}

constexpr int kChunk = 32;    // keys (pass 1) or queries (pass 2) per step
constexpr int kSub = 2;       // steps per LDS stage (one barrier per stage)
constexpr int kStage = kChunk * kSub;
constexpr int kWaves = 4;      // waves per workgroup; the workgroup shares each chunk
constexpr int kThreads = 64 * kWaves;
constexpr int kRows = 16;     // queries (pass 1) or keys (pass 2) per operand block
constexpr int kRowBlocks = 3; // operand blocks per wave: each loaded chunk serves 48 rows
constexpr float kSlack = 8.f; // row pass: log2 headroom before the running max is moved

// One stage (kStage rows) of a [T, D] bf16 operand, loaded once per workgroup
// (kPer 16-byte pieces per thread) into one of two LDS tiles.  Rows are padded by
// 16 bytes, so the MFMA operand reads (16 rows, 16 bytes per lane) fall in
// distinct banks.  Rows past T read zeros.
template <int D>
struct ChunkTiles {
  static constexpr int kRowB = D * 2 + 16;
  static constexpr int kTileB = kStage * kRowB;
  static constexpr int kPieces = kStage * D / 8;
  static constexpr int kPer = (kPieces + kThreads - 1) / kThreads;
  unsigned char* lds;   // two tiles of kTileB bytes
  u32x4 stage[kPer];
  __device__ void fetch(__amdgpu_buffer_rsrc_t r, int row0) {
#pragma unroll
    for (int p = 0; p < kPer; ++p) {
      const int pc = threadIdx.x + kThreads * p, row = pc / (D / 8), col = pc % (D / 8);
      if (kPieces % kThreads == 0 || pc < kPieces)
        stage[p] = __builtin_amdgcn_raw_buffer_load_b128(r, ((row0 + row) * D + 8 * col) * 2, 0, 0);
    }
  }
  __device__ void stash(int t) {
#pragma unroll
    for (int p = 0; p < kPer; ++p) {
      const int pc = threadIdx.x + kThreads * p, row = pc / (D / 8), col = pc % (D / 8);
      if (kPieces % kThreads == 0 || pc < kPieces)
        *reinterpret_cast<u32x4*>(lds + t * kTileB + row * kRowB + col * 16) = stage[p];
    }
  }
  // operand row `row` of tile t, values 32 kk + 8 g .. + 8
  __device__ bf16x8 operand(int t, int row, int kk, int g) const {
    return *reinterpret_cast<const bf16x8*>(lds + t * kTileB + row * kRowB + (32 * kk + 8 * g) * 2);
  }
};

template <int D, int RB>
// Three waves per SIMD in both passes: the MFMA results stay in VGPRs (168 in
// all) and a third wave hides the softmax's latency.  A wave raises its
// priority for its MFMA block, so the SIMD's waves take turns: one issues
// MFMAs while the others run their exponentials.
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(3))) void prefill_lse_kernel(const uint16_t* __restrict__ q,
                                                          const uint16_t* __restrict__ k, int T, int Hq,
                                                          int Hkv, float qscale, float* __restrict__ lse) {
  constexpr int KK = D / 32;
  const int b = blockIdx.z, h = blockIdx.y, kvh = h / (Hq / Hkv);
  const int lane = threadIdx.x & 63, g = lane >> 4, hn = lane & 15;
  const int wid = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);   // wave-uniform: scalar branches
  const int wq0 = blockIdx.x * kWaves * kRows * RB;                    // the workgroup's first query
  if (wq0 >= T) return;   // the whole workgroup
  const int q0 = wq0 + wid * kRows * RB;
  const auto qr = span_rsrc(q + (size_t(b) * Hq + h) * size_t(T) * D, T * D * 2);
  const auto kr = span_rsrc(k + (size_t(b) * Hkv + kvh) * size_t(T) * D, T * D * 2);
  bf16x8 qa[RB][KK];   // query rows q0 + 16 r + hn (zeros past T), dims 32 kk + 8 g ..
#pragma unroll
  for (int r = 0; r < RB; ++r)
#pragma unroll
    for (int kk = 0; kk < KK; ++kk) qa[r][kk] = load_row8(qr, ((q0 + kRows * r + hn) * D + 32 * kk + 8 * g) * 2);
  float m[RB][4], l[RB][4];
#pragma unroll
  for (int r = 0; r < RB; ++r)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      m[r][i] = -INFINITY;
      l[r][i] = 0.f;
    }
  // A wave past T has no rows; it still loads and synchronises with the others.
  const int qlast = q0 < T ? min(q0 + kRows * RB, T) - 1 : -1;
  const int wlast = min(wq0 + kWaves * kRows * RB, T) - 1;   // the workgroup walks keys 0..wlast
  // Each stage of keys is loaded once per workgroup into LDS; one barrier per stage.
  __shared__ __attribute__((aligned(16))) unsigned char ktiles[2 * ChunkTiles<D>::kTileB];
  ChunkTiles<D> kc{ktiles};
  kc.fetch(kr, 0);
  kc.stash(0);
  // the query operands are complete here, so no wait in the loop counts them
  // (it would also wait for the next stage's fetch)
#pragma unroll
  for (int r = 0; r < RB; ++r)
#pragma unroll
    for (int kk = 0; kk < KK; ++kk) asm volatile("" ::"v"(qa[r][kk]));
  __syncthreads();
  int t = 0;
  for (int k0s = 0; k0s <= wlast; k0s += kStage, t ^= 1) {
    const bool more = k0s + kStage <= wlast;
    if (more) kc.fetch(kr, k0s + kStage);
#pragma unroll
    for (int sub = 0; sub < kSub; ++sub) {
      const int k0 = k0s + kChunk * sub;
      if (k0 <= qlast) {
        // keys k0 + hn and k0 + 16 + hn (masked by causality past T), shared by
        // the wave's RB blocks of 16 queries
        bf16x8 ka[KK], kb[KK];
#pragma unroll
        for (int kk = 0; kk < KK; ++kk) {
          ka[kk] = kc.operand(t, kChunk * sub + hn, kk, g);
          kb[kk] = kc.operand(t, kChunk * sub + 16 + hn, kk, g);
        }
        __builtin_amdgcn_s_setprio(1);   // the MFMA block goes first among the SIMD's waves
        f32x4 c0[RB], c1[RB];
#pragma unroll
        for (int r = 0; r < RB; ++r) {
          c0[r] = f32x4{0.f, 0.f, 0.f, 0.f};
          c1[r] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
          for (int kk = 0; kk < KK; ++kk) {
            c0[r] = mfma_bf16(qa[r][kk], ka[kk], c0[r]);
            c1[r] = mfma_bf16(qa[r][kk], kb[kk], c1[r]);
          }
        }
        __builtin_amdgcn_s_setprio(0);
#pragma unroll
        for (int r = 0; r < RB; ++r) {
          if (k0 > q0 + kRows * r + kRows - 1) continue;   // the whole block is before these keys (uniform)
          if (k0 + kChunk - 1 <= q0 + kRows * r) {
            // every key of the chunk is at or before every row of the block: no
            // mask.  The running max moves only when a score of the block passes
            // it by more than kSlack (one vote per block); otherwise the chunk
            // adds its terms against the old max, up to 2^kSlack each.
            float e0[4], e1[4];
            bool up = false;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
              e0[i] = fmaf(c0[r][i], qscale, -m[r][i]);
              e1[i] = fmaf(c1[r][i], qscale, -m[r][i]);
              up |= fmaxf(e0[i], e1[i]) > kSlack;   // also true while m is -inf
            }
            if (__builtin_amdgcn_ballot_w64(up)) {
#pragma unroll
              for (int i = 0; i < 4; ++i) {
                const float s0 = c0[r][i] * qscale, s1 = c1[r][i] * qscale;
                const float mn = fmaxf(m[r][i], fmaxf(s0, s1));
                l[r][i] = fmaf(l[r][i], exp2_hw(m[r][i] - mn), exp2_hw(s0 - mn) + exp2_hw(s1 - mn));
                m[r][i] = mn;
              }
            } else {
#pragma unroll
              for (int i = 0; i < 4; ++i) l[r][i] += exp2_hw(e0[i]) + exp2_hw(e1[i]);
            }
            continue;
          }
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const int row = q0 + kRows * r + 4 * g + i;
            const bool v0 = k0 + hn <= row, v1 = k0 + 16 + hn <= row;
            const float s0 = v0 ? c0[r][i] * qscale : -INFINITY, s1 = v1 ? c1[r][i] * qscale : -INFINITY;
            const float mn = fmaxf(m[r][i], fmaxf(s0, s1));
            if (mn != -INFINITY) {
              l[r][i] = (m[r][i] == -INFINITY ? 0.f : l[r][i] * exp2_hw(m[r][i] - mn)) + (v0 ? exp2_hw(s0 - mn) : 0.f) +
                        (v1 ? exp2_hw(s1 - mn) : 0.f);
              m[r][i] = mn;
            }
          }
        }
      }
    }
    if (more) kc.stash(t ^ 1);
    __syncthreads();
  }
#pragma unroll
  for (int r = 0; r < RB; ++r)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
#pragma unroll
      for (int off = 1; off < 16; off <<= 1) {
        const float mo = __shfl_xor(m[r][i], off, 64), lo = __shfl_xor(l[r][i], off, 64);
        merge_ms(m[r][i], l[r][i], mo, lo);
      }
      const int row = q0 + kRows * r + 4 * g + i;
      if (hn == 0 && row < T) lse[(size_t(b) * Hq + h) * T + row] = m[r][i] + __log2f(l[r][i]);
    }
}

template <int D, int RB>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(3))) void prefill_colsum_kernel(const uint16_t* __restrict__ q,
                                                             const uint16_t* __restrict__ k, int T, int Hq,
                                                             int Hkv, float qscale,
                                                             const float* __restrict__ lse,
                                                             float* __restrict__ wt) {
  constexpr int KK = D / 32;
  const int b = blockIdx.z, h = blockIdx.y, kvh = h / (Hq / Hkv);
  const int lane = threadIdx.x & 63, g = lane >> 4, hn = lane & 15;
  const int wid = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);   // wave-uniform: scalar branches
  const int wt0 = blockIdx.x * kWaves * kRows * RB;                    // the workgroup's first key
  if (wt0 >= T) return;   // the whole workgroup
  const int t0 = wt0 + wid * kRows * RB;
  const auto qr = span_rsrc(q + (size_t(b) * Hq + h) * size_t(T) * D, T * D * 2);
  const auto kr = span_rsrc(k + (size_t(b) * Hkv + kvh) * size_t(T) * D, T * D * 2);
  const auto lr = span_rsrc(lse + (size_t(b) * Hq + h) * T, T * 4);
  bf16x8 ka[RB][KK];   // key rows t0 + 16 r + hn
#pragma unroll
  for (int r = 0; r < RB; ++r)
#pragma unroll
    for (int kk = 0; kk < KK; ++kk) ka[r][kk] = load_row8(kr, ((t0 + kRows * r + hn) * D + 32 * kk + 8 * g) * 2);
  float acc[RB][4];
#pragma unroll
  for (int r = 0; r < RB; ++r)
#pragma unroll
    for (int i = 0; i < 4; ++i) acc[r][i] = 0.f;
  // Each stage of queries (and their lse values) is loaded once per workgroup
  // into LDS, one barrier per stage; the workgroup walks the query stages from
  // the last one down to wt0.
  // Queries past T read zeros and lse 0 and are masked.
  __shared__ __attribute__((aligned(16))) unsigned char qtiles[2 * ChunkTiles<D>::kTileB];
  __shared__ float ltiles[2][kStage];
  ChunkTiles<D> qc{qtiles};
  float lstage = 0.f;
  auto fetch = [&](int q0) {
    qc.fetch(qr, q0);
    if (threadIdx.x < kStage)
      lstage = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(lr, (q0 + threadIdx.x) * 4, 0, 0));
  };
  auto stash = [&](int t) {
    qc.stash(t);
    if (threadIdx.x < kStage) ltiles[t][threadIdx.x] = lstage;
  };
  const int qtop = (T - 1) & ~(kStage - 1);   // the walk runs down from the last stage to wt0
  fetch(qtop);
  stash(0);
  // the key operands are complete here, so no wait in the loop counts them
#pragma unroll
  for (int r = 0; r < RB; ++r)
#pragma unroll
    for (int kk = 0; kk < KK; ++kk) asm volatile("" ::"v"(ka[r][kk]));
  __syncthreads();
  int t = 0;
  for (int q0s = qtop; q0s >= wt0; q0s -= kStage, t ^= 1) {
    const bool more = q0s - kStage >= wt0;
    if (more) fetch(q0s - kStage);
#pragma unroll
    for (int sub = 0; sub < kSub; ++sub) {
      const int q0 = q0s + kChunk * sub;
      if (q0 + kChunk - 1 >= t0 && t0 < T) {   // some query of the chunk is at or after the wave's first key
        // queries q0 + hn and q0 + 16 + hn, shared by the wave's RB blocks of 16 keys
        bf16x8 qa[KK], qb[KK];
#pragma unroll
        for (int kk = 0; kk < KK; ++kk) {
          qa[kk] = qc.operand(t, kChunk * sub + hn, kk, g);
          qb[kk] = qc.operand(t, kChunk * sub + 16 + hn, kk, g);
        }
        const float l0 = ltiles[t][kChunk * sub + hn], l1 = ltiles[t][kChunk * sub + 16 + hn];
        __builtin_amdgcn_s_setprio(1);   // the MFMA block goes first among the SIMD's waves
        f32x4 c0[RB], c1[RB];
#pragma unroll
        for (int r = 0; r < RB; ++r) {
          c0[r] = f32x4{0.f, 0.f, 0.f, 0.f};
          c1[r] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
          for (int kk = 0; kk < KK; ++kk) {
            c0[r] = mfma_bf16(ka[r][kk], qa[kk], c0[r]);
            c1[r] = mfma_bf16(ka[r][kk], qb[kk], c1[r]);
          }
        }
        __builtin_amdgcn_s_setprio(0);
        const int qa_i = q0 + hn, qb_i = q0 + 16 + hn;
#pragma unroll
        for (int r = 0; r < RB; ++r) {
          if (q0 + kChunk <= T && q0 >= t0 + kRows * r + kRows - 1) {
            // every query of the chunk exists and is at or after every key of the block
#pragma unroll
            for (int i = 0; i < 4; ++i) {
              acc[r][i] += exp2_hw(fmaf(c0[r][i], qscale, -l0));
              acc[r][i] += exp2_hw(fmaf(c1[r][i], qscale, -l1));
            }
            continue;
          }
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const int key = t0 + kRows * r + 4 * g + i;
            if (qa_i >= key && qa_i < T) acc[r][i] += exp2_hw(fmaf(c0[r][i], qscale, -l0));
            if (qb_i >= key && qb_i < T) acc[r][i] += exp2_hw(fmaf(c1[r][i], qscale, -l1));
          }
        }
      }
    }
    if (more) stash(t ^ 1);
    __syncthreads();
  }
#pragma unroll
  for (int r = 0; r < RB; ++r)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      float x = acc[r][i];
#pragma unroll
      for (int off = 1; off < 16; off <<= 1) x += __shfl_xor(x, off, 64);
      const int key = t0 + kRows * r + 4 * g + i;
      if (hn == 0 && key < T) wt[(size_t(b) * Hq + h) * T + key] = x;
    }
}

// S[w] of sequence b: the window's token weights of every head (heads in
// order per token, then a fixed tree over the window's tokens).
__global__ __launch_bounds__(256) void prefill_window_kernel(PoolView pv, int layer, int T,
                                                             const float* __restrict__ wt) {
  __shared__ float s_part[256];
  const int w = blockIdx.x, b = blockIdx.y, tid = threadIdx.x;
  const int seg = layer * pv.B + b;
  float x = 0.f;
  for (int t = tid; t < pv.W; t += 256) {
    const int tok = w * pv.W + t;
    if (tok < T) {
      const float* p = wt + size_t(b) * pv.Hq * T + tok;
      for (int h = 0; h < pv.Hq; ++h) x += p[size_t(h) * T];
    }
  }
  s_part[tid] = x;
  __syncthreads();
  for (int s = 128; s > 0; s >>= 1) {
    if (tid < s) s_part[tid] += s_part[tid + s];
    __syncthreads();
  }
  if (tid == 0) pv.scores[size_t(seg) * pv.maxw + w] = s_part[0];
}

}  // namespace

hipError_t launch_prefill_scores(const PoolView& pv, int layer, const uint16_t* q, const uint16_t* k,
                                 int T, float* lse, float* wt, hipStream_t s) {
  const float qscale = 1.4426950408889634f / sqrtf(float(pv.D));
  const dim3 grid((T + kWaves * kRows * kRowBlocks - 1) / (kWaves * kRows * kRowBlocks), pv.Hq, pv.B);
  if (pv.D == 128) {
    hipLaunchKernelGGL((prefill_lse_kernel<128, kRowBlocks>), grid, dim3(kThreads), 0, s, q, k, T, pv.Hq, pv.Hkv,
                       qscale, lse);
    hipLaunchKernelGGL((prefill_colsum_kernel<128, kRowBlocks>), grid, dim3(kThreads), 0, s, q, k, T, pv.Hq, pv.Hkv,
                       qscale, lse, wt);
  } else {
    hipLaunchKernelGGL((prefill_lse_kernel<64, kRowBlocks>), grid, dim3(kThreads), 0, s, q, k, T, pv.Hq, pv.Hkv,
                       qscale, lse);
    hipLaunchKernelGGL((prefill_colsum_kernel<64, kRowBlocks>), grid, dim3(kThreads), 0, s, q, k, T, pv.Hq, pv.Hkv,
                       qscale, lse, wt);
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int n = (T + pv.W - 1) / pv.W;
  hipLaunchKernelGGL(prefill_window_kernel, dim3(n, pv.B), dim3(256), 0, s, pv, layer, T, wt);
  return hipGetLastError();
}

}  // namespace kvtier
