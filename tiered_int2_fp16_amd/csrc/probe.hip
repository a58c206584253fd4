// Streaming-read probe for gfx950: the bandwidth a plain read of a given
// number of bytes reaches in one launch on this GPU, beside the nominal HBM
// peak.  A measurement aid, not a step of the method: decode attention
// re-reads the cache from HBM at every step ("Technische Samenvatting: RDKV",
// 1 Probleemstelling), so the attainable rate of one cold read of one step's
// bytes bounds what the attention kernel can reach at that size.
//
// Workgroup w of the grid reads its contiguous share of the bytes with 16-byte
// buffer loads, 16 loads per thread in flight before any is used (a share of
// up to 64 KB is one round of loads); lanes past the share read zeros without
// touching memory.  Each wave folds what it read into one word and stores it,
// so the loads cannot be optimised away.
#include <hip/hip_ext.h>

#include "launch.h"

namespace kvtier {

namespace {

__device__ inline __amdgpu_buffer_rsrc_t probe_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, int(bytes), 0x00020000);
}

}  // namespace

__global__ __launch_bounds__(256) void stream_probe_kernel(const uint8_t* __restrict__ src, uint64_t bytes,
                                                           uint32_t* __restrict__ sink) {
  constexpr int kBatch = 16;
  constexpr uint32_t kRound = 256u * 16u * kBatch;   // bytes one round of a workgroup reads
  const uint64_t share = ((bytes + gridDim.x - 1) / gridDim.x + 15) & ~uint64_t(15);
  const uint64_t beg = share * blockIdx.x;
  const uint64_t end = beg + share < bytes ? beg + share : bytes;
  const uint32_t mine = beg < end ? uint32_t(end - beg) : 0u;
  const auto rs = probe_rsrc(src + (beg < bytes ? beg : 0), mine);
  uint32_t acc = 0;
  for (uint32_t r = 0; r < mine; r += kRound) {
    uint4 v[kBatch];
#pragma unroll
    for (int j = 0; j < kBatch; ++j)
      v[j] = __builtin_bit_cast(
          uint4, __builtin_amdgcn_raw_buffer_load_b128(rs, int(r + (j * 256u + threadIdx.x) * 16u), 0, 0));
#pragma unroll
    for (int j = 0; j < kBatch; ++j) acc ^= v[j].x ^ v[j].y ^ v[j].z ^ v[j].w;
  }
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) acc ^= __shfl_xor(acc, off, 64);
  if ((threadIdx.x & 63) == 0) sink[blockIdx.x * 4 + (threadIdx.x >> 6)] = acc;
}

hipError_t launch_stream_probe(const void* src, uint64_t bytes, int workgroups, uint32_t* sink,
                               hipEvent_t ev_start, hipEvent_t ev_stop, hipStream_t s) {
  if (ev_start || ev_stop)
    hipExtLaunchKernelGGL(stream_probe_kernel, dim3(workgroups), dim3(256), 0, s, ev_start, ev_stop, 0u,
                          static_cast<const uint8_t*>(src), bytes, sink);
  else
    hipLaunchKernelGGL(stream_probe_kernel, dim3(workgroups), dim3(256), 0, s, static_cast<const uint8_t*>(src),
                       bytes, sink);
  return hipGetLastError();
}

}  // namespace kvtier
