// Host launchers of the gfx950 kernels (one translation unit per kernel family).
// Each returns hipSuccess or the launch error.
#pragma once

#include <hip/hip_runtime.h>

#include "device_common.h"

namespace kvtier {

hipError_t launch_prefill(const PoolView& pv, int layer, const uint16_t* k, const uint16_t* v,
                          int tokens, const float* prior, hipStream_t s);
hipError_t launch_demote(const PoolView& pv, int layer, const int32_t* items, int stride,
                         const int32_t* counts, hipStream_t s);
hipError_t launch_promote(const PoolView& pv, int layer, const int32_t* items, int stride,
                          const int32_t* counts, hipStream_t s);
hipError_t launch_transitions(const PoolView& pv, int layer, const int32_t* d_items, int d_stride,
                              const int32_t* d_counts, const int32_t* p_items, int p_stride,
                              const int32_t* p_counts, hipStream_t s);
hipError_t launch_plan(const PoolView& pv, int layer, const int32_t* d_items, int d_stride,
                       const int32_t* d_counts, const int32_t* p_items, int p_stride,
                       const int32_t* p_counts, hipStream_t s);
hipError_t launch_moves(const PoolView& pv, int layer, int cap_d, int cap_p, hipStream_t s);
hipError_t launch_read(const PoolView& pv, int layer, int b, int window, bool ledger, void* dst,
                       hipStream_t s);

struct AttnArgs {
  int layer;
  const uint16_t* q;
  const uint16_t* k_new;
  const uint16_t* v_new;
  float* out;
  float* mass;
  float* partials;      // [batch][kv_heads][splits][group][D]
  float2* ml;           // [batch][q_heads][splits]: (max, sum)
  float2* tile_mass;    // [batch][max_windows*W/32][q_heads]: (raw mass, max)
  float2* app_mass;     // [batch][q_heads]
  int32_t* app_info;    // [batch][8] append decision of this step (workspace)
  int splits;
  int plan_words;       // page-table entries staged in LDS: max_windows rounded up to 256
  int acc_scores;       // combine also adds the window masses to the scores
  hipEvent_t ev_start;  // optional dispatch timing events (may be null)
  hipEvent_t ev_stop;
};
hipError_t launch_attn(const PoolView& pv, const AttnArgs& a, hipStream_t s);

hipError_t launch_prefill_scores(const PoolView& pv, int layer, const uint16_t* q, const uint16_t* k,
                                 int T, float* lse, float* wt, hipStream_t s);
hipError_t launch_route_diagnostics(const PoolView& pv, int layer, const int32_t* counts,
                                    const float* shadow_mass, float* diag, hipStream_t s);
hipError_t launch_score_route(const PoolView& pv, int layer, const float* mass, int do_route,
                              double budget_frac, double hi_frac, int32_t* transitions,
                              int32_t* counts, hipStream_t s);

hipError_t launch_stream_probe(const void* src, uint64_t bytes, int workgroups, uint32_t* sink,
                               hipEvent_t ev_start, hipEvent_t ev_stop, hipStream_t s);

}  // namespace kvtier
