// C ABI of the window-tiered KV path: host-side validation, then launches.
// Declarations, argument meaning, layouts and error behaviour: include/kvtier.h.
#include <cmath>
#include <cstdio>
#include <cstring>
#include <mutex>
#include <new>
#include <string>
#include <vector>

#include "host_core.h"
#include "kvtier.h"
#include "launch.h"

using namespace kvtier;

struct kv_pool {
  Geometry g;
  char* arena = nullptr;
  size_t arena_bytes = 0;
  int splits = 1;
  int device = 0;
  int cus = 1;
  std::vector<hipEvent_t> ev_start, ev_stop;  // attention dispatch timing
  int ev_used = 0;
  ~kv_pool() {
    for (hipEvent_t e : ev_start) hipEventDestroy(e);
    for (hipEvent_t e : ev_stop) hipEventDestroy(e);
  }
};

namespace {

thread_local std::string g_last_error;

kv_status fail(kv_status s, const std::string& msg) {
  g_last_error = msg;
  return s;
}

kv_status hip_fail(hipError_t e, const char* what) {
  return fail(KV_EDEVICE, std::string(what) + ": " + hipGetErrorString(e));
}

PoolView view(const kv_pool* p) {
  const Geometry& g = p->g;
  PoolView v;
  v.bf16 = reinterpret_cast<uint16_t*>(p->arena + g.off[KV_REGION_BF16]);
  v.ledger = reinterpret_cast<uint8_t*>(p->arena + g.off[KV_REGION_LEDGER]);
  v.pages = reinterpret_cast<uint32_t*>(p->arena + g.off[KV_REGION_PAGES]);
  v.scores = reinterpret_cast<float*>(p->arena + g.off[KV_REGION_SCORES]);
  v.tokens = reinterpret_cast<int32_t*>(p->arena + g.off[KV_REGION_TOKENS]);
  v.work = reinterpret_cast<int32_t*>(p->arena + g.off[KV_REGION_WORK]);
  v.err = reinterpret_cast<int32_t*>(p->arena + g.off[KV_REGION_ERR]);
  v.B = g.cfg.batch;
  v.L = g.cfg.layers;
  v.Hq = g.cfg.q_heads;
  v.Hkv = g.cfg.kv_heads;
  v.D = g.cfg.head_dim;
  v.W = g.cfg.window;
  v.maxw = g.cfg.max_windows;
  v.R = g.cfg.n_recent;
  v.nb = g.cfg.bf16_slots;
  v.nl = g.cfg.ledger_slots;
  v.G = g.group;
  v.lbits = g.cfg.ledger_bits;
  v.work_items = int(g.work_items);
  v.work_counts = int(g.work_counts);
  v.cus = p->cus;
  return v;
}

bool aligned(const void* p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

}  // namespace

// Attention workspace of kv_decode_step_noalloc: a static device array, one
// copy per GPU the library runs on.  In host code `scratch` names a host-side
// stand-in, not device memory: kernels and copies get the device address that
// hipGetSymbolAddress returns for the current device, kept per device below.
static __device__ __align__(256) uint8_t scratch[KV_NOALLOC_SCRATCH_BYTES];

namespace {

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

// Device address of `scratch` on device `dev` (which must be current),
// looked up on the first call for that device.
kv_status scratch_address(int dev, void** out) {
  if (dev < 0 || dev >= kMaxDevices) return fail(KV_EDEVICE, "device index beyond the scratch table");
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return hip_fail(e, "hipGetSymbolAddress(scratch)");
    if (!p) return fail(KV_EDEVICE, "hipGetSymbolAddress(scratch) gave a null address");
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return KV_OK;
}

kv_status check_pool_layer(const kv_pool* p, int32_t layer) {
  if (!p) return fail(KV_EINVAL, "pool is NULL");
  if (layer < 0 || layer >= p->g.cfg.layers) return fail(KV_EINVAL, "layer out of range");
  return KV_OK;
}

kv_status set_device(const kv_pool* p) {
  int cur = -1;
  if (hipGetDevice(&cur) != hipSuccess) return fail(KV_EDEVICE, "hipGetDevice failed");
  if (cur != p->device) {
    hipError_t e = hipSetDevice(p->device);
    if (e != hipSuccess) return hip_fail(e, "hipSetDevice");
  }
  return KV_OK;
}

}  // namespace

extern "C" {

size_t kv_pool_arena_bytes(const kv_pool_config* cfg) {
  if (!cfg) {
    g_last_error = "cfg is NULL";
    return 0;
  }
  Geometry g;
  std::string err;
  if (!geometry_init(*cfg, &g, &err)) {
    g_last_error = err;
    return 0;
  }
  return g.total;
}

size_t kv_ledger_entry_bytes(int32_t window, int32_t head_dim, int32_t ledger_bits) {
  if (window <= 0 || head_dim <= 0 || window % 32 || head_dim % 32) return 0;
  if (ledger_bits == 0) ledger_bits = 2;
  if (ledger_bits != 2 && ledger_bits != 4 && ledger_bits != 8) return 0;
  return size_t(ledger_bits + 1) * window * head_dim / 4;
}

kv_status kv_pool_create(const kv_pool_config* cfg, void* arena, size_t arena_bytes, void* stream,
                         kv_pool** out) {
  if (!cfg || !out) return fail(KV_EINVAL, "cfg and out must not be NULL");
  *out = nullptr;
  Geometry g;
  std::string err;
  if (!geometry_init(*cfg, &g, &err)) return fail(KV_EINVAL, err);
  if (!arena) return fail(KV_EINVAL, "arena is NULL");
  if (!aligned(arena, 256)) return fail(KV_EINVAL, "arena must be 256-byte aligned");
  if (arena_bytes < g.total)
    return fail(KV_ENOMEM, "arena has " + std::to_string(arena_bytes) + " bytes, needs " +
                               std::to_string(g.total));
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_fail(e, "hipGetDevice");
  int cus = 0;
  e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
  if (e != hipSuccess) return hip_fail(e, "hipDeviceGetAttribute");
  // set-up of kv_decode_step_noalloc: this device's scratch address, once
  void* scratch_ptr = nullptr;
  if (kv_status st = scratch_address(dev, &scratch_ptr)) return st;
  // clear page table, scores, token counts, work region and error word
  char* base = static_cast<char*>(arena);
  const size_t meta0 = g.off[KV_REGION_PAGES];
  e = hipMemsetAsync(base + meta0, 0, g.total - meta0, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, "hipMemsetAsync");
  kv_pool* p = new (std::nothrow) kv_pool;
  if (!p) return fail(KV_ENOMEM, "host allocation failed");
  p->g = g;
  p->arena = base;
  p->arena_bytes = arena_bytes;
  p->splits = attn_splits(g, cus);
  p->cus = cus > 0 ? cus : 1;
  p->device = dev;
  *out = p;
  return KV_OK;
}

kv_status kv_pool_destroy(kv_pool* pool) {
  delete pool;
  return KV_OK;
}

kv_status kv_pool_region(const kv_pool* pool, int32_t which, size_t* offset, size_t* bytes) {
  if (!pool) return fail(KV_EINVAL, "pool is NULL");
  if (which < 0 || which >= KV_REGION_COUNT) return fail(KV_EINVAL, "unknown region");
  if (offset) *offset = pool->g.off[which];
  if (bytes) *bytes = pool->g.size[which];
  return KV_OK;
}

kv_status kv_prefill(kv_pool* pool, int32_t layer, const void* k, const void* v, int32_t tokens,
                     const float* prior, void* stream) {
  kv_status st = check_pool_layer(pool, layer);
  if (st) return st;
  const kv_pool_config& c = pool->g.cfg;
  if (!k || !v) return fail(KV_EINVAL, "k and v must not be NULL");
  if (!aligned(k, 16) || !aligned(v, 16)) return fail(KV_EINVAL, "k and v must be 16-byte aligned");
  if (tokens < 1) return fail(KV_EINVAL, "tokens must be >= 1");
  const int n = (tokens + c.window - 1) / c.window;
  if (n > c.max_windows) return fail(KV_EINVAL, "context exceeds max_windows");
  if (n > c.bf16_slots) return fail(KV_EINVAL, "context exceeds bf16_slots");
  if ((st = set_device(pool))) return st;
  hipError_t e = launch_prefill(view(pool), layer, static_cast<const uint16_t*>(k),
                                static_cast<const uint16_t*>(v), tokens, prior,
                                static_cast<hipStream_t>(stream));
  return e == hipSuccess ? KV_OK : hip_fail(e, "prefill launch");
}

size_t kv_prefill_scores_workspace_bytes(const kv_pool* pool, int32_t tokens) {
  if (!pool || tokens < 1) return 0;
  return size_t(2) * 4 * size_t(pool->g.cfg.batch) * size_t(pool->g.cfg.q_heads) * size_t(tokens);
}

kv_status kv_prefill_scores(kv_pool* pool, int32_t layer, const void* q, const void* k, int32_t tokens,
                            void* workspace, size_t workspace_bytes, void* stream) {
  kv_status st = check_pool_layer(pool, layer);
  if (st) return st;
  const kv_pool_config& c = pool->g.cfg;
  if (!q || !k || !workspace) return fail(KV_EINVAL, "q, k and workspace must not be NULL");
  if (!aligned(q, 16) || !aligned(k, 16) || !aligned(workspace, 16))
    return fail(KV_EINVAL, "q, k and workspace must be 16-byte aligned");
  if (tokens < 1) return fail(KV_EINVAL, "tokens must be >= 1");
  if ((tokens + c.window - 1) / c.window > c.max_windows) return fail(KV_EINVAL, "context exceeds max_windows");
  if (int64_t(tokens) * c.head_dim * 2 >= (int64_t(1) << 31))
    return fail(KV_EINVAL, "tokens * head_dim * 2 must stay below 2^31");
  const size_t need = kv_prefill_scores_workspace_bytes(pool, tokens);
  if (workspace_bytes < need)
    return fail(KV_ENOMEM, "workspace has " + std::to_string(workspace_bytes) + " bytes, needs " +
                               std::to_string(need));
  if ((st = set_device(pool))) return st;
  float* lse = static_cast<float*>(workspace);
  float* wt = lse + size_t(c.batch) * c.q_heads * tokens;
  hipError_t e = launch_prefill_scores(view(pool), layer, static_cast<const uint16_t*>(q),
                                       static_cast<const uint16_t*>(k), tokens, lse, wt,
                                       static_cast<hipStream_t>(stream));
  return e == hipSuccess ? KV_OK : hip_fail(e, "prefill scores launch");
}

static kv_status transition(kv_pool* pool, int32_t layer, const int32_t* items, int32_t stride,
                            const int32_t* counts, void* stream, bool promote) {
  kv_status st = check_pool_layer(pool, layer);
  if (st) return st;
  if (!items || !counts) return fail(KV_EINVAL, "items and counts must not be NULL");
  if (stride < 1) return fail(KV_EINVAL, "stride must be >= 1");
  if (!promote && pool->g.cfg.ledger_slots == 0)
    return fail(KV_EINVAL, "pool has no ledger slots");
  if ((st = set_device(pool))) return st;
  hipError_t e = promote ? launch_promote(view(pool), layer, items, stride, counts,
                                          static_cast<hipStream_t>(stream))
                         : launch_demote(view(pool), layer, items, stride, counts,
                                         static_cast<hipStream_t>(stream));
  return e == hipSuccess ? KV_OK : hip_fail(e, promote ? "promote launch" : "demote launch");
}

kv_status kv_demote_quantize(kv_pool* pool, int32_t layer, const int32_t* items, int32_t stride,
                             const int32_t* counts, void* stream) {
  return transition(pool, layer, items, stride, counts, stream, false);
}

kv_status kv_promote_dequantize(kv_pool* pool, int32_t layer, const int32_t* items, int32_t stride,
                                const int32_t* counts, void* stream) {
  return transition(pool, layer, items, stride, counts, stream, true);
}

kv_status kv_apply_transitions(kv_pool* pool, int32_t layer, const int32_t* demote_items,
                               int32_t demote_stride, const int32_t* demote_counts,
                               const int32_t* promote_items, int32_t promote_stride,
                               const int32_t* promote_counts, void* stream) {
  kv_status st = check_pool_layer(pool, layer);
  if (st) return st;
  if (!demote_items || !demote_counts || !promote_items || !promote_counts)
    return fail(KV_EINVAL, "item lists and counts must not be NULL");
  if (demote_stride < 1 || promote_stride < 1) return fail(KV_EINVAL, "strides must be >= 1");
  if (pool->g.cfg.ledger_slots == 0) return fail(KV_EINVAL, "pool has no ledger slots");
  if ((st = set_device(pool))) return st;
  hipError_t e = launch_transitions(view(pool), layer, demote_items, demote_stride, demote_counts,
                                    promote_items, promote_stride, promote_counts,
                                    static_cast<hipStream_t>(stream));
  return e == hipSuccess ? KV_OK : hip_fail(e, "transitions launch");
}

kv_status kv_plan_transitions(kv_pool* pool, int32_t layer, const int32_t* demote_items,
                              int32_t demote_stride, const int32_t* demote_counts,
                              const int32_t* promote_items, int32_t promote_stride,
                              const int32_t* promote_counts, void* stream) {
  kv_status st = check_pool_layer(pool, layer);
  if (st) return st;
  if (!demote_items || !demote_counts || !promote_items || !promote_counts)
    return fail(KV_EINVAL, "item lists and counts must not be NULL");
  if (demote_stride < 1 || promote_stride < 1) return fail(KV_EINVAL, "strides must be >= 1");
  if (pool->g.cfg.ledger_slots == 0) return fail(KV_EINVAL, "pool has no ledger slots");
  if ((st = set_device(pool))) return st;
  hipError_t e = launch_plan(view(pool), layer, demote_items, demote_stride, demote_counts, promote_items,
                             promote_stride, promote_counts, static_cast<hipStream_t>(stream));
  return e == hipSuccess ? KV_OK : hip_fail(e, "plan launch");
}

kv_status kv_move_planned(kv_pool* pool, int32_t layer, void* stream) {
  kv_status st = check_pool_layer(pool, layer);
  if (st) return st;
  if (pool->g.cfg.ledger_slots == 0) return fail(KV_EINVAL, "pool has no ledger slots");
  if ((st = set_device(pool))) return st;
  const int m = pool->g.cfg.max_windows;
  hipError_t e = launch_moves(view(pool), layer, m, m, static_cast<hipStream_t>(stream));
  return e == hipSuccess ? KV_OK : hip_fail(e, "move launch");
}

size_t kv_attn_workspace_bytes(const kv_pool* pool) {
  if (!pool) return 0;
  return attn_workspace(pool->g, pool->splits).total;
}

static kv_status attention(kv_pool* pool, int32_t layer, const void* q, const void* k_new,
                           const void* v_new, float* out, float* mass, void* workspace,
                           size_t workspace_bytes, int acc_scores, void* stream) {
  kv_status st = check_pool_layer(pool, layer);
  if (st) return st;
  if (!q || !out) return fail(KV_EINVAL, "q and out must not be NULL");
  if ((k_new == nullptr) != (v_new == nullptr)) return fail(KV_EINVAL, "k_new and v_new go together");
  if (!aligned(q, 16) || (k_new && (!aligned(k_new, 16) || !aligned(v_new, 16))))
    return fail(KV_EINVAL, "q, k_new, v_new must be 16-byte aligned");
  if (!aligned(out, 16)) return fail(KV_EINVAL, "out must be 16-byte aligned");
  const AttnWorkspace ws = attn_workspace(pool->g, pool->splits);
  if (!workspace) return fail(KV_EINVAL, "workspace is NULL");
  if (!aligned(workspace, 256)) return fail(KV_EINVAL, "workspace must be 256-byte aligned");
  if (workspace_bytes < ws.total)
    return fail(KV_ENOMEM, "workspace has " + std::to_string(workspace_bytes) + " bytes, needs " +
                               std::to_string(ws.total));
  if ((st = set_device(pool))) return st;
  char* wsb = static_cast<char*>(workspace);
  AttnArgs a;
  a.layer = layer;
  a.q = static_cast<const uint16_t*>(q);
  a.k_new = static_cast<const uint16_t*>(k_new);
  a.v_new = static_cast<const uint16_t*>(v_new);
  a.out = out;
  a.mass = mass;
  a.partials = reinterpret_cast<float*>(wsb + ws.partials);
  a.ml = reinterpret_cast<float2*>(wsb + ws.ml);
  a.tile_mass = reinterpret_cast<float2*>(wsb + ws.tile_mass);
  a.app_mass = reinterpret_cast<float2*>(wsb + ws.app_mass);
  a.app_info = reinterpret_cast<int32_t*>(wsb + ws.app_info);
  a.splits = pool->splits;
  a.plan_words = (pool->g.cfg.max_windows + 255) & ~255;
  a.acc_scores = acc_scores;
  a.ev_start = a.ev_stop = nullptr;
  if (!pool->ev_start.empty() && pool->ev_used < int(pool->ev_start.size())) {
    a.ev_start = pool->ev_start[pool->ev_used];
    a.ev_stop = pool->ev_stop[pool->ev_used];
    ++pool->ev_used;
  }
  hipError_t e = launch_attn(view(pool), a, static_cast<hipStream_t>(stream));
  return e == hipSuccess ? KV_OK : hip_fail(e, "attention launch");
}

kv_status kv_tiered_decode_attn(kv_pool* pool, int32_t layer, const void* q, const void* k_new,
                                const void* v_new, float* out, float* mass, void* workspace,
                                size_t workspace_bytes, void* stream) {
  return attention(pool, layer, q, k_new, v_new, out, mass, workspace, workspace_bytes, 0, stream);
}

kv_status kv_decode_step(kv_pool* pool, int32_t layer, const void* q, const void* k_new,
                         const void* v_new, float* out, float* mass, void* workspace,
                         size_t workspace_bytes, void* stream) {
  return attention(pool, layer, q, k_new, v_new, out, mass, workspace, workspace_bytes, 1, stream);
}

kv_status kv_decode_step_noalloc(kv_pool* pool, int32_t layer, const void* q, const void* k_new,
                                 const void* v_new, float* out, float* mass, void* stream) {
  kv_status st = check_pool_layer(pool, layer);
  if (st) return st;
  const size_t need = attn_workspace(pool->g, pool->splits).total;
  if (need > size_t(KV_NOALLOC_SCRATCH_BYTES))
    return fail(KV_ENOMEM, "the step needs " + std::to_string(need) + " bytes of workspace; the static scratch holds " +
                               std::to_string(size_t(KV_NOALLOC_SCRATCH_BYTES)) + " (use kv_decode_step)");
  void* ws = nullptr;
  {
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    ws = (pool->device >= 0 && pool->device < kMaxDevices) ? g_scratch_ptr[pool->device] : nullptr;
  }
  if (!ws) return fail(KV_EDEVICE, "no scratch address for the pool's device");
  return attention(pool, layer, q, k_new, v_new, out, mass, ws, size_t(KV_NOALLOC_SCRATCH_BYTES), 1, stream);
}

kv_status kv_attn_profile(kv_pool* pool, int32_t capacity) {
  if (!pool) return fail(KV_EINVAL, "pool is NULL");
  if (capacity < 0 || capacity > (1 << 20)) return fail(KV_EINVAL, "capacity out of range");
  kv_status st = set_device(pool);
  if (st) return st;
  for (hipEvent_t e : pool->ev_start) hipEventDestroy(e);
  for (hipEvent_t e : pool->ev_stop) hipEventDestroy(e);
  pool->ev_start.clear();
  pool->ev_stop.clear();
  pool->ev_used = 0;
  for (int i = 0; i < capacity; ++i) {
    hipEvent_t a = nullptr, b = nullptr;
    hipError_t e = hipEventCreate(&a);
    if (e == hipSuccess) e = hipEventCreate(&b);
    if (e != hipSuccess) return hip_fail(e, "hipEventCreate");
    pool->ev_start.push_back(a);
    pool->ev_stop.push_back(b);
  }
  return KV_OK;
}

kv_status kv_attn_timings(kv_pool* pool, float* ms, int32_t cap, int32_t* n) {
  if (!pool || !n || (cap > 0 && !ms)) return fail(KV_EINVAL, "bad arguments");
  kv_status st = set_device(pool);
  if (st) return st;
  hipError_t e = hipDeviceSynchronize();
  if (e != hipSuccess) return hip_fail(e, "hipDeviceSynchronize");
  const int cnt = pool->ev_used < cap ? pool->ev_used : cap;
  for (int i = 0; i < cnt; ++i) {
    float t = 0.f;
    e = hipEventElapsedTime(&t, pool->ev_start[i], pool->ev_stop[i]);
    if (e != hipSuccess) return hip_fail(e, "hipEventElapsedTime");
    ms[i] = t;
  }
  *n = cnt;
  pool->ev_used = 0;
  return KV_OK;
}

kv_status kv_score_route(kv_pool* pool, int32_t layer, const float* mass, int32_t do_route,
                         double budget_frac, double hi_frac, int32_t* transitions, int32_t* counts,
                         void* stream) {
  kv_status st = check_pool_layer(pool, layer);
  if (st) return st;
  if (do_route) {
    if (!(budget_frac >= 0.0 && budget_frac <= 1.0) || !(hi_frac >= 0.0 && hi_frac <= 1.0))
      return fail(KV_EBUDGET, "budget_frac and hi_frac must lie in [0, 1]");
  }
  if ((st = set_device(pool))) return st;
  hipError_t e = launch_score_route(view(pool), layer, mass, do_route, budget_frac, hi_frac,
                                    transitions, counts, static_cast<hipStream_t>(stream));
  return e == hipSuccess ? KV_OK : hip_fail(e, "score/route launch");
}

kv_status kv_route_diagnostics(kv_pool* pool, int32_t layer, const int32_t* counts,
                               const float* shadow_mass, float* diag, void* stream) {
  kv_status st = check_pool_layer(pool, layer);
  if (st) return st;
  if (!diag) return fail(KV_EINVAL, "diag must not be NULL");
  if (!counts && !shadow_mass) return fail(KV_EINVAL, "give counts, shadow_mass or both");
  if ((st = set_device(pool))) return st;
  hipError_t e = launch_route_diagnostics(view(pool), layer, counts, shadow_mass, diag,
                                          static_cast<hipStream_t>(stream));
  return e == hipSuccess ? KV_OK : hip_fail(e, "diagnostics launch");
}

kv_status kv_read_ledger(kv_pool* pool, int32_t layer, int32_t b, int32_t window, void* dst,
                         void* stream) {
  kv_status st = check_pool_layer(pool, layer);
  if (st) return st;
  if (b < 0 || b >= pool->g.cfg.batch) return fail(KV_EINVAL, "sequence out of range");
  if (window < 0 || window >= pool->g.cfg.max_windows) return fail(KV_EINVAL, "window out of range");
  if (!dst || !aligned(dst, 16)) return fail(KV_EINVAL, "dst must be non-NULL and 16-byte aligned");
  if ((st = set_device(pool))) return st;
  hipError_t e = launch_read(view(pool), layer, b, window, true, dst, static_cast<hipStream_t>(stream));
  return e == hipSuccess ? KV_OK : hip_fail(e, "read launch");
}

kv_status kv_read_window(kv_pool* pool, int32_t layer, int32_t b, int32_t window, void* dst,
                         void* stream) {
  kv_status st = check_pool_layer(pool, layer);
  if (st) return st;
  if (b < 0 || b >= pool->g.cfg.batch) return fail(KV_EINVAL, "sequence out of range");
  if (window < 0 || window >= pool->g.cfg.max_windows) return fail(KV_EINVAL, "window out of range");
  if (!dst || !aligned(dst, 16)) return fail(KV_EINVAL, "dst must be non-NULL and 16-byte aligned");
  if ((st = set_device(pool))) return st;
  hipError_t e = launch_read(view(pool), layer, b, window, false, dst, static_cast<hipStream_t>(stream));
  return e == hipSuccess ? KV_OK : hip_fail(e, "read launch");
}

kv_status kv_stream_probe(const void* src, size_t bytes, size_t stride, int32_t count, int32_t workgroups,
                          uint32_t* sink, void* stream, float* ms) {
  if (!src || !sink) return fail(KV_EINVAL, "src and sink must not be NULL");
  if (bytes < 1 || count < 1) return fail(KV_EINVAL, "bytes and count must be >= 1");
  if (workgroups < 1 || workgroups > 65536) return fail(KV_EINVAL, "workgroups must be in [1, 65536]");
  if ((bytes + size_t(workgroups) - 1) / size_t(workgroups) > (size_t(1) << 31))
    return fail(KV_EINVAL, "a workgroup's share must stay within 2 GiB");
  hipStream_t s = static_cast<hipStream_t>(stream);
  std::vector<hipEvent_t> ev(ms ? 2 * size_t(count) : 0, nullptr);
  auto release = [&]() {
    for (hipEvent_t e : ev)
      if (e) hipEventDestroy(e);
  };
  for (hipEvent_t& e : ev) {
    const hipError_t r = hipEventCreate(&e);
    if (r != hipSuccess) {
      release();
      return hip_fail(r, "hipEventCreate");
    }
  }
  const char* base = static_cast<const char*>(src);
  for (int32_t i = 0; i < count; ++i) {
    const hipError_t r = launch_stream_probe(base + size_t(i) * stride, bytes, workgroups, sink,
                                             ms ? ev[2 * i] : nullptr, ms ? ev[2 * i + 1] : nullptr, s);
    if (r != hipSuccess) {
      release();
      return hip_fail(r, "stream probe launch");
    }
  }
  if (ms) {
    hipError_t r = hipStreamSynchronize(s);
    for (int32_t i = 0; r == hipSuccess && i < count; ++i) r = hipEventElapsedTime(&ms[i], ev[2 * i], ev[2 * i + 1]);
    release();
    if (r != hipSuccess) return hip_fail(r, "timing the stream probe");
  }
  return KV_OK;
}

kv_status kv_pool_check(kv_pool* pool, void* stream, int32_t* bits) {
  if (!pool) return fail(KV_EINVAL, "pool is NULL");
  kv_status st = set_device(pool);
  if (st) return st;
  hipStream_t s = static_cast<hipStream_t>(stream);
  int32_t word = 0;
  int32_t* err = reinterpret_cast<int32_t*>(pool->arena + pool->g.off[KV_REGION_ERR]);
  hipError_t e = hipMemcpyAsync(&word, err, 4, hipMemcpyDeviceToHost, s);
  if (e == hipSuccess) e = hipStreamSynchronize(s);
  if (e != hipSuccess) return hip_fail(e, "reading the error word");
  if (bits) *bits = word;
  if (word) {
    const int32_t zero = 0;
    e = hipMemcpyAsync(err, &zero, 4, hipMemcpyHostToDevice, s);
    if (e == hipSuccess) e = hipStreamSynchronize(s);
    if (e != hipSuccess) return hip_fail(e, "clearing the error word");
    char buf[64];
    std::snprintf(buf, sizeof buf, "device state error bits 0x%x", unsigned(word));
    return fail(KV_ESTATE, buf);
  }
  return KV_OK;
}

kv_status kv_tier_counts(int32_t n, int32_t n_recent, double budget_frac, double hi_frac,
                         int32_t ledger_bits, int32_t* n_hi, int32_t* n_lo) {
  if (!n_hi || !n_lo || n < 0 || n_recent < 0) return fail(KV_EINVAL, "bad arguments");
  if (ledger_bits == 0) ledger_bits = 2;
  if (ledger_bits != 2 && ledger_bits != 4 && ledger_bits != 8)
    return fail(KV_EINVAL, "ledger_bits must be 0 (= 2), 2, 4 or 8");
  int hi = 0, lo = 0;
  tier_counts(n, n_recent, budget_frac, hi_frac, ledger_bits, &hi, &lo);
  *n_hi = hi;
  *n_lo = lo;
  return KV_OK;
}

const char* kv_last_error(void) { return g_last_error.c_str(); }

}  // extern "C"
