/*
 * kvtier.h - C ABI of the window-tiered KV-cache decode path for MI355X (gfx950).
 *
 * The method (QEvict technical summary, gist.science paper 2608.05326,
 * "Methodologie: QEvict" and "Kernmechanismen"): the cached history of each
 * (sequence, layer) segment is cut into windows of consecutive tokens; every
 * window sits in one of three tiers -
 *   F  full precision (bf16 here),
 *   Q  recoverable low-bit (INT2 in the summary's experiments; INT4 or INT8
 *      per pool here), backed by a write-once quantisation ledger,
 *   E  evicted, for good -
 * and windows move between tiers under a byte budget by their cumulative
 * attention score.  One decode step attends over F and Q windows and emits the
 * attention mass each window receives.
 *
 * Conventions for every call below
 *   - Pointers are DEVICE pointers unless marked [host].
 *   - `stream` is a hipStream_t passed as void* (NULL = the null stream).
 *     Calls enqueue work and return without synchronising, except
 *     kv_pool_create (no sync either, but it validates), kv_pool_check and
 *     kv_last_error.
 *   - Arguments are validated on the host before anything is enqueued; a bad
 *     argument returns KV_EINVAL (or KV_ENOMEM for a too-small buffer) and
 *     enqueues nothing.  A failed launch returns KV_EDEVICE.
 *   - Conditions only the device can see (a demotion of a window that is not
 *     bf16, a pool out of slots, ...) set bits of the pool's device error word,
 *     skip the offending item and leave the state consistent; kv_pool_check
 *     reports them as KV_ESTATE.
 *   - No C++ exception crosses this ABI.  The library never allocates device
 *     memory: the caller owns the arena and every buffer passed in.
 *   - One pool is used from one stream at a time; calls on one pool must not
 *     overlap.
 */
#ifndef KVTIER_H
#define KVTIER_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef struct kv_pool kv_pool;  /* opaque host handle owned by the library */
typedef int32_t kv_status;

enum {
  KV_OK = 0,
  KV_EINVAL = 1,   /* invalid argument or configuration */
  KV_ENOMEM = 2,   /* a caller buffer is smaller than required */
  KV_EBUDGET = 3,  /* budget fractions outside [0, 1] */
  KV_ESTATE = 4,   /* device-side state error (see kv_pool_check) */
  KV_EDEVICE = 5   /* HIP runtime error */
};

/* Window tiers as stored in the page table. */
enum { KV_TIER_E = 0, KV_TIER_Q = 1, KV_TIER_F = 2 };

/* Device error word bits (kv_pool_check). */
enum {
  KV_ERR_DEMOTE_STATE = 1,     /* demote item not a full bf16 window */
  KV_ERR_PROMOTE_STATE = 2,    /* promote item not ledger-tier with a ledger entry */
  KV_ERR_NO_BF16_SLOT = 4,     /* no free bf16 slot in the segment */
  KV_ERR_NO_LEDGER_SLOT = 8,   /* no free ledger slot in the segment */
  KV_ERR_APPEND_STATE = 16,    /* append into a window that is not bf16 */
  KV_ERR_ITEM_RANGE = 32,      /* item window index out of range */
  KV_ERR_READ_MISSING = 64,    /* kv_read_* of a window without that copy */
  KV_ERR_CAPACITY = 128        /* append beyond max_windows */
};

/* Pool geometry [host].  A segment is one (sequence b, layer l) pair; segment
 * index = l * batch + b.  Limits: q_heads % kv_heads == 0 with group size
 * q_heads / kv_heads in {1, 2, 4, 7, 8}; head_dim in {64, 128}; window a
 * multiple of 32 in [32, 256]; 1 <= max_windows <= 4096 with
 * max_windows * window / 32 <= 8192; bf16_slots <= 16383
 * and ledger_slots <= 32767 per segment; n_recent >= 1 (the newest window,
 * which appends write into, always stays bf16); ledger_bits 0 (= 2),
 * 2, 4 or 8.
 * ledger_bits is the code width of the pool's quantised tier: INT2 is the
 * width of the QEvict summary's experiments ("Methodologie: QEvict", tier 2);
 * 2, 4 and 8 are the packed widths the RDKV summary groups its stream by
 * ("2.3 Efficiente Gepakte Decode (TriZone)", Zone A).  Every window of a pool
 * uses the same width.  Value limits of the quantised tier at b bits (values
 * beyond them are invalid input: the attention's fp16 operands overflow):
 * |q| < 65504 / 2^b, K group range * |q| < 65504 * (2^b - 1) / 2^b, and V group
 * range < 65504 * (2^b - 1) / 2^(b+3) (b = 2: 6141, 4: 7676, 8: 8156). */
typedef struct {
  int32_t batch, layers, q_heads, kv_heads;
  int32_t head_dim;
  int32_t window;        /* tokens per window */
  int32_t max_windows;   /* windows per segment, including growth by decode */
  int32_t n_recent;      /* newest windows that always stay bf16 */
  int32_t bf16_slots;    /* bf16 window slots per segment */
  int32_t ledger_slots;  /* ledger slots per segment */
  int32_t ledger_bits;   /* code width of the ledger: 2 (or 0), 4, 8 */
} kv_pool_config;

/* Arena regions (kv_pool_region).  All regions are 256-byte aligned.
 *  KV_REGION_BF16    bf16 window slots: [segment][bf16_slot][kv_head] blocks of
 *                    2*W*D bf16 values in 32-token tiles laid out for the
 *                    matrix cores (K part, then V part of each tile; the
 *                    placement is internal - kv_read_window gives [W][D]).
 *  KV_REGION_LEDGER  ledger slots: [segment][ledger_slot][kv_head] entries of
 *                    (b+1)*W*D/4 bytes in 32-token tiles (b-bit K and V codes,
 *                    fp16 K scale/min per channel, fp16 V scale/min per token
 *                    and 32-channel group; placement internal - kv_read_ledger
 *                    gives the canonical layout below).
 *  KV_REGION_PAGES   uint32 [segment][max_windows] page-table entries:
 *                    bits 0-1 tier, bit 2 has-ledger, bits 3-16 bf16 slot,
 *                    bits 17-31 ledger slot.
 *  KV_REGION_SCORES  float [segment][max_windows] cumulative scores.
 *  KV_REGION_TOKENS  int32 [segment] tokens cached.
 *  KV_REGION_WORK    library scratch (each layer's transition work lists and their item counts).
 *  KV_REGION_ERR     int32 device error word. */
enum {
  KV_REGION_BF16 = 0, KV_REGION_LEDGER = 1, KV_REGION_PAGES = 2, KV_REGION_SCORES = 3,
  KV_REGION_TOKENS = 4, KV_REGION_WORK = 5, KV_REGION_ERR = 6, KV_REGION_COUNT = 7
};

/* Bytes of the device arena a pool of this geometry needs; 0 if `cfg` is
 * invalid (kv_last_error says why). [host, pure] */
size_t kv_pool_arena_bytes(const kv_pool_config* cfg);

/* Bytes of one ledger entry (one window, one kv head) of b-bit codes:
 * (b+1)*W*D/4, i.e. the codes plus an fp16 scale and min per 32 values = b+1
 * bits per value (ledger_bits 0 means 2); 0 for an invalid argument. [host] */
size_t kv_ledger_entry_bytes(int32_t window, int32_t head_dim, int32_t ledger_bits);

/* Create a pool over a caller-owned device arena of at least
 * kv_pool_arena_bytes(cfg) bytes, 256-byte aligned: the window pool of the
 * three-tier cache ("Technische Samenvatting: QEvict", "Methodologie: QEvict":
 * consecutive windows, each in the full-precision, recoverable quantised or
 * evicted tier under a fixed budget; "Kernmechanismen", window-level routing
 * and the write-once quantisation ledger), with a page table (window -> tier,
 * bf16 slot, ledger slot) per segment.  Enqueues the clearing of the metadata
 * regions (every window evicted, no tokens, zero scores, zero error word) on
 * `stream`.  Also looks up, once per device, the address of the static
 * scratch of kv_decode_step_noalloc.  *out receives the handle. */
kv_status kv_pool_create(const kv_pool_config* cfg, void* arena, size_t arena_bytes,
                         void* stream, kv_pool** out);

/* Release the host handle (the arena stays the caller's). NULL is a no-op. */
kv_status kv_pool_destroy(kv_pool* pool);

/* Byte offset and size of a region inside the arena. [host] */
kv_status kv_pool_region(const kv_pool* pool, int32_t which, size_t* offset, size_t* bytes);

/* Initial window scores from the prefill attention ("Technische Samenvatting: RDKV",
 * 2.1: a token's weight is the attention it receives over all query positions,
 * w_t = sum_tau a_{tau,t}; 2.2 phase 1: computed once after the prefill with the
 * full cache), as QEvict's cumulative scores start ("Technische Samenvatting:
 * QEvict", Kernmechanismen): S[w] = sum over query heads and over the window's
 * tokens of w_t, for the ceil(tokens/W) windows of every sequence of `layer`.
 *   q  bf16 [batch][q_heads][tokens][D]: the prefill queries of the layer;
 *   k  bf16 [batch][kv_heads][tokens][D]: its keys (those given to kv_prefill);
 *      causal attention, query head h reading kv head h / (q_heads / kv_heads),
 *      logits q.k / sqrt(D).
 *   workspace  caller-owned device memory of kv_prefill_scores_workspace_bytes:
 *      float lse [batch][q_heads][tokens] (log2-sum-exp of each query row), then
 *      float w [batch][q_heads][tokens] (the token weights of each head).
 * Replaces the scores kv_prefill set; other state is untouched.  KV_EINVAL for
 * NULL or unaligned pointers, tokens < 1, ceil(tokens/W) > max_windows or
 * tokens*D*2 >= 2^31; KV_ENOMEM for a short workspace. */
size_t kv_prefill_scores_workspace_bytes(const kv_pool* pool, int32_t tokens);
kv_status kv_prefill_scores(kv_pool* pool, int32_t layer, const void* q, const void* k,
                            int32_t tokens, void* workspace, size_t workspace_bytes,
                            void* stream);

/* Load a prefilled context into `layer`: k, v bf16 [batch][kv_heads][tokens][D].
 * Every window of every sequence becomes a bf16 window (window w in bf16
 * slot w), tokens = `tokens`, scores = prior (float [batch][ceil(tokens/W)],
 * or zeros when NULL).  Needs ceil(tokens/W) <= min(max_windows, bf16_slots). */
kv_status kv_prefill(kv_pool* pool, int32_t layer, const void* k, const void* v,
                     int32_t tokens, const float* prior, void* stream);

/* Demote windows from bf16 to the ledger tier ("Kernmechanismen", demotion;
 * write-once ledger).  items: int32 [batch][stride] window indices of `layer`, counts:
 * int32 [batch] items per sequence (device, so a router's output can be passed
 * straight in).  A window without a ledger entry is quantised now into the
 * lowest free ledger slot (per 32-value groups: K per channel over 32 tokens,
 * V per token over 32 channels; fp16 scale = (max-min)/L and min, L =
 * 2^ledger_bits - 1; codes round-half-even((x - min)/scale) in float32,
 * clamped to 0..L); a window that
 * already has one keeps it unchanged.  Its bf16 slot is freed.  Items are
 * processed in order per sequence. */
kv_status kv_demote_quantize(kv_pool* pool, int32_t layer, const int32_t* items,
                             int32_t stride, const int32_t* counts, void* stream);

/* Promote windows from the ledger tier back to bf16 ("Kernmechanismen", promotion): the
 * ledger entry is dequantised, bf16_rne(fmaf(code, scale, min)), into the
 * lowest free bf16 slot; the ledger entry is kept.  Same item format as
 * kv_demote_quantize.  Enqueue demotions first: a promotion can reuse a slot
 * a demotion frees. */
kv_status kv_promote_dequantize(kv_pool* pool, int32_t layer, const int32_t* items,
                                int32_t stride, const int32_t* counts, void* stream);

/* A routing event's moves in one call ("Kernmechanismen": demotion,
 * promotion, window-level routing): exactly
 * kv_demote_quantize(demote lists) followed by kv_promote_dequantize(promote
 * lists) on the same stream - the same pages, ledger entries, bf16 slots and
 * error bits - with one plan launch for both lists instead of two.  The
 * lists have the format of those calls (kv_score_route writes such a pair).
 * KV_EINVAL for NULL lists or counts, a stride < 1 or a pool without ledger
 * slots. */
kv_status kv_apply_transitions(kv_pool* pool, int32_t layer, const int32_t* demote_items,
                               int32_t demote_stride, const int32_t* demote_counts,
                               const int32_t* promote_items, int32_t promote_stride,
                               const int32_t* promote_counts, void* stream);

/* kv_apply_transitions in two calls, so that a caller can plan a layer's
 * moves ahead of time, on another stream, while other layers' kernels run
 * ("Kernmechanismen": the moves of a routing event are known before the
 * layers are visited).  kv_plan_transitions validates both lists, assigns
 * the slots and rewrites the layer's page table at once, exactly as
 * kv_apply_transitions does, and leaves the layer's work lists in the pool;
 * kv_move_planned then moves the bytes those lists name (quantise, then
 * dequantise).  Between the two calls nothing may read or write the layer's
 * windows (no attention, append, read-back or other move of that layer):
 * the page table already shows the moves while the bytes are not yet there.
 * Each layer has its own work lists, so plans of different layers can run
 * ahead of each other's moves; a second plan of the same layer replaces the
 * first.  Each plan is moved once: a second kv_move_planned of the same plan
 * would quantise slots the first one may already have refilled (a pool's
 * lists are empty until its first plan, so a move before any plan does
 * nothing).  Arguments and errors of kv_plan_transitions as kv_apply_transitions;
 * kv_move_planned: KV_EINVAL for a pool without ledger slots. */
kv_status kv_plan_transitions(kv_pool* pool, int32_t layer, const int32_t* demote_items,
                              int32_t demote_stride, const int32_t* demote_counts,
                              const int32_t* promote_items, int32_t promote_stride,
                              const int32_t* promote_counts, void* stream);
kv_status kv_move_planned(kv_pool* pool, int32_t layer, void* stream);

/* Workspace bytes kv_tiered_decode_attn needs for this pool. [host] */
size_t kv_attn_workspace_bytes(const kv_pool* pool);

/* One decode step of grouped-query attention for every sequence of `layer`
 * over its bf16 and ledger windows; evicted windows take no part (the softmax
 * normaliser runs over the remaining tokens).  Query head h reads kv head
 * h / (q_heads / kv_heads).  ("Technische Samenvatting: QEvict",
 * "Methodologie: QEvict": quantised windows stay reachable by attention, only
 * evicted ones are gone; "Kernmechanismen", Implementatie: grouped-query
 * attention; Cumulatieve Scoring: the attention each window receives is what
 * the scores accumulate, emitted here as `mass`.  Ledger tiles are decoded in
 * registers inside the kernel rather than dequantised into a rebuilt cache
 * first, the cost the summary's "Resultaten" names for its FlashAttention-2
 * path.)
 *   q      bf16 [batch][q_heads][D]
 *   k_new, v_new  bf16 [batch][kv_heads][D], the token this step appends (it
 *          is attended and then stored in the newest window, opening a new
 *          bf16 window when the last one is full); both NULL = no append.
 *   out    float [batch][q_heads][D], 16-byte aligned
 *   mass   float [batch][q_heads][max_windows] or NULL: the softmax probability
 *          summed over each window's tokens (0 for evicted windows; entries at
 *          or past the window count are not written).
 *   workspace  >= kv_attn_workspace_bytes(pool) bytes, 256-byte aligned; its
 *          contents need not be preserved between calls. */
kv_status kv_tiered_decode_attn(kv_pool* pool, int32_t layer, const void* q,
                                const void* k_new, const void* v_new,
                                float* out, float* mass,
                                void* workspace, size_t workspace_bytes, void* stream);

/* One decode step: kv_tiered_decode_attn, with the cumulative score update of
 * kv_score_route (S[w] += sum over the layer's query heads of mass[h][w],
 * heads in order, for live windows) fused into its combining kernel
 * ("Technische Samenvatting: QEvict", "Kernmechanismen", Cumulatieve Scoring:
 * a window's importance is its attention accumulated over time).  Same
 * arguments; mass may be NULL (the scores are still updated).  S ends up
 * bit-identical to kv_tiered_decode_attn followed by kv_score_route. */
kv_status kv_decode_step(kv_pool* pool, int32_t layer, const void* q,
                         const void* k_new, const void* v_new,
                         float* out, float* mass,
                         void* workspace, size_t workspace_bytes, void* stream);

/* kv_decode_step without a workspace argument, for callers that cannot
 * allocate device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid hipMalloc).  The attention workspace is a static
 * device array of KV_NOALLOC_SCRATCH_BYTES in the library, one per GPU, held
 * until the process ends; its device address is looked up once per device by
 * kv_pool_create.  The call allocates nothing (no hipMalloc, no hipFree, no
 * allocating library routine) and returns KV_ENOMEM, enqueuing nothing, when
 * kv_attn_workspace_bytes(pool) exceeds KV_NOALLOC_SCRATCH_BYTES.  Every call
 * on one GPU shares that GPU's array, and its contents are those the last
 * call left (nothing in it needs to start at zero): calls that overlap on one
 * GPU, from any pool or stream, race and must be serialised by the caller.
 * Other arguments, results and errors as kv_decode_step. */
enum { KV_NOALLOC_SCRATCH_BYTES = 16 << 20 };
kv_status kv_decode_step_noalloc(kv_pool* pool, int32_t layer, const void* q,
                                 const void* k_new, const void* v_new,
                                 float* out, float* mass, void* stream);

/* Kernel timing of kv_tiered_decode_attn and kv_decode_step (a profiling aid).  capacity > 0
 * makes each later attention dispatch carry its own start/stop events
 * (hipExtLaunchKernel), for up to `capacity` dispatches between reads;
 * capacity 0 turns timing off.  Creates HIP events, never device memory. */
kv_status kv_attn_profile(kv_pool* pool, int32_t capacity);

/* Synchronise the device, copy the durations (milliseconds) of the attention
 * dispatches timed since the last call into ms [host, cap entries] and their
 * number into *n [host]; restart the count. */
kv_status kv_attn_timings(kv_pool* pool, float* ms, int32_t cap, int32_t* n);

/* Cumulative scoring and routing of `layer` ("Kernmechanismen", cumulative
 * scoring; "Methodologie: QEvict", three tiers under a fixed budget).
 *   mass   float [batch][q_heads][max_windows] from kv_tiered_decode_attn, or
 *          NULL: S[w] += sum over heads of mass[h][w] for live windows.
 *   do_route != 0: route every window.  With n windows, R = n_recent:
 *            n_hi = min(n, max(R, floor(hi_frac * n)))
 *            n_lo = max(0, min(n - n_hi, floor((budget_frac * n - n_hi) * 16 / (b + 1))))
 *          (double precision, in this order; b = ledger_bits, so 16 / 3 for
 *          INT2: bf16 bits per value over ledger bits per value); the R newest
 *          windows are bf16; the other live windows ranked by (S descending,
 *          index ascending): the first n_hi - R stay/become bf16, the next
 *          n_lo go to the ledger tier, the rest
 *          are evicted now.  Demotions and promotions are written as lists for
 *          kv_demote_quantize / kv_promote_dequantize:
 *   transitions  int32 [3][batch][max_windows]: demote, promote, evict lists
 *          (ascending window order)
 *   counts int32 [4][batch]: demotions, promotions, evictions, demotions that
 *          will quantise (no ledger entry yet). */
kv_status kv_score_route(kv_pool* pool, int32_t layer, const float* mass, int32_t do_route,
                         double budget_frac, double hi_frac,
                         int32_t* transitions, int32_t* counts, void* stream);

/* Routing diagnostics of `layer` ("Technische Samenvatting: QEvict", "Kernbijdragen"
 * item 1: future missed mass, Global LIR, selection churn), one row per sequence of
 *   diag   float [batch][5], caller-owned and zeroed before the first call; [1] and [2]
 *          accumulate over calls.
 *   counts int32 [4][batch] of the routing event just taken by kv_score_route (its
 *          evictions are in the page table), or NULL:
 *            diag[0] = selection churn = (demotions + promotions + evictions) / windows
 *                      live before the event (live now + evictions), 0 with none live;
 *            diag[1] += promotions (windows back in bf16);
 *            diag[2] += demotions (windows that left bf16);
 *            diag[3] = Global LIR = diag[1] / diag[2], 0 while diag[2] is 0.
 *   shadow_mass float [batch][q_heads][max_windows]: the window masses of one decode step
 *          of a cache holding every window in bf16 (another pool routed at a full
 *          budget, fed the same tokens), or NULL:
 *            diag[4] = future missed mass = (1 / q_heads) * sum over heads and over the
 *                      windows this pool has evicted of shadow_mass.
 *          Call it with this pool in the state that step ran with.
 * Ratios are IEEE float32 quotients of the integer counts.  KV_EINVAL if diag is NULL
 * or both counts and shadow_mass are. */
kv_status kv_route_diagnostics(kv_pool* pool, int32_t layer, const int32_t* counts,
                               const float* shadow_mass, float* diag, void* stream);

/* Copy window `window` of sequence b, layer l, in the canonical layouts:
 * kv_read_ledger writes kv_heads ledger entries of (b+1)*W*D/4 bytes to dst,
 * each Kc [W][D*b/8], Vc [W][D*b/8] (b-bit code of (t, d) in byte d*b/8, bits
 * (d*b)%8 .. +b-1), Ks, Km fp16 [W/32][D], Vs, Vm fp16 [W][D/32];
 * kv_read_window writes bf16 K then V
 * [kv_heads][2][W][D].
 * A window without that copy sets KV_ERR_READ_MISSING and writes zeros. */
kv_status kv_read_ledger(kv_pool* pool, int32_t layer, int32_t b, int32_t window,
                         void* dst, void* stream);
kv_status kv_read_window(kv_pool* pool, int32_t layer, int32_t b, int32_t window,
                         void* dst, void* stream);

/* The router's tier counts for a segment of n windows and a ledger of
 * ledger_bits-bit codes (0 means 2): the formula of kv_score_route, evaluated
 * on the host in the same double-precision order. [host, pure] */
kv_status kv_tier_counts(int32_t n, int32_t n_recent, double budget_frac, double hi_frac,
                         int32_t ledger_bits, int32_t* n_hi, int32_t* n_lo);

/* Streaming-read probe, a measurement aid and not a step of the method: the
 * rate one cold launch of a plain read reaches on this GPU, the attainable
 * ceiling beside the nominal HBM peak for a decode step that re-reads its
 * cache ("Technische Samenvatting: RDKV", 1 Probleemstelling).  Enqueues
 * `count` launches back to back on `stream`; launch i reads `bytes` bytes at
 * src + i * stride with `workgroups` workgroups of 256 threads (each
 * workgroup a contiguous share, 16-byte loads, 16 per thread in flight) and
 * stores one word per wave into sink (uint32 [workgroups * 4], device).  With
 * ms != NULL [host, count entries] every launch carries start/stop events
 * (hipExtLaunchKernel); the call then synchronises the stream and writes each
 * launch's duration in milliseconds.  KV_EINVAL for NULL src or sink, bytes
 * or count < 1, workgroups outside [1, 65536] or a share above 2 GiB. */
kv_status kv_stream_probe(const void* src, size_t bytes, size_t stride, int32_t count,
                          int32_t workgroups, uint32_t* sink, void* stream, float* ms);

/* Synchronise `stream`, read and clear the device error word.  Returns KV_OK or
 * KV_ESTATE (kv_last_error lists the bits); *bits (may be NULL) gets them. */
kv_status kv_pool_check(kv_pool* pool, void* stream, int32_t* bits);

/* Message of the last failing call on this thread ("" if none). [host] */
const char* kv_last_error(void);

#ifdef __cplusplus
}
#endif
#endif /* KVTIER_H */
