/*
 * dla.h -- C ABI of the Dynamic Linear Attention (DLA) layer forward pass on
 * AMD Instinct MI355X (gfx950).
 *
 * The layer is multi-state linear attention over a fixed-capacity,
 * chronologically ordered cache of outer-product states S = sum v_s k_s^T
 * (d_v x d_k), read as o_t = sum_j lam_t[j] S_(j) q_t with slot j the j-th
 * most recent state.  Sources (reading notes "Dynamic Linear Attention |
 * Chlience Paper Archive"): section 5.1 builds the per-token state and either
 * merges it into the current state or opens a new one; section 5.2 keeps at
 * most C states and greedily merges an adjacent pair when the cache is over
 * capacity; section 5.3 reads the bounded cache with query-dependent weights;
 * section 1 gives the single-state recurrence whose state includes token t
 * when o_t is read.  The ai-feeds.com summary "Dynamic Linear Attention"
 * (method section) adds that the layer consumes an online token stream, that
 * two consecutive low-information tokens are merged, that a merged state
 * keeps the original timestamp, and that the updated state set is handed on
 * to decoding.
 *
 * Fixed choices (the pages leave them open):
 *   - token information s_t = 1 - cos(k_t, k_{t-1}), float, s = 1 without a
 *     previous key or with a zero-norm key (dot and norms summed in double,
 *     rounded once to float);
 *   - token t opens a new state unless s_t < tau and s_{t-1} < tau;
 *     an empty cache always opens one;
 *   - information sums are int64 multiples of 2^-32 (exact);
 *   - after an append that leaves C+1 states, the adjacent pair with the
 *     smallest summed information is merged (earliest pair on ties); the
 *     merged state keeps the earlier start.  A cache set to
 *     DLA_MERGE_DENSITY merges instead the pair of lowest information
 *     density (I_i + I_{i+1}) / (n_i + n_{i+1}), n the token counts: the
 *     criterion the reading notes write in section 5.2, compared exactly,
 *     earliest pair on ties;
 *   - o_t is read after the update and any merge;
 *   - lam is indexed by cache slot, slot 0 = most recent state.
 *
 * The Log-Linear fixed schedule (a cache set to DLA_FENWICK).  The reading
 * notes quote Log-Linear Attention in section 2 as the multi-state method
 * whose buckets come from a Fenwick-tree decomposition of the prefix, with
 * o_t = sum_l lam_t^(l) S_t^(l) q_t, and contrast it with DLA in section 5.4
 * (buckets by position: recent tokens fine, old ones coarse).  The pages do
 * not spell out the buckets; this library takes the binary decomposition:
 *   - level 0 is token t itself; level l >= 1 is the bucket of the 2^(l-1)
 *     earlier tokens that agree with t above bit l-1 and have bit l-1 clear
 *     where t has it set (empty if bit l-1 of t is clear), i.e. key s < t
 *     sits at level 1 + (highest bit in which s and t differ);
 *   - lam_t[l] weights level l (not a slot), so lam needs
 *     L(T) = bit_length(T - 1) + 1 columns: C >= L(T);
 *   - no token information is computed and tau is ignored;
 *   - dla_prefill and dla_decode_step continue the streams from t_seen, on
 *     a cache that fixed-schedule calls left (or an empty one).
 *
 * Conventions for every entry point
 *   - Pointers named as device pointers must point to device memory the
 *     caller allocated; the library never allocates, frees or synchronises.
 *   - `stream` is a hipStream_t (NULL = the null stream).  Work is enqueued
 *     on it and the call returns at once; buffers must stay alive until the
 *     stream work completes.  A cache must not be used on two streams at once.
 *   - All argument checks run on the host before anything is enqueued; on any
 *     error status nothing was enqueued.  dla_last_error() then describes the
 *     problem (thread-local string).
 *   - Tensors are row-major and contiguous; every device pointer must be
 *     16-byte aligned.
 *   - NaN or Inf inputs are outside the contract.
 */
#ifndef DLA_H
#define DLA_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define DLA_ABI_VERSION 7
#define DLA_MAX_C 64        /* largest supported cache capacity */
#define DLA_CHUNK 64        /* tokens per prefill chunk */
/* bytes of the static per-device scratch of dla_prefill_noalloc (64 MiB) */
#define DLA_NOALLOC_SCRATCH_BYTES (64ull << 20)

/* Chunk-kernel choice of dla_set_prefill_path (testing and profiling). */
#define DLA_PATH_AUTO 0       /* the library's choice (the default) */
#define DLA_PATH_STREAMED 1   /* the streamed chunk kernel for every shape */
#define DLA_PATH_UNSPLIT 2    /* the library's kernel, never split along the sequence */

typedef enum dla_status {
    DLA_OK = 0,
    DLA_ERR_ARG = 1,          /* bad pointer, size, alignment or mismatch */
    DLA_ERR_UNSUPPORTED = 2,  /* valid request outside what this library supports */
    DLA_ERR_WORKSPACE = 3,    /* workspace missing or too small */
    DLA_ERR_HIP = 4           /* a HIP launch failed; see dla_last_error() */
} dla_status;

typedef enum dla_dtype {
    DLA_F32 = 0,   /* float32 inputs and outputs */
    DLA_BF16 = 1   /* bfloat16 inputs and outputs */
} dla_dtype;

/* Which adjacent pair a capacity merge joins. */
typedef enum dla_merge_rule {
    DLA_MERGE_SUM = 0,       /* smallest summed information I_i + I_{i+1} (the default) */
    DLA_MERGE_DENSITY = 1,   /* lowest information density (I_i + I_{i+1}) / (n_i + n_{i+1}) */
    DLA_FENWICK = 2          /* the Log-Linear fixed schedule (dla_prefill), no information rule */
} dla_merge_rule;

/* How a token's information is scored, and so where boundaries fall. */
typedef enum dla_score_rule {
    DLA_SCORE_COSINE = 0,    /* s_t = 1 - cos(k_t, k_{t-1}); a state opens unless s_t and s_{t-1} are both below tau (the default) */
    DLA_SCORE_STATE = 1      /* the state information score I_t (reading notes, section 5.1); a state opens when I_t >= tau */
} dla_score_rule;

/*
 * Cache: caller-owned device memory holding, for every stream (b, h), up to
 * C states in physical slots plus the stream's metadata.  The struct is a
 * plain view; dla_cache_init fills it.
 *
 * State storage (the cache's state dtype):
 *   DLA_F32   every state is float32 in its physical slot;
 *   DLA_BF16  the closed states (all but the most recent) are bfloat16 in
 *             their physical slots, and the most recent ("active") state,
 *             the one tokens are added to, is float32 in a separate region
 *             of one state per stream (its slot's bfloat16 copy is written
 *             when it closes).  About half the bytes a decode step streams.
 *
 * Buffer layout (offsets from dla_cache_layout):
 *   states  at states_offset: [B*H][C][d_v][d_k] in the state dtype, physical slots;
 *   active  at active_offset (DLA_BF16 only): [B*H][d_v][d_k] float32;
 *   meta    at meta_offset + bh * meta_stride, per stream:
 *     int32  m            live states (0..C)
 *     int32  has_prev     1 once the stream has seen a key
 *     float  s_prev       information of the last token (1 if none)
 *     int64  t_seen       tokens consumed so far (state starts are counted on it)
 *     uint8  order[64]    physical slot of live state i, i = 0 oldest
 *     int64  info[64]     summed information of live state i, units of 2^-32
 *     int32  count[64]    tokens in live state i
 *     int64  start[64]    index of the first token of live state i
 *     float  k_prev[d_k]  last key seen
 * A checkpoint of a stream is a copy of this buffer.
 */
typedef struct dla_cache {
    int32_t B, H, C, d_k, d_v;
    int32_t merge_rule;   /* a dla_merge_rule; dla_cache_init sets DLA_MERGE_SUM */
    int32_t state_dtype;  /* DLA_F32 or DLA_BF16 (set by dla_cache_init) */
    int32_t score_rule;   /* a dla_score_rule; dla_cache_init sets DLA_SCORE_COSINE */
    void *base;           /* device pointer */
    uint64_t bytes;
} dla_cache;

typedef struct dla_cache_layout_t {
    uint64_t states_offset;
    uint64_t active_offset;   /* DLA_BF16 state dtype; equal to meta_offset for DLA_F32 (no region) */
    uint64_t meta_offset;
    uint64_t meta_stride;
    uint32_t off_m, off_has_prev, off_s_prev, off_t_seen;
    uint32_t off_order, off_info, off_count, off_start, off_k_prev;
} dla_cache_layout_t;

/* Optional starting content of a cache (device pointers, oldest state first). */
typedef struct dla_cache_preload {
    int32_t m0;               /* live states per stream, 0..C */
    int32_t reserved;
    const float *states;      /* [B*H][m0][d_v][d_k] float32 */
    const int64_t *info;      /* [B*H][m0] summed information, units of 2^-32 */
    const int32_t *count;     /* [B*H][m0] tokens per state */
    const int64_t *start;     /* [B*H][m0] first token of each state */
    int64_t t_seen;           /* tokens every stream has already consumed */
} dla_cache_preload;

/*
 * Optional schedule export (device pointers, any may be NULL).
 * Prefill (T tokens per stream):
 *   s [B*H][T]        token information
 *   boundary [B*H][T] 1 if the token opened a state
 *   seg_id [B*H][T]   states opened so far in this call, minus one
 *   m_t [B*H][T]      live states after the token
 *   ev_t, ev_i [B*H][T], n_ev [B*H]: the capacity merges in order: token and
 *                     chronological index of the earlier state of the pair
 *                     (ev_t and ev_i are given together or not at all)
 * Decode step: s, boundary, m_t and ev_i are [B*H] (ev_i = -1 without a
 * merge); seg_id, ev_t and n_ev are ignored.
 */
typedef struct dla_schedule_out {
    float *s;
    uint8_t *boundary;
    int32_t *seg_id;
    int32_t *m_t;
    int32_t *ev_t;
    int32_t *ev_i;
    int32_t *n_ev;
} dla_schedule_out;

/* Version of this ABI (DLA_ABI_VERSION). */
int32_t dla_abi_version(void);

/*
 * Bytes of a cache for the given shape and state dtype; 0 if either is
 * invalid (then dla_last_error is left as it was).  The cache is the
 * fixed-capacity state set M = {(S_i, n_i, I_i)}, m <= C, of the reading
 * notes' section 5.2 (capacity-bounded memory), one per stream, with the
 * metadata an online stream carries from call to call (ai-feeds.com summary,
 * method section).  Host only.
 */
uint64_t dla_cache_bytes(int32_t B, int32_t H, int32_t C, int32_t d_k, int32_t d_v,
                         dla_dtype state_dtype);

/* Offsets of the cache buffer's parts (the layout of dla_cache above, the
 * state set of section 5.2).  Host only.  DLA_ERR_ARG on a bad shape or dtype
 * or a NULL out. */
dla_status dla_cache_layout(int32_t B, int32_t H, int32_t C, int32_t d_k, int32_t d_v,
                            dla_dtype state_dtype, dla_cache_layout_t *out);

/*
 * Make `base` (device, >= dla_cache_bytes bytes for the same state dtype,
 * 256-byte aligned) an empty cache, or one holding `preload` (may be NULL),
 * and fill *cache: the empty state set the layer starts from, or a given one
 * (reading notes, section 5.2: the cache M of at most C states, each with its
 * token count n_i and information sum I_i; ai-feeds.com summary, method
 * section: the state set handed on to decoding).  Supported: C in [1, 64],
 * d_k in {64, 128, 256}, d_v a positive multiple of 16 up to 4096,
 * state_dtype DLA_F32 or DLA_BF16 (preloaded closed states are rounded to
 * bfloat16, to nearest even; the most recent stays float32).  A preloaded
 * stream has no previous key, so its next token has s = 1.  Enqueues one
 * kernel on `stream`; the preload buffers must stay alive until it ran.
 * DLA_ERR_ARG on a NULL cache, bad shape, misaligned or short buffer, bad
 * preload (m0 outside [0, C], NULL or misaligned pointers); DLA_ERR_HIP when
 * the launch fails.
 */
dla_status dla_cache_init(dla_cache *cache, void *base, uint64_t bytes, int32_t B,
                          int32_t H, int32_t C, int32_t d_k, int32_t d_v, dla_dtype state_dtype,
                          const dla_cache_preload *preload, void *stream);

/*
 * Merge rule of the cache's streams from the next prefill or decode call on:
 * DLA_MERGE_SUM or DLA_MERGE_DENSITY (reading notes "Dynamic Linear Attention
 * | Chlience Paper Archive", section 5.2: the pair of lowest information
 * density is merged), or DLA_FENWICK, the Log-Linear fixed schedule
 * (sections 2 and 5.4; see the top of this header).  Host only: it sets cache->merge_rule, which a caller
 * may also set directly; prefill and decode reject any other value with
 * DLA_ERR_ARG.  DLA_ERR_ARG for a NULL cache or an unknown rule (the cache is
 * then unchanged).
 */
dla_status dla_cache_set_merge_rule(dla_cache *cache, int32_t rule);

/*
 * Score rule of the cache's streams from the next prefill or decode call on.
 * DLA_SCORE_COSINE (the default) is the cosine score of consecutive keys with
 * the two-low-tokens boundary rule (top of this header).  DLA_SCORE_STATE is
 * the State Information Score of the reading notes, section 5.1: the
 * per-token state v_t k_t^T is compared with the current (most recent) state
 * S of the cache, both divided by their root mean square (RMSNorm with unit
 * gain), I_t = ||N(v_t k_t^T) - N(S)||_F / (||N(S)||_F + 1e-6), rounded to
 * float, and token t opens a new state when I_t >= tau (b_t = [I_t >= tau],
 * same section); I_t = 2 without a current state or for a zero matrix.  The
 * information sums and capacity merges are those of the merge rule, with I_t
 * in place of s_t.  Supported with DLA_SCORE_STATE: d_k and d_v in
 * {64, 128, 256}, not both 256, with bfloat16 io, d_k and d_v in {64, 128}
 * with float32 io (prefill and decode return DLA_ERR_UNSUPPORTED otherwise).  The fixed
 * schedule computes no score and ignores the rule.  Host only: it sets
 * cache->score_rule; DLA_ERR_ARG for a NULL cache or an unknown rule.
 */
dla_status dla_cache_set_score_rule(dla_cache *cache, int32_t rule);

/* Workspace bytes dla_prefill needs for this shape (the schedule of section
 * 5.1-5.2, the chunk operands of the section 5.3 read and, for a sweep grid
 * small enough to be split along the sequence, the slots of its block sets);
 * 0 if the shape is invalid.  Host only. */
uint64_t dla_prefill_workspace_bytes(int32_t B, int32_t H, int32_t T, int32_t C,
                                     int32_t d_k, int32_t d_v);

/*
 * Prefill: consume T tokens of every stream on top of what the cache holds
 * (an empty cache from dla_cache_init, or the states, metadata and last key
 * that earlier prefill and decode calls or a preload left), write o for every
 * token and leave the final states and metadata in the cache, ready for
 * dla_decode_step or another prefill.  The result is the one a single call
 * over all the tokens so far would give (reading notes, section 5: the cache
 * is the running state of an online stream).  To start a stream afresh,
 * initialise the cache again.
 *   q, k    [B*H][T][d_k]   io dtype, device
 *   v, o    [B*H][T][d_v]   io dtype, device
 *   lam     [B*H][T][C]     io dtype, device; lam[.][t][j] weights slot j
 *   tau     boundary threshold
 *   io      DLA_F32 (d_k in {64, 128}) or DLA_BF16 (d_k in {64, 128, 256})
 *   workspace  device, >= dla_prefill_workspace_bytes, 256-byte aligned;
 *              scratch owned by the call until the stream work completes
 *   sched   optional schedule export, may be NULL
 * T must be in [1, 2^24].  On a cache with bfloat16 state storage the
 * register-resident sweep (bfloat16 io, C <= 32) rounds each closed state to
 * bfloat16 when it closes or takes a merge; the streamed kernel (float32 io,
 * or C > 32) widens the live states into the workspace, runs in float32 and
 * rounds each closed state once at the end of the call.
 *
 * With the cache's rule DLA_FENWICK the call follows the Log-Linear fixed
 * schedule (top of this header), continuing each stream from t0 = t_seen on a
 * cache that fixed-schedule calls left (or an empty one).  lam[.][t][l]
 * weights level l.  C must be at least bit_length(T - 1) + 1 (DLA_ERR_ARG
 * otherwise); a stream whose positions need more, bit_length(t0 + T - 1) + 1
 * > C, is refused on the device: its outputs are NaN and its cache is left
 * unchanged.  float32 state storage only (each bucket is built by a cascade
 * of merges, which bfloat16 storage would round once per carry level); tau is
 * ignored, and a sched with any non-NULL field returns DLA_ERR_UNSUPPORTED
 * (the export describes the information schedule).  The final cache holds the
 * buckets of the prefix [0, t0 + T), oldest first: popcount(t0 + T) states
 * with their starts and counts, information 0, no previous key.
 */
dla_status dla_prefill(const void *q, const void *k, const void *v, const void *lam,
                       void *o, int32_t T, float tau, dla_dtype io, const dla_cache *cache,
                       void *workspace, uint64_t workspace_bytes,
                       const dla_schedule_out *sched, void *stream);

/*
 * dla_prefill without a workspace, for callers that cannot allocate device
 * memory (code under HIP graph capture, tight serving loops, harnesses that
 * forbid hipMalloc): the same computation, arguments and results as
 * dla_prefill, with the workspace taken from a static scratch array of
 * DLA_NOALLOC_SCRATCH_BYTES bytes that the library holds on each device it
 * runs on, from its load there until the process ends.  The call allocates
 * and frees nothing.
 *   - The scratch is the one of the device current on the calling thread;
 *     `stream` must belong to that device (DLA_ERR_ARG otherwise).
 *   - A call whose dla_prefill_workspace_bytes, less the slots of a split
 *     sweep (which the call then runs unsplit, with the same results),
 *     exceeds DLA_NOALLOC_SCRATCH_BYTES returns DLA_ERR_WORKSPACE with
 *     nothing enqueued (use dla_prefill with a workspace then).
 *   - Every call on a device shares that device's scratch, which keeps the
 *     last call's contents (nothing in it needs to start at zero): calls that
 *     overlap on one device race, so calls on different streams of one device
 *     must be ordered by the caller.
 */
dla_status dla_prefill_noalloc(const void *q, const void *k, const void *v, const void *lam,
                               void *o, int32_t T, float tau, dla_dtype io, const dla_cache *cache,
                               const dla_schedule_out *sched, void *stream);

/*
 * Name of the chunk kernel (the MFMA sweep of the section 5.3 read after the
 * schedule kernels) that dla_prefill launches for this shape and io dtype on
 * this thread (see dla_set_prefill_path), e.g. "k_prefill_rs<128,16,8>"
 * (template arguments d_k, value columns per block, state slots per wave).
 * For profilers and benchmarks; host only.
 * The string is thread-local and valid until the next call on this thread;
 * NULL for a shape dla_prefill would reject.
 */
const char *dla_prefill_kernel(dla_dtype io, int32_t B, int32_t H, int32_t C, int32_t d_k, int32_t d_v);

/*
 * Decode step: consume one token of every stream on top of the cache and
 * write o.  q, k [B*H][d_k]; v, o [B*H][d_v]; lam [B*H][C]; io dtype, device.
 * Supported: d_k and d_v each in {64, 128, 256}, any io dtype
 * (DLA_ERR_UNSUPPORTED for another d_v).  The step is the layer's online
 * form: the token's information and boundary (reading notes, section 5.1),
 * the capacity merge (section 5.2), the read o = sum_j lam[j] S_(j) q after
 * the update (sections 5.3 and 1); the updated state set stays in the cache
 * for the next step (ai-feeds.com summary, method section).  Enqueues one
 * kernel on `stream`; DLA_ERR_ARG on a bad cache, NULL or misaligned
 * pointers or a NaN tau, DLA_ERR_HIP when the launch fails.
 *
 * With the cache's rule DLA_FENWICK the step follows the Log-Linear fixed
 * schedule (top of this header) on a cache that fixed-schedule calls left (or
 * an empty one): token t = t_seen is read at level 0 and each bucket of
 * [0, t) at its level, with lam[.][l] the weight of level l; then the token
 * joins the buckets its carry completes (with z trailing ones in t, the last
 * z buckets and the token become one state; z = 0 opens a state).  float32
 * state storage only and no schedule export (DLA_ERR_UNSUPPORTED); tau is
 * ignored.  A stream at t >= 2^(C-1) needs a level weight the cache does not
 * have, and so does a cache no fixed-schedule call left that has no free
 * slot: that stream's output row is NaN and its cache is left unchanged.
 */
dla_status dla_decode_step(const void *q, const void *k, const void *v, const void *lam,
                           void *o, float tau, dla_dtype io, const dla_cache *cache,
                           const dla_schedule_out *sched, void *stream);

/*
 * Testing and profiling hook: which chunk kernel the dla_prefill calls made
 * on this thread launch.  DLA_PATH_AUTO (the default) lets the library
 * choose (the register-resident sweep for bfloat16 io, C <= 32 and
 * d_k <= 128, the streamed kernel otherwise); DLA_PATH_STREAMED runs the
 * streamed kernel for every shape; DLA_PATH_UNSPLIT runs the library's
 * choice but never splits the register-resident sweep along the sequence
 * (which it does with float32 state storage when the sweep's grid would fill
 * at most half of the device's block slots: the same results, bit for bit).  value_columns = 0 lets the library choose
 * the streamed kernel's d_v slice width, 16 or 32 forces it where d_v allows
 * and its LDS fits.  Both kernels compute the same layer (reading notes,
 * sections 5.1-5.3); production callers never need this.  Host only;
 * DLA_ERR_ARG for an unknown path or width (nothing changes then).
 */
dla_status dla_set_prefill_path(int32_t path, int32_t value_columns);

/*
 * Benchmark hook.  While set, every dla_prefill call made on this thread
 * records the event `before` right before its chunk kernel (the MFMA
 * prefill sweep, after the schedule kernels) and `after` right after it, on
 * the call's stream.  Both are hipEvent_t handles owned by the caller; pass
 * NULL, NULL to stop.  DLA_ERR_ARG if exactly one is NULL.
 */
dla_status dla_set_prefill_events(void *before, void *after);

/* Static text for a status code (host only). */
const char *dla_status_str(dla_status s);

/* Detail of the last non-OK status returned on this thread ("" if none;
 * host only).  The string is thread-local and valid until the next call. */
const char *dla_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* DLA_H */
