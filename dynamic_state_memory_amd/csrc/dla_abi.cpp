// dla_abi.cpp -- host side of the C ABI declared in include/dla.h: argument
// checks, workspace carving, launch configuration, status codes.  Every check
// runs before anything is enqueued; the library allocates nothing and never
// synchronises.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cstdarg>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <mutex>

#include "dla.h"
#include "dla_internal.h"

using namespace dla;

namespace {

thread_local char g_err[512] = "";
thread_local hipEvent_t g_ev_before = nullptr, g_ev_after = nullptr;
// testing and profiling override of the chunk-kernel choice (dla_set_prefill_path)
thread_local int g_path_override = DLA_PATH_AUTO, g_dvt_override = 0;

dla_status fail(dla_status s, const char *fmt, ...)
{
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(g_err, sizeof(g_err), fmt, ap);
    va_end(ap);
    return s;
}

dla_status ok()
{
    g_err[0] = '\0';
    return DLA_OK;
}

bool aligned(const void *p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

constexpr size_t kLdsBytes = 160 * 1024;    // LDS of one compute unit

int bit_length(int64_t x) { int n = 0; for (; x > 0; x >>= 1) ++n; return n; }

// Shape check shared by every entry point.  Returns DLA_OK or a status and message.
dla_status check_shape(int32_t B, int32_t H, int32_t C, int32_t dk, int32_t dv)
{
    if (B < 1 || H < 1) return fail(DLA_ERR_ARG, "B and H must be >= 1 (got %d, %d)", B, H);
    if (static_cast<int64_t>(B) * H > (1 << 24)) return fail(DLA_ERR_ARG, "B*H too large");
    if (C < 1 || C > DLA_MAX_C) return fail(DLA_ERR_ARG, "C must be in [1, %d] (got %d)", DLA_MAX_C, C);
    if (dk != 64 && dk != 128 && dk != 256)
        return fail(DLA_ERR_UNSUPPORTED, "d_k must be 64, 128 or 256 (got %d)", dk);
    if (dv < 16 || dv % 16 != 0 || dv > 4096)
        return fail(DLA_ERR_UNSUPPORTED, "d_v must be a multiple of 16 in [16, 4096] (got %d)", dv);
    return DLA_OK;
}

struct Sizes {
    uint64_t s, qs, flag, tile_cnt, tile_sum, seg_t, seg_P, seg_q0, nseg, events, chunk_ev, init_m, init_order, init_t,
        shadow;
    uint64_t ev_stride;
    uint64_t rec;
    uint64_t seg;
    int seg_sets;
    uint64_t total;
};

Sizes workspace_sizes(int64_t BH, int64_t T, int64_t C, int64_t dk, int64_t dv)
{
    const int64_t NT = (T + kScoreTile - 1) / kScoreTile;
    const int64_t NCH = (T + kChunk - 1) / kChunk;
    Sizes z;
    z.s = align_up(4ull * BH * T, 256);
    z.qs = align_up(8ull * BH * T, 256);
    z.flag = align_up(1ull * BH * T, 256);
    z.tile_cnt = align_up(4ull * BH * NT, 256);
    z.tile_sum = align_up(8ull * BH * NT, 256);
    z.seg_t = align_up(4ull * BH * (T + 1), 256);
    z.seg_P = align_up(8ull * BH * (T + 1), 256);
    z.seg_q0 = align_up(8ull * BH * T, 256);
    z.nseg = align_up(4ull * BH, 256);
    z.ev_stride = static_cast<uint64_t>(std::max<int64_t>(T, kChunk));
    z.events = align_up(8ull * BH * z.ev_stride, 256);
    z.chunk_ev = align_up(4ull * BH * (NCH + 1), 256);
    z.init_m = align_up(4ull * BH, 256);
    z.init_order = align_up(64ull * BH, 256);
    z.init_t = align_up(8ull * BH, 256);
    z.shadow = align_up(2ull * BH * C * dv * dk, 256);
    // chunk records (register-resident path), or the fp32 working copy of a
    // bf16-state cache's states (streamed path)
    z.rec = align_up(std::max<uint64_t>(static_cast<uint64_t>(BH) * NCH * rs_record_bytes(dk), 4ull * BH * C * dv * dk), 256);
    // slots of the block sets of a sweep split along the sequence (one per
    // set but the last): only for a grid of at most 256 blocks of the
    // register-resident sweep (16 value columns per block), at most one set
    // per 8 chunks; last in the workspace, so that the allocation-free call
    // can leave them out and run unsplit
    z.seg_sets = (C <= 32 && dk <= 128 && BH * ((dv + 15) / 16) <= 256)
                     ? static_cast<int>(std::min<int64_t>(kSegScratch, std::max<int64_t>(0, NCH / 8 - 1)))
                     : 0;
    z.seg = align_up(4ull * z.seg_sets * BH * C * dv * dk, 256);
    z.total = z.s + z.qs + z.flag + z.tile_cnt + z.tile_sum + z.seg_t + z.seg_P + z.seg_q0 + z.nseg +
              z.events + z.chunk_ev + z.init_m + z.init_order + z.init_t + z.shadow + z.rec + z.seg;
    return z;
}

Workspace carve(void *base, const Sizes &z, bool with_seg)
{
    uint8_t *p = static_cast<uint8_t *>(base);
    Workspace w;
    w.s = reinterpret_cast<float *>(p); p += z.s;
    w.qs = reinterpret_cast<int64_t *>(p); p += z.qs;
    w.flag = p; p += z.flag;
    w.tile_cnt = reinterpret_cast<int32_t *>(p); p += z.tile_cnt;
    w.tile_sum = reinterpret_cast<int64_t *>(p); p += z.tile_sum;
    w.seg_t = reinterpret_cast<int32_t *>(p); p += z.seg_t;
    w.seg_P = reinterpret_cast<int64_t *>(p); p += z.seg_P;
    w.seg_q0 = reinterpret_cast<int64_t *>(p); p += z.seg_q0;
    w.nseg = reinterpret_cast<int32_t *>(p); p += z.nseg;
    w.events = reinterpret_cast<int2 *>(p); p += z.events;
    w.chunk_ev = reinterpret_cast<int32_t *>(p); p += z.chunk_ev;
    w.init_m = reinterpret_cast<int32_t *>(p); p += z.init_m;
    w.init_order = p; p += z.init_order;
    w.init_t = reinterpret_cast<int64_t *>(p); p += z.init_t;
    w.ev_stride = z.ev_stride;
    w.shadow = p; p += z.shadow;
    w.rec = p;
    w.work = reinterpret_cast<float *>(p);
    p += z.rec;
    w.seg_states = with_seg && z.seg ? reinterpret_cast<float *>(p) : nullptr;
    w.seg_sets = with_seg ? z.seg_sets : 0;
    p += z.seg;
    (void)p;
    return w;
}

// Offsets of a cache buffer's parts: the slots (fp32, or bf16 closed states),
// the fp32 active-state region (bf16 storage only; empty otherwise) and the
// per-stream metadata.
struct CacheOffsets {
    uint64_t states, active, meta, total;
};

CacheOffsets cache_offsets(int64_t BH, int64_t C, int64_t dk, int64_t dv, bool bf16)
{
    CacheOffsets o;
    o.states = 0;
    o.active = align_up((bf16 ? 2ull : 4ull) * BH * C * dv * dk, 256);
    o.meta = align_up(o.active + (bf16 ? 4ull * BH * dv * dk : 0ull), 256);
    o.total = o.meta + BH * meta_stride_bytes(dk);
    return o;
}

bool valid_state_dtype(int d) { return d == DLA_F32 || d == DLA_BF16; }

dla_status check_cache(const dla_cache *c)
{
    if (!c) return fail(DLA_ERR_ARG, "cache is NULL");
    dla_status s = check_shape(c->B, c->H, c->C, c->d_k, c->d_v);
    if (s != DLA_OK) return s;
    if (!c->base || !aligned(c->base, 256)) return fail(DLA_ERR_ARG, "cache base is NULL or not 256-byte aligned");
    if (!valid_state_dtype(c->state_dtype)) return fail(DLA_ERR_ARG, "unknown state dtype %d", c->state_dtype);
    if (c->bytes < dla_cache_bytes(c->B, c->H, c->C, c->d_k, c->d_v, static_cast<dla_dtype>(c->state_dtype)))
        return fail(DLA_ERR_ARG, "cache buffer too small (%llu bytes)", static_cast<unsigned long long>(c->bytes));
    if (c->merge_rule != DLA_MERGE_SUM && c->merge_rule != DLA_MERGE_DENSITY && c->merge_rule != DLA_FENWICK)
        return fail(DLA_ERR_ARG, "unknown merge rule %d", c->merge_rule);
    if (c->score_rule != DLA_SCORE_COSINE && c->score_rule != DLA_SCORE_STATE)
        return fail(DLA_ERR_ARG, "unknown score rule %d", c->score_rule);
    return DLA_OK;
}

// Shapes the state information score supports (its schedule kernel holds a
// stream's current state in registers and the chunk in LDS).
dla_status check_state_score(const dla_cache *c, bool io_bf16)
{
    if (c->score_rule != DLA_SCORE_STATE || c->merge_rule == DLA_FENWICK) return DLA_OK;
    const bool w = (c->d_v == 64 || c->d_v == 128 || c->d_v == 256);
    if (!w) return fail(DLA_ERR_UNSUPPORTED, "the state score supports d_v in {64, 128, 256} (got %d)", c->d_v);
    if (!io_bf16 && (c->d_k > 128 || c->d_v > 128))
        return fail(DLA_ERR_UNSUPPORTED, "the state score with float32 io supports d_k, d_v in {64, 128}");
    if (c->d_k == 256 && c->d_v == 256)
        return fail(DLA_ERR_UNSUPPORTED,
                    "the state score at d_k = d_v = 256 is not supported (the current state, 64 K floats, held by "
                    "one block's registers, would spill)");
    return DLA_OK;
}

CacheGeom geom(const dla_cache *c)
{
    CacheGeom g;
    g.B = c->B; g.H = c->H; g.C = c->C; g.dk = c->d_k; g.dv = c->d_v;
    g.state_bf16 = c->state_dtype == DLA_BF16;
    g.meta_stride = meta_stride_bytes(c->d_k);
    return g;
}

dla_status hip_status(hipError_t e, const char *what)
{
    if (e == hipSuccess) return ok();
    return fail(DLA_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

int choose_dvt(int64_t BH, int dv)
{
    if (g_dvt_override != 0 && dv % g_dvt_override == 0) return g_dvt_override;
    if (dv % 32 != 0) return 16;
    // prefer the wider slice when it still gives about one block per compute unit
    return BH * (dv / 32) >= 200 ? 32 : 16;
}

// Which chunk kernel a prefill of this shape runs, with its value-column
// slice width and LDS need.  bf16 inputs with C <= 32 and d_k <= 128 keep the
// state stack in registers; the streamed kernel covers the rest (or every
// shape while dla_set_prefill_path asks for it on this thread).  The streamed
// kernel takes 32-column slices only where their LDS fits a compute unit.
struct PrefillPlan {
    int register_resident;
    int dvt;
    size_t lds;
    char name[48];
};

PrefillPlan plan_prefill(bool io_bf16, int64_t BH, int C, int dk, int dv)
{
    PrefillPlan p;
    p.dvt = choose_dvt(BH, dv);
    p.register_resident = io_bf16 && C <= 32 && dk <= 128 && g_path_override != DLA_PATH_STREAMED;
    if (p.register_resident) {
        p.dvt = prefill_rs_dvt(dk, C, p.dvt);
        p.lds = prefill_rs_smem_bytes(dk, p.dvt, C);
        const int spw = prefill_rs_spw(C);
        std::snprintf(p.name, sizeof(p.name), "k_prefill_rs<%d,%d,%d>", dk, p.dvt, spw);
    } else {
        if (p.dvt == 32 && prefill_smem_bytes(io_bf16, dk, 32) > kLdsBytes) p.dvt = 16;
        p.lds = prefill_smem_bytes(io_bf16, dk, p.dvt);
        std::snprintf(p.name, sizeof(p.name), "k_prefill<%s,%d,%d>", io_bf16 ? "bf16" : "f32", dk, p.dvt);
    }
    return p;
}

thread_local char g_kernel_name[48];

// Static scratch of dla_prefill_noalloc: the prefill workspace for callers
// that cannot allocate.  One copy per device, held from the library's load on
// that device until the process ends.  Host code never passes the array's
// name to a kernel (on the host it is only a stand-in for the symbol): it uses
// the device address that hipGetSymbolAddress returns, looked up once per
// device with that device current.
static __device__ __align__(256) uint8_t scratch[DLA_NOALLOC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void *g_scratch_ptr[kMaxDevices];

// Block slots of the sweep on the current device (two blocks per compute
// unit), looked up once per device.
int g_block_slots[kMaxDevices];

dla_status device_block_slots(int *out)
{
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return fail(DLA_ERR_HIP, "hipGetDevice: %s", hipGetErrorString(e));
    if (dev < 0 || dev >= kMaxDevices) return fail(DLA_ERR_UNSUPPORTED, "device %d: at most %d devices", dev, kMaxDevices);
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_block_slots[dev]) {
        int cus = 0;
        e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
        if (e != hipSuccess || cus <= 0)
            return fail(DLA_ERR_HIP, "hipDeviceGetAttribute(compute units): %s", hipGetErrorString(e));
        g_block_slots[dev] = 2 * cus;
    }
    *out = g_block_slots[dev];
    return DLA_OK;
}

// The scratch address of the device current on this thread, which must be
// the device of `stream`.
dla_status device_scratch(hipStream_t stream, void **out)
{
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return fail(DLA_ERR_HIP, "hipGetDevice: %s", hipGetErrorString(e));
    if (dev < 0 || dev >= kMaxDevices) return fail(DLA_ERR_UNSUPPORTED, "device %d: at most %d devices", dev, kMaxDevices);
    if (stream) {
        hipDevice_t sdev = -1;
        e = hipStreamGetDevice(stream, &sdev);
        if (e != hipSuccess) return fail(DLA_ERR_HIP, "hipStreamGetDevice: %s", hipGetErrorString(e));
        if (sdev != dev)
            return fail(DLA_ERR_ARG, "the stream belongs to device %d, the current device is %d", sdev, dev);
    }
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch_ptr[dev]) {
        void *ptr = nullptr;
        e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
        if (e != hipSuccess || !ptr)
            return fail(DLA_ERR_HIP, "hipGetSymbolAddress(scratch): %s", hipGetErrorString(e));
        g_scratch_ptr[dev] = ptr;
    }
    *out = g_scratch_ptr[dev];
    return DLA_OK;
}

}  // namespace

extern "C" {

int32_t dla_abi_version(void) { return DLA_ABI_VERSION; }

uint64_t dla_cache_bytes(int32_t B, int32_t H, int32_t C, int32_t d_k, int32_t d_v, dla_dtype state_dtype)
{
    char saved[sizeof(g_err)];
    std::memcpy(saved, g_err, sizeof(g_err));
    const bool bad = check_shape(B, H, C, d_k, d_v) != DLA_OK || !valid_state_dtype(state_dtype);
    std::memcpy(g_err, saved, sizeof(g_err));
    if (bad) return 0;
    return cache_offsets(static_cast<int64_t>(B) * H, C, d_k, d_v, state_dtype == DLA_BF16).total;
}

dla_status dla_cache_layout(int32_t B, int32_t H, int32_t C, int32_t d_k, int32_t d_v, dla_dtype state_dtype,
                            dla_cache_layout_t *out)
{
    dla_status s = check_shape(B, H, C, d_k, d_v);
    if (s != DLA_OK) return s;
    if (!valid_state_dtype(state_dtype)) return fail(DLA_ERR_ARG, "unknown state dtype %d", static_cast<int>(state_dtype));
    if (!out) return fail(DLA_ERR_ARG, "out is NULL");
    const CacheOffsets co = cache_offsets(static_cast<int64_t>(B) * H, C, d_k, d_v, state_dtype == DLA_BF16);
    out->states_offset = co.states;
    out->active_offset = co.active;
    out->meta_offset = co.meta;
    out->meta_stride = meta_stride_bytes(d_k);
    out->off_m = kOffM;
    out->off_has_prev = kOffHasPrev;
    out->off_s_prev = kOffSPrev;
    out->off_t_seen = kOffTSeen;
    out->off_order = kOffOrder;
    out->off_info = kOffInfo;
    out->off_count = kOffCount;
    out->off_start = kOffStart;
    out->off_k_prev = kOffKprev;
    return ok();
}

dla_status dla_cache_init(dla_cache *cache, void *base, uint64_t bytes, int32_t B, int32_t H, int32_t C,
                          int32_t d_k, int32_t d_v, dla_dtype state_dtype, const dla_cache_preload *preload,
                          void *stream)
{
    if (!cache) return fail(DLA_ERR_ARG, "cache is NULL");
    dla_status s = check_shape(B, H, C, d_k, d_v);
    if (s != DLA_OK) return s;
    if (!valid_state_dtype(state_dtype)) return fail(DLA_ERR_ARG, "unknown state dtype %d", static_cast<int>(state_dtype));
    if (!base || !aligned(base, 256)) return fail(DLA_ERR_ARG, "base is NULL or not 256-byte aligned");
    if (bytes < dla_cache_bytes(B, H, C, d_k, d_v, state_dtype))
        return fail(DLA_ERR_ARG, "buffer of %llu bytes is smaller than dla_cache_bytes",
                    static_cast<unsigned long long>(bytes));
    PreloadArgs pre = {0, nullptr, nullptr, nullptr, nullptr, 0};
    if (preload) {
        if (preload->m0 < 0 || preload->m0 > C) return fail(DLA_ERR_ARG, "preload m0 must be in [0, C]");
        if (preload->t_seen < 0) return fail(DLA_ERR_ARG, "preload t_seen must be >= 0");
        if (preload->m0 > 0) {
            if (!preload->states || !preload->info || !preload->count || !preload->start)
                return fail(DLA_ERR_ARG, "preload pointers must be non-NULL when m0 > 0");
            if (!aligned(preload->states, 16) || !aligned(preload->info, 8) || !aligned(preload->count, 4) ||
                !aligned(preload->start, 8))
                return fail(DLA_ERR_ARG, "preload pointers misaligned");
        }
        pre.m0 = preload->m0;
        pre.states = preload->states;
        pre.info = preload->info;
        pre.count = preload->count;
        pre.start = preload->start;
        pre.t_seen = preload->t_seen;
    }
    cache->B = B; cache->H = H; cache->C = C; cache->d_k = d_k; cache->d_v = d_v;
    cache->merge_rule = DLA_MERGE_SUM;
    cache->state_dtype = state_dtype;
    cache->score_rule = DLA_SCORE_COSINE;
    cache->base = base;
    cache->bytes = bytes;
    const CacheGeom g = geom(cache);
    const CacheOffsets co = cache_offsets(static_cast<int64_t>(B) * H, C, d_k, d_v, g.state_bf16);
    uint8_t *b8 = static_cast<uint8_t *>(base);
    float *states = reinterpret_cast<float *>(b8 + co.states);
    float *active = g.state_bf16 ? reinterpret_cast<float *>(b8 + co.active) : nullptr;
    uint8_t *meta = b8 + co.meta;
    return hip_status(launch_cache_init(states, active, meta, g, pre, static_cast<hipStream_t>(stream)),
                      "cache init launch");
}

dla_status dla_cache_set_merge_rule(dla_cache *cache, int32_t rule)
{
    if (!cache) return fail(DLA_ERR_ARG, "cache is NULL");
    if (rule != DLA_MERGE_SUM && rule != DLA_MERGE_DENSITY && rule != DLA_FENWICK)
        return fail(DLA_ERR_ARG, "unknown merge rule %d", rule);
    cache->merge_rule = rule;
    return ok();
}

uint64_t dla_prefill_workspace_bytes(int32_t B, int32_t H, int32_t T, int32_t C, int32_t d_k, int32_t d_v)
{
    char saved[sizeof(g_err)];
    std::memcpy(saved, g_err, sizeof(g_err));
    const bool bad = check_shape(B, H, C, d_k, d_v) != DLA_OK || T < 1 || T > (1 << 24);
    std::memcpy(g_err, saved, sizeof(g_err));
    if (bad) return 0;
    return workspace_sizes(static_cast<int64_t>(B) * H, T, C, d_k, d_v).total;
}

}  // extern "C"

namespace {

// Every check of a prefill call, then the launches.  With `scratch_only` the
// workspace is the library's static scratch of the stream's device (the
// arguments workspace and workspace_bytes are ignored): the call allocates
// nothing.
dla_status prefill_call(const void *q, const void *k, const void *v, const void *lam, void *o, int32_t T, float tau,
                        dla_dtype io, const dla_cache *cache, void *workspace, uint64_t workspace_bytes,
                        const dla_schedule_out *sched, void *stream, bool scratch_only)
{
    dla_status s = check_cache(cache);
    if (s != DLA_OK) return s;
    if (!q || !k || !v || !lam || !o) return fail(DLA_ERR_ARG, "q, k, v, lam and o must be non-NULL");
    if (!aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16) || !aligned(lam, 16) || !aligned(o, 16))
        return fail(DLA_ERR_ARG, "q, k, v, lam and o must be 16-byte aligned");
    if (T < 1 || T > (1 << 24)) return fail(DLA_ERR_ARG, "T must be in [1, 2^24] (got %d)", T);
    if (io != DLA_F32 && io != DLA_BF16) return fail(DLA_ERR_ARG, "unknown io dtype %d", static_cast<int>(io));
    if (io == DLA_F32 && cache->d_k > 128)
        return fail(DLA_ERR_UNSUPPORTED,
                    "float32 prefill supports d_k in {64, 128} (the streamed kernel's chunk operands at d_k = 256 "
                    "need %zu bytes of LDS, a compute unit has %zu)",
                    prefill_smem_bytes(0, 256, 16), kLdsBytes);
    if (tau != tau) return fail(DLA_ERR_ARG, "tau is NaN");
    if (sched && ((sched->ev_t == nullptr) != (sched->ev_i == nullptr)))
        return fail(DLA_ERR_ARG, "schedule export: ev_t and ev_i go together");
    const int64_t BH = static_cast<int64_t>(cache->B) * cache->H;
    const Sizes z = workspace_sizes(BH, T, cache->C, cache->d_k, cache->d_v);
    // (the allocation-free call runs the sweep unsplit when the split's slots
    // do not fit its scratch)
    bool with_seg = true;
    if (scratch_only) {
        if (z.total - z.seg > DLA_NOALLOC_SCRATCH_BYTES)
            return fail(DLA_ERR_WORKSPACE,
                        "this call needs %llu bytes of scratch; the static scratch holds %llu (use dla_prefill "
                        "with a workspace)",
                        static_cast<unsigned long long>(z.total - z.seg),
                        static_cast<unsigned long long>(DLA_NOALLOC_SCRATCH_BYTES));
        with_seg = z.total <= DLA_NOALLOC_SCRATCH_BYTES;
    } else {
        if (!workspace || !aligned(workspace, 256))
            return fail(DLA_ERR_WORKSPACE, "workspace NULL or not 256-byte aligned");
        if (workspace_bytes < z.total)
            return fail(DLA_ERR_WORKSPACE, "workspace of %llu bytes, %llu needed",
                        static_cast<unsigned long long>(workspace_bytes), static_cast<unsigned long long>(z.total));
    }
    PrefillArgs a;
    a.q = q; a.k = k; a.v = v; a.lam = lam; a.o = o;
    a.T = T;
    a.tau = tau;
    a.io_bf16 = io == DLA_BF16;
    a.merge_rule = cache->merge_rule;
    a.score_rule = cache->merge_rule == DLA_FENWICK ? DLA_SCORE_COSINE : cache->score_rule;
    s = check_state_score(cache, a.io_bf16);
    if (s != DLA_OK) return s;
    if (a.score_rule == DLA_SCORE_STATE && state_score_smem_bytes(a.io_bf16, cache->d_k, cache->d_v) > kLdsBytes)
        return fail(DLA_ERR_UNSUPPORTED, "the state score's chunk operands at this shape need more LDS than a compute unit has");
    const PrefillPlan plan = plan_prefill(a.io_bf16, BH, cache->C, cache->d_k, cache->d_v);
    a.dvt = plan.dvt;
    a.register_resident = plan.register_resident;
    if (plan.lds > kLdsBytes)
        return fail(DLA_ERR_UNSUPPORTED, "shape needs more LDS than a compute unit has");
    a.g = geom(cache);
    if (a.merge_rule == DLA_FENWICK) {
        const int levels = bit_length(T - 1) + 1;
        if (cache->C < levels)
            return fail(DLA_ERR_ARG, "the fixed schedule over %d tokens needs C >= %d levels (C = %d)", T, levels,
                        cache->C);
        // every bucket is built by a cascade of merges, and with bf16 storage
        // each one re-rounds the closed values it reads: about one rounding per
        // carry level, past the bf16 output gate already at T ~ 1500
        if (a.g.state_bf16)
            return fail(DLA_ERR_UNSUPPORTED, "the fixed schedule needs float32 state storage");
        if (sched && (sched->s || sched->boundary || sched->seg_id || sched->m_t || sched->ev_t || sched->ev_i ||
                      sched->n_ev))
            return fail(DLA_ERR_UNSUPPORTED, "no schedule export for the fixed schedule");
    }
    const CacheOffsets co = cache_offsets(BH, cache->C, cache->d_k, cache->d_v, a.g.state_bf16);
    uint8_t *b8 = static_cast<uint8_t *>(cache->base);
    a.states = reinterpret_cast<float *>(b8 + co.states);
    a.active = a.g.state_bf16 ? reinterpret_cast<float *>(b8 + co.active) : nullptr;
    a.meta = b8 + co.meta;
    hipStream_t st = static_cast<hipStream_t>(stream);
    if (scratch_only) {
        dla_status ss = device_scratch(st, &workspace);
        if (ss != DLA_OK) return ss;
    }
    a.ws = carve(workspace, z, with_seg);
    a.seg_slots = 0;
    if (a.register_resident && g_path_override != DLA_PATH_UNSPLIT) {
        s = device_block_slots(&a.seg_slots);
        if (s != DLA_OK) return s;
    }
    a.ev_before = g_ev_before;
    a.ev_after = g_ev_after;
    if (sched) a.sched = *sched;
    else std::memset(&a.sched, 0, sizeof(a.sched));
    // schedule fields the prefill kernels never fill are ignored; s and boundary
    // are copied from the workspace afterwards
    hipError_t e = launch_prefill(a, st);
    if (e != hipSuccess) return hip_status(e, "prefill launch");
    if (sched && sched->s) {
        e = hipMemcpyAsync(sched->s, a.ws.s, 4ull * BH * T, hipMemcpyDeviceToDevice, st);
        if (e != hipSuccess) return hip_status(e, "schedule copy");
    }
    if (sched && sched->boundary) {
        e = hipMemcpyAsync(sched->boundary, a.ws.flag, 1ull * BH * T, hipMemcpyDeviceToDevice, st);
        if (e != hipSuccess) return hip_status(e, "schedule copy");
    }
    return ok();
}

}  // namespace

extern "C" {

dla_status dla_prefill(const void *q, const void *k, const void *v, const void *lam, void *o, int32_t T,
                       float tau, dla_dtype io, const dla_cache *cache, void *workspace,
                       uint64_t workspace_bytes, const dla_schedule_out *sched, void *stream)
{
    return prefill_call(q, k, v, lam, o, T, tau, io, cache, workspace, workspace_bytes, sched, stream, false);
}

dla_status dla_prefill_noalloc(const void *q, const void *k, const void *v, const void *lam, void *o, int32_t T,
                               float tau, dla_dtype io, const dla_cache *cache, const dla_schedule_out *sched,
                               void *stream)
{
    return prefill_call(q, k, v, lam, o, T, tau, io, cache, nullptr, 0, sched, stream, true);
}

const char *dla_prefill_kernel(dla_dtype io, int32_t B, int32_t H, int32_t C, int32_t d_k, int32_t d_v)
{
    char saved[sizeof(g_err)];
    std::memcpy(saved, g_err, sizeof(g_err));
    const bool bad = check_shape(B, H, C, d_k, d_v) != DLA_OK || (io != DLA_F32 && io != DLA_BF16);
    std::memcpy(g_err, saved, sizeof(g_err));
    if (bad) return nullptr;
    const PrefillPlan p = plan_prefill(io == DLA_BF16, static_cast<int64_t>(B) * H, C, d_k, d_v);
    std::memcpy(g_kernel_name, p.name, sizeof(g_kernel_name));
    return g_kernel_name;
}

dla_status dla_decode_step(const void *q, const void *k, const void *v, const void *lam, void *o, float tau,
                           dla_dtype io, const dla_cache *cache, const dla_schedule_out *sched, void *stream)
{
    dla_status s = check_cache(cache);
    if (s != DLA_OK) return s;
    if (!q || !k || !v || !lam || !o) return fail(DLA_ERR_ARG, "q, k, v, lam and o must be non-NULL");
    if (!aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16) || !aligned(lam, 16) || !aligned(o, 16))
        return fail(DLA_ERR_ARG, "q, k, v, lam and o must be 16-byte aligned");
    if (io != DLA_F32 && io != DLA_BF16) return fail(DLA_ERR_ARG, "unknown io dtype %d", static_cast<int>(io));
    if (cache->d_v != 64 && cache->d_v != 128 && cache->d_v != 256)
        return fail(DLA_ERR_UNSUPPORTED, "decode supports d_v in {64, 128, 256} (got %d)", cache->d_v);
    if (cache->merge_rule == DLA_FENWICK) {
        if (cache->state_dtype != DLA_F32)
            return fail(DLA_ERR_UNSUPPORTED, "the fixed schedule needs float32 state storage");
        if (sched && (sched->s || sched->boundary || sched->m_t || sched->ev_i))
            return fail(DLA_ERR_UNSUPPORTED, "no schedule export for the fixed schedule");
    }
    if (tau != tau) return fail(DLA_ERR_ARG, "tau is NaN");
    DecodeArgs a;
    a.q = q; a.k = k; a.v = v; a.lam = lam; a.o = o;
    a.tau = tau;
    a.io_bf16 = io == DLA_BF16;
    a.merge_rule = cache->merge_rule;
    a.score_rule = cache->merge_rule == DLA_FENWICK ? DLA_SCORE_COSINE : cache->score_rule;
    s = check_state_score(cache, a.io_bf16);
    if (s != DLA_OK) return s;
    a.g = geom(cache);
    const int64_t BH = static_cast<int64_t>(cache->B) * cache->H;
    const CacheOffsets co = cache_offsets(BH, cache->C, cache->d_k, cache->d_v, a.g.state_bf16);
    uint8_t *b8 = static_cast<uint8_t *>(cache->base);
    a.states = reinterpret_cast<float *>(b8 + co.states);
    a.active = a.g.state_bf16 ? reinterpret_cast<float *>(b8 + co.active) : nullptr;
    a.meta = b8 + co.meta;
    a.sched.s = sched ? sched->s : nullptr;
    a.sched.boundary = sched ? sched->boundary : nullptr;
    a.sched.m_t = sched ? sched->m_t : nullptr;
    a.sched.ev_i = sched ? sched->ev_i : nullptr;
    return hip_status(launch_decode(a, static_cast<hipStream_t>(stream)), "decode launch");
}

dla_status dla_cache_set_score_rule(dla_cache *cache, int32_t rule)
{
    if (!cache) return fail(DLA_ERR_ARG, "cache is NULL");
    if (rule != DLA_SCORE_COSINE && rule != DLA_SCORE_STATE) return fail(DLA_ERR_ARG, "unknown score rule %d", rule);
    cache->score_rule = rule;
    return ok();
}

dla_status dla_set_prefill_path(int32_t path, int32_t value_columns)
{
    if (path != DLA_PATH_AUTO && path != DLA_PATH_STREAMED && path != DLA_PATH_UNSPLIT)
        return fail(DLA_ERR_ARG, "unknown prefill path %d", path);
    if (value_columns != 0 && value_columns != 16 && value_columns != 32)
        return fail(DLA_ERR_ARG, "value_columns must be 0, 16 or 32 (got %d)", value_columns);
    g_path_override = path;
    g_dvt_override = value_columns;
    return ok();
}

dla_status dla_set_prefill_events(void *before, void *after)
{
    if ((before == nullptr) != (after == nullptr))
        return fail(DLA_ERR_ARG, "pass both events or neither");
    g_ev_before = static_cast<hipEvent_t>(before);
    g_ev_after = static_cast<hipEvent_t>(after);
    return ok();
}

const char *dla_status_str(dla_status s)
{
    switch (s) {
    case DLA_OK: return "ok";
    case DLA_ERR_ARG: return "invalid argument";
    case DLA_ERR_UNSUPPORTED: return "unsupported shape or dtype";
    case DLA_ERR_WORKSPACE: return "workspace missing or too small";
    case DLA_ERR_HIP: return "HIP error";
    }
    return "unknown status";
}

const char *dla_last_error(void) { return g_err; }

}  // extern "C"
