// dla_internal.h -- definitions shared by the host ABI and the kernels of
// libdla (cache metadata layout, workspace carving, launcher signatures).
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "dla.h"

namespace dla {

constexpr int kChunk = DLA_CHUNK;   // tokens per prefill chunk (mask width)
constexpr int kMaxC = DLA_MAX_C;    // lanes of the greedy wave = largest capacity
constexpr int kScoreTile = 256;     // tokens per block of the score/compaction passes

// Per-stream metadata record (see dla.h for the meaning of each field).
struct MetaHead {
    int32_t m;
    int32_t has_prev;
    float s_prev;
    int32_t pad0;
    int64_t t_seen;
    int64_t pad1;
};
static_assert(sizeof(MetaHead) == 32, "metadata head is 32 bytes");
constexpr uint32_t kOffM = 0;
constexpr uint32_t kOffHasPrev = 4;
constexpr uint32_t kOffSPrev = 8;
constexpr uint32_t kOffTSeen = 16;
constexpr uint32_t kOffOrder = 32;                     // uint8[64]
constexpr uint32_t kOffInfo = kOffOrder + 64;          // int64[64]
constexpr uint32_t kOffCount = kOffInfo + 8 * 64;      // int32[64]
constexpr uint32_t kOffStart = kOffCount + 4 * 64;     // int64[64]
constexpr uint32_t kOffKprev = kOffStart + 8 * 64;     // float[d_k]

inline uint64_t align_up(uint64_t x, uint64_t a) { return (x + a - 1) / a * a; }
inline uint64_t meta_stride_bytes(int dk) { return align_up(kOffKprev + 4ull * dk, 256); }

struct CacheGeom {
    int B, H, C, dk, dv;
    int state_bf16;     // closed states bf16 in their slots, the active one fp32 in its own region
    size_t meta_stride;
};

struct PreloadArgs {
    int m0;
    const float *states;
    const int64_t *info;
    const int32_t *count;
    const int64_t *start;
    int64_t t_seen;
};

// Prefill workspace, carved from one caller buffer (see carve_workspace).
struct Workspace {
    float *s;            // [BH][T] token information
    int64_t *qs;         // [BH][T] information, 2^-32 fixed point
    uint8_t *flag;       // [BH][T] boundary flags
    int32_t *tile_cnt;   // [BH][NT]
    int64_t *tile_sum;   // [BH][NT]
    int32_t *seg_t;      // [BH][T+1] boundary tokens (+ sentinel T)
    int64_t *seg_P;      // [BH][T+1] information before each boundary (+ total)
    int64_t *seg_q0;     // [BH][T] information of each boundary token
    int32_t *nseg;       // [BH]
    int2 *events;        // [BH][ev_stride] (token, state merged away or -1)
    size_t ev_stride;    // events per stream: max(T, 64) (fixed-schedule calls can have more events than tokens)
    int32_t *chunk_ev;   // [BH][NCH+1] first event of each chunk
    int32_t *init_m;     // [BH] live states when the call starts (saved by the greedy scan)
    uint8_t *init_order; // [BH][64] their physical slots, oldest first
    int64_t *init_t;     // [BH] position the call starts at (fixed schedule)
    void *shadow;        // [BH][C][dv][dk] fp16 copy of the states (bf16 io)
    // per-chunk operands built by the chunk pre-pass (register-resident path)
    // [BH][NCH] chunk records of the register-resident prefill, each
    // rs_record_bytes(d_k) long: fp16 query fragments [4][DK/32][64][8],
    // bf16 read weights [32][64] (row i: lam_t of the slot that the state
    // with chronological index i at the chunk start is read with at token t,
    // times 2^e for the query scaling 2^-e of the fragments), bf16 fragments
    // of (Q K^T) o W [4][2][64][8], bf16 fragments of K^T [DK/16][2][64][8]
    void *rec;
    // streamed path on a cache with bf16 closed states: the fp32 working copy
    // of the states [BH][C][dv][dk], in the same bytes as rec (unused there)
    float *work;
    // register-resident sweep split along the sequence: the slots of every
    // block set but the last [kSegScratch][BH][C][dv][dk] fp32 (NULL when the
    // shape's grid is too large to be split)
    float *seg_states;
    int seg_sets;        // block sets with slots there (the split has at most one more)
};
constexpr int kSegScratch = 3;  // block sets with slots of their own (at most 4 sets)
constexpr int kPrepCmax = 32;   // read-weight rows kept per chunk by the pre-pass
// chunk record of the register-resident prefill: query fragments, read weights,
// weighted-score fragments, key fragments (bytes; each part a multiple of 16)
constexpr size_t rs_rec_q_bytes(int dk) { return 2ull * 64 * dk; }
constexpr size_t rs_rec_a_bytes(int dk) { return rs_rec_q_bytes(dk) + 2ull * 32 * 64; }
constexpr size_t rs_rec_b_bytes(int dk) { return 2ull * 64 * 64 + 2ull * 64 * dk; }
constexpr size_t rs_record_bytes(int dk) { return rs_rec_a_bytes(dk) + rs_rec_b_bytes(dk); }

struct PrefillArgs {
    const void *q, *k, *v, *lam;
    void *o;
    int T;
    float tau;
    int io_bf16;
    int merge_rule;                   // DLA_MERGE_SUM, DLA_MERGE_DENSITY or DLA_FENWICK
    int score_rule;                   // DLA_SCORE_COSINE or DLA_SCORE_STATE
    int dvt;
    CacheGeom g;
    float *states;                    // slots (bf16 data when g.state_bf16)
    float *active;                    // [BH][dv][dk] fp32 active states (g.state_bf16), else NULL
    uint8_t *meta;
    Workspace ws;
    dla_schedule_out sched;
    hipEvent_t ev_before, ev_after;   // optional, recorded around the chunk kernel
    int register_resident;            // 1: k_prefill_rs, 0: k_prefill (states streamed)
    int seg_slots;                    // block slots of the device (two per compute unit) for
                                      // splitting a small sweep grid along the sequence; 0: no split
};

struct DecodeSched {
    float *s;
    uint8_t *boundary;
    int32_t *m_t;
    int32_t *ev_i;
};

struct DecodeArgs {
    const void *q, *k, *v, *lam;
    void *o;
    float tau;
    int io_bf16;
    int merge_rule;                   // DLA_MERGE_SUM or DLA_MERGE_DENSITY
    int score_rule;                   // DLA_SCORE_COSINE or DLA_SCORE_STATE
    CacheGeom g;
    float *states;                    // slots (bf16 data when g.state_bf16)
    float *active;                    // [BH][dv][dk] fp32 active states (g.state_bf16), else NULL
    uint8_t *meta;
    DecodeSched sched;
};

hipError_t launch_cache_init(float *states, float *active, uint8_t *meta, const CacheGeom &g,
                             const PreloadArgs &pre, hipStream_t stream);
hipError_t launch_prefill(const PrefillArgs &a, hipStream_t stream);
hipError_t launch_decode(const DecodeArgs &a, hipStream_t stream);
size_t prefill_smem_bytes(int io_bf16, int dk, int dvt);
hipError_t launch_prefill_rs(const PrefillArgs &a, hipStream_t stream);
hipError_t launch_fenwick_schedule(const PrefillArgs &a, hipStream_t stream);
hipError_t launch_fen_refused(const PrefillArgs &a, hipStream_t stream);   // NaN outputs of refused streams
size_t prefill_rs_smem_bytes(int dk, int dvt, int C);
hipError_t launch_state_score(const PrefillArgs &a, hipStream_t stream);   // scores of the state rule
size_t state_score_smem_bytes(int io_bf16, int dk, int dv);
int prefill_rs_dvt(int dk, int C, int dvt_wanted);
int prefill_rs_spw(int C);      // closed-state slots per wave of the register-resident sweep

}  // namespace dla
