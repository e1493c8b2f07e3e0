// dla_kernels.hip -- gfx950 kernels of the Dynamic Linear Attention (DLA)
// layer forward pass: token score, boundary compaction, greedy capacity scan,
// chunked MFMA prefill, streaming decode step, cache initialisation.
//
// Method (reading notes "Dynamic Linear Attention | Chlience Paper Archive"):
//   section 5.1  per-token state v k^T; a low-information token joins the
//                current state, otherwise it opens a new one;
//   section 5.2  at most C states, chronological; when over capacity the
//                adjacent pair with the least information is merged
//                (S_i += S_{i+1}, counts and information summed);
//   section 5.3  o_t = sum_i lam_{t,i} S_i q_t over the bounded cache;
//   section 1    the state already holds token t when o_t is read.
// ai-feeds.com summary "Dynamic Linear Attention", method section: the
// information signal may be the feature change of the key, two consecutive
// low-information tokens merge, and a merged state keeps its original
// timestamp.  The fixed choices (cosine score, summed-information key,
// slot-indexed lam) are listed in include/dla.h.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <stdint.h>

#include "dla_device.h"
#include "dla_internal.h"

namespace dla {

// ------------------------------------------------------------ cache init

// One block per stream: metadata reset, optional preload of the first m0 states.
__global__ __launch_bounds__(256) void k_cache_init(float *__restrict__ states, float *__restrict__ active,
                                                     uint8_t *__restrict__ meta_base,
                                                     CacheGeom g, PreloadArgs pre)
{
    const int bh = blockIdx.x;
    const int tid = threadIdx.x;
    uint8_t *meta = meta_base + static_cast<size_t>(bh) * g.meta_stride;
    MetaHead *head = reinterpret_cast<MetaHead *>(meta);
    uint8_t *order = meta + kOffOrder;
    int64_t *info = reinterpret_cast<int64_t *>(meta + kOffInfo);
    int32_t *count = reinterpret_cast<int32_t *>(meta + kOffCount);
    int64_t *start = reinterpret_cast<int64_t *>(meta + kOffStart);
    float *kprev = reinterpret_cast<float *>(meta + kOffKprev);
    const int m0 = pre.m0;
    if (tid == 0) {
        head->m = m0;
        head->has_prev = 0;
        head->s_prev = 1.0f;
        head->pad0 = 0;
        head->t_seen = pre.t_seen;
        head->pad1 = 0;
    }
    if (tid < kMaxC) {
        order[tid] = static_cast<uint8_t>(tid);
        const bool live = tid < m0;
        info[tid] = live ? pre.info[static_cast<size_t>(bh) * m0 + tid] : 0;
        count[tid] = live ? pre.count[static_cast<size_t>(bh) * m0 + tid] : 0;
        start[tid] = live ? pre.start[static_cast<size_t>(bh) * m0 + tid] : 0;
    }
    for (int i = tid; i < g.dk; i += blockDim.x) kprev[i] = 0.0f;
    if (m0 > 0 && !g.state_bf16) {
        const size_t n4 = static_cast<size_t>(m0) * g.dv * g.dk / 4;
        const float4 *src = reinterpret_cast<const float4 *>(pre.states) + bh * n4;
        float4 *dst = reinterpret_cast<float4 *>(states) +
                      static_cast<size_t>(bh) * g.C * g.dv * g.dk / 4;
        for (size_t i = tid; i < n4; i += blockDim.x) dst[i] = src[i];
    } else if (m0 > 0) {
        // closed states (all but the most recent) rounded to bf16 into slots
        // 0 .. m0 - 2; the most recent one stays fp32 in the active region
        const size_t ss4 = static_cast<size_t>(g.dv) * g.dk / 4;     // one state, in float4
        const float4 *src = reinterpret_cast<const float4 *>(pre.states) + bh * m0 * ss4;
        uint2 *dst = reinterpret_cast<uint2 *>(states) + static_cast<size_t>(bh) * g.C * ss4;
        for (size_t i = tid; i < (m0 - 1) * ss4; i += blockDim.x) dst[i] = pack_bf16x4(src[i]);
        float4 *act = reinterpret_cast<float4 *>(active) + static_cast<size_t>(bh) * ss4;
        for (size_t i = tid; i < ss4; i += blockDim.x) act[i] = src[(m0 - 1) * ss4 + i];
    }
}

// ------------------------------------------------------------ token score

// Grid (tiles of 256 tokens, streams).  s_t = 1 - cos(k_t, k_{t-1}) from
// double sums; boundary b_t = empty cache or not (s_t < tau and s_{t-1} < tau);
// per-tile boundary count and information sum for the compaction pass.
template <typename TIO, int DK>
__global__ __launch_bounds__(256) void k_score(const TIO *__restrict__ K, int T, float tau,
                                               float *__restrict__ s_out,
                                               int64_t *__restrict__ qs_out,
                                               uint8_t *__restrict__ flag_out,
                                               int32_t *__restrict__ tile_cnt,
                                               int64_t *__restrict__ tile_sum, int NT,
                                               const uint8_t *__restrict__ meta_base, size_t meta_stride)
{
    constexpr int G = DK / 8;        // lanes per token, 8 elements each
    constexpr int TPW = 64 / G;      // tokens per wave pass
    __shared__ float s_lds[kScoreTile + 1];
    __shared__ int32_t red_c[4];
    __shared__ int64_t red_q[4];
    const int bh = blockIdx.y, tile = blockIdx.x;
    const int t0 = tile * kScoreTile;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int gi = lane / G, gl = lane % G;
    const TIO *Kb = K + static_cast<size_t>(bh) * T * DK;
    // the stream as the cache leaves it: token 0 is scored against its last
    // key (if it has seen one) and is a boundary only by the usual rule
    // unless the cache is empty
    const uint8_t *meta = meta_base + static_cast<size_t>(bh) * meta_stride;
    const MetaHead *head = reinterpret_cast<const MetaHead *>(meta);
    const float *kprev = reinterpret_cast<const float *>(meta + kOffKprev);
    const int has_prev = head->has_prev, m_init = head->m;
    const float s_prev = head->s_prev;

    // j indexes tokens t0 - 1 .. t0 + 255
    for (int base = wave * TPW; base < kScoreTile + 1; base += 4 * TPW) {
        const int j = base + gi;
        const int t = t0 - 1 + j;
        const bool valid = j < kScoreTile + 1 && t >= 0 && t < T;
        double d = 0.0, a = 0.0, b = 0.0;
        if (valid && t > 0) {
            const TIO *kt = Kb + static_cast<size_t>(t) * DK + gl * 8;
            const TIO *kp = kt - DK;
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                const double x = to_f(kt[e]);
                const double y = to_f(kp[e]);
                d += x * y;
                a += x * x;
                b += y * y;
            }
        } else if (valid && has_prev) {
            // token 0 of the call against the last key the cache kept
            const TIO *kt = Kb + gl * 8;
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                const double x = to_f(kt[e]);
                const double y = kprev[gl * 8 + e];
                d += x * y;
                a += x * x;
                b += y * y;
            }
        }
        d = group_sum_dpp<G>(d);
        a = group_sum_dpp<G>(a);
        b = group_sum_dpp<G>(b);
        if (valid && gl == 0) s_lds[j] = (t == 0 && !has_prev) ? 1.0f : cosine_distance(d, a, b);
    }
    __syncthreads();

    const int t = t0 + tid;
    int32_t c = 0;
    int64_t q = 0;
    if (t < T) {
        const float s = s_lds[tid + 1];
        const float sp = (t == 0) ? s_prev : s_lds[tid];
        const int bnd = (t == 0 && m_init == 0) || !((s < tau) && (sp < tau));
        q = fixed_point(s);
        const size_t row = static_cast<size_t>(bh) * T + t;
        s_out[row] = s;
        qs_out[row] = q;
        flag_out[row] = static_cast<uint8_t>(bnd);
        c = bnd;
    }
    c = wave_sum(c);
    q = wave_sum(q);
    if (lane == 0) { red_c[wave] = c; red_q[wave] = q; }
    __syncthreads();
    if (tid == 0) {
        tile_cnt[static_cast<size_t>(bh) * NT + tile] = red_c[0] + red_c[1] + red_c[2] + red_c[3];
        tile_sum[static_cast<size_t>(bh) * NT + tile] = red_q[0] + red_q[1] + red_q[2] + red_q[3];
    }
}

// ------------------------------------------------------ boundary compaction

// Grid (tiles, streams).  Lists every boundary token j of a stream with the
// exclusive prefix of information before it, so that the greedy scan sees
// whole segments (a boundary and the low tokens after it).
__global__ __launch_bounds__(256) void k_compact(int T, int NT, const uint8_t *__restrict__ flag,
                                                 const int64_t *__restrict__ qs,
                                                 const int32_t *__restrict__ tile_cnt,
                                                 const int64_t *__restrict__ tile_sum,
                                                 int32_t *__restrict__ seg_t,
                                                 int64_t *__restrict__ seg_P,
                                                 int64_t *__restrict__ seg_q0,
                                                 int32_t *__restrict__ nseg,
                                                 int32_t *__restrict__ seg_id_out)
{
    __shared__ int32_t wc[4];
    __shared__ int64_t wq[4];
    __shared__ int32_t base_c_s;
    __shared__ int64_t base_q_s;
    const int bh = blockIdx.y, tile = blockIdx.x;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;

    int32_t c = 0;
    int64_t p = 0;
    for (int i = tid; i < tile; i += 256) {
        c += tile_cnt[static_cast<size_t>(bh) * NT + i];
        p += tile_sum[static_cast<size_t>(bh) * NT + i];
    }
    c = wave_sum(c);
    p = wave_sum(p);
    if (lane == 0) { wc[wave] = c; wq[wave] = p; }
    __syncthreads();
    if (tid == 0) {
        base_c_s = wc[0] + wc[1] + wc[2] + wc[3];
        base_q_s = wq[0] + wq[1] + wq[2] + wq[3];
    }
    __syncthreads();
    const int32_t base_c = base_c_s;
    const int64_t base_q = base_q_s;

    const int t = tile * kScoreTile + tid;
    const size_t row = static_cast<size_t>(bh) * T + t;
    const int32_t f = (t < T) ? flag[row] : 0;
    const int64_t q = (t < T) ? qs[row] : 0;
    const int32_t fi = wave_incl_scan(f, lane);
    const int64_t qi = wave_incl_scan(q, lane);
    __syncthreads();
    if (lane == 63) { wc[wave] = fi; wq[wave] = qi; }
    __syncthreads();
    int32_t off_c = 0;
    int64_t off_q = 0;
    for (int w = 0; w < wave; ++w) { off_c += wc[w]; off_q += wq[w]; }
    const int32_t ex_c = base_c + off_c + fi - f;
    const int64_t ex_q = base_q + off_q + qi - q;
    const size_t sbase = static_cast<size_t>(bh) * (T + 1);
    if (t < T && f) {
        seg_t[sbase + ex_c] = t;
        seg_P[sbase + ex_c] = ex_q;
        seg_q0[static_cast<size_t>(bh) * T + ex_c] = q;
    }
    if (seg_id_out && t < T) seg_id_out[row] = ex_c + f - 1;
    if (tile == NT - 1 && tid == 255) {
        // totals of the whole stream: sentinel entry after the last segment
        const int32_t tot_c = ex_c + f;
        const int64_t tot_q = ex_q + q;
        nseg[bh] = tot_c;
        seg_t[sbase + tot_c] = T;
        seg_P[sbase + tot_c] = tot_q;
    }
}

// ----------------------------------------------------- greedy capacity scan

// One wave per stream; lane i holds live state i (oldest first).  Walks the
// segments in order: the boundary token is appended as a new state; if that
// leaves C+1 states the adjacent pair with the smallest summed information
// is merged (earliest pair on ties, the earlier start kept); the rest of the
// segment joins the most recent state.  Emits one event per boundary for the
// prefill kernel: (token, identity of the state merged away or -1), where the
// identity is its index among the states alive at its chunk's start, or
// 64 + its start offset within the chunk when it was opened in that chunk --
// except for a boundary whose new state the merge joins at once to the state
// before it (the newest pair): for the chunk kernels that is the token
// joining the most recent state, as a token without a boundary does.
__global__ __launch_bounds__(64) void k_greedy(int T, int C, int NCH,
                                               const int32_t *__restrict__ seg_t,
                                               const int64_t *__restrict__ seg_P,
                                               const int64_t *__restrict__ seg_q0,
                                               const int32_t *__restrict__ nseg_arr,
                                               int2 *__restrict__ events,
                                               int32_t *__restrict__ chunk_ev,
                                               const float *__restrict__ s_all,
                                               uint8_t *__restrict__ meta_base, size_t meta_stride,
                                               int32_t *__restrict__ ev_t_out,
                                               int32_t *__restrict__ ev_i_out,
                                               int32_t *__restrict__ n_ev_out, int merge_rule,
                                               int32_t *__restrict__ init_m_out,
                                               uint8_t *__restrict__ init_order_out)
{
    const int bh = blockIdx.x;
    const int lane = threadIdx.x;
    const size_t sbase = static_cast<size_t>(bh) * (T + 1);
    const int nseg = nseg_arr[bh];
    uint8_t *meta = meta_base + static_cast<size_t>(bh) * meta_stride;
    MetaHead *head = reinterpret_cast<MetaHead *>(meta);
    int64_t *info = reinterpret_cast<int64_t *>(meta + kOffInfo);
    int32_t *count = reinterpret_cast<int32_t *>(meta + kOffCount);
    int64_t *start = reinterpret_cast<int64_t *>(meta + kOffStart);
    // the stream as the cache leaves it (states with absolute token starts);
    // the live count and slots are kept for the chunk kernels, since the
    // metadata is rewritten at the end
    const int m_init = head->m;
    const int64_t t_seen = head->t_seen;
    int64_t I = lane < m_init ? info[lane] : 0;
    int32_t n = lane < m_init ? count[lane] : 0;
    int64_t st = lane < m_init ? start[lane] : 0;
    int32_t oi = -1;
    int m = m_init, cur_chunk = -1, nev = 0, nmerge = 0;
    if (lane == 0) init_m_out[bh] = m_init;
    init_order_out[static_cast<size_t>(bh) * kMaxC + lane] = meta[kOffOrder + lane];
    // the tokens before the call's first boundary join the most recent state
    if (m_init > 0 && lane == m_init - 1) {
        I += seg_P[sbase];
        n += seg_t[sbase];
    }

    for (int b0 = 0; b0 < nseg; b0 += 64) {
        const int j = b0 + lane;
        int32_t tj = 0, tn = 0;
        int64_t Pj = 0, Pn = 0, q0 = 0;
        if (j < nseg) {
            tj = seg_t[sbase + j];
            tn = seg_t[sbase + j + 1];
            Pj = seg_P[sbase + j];
            Pn = seg_P[sbase + j + 1];
            q0 = seg_q0[static_cast<size_t>(bh) * T + j];
        }
        const int cnt = min(64, nseg - b0);
        for (int jj = 0; jj < cnt; ++jj) {
            if (m == C && merge_rule != DLA_MERGE_DENSITY) {
                // A full cache under the summed key: the boundary of segment j
                // merges into the newest pair (the most recent state and its
                // own new state) when that pair's key is below the key of the
                // pair before it (q_j < I_{m-2}) and below every older pair's
                // key (their minimum M, which such merges leave alone), the most
                // recent state grown by every segment since jj.  The run of such
                // segments is taken at once: each merges its new state away at
                // once, so the state list keeps its shape and only the most
                // recent state's information and count grow.
                const int64_t Iprev = m >= 2 ? readlane_any(I, m - 2) : INT64_MAX;
                const int64_t Ilast = readlane_any(I, m - 1);
                const int64_t I_nx = lane_down1(I);
                const int64_t M = wave_min_i64(lane + 2 < m ? I + I_nx : INT64_MAX);
                const int64_t Pfirst = readlane_any(Pj, jj);
                const bool in = lane >= jj && lane < cnt;
                const bool joins = q0 < Iprev && Ilast + (Pj - Pfirst) + q0 < M;
                const uint64_t stop = __ballot(in && !joins);
                const int je = stop ? __builtin_ctzll(stop) : cnt;
                if (je > jj) {
                    // lane j of the run: its merge for the schedule export, and
                    // the event offset of every chunk from the one after the
                    // previous segment's on (a run emits no event: see below)
                    const int tprev = static_cast<int>(dpp32_rows<0x138, 0xF>(static_cast<uint32_t>(tj)));
                    if (in && lane < je) {
                        const int cj = tj / kChunk;
                        const int k = lane - jj;
                        if (ev_t_out) {
                            ev_t_out[static_cast<size_t>(bh) * T + nmerge + k] = tj;
                            ev_i_out[static_cast<size_t>(bh) * T + nmerge + k] = m - 1;
                        }
                        for (int kk = (lane == jj ? cur_chunk : tprev / kChunk) + 1; kk <= cj; ++kk)
                            chunk_ev[static_cast<size_t>(bh) * (NCH + 1) + kk] = nev;
                    }
                    const int last_chunk = readlane_any(tj, je - 1) / kChunk;
                    if (last_chunk != cur_chunk) {
                        oi = lane < m ? lane : -1;
                        cur_chunk = last_chunk;
                    }
                    const int64_t addI = readlane_any(Pn, je - 1) - Pfirst;
                    const int addn = readlane_any(tn, je - 1) - readlane_any(tj, jj);
                    if (lane == m - 1) { I += addI; n += addn; }
                    nmerge += je - jj;
                    jj = je;
                    if (jj >= cnt) break;
                }
                // (segment jj, whose merge lands elsewhere, takes the step below)
            }
            // segment jj of this batch, broadcast from its lane (jj is uniform)
            const int t = readlane_any(tj, jj);
            const int tnext = readlane_any(tn, jj);
            const int64_t qj = readlane_any(q0, jj);
            const int64_t remI = readlane_any(Pn, jj) - readlane_any(Pj, jj) - qj;
            const int remn = tnext - t - 1;
            const int c = t / kChunk;
            if (c != cur_chunk) {
                for (int kk = cur_chunk + 1 + lane; kk <= c; kk += 64)
                    chunk_ev[static_cast<size_t>(bh) * (NCH + 1) + kk] = nev;
                oi = lane < m ? lane : -1;
                cur_chunk = c;
            }
            int dead = -1, istar = -1;
            if (m < C) {
                if (lane == m) { I = qj; n = 1; st = t_seen + t; oi = -1; }
                ++m;
            } else {
                const int64_t I_nx = lane_down1(I);
                const int32_t n_nx = lane_down1(n);
                const int64_t st_nx = lane_down1(st);
                const int32_t oi_nx = lane_down1(oi);
                const bool inside = lane + 1 < m;
                const int64_t pI = inside ? I_nx : qj;
                const int32_t pn = inside ? n_nx : 1;
                const int64_t pst = inside ? st_nx : t_seen + t;
                const int32_t poi = inside ? oi_nx : -1;
                if (merge_rule == DLA_MERGE_DENSITY) {
                    // lowest information density (I_i + I_{i+1}) / (n_i + n_{i+1})
                    istar = wave_argmin_frac(I + pI, static_cast<int64_t>(n) + pn, lane < m);
                } else {
                    const int64_t key = lane < m ? I + pI : INT64_MAX;
                    const int64_t kmin = wave_min_i64(key);
                    const uint64_t hit = __ballot(key == kmin);
                    istar = __ffsll(static_cast<unsigned long long>(hit)) - 1;
                }
                const int32_t d_oi = readlane_any(poi, istar);
                const int64_t d_st = readlane_any(pst, istar);
                dead = d_oi >= 0 ? d_oi : 64 + static_cast<int>(d_st - t_seen - cur_chunk * kChunk);
                if (lane == istar) { I += pI; n += pn; }
                else if (lane > istar && lane < m) { I = pI; n = pn; st = pst; oi = poi; }
            }
            // (a new state merged at once into the state before it -- the
            // newest pair -- is the token joining the most recent state: the
            // chunk kernels get no event for it)
            const bool joined = istar >= 0 && istar == m - 1;
            if (lane == 0) {
                if (!joined) events[static_cast<size_t>(bh) * T + nev] = make_int2(t, dead);
                if (ev_t_out && istar >= 0) {
                    ev_t_out[static_cast<size_t>(bh) * T + nmerge] = t;
                    ev_i_out[static_cast<size_t>(bh) * T + nmerge] = istar;
                }
            }
            if (!joined) ++nev;
            if (istar >= 0) ++nmerge;
            if (lane == m - 1) { I += remI; n += remn; }
        }
    }
    for (int kk = cur_chunk + 1 + lane; kk <= NCH; kk += 64)
        chunk_ev[static_cast<size_t>(bh) * (NCH + 1) + kk] = nev;
    if (n_ev_out && lane == 0) n_ev_out[bh] = nmerge;

    info[lane] = lane < m ? I : 0;
    count[lane] = lane < m ? n : 0;
    start[lane] = lane < m ? st : 0;
    if (lane == 0) {
        head->m = m;
        head->has_prev = 1;
        head->s_prev = s_all[static_cast<size_t>(bh) * T + T - 1];
        head->pad0 = 0;
        head->t_seen = t_seen + T;
        head->pad1 = 0;
    }
}

// Copies the last key of every stream into its cache metadata (float).
template <typename TIO>
__global__ void k_store_kprev(const TIO *__restrict__ K, int T, int dk, uint8_t *__restrict__ meta_base,
                              size_t meta_stride)
{
    const int bh = blockIdx.x;
    float *kp = reinterpret_cast<float *>(meta_base + static_cast<size_t>(bh) * meta_stride + kOffKprev);
    const TIO *src = K + (static_cast<size_t>(bh) * T + T - 1) * dk;
    for (int i = threadIdx.x; i < dk; i += blockDim.x) kp[i] = to_f(src[i]);
}

// ------------------------------------------------------------ Log-Linear fixed schedule
//
// The Log-Linear form quoted in "Dynamic Linear Attention | Chlience Paper
// Archive", section 2: the prefix seen by query t is split into Fenwick-tree
// buckets and o_t = sum_l lam_t^(l) S_t^(l) q_t.  Reading: the token itself is
// level 0 and the rest of the prefix is the binary decomposition of t, oldest
// (largest) bucket first; key s < t is at level 1 + (highest bit in which s
// and t differ).
//
// The chunk kernels see this schedule as chunk-level events in the greedy
// scan's encoding.  Within a chunk the reads take their weights from the
// pre-pass (a formula of the positions), so the events only have to say what
// the states are at each chunk end: whole chunks, each piece inside one
// bucket of every later token.  A chunk with an even index opens a state at
// its first token and merges the older pieces that have become one bucket
// (several events on one token: one boundary, several merges); a chunk with
// an odd index joins the state of the chunk before it (no event).  The last
// chunk leaves the buckets of the whole prefix: a full last chunk with an odd
// index opens a state and merges it and the carried pieces away; a partial one
// opens a state at the start of each of its buckets.

// Pieces live at the start of chunk c (before its events).
__device__ __forceinline__ int fen_m0(int c) { return c == 0 ? 0 : __popc((c & 1) ? c : c - 1); }

// Events of chunk c, written at ev when ev is not NULL; returns their number.
__device__ int fen_chunk_events(int c, int T, int NCH, int2 *ev)
{
    const int c0 = c * kChunk, n = min(kChunk, T - c0), m0 = fen_m0(c);
    const bool last = c == NCH - 1;
    int cnt = 0;
    auto put = [&](int p, int d) {
        if (ev) ev[cnt] = make_int2(p, d);
        ++cnt;
    };
    if (last && n == kChunk && (c & 1)) {
        // the chunk and the z pieces it completes become one bucket
        const int z = __ffs(c + 1) - 1;
        for (int d = m0 - z + 1; d < m0; ++d) put(c0, d);
        put(c0, 64);
        return cnt;
    }
    if ((c & 1) && !(last && n < kChunk)) return 0;
    if (c >= 2 && !(c & 1)) {
        // the z most recent pieces (a chunk pair and its carries) are one bucket now
        const int z = __ffs(c) - 1;
        for (int d = m0 - z + 1; d < m0; ++d) put(c0, d);
    }
    if (cnt == 0) put(c0, -1);
    if (last && n < kChunk) {
        int p = 0;
        for (int b = 5; b >= 0; --b)
            if ((n >> b) & 1) {
                if (p > 0) put(c0 + p, -1);
                p += 1 << b;
            }
    }
    return cnt;
}

// A call continuing a stream at position t0 > 0 keeps the pieces exactly the
// buckets of [0, t) at every chunk end (its chunks are not aligned to the
// bucket sizes).  Call chunk c goes from the buckets of ts = t0 + 64 c to
// those of te: the two share their buckets above bit h, the highest bit in
// which ts and te differ; te's bucket of bit h starts where ts's buckets below
// h start, so those merge into the oldest of them and the chunk's first tokens
// join it (or, if ts has no bucket below h, the chunk opens it); te's buckets
// below h lie inside the chunk and each opens a state.  Merges ride on the
// first boundary; with no boundary they ride on one at the chunk start whose
// own state is merged away last.
__device__ int fen_cont_events(int64_t t0, int c, int T, int2 *ev)
{
    const int c0 = c * kChunk;
    const int64_t ts = t0 + c0, te = ts + min(kChunk, T - c0);
    const int m0 = __popcll(ts);
    const int h = 63 - __clzll(static_cast<unsigned long long>(ts ^ te));
    const int k = __popcll(ts >> (h + 1));
    const bool below = (ts & ((1ll << h) - 1)) != 0;
    int cnt = 0;
    auto put = [&](int p, int d) {
        if (ev) ev[cnt] = make_int2(p, d);
        ++cnt;
    };
    // boundaries: te's bucket of bit h when ts has nothing below h, then te's
    // buckets below h (positions within the chunk, increasing)
    int first = -1;
    if (!below) first = 0;
    else
        for (int b = h - 1; b >= 0; --b)
            if ((te >> b) & 1) {
                first = static_cast<int>((te & ~((2ll << b) - 1)) - ts);
                break;
            }
    if (first >= 0) {
        if (below && k + 1 < m0)
            for (int d = k + 1; d < m0; ++d) put(c0 + first, d);
        else
            put(c0 + first, -1);
        for (int b = h - 1; b >= 0; --b)
            if ((te >> b) & 1) {
                const int p = static_cast<int>((te & ~((2ll << b) - 1)) - ts);
                if (p > first) put(c0 + p, -1);
            }
    } else if (k + 1 < m0) {
        for (int d = k + 1; d < m0; ++d) put(c0, d);
        put(c0, 64);
    }
    return cnt;
}

// One block per stream: the events and per-chunk event offsets of the whole
// stream (a block-wide scan over the chunks), and the metadata of the final
// cache, the buckets of [0, t0 + T).  The stream continues from t0 = t_seen
// with the pieces the cache holds (the buckets of [0, t0), as fixed-schedule
// calls leave them).  A stream that would need a level weight past column
// C - 1 is refused: init_m = -1 marks it for the chunk kernels, which then
// leave its cache as it was and its outputs NaN.
__global__ __launch_bounds__(256) void k_fenwick_schedule(int T, int NCH, int C, int dk, size_t ev_stride,
                                                          int2 *__restrict__ events, int32_t *__restrict__ chunk_ev,
                                                          uint8_t *__restrict__ meta_base, size_t meta_stride,
                                                          int32_t *__restrict__ init_m_out,
                                                          uint8_t *__restrict__ init_order_out,
                                                          int64_t *__restrict__ t0_out)
{
    const int bh = blockIdx.x, tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    __shared__ int wsum[4];
    uint8_t *meta = meta_base + static_cast<size_t>(bh) * meta_stride;
    MetaHead *head = reinterpret_cast<MetaHead *>(meta);
    const int64_t t0 = head->t_seen;
    const int m_init = head->m;
    const int64_t tend = t0 + T;
    // levels 0 .. bit_length(tend - 1) must have a column
    const bool refused = C < 64 && tend - 1 >= (1ll << (C - 1));
    __syncthreads();          // every thread has read the head before it changes
    if (tid == 0) t0_out[bh] = t0;
    if (refused) {
        for (int c = tid; c <= NCH; c += 256) chunk_ev[static_cast<size_t>(bh) * (NCH + 1) + c] = 0;
        if (tid == 0) init_m_out[bh] = -1;
        return;
    }
    int carry = 0;
    for (int base = 0; base < NCH; base += 256) {
        const int c = base + tid;
        const int cnt = c >= NCH ? 0 : t0 > 0 ? fen_cont_events(t0, c, T, nullptr) : fen_chunk_events(c, T, NCH, nullptr);
        int x = cnt;
#pragma unroll
        for (int off = 1; off < 64; off <<= 1) {
            const int y = __shfl_up(x, off);
            if (lane >= off) x += y;
        }
        if (lane == 63) wsum[wave] = x;
        __syncthreads();
        int before = carry;
        for (int w = 0; w < wave; ++w) before += wsum[w];
        const int total = carry + wsum[0] + wsum[1] + wsum[2] + wsum[3];
        if (c < NCH) {
            const int e0 = before + x - cnt;
            chunk_ev[static_cast<size_t>(bh) * (NCH + 1) + c] = e0;
            int2 *ev = events + static_cast<size_t>(bh) * ev_stride + e0;
            if (t0 > 0) fen_cont_events(t0, c, T, ev);
            else fen_chunk_events(c, T, NCH, ev);
        }
        __syncthreads();
        carry = total;
    }
    if (tid == 0) chunk_ev[static_cast<size_t>(bh) * (NCH + 1) + NCH] = carry;

    // the pieces the call starts from (their slots are kept for the sweep,
    // which rewrites the order)
    if (tid < kMaxC) init_order_out[static_cast<size_t>(bh) * kMaxC + tid] = meta[kOffOrder + tid];
    __syncthreads();
    if (tid < kMaxC) {
        // bucket tid of [0, tend): the tid-th set bit of tend from the top
        int64_t st = 0, cnt = 0;
        int seen = 0;
        for (int b = 62; b >= 0; --b)
            if ((tend >> b) & 1) {
                if (seen == tid) cnt = 1ll << b;
                if (seen < tid) st += 1ll << b;
                ++seen;
            }
        if (tid >= seen) st = 0;
        reinterpret_cast<int64_t *>(meta + kOffInfo)[tid] = 0;
        reinterpret_cast<int32_t *>(meta + kOffCount)[tid] = static_cast<int32_t>(cnt);
        reinterpret_cast<int64_t *>(meta + kOffStart)[tid] = st;
    }
    for (int i = tid; i < dk; i += blockDim.x) reinterpret_cast<float *>(meta + kOffKprev)[i] = 0.0f;
    if (tid == 0) {
        head->m = __popcll(tend);
        head->has_prev = 0;
        head->s_prev = 0.0f;
        head->pad0 = 0;
        head->t_seen = tend;
        head->pad1 = 0;
        init_m_out[bh] = m_init;
    }
}

// ------------------------------------------------------------ prefill

template <typename TIO, int DK, int DVT>
struct PrefillSmem {
    static constexpr int PAD = 16 / sizeof(TIO);
    TIO q[kChunk][DK + PAD];
    TIO k[kChunk][DK + PAD];
    TIO kt[DK][kChunk + PAD];
    TIO vt[DVT][kChunk + PAD];
    TIO pw[kChunk][kChunk + PAD];
    float lam[kChunk][kMaxC];
    // the read weights of the states live at the chunk start, used only by
    // the inter-chunk read, and the four waves' partial reads written after
    // it (a barrier between): one region
    union {
        float wold[kMaxC][kChunk];
        float ored[4][kChunk][DVT];
    };
    uint64_t om[kChunk];
    uint64_t nm[kChunk];
    int32_t order[kMaxC];
    int32_t new_order[kMaxC];
    int32_t merge_dst[kMaxC];
    int32_t merge_src[kMaxC];
    int32_t grp_lo[kChunk + 1];
    int32_t grp_hi[kChunk + 1];
    int32_t grp_slot[kChunk + 1];
    int32_t grp_add[kChunk + 1];
    int32_t changed[kMaxC + kChunk + 1];
    int32_t shexp[kMaxC];         // power-of-two exponent of each fp16 state copy
    float red[4];
    int32_t n_merge, n_grp, n_changed, m_new, qexp;
};

// One block (4 waves) per (stream, d_v tile of DVT columns); sweeps the
// stream's chunks of 64 tokens in order.  Per chunk:
//   1. token masks from the chunk's events: bit i of om_t = state i of the
//      chunk start still live at t, bit p of nm_t = state opened at chunk
//      position p still live at t;
//   2. inter-chunk read: O[t] = sum_i lam_t[slot_t(i)] S_i q_t over the states
//      live at the chunk start (states merged during the chunk share the
//      weight of the state they joined); each wave takes every 4th state;
//   3. intra-chunk product: O += ((Q K^T) o W) V with W[t][s] =
//      lam_t[#{live chunk starts > s}] for s <= t;
//   4. o store; then chunk-end update: old merges S_a += S_b, every group of
//      chunk tokens adds (or sets) V_g^T K_g into its final state, and the
//      operand copies of the changed states are refreshed.
// States are fp32 in the cache.  With bf16 inputs the read streams an fp16
// copy of each state, normalised by a power of two kept in LDS, against the
// query chunk scaled by a power of two; both exponents are folded into the
// read weights.  The intra-chunk product and the state updates multiply the
// exact bf16 inputs (fp32 accumulation).  With fp32 inputs everything is fp32.
// The fp16 operand copy of the state in physical slot `slot` (this block's
// d_v slice), normalised by a power of two kept in S.shexp: a block-wide
// maximum, then the scaled copy.  Every thread of the block takes part.
template <int DK, int DVT, typename Smem, typename RT>
__device__ void shadow_state(Smem &S, int slot, const float *st_base, RT *shadow_base, size_t slot_stride,
                             int tid, int lane, int wave)
{
    const float4 *src = reinterpret_cast<const float4 *>(st_base + slot * slot_stride);
    float mx = 0.0f;
    for (int idx = tid; idx < DVT * DK / 4; idx += 256) {
        const float4 a = src[idx];
        mx = fmaxf(mx, fmaxf(fmaxf(fabsf(a.x), fabsf(a.y)), fmaxf(fabsf(a.z), fabsf(a.w))));
    }
    mx = wave_max(mx);
    __syncthreads();
    if (lane == 0) S.red[wave] = mx;
    __syncthreads();
    const int e = f16_exponent(fmaxf(fmaxf(S.red[0], S.red[1]), fmaxf(S.red[2], S.red[3])));
    RT *dst = shadow_base + slot * slot_stride;
    for (int idx = tid; idx < DVT * DK / 8; idx += 256) {
        const float4 a = src[2 * idx];
        const float4 b = src[2 * idx + 1];
        f16x8 o;
        o[0] = static_cast<_Float16>(ldexpf(a.x, -e)); o[1] = static_cast<_Float16>(ldexpf(a.y, -e));
        o[2] = static_cast<_Float16>(ldexpf(a.z, -e)); o[3] = static_cast<_Float16>(ldexpf(a.w, -e));
        o[4] = static_cast<_Float16>(ldexpf(b.x, -e)); o[5] = static_cast<_Float16>(ldexpf(b.y, -e));
        o[6] = static_cast<_Float16>(ldexpf(b.z, -e)); o[7] = static_cast<_Float16>(ldexpf(b.w, -e));
        reinterpret_cast<f16x8 *>(dst)[idx] = o;
    }
    if (tid == 0) S.shexp[slot] = e;
}

template <typename TIO, int DK, int DVT>
__global__ __launch_bounds__(256, 1) void k_prefill(
    const TIO *__restrict__ Q, const TIO *__restrict__ K, const TIO *__restrict__ V,
    const TIO *__restrict__ LAM, TIO *__restrict__ O, int T, int C, int DV, int nblk_dv,
    float *__restrict__ states, typename ReadT<TIO>::type *__restrict__ shadow,
    const int2 *__restrict__ events, const int32_t *__restrict__ chunk_ev,
    uint8_t *__restrict__ meta_base, size_t meta_stride, int32_t *__restrict__ m_t_out,
    const int32_t *__restrict__ init_m, const uint8_t *__restrict__ init_order, int fen, size_t ev_stride,
    const int64_t *__restrict__ init_t)
{
    constexpr int KS = DK / 32;     // reduction steps over d_k
    constexpr int NTV = DVT / 16;   // 16-wide tiles over the d_v slice
    constexpr int MT = kChunk / 16; // 16-row tiles over the chunk
    constexpr int EPV = 16 / sizeof(TIO);
    constexpr bool kHalfRead = sizeof(TIO) == 2;
    typedef typename ReadT<TIO>::type RT;
    typedef PrefillSmem<TIO, DK, DVT> Smem;
    extern __shared__ __align__(16) unsigned char smem_raw[];
    Smem &S = *reinterpret_cast<Smem *>(smem_raw);

    // blocks of one stream are given consecutive ids on one XCD when possible
    const int nblk = gridDim.x;
    int lin = blockIdx.x;
    if ((nblk & 7) == 0) lin = (blockIdx.x & 7) * (nblk >> 3) + (blockIdx.x >> 3);
    const int bh = lin / nblk_dv;
    const int dv0 = (lin % nblk_dv) * DVT;

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int lr = lane & 15, lg = lane >> 4;
    const int NCH = (T + kChunk - 1) / kChunk;
    const size_t tok0 = static_cast<size_t>(bh) * T;
    // a state's d_v slice for this block starts at state(p) + dv0*DK
    float *st_base = states + static_cast<size_t>(bh) * C * DV * DK + static_cast<size_t>(dv0) * DK;
    const RT *rd_base;
    if constexpr (kHalfRead)
        rd_base = shadow + static_cast<size_t>(bh) * C * DV * DK + static_cast<size_t>(dv0) * DK;
    else
        rd_base = reinterpret_cast<const RT *>(st_base);
    const size_t slot_stride = static_cast<size_t>(DV) * DK;

    int m0 = 0;
    if (tid < kMaxC) { S.order[tid] = tid; S.shexp[tid] = 0; }
    // the states the cache holds when the call starts (their fp32 values are
    // in the cache already; with bf16 io their fp16 operand copies are made here)
    const int m_init = init_m[bh];
    // fixed schedule (fen): a refused stream is left as it was (its outputs are
    // set apart later); the position the call starts at
    if (m_init < 0) return;
    const int64_t t0 = fen ? init_t[bh] : 0;
    const int2 *ev_s = events + static_cast<size_t>(bh) * ev_stride;
    if (tid < m_init) S.order[tid] = init_order[static_cast<size_t>(bh) * kMaxC + tid];
    m0 = m_init;
    if constexpr (kHalfRead) {
        __syncthreads();
        for (int i = 0; i < m_init; ++i)
            shadow_state<DK, DVT>(S, S.order[i], st_base, shadow + static_cast<size_t>(bh) * C * DV * DK +
                                  static_cast<size_t>(dv0) * DK, slot_stride, tid, lane, wave);
    }

    for (int ch = 0; ch < NCH; ++ch) {
        const int c0 = ch * kChunk;
        const int nvalid = min(kChunk, T - c0);
        __syncthreads();
        // ---- 1. load the chunk and build token masks
        float qmax = 0.0f;
        for (int idx = tid; idx < kChunk * DK / EPV; idx += 256) {
            const int r = idx / (DK / EPV), cv = (idx % (DK / EPV)) * EPV;
            uint4 qv = make_uint4(0, 0, 0, 0), kv = qv;
            if (r < nvalid) {
                const size_t off = (tok0 + c0 + r) * DK + cv;
                qv = *reinterpret_cast<const uint4 *>(Q + off);
                kv = *reinterpret_cast<const uint4 *>(K + off);
            }
            *reinterpret_cast<uint4 *>(&S.q[r][cv]) = qv;
            *reinterpret_cast<uint4 *>(&S.k[r][cv]) = kv;
            const TIO *qe = reinterpret_cast<const TIO *>(&qv);
#pragma unroll
            for (int e = 0; e < EPV; ++e) qmax = fmaxf(qmax, fabsf(to_f(qe[e])));
            const TIO *ke = reinterpret_cast<const TIO *>(&kv);
#pragma unroll
            for (int e = 0; e < EPV; ++e) S.kt[cv + e][r] = ke[e];
        }
        for (int idx = tid; idx < kChunk * DVT / EPV; idx += 256) {
            const int r = idx / (DVT / EPV), cv = (idx % (DVT / EPV)) * EPV;
            uint4 vv = make_uint4(0, 0, 0, 0);
            if (r < nvalid) vv = *reinterpret_cast<const uint4 *>(V + (tok0 + c0 + r) * DV + dv0 + cv);
            const TIO *ve = reinterpret_cast<const TIO *>(&vv);
#pragma unroll
            for (int e = 0; e < EPV; ++e) S.vt[cv + e][r] = ve[e];
        }
        for (int idx = tid; idx < kChunk * C; idx += 256) {
            const int r = idx / C, j = idx % C;
            S.lam[r][j] = r < nvalid ? to_f(LAM[(tok0 + c0 + r) * C + j]) : 0.0f;
        }
        if (tid < kChunk) {
            const int e0 = chunk_ev[static_cast<size_t>(bh) * (NCH + 1) + ch];
            const int e1 = chunk_ev[static_cast<size_t>(bh) * (NCH + 1) + ch + 1];
            uint64_t om = low_bits(m0), nm = 0;
            for (int e = e0; e < e1; ++e) {
                const int2 ev = ev_s[e];
                const int pos = ev.x - c0;
                if (tid >= pos) {
                    nm |= 1ull << pos;
                    if (ev.y >= 64) nm &= ~(1ull << (ev.y - 64));
                    else if (ev.y >= 0) om &= ~(1ull << ev.y);
                }
            }
            S.om[tid] = om;
            S.nm[tid] = nm;
            if (m_t_out && dv0 == 0 && tid < nvalid)
                m_t_out[tok0 + c0 + tid] = __popcll(om) + __popcll(nm);
        }
        qmax = wave_max(qmax);
        if (lane == 0) S.red[wave] = qmax;
        __syncthreads();
        const int qexp = kHalfRead ? f16_exponent(fmaxf(fmaxf(S.red[0], S.red[1]), fmaxf(S.red[2], S.red[3]))) : 0;
        const int64_t ts = t0 + c0;         // absolute position of the chunk's first token
        for (int idx = tid; idx < m0 * kChunk; idx += 256) {
            const int i = idx / kChunk, t = idx % kChunk;
            float w;
            if (fen) {
                // piece i of the fixed schedule (as in the register path's
                // pre-pass): the i-th bucket of the chunk count it was formed
                // for (from position 0) or of [0, ts) (continuing), read at
                // its level; rows past the stream's end weigh 0
                const int64_t cp = t0 > 0 ? ts : static_cast<int64_t>((ch & 1) ? ch : ch - 1) * kChunk;
                int seen = 0;
                int64_t first = 0;
                for (int b = 62; b >= 0; --b)
                    if ((cp >> b) & 1) {
                        if (seen == i) first = cp & ~((2ll << b) - 1);
                        ++seen;
                    }
                w = t < nvalid ? S.lam[t][64 - __clzll(static_cast<unsigned long long>((ts + t) ^ first))] : 0.0f;
            } else {
                w = S.lam[t][__popcll(shr64(S.om[t], i + 1)) + __popcll(S.nm[t])];
            }
            S.wold[i][t] = kHalfRead ? ldexpf(w, S.shexp[S.order[i]] + qexp) : w;
        }
        // Q fragments of the whole chunk (A operand of the inter-chunk read)
        Frag<RT> qf[MT][KS];
#pragma unroll
        for (int mt = 0; mt < MT; ++mt)
#pragma unroll
            for (int ks = 0; ks < KS; ++ks) read_frag_from(qf[mt][ks], &S.q[16 * mt + lr][32 * ks + 8 * lg], qexp);
        __syncthreads();

        // ---- 2. inter-chunk read over the states live at the chunk start
        floatx4 Oi[MT][NTV];
#pragma unroll
        for (int mt = 0; mt < MT; ++mt)
#pragma unroll
            for (int nt = 0; nt < NTV; ++nt) Oi[mt][nt] = floatx4{0.f, 0.f, 0.f, 0.f};
        {
            Frag<RT> bc[KS][NTV], bn[KS][NTV];
            int i = wave;
            if (i < m0) {
                const RT *sp = rd_base + S.order[i] * slot_stride;
#pragma unroll
                for (int ks = 0; ks < KS; ++ks)
#pragma unroll
                    for (int nt = 0; nt < NTV; ++nt)
                        load_frag(bc[ks][nt], sp + (16 * nt + lr) * DK + 32 * ks + 8 * lg);
            }
            for (; i < m0; i += 4) {
                if (i + 4 < m0) {
                    const RT *sp = rd_base + S.order[i + 4] * slot_stride;
#pragma unroll
                    for (int ks = 0; ks < KS; ++ks)
#pragma unroll
                        for (int nt = 0; nt < NTV; ++nt)
                            load_frag(bn[ks][nt], sp + (16 * nt + lr) * DK + 32 * ks + 8 * lg);
                }
                floatx4 P[MT][NTV];
#pragma unroll
                for (int mt = 0; mt < MT; ++mt)
#pragma unroll
                    for (int nt = 0; nt < NTV; ++nt) P[mt][nt] = floatx4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int ks = 0; ks < KS; ++ks)
#pragma unroll
                    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
                        for (int nt = 0; nt < NTV; ++nt) mma32(P[mt][nt], qf[mt][ks], bc[ks][nt]);
#pragma unroll
                for (int mt = 0; mt < MT; ++mt) {
                    const float4 w = *reinterpret_cast<const float4 *>(&S.wold[i][16 * mt + 4 * lg]);
#pragma unroll
                    for (int nt = 0; nt < NTV; ++nt) {
                        Oi[mt][nt][0] += w.x * P[mt][nt][0];
                        Oi[mt][nt][1] += w.y * P[mt][nt][1];
                        Oi[mt][nt][2] += w.z * P[mt][nt][2];
                        Oi[mt][nt][3] += w.w * P[mt][nt][3];
                    }
                }
#pragma unroll
                for (int ks = 0; ks < KS; ++ks)
#pragma unroll
                    for (int nt = 0; nt < NTV; ++nt) bc[ks][nt] = bn[ks][nt];
            }
        }
        __syncthreads();          // every wave is done with the read weights
#pragma unroll
        for (int mt = 0; mt < MT; ++mt)
#pragma unroll
            for (int nt = 0; nt < NTV; ++nt)
#pragma unroll
                for (int r = 0; r < 4; ++r) S.ored[wave][16 * mt + 4 * lg + r][16 * nt + lr] = Oi[mt][nt][r];

        // ---- 3. intra-chunk slot-weighted causal product (wave w: rows 16w..16w+15)
        {
            const int w = wave;
            Frag<TIO> qa[KS];
#pragma unroll
            for (int ks = 0; ks < KS; ++ks) load_frag(qa[ks], &S.q[16 * w + lr][32 * ks + 8 * lg]);
#pragma unroll
            for (int nt = 0; nt < MT; ++nt) {
                floatx4 A = floatx4{0.f, 0.f, 0.f, 0.f};
                if (nt <= w) {
#pragma unroll
                    for (int ks = 0; ks < KS; ++ks) {
                        Frag<TIO> kb;
                        load_frag(kb, &S.k[16 * nt + lr][32 * ks + 8 * lg]);
                        mma32(A, qa[ks], kb);
                    }
                }
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const int t = 16 * w + 4 * lg + r;
                    const int s = 16 * nt + lr;
                    float val = 0.0f;
                    if (s <= t) {
                        const int slot = !fen ? __popcll(shr64(S.nm[t], s + 1))
                                              : (s == t || t >= nvalid) ? 0
                                                                        : 64 - __clzll(static_cast<unsigned long long>(
                                                                                   (ts + t) ^ (ts + s)));
                        val = A[r] * S.lam[t][slot];
                    }
                    S.pw[t][s] = from_f<TIO>(val);
                }
            }
        }
        __syncthreads();
        {
            const int w = wave;
            floatx4 Oa[NTV];
#pragma unroll
            for (int nt = 0; nt < NTV; ++nt)
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const int t = 16 * w + 4 * lg + r, col = 16 * nt + lr;
                    Oa[nt][r] = S.ored[0][t][col] + S.ored[1][t][col] + S.ored[2][t][col] + S.ored[3][t][col];
                }
#pragma unroll
            for (int ks = 0; ks < kChunk / 32; ++ks) {
                if (32 * ks <= 16 * w + 15) {
                    Frag<TIO> a;
                    load_frag(a, &S.pw[16 * w + lr][32 * ks + 8 * lg]);
#pragma unroll
                    for (int nt = 0; nt < NTV; ++nt) {
                        Frag<TIO> b;
                        load_frag(b, &S.vt[16 * nt + lr][32 * ks + 8 * lg]);
                        mma32(Oa[nt], a, b);
                    }
                }
            }
            // ---- 4a. output
#pragma unroll
            for (int nt = 0; nt < NTV; ++nt)
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const int t = 16 * w + 4 * lg + r;
                    if (t < nvalid) O[(tok0 + c0 + t) * DV + dv0 + 16 * nt + lr] = from_f<TIO>(Oa[nt][r]);
                }
        }

        // ---- 4b. chunk-end state update
        if (tid == 0) {
            const int tl = nvalid - 1;
            const uint64_t oa = S.om[tl], na = S.nm[tl];
            uint64_t used = 0;
            int nold = 0, last_old = -1, nmg = 0, tgt = -1;
            for (int i = 0; i < m0; ++i) {
                if ((oa >> i) & 1ull) {
                    S.new_order[nold++] = S.order[i];
                    used |= 1ull << S.order[i];
                    last_old = i;
                    tgt = i;
                } else if (tgt >= 0) {   // old state 0 is never merged away
                    S.merge_dst[nmg] = S.order[tgt];
                    S.merge_src[nmg] = S.order[i];
                    ++nmg;
                }
            }
            int ng = 0, mnew = nold, nch = 0;
            for (int i = 0; i < nmg; ++i) S.changed[nch++] = S.merge_dst[i];
            const int first_new = na ? __ffsll(static_cast<unsigned long long>(na)) - 1 : nvalid;
            if (first_new > 0 && last_old >= 0) {
                S.grp_lo[ng] = 0; S.grp_hi[ng] = first_new;
                S.grp_slot[ng] = S.order[last_old]; S.grp_add[ng] = 1;
                S.changed[nch++] = S.order[last_old];
                ++ng;
            }
            uint64_t rest = na;
            while (rest) {
                const int p = __ffsll(static_cast<unsigned long long>(rest)) - 1;
                rest &= rest - 1;
                const int q = rest ? __ffsll(static_cast<unsigned long long>(rest)) - 1 : nvalid;
                const int slot = __ffsll(static_cast<unsigned long long>(~used)) - 1;
                if (slot < 0 || slot >= C) break;   // cannot happen: at most C states live
                used |= 1ull << slot;
                S.new_order[mnew++] = slot;
                S.grp_lo[ng] = p; S.grp_hi[ng] = q; S.grp_slot[ng] = slot; S.grp_add[ng] = 0;
                S.changed[nch++] = slot;
                ++ng;
            }
            S.n_merge = nmg;
            S.n_grp = ng;
            S.n_changed = nch;
            S.m_new = mnew;
        }
        __syncthreads();
        // merges of states that were live at the chunk start (fp32, in place)
        for (int g = 0; g < S.n_merge; ++g) {
            float4 *dst = reinterpret_cast<float4 *>(st_base + S.merge_dst[g] * slot_stride);
            const float4 *src = reinterpret_cast<const float4 *>(st_base + S.merge_src[g] * slot_stride);
            for (int idx = tid; idx < DVT * DK / 4; idx += 256) {
                float4 a = dst[idx];
                const float4 b = src[idx];
                a.x += b.x; a.y += b.y; a.z += b.z; a.w += b.w;
                dst[idx] = a;
            }
        }
        __syncthreads();
        // V_g^T K_g of every group of chunk tokens into its final state
        for (int g = 0; g < S.n_grp; ++g) {
            const int lo = S.grp_lo[g], hi = S.grp_hi[g];
            float *dst = st_base + S.grp_slot[g] * slot_stride;
            const bool add = S.grp_add[g] != 0;
            for (int tile = wave; tile < NTV * (DK / 16); tile += 4) {
                const int mt = tile % NTV, nt = tile / NTV;
                floatx4 acc = floatx4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int ks = 0; ks < kChunk / 32; ++ks) {
                    const int base = 32 * ks + 8 * lg;
                    if (32 * ks < hi && 32 * ks + 32 > lo) {
                        Frag<TIO> a, b;
                        load_frag(a, &S.vt[16 * mt + lr][base]);
                        mask_frag(a, base, lo, hi);
                        load_frag(b, &S.kt[16 * nt + lr][base]);
                        mma32(acc, a, b);
                    }
                }
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    float *p = dst + (16 * mt + 4 * lg + r) * DK + 16 * nt + lr;
                    *p = add ? (*p + acc[r]) : acc[r];
                }
            }
        }
        __syncthreads();
        if constexpr (kHalfRead) {
            // fp16 operand copies of the changed states, normalised per state
            for (int c = 0; c < S.n_changed; ++c)
                shadow_state<DK, DVT>(S, S.changed[c], st_base, shadow + static_cast<size_t>(bh) * C * DV * DK +
                                      static_cast<size_t>(dv0) * DK, slot_stride, tid, lane, wave);
        }
        __syncthreads();
        if (tid < kMaxC) S.order[tid] = tid < S.m_new ? S.new_order[tid] : 0;
        m0 = S.m_new;
    }
    __syncthreads();
    if (dv0 == 0 && tid < kMaxC) {
        uint8_t *order = meta_base + static_cast<size_t>(bh) * meta_stride + kOffOrder;
        order[tid] = static_cast<uint8_t>(tid < m0 ? S.order[tid] : 0xFF);
    }
}

// ------------------------------------------------------------ decode step

// One block per stream.  Wave 0 runs the scalar step (score, boundary,
// greedy merge on the metadata); then every thread streams the live states
// once: o = sum_i lam[slot(i)] S_i q + lam[0] v (k . q), adding v k^T into
// the most recent state, or writing the new state v k^T into a free slot,
// and applying a capacity merge S_a += S_b while the data passes through.
// The states are read and written with nontemporal hints: a step touches
// each of them once, so they should not displace other data in the caches.
//
// Thread tid owns columns 4 (tid % G) .. + 3 of the rows tid / G + R j of
// every state (G = DK / 4 threads per row, R rows per pass, P passes); the
// passes go in batches of at most 16 loads per thread, batch by batch over
// all the states, so that large states do not need more registers.
template <int DK, int DV>
struct DecodeShape {
    static constexpr int G = DK / 4;          // threads per state row (float4 each)
    static constexpr int R = 256 / G;         // rows per pass
    static constexpr int P = DV / R;          // passes per state
    static constexpr int PB = P < 16 ? P : 16; // passes per batch
    static_assert(DV % R == 0 && P % PB == 0, "whole passes and batches");
};

template <typename TIO, int DK, int DV, bool BF>
__global__ __launch_bounds__(256) void k_decode(const TIO *__restrict__ Qg, const TIO *__restrict__ Kg,
                                                const TIO *__restrict__ Vg, const TIO *__restrict__ Lg,
                                                TIO *__restrict__ Og, float tau, int C,
                                                float *__restrict__ states, float *__restrict__ active,
                                                uint8_t *__restrict__ meta_base,
                                                size_t meta_stride, DecodeSched sched, int merge_rule,
                                                int score_rule)
{
    typedef DecodeShape<DK, DV> Sh;
    constexpr int G = Sh::G, R = Sh::R, P = Sh::P, PB = Sh::PB;
    constexpr size_t SS = static_cast<size_t>(DK) * DV;   // elements per state
    __shared__ __align__(16) float qs[DK];
    __shared__ __align__(16) float ks[DK];
    __shared__ float kp[DK], vs[DV], lw[kMaxC];
    __shared__ float wlog[kMaxC];
    __shared__ int32_t order_s[kMaxC];
    __shared__ double red[4][4];
    __shared__ double fsq[4];
    __shared__ float orow[DV];
    __shared__ int32_t ctl[8];        // mode, add_slot, set_slot, merge_i, m, ...
    __shared__ float sc_kq;

    const int bh = blockIdx.x;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    uint8_t *meta = meta_base + static_cast<size_t>(bh) * meta_stride;
    MetaHead *head = reinterpret_cast<MetaHead *>(meta);
    uint8_t *order = meta + kOffOrder;
    int64_t *info = reinterpret_cast<int64_t *>(meta + kOffInfo);
    int32_t *count = reinterpret_cast<int32_t *>(meta + kOffCount);
    int64_t *start = reinterpret_cast<int64_t *>(meta + kOffStart);
    float *kprev = reinterpret_cast<float *>(meta + kOffKprev);

    if (tid < DK) {
        qs[tid] = to_f(Qg[static_cast<size_t>(bh) * DK + tid]);
        ks[tid] = to_f(Kg[static_cast<size_t>(bh) * DK + tid]);
        kp[tid] = kprev[tid];
    }
    if (tid < DV) vs[tid] = to_f(Vg[static_cast<size_t>(bh) * DV + tid]);
    if (tid < C) lw[tid] = to_f(Lg[static_cast<size_t>(bh) * C + tid]);
    __syncthreads();
    const bool state_score = score_rule == DLA_SCORE_STATE;
    {
        double d = 0.0, a = 0.0, b = 0.0, kq = 0.0;
        if (tid < DK) {
            const double x = ks[tid], y = kp[tid];
            d = x * y; a = x * x; b = y * y;
            kq = x * static_cast<double>(qs[tid]);
        }
        if (state_score) {
            // the state information score needs x = v^T S k and |S|_F^2 of the
            // current (most recent) state, read once before the step; a and b
            // then carry |k|^2 and |v|^2
            const int m0 = head->m;
            d = 0.0;
            a = tid < DK ? static_cast<double>(ks[tid]) * ks[tid] : 0.0;
            b = tid < DV ? static_cast<double>(vs[tid]) * vs[tid] : 0.0;
            double f = 0.0;
            if (m0 > 0) {
                const int col = (tid % G) * 4, row0 = tid / G;
                const float4 k4 = *reinterpret_cast<const float4 *>(&ks[col]);
                const float *src;
                if constexpr (BF) src = active + static_cast<size_t>(bh) * SS;
                else src = states + (static_cast<size_t>(bh) * C + order[m0 - 1]) * SS;
#pragma unroll 4
                for (int j = 0; j < P; ++j) {
                    const int row = row0 + R * j;
                    const float4 x = *reinterpret_cast<const float4 *>(src + static_cast<size_t>(row) * DK + col);
                    d += static_cast<double>(vs[row]) * (static_cast<double>(x.x) * k4.x + static_cast<double>(x.y) * k4.y +
                                                         static_cast<double>(x.z) * k4.z + static_cast<double>(x.w) * k4.w);
                    f += static_cast<double>(x.x) * x.x + static_cast<double>(x.y) * x.y +
                         static_cast<double>(x.z) * x.z + static_cast<double>(x.w) * x.w;
                }
            }
            d = wave_sum(d); a = wave_sum(a); b = wave_sum(b); kq = wave_sum(kq); f = wave_sum(f);
            if (lane == 0) { red[wave][0] = d; red[wave][1] = a; red[wave][2] = b; red[wave][3] = kq; fsq[wave] = f; }
        } else {
            d = wave_sum(d); a = wave_sum(a); b = wave_sum(b); kq = wave_sum(kq);
            if (lane == 0) { red[wave][0] = d; red[wave][1] = a; red[wave][2] = b; red[wave][3] = kq; }
        }
    }
    __syncthreads();
    if (wave == 0) {
        const double d = red[0][0] + red[1][0] + red[2][0] + red[3][0];
        const double a = red[0][1] + red[1][1] + red[2][1] + red[3][1];
        const double b = red[0][2] + red[1][2] + red[2][2] + red[3][2];
        const double kq = red[0][3] + red[1][3] + red[2][3] + red[3][3];
        const int m = head->m;
        const int has_prev = head->has_prev;
        const float s_prev = head->s_prev;
        const int64_t t_seen = head->t_seen;
        float s;
        int bnd;
        if (state_score) {
            // I = sqrt(2 D (1 - c)) / (sqrt(D) + 1e-6), c = x / (|v| |k| |S|_F)
            const double F = fsq[0] + fsq[1] + fsq[2] + fsq[3];
            const double nn = a * b, Dd = static_cast<double>(DK) * DV;
            if (m == 0 || nn == 0.0 || F <= 0.0) s = 2.0f;
            else s = static_cast<float>(sqrt(fmax(0.0, 2.0 * Dd * (1.0 - d / sqrt(nn * F)))) / (sqrt(Dd) + 1e-6));
            bnd = (m == 0) || (s >= tau);
        } else {
            s = has_prev ? cosine_distance(d, a, b) : 1.0f;
            bnd = (m == 0) || !((s < tau) && (s_prev < tau));
        }
        const int64_t qv = fixed_point(s);
        int64_t I = lane < m ? info[lane] : 0;
        int32_t n = lane < m ? count[lane] : 0;
        int64_t stt = lane < m ? start[lane] : 0;
        int32_t ord = lane < m ? static_cast<int32_t>(order[lane]) : 0;
        uint64_t usedmask = 0;
        for (int i = 0; i < m; ++i) usedmask |= 1ull << __shfl(ord, i);
        int mode, add_slot = -1, set_slot = -1, merge_i = -1, m_new = m, post_slot = 0;
        if (!bnd) {
            mode = 0;                                  // join the most recent state
            add_slot = __shfl(ord, m - 1);
            post_slot = m - 1 - lane;
            if (lane == m - 1) { I += qv; n += 1; }
        } else if (m < C) {
            mode = 1;                                  // open a state in a free slot
            set_slot = __ffsll(static_cast<unsigned long long>(~usedmask)) - 1;
            post_slot = m - lane;
            if (lane == m) { I = qv; n = 1; stt = t_seen; ord = set_slot; }
            m_new = m + 1;
        } else {
            const int64_t I_nx = lane_down1(I);
            const bool inside = lane + 1 < m;
            const int64_t pI = inside ? I_nx : qv;
            if (merge_rule == DLA_MERGE_DENSITY) {
                // lowest information density (I_i + I_{i+1}) / (n_i + n_{i+1})
                const int32_t n_down = lane_down1(n);
                const int64_t pn = inside ? n_down : 1;
                merge_i = wave_argmin_frac(I + pI, static_cast<int64_t>(n) + pn, lane < m);
            } else {
                const int64_t key = lane < m ? I + pI : INT64_MAX;
                const int64_t kmin = wave_min_i64(key);
                merge_i = __ffsll(static_cast<unsigned long long>(__ballot(key == kmin))) - 1;
            }
            post_slot = m - 1 - (lane <= merge_i ? lane : lane - 1);
            if (merge_i == m - 1) {
                mode = 3;                              // the new token joins the most recent state
                add_slot = __shfl(ord, m - 1);
                if (lane == m - 1) { I += qv; n += 1; }
            } else {
                mode = 2;                              // merge (i, i+1), new state into the freed slot
                const int32_t freed = __shfl(ord, merge_i + 1);
                set_slot = freed;
                const int32_t n_nx = lane_down1(n);
                const int64_t st_nx = lane_down1(stt);
                const int32_t ord_nx = lane_down1(ord);
                if (lane == merge_i) { I += I_nx; n += n_nx; }
                else if (lane > merge_i && lane < m - 1) { I = I_nx; n = n_nx; stt = st_nx; ord = ord_nx; }
                else if (lane == m - 1) { I = qv; n = 1; stt = t_seen; ord = freed; }
            }
        }
        if (lane < m) {
            wlog[lane] = lw[post_slot];
            order_s[lane] = static_cast<int32_t>(order[lane]);
        }
        if (lane == 0) {
            ctl[0] = mode; ctl[1] = add_slot; ctl[2] = set_slot; ctl[3] = merge_i; ctl[4] = m;
            sc_kq = static_cast<float>(kq) * lw[0];
        }
        // new metadata
        if (lane < kMaxC) {
            info[lane] = lane < m_new ? I : 0;
            count[lane] = lane < m_new ? n : 0;
            start[lane] = lane < m_new ? stt : 0;
            order[lane] = static_cast<uint8_t>(lane < m_new ? ord : 0xFF);
        }
        if (lane == 0) {
            head->m = m_new;
            head->has_prev = 1;
            head->s_prev = s;
            head->t_seen = t_seen + 1;
            if (sched.s) sched.s[bh] = s;
            if (sched.boundary) sched.boundary[bh] = static_cast<uint8_t>(bnd);
            if (sched.m_t) sched.m_t[bh] = m_new;
            if (sched.ev_i) sched.ev_i[bh] = merge_i;
        }
    }
    __syncthreads();
    if (tid < DK) kprev[tid] = ks[tid];
    const int mode = ctl[0], add_slot = ctl[1], set_slot = ctl[2], merge_i = ctl[3], m = ctl[4];
    const int col = (tid % G) * 4, row0 = tid / G;
    const float4 q4 = *reinterpret_cast<const float4 *>(&qs[col]);
    const float4 k4 = *reinterpret_cast<const float4 *>(&ks[col]);
    float acc[P];
#pragma unroll
    for (int j = 0; j < P; ++j) acc[j] = 0.0f;
    if constexpr (!BF) {
        float *sb = states + static_cast<size_t>(bh) * C * SS;
#pragma unroll 1
        for (int b = 0; b < P; b += PB) {
            for (int i = 0; i < m; ++i) {
                const int p = order_s[i];
                const float w = wlog[i];
                float4 *sp = reinterpret_cast<float4 *>(sb + static_cast<size_t>(p) * SS);
                float4 x[PB];
#pragma unroll
                for (int j = 0; j < PB; ++j) {
                    const floatx4 t = __builtin_nontemporal_load(reinterpret_cast<const floatx4 *>(sp) +
                                                                 ((row0 + R * (b + j)) * DK + col) / 4);
                    x[j] = make_float4(t[0], t[1], t[2], t[3]);
                }
#pragma unroll
                for (int j = 0; j < PB; ++j)
                    acc[b + j] += w * (x[j].x * q4.x + x[j].y * q4.y + x[j].z * q4.z + x[j].w * q4.w);
                if (p == add_slot) {
#pragma unroll
                    for (int j = 0; j < PB; ++j) {
                        const float vr = vs[row0 + R * (b + j)];
                        float4 y = x[j];
                        y.x += vr * k4.x; y.y += vr * k4.y; y.z += vr * k4.z; y.w += vr * k4.w;
                        __builtin_nontemporal_store(floatx4{y.x, y.y, y.z, y.w},
                                                    reinterpret_cast<floatx4 *>(sp) + ((row0 + R * (b + j)) * DK + col) / 4);
                    }
                }
                if (mode == 2 && i == merge_i + 1) {
                    float4 *dp = reinterpret_cast<float4 *>(sb + static_cast<size_t>(order_s[merge_i]) * SS);
#pragma unroll
                    for (int j = 0; j < PB; ++j) {
                        const int idx = ((row0 + R * (b + j)) * DK + col) / 4;
                        float4 a = dp[idx];
                        a.x += x[j].x; a.y += x[j].y; a.z += x[j].z; a.w += x[j].w;
                        __builtin_nontemporal_store(floatx4{a.x, a.y, a.z, a.w}, reinterpret_cast<floatx4 *>(dp) + idx);
                    }
                }
            }
            if (set_slot >= 0) {
                float4 *sp = reinterpret_cast<float4 *>(sb + static_cast<size_t>(set_slot) * SS);
#pragma unroll
                for (int j = 0; j < PB; ++j) {
                    const float vr = vs[row0 + R * (b + j)];
                    __builtin_nontemporal_store(floatx4{vr * k4.x, vr * k4.y, vr * k4.z, vr * k4.w},
                                                reinterpret_cast<floatx4 *>(sp) + ((row0 + R * (b + j)) * DK + col) / 4);
                }
            }
        }
    } else {
        // closed states bf16 in their slots, the active one (chronological
        // index m - 1) fp32 in the stream's active region; each state is read
        // once, and every change is applied while it passes
        typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
        const int act_i = m - 1;
        floatx4 *ab = reinterpret_cast<floatx4 *>(active + static_cast<size_t>(bh) * SS);
        u32x2 *sb = reinterpret_cast<u32x2 *>(states) + static_cast<size_t>(bh) * C * SS / 4;
#pragma unroll 1
        for (int b = 0; b < P; b += PB) {
            for (int i = 0; i < m; ++i) {
                const int p = order_s[i];
                const float w = wlog[i];
                float4 x[PB];
                if (i == act_i) {
#pragma unroll
                    for (int j = 0; j < PB; ++j) {
                        const floatx4 t = __builtin_nontemporal_load(ab + ((row0 + R * (b + j)) * DK + col) / 4);
                        x[j] = make_float4(t[0], t[1], t[2], t[3]);
                    }
                } else {
                    const u32x2 *sp = sb + static_cast<size_t>(p) * SS / 4;
#pragma unroll
                    for (int j = 0; j < PB; ++j) {
                        const u32x2 t = __builtin_nontemporal_load(sp + ((row0 + R * (b + j)) * DK + col) / 4);
                        x[j] = unpack_bf16x4(make_uint2(t[0], t[1]));
                    }
                }
#pragma unroll
                for (int j = 0; j < PB; ++j)
                    acc[b + j] += w * (x[j].x * q4.x + x[j].y * q4.y + x[j].z * q4.z + x[j].w * q4.w);
                // where a bf16 result goes: the active state closing into its own
                // slot, or the state merging away added into the slot of merge_i
                int dst_slot = -1;
                bool add_into = false;
                if (i == act_i) {
                    if (mode == 0 || mode == 3) {
                        // the token joins the active state
#pragma unroll
                        for (int j = 0; j < PB; ++j) {
                            const float vr = vs[row0 + R * (b + j)];
                            const float4 y = x[j];
                            __builtin_nontemporal_store(floatx4{y.x + vr * k4.x, y.y + vr * k4.y, y.z + vr * k4.z,
                                                                y.w + vr * k4.w},
                                                        ab + ((row0 + R * (b + j)) * DK + col) / 4);
                        }
                    } else if (mode == 2 && merge_i + 1 == act_i) {
                        dst_slot = order_s[merge_i];       // merged into the closed state before it
                        add_into = true;
                    } else {
                        dst_slot = p;                      // closes: a new state becomes the active one
                    }
                } else if (mode == 2 && i == merge_i + 1) {
                    dst_slot = order_s[merge_i];
                    add_into = true;
                }
                if (dst_slot >= 0) {
                    u32x2 *dp = sb + static_cast<size_t>(dst_slot) * SS / 4;
#pragma unroll
                    for (int j = 0; j < PB; ++j) {
                        const int idx = ((row0 + R * (b + j)) * DK + col) / 4;
                        float4 y = x[j];
                        if (add_into) {
                            const u32x2 t = dp[idx];
                            const float4 a4 = unpack_bf16x4(make_uint2(t[0], t[1]));
                            y.x += a4.x; y.y += a4.y; y.z += a4.z; y.w += a4.w;
                        }
                        const uint2 u = pack_bf16x4(y);
                        __builtin_nontemporal_store(u32x2{u.x, u.y}, dp + idx);
                    }
                }
            }
            if (mode == 1 || mode == 2) {
                // the new state v k^T is the active one now
#pragma unroll
                for (int j = 0; j < PB; ++j) {
                    const float vr = vs[row0 + R * (b + j)];
                    __builtin_nontemporal_store(floatx4{vr * k4.x, vr * k4.y, vr * k4.z, vr * k4.w},
                                                ab + ((row0 + R * (b + j)) * DK + col) / 4);
                }
            }
        }
    }
    (void)mode;
#pragma unroll
    for (int j = 0; j < P; ++j) {
        float x = acc[j];
#pragma unroll
        for (int off = G / 2; off > 0; off >>= 1) x += __shfl_xor(x, off);
        if (tid % G == 0) orow[row0 + R * j] = x;
    }
    __syncthreads();
    if (tid < DV) Og[static_cast<size_t>(bh) * DV + tid] = from_f<TIO>(orow[tid] + sc_kq * vs[tid]);
}

// ------------------------------------------------------------ decode, fixed schedule
//
// One token of every stream under the Log-Linear fixed schedule (the Fenwick
// buckets described at k_fenwick_schedule).  The cache holds the buckets of
// [0, t), t = t_seen, oldest first.  Token t is read at level 0 and bucket i
// at level 1 + (highest bit in which its start and t differ); then the token
// joins the buckets its carry completes: with z trailing ones in t, the last
// z buckets and the token become one bucket (z = 0: the token opens a state).
// Each state is read once; the ones that merge are summed in registers on
// the way and the sum is written once, into the slot of the oldest of them.
// A stream at t >= 2^(C-1) would need a level weight the cache does not
// have: its output row is NaN and its cache is left as it was.
template <typename TIO, int DK, int DV>
__global__ __launch_bounds__(256) void k_decode_fenwick(const TIO *__restrict__ Qg, const TIO *__restrict__ Kg,
                                                        const TIO *__restrict__ Vg, const TIO *__restrict__ Lg,
                                                        TIO *__restrict__ Og, int C, float *__restrict__ states,
                                                        uint8_t *__restrict__ meta_base, size_t meta_stride)
{
    typedef DecodeShape<DK, DV> Sh;
    constexpr int G = Sh::G, R = Sh::R, P = Sh::P, PB = Sh::PB;
    constexpr size_t SS = static_cast<size_t>(DK) * DV;
    __shared__ __align__(16) float qs[DK];
    __shared__ __align__(16) float ks[DK];
    __shared__ float vs[DV], lw[kMaxC];
    __shared__ float wlog[kMaxC];
    __shared__ int32_t order_s[kMaxC];
    __shared__ double red[4];
    __shared__ float orow[DV];
    __shared__ int32_t ctl[4];        // m, first merging index, destination slot, refused
    __shared__ float sc_kq;

    const int bh = blockIdx.x;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    uint8_t *meta = meta_base + static_cast<size_t>(bh) * meta_stride;
    MetaHead *head = reinterpret_cast<MetaHead *>(meta);
    uint8_t *order = meta + kOffOrder;
    int64_t *info = reinterpret_cast<int64_t *>(meta + kOffInfo);
    int32_t *count = reinterpret_cast<int32_t *>(meta + kOffCount);
    int64_t *start = reinterpret_cast<int64_t *>(meta + kOffStart);

    if (tid < DK) {
        qs[tid] = to_f(Qg[static_cast<size_t>(bh) * DK + tid]);
        ks[tid] = to_f(Kg[static_cast<size_t>(bh) * DK + tid]);
    }
    if (tid < DV) vs[tid] = to_f(Vg[static_cast<size_t>(bh) * DV + tid]);
    if (tid < C) lw[tid] = to_f(Lg[static_cast<size_t>(bh) * C + tid]);
    __syncthreads();
    {
        double kq = tid < DK ? static_cast<double>(ks[tid]) * static_cast<double>(qs[tid]) : 0.0;
        kq = wave_sum(kq);
        if (lane == 0) red[wave] = kq;
    }
    __syncthreads();
    if (wave == 0) {
        const double kq = red[0] + red[1] + red[2] + red[3];
        const int m = head->m;
        const int64_t t = head->t_seen;
        int32_t n = lane < m ? count[lane] : 0;
        int64_t stt = lane < m ? start[lane] : 0;
        int32_t ord = lane < m ? static_cast<int32_t>(order[lane]) : 0;
        if (lane < m) {
            const int lv = 64 - __clzll(static_cast<unsigned long long>(t ^ stt));
            wlog[lane] = lv < C ? lw[lv] : 0.0f;
            order_s[lane] = ord;
        }
        uint64_t usedmask = 0;
        for (int i = 0; i < m; ++i) usedmask |= 1ull << __shfl(ord, i);
        const int z = __ffsll(static_cast<unsigned long long>(~t)) - 1;       // trailing ones of t
        const int first = z == 0 ? m : max(m - z, 0);
        // (a cache that no fixed-schedule call left -- too many states for a
        // new one -- is refused the same way, so no slot past C is written)
        const bool refused = (C < 64 && t >= (1ll << (C - 1))) || m > C || (first == m && m >= C);
        int dst, m_new;
        if (first == m) {
            dst = __ffsll(static_cast<unsigned long long>(~usedmask)) - 1;  // lowest free slot
            m_new = m + 1;
            if (lane == m) { n = 1; stt = t; ord = dst; }
        } else {
            dst = __shfl(ord, first);
            m_new = first + 1;
            const int32_t tot = wave_sum<int32_t>(lane >= first && lane < m ? n : 0);
            if (lane == first) n = tot + 1;
        }
        if (lane == 0) {
            ctl[0] = m; ctl[1] = first; ctl[2] = dst; ctl[3] = refused;
            sc_kq = static_cast<float>(kq) * lw[0];
        }
        if (!refused) {
            if (lane < kMaxC) {
                info[lane] = 0;
                count[lane] = lane < m_new ? n : 0;
                start[lane] = lane < m_new ? stt : 0;
                order[lane] = static_cast<uint8_t>(lane < m_new ? ord : 0xFF);
            }
            if (lane == 0) {
                head->m = m_new;
                head->has_prev = 0;
                head->s_prev = 0.0f;
                head->t_seen = t + 1;
            }
        }
    }
    __syncthreads();
    const int m = ctl[0], first = ctl[1], dst = ctl[2];
    if (ctl[3]) {
        if (tid < DV) Og[static_cast<size_t>(bh) * DV + tid] = from_f<TIO>(__builtin_nanf(""));
        return;
    }
    const int col = (tid % G) * 4, row0 = tid / G;
    const float4 q4 = *reinterpret_cast<const float4 *>(&qs[col]);
    const float4 k4 = *reinterpret_cast<const float4 *>(&ks[col]);
    float acc[P];
#pragma unroll
    for (int j = 0; j < P; ++j) acc[j] = 0.0f;
    float *sb = states + static_cast<size_t>(bh) * C * SS;
    auto batch = [&](const int b) {
        float4 sum[PB];
#pragma unroll
        for (int j = 0; j < PB; ++j) {
            const float vr = vs[row0 + R * (b + j)];
            sum[j] = make_float4(vr * k4.x, vr * k4.y, vr * k4.z, vr * k4.w);
        }
        for (int i = 0; i < m; ++i) {
            const int p = order_s[i];
            const float w = wlog[i];
            const floatx4 *sp = reinterpret_cast<const floatx4 *>(sb + static_cast<size_t>(p) * SS);
            float4 x[PB];
#pragma unroll
            for (int j = 0; j < PB; ++j) {
                const floatx4 u = __builtin_nontemporal_load(sp + ((row0 + R * (b + j)) * DK + col) / 4);
                x[j] = make_float4(u[0], u[1], u[2], u[3]);
            }
#pragma unroll
            for (int j = 0; j < PB; ++j)
                acc[b + j] += w * (x[j].x * q4.x + x[j].y * q4.y + x[j].z * q4.z + x[j].w * q4.w);
            if (i >= first) {
#pragma unroll
                for (int j = 0; j < PB; ++j) {
                    sum[j].x += x[j].x; sum[j].y += x[j].y; sum[j].z += x[j].z; sum[j].w += x[j].w;
                }
            }
        }
        // the token's bucket (its own slot was read above by the same threads)
        floatx4 *dp = reinterpret_cast<floatx4 *>(sb + static_cast<size_t>(dst) * SS);
#pragma unroll
        for (int j = 0; j < PB; ++j)
            __builtin_nontemporal_store(floatx4{sum[j].x, sum[j].y, sum[j].z, sum[j].w},
                                        dp + ((row0 + R * (b + j)) * DK + col) / 4);
    };
    if constexpr (P == PB) {
        batch(0);
    } else {
#pragma unroll 1
        for (int b = 0; b < P; b += PB) batch(b);
    }
#pragma unroll
    for (int j = 0; j < P; ++j) {
        float x = acc[j];
#pragma unroll
        for (int off = G / 2; off > 0; off >>= 1) x += __shfl_xor(x, off);
        if (tid % G == 0) orow[row0 + R * j] = x;
    }
    __syncthreads();
    if (tid < DV) Og[static_cast<size_t>(bh) * DV + tid] = from_f<TIO>(orow[tid] + sc_kq * vs[tid]);
}

// ------------------------------------------------------------ launchers

hipError_t launch_cache_init(float *states, float *active, uint8_t *meta, const CacheGeom &g,
                             const PreloadArgs &pre, hipStream_t stream)
{
    hipLaunchKernelGGL(k_cache_init, dim3(g.B * g.H), dim3(256), 0, stream, states, active, meta, g, pre);
    return hipGetLastError();
}

template <typename TIO, int DK>
static hipError_t prefill_schedule(const PrefillArgs &a, hipStream_t stream)
{
    const int BH = a.g.B * a.g.H, T = a.T;
    const int NT = (T + kScoreTile - 1) / kScoreTile;
    const int NCH = (T + kChunk - 1) / kChunk;
    const TIO *K = static_cast<const TIO *>(a.k);
    if (a.score_rule == DLA_SCORE_STATE) {
        hipError_t e = launch_state_score(a, stream);
        if (e != hipSuccess) return e;
    } else {
        hipLaunchKernelGGL((k_score<TIO, DK>), dim3(NT, BH), dim3(256), 0, stream, K, T, a.tau, a.ws.s,
                           a.ws.qs, a.ws.flag, a.ws.tile_cnt, a.ws.tile_sum, NT, a.meta, a.g.meta_stride);
    }
    hipLaunchKernelGGL(k_compact, dim3(NT, BH), dim3(256), 0, stream, T, NT, a.ws.flag, a.ws.qs,
                       a.ws.tile_cnt, a.ws.tile_sum, a.ws.seg_t, a.ws.seg_P, a.ws.seg_q0, a.ws.nseg,
                       a.sched.seg_id);
    hipLaunchKernelGGL(k_greedy, dim3(BH), dim3(64), 0, stream, T, a.g.C, NCH, a.ws.seg_t, a.ws.seg_P,
                       a.ws.seg_q0, a.ws.nseg, a.ws.events, a.ws.chunk_ev, a.ws.s, a.meta, a.g.meta_stride,
                       a.sched.ev_t, a.sched.ev_i, a.sched.n_ev, a.merge_rule, a.ws.init_m, a.ws.init_order);
    hipLaunchKernelGGL((k_store_kprev<TIO>), dim3(BH), dim3(128), 0, stream, K, T, DK, a.meta,
                       a.g.meta_stride);
    return hipGetLastError();
}

template <typename TIO, int DK, int DVT>
static hipError_t prefill_main(const PrefillArgs &a, hipStream_t stream)
{
    const int BH = a.g.B * a.g.H;
    const int nblk_dv = a.g.dv / DVT;
    const size_t smem = sizeof(PrefillSmem<TIO, DK, DVT>);
    static bool attr_set = false;   // idempotent; a race only repeats the same call
    if (!attr_set) {
        hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void *>(&k_prefill<TIO, DK, DVT>),
                                           hipFuncAttributeMaxDynamicSharedMemorySize,
                                           static_cast<int>(smem));
        if (e != hipSuccess) return e;
        attr_set = true;
    }
    if (a.ev_before) {
        hipError_t e = hipEventRecord(a.ev_before, stream);
        if (e != hipSuccess) return e;
    }
    hipLaunchKernelGGL((k_prefill<TIO, DK, DVT>), dim3(BH * nblk_dv), dim3(256), smem, stream,
                       static_cast<const TIO *>(a.q), static_cast<const TIO *>(a.k),
                       static_cast<const TIO *>(a.v), static_cast<const TIO *>(a.lam),
                       static_cast<TIO *>(a.o), a.T, a.g.C, a.g.dv, nblk_dv, a.states,
                       static_cast<typename ReadT<TIO>::type *>(a.ws.shadow), a.ws.events, a.ws.chunk_ev, a.meta,
                       a.g.meta_stride, a.sched.m_t, a.ws.init_m, a.ws.init_order, a.merge_rule == DLA_FENWICK ? 1 : 0,
                       a.merge_rule == DLA_FENWICK ? a.ws.ev_stride : static_cast<size_t>(a.T), a.ws.init_t);
    hipError_t e = hipGetLastError();
    if (e == hipSuccess && a.ev_after) e = hipEventRecord(a.ev_after, stream);
    return e;
}

// A cache with bf16 closed states on the streamed prefill: the live states are
// widened into an fp32 working copy (closed ones from their bf16 slots, the
// most recent from the fp32 active region), the streamed kernels run on the
// copy, and the final live states are narrowed back: the closed ones rounded
// once to bf16 (nearest even) into their slots, the most recent into the
// active region.  Grid (element blocks, slot, stream); a block whose slot
// holds no live state does nothing.
template <bool NARROW>
__global__ __launch_bounds__(256) void k_state_copy(uint16_t *__restrict__ slots, float *__restrict__ active,
                                                    float *__restrict__ work, const uint8_t *__restrict__ meta_base,
                                                    size_t meta_stride, int C, int D2)
{
    const int p = blockIdx.y, bh = blockIdx.z;
    const uint8_t *meta = meta_base + static_cast<size_t>(bh) * meta_stride;
    const int m = reinterpret_cast<const MetaHead *>(meta)->m;
    int idx = -1;                    // chronological index of the state in slot p
    for (int i = 0; i < m; ++i)
        if (meta[kOffOrder + i] == p) idx = i;
    if (idx < 0) return;
    const bool last = idx == m - 1;
    float4 *w4 = reinterpret_cast<float4 *>(work + (static_cast<size_t>(bh) * C + p) * D2);
    uint2 *s4 = reinterpret_cast<uint2 *>(slots + (static_cast<size_t>(bh) * C + p) * D2);
    float4 *a4 = reinterpret_cast<float4 *>(active + static_cast<size_t>(bh) * D2);
    for (int e = blockIdx.x * 256 + threadIdx.x; e < D2 / 4; e += gridDim.x * 256) {
        if constexpr (NARROW) {
            if (last) a4[e] = w4[e];
            else s4[e] = pack_bf16x4(w4[e]);
        } else {
            w4[e] = last ? a4[e] : unpack_bf16x4(s4[e]);
        }
    }
}

template <bool NARROW>
static hipError_t state_copy(const PrefillArgs &a, hipStream_t stream)
{
    const int D2 = a.g.dv * a.g.dk;
    const int gx = std::min((D2 / 4 + 255) / 256, 16);
    hipLaunchKernelGGL(k_state_copy<NARROW>, dim3(gx, a.g.C, a.g.B * a.g.H), dim3(256), 0, stream,
                       reinterpret_cast<uint16_t *>(a.states), a.active, a.ws.work, a.meta, a.g.meta_stride, a.g.C,
                       D2);
    return hipGetLastError();
}

// The outputs of streams the fixed schedule refused (a level weight past
// column C - 1 would be needed; marked init_m < 0): NaN, as the decode step
// reports the same condition.  Their caches were left as they were.
template <typename TIO>
__global__ __launch_bounds__(256) void k_fen_refused(TIO *__restrict__ O, int T, int DV,
                                                     const int32_t *__restrict__ init_m)
{
    const int bh = blockIdx.y;
    if (init_m[bh] >= 0) return;
    const size_t n = static_cast<size_t>(T) * DV;
    TIO *o = O + static_cast<size_t>(bh) * n;
    for (size_t i = static_cast<size_t>(blockIdx.x) * 256 + threadIdx.x; i < n; i += static_cast<size_t>(gridDim.x) * 256)
        o[i] = from_f<TIO>(__builtin_nanf(""));
}

hipError_t launch_fen_refused(const PrefillArgs &a, hipStream_t stream)
{
    const int gx = static_cast<int>(std::min<int64_t>((static_cast<int64_t>(a.T) * a.g.dv + 255) / 256, 64));
    const dim3 grid(gx, a.g.B * a.g.H);
    if (a.io_bf16)
        hipLaunchKernelGGL(k_fen_refused<__bf16>, grid, dim3(256), 0, stream, static_cast<__bf16 *>(a.o), a.T, a.g.dv,
                           a.ws.init_m);
    else
        hipLaunchKernelGGL(k_fen_refused<float>, grid, dim3(256), 0, stream, static_cast<float *>(a.o), a.T, a.g.dv,
                           a.ws.init_m);
    return hipGetLastError();
}

hipError_t launch_fenwick_schedule(const PrefillArgs &a, hipStream_t stream)
{
    const int NCH = (a.T + kChunk - 1) / kChunk;
    hipLaunchKernelGGL(k_fenwick_schedule, dim3(a.g.B * a.g.H), dim3(256), 0, stream, a.T, NCH, a.g.C, a.g.dk,
                       a.ws.ev_stride, a.ws.events, a.ws.chunk_ev, a.meta, a.g.meta_stride, a.ws.init_m,
                       a.ws.init_order, a.ws.init_t);
    return hipGetLastError();
}

// The streamed chunk kernel of key width DK, slice width a.dvt.
template <typename TIO, int DK>
static hipError_t prefill_main_dk(const PrefillArgs &a, hipStream_t stream)
{
    if constexpr (sizeof(PrefillSmem<TIO, DK, 32>) <= 160 * 1024)
        if (a.dvt == 32) return prefill_main<TIO, DK, 32>(a, stream);
    return prefill_main<TIO, DK, 16>(a, stream);
}

template <typename TIO>
static hipError_t prefill_typed(const PrefillArgs &a, hipStream_t stream)
{
    hipError_t e;
    const bool fen = a.merge_rule == DLA_FENWICK;
    if (fen) e = launch_fenwick_schedule(a, stream);
    else if (a.g.dk == 64) e = prefill_schedule<TIO, 64>(a, stream);
    else if (a.g.dk == 128) e = prefill_schedule<TIO, 128>(a, stream);
    else if constexpr (sizeof(TIO) == 2) e = prefill_schedule<TIO, 256>(a, stream);
    else return hipErrorInvalidValue;
    if (e != hipSuccess) return e;
    if (a.g.dk == 64) e = prefill_main_dk<TIO, 64>(a, stream);
    else if (a.g.dk == 128) e = prefill_main_dk<TIO, 128>(a, stream);
    else if constexpr (sizeof(TIO) == 2) e = prefill_main_dk<TIO, 256>(a, stream);
    else return hipErrorInvalidValue;
    if (e != hipSuccess || !fen) return e;
    return launch_fen_refused(a, stream);
}

static hipError_t prefill_register_resident(const PrefillArgs &a, hipStream_t stream)
{
    hipError_t e;
    if (a.merge_rule == DLA_FENWICK) {
        e = launch_fenwick_schedule(a, stream);
    } else {
        e = a.g.dk == 128 ? prefill_schedule<__bf16, 128>(a, stream) : prefill_schedule<__bf16, 64>(a, stream);
    }
    if (e != hipSuccess) return e;
    return launch_prefill_rs(a, stream);
}

hipError_t launch_prefill(const PrefillArgs &a, hipStream_t stream)
{
    if (a.register_resident) return prefill_register_resident(a, stream);
    if (a.g.state_bf16) {
        // the streamed kernels on an fp32 working copy of the states
        hipError_t e = state_copy<false>(a, stream);
        if (e != hipSuccess) return e;
        PrefillArgs b = a;
        b.states = a.ws.work;
        e = b.io_bf16 ? prefill_typed<__bf16>(b, stream) : prefill_typed<float>(b, stream);
        if (e != hipSuccess) return e;
        return state_copy<true>(a, stream);
    }
    if (a.io_bf16) return prefill_typed<__bf16>(a, stream);
    return prefill_typed<float>(a, stream);
}

template <typename TIO, int DK, int DV>
static void decode_launch(const DecodeArgs &a, hipStream_t stream)
{
    const int BH = a.g.B * a.g.H;
    const TIO *q = static_cast<const TIO *>(a.q), *k = static_cast<const TIO *>(a.k);
    const TIO *v = static_cast<const TIO *>(a.v), *l = static_cast<const TIO *>(a.lam);
    TIO *o = static_cast<TIO *>(a.o);
    if (a.merge_rule == DLA_FENWICK)
        hipLaunchKernelGGL((k_decode_fenwick<TIO, DK, DV>), dim3(BH), dim3(256), 0, stream, q, k, v, l, o, a.g.C,
                           a.states, a.meta, a.g.meta_stride);
    else if (a.g.state_bf16)
        hipLaunchKernelGGL((k_decode<TIO, DK, DV, true>), dim3(BH), dim3(256), 0, stream, q, k, v, l, o, a.tau,
                           a.g.C, a.states, a.active, a.meta, a.g.meta_stride, a.sched, a.merge_rule, a.score_rule);
    else
        hipLaunchKernelGGL((k_decode<TIO, DK, DV, false>), dim3(BH), dim3(256), 0, stream, q, k, v, l, o, a.tau,
                           a.g.C, a.states, a.active, a.meta, a.g.meta_stride, a.sched, a.merge_rule, a.score_rule);
}

template <typename TIO, int DK>
static hipError_t decode_dk(const DecodeArgs &a, hipStream_t stream)
{
    switch (a.g.dv) {
    case 64: decode_launch<TIO, DK, 64>(a, stream); break;
    case 128: decode_launch<TIO, DK, 128>(a, stream); break;
    case 256: decode_launch<TIO, DK, 256>(a, stream); break;
    default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

template <typename TIO>
static hipError_t decode_typed(const DecodeArgs &a, hipStream_t stream)
{
    switch (a.g.dk) {
    case 64: return decode_dk<TIO, 64>(a, stream);
    case 128: return decode_dk<TIO, 128>(a, stream);
    case 256: return decode_dk<TIO, 256>(a, stream);
    default: return hipErrorInvalidValue;
    }
}

hipError_t launch_decode(const DecodeArgs &a, hipStream_t stream)
{
    if (a.io_bf16) return decode_typed<__bf16>(a, stream);
    return decode_typed<float>(a, stream);
}

size_t prefill_smem_bytes(int io_bf16, int dk, int dvt)
{
    if (io_bf16) {
        if (dk == 64) return dvt == 32 ? sizeof(PrefillSmem<__bf16, 64, 32>) : sizeof(PrefillSmem<__bf16, 64, 16>);
        if (dk == 128) return dvt == 32 ? sizeof(PrefillSmem<__bf16, 128, 32>) : sizeof(PrefillSmem<__bf16, 128, 16>);
        return dvt == 32 ? sizeof(PrefillSmem<__bf16, 256, 32>) : sizeof(PrefillSmem<__bf16, 256, 16>);
    }
    if (dk == 64) return dvt == 32 ? sizeof(PrefillSmem<float, 64, 32>) : sizeof(PrefillSmem<float, 64, 16>);
    if (dk == 128) return dvt == 32 ? sizeof(PrefillSmem<float, 128, 32>) : sizeof(PrefillSmem<float, 128, 16>);
    return dvt == 32 ? sizeof(PrefillSmem<float, 256, 32>) : sizeof(PrefillSmem<float, 256, 16>);
}

}  // namespace dla
