// dla_prefill_rs.hip -- chunked DLA prefill with the state stack held in
// registers (bf16 inputs, capacity C <= 32).
//
// Read and update follow the reading notes "Dynamic Linear Attention |
// Chlience Paper Archive": section 5.3 (o_t = sum_i lam_{t,i} S_i q_t over the
// bounded cache), section 5.1 (a low-information token is added to the most
// recent state, a boundary token opens one) and section 5.2 (adjacent merges
// S_i += S_{i+1} when over capacity).  The schedule comes from the greedy
// scan kernel as one event per boundary token.
//
// Two kernels:
//   k_chunk_prep  one block per (stream, 64-token chunk), all chunks in
//                 parallel: the operands of the chunk that do not depend on
//                 the state values, in MFMA-fragment order -- the query as
//                 fp16 scaled by a power of two, the read weight of every
//                 state live at the chunk start for every token (from the
//                 schedule alone), K transposed, and the intra-chunk
//                 slot-weighted causal product P = (Q K^T) o W,
//                 W[t][s] = lam_t[#live chunk starts > s].
//   k_prefill_rs  one block (4 waves) per (stream, d_v slice of DVT columns)
//                 sweeping the stream's chunks in order.  It keeps every
//                 closed state (all but the most recent) of the slice as fp16
//                 MFMA operands in the registers of the wave that owns its
//                 physical slot (slot p -> wave p % 4, register set p / 4),
//                 normalised by a power of two kept in LDS, and the most
//                 recent ("active") state as fp32 MFMA accumulators (d_k rows
//                 32w..32w+31 in wave w) plus an fp16 operand copy.  A chunk
//                 without events touches no state memory: read, P V, then
//                 V_c^T K_c accumulated into the active state's registers.  In
//                 a chunk with events the wave owning each changed slot builds
//                 its new fp32 value in registers (own value, merged-in
//                 values, V_g^T K_g of its tokens), writes it to the fp32 cache
//                 and converts it into its register copy.  A grid that would
//                 fill at most half of the device's block slots (few streams)
//                 is split along the sequence into up to four block sets per
//                 stream (float32 state storage):
//                 set s takes the chunks before its range for their
//                 state updates only (no reads, no outputs, only the key
//                 operands staged) and then sweeps its range in full, in a
//                 copy of the slots of its own (the last set in the cache).
//                 The updates are the same in every set, so the results equal
//                 the unsplit sweep's bit for bit.
//
// Operand order of the read: the reduction index d_k of a 32-wide step is
// split over lane groups g = lane / 16 as {4g..4g+3, 16+4g..16+4g+3}, the
// order in which a 16x16 accumulator pair holds rows; the query fragments use
// the same order, so the active state goes from accumulator to operand in place.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <algorithm>
#include <cstddef>
#include <cmath>
#include <type_traits>

#include "dla_device.h"
#include "dla_internal.h"

namespace dla {

// fp16 operand in the permuted reduction order from row[c0..c0+3] and
// row[c0+16..c0+19].
__device__ __forceinline__ void perm_frag_f16(Frag<_Float16> &f, const _Float16 *row, int c0)
{
    const uint2 a = *reinterpret_cast<const uint2 *>(row + c0);
    const uint2 b = *reinterpret_cast<const uint2 *>(row + c0 + 16);
    const _Float16 *xa = reinterpret_cast<const _Float16 *>(&a);
    const _Float16 *xb = reinterpret_cast<const _Float16 *>(&b);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        f.v[j] = xa[j];
        f.v[4 + j] = xb[j];
    }
}

template <int NTV>
__device__ __forceinline__ int refresh_active(const floatx4 (&am)[NTV][2], Frag<_Float16> (&af)[NTV])
{
    float mx = 0.0f;
#pragma unroll
    for (int nt = 0; nt < NTV; ++nt)
#pragma unroll
        for (int h = 0; h < 2; ++h)
#pragma unroll
            for (int j = 0; j < 4; ++j) mx = fmaxf(mx, fabsf(am[nt][h][j]));
    const int e = f16_exponent(wave_max(mx));
#pragma unroll
    for (int nt = 0; nt < NTV; ++nt)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            af[nt].v[j] = static_cast<_Float16>(ldexpf(am[nt][0][j], -e));
            af[nt].v[4 + j] = static_cast<_Float16>(ldexpf(am[nt][1][j], -e));
        }
    return e;
}

// Four 16-bit elements, the result of a transposed 8-byte LDS read.
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) i16x4 lds_i16x4;

// ------------------------------------------------------------ chunk pre-pass

// FEN: the Log-Linear fixed schedule (the schedule kernel's chunk events);
// key s is read by query t with lam_t[level], level 0 for s = t and
// 1 + (highest bit in which s and t differ) otherwise, the same for every key
// of a piece live at the chunk start.
template <int DK, bool FEN>
__global__ __launch_bounds__(256) void k_chunk_prep(
    const __bf16 *__restrict__ Q, const __bf16 *__restrict__ K, const __bf16 *__restrict__ LAM, int T, int C,
    const int2 *__restrict__ events, const int32_t *__restrict__ chunk_ev, uint8_t *__restrict__ rec,
    int32_t *__restrict__ m_t_out, const int32_t *__restrict__ init_m, const int64_t *__restrict__ init_t)
{
    constexpr int KS = DK / 32;
    // 40 KB of LDS: four blocks per compute unit.  The weighted scores P
    // reuse the query rows (wave w writes P rows 16w.. only after it has read
    // its own query rows, and every other query read ends at a barrier
    // before), and lam is kept in its bf16 input precision.
    __shared__ __align__(16) __bf16 q[kChunk][DK + 8];
    __shared__ __align__(16) __bf16 k[kChunk][DK + 8];
    __shared__ __bf16 lam[kChunk][kPrepCmax + 2];
    static_assert(DK >= kChunk, "the weighted-score rows fit the query rows");
    __bf16 (*pw)[DK + 8] = q;
    __shared__ uint64_t om[kChunk];
    __shared__ uint64_t nm[kChunk];
    __shared__ int2 evs[kChunk];
    __shared__ float red[4];
    const int ch = blockIdx.x, bh = blockIdx.y;
    const int NCH = gridDim.x;
    const int c0 = ch * kChunk;
    const int nvalid = min(kChunk, T - c0);
    const size_t tok0 = static_cast<size_t>(bh) * T;
    const size_t cb = static_cast<size_t>(bh) * NCH + ch;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    // this chunk's record: query fragments, read weights, weighted-score
    // fragments, key fragments (written with nontemporal hints: the sweep
    // reads a record only after many others have been written)
    uint8_t *rb = rec + cb * rs_record_bytes(DK);
    f16x8 *q16f = reinterpret_cast<f16x8 *>(rb);
    __bf16 *wrow = reinterpret_cast<__bf16 *>(rb + rs_rec_q_bytes(DK));
    bf16x8 *pwf = reinterpret_cast<bf16x8 *>(rb + rs_rec_a_bytes(DK));
    bf16x8 *ktf = reinterpret_cast<bf16x8 *>(rb + rs_rec_a_bytes(DK) + 2 * kChunk * kChunk);
    const int lr = lane & 15, lg = lane >> 4;
    // fixed schedule: the position the call starts at (a refused stream is
    // left alone: its outputs are set apart and its records never read)
    int64_t t0 = 0;
    if constexpr (FEN) {
        if (init_m[bh] < 0) return;
        t0 = init_t[bh];
    }
    const int64_t ts = t0 + c0;         // absolute position of the chunk's first token

    float qmax = 0.0f;
#pragma unroll
    for (int j = 0; j < DK / 32; ++j) {
        const int idx = tid + 256 * j;
        const int r = idx & (kChunk - 1), cv = (idx / kChunk) * 8;
        uint4 qv = make_uint4(0, 0, 0, 0), kv = qv;
        if (r < nvalid) {
            const size_t off = (tok0 + c0 + r) * DK + cv;
            qv = *reinterpret_cast<const uint4 *>(Q + off);
            kv = *reinterpret_cast<const uint4 *>(K + off);
        }
        *reinterpret_cast<uint4 *>(&q[r][cv]) = qv;
        *reinterpret_cast<uint4 *>(&k[r][cv]) = kv;
        const __bf16 *qe = reinterpret_cast<const __bf16 *>(&qv);
#pragma unroll
        for (int e = 0; e < 8; ++e) qmax = fmaxf(qmax, fabsf(static_cast<float>(qe[e])));
    }
#pragma unroll
    for (int j = 0; j < kPrepCmax / 4; ++j) {
        const int idx = tid + 256 * j;
        const int r = idx & (kChunk - 1), c = idx / kChunk;
        lam[r][c] = (c < C && r < nvalid) ? LAM[(tok0 + c0 + r) * C + c] : static_cast<__bf16>(0.0f);
    }
    const int e0 = chunk_ev[static_cast<size_t>(bh) * (NCH + 1) + ch];
    const int nev = chunk_ev[static_cast<size_t>(bh) * (NCH + 1) + ch + 1] - e0;
    // states live at the chunk start: those the cache held when the call
    // started, plus one per boundary before the chunk, capped at C by the merges
    // (fixed schedule from position 0: the chunk-level pieces; from t0 > 0:
    // the buckets of [0, ts))
    const int m0 = FEN ? (t0 > 0 ? __popcll(ts) : ch == 0 ? 0 : __popc((ch & 1) ? ch : ch - 1))
                       : min(C, init_m[bh] + e0);
    if (!FEN && tid < nev) evs[tid] = events[tok0 + e0 + tid];
    qmax = wave_max(qmax);
    if (lane == 0) red[wave] = qmax;
    __syncthreads();
    const int qexp = f16_exponent(fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3])));
    if (!FEN && tid < kChunk) {
        // bit i of o: the state with chronological index i at the chunk start
        // is live after token tid; bit p of m: the state opened at chunk
        // position p is live after token tid
        uint64_t o = low_bits(m0), m = 0;
        for (int e = 0; e < nev; ++e) {
            const int2 ev = evs[e];
            const int pos = ev.x - c0;
            if (tid >= pos) {
                m |= 1ull << pos;
                if (ev.y >= 64) m &= ~(1ull << (ev.y - 64));
                else if (ev.y >= 0) o &= ~(1ull << ev.y);
            }
        }
        om[tid] = o;
        nm[tid] = m;
        if (m_t_out && tid < nvalid) m_t_out[tok0 + c0 + tid] = __popcll(o) + __popcll(m);
    }
    // fp16 query fragments (permuted reduction order)
#pragma unroll
    for (int j = 0; j < KS; ++j) {
        const int f = tid + 256 * j;                   // (mt, ks, lane)
        const int l = f & 63, ks = (f >> 6) % KS, mt = (f >> 6) / KS;
        const __bf16 *row = q[16 * mt + (l & 15)];
        const int cc = 32 * ks + 4 * (l >> 4);
        f16x8 h;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            h[e] = static_cast<_Float16>(ldexpf(static_cast<float>(row[cc + e]), -qexp));
            h[4 + e] = static_cast<_Float16>(ldexpf(static_cast<float>(row[cc + 16 + e]), -qexp));
        }
        __builtin_nontemporal_store(h, &q16f[f]);
    }
    // K^T fragments: d_k rows of a 16-tile, 8 consecutive tokens per lane, by
    // two transposed 8-byte LDS reads (each wave one (tile, kk) pair per step:
    // in a 16-lane group, lane i receives element i % 4 of the reads of lanes
    // 4 k + i / 4, so lane q reads row t0 + q / 4, columns 16 tile + 4 (q % 4) ..)
#pragma unroll
    for (int j = 0; j < DK / 32; ++j) {
        const int f = tid + 256 * j;                   // (tile, kk, lane)
        const int l = f & 63, kk = (f >> 6) & 1, tile = f >> 7;
        const int q = l & 15, t0 = 32 * kk + 8 * (l >> 4);
        const __bf16 *p0 = &k[t0 + (q >> 2)][16 * tile + 4 * (q & 3)];
        const i16x4 a = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4 *)(p0));
        const i16x4 b = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4 *)(p0 + 4 * (DK + 8)));
        __builtin_nontemporal_store(__builtin_bit_cast(bf16x8, __builtin_shufflevector(a, b, 0, 1, 2, 3, 4, 5, 6, 7)),
                                    &ktf[f]);
    }
    __syncthreads();
    // P = (Q K^T) o W on the causal triangle (wave w: rows 16w..16w+15)
    {
        const int w = wave;
        Frag<__bf16> qa[KS];
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) load_frag(qa[ks], &q[16 * w + lr][32 * ks + 8 * lg]);
#pragma unroll
        for (int nt = 0; nt < kChunk / 16; ++nt) {
            floatx4 A = floatx4{0.f, 0.f, 0.f, 0.f};
            if (nt <= w) {
#pragma unroll
                for (int ks = 0; ks < KS; ++ks) {
                    Frag<__bf16> kb;
                    load_frag(kb, &k[16 * nt + lr][32 * ks + 8 * lg]);
                    mma32(A, qa[ks], kb);
                }
            }
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int t = 16 * w + 4 * lg + r;
                const int s = 16 * nt + lr;
                float val = 0.0f;
                if (s <= t) {
                    // (fixed schedule: the level of absolute positions; rows
                    // past the stream's end hold zero scores, read column 0)
                    const int col = !FEN ? __popcll(shr64(nm[t], s + 1))
                                         : (s == t || t >= nvalid) ? 0
                                                                   : 64 - __clzll(static_cast<unsigned long long>(
                                                                              (ts + t) ^ (ts + s)));
                    val = A[r] * static_cast<float>(lam[t][col]);
                }
                pw[t][s] = static_cast<__bf16>(val);
            }
        }
    }
    __syncthreads();
#pragma unroll
    for (int j = 0; j < 2; ++j) {
        const int f = tid + 256 * j;                   // (mt, ks2, lane)
        const int l = f & 63, ks2 = (f >> 6) & 1, mt = f >> 7;
        __builtin_nontemporal_store(*reinterpret_cast<const bf16x8 *>(&pw[16 * mt + (l & 15)][32 * ks2 + 8 * (l >> 4)]), &pwf[f]);
    }
    // read weights by chronological index: a state live at the chunk start is
    // read at token t with the slot of the nearest older state still live
    // (itself, or the state it was merged into), i.e. after every live state
    // that is more recent, old or new; 0 for rows without a state.  They
    // carry the factor 2^qexp that undoes the query scaling (exact in bf16).
#pragma unroll
    for (int j = 0; j < kPrepCmax / 4; ++j) {
        const int idx = tid + 256 * j;
        const int t = idx & (kChunk - 1), i = idx / kChunk;
        float w = 0.0f;
        if (FEN && i < m0 && t < nvalid) {
            // (rows past the stream's end keep weight 0: their level could
            // exceed the last column)
            // piece i: from position 0, the bucket of the i-th set bit (from
            // the top) of the chunk count it was formed for, its first chunk
            // the bits above; from t0 > 0, the i-th bucket of [0, ts)
            const int64_t cp = t0 > 0 ? ts : static_cast<int64_t>((ch & 1) ? ch : ch - 1) * kChunk;
            int seen = 0;
            int64_t first = 0;
            for (int b = 62; b >= 0; --b)
                if ((cp >> b) & 1) {
                    if (seen == i) first = cp & ~((2ll << b) - 1);
                    ++seen;
                }
            const int col = 64 - __clzll(static_cast<unsigned long long>((ts + t) ^ first));
            w = ldexpf(static_cast<float>(lam[t][col]), qexp);
        } else if (i < m0) {
            w = ldexpf(static_cast<float>(lam[t][__popcll(shr64(om[t], i + 1)) + __popcll(nm[t])]), qexp);
        }
        wrow[i * kChunk + (t % 16) * (kChunk / 16) + t / 16] = static_cast<__bf16>(w);
    }
}

// ------------------------------------------------------------ the sweep

constexpr int kRsWaves = 4;                    // waves per sweep block; two blocks share a CU
constexpr int kRsThreads = 64 * kRsWaves;

// A chunk's operands written by k_chunk_prep, copied verbatim into LDS by
// global->LDS loads (each 16-byte piece lands at the offset it has in the
// global chunk).  Part A is read from the chunk start to the end of the
// inter-chunk read, part B from then on, so part A of the next chunk is
// loaded while part B is in use and the other way round (one buffer each).
template <int DK>
struct RsStageA {
    _Float16 qf[kChunk / 16][DK / 32][64][8];   // query fragments (permuted reduction order)
    // read weights by chronological index of the state; within a row, the
    // weight of token t sits at 4 (t % 16) + t / 16 (a lane's four row tiles
    // side by side)
    __bf16 wr[kPrepCmax][kChunk];
};
template <int DK>
struct RsStageB {
    __bf16 pwf[kChunk / 16][2][64][8];           // fragments of (Q K^T) o W
    __bf16 ktf[DK / 16][2][64][8];               // fragments of K^T
};
static_assert(sizeof(RsStageA<128>) == rs_rec_a_bytes(128) && sizeof(RsStageB<128>) == rs_rec_b_bytes(128) &&
                  sizeof(RsStageA<64>) == rs_rec_a_bytes(64) && sizeof(RsStageB<64>) == rs_rec_b_bytes(64),
              "the LDS stages mirror the two parts of a chunk record");

// The chunk's V slice, row-major (token, column), copied into LDS by
// global->LDS loads at the chunk start and read after the middle barrier.
template <int DVT>
struct RsStageV {
    __bf16 v[kChunk][DVT];
};

// Everything else the sweep keeps in LDS.  The stages are separate __shared__
// variables so that the compiler can tell that loads in flight into one never
// touch the other.
template <int DK, int DVT, int CMAX>
struct RsSmem {
    // in a chunk with events, after the read, the active state passes through it
    floatx4 abuf[(DK / 16) * (DVT / 16) * 64];
    floatx4 ored[kRsWaves][kChunk / 16][DVT / 16][64];  // partial reads: wave, row tile, column tile, lane
    int32_t order[kMaxC];       // physical slot of each live state, oldest first
    int32_t new_order[kMaxC];
    // per physical slot, what a chunk with events does to the state in it:
    // its new value is (own value if jbase) + (values of the slots in jsrc,
    // merged into it) + (V^T K of the chunk tokens [jlo, jhi))
    int32_t jbase[kMaxC];
    uint32_t jsrc[kMaxC];
    int32_t jlo[kMaxC];
    int32_t jhi[kMaxC];
    int32_t shexp[kMaxC];
    // read weights of physical slot p: row jrow[p] of the chunk's weight table
    // (the chronological index of its state) times wsc[p] = 2^(state
    // exponent); 0 for a slot without a closed state (rewritten after every
    // chunk with events, when each owner wave copies its slots' values into
    // registers)
    int32_t jrow[CMAX];
    float wsc[CMAX];
    int32_t nev;                // events of the chunk
    uint32_t jobs;              // slots whose new value an owner wave builds
    uint32_t closed_new;        // slots of the closed states after the chunk
    int32_t m_new, act_new, an_case;
};

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) void lds_void_t;
typedef __attribute__((address_space(1))) const void glb_void_t;

// One 16-byte piece per lane from global memory straight into LDS: lane l
// reads base + off (base and lds_wave the same for the whole wave, off its
// own) and its piece lands at lds_wave + 16 l.  Issued as a buffer load
// (base in a buffer resource, off as the lane's offset) rather than a global
// one: the compiler counts a global load into LDS as a possible LDS access
// too, and while one is in flight it waits for every LDS read at once
// (lgkmcnt 0) instead of for the one it needs; a buffer load into LDS is
// counted as a vector memory load only.
__device__ __forceinline__ void load_to_lds16(const void *base, uint32_t off, void *lds_wave)
{
    // raw buffer, no stride, no range limit in practice (the offsets stay
    // within the caller's buffers); word 3 as for gfx9 raw buffers
    const __amdgpu_buffer_rsrc_t r =
        __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), static_cast<short>(0), 0x7fffffff, 0x00020000);
    __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_void_t *)(lds_wave), 16, off, 0, 0, 0);
}

__device__ __forceinline__ void wait_vmem() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }

// A constant made in registers where it is used: with the register file full
// the compiler would otherwise keep such a value in scratch memory and reload
// it, and the reload waits for every vector memory load in flight (the loads
// of the next chunk's operands included).
__device__ __forceinline__ int fresh_i32(int v)
{
    asm volatile("" : "+v"(v));
    return v;
}

// base (the same for the whole wave) plus a per-lane byte offset: the form
// the global instructions take as an SGPR base and a 32-bit VGPR offset.  The
// empty asm makes the offset opaque at each use, so that the compiler does
// not hoist base + offset out of the chunk loop as a 64-bit per-lane address
// (with the register file full it would spill it and reload it from scratch
// on every chunk).
template <typename P>
__device__ __forceinline__ P *at_bytes(P *base, uint32_t off)
{
    typedef typename std::conditional<std::is_const<P>::value, const char, char>::type B;
    asm volatile("" : "+v"(off));
    return reinterpret_cast<P *>(reinterpret_cast<B *>(base) + off);
}

// Pieces j of an array of N 16-byte pieces: thread tid moves piece tid + NT j
// (wave w's instruction fills pieces 64 w + NT j .. + 63).
template <int N>
__device__ __forceinline__ void stage_array(const u32x4 *src, u32x4 *dst, int tid, int wave)
{
    const int wv = __builtin_amdgcn_readfirstlane(wave);   // (uniform: the buffer base is a scalar)
#pragma unroll
    for (int j = 0; j < (N + kRsThreads - 1) / kRsThreads; ++j)
        if (N % kRsThreads == 0 || 64 * wv + kRsThreads * j < N)
            load_to_lds16(src + 64 * wv + kRsThreads * j, 16u * (fresh_i32(tid) & 63), dst + 64 * wv + kRsThreads * j);
}

// part A / part B of chunk record cb into the stages
template <int DK>
__device__ __forceinline__ void stage_a(RsStageA<DK> &X, const uint8_t *rec, size_t cb, int tid, int wave)
{
    stage_array<rs_rec_a_bytes(DK) / 16>(reinterpret_cast<const u32x4 *>(rec + cb * rs_record_bytes(DK)),
                                         reinterpret_cast<u32x4 *>(&X), tid, wave);
}

template <int DK>
__device__ __forceinline__ void stage_b(RsStageB<DK> &Y, const uint8_t *rec, size_t cb, int tid, int wave)
{
    stage_array<rs_rec_b_bytes(DK) / 16>(
        reinterpret_cast<const u32x4 *>(rec + cb * rs_record_bytes(DK) + rs_rec_a_bytes(DK)),
        reinterpret_cast<u32x4 *>(&Y), tid, wave);
}

// only the K^T fragments of part B (a chunk taken for its updates only)
template <int DK>
__device__ __forceinline__ void stage_b_keys(RsStageB<DK> &Y, const uint8_t *rec, size_t cb, int tid, int wave)
{
    constexpr size_t kt = offsetof(RsStageB<DK>, ktf);
    stage_array<(rs_rec_b_bytes(DK) - kt) / 16>(
        reinterpret_cast<const u32x4 *>(rec + cb * rs_record_bytes(DK) + rs_rec_a_bytes(DK) + kt),
        reinterpret_cast<u32x4 *>(reinterpret_cast<uint8_t *>(&Y) + kt), tid, wave);
}

// The V slice of the chunk starting at token c0 into LDS: 16-byte piece p
// (row p / (DVT / 8), columns 8 (p % (DVT / 8)) ..) from thread p; rows past
// the end of the stream repeat its last row (their products meet zero keys
// and zero intra-chunk weights).
template <int DVT>
__device__ __forceinline__ void stage_v(RsStageV<DVT> &Vs, const __bf16 *V, size_t tok0, int c0, int T, int DV,
                                        int dv0, int tid, int wave)
{
    constexpr int PPR = DVT / 8;                 // pieces per row
    static_assert(kChunk * PPR <= kRsThreads, "one piece per thread");
    if (tid < kChunk * PPR) {
        // (the thread index made opaque here: no per-lane 64-bit address is
        // formed once and held, or spilled, across the chunk loop)
        const int t = fresh_i32(tid);
        const int r = min(t / PPR, T - 1 - c0);
        const uint32_t off = 2u * (static_cast<uint32_t>(r) * static_cast<uint32_t>(DV) + 8u * (t % PPR));
        load_to_lds16(V + (tok0 + c0) * DV + dv0, off,
                      reinterpret_cast<char *>(&Vs) + 1024 * __builtin_amdgcn_readfirstlane(wave));
    }
}


// Lane (g, i) = (lane / 16, lane % 16)'s operand of token step kk (32 tokens)
// and column tile nt of the V slice held row-major in LDS: V[32 kk + 8 g + j]
// [16 nt + i], j = 0..7, the B operand of P V and the update.  Two transposed
// 8-byte reads: in each 16-lane group, lane i receives element i % 4 of the
// reads of lanes 4 k + i / 4 (k = 0..3), so lane q reads row 32 kk + 8 g +
// q / 4 (+ 4 in the second read), columns 16 nt + 4 (q % 4) .. + 3.
template <int DVT>
__device__ __forceinline__ Frag<__bf16> v_frag(const RsStageV<DVT> &Vs, int nt, int kk, int lane)
{
    const int g = lane >> 4, q = lane & 15;
    const __bf16 *p0 = &Vs.v[32 * kk + 8 * g + (q >> 2)][16 * nt + 4 * (q & 3)];
    const i16x4 a = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4 *)(p0));
    const i16x4 b = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4 *)(p0 + 4 * DVT));
    Frag<__bf16> f;
    f.v = __builtin_bit_cast(bf16x8, __builtin_shufflevector(a, b, 0, 1, 2, 3, 4, 5, 6, 7));
    return f;
}

// The closed-state part of the inter-chunk read over the wave's first NP slot
// pairs: one 16-token row tile at a time (a quarter of the query fragments
// live), two independent product chains per pair, each product weighted per
// token with the slot's read weight: row wrow[r] of the chunk's weight table
// times wscl[r] (0 for a slot without a closed state).  Straight-line
// code: the products of one pair overlap the weighting of the previous one.
// The products are formed transposed, state fragment times query fragment
// (the two operand layouts of the 16x16x32 product are the same), so lane
// (lr, lg) holds token lr of the tile, columns 4 lg .. 4 lg + 3: its weight
// is one number per slot and tile.
template <int DK, int DVT, int SPW, int NP>
__device__ __forceinline__ void rs_read_closed(floatx4 (&Oi)[kChunk / 16][DVT / 16],
                                               const Frag<_Float16> (&stk)[SPW][DK / 32][DVT / 16],
                                               const RsStageA<DK> &X, const int (&wrow)[SPW], const float (&wscl)[SPW], int wave, int lane,
                                               int lr)
{
    constexpr int KS = DK / 32;
    constexpr int NTV = DVT / 16;
    constexpr int NW = kRsWaves;
    static_assert(2 * NP <= SPW, "pairs of the wave's slots");
    // the query fragments of a row tile rotate through one set of registers:
    // the last pair of a tile loads each fragment of the next tile as soon as
    // its own products with that fragment have issued, so the next tile's
    // loads are in flight under the tile's last products and weighting
    Frag<_Float16> qf[KS];
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) load_frag(qf[ks], X.qf[0][ks][lane]);
#pragma unroll
    for (int mt = 0; mt < kChunk / 16; ++mt) {
#pragma unroll
        for (int r2 = 0; r2 < 2 * NP; r2 += 2) {
            floatx4 P0[NTV], P1[NTV];
#pragma unroll
            for (int nt = 0; nt < NTV; ++nt) {
                P0[nt] = floatx4{0.f, 0.f, 0.f, 0.f};
                P1[nt] = floatx4{0.f, 0.f, 0.f, 0.f};
            }
#pragma unroll
            for (int ks = 0; ks < KS; ++ks) {
#pragma unroll
                for (int nt = 0; nt < NTV; ++nt) {
                    mma32(P0[nt], stk[r2][ks][nt], qf[ks]);
                    mma32(P1[nt], stk[r2 + 1][ks][nt], qf[ks]);
                }
                if (r2 + 2 == 2 * NP && mt + 1 < kChunk / 16) load_frag(qf[ks], X.qf[mt + 1][ks][lane]);
            }
            const float w0 = static_cast<float>(X.wr[wrow[r2]][(kChunk / 16) * lr + mt]) * wscl[r2];
            const float w1 = static_cast<float>(X.wr[wrow[r2 + 1]][(kChunk / 16) * lr + mt]) * wscl[r2 + 1];
#pragma unroll
            for (int nt = 0; nt < NTV; ++nt)
#pragma unroll
                for (int i = 0; i < 4; ++i) Oi[mt][nt][i] = fmaf(w1, P1[nt][i], fmaf(w0, P0[nt][i], Oi[mt][nt][i]));
        }
    }
}

// What one block carries from chunk to chunk (registers after inlining).
template <int DK, int DVT, int SPW>
struct RsCarry {
    Frag<_Float16> stk[SPW][DK / 32][DVT / 16];  // closed states of the wave's slots (fp16, normalised)
    floatx4 am[DVT / 16][2];                     // active state, d_k rows 32 kb .. 32 kb + 31 (fp32)
    Frag<_Float16> af[DVT / 16];                 // its fp16 operand copy
    int wrow[SPW];                               // read-weight rows of the wave's slots (uniform)
    float wscl[SPW];                             // and their scales (uniform)
    int2 evnext;                                 // event lane of the next chunk's window (wave 0)
    int ea;                                      // exponent of this wave's active-state operand
    int m0, act;                                 // live states, the active state's slot (uniform)
    int ewin;                                    // index of this chunk's first event in the stream
    uint32_t closed;                             // physical slots of the closed states (uniform)
};

// Four consecutive values of a state in the cache at element offset e of a
// stream's slice: fp32, or bf16 for the closed states of a bf16 cache
// (rounded to nearest even when stored).
template <bool SBF>
__device__ __forceinline__ float4 cache_load4(const void *base, size_t e)
{
    if constexpr (SBF) return unpack_bf16x4(*reinterpret_cast<const uint2 *>(static_cast<const uint16_t *>(base) + e));
    else return *reinterpret_cast<const float4 *>(static_cast<const float *>(base) + e);
}
template <bool SBF>
__device__ __forceinline__ void cache_store4(void *base, size_t e, float4 v)
{
    if constexpr (SBF)
        *reinterpret_cast<uint2 *>(static_cast<uint16_t *>(base) + e) = pack_bf16x4(v);
    else
        *reinterpret_cast<float4 *>(static_cast<float *>(base) + e) = v;
}

// Per-lane byte offset, recomputed at each use from an opaque copy of the
// thread index (kept live anyway) rather than held, or spilled, across chunks:
// lane (lr, lg) of wave w's output piece (token 16 w + lr, columns
// 4 lg .. 4 lg + 3) within a chunk.
__device__ __forceinline__ uint32_t o_offset(int tid, int DV)
{
    uint32_t t = static_cast<uint32_t>(tid);
    asm volatile("" : "+v"(t));
    const uint32_t w = t >> 6, l = t & 63;
    return 2u * ((16u * w + (l & 15u)) * static_cast<uint32_t>(DV) + 4u * (l >> 4));
}

// The chunk ranges of the block sets a stream's sweep is split into (see
// k_prefill_rs): set s sweeps chunks [first[s], first[s + 1]) in full.
constexpr int kMaxSeg = kSegScratch + 1;
struct RsSegments {
    int n;
    int first[kMaxSeg + 1];
};

// Per-block constants of the sweep.
struct RsParams {
    const __bf16 *V;
    __bf16 *O;
    int T, C, DV;
    const int2 *events;         // the stream's events
    int evtot;                  // events of the stream
    const uint8_t *rec;         // chunk records
    int bh, dv0, tid, lane, wave, lr, lg, NCH;
    size_t tok0, slot_stride;
    int c_begin, c_end;         // this block's chunks: [0, c_begin) update only, then [c_begin, c_end) in full
    int m_init;                 // states the cache held when the call started
    const uint8_t *init_order;  // their physical slots, oldest first
    void *st_base;              // the stream's slice of the slots (fp32, or bf16 closed states)
    float *act_base;            // its slice of the fp32 active-state region (bf16 cache), else NULL
};

// One chunk of the sweep: its part A operands are in X, its part B operands
// are loaded into Y at its start; part A of the next chunk goes into X once
// the inter-chunk read is done.
//
// Work split over the 4 waves: wave w owns the physical slots p = 4 r + w
// (closed states in registers), holds d_k rows 32 (w - AW) .. + 31 of the
// active state (d_k = 128: every wave), and reduces and stores the outputs of
// tokens 16 w .. 16 w + 15.
template <int DK, int DVT, int SPW, bool SBF, bool CONT, bool MAYUPD>
__device__ __forceinline__ void rs_chunk(const int ch, RsStageA<DK> &X, RsStageB<DK> &Y, RsStageV<DVT> &Vs,
                                         RsSmem<DK, DVT, kRsWaves * SPW> &S, const RsParams &A,
                                         RsCarry<DK, DVT, SPW> &c, const bool upd_chunk)
{
    // a chunk taken for its state updates only (the instance for split grids)
    const bool upd = MAYUPD && upd_chunk;
    constexpr int KS = DK / 32;
    constexpr int NTV = DVT / 16;
    constexpr int MT = kChunk / 16;
    constexpr int NW = kRsWaves;
    constexpr int AW = NW - KS;                  // first wave holding rows of the active state
    static_assert(MT == NW, "one 16-token row tile per wave");
    __bf16 *O = A.O;
    const int T = A.T, DV = A.DV;
    const int bh = A.bh, dv0 = A.dv0, tid = A.tid, lane = A.lane, wave = A.wave, lr = A.lr, lg = A.lg;
    const int NCH = A.NCH;
    const size_t tok0 = A.tok0, slot_stride = A.slot_stride;
    auto &stk = c.stk;
    auto &am = c.am;
    auto &af = c.af;
    floatx4 Oprev[NTV];                          // this chunk's outputs (rows 16 wave ..)
    const bool act_wave = wave >= AW;
    const int kb = wave - AW;                    // the active wave's 32-row d_k block

    // chunk -1 (a call starting from a non-empty cache) has no tokens and
    // stores nothing: it runs on chunk 0's operands, and only its event
    // path matters, which loads the closed states the cache holds
    const bool virt = CONT && ch < 0;
    const int c0 = ch * kChunk;
    const int nvalid = virt ? 0 : min(kChunk, T - c0);
    const int2 evcur = c.evnext;
    const bool more = ch + 1 < A.c_end;
    const size_t cb = static_cast<size_t>(bh) * NCH + (virt ? 0 : ch);
    // part A of chunk ch has landed (every wave's share) and every wave is
    // done with chunk ch - 1 (so part B may be overwritten)
    wait_vmem();
    __syncthreads();
    // ---- part B of this chunk
    if (upd) stage_b_keys<DK>(Y, A.rec, cb, tid, wave);
    else stage_b<DK>(Y, A.rec, cb, tid, wave);
    // the chunk's events: the lanes of wave 0's window (the next 64 events of
    // the stream, at most 64 per chunk) whose token lies in the chunk
    if (wave == 0) {
        const int n = __popcll(__ballot(evcur.x < c0 + kChunk));
        if (lane == 0) S.nev = n;
    }
    // ---- this chunk's V (transposed) and events into LDS
    stage_v<DVT>(Vs, A.V, tok0, virt ? 0 : c0, T, DV, dv0, tid, wave);
    // ---- inter-chunk read: closed states from registers, then the active state
    floatx4 Oi[MT][NTV];
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
        for (int nt = 0; nt < NTV; ++nt) Oi[mt][nt] = floatx4{0.f, 0.f, 0.f, 0.f};
    // the wave's slot pairs up to the last one holding a closed state (slots
    // are taken lowest-free, so the live ones gather at the low end; a slot
    // without a closed state inside the range has weight 0 and finite
    // operands): one uniform branch per chunk picks a straight-line read
    uint32_t mine = 0;          // which of the wave's slots hold a closed state (uniform)
#pragma unroll
    for (int r = 0; r < SPW; ++r) mine |= ((c.closed >> (NW * r + wave)) & 1u) << r;
    static_assert(SPW % 2 == 0 && SPW <= 8, "slots are read in pairs");
    const int npair = mine ? (33 - __builtin_clz(mine)) / 2 : 0;
    // (the two blocks on a compute unit share its SIMDs: the closed-state
    // read, a long run of independent products, issues at the lowest wave
    // priority, everything else at a higher one, so that one block's short
    // dependent phases take the issue slots they need while the other block
    // reads and the products fill the rest)
    // (a chunk taken for its state updates only reads nothing: npair = 0)
    __builtin_amdgcn_s_setprio(0);
    switch (upd ? 0 : npair) {
    case 0: break;
    case 1: rs_read_closed<DK, DVT, SPW, 1>(Oi, stk, X, c.wrow, c.wscl, wave, lane, lr); break;
    case 2: rs_read_closed<DK, DVT, SPW, (SPW >= 4 ? 2 : 1)>(Oi, stk, X, c.wrow, c.wscl, wave, lane, lr); break;
    case 3: rs_read_closed<DK, DVT, SPW, (SPW >= 6 ? 3 : 1)>(Oi, stk, X, c.wrow, c.wscl, wave, lane, lr); break;
    default: rs_read_closed<DK, DVT, SPW, SPW / 2>(Oi, stk, X, c.wrow, c.wscl, wave, lane, lr); break;
    }
    __builtin_amdgcn_s_setprio(2);
    if (!upd && c.act >= 0 && act_wave) {
        // the most recent state's weights of token 16 mt + lr, times 2^ea
        const uint2 wb = *reinterpret_cast<const uint2 *>(&X.wr[c.m0 > 0 ? c.m0 - 1 : 0][(kChunk / 16) * (fresh_i32(tid) & 15)]);
        const float wa[4] = {ldexpf(__uint_as_float(wb.x << 16), c.ea), ldexpf(__uint_as_float(wb.x & 0xffff0000u), c.ea),
                             ldexpf(__uint_as_float(wb.y << 16), c.ea), ldexpf(__uint_as_float(wb.y & 0xffff0000u), c.ea)};
        static_assert(MT == 4, "one weight per row tile in the lane's 8 bytes");
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) {
            Frag<_Float16> qa;
            load_frag(qa, X.qf[mt][kb][lane]);
#pragma unroll
            for (int nt = 0; nt < NTV; ++nt) {
                floatx4 P = floatx4{0.f, 0.f, 0.f, 0.f};
                mma32(P, af[nt], qa);
#pragma unroll
                for (int i = 0; i < 4; ++i) Oi[mt][nt][i] = fmaf(wa[mt], P[i], Oi[mt][nt][i]);
            }
        }
    }
    if (!upd) {
#pragma unroll
        for (int mt = 0; mt < MT; ++mt)
#pragma unroll
            for (int nt = 0; nt < NTV; ++nt) S.ored[wave][mt][nt][lane] = Oi[mt][nt];
    }
    // part B has landed and every wave is done with part A
    wait_vmem();
    __syncthreads();
    const int nev = __builtin_amdgcn_readfirstlane(S.nev);
    const bool has_ev = virt || nev > 0;
    // ---- part A of the next chunk; its events into registers
    if (more) {
        // (not for a next chunk that is taken for its updates only)
        if (!(upd && ch + 1 < A.c_begin)) stage_a<DK>(X, A.rec, cb + (virt ? 0 : 1), tid, wave);
        // wave 0: the window of the next chunk (past the stream's last event a
        // lane holds a token no chunk reaches)
        // (the sentinel is the destination's old value: a select on the loaded
        // value would wait for the load here)
        c.evnext = make_int2(fresh_i32(0x7fffffff), fresh_i32(-1));
        const int en = c.ewin + nev;
        if (wave == 0 && en + lane < A.evtot) c.evnext = *at_bytes(A.events + en, 8u * (fresh_i32(tid) & 63));
    }
    // ---- reduce the partial reads of rows 16 w .., add P V
    if (!upd) {
        const int w = wave;
#pragma unroll
        for (int nt = 0; nt < NTV; ++nt) {
            floatx4 sum = S.ored[0][w][nt][lane];
#pragma unroll
            for (int u = 1; u < NW; ++u) sum += S.ored[u][w][nt][lane];
            Oprev[nt] = sum;
        }
#pragma unroll
        for (int ks = 0; ks < kChunk / 32; ++ks) {
            if (32 * ks <= 16 * w + 15) {
                Frag<__bf16> a;
                load_frag(a, Y.pwf[w][ks][lane]);
#pragma unroll
                for (int nt = 0; nt < NTV; ++nt) {
                    Frag<__bf16> b;
                    b = v_frag<DVT>(Vs, nt, ks, lane);
                    mma32(Oprev[nt], b, a);
                }
            }
        }
        __bf16 *ob = O + (tok0 + c0) * DV + dv0;
        const uint32_t oo = o_offset(tid, DV);
        if (nvalid == kChunk || 16 * w + lr < nvalid) {
#pragma unroll
            for (int nt = 0; nt < NTV; ++nt) {
                const bf16x4 h = {static_cast<__bf16>(Oprev[nt][0]), static_cast<__bf16>(Oprev[nt][1]),
                                  static_cast<__bf16>(Oprev[nt][2]), static_cast<__bf16>(Oprev[nt][3])};
                *at_bytes(reinterpret_cast<bf16x4 *>(ob + 16 * nt), oo) = h;
            }
        }
    }

    // ---- chunk-end update
    if (!has_ev) {
        // every token of the chunk joins the active state: V_c^T K_c into its registers
        if (act_wave) {
#pragma unroll
            for (int kk = 0; kk < kChunk / 32; ++kk)
#pragma unroll
                for (int h = 0; h < 2; ++h) {
                    Frag<__bf16> a;
                    load_frag(a, Y.ktf[2 * kb + h][kk][lane]);
#pragma unroll
                    for (int nt = 0; nt < NTV; ++nt) {
                        Frag<__bf16> b;
                        b = v_frag<DVT>(Vs, nt, kk, lane);
                        mma32(am[nt][h], a, b);
                    }
                }
            // (its fp16 copy serves the reads: in update-only chunks, only for
            // the first full chunk after them)
            if (!upd || ch + 1 >= A.c_begin) c.ea = refresh_active<NTV>(am, af);
        }
        c.ewin += nev;
        return;
    }

    // ---- chunk with events.  The bookkeeping (one thread) turns the chunk's
    // merges and new starts into per-slot jobs; the active-state waves pass
    // the active state to LDS; then the wave owning each changed closed slot
    // builds its new fp32 value in registers (old values + merged-in values +
    // V^T K of its tokens), writes it to the cache and converts it into its
    // fp16 operand copy, and the active-state waves form the new active state.
    const int m0 = c.m0, act = c.act;
    // the active state (d_k rows in 16-row tiles) passes through abuf; a new
    // active state built by an owner wave (rare) through the partial reads,
    // which it writes only after the barrier that follows every wave's reduce
    floatx4 *actbuf = S.abuf;                                       // [DK / 16][NTV][64]
    floatx4 *anbuf = &S.ored[0][0][0][0];                           // [DK / 16][NTV][64]
    static_assert((DK / 16) * NTV * 64 <= NW * MT * NTV * 64, "a state slice fits the partial-read buffer");
    if (wave == 0 && virt) {
        // chunk -1: each closed state the cache holds is a job that keeps its
        // own value (read from the cache into its owner's registers); the
        // most recent one, already in the accumulators, stays the active state
        const int mi = A.m_init;
        const int ord = lane < mi ? A.init_order[lane] : 255;
        uint32_t jobs = 0;
        for (int i = 0; i + 1 < mi; ++i) jobs |= 1u << __builtin_amdgcn_readlane(ord, i);
        const int an = __builtin_amdgcn_readlane(ord, mi - 1);
        if (lane < mi) S.new_order[lane] = ord;
        if (lane + 1 < mi) {
            S.jbase[ord] = 1;
            S.jsrc[ord] = 0;
            S.jlo[ord] = 0;
            S.jhi[ord] = 0;
        }
        if (lane == 0) {
            S.jlo[an] = 0;
            S.jhi[an] = 0;
            S.jobs = jobs;
            S.closed_new = jobs;
            S.m_new = mi;
            S.act_new = an;
            S.an_case = 0;
        }
    } else if (wave == 0) {
        // the chunk's events are in the registers of lanes 0 .. nev - 1: the
        // live states at its end (bit i of oa: old state i, bit p of na: the
        // state opened at chunk position p) and the slots the old ones keep
        uint64_t oa = low_bits(m0), na = 0;
        uint32_t used = c.closed | (act >= 0 ? 1u << act : 0u);
        for (int e = 0; e < nev; ++e) {
            const int pos = __builtin_amdgcn_readlane(evcur.x, e) - c0;
            const int d = __builtin_amdgcn_readlane(evcur.y, e);
            na |= 1ull << pos;
            if (d >= 64) {
                na &= ~(1ull << (d - 64));
            } else if (d >= 0) {
                oa &= ~(1ull << d);
                used &= ~(1u << S.order[d]);
            }
        }
        // old states still live keep their value and their order (lane i: old state i)
        const int ln = fresh_i32(tid) & 63;     // (= lane, formed here rather than held)
        if (ln < m0 && ((oa >> ln) & 1ull)) {
            const int p = S.order[ln];
            // (position: the live old states in lower lanes, counted by mbcnt)
            S.new_order[__builtin_amdgcn_mbcnt_hi(static_cast<uint32_t>(oa >> 32),
                                                  __builtin_amdgcn_mbcnt_lo(static_cast<uint32_t>(oa), 0u))] = p;
            S.jbase[p] = 1;
            S.jsrc[p] = 0;
            S.jlo[p] = 0;
            S.jhi[p] = 0;
        }
        uint32_t jobs = 0;
        // a state merged away joins the nearest older live state (the oldest
        // state is never merged away) and is no longer read
        for (uint64_t dead = low_bits(m0) & ~oa; dead; dead &= dead - 1) {
            const int i = __builtin_ctzll(dead);
            const uint64_t older = oa & low_bits(i);
            const int tp = S.order[older ? 63 - __builtin_clzll(older) : 0];
            const int dp = S.order[i];
            if (lane == 0) {
                S.jsrc[tp] |= 1u << dp;
                S.jrow[dp] = 0;
                S.wsc[dp] = 0.0f;
            }
            jobs |= 1u << tp;
        }
        const int nold = __popcll(oa);
        const int last_p = nold ? S.order[63 - __builtin_clzll(oa)] : -1;
        const int first_new = na ? __builtin_ctzll(na) : nvalid;
        if (first_new > 0 && nold > 0) {
            // the chunk's tokens before its first new state join the last old state
            if (lane == 0) S.jhi[last_p] = first_new;
            jobs |= 1u << last_p;
        }
        int mnew = nold, an = last_p;
        for (uint64_t rest = na; rest;) {
            const int pos = __builtin_ctzll(rest);
            rest &= rest - 1;
            const int q = rest ? __builtin_ctzll(rest) : nvalid;
            const int slot = __builtin_ctz(~used);        // lowest free slot (at most C states live)
            used |= 1u << slot;
            if (lane == 0) {
                S.new_order[mnew] = slot;
                S.jbase[slot] = 0;
                S.jsrc[slot] = 0;
                S.jlo[slot] = pos;
                S.jhi[slot] = q;
            }
            ++mnew;
            an = slot;
            jobs |= 1u << slot;
        }
        // the previous active state, still live but no longer the most recent, closes
        if (act >= 0 && act != an && ((oa >> (m0 - 1)) & 1ull)) jobs |= 1u << act;
        // the new active state: 0 = the same state (tokens added), 1 = a new
        // state (set from its tokens; it may sit in the slot of the previous
        // active state when that one was merged away), 2 = an older state
        // (built by its owner)
        const int an_case = na ? 1 : (an == act ? 0 : 2);
        if (an_case != 2) jobs &= ~(1u << an);
        if (lane == 0) {
            S.jobs = jobs;
            S.closed_new = used & ~(1u << an);
            S.m_new = mnew;
            S.act_new = an;
            S.an_case = an_case;
        }
    }
    if (act >= 0 && act_wave) {
#pragma unroll
        for (int nt = 0; nt < NTV; ++nt)
#pragma unroll
            for (int h = 0; h < 2; ++h) actbuf[((2 * kb + h) * NTV + nt) * 64 + lane] = am[nt][h];
    }
    // LDS-only barriers from here on: the loads in flight (next chunk's
    // operands) and the stores of this chunk drain behind them; a state's
    // fp32 value written here is read by another wave only in a later chunk,
    // after the chunk-start barrier that waits for every wave's stores
    lds_barrier();
    const int an = S.act_new, an_case = S.an_case;
    uint32_t mine_jobs = 0;     // the wave's slots with a job (uniform)
    {
        const uint32_t jobs = __builtin_amdgcn_readfirstlane(S.jobs);
#pragma unroll
        for (int r = 0; r < SPW; ++r) mine_jobs |= ((jobs >> (NW * r + wave)) & 1u) << r;
    }
#pragma unroll
    for (int r = 0; r < SPW; ++r) {
        if (!((mine_jobs >> r) & 1u)) continue;
        const int p = NW * r + wave;
        // the new value in d_k tiles (rows 16 kt + 4 lg + e, column 16 nt + lr)
        floatx4 acc[DK / 16][NTV];
        const int jbase = __builtin_amdgcn_readfirstlane(S.jbase[p]);
        const uint32_t jsrc = __builtin_amdgcn_readfirstlane(S.jsrc[p]);
        const int lo = __builtin_amdgcn_readfirstlane(S.jlo[p]), hi = __builtin_amdgcn_readfirstlane(S.jhi[p]);
        const uint32_t parts = (jbase ? 1u << p : 0u) | jsrc;
#pragma unroll
        for (int kt = 0; kt < DK / 16; ++kt)
#pragma unroll
            for (int nt = 0; nt < NTV; ++nt) acc[kt][nt] = floatx4{0.f, 0.f, 0.f, 0.f};
        for (uint32_t pm = parts; pm; pm &= pm - 1) {
            const int q = __builtin_ctz(pm);
            if (q == act) {
#pragma unroll
                for (int kt = 0; kt < DK / 16; ++kt)
#pragma unroll
                    for (int nt = 0; nt < NTV; ++nt) acc[kt][nt] += actbuf[(kt * NTV + nt) * 64 + lane];
            } else {
#pragma unroll
                for (int kt = 0; kt < DK / 16; ++kt)
#pragma unroll
                    for (int nt = 0; nt < NTV; ++nt) {
                        const float4 v = cache_load4<SBF>(A.st_base, q * slot_stride + (16 * nt + lr) * DK + 16 * kt + 4 * lg);
                        acc[kt][nt] += floatx4{v.x, v.y, v.z, v.w};
                    }
            }
        }
        if (hi > lo) {
#pragma unroll
            for (int kk = 0; kk < kChunk / 32; ++kk) {
                if (32 * kk >= hi || 32 * kk + 32 <= lo) continue;
                Frag<__bf16> b[NTV];
#pragma unroll
                for (int nt = 0; nt < NTV; ++nt) b[nt] = v_frag<DVT>(Vs, nt, kk, lane);
#pragma unroll
                for (int kt = 0; kt < DK / 16; ++kt) {
                    Frag<__bf16> a;
                    load_frag(a, Y.ktf[kt][kk][lane]);
                    mask_frag(a, 32 * kk + 8 * lg, lo, hi);
#pragma unroll
                    for (int nt = 0; nt < NTV; ++nt) mma32(acc[kt][nt], a, b[nt]);
                }
            }
        }
        if (p == an) {
            // an older state becomes the active one: hand it to the active-state waves
#pragma unroll
            for (int kt = 0; kt < DK / 16; ++kt)
#pragma unroll
                for (int nt = 0; nt < NTV; ++nt) anbuf[(kt * NTV + nt) * 64 + lane] = acc[kt][nt];
            continue;
        }
        // fp32 value into the cache (a new state's slot may be the slot of a
        // state merged away in this chunk, which another wave may still be
        // reading: new states are written after the next barrier), normalised
        // fp16 copy into the registers
        float mx = 0.0f;
#pragma unroll
        for (int kt = 0; kt < DK / 16; ++kt)
#pragma unroll
            for (int nt = 0; nt < NTV; ++nt) {
                const floatx4 v = acc[kt][nt];
                if (jbase)
                    cache_store4<SBF>(A.st_base, p * slot_stride + (16 * nt + lr) * DK + 16 * kt + 4 * lg,
                                 make_float4(v[0], v[1], v[2], v[3]));
                mx = fmaxf(mx, fmaxf(fmaxf(fabsf(v[0]), fabsf(v[1])), fmaxf(fabsf(v[2]), fabsf(v[3]))));
            }
        const int e = f16_exponent(wave_max(mx));
        if (lane == 0) S.shexp[p] = e;
#pragma unroll
        for (int ks = 0; ks < KS; ++ks)
#pragma unroll
            for (int nt = 0; nt < NTV; ++nt)
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    stk[r][ks][nt].v[j] = static_cast<_Float16>(ldexpf(acc[2 * ks][nt][j], -e));
                    stk[r][ks][nt].v[4 + j] = static_cast<_Float16>(ldexpf(acc[2 * ks + 1][nt][j], -e));
                }
    }
    // every merged-in value has been read (the loads have returned, their
    // values are used) and anbuf is written by the owner of an
    lds_barrier();
    // new closed states: their fp32 values into the cache (recomputed from their tokens)
#pragma unroll
    for (int r = 0; r < SPW; ++r) {
        if (!((mine_jobs >> r) & 1u)) continue;
        const int p = NW * r + wave;
        if (p == an || S.jbase[p]) continue;
        const int lo = __builtin_amdgcn_readfirstlane(S.jlo[p]), hi = __builtin_amdgcn_readfirstlane(S.jhi[p]);
        floatx4 acc[DK / 16][NTV];
#pragma unroll
        for (int kt = 0; kt < DK / 16; ++kt)
#pragma unroll
            for (int nt = 0; nt < NTV; ++nt) acc[kt][nt] = floatx4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int kk = 0; kk < kChunk / 32; ++kk) {
            if (32 * kk >= hi || 32 * kk + 32 <= lo) continue;
            Frag<__bf16> b[NTV];
#pragma unroll
            for (int nt = 0; nt < NTV; ++nt) b[nt] = v_frag<DVT>(Vs, nt, kk, lane);
#pragma unroll
            for (int kt = 0; kt < DK / 16; ++kt) {
                Frag<__bf16> a;
                load_frag(a, Y.ktf[kt][kk][lane]);
                mask_frag(a, 32 * kk + 8 * lg, lo, hi);
#pragma unroll
                for (int nt = 0; nt < NTV; ++nt) mma32(acc[kt][nt], a, b[nt]);
            }
        }
#pragma unroll
        for (int kt = 0; kt < DK / 16; ++kt)
#pragma unroll
            for (int nt = 0; nt < NTV; ++nt)
                cache_store4<SBF>(A.st_base, p * slot_stride + (16 * nt + lr) * DK + 16 * kt + 4 * lg,
                             make_float4(acc[kt][nt][0], acc[kt][nt][1], acc[kt][nt][2], acc[kt][nt][3]));
    }
    // the new active state into the accumulators
    if (act_wave) {
        if (an_case == 2) {
#pragma unroll
            for (int nt = 0; nt < NTV; ++nt)
#pragma unroll
                for (int h = 0; h < 2; ++h) am[nt][h] = anbuf[((2 * kb + h) * NTV + nt) * 64 + lane];
        } else {
            const int lo = S.jlo[an], hi = S.jhi[an];
            if (an_case == 1) {
#pragma unroll
                for (int nt = 0; nt < NTV; ++nt) {
                    am[nt][0] = floatx4{0.f, 0.f, 0.f, 0.f};
                    am[nt][1] = floatx4{0.f, 0.f, 0.f, 0.f};
                }
            }
#pragma unroll
            for (int kk = 0; kk < kChunk / 32; ++kk) {
                if (32 * kk >= hi || 32 * kk + 32 <= lo) continue;
#pragma unroll
                for (int h = 0; h < 2; ++h) {
                    Frag<__bf16> a;
                    load_frag(a, Y.ktf[2 * kb + h][kk][lane]);
                    mask_frag(a, 32 * kk + 8 * lg, lo, hi);
#pragma unroll
                    for (int nt = 0; nt < NTV; ++nt) {
                        Frag<__bf16> b;
                        b = v_frag<DVT>(Vs, nt, kk, lane);
                        mma32(am[nt][h], a, b);
                    }
                }
            }
        }
        if (!upd || ch + 1 >= A.c_begin) c.ea = refresh_active<NTV>(am, af);
    }
    const int mnew = __builtin_amdgcn_readfirstlane(S.m_new);
    const uint32_t cl = __builtin_amdgcn_readfirstlane(S.closed_new);
    lds_barrier();
    // the new order; read weights of the closed states from the next chunk on
    // (their exponents are final; the slots merged away were cleared)
    if (tid < mnew) {
        const int p = S.new_order[tid];
        S.order[tid] = p;
        const bool closed = tid + 1 < mnew;
        S.jrow[p] = closed ? tid : 0;
        S.wsc[p] = closed ? ldexpf(1.0f, S.shexp[p]) : 0.0f;
    }
    // every owner wave takes its slots' read weights into registers
    lds_barrier();
#pragma unroll
    for (int r = 0; r < SPW; ++r) {
        c.wrow[r] = __builtin_amdgcn_readfirstlane(S.jrow[NW * r + wave]);
        c.wscl[r] = __int_as_float(__builtin_amdgcn_readfirstlane(__float_as_int(S.wsc[NW * r + wave])));
    }
    c.m0 = mnew;
    c.act = an;
    c.closed = cl;
    c.ewin += nev;
}

template <int DK, int DVT, int SPW, bool SBF, bool CONT, bool SPLIT>
__global__ __launch_bounds__(kRsThreads, 2) void k_prefill_rs(
    const __bf16 *__restrict__ V, __bf16 *__restrict__ O, int T, int C, int DV, int nblk_dv,
    float *__restrict__ states, float *__restrict__ active, const int2 *__restrict__ events, size_t ev_stride,
    const int32_t *__restrict__ chunk_ev, const uint8_t *__restrict__ rec,
    uint8_t *__restrict__ meta_base, size_t meta_stride, const int32_t *__restrict__ init_m,
    const uint8_t *__restrict__ init_order, const RsSegments seg, float *__restrict__ seg_states)
{
    constexpr int KS = DK / 32;
    constexpr int NTV = DVT / 16;
    constexpr int CMAX = kRsWaves * SPW;
    static_assert(KS <= kRsWaves, "one wave per 32-row block of the active state");
    static_assert(kChunk * DVT / 8 <= kRsThreads, "one 16-byte V piece per thread");
    static_assert(CMAX <= kPrepCmax, "a chunk record holds lam for 32 slots");
    __shared__ RsStageA<DK> stA;
    __shared__ RsStageB<DK> stB;
    __shared__ RsStageV<DVT> stV;
    __shared__ RsSmem<DK, DVT, CMAX> S;

    const int nblk = gridDim.x;
    int lin = blockIdx.x;
    if ((nblk & 7) == 0) lin = (blockIdx.x & 7) * (nblk >> 3) + (blockIdx.x >> 3);
    // block lin: segment sg = lin / (BH nblk_dv) of stream (lin / nblk_dv) % BH
    const int BHn = nblk / (seg.n * nblk_dv);
    const int sg = lin / (BHn * nblk_dv);
    lin -= sg * BHn * nblk_dv;
    RsParams A;
    A.V = V; A.O = O; A.T = T; A.C = C; A.DV = DV;
    A.rec = rec;
    A.bh = lin / nblk_dv;
    A.events = events + static_cast<size_t>(A.bh) * ev_stride;
    A.dv0 = (lin % nblk_dv) * DVT;
    A.tid = threadIdx.x;
    A.lane = A.tid & 63;
    A.wave = __builtin_amdgcn_readfirstlane(A.tid >> 6);
    A.lr = A.lane & 15;
    A.lg = A.lane >> 4;
    A.NCH = (T + kChunk - 1) / kChunk;
    A.tok0 = static_cast<size_t>(A.bh) * T;
    A.slot_stride = static_cast<size_t>(DV) * DK;
    {
        const size_t off = static_cast<size_t>(A.bh) * C * DV * DK + static_cast<size_t>(A.dv0) * DK;
        A.st_base = SBF ? static_cast<void *>(reinterpret_cast<uint16_t *>(states) + off)
                        : static_cast<void *>(states + off);
        A.act_base = SBF ? active + static_cast<size_t>(A.bh) * DV * DK + static_cast<size_t>(A.dv0) * DK
                         : nullptr;
    }
    A.evtot = chunk_ev[static_cast<size_t>(A.bh) * (A.NCH + 1) + A.NCH];
    const int tid = A.tid, wave = A.wave, lr = A.lr, lg = A.lg, NCH = A.NCH;

    RsCarry<DK, DVT, SPW> c;
#pragma unroll
    for (int r = 0; r < SPW; ++r)
#pragma unroll
        for (int ks = 0; ks < KS; ++ks)
#pragma unroll
            for (int nt = 0; nt < NTV; ++nt) zero_frag(c.stk[r][ks][nt]);
#pragma unroll
    for (int nt = 0; nt < NTV; ++nt) {
        c.am[nt][0] = floatx4{0.f, 0.f, 0.f, 0.f};
        c.am[nt][1] = floatx4{0.f, 0.f, 0.f, 0.f};
        zero_frag(c.af[nt]);
    }
    if (tid < CMAX) { S.jrow[tid] = 0; S.wsc[tid] = 0.0f; }
#pragma unroll
    for (int r = 0; r < SPW; ++r) {
        c.wrow[r] = 0;
        c.wscl[r] = 0.0f;
    }
    c.ea = 0;
    c.m0 = 0;
    c.act = -1;
    c.closed = 0;
    if (tid < kMaxC) { S.order[tid] = tid; S.shexp[tid] = 0; }

    // the states the cache holds when the call starts (oldest first, in the
    // physical slots the greedy scan recorded): the closed ones into their
    // owner waves' fp16 operand registers, the most recent one into the
    // active-state accumulators
    // the states the cache holds when the call starts: the most recent one
    // into the active-state accumulators here, the closed ones through the
    // event path of a chunk -1 (which loads each from the cache into its
    // owner wave's registers)
    A.m_init = init_m[A.bh];
    A.init_order = init_order + static_cast<size_t>(A.bh) * kMaxC;
    // two instances are launched: CONT for streams whose cache holds states,
    // the other for empty ones (the sweep without the start-up code); a block
    // of the other kind leaves at once (the whole block: no barrier is met)
    // (a stream the fixed schedule refused, m_init < 0, is left to a later kernel)
    if (A.m_init < 0 || (A.m_init > 0) != CONT) return;
    // segments (float32 state storage): the stream is swept by seg.n block
    // sets; set sg takes chunks [0, first[sg]) for their state updates only
    // (the same updates and merges, in the same order, as any set) and chunks
    // [first[sg], first[sg + 1]) in full, in slots of its own (the last set
    // in the cache), which start as a copy of the cache's.
    const bool split = SPLIT && !SBF && seg.n > 1;
    const bool last_set = sg == seg.n - 1;
    if (!split && !last_set) return;
    A.c_begin = split ? seg.first[sg] : 0;
    A.c_end = split ? seg.first[sg + 1] : NCH;
    if (split && !last_set) {
        float *own = seg_states + (static_cast<size_t>(sg) * BHn + A.bh) * C * DV * DK + static_cast<size_t>(A.dv0) * DK;
        if (CONT) {
            // the states the cache holds: this block's rows of every slot
            const float *from = static_cast<const float *>(A.st_base);
            constexpr int PER = DVT * DK / 4;          // 16-byte pieces of a slot's rows
            for (int i = tid; i < C * PER; i += kRsThreads) {
                const int p = i / PER, e = i % PER;
                reinterpret_cast<float4 *>(own + p * A.slot_stride)[e] =
                    reinterpret_cast<const float4 *>(from + p * A.slot_stride)[e];
            }
            __syncthreads();
        }
        A.st_base = own;
    }
    if (CONT) {
        c.act = A.init_order[A.m_init - 1];
        if (A.m_init == 1) {
            c.m0 = 1;
            if (tid == 0) S.order[0] = c.act;
        }
        const int kb = wave - (kRsWaves - KS);
        if (kb >= 0) {
            const float *src = SBF ? A.act_base : static_cast<const float *>(A.st_base) + c.act * A.slot_stride;
#pragma unroll
            for (int nt = 0; nt < NTV; ++nt)
#pragma unroll
                for (int h = 0; h < 2; ++h) {
                    const float4 v = *reinterpret_cast<const float4 *>(src + (16 * nt + lr) * DK + 32 * kb + 16 * h + 4 * lg);
                    c.am[nt][h] = floatx4{v.x, v.y, v.z, v.w};
                }
            c.ea = refresh_active<NTV>(c.am, c.af);
        }
    }

    // chunk 0: part A into LDS, events into registers
    stage_a<DK>(stA, rec, static_cast<size_t>(A.bh) * NCH, tid, wave);
    // wave 0: the window of chunk 0 (the stream's first 64 events)
    c.ewin = 0;
    c.evnext = make_int2(0x7fffffff, -1);
    if (wave == 0 && A.lane < A.evtot) c.evnext = A.events[A.lane];

    // (a later block set first takes the chunks before its range for their
    // updates only; only a stream that starts from an empty cache is split)
    // (the update-only chunk code is in the instance launched for split grids
    // only, so that it takes no registers from the other instances' sweep)
    for (int ch = (CONT && A.m_init > 1) ? -1 : 0; ch < A.c_end; ++ch)
        rs_chunk<DK, DVT, SPW, SBF, CONT, SPLIT>(ch, stA, stB, stV, S, A, c, ch < A.c_begin);

    // the active state's accumulators are the last state of the final cache
    const int kb = wave - (kRsWaves - KS);
    if (c.act >= 0 && kb >= 0) {
        // (fp32 in its slot, or in the active-state region of a bf16 cache)
        float *dst = SBF ? A.act_base : static_cast<float *>(A.st_base) + c.act * A.slot_stride;
#pragma unroll
        for (int nt = 0; nt < NTV; ++nt)
#pragma unroll
            for (int h = 0; h < 2; ++h)
                *reinterpret_cast<float4 *>(dst + (16 * nt + lr) * DK + 32 * kb + 16 * h + 4 * lg) =
                    make_float4(c.am[nt][h][0], c.am[nt][h][1], c.am[nt][h][2], c.am[nt][h][3]);
    }
    __syncthreads();
    if (last_set && A.dv0 == 0 && tid < kMaxC) {
        uint8_t *order = meta_base + static_cast<size_t>(A.bh) * meta_stride + kOffOrder;
        order[tid] = static_cast<uint8_t>(tid < c.m0 ? S.order[tid] : 0xFF);
    }
}

template <int DK, int DVT, int SPW>
static hipError_t launch_rs(const PrefillArgs &a, hipStream_t stream)
{
    const int BH = a.g.B * a.g.H;
    // the greedy scan writes T events per stream at most, the fixed schedule
    // up to max(T, 64)
    const size_t ev_stride = a.merge_rule == DLA_FENWICK ? a.ws.ev_stride : static_cast<size_t>(a.T);
    const int nblk_dv = a.g.dv / DVT;
    const int NCH = (a.T + kChunk - 1) / kChunk;
#define DLA_PREP_LAUNCH(FEN_)                                                                               \
    hipLaunchKernelGGL((k_chunk_prep<DK, FEN_>), dim3(NCH, BH), dim3(256), 0, stream,                      \
                       static_cast<const __bf16 *>(a.q), static_cast<const __bf16 *>(a.k),                  \
                       static_cast<const __bf16 *>(a.lam), a.T, a.g.C, a.ws.events, a.ws.chunk_ev,          \
                       static_cast<uint8_t *>(a.ws.rec), a.sched.m_t, a.ws.init_m, a.ws.init_t)
    if (a.merge_rule == DLA_FENWICK) DLA_PREP_LAUNCH(true);
    else DLA_PREP_LAUNCH(false);
#undef DLA_PREP_LAUNCH
    hipError_t e0 = hipGetLastError();
    if (e0 != hipSuccess) return e0;
    if (a.ev_before) {
        hipError_t e = hipEventRecord(a.ev_before, stream);
        if (e != hipSuccess) return e;
    }
    // A grid that fills at most half the block slots is split along the
    // sequence into seg.n block sets (float32 state storage).  Set s sweeps chunks
    // [first[s], first[s + 1]) in full after chunks [0, first[s]) for their
    // updates only, which cost a fraction x of a full chunk; the ranges are
    // chosen so that every set has the same work: first[s] = tau (1 - (1 -
    // x)^s) / x with tau = NCH x / (1 - (1 - x)^n).
    RsSegments seg{};
    seg.n = 1;
    {
        const int blocks = BH * nblk_dv;
        int n = a.seg_slots > 0 ? std::min(kMaxSeg, a.seg_slots / blocks) : 1;
        n = std::min(std::min(n, NCH / 8), 1 + a.ws.seg_sets);
        if (n >= 2 && a.ws.seg_states && !a.g.state_bf16) {
            constexpr double x = 0.3;
            const double tau = NCH * x / (1.0 - std::pow(1.0 - x, n));
            seg.n = n;
            seg.first[0] = 0;
            for (int k = 1; k < n; ++k) {
                const int f = static_cast<int>(std::lround(tau * (1.0 - std::pow(1.0 - x, k)) / x));
                seg.first[k] = std::min(std::max(f, seg.first[k - 1] + 1), NCH - (n - k));
            }
            seg.first[n] = NCH;
        } else {
            seg.first[1] = NCH;
        }
    }
#define DLA_RS_LAUNCH(SBF_, CONT_, SPLIT_)                                                                  \
    hipLaunchKernelGGL((k_prefill_rs<DK, DVT, SPW, SBF_, CONT_, SPLIT_>), dim3(seg.n * BH * nblk_dv), dim3(kRsThreads), 0, stream, \
                       static_cast<const __bf16 *>(a.v), static_cast<__bf16 *>(a.o), a.T, a.g.C, a.g.dv, nblk_dv,    \
                       a.states, a.active, a.ws.events, ev_stride, a.ws.chunk_ev,                                   \
                       static_cast<const uint8_t *>(a.ws.rec), a.meta, a.g.meta_stride, a.ws.init_m, a.ws.init_order, \
                       seg, a.ws.seg_states)
    // streams starting from an empty cache, then those continuing one
    if (a.g.state_bf16) {
        DLA_RS_LAUNCH(true, false, false);
        DLA_RS_LAUNCH(true, true, false);
    } else {
        if (seg.n > 1) {
            DLA_RS_LAUNCH(false, false, true);
            DLA_RS_LAUNCH(false, true, true);
        } else {
            DLA_RS_LAUNCH(false, false, false);
            DLA_RS_LAUNCH(false, true, false);
        }
    }
#undef DLA_RS_LAUNCH
    hipError_t e = hipGetLastError();
    if (e == hipSuccess && a.ev_after) e = hipEventRecord(a.ev_after, stream);
    if (e == hipSuccess && a.merge_rule == DLA_FENWICK) e = launch_fen_refused(a, stream);
    return e;
}

// The register-resident sweep works on 16-column slices of d_v (4 waves, each
// holding C/4 states of the slice, C rounded up to 8, 16 or 32; two blocks
// share a compute unit).
int prefill_rs_dvt(int, int, int) { return 16; }

int prefill_rs_spw(int C) { return (C <= 8 ? 8 : C <= 16 ? 16 : 32) / kRsWaves; }

template <int DK>
static hipError_t launch_rs_dk(const PrefillArgs &a, hipStream_t stream)
{
    switch (prefill_rs_spw(a.g.C)) {
    case 2: return launch_rs<DK, 16, 2>(a, stream);
    case 4: return launch_rs<DK, 16, 4>(a, stream);
    default: return launch_rs<DK, 16, 8>(a, stream);
    }
}

hipError_t launch_prefill_rs(const PrefillArgs &a, hipStream_t stream)
{
    return a.g.dk == 128 ? launch_rs_dk<128>(a, stream) : launch_rs_dk<64>(a, stream);
}

template <int DK, int DVT, int CMAX>
constexpr size_t rs_lds_bytes()
{
    return sizeof(RsStageA<DK>) + sizeof(RsStageB<DK>) + sizeof(RsStageV<DVT>) + sizeof(RsSmem<DK, DVT, CMAX>);
}

size_t prefill_rs_smem_bytes(int dk, int, int C)
{
    const int cmax = C <= 8 ? 8 : (C <= 16 ? 16 : 32);
    if (dk == 128) return cmax == 8 ? rs_lds_bytes<128, 16, 8>() : cmax == 16 ? rs_lds_bytes<128, 16, 16>()
                                                                             : rs_lds_bytes<128, 16, 32>();
    return cmax == 8 ? rs_lds_bytes<64, 16, 8>() : cmax == 16 ? rs_lds_bytes<64, 16, 16>() : rs_lds_bytes<64, 16, 32>();
}

}  // namespace dla
