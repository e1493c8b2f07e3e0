// dla_state_score.hip -- the state information score of the DLA prefill
// (a cache whose score rule is DLA_SCORE_STATE).
//
// Reading notes "Dynamic Linear Attention | Chlience Paper Archive", section
// 5.1: each token builds its per-token state v_t k_t^T and compares it with
// the current (most recent) memory state S; both are RMS-normalised, and
//     I_t = ||N(v_t k_t^T) - N(S)||_F / (||N(S)||_F + eps),   eps = 1e-6;
// the token opens a new state when I_t >= tau (an empty cache always does).
// With both matrices non-zero each normalised matrix has Frobenius norm
// sqrt(D), D = d_k d_v, so
//     I_t = sqrt(2 D (1 - c)) / (sqrt(D) + eps),
//     c = <v_t k_t^T, S>_F / (|v_t| |k_t| |S|_F) = x / sqrt(nn F),
// with x = v_t^T S k_t, nn = |v_t|^2 |k_t|^2 and F = |S|_F^2; a zero matrix or
// an empty cache gives I_t = 2.
//
// The score depends on the current state, and which state is current depends
// on the earlier boundaries and capacity merges (section 5.2): a token that
// joins, or whose new state the capacity merge joins to the state before it,
// extends the current state; any other boundary restarts it at the token.
// The current state is therefore always a suffix [a, t) of the stream.  One
// block per stream sweeps the 64-token chunks in order, with the part of the
// current state that precedes the chunk, S_pre = sum over [a, c0) of v k^T,
// held as fp32 MFMA accumulators, its 16 x 16 tiles spread over the block's
// waves (eight waves by key columns, or four by value rows for the larger
// shapes):
//   1. u_t = v_t^T S_pre k_t for the chunk's tokens: Y = S_pre K^T on MFMA,
//      S_pre split into two fp16 halves (22 significant bits) and K exact in
//      fp16 (bf16 inputs) or split as well (fp32 inputs), then u_t = v_t . Y_t
//      (each wave's part over its tiles, summed in the scan);
//   2. the chunk's Gram products H[t][s] = (v_t . v_s)(k_t . k_s) on MFMA and
//      their row sums in fp64 (the part of x_t inside the chunk while the
//      current state began before it);
//   3. one wave scores the tokens in passes, a lane per token: a pass scores
//      every token against the current state as if none restarted it (x_t
//      from the row sums, or from the Gram row from the state's start when it
//      began inside the chunk; |S|_F^2 as a prefix sum of 2 x + |v|^2 |k|^2),
//      then walks the boundaries in order with the greedy merge decision
//      (same rule and arithmetic as the greedy scan kernel): a boundary
//      merged into the newest pair keeps the pass going (a run of them is
//      taken at once), any other restarts the current state at the boundary
//      token and the next pass begins after it;
//   4. S_pre of the next chunk: the tokens of the chunk from the current
//      state's start on are added (the accumulators are cleared first if the
//      current state restarted inside the chunk).
// The kernel writes what the cosine score kernel writes (scores, their 2^-32
// fixed-point values, boundary flags, per-tile boundary counts and sums); the
// boundary compaction and the greedy scan then build the schedule exactly as
// for the cosine score.  It reads the cache (the states it holds when the
// call starts) and writes nothing into it.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "dla_device.h"
#include "dla_internal.h"

namespace dla {

namespace {

constexpr int kSsMaxWaves = 8;

// Waves per block: eight (two per SIMD, 256 registers each) where the
// per-wave state fits, four (512 registers each) for the larger shapes.
template <typename TIO, int DK, int DV>
constexpr int ss_waves()
{
    return (sizeof(TIO) == 2 ? (DK * DV <= 128 * 64 || (DK == 256 && DV == 64)) : DK * DV <= 64 * 128) ? 8 : 4;
}

// The d_v x d_k tiles of S_pre over the NW waves: JW waves along d_k, IW along
// d_v; wave w holds the tiles (d_v tile iw + IW i, d_k tile jw + JW j) with
// jw = w % JW, iw = w / JW.  Eight waves split d_k first, so that each wave
// reads the key columns of its own d_k tiles only; four waves (the larger
// shapes, whose registers are the limit) split d_v.
template <int DK, int DV, int NW>
struct SsSplit {
    static constexpr int NJT = DK / 16, NIT = DV / 16;
    static constexpr int JW = NW == 4 ? 1 : (NJT < NW ? NJT : NW);
    static constexpr int IW = NW / JW;
    static constexpr int JPW = NJT / JW, IPW = NIT / IW;
    static_assert(JW * IW == NW && JPW * JW == NJT && IPW * IW == NIT, "whole tiles per wave");
};

template <typename TIO, int DK, int DV>
struct SsSmem {
    static constexpr int PAD = 16 / sizeof(TIO);
    TIO kr[kChunk][DK + PAD];       // K of the chunk, row-major
    TIO vr[kChunk][DV + PAD];       // V of the chunk, row-major
    TIO kt[DK][kChunk + PAD];       // K transposed
    TIO vt[DV][kChunk + PAD];       // V transposed
    // K of the chunk scaled by 2^-ek in fp16 (bf16 inputs: exact while within
    // fp16's normal range of the chunk's largest element), the operand of u_t
    _Float16 kh[sizeof(TIO) == 2 ? kChunk : 1][DK + 8];
    float H[kChunk][kChunk + 1];    // Gram products (lower triangle)
    double rowsum[kChunk];          // sum of H[t][s] over s < t
    float upart[kSsMaxWaves][kChunk];   // partial u_t of the waves
    float nn[kChunk];               // |v_t|^2 |k_t|^2
    float s_c[kChunk];              // scores of the chunk
    uint8_t f_c[kChunk];            // boundary flags of the chunk
    float red[kSsMaxWaves], kred[kSsMaxWaves];
    double dred[kSsMaxWaves];
    int64_t a_s;                    // start of the current state after the chunk (from the scan)
};

// fp16 halves of x * 2^-e: hi = fp16(x'), lo = fp16(x' - hi).
__device__ __forceinline__ void split16(float x, int e, _Float16 &hi, _Float16 &lo)
{
    const float y = ldexpf(x, -e);
    hi = static_cast<_Float16>(y);
    lo = static_cast<_Float16>(y - static_cast<float>(hi));
}

template <typename TIO, int DK, int DV>
__global__ __launch_bounds__((64 * ss_waves<TIO, DK, DV>()), 1) void k_state_score(
    const TIO *__restrict__ K, const TIO *__restrict__ V, int T, float tau, int C, int merge_rule,
    const float *__restrict__ states, const float *__restrict__ active, int state_bf16,
    const uint8_t *__restrict__ meta_base, size_t meta_stride,
    float *__restrict__ s_out, int64_t *__restrict__ qs_out, uint8_t *__restrict__ flag_out,
    int32_t *__restrict__ tile_cnt, int64_t *__restrict__ tile_sum, int NT)
{
    constexpr int NW = ss_waves<TIO, DK, DV>();
    constexpr int kSsThreads = 64 * NW;
    typedef SsSplit<DK, DV, NW> Sp;
    constexpr int IPW = Sp::IPW, JPW = Sp::JPW, IW = Sp::IW, JW = Sp::JW;
    constexpr bool kF32 = sizeof(TIO) == 4;
    extern __shared__ __align__(16) unsigned char smem_raw[];
    typedef SsSmem<TIO, DK, DV> Smem;
    Smem &S = *reinterpret_cast<Smem *>(smem_raw);

    const int bh = blockIdx.x;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int lr = lane & 15, lg = lane >> 4;
    const int jw = wave % JW, iw = wave / JW;
    const int NCH = (T + kChunk - 1) / kChunk;
    const size_t tok0 = static_cast<size_t>(bh) * T;
    const double D = static_cast<double>(DK) * DV;
    const double sqD = sqrt(D);

    // the stream as the cache holds it: its states' information and counts
    // (the greedy lanes) and its most recent state (the current one)
    const uint8_t *meta = meta_base + static_cast<size_t>(bh) * meta_stride;
    const MetaHead *head = reinterpret_cast<const MetaHead *>(meta);
    const int m_init = head->m;
    int64_t I = 0;
    int32_t n = 0;
    if (wave == 0 && lane < m_init) {
        I = reinterpret_cast<const int64_t *>(meta + kOffInfo)[lane];
        n = reinterpret_cast<const int32_t *>(meta + kOffCount)[lane];
    }
    int m = m_init;
    // S_pre accumulators: acc[i][j], the tile of d_v tile it = iw + IW i and
    // d_k tile jt = jw + JW j, holds S[16 it + lr][16 jt + 4 lg + r]
    floatx4 acc[IPW][JPW];
#pragma unroll
    for (int i = 0; i < IPW; ++i)
#pragma unroll
        for (int j = 0; j < JPW; ++j) acc[i][j] = floatx4{0.f, 0.f, 0.f, 0.f};
    double F = 0.0;          // |S_cur|_F^2 (wave 0)
    int64_t a = 0;           // start of the current state (absolute token of this call; < 0: before it)
    if (m_init > 0) {
        // (m_init is the same for the whole block)
        const int slot = meta[kOffOrder + m_init - 1];
        const float *src = state_bf16 ? active + static_cast<size_t>(bh) * DV * DK
                                      : states + (static_cast<size_t>(bh) * C + slot) * DV * DK;
        double sqd = 0.0;
#pragma unroll
        for (int i = 0; i < IPW; ++i)
#pragma unroll
            for (int j = 0; j < JPW; ++j) {
                const int row = 16 * (iw + IW * i) + lr, jt = jw + JW * j;
                const float4 x = *reinterpret_cast<const float4 *>(src + static_cast<size_t>(row) * DK + 16 * jt + 4 * lg);
                acc[i][j] = floatx4{x.x, x.y, x.z, x.w};
                sqd += static_cast<double>(x.x) * x.x + static_cast<double>(x.y) * x.y +
                       static_cast<double>(x.z) * x.z + static_cast<double>(x.w) * x.w;
            }
        sqd = wave_sum(sqd);
        if (lane == 0) S.dred[wave] = sqd;
        __syncthreads();
        F = 0.0;
#pragma unroll
        for (int w = 0; w < NW; ++w) F += S.dred[w];
        a = -1;
    }
    int32_t tcnt = 0;
    int64_t tsum = 0;
    // the chunk's K and V rows as 16-byte pieces: lane l holds token l's
    // pieces wave + 8 i (so that the transposed LDS writes of a wave touch 64
    // consecutive tokens of one row of K^T or V^T)
    constexpr int EPV = 16 / sizeof(TIO);
    constexpr int NKP = kChunk * DK / EPV / kSsThreads;
    constexpr int NVP = kChunk * DV / EPV / kSsThreads;
    static_assert(NKP * kSsThreads * EPV == kChunk * DK && NVP * kSsThreads * EPV == kChunk * DV && kChunk == 64,
                  "whole pieces, one token per lane");
    constexpr bool kPrefetch = NKP + NVP <= 8;
    uint4 kp[NKP], vp[NVP];
    auto load_chunk = [&](int c, uint4 (&kq)[NKP], uint4 (&vq)[NVP]) {
        const int cbase = c * kChunk, nv = min(kChunk, T - cbase);
        // (rows past the stream's end load its last row and are zeroed when
        // staged: a select here would wait for the load)
        const size_t row = tok0 + cbase + min(lane, nv - 1);
#pragma unroll
        for (int i = 0; i < NKP; ++i)
            kq[i] = *reinterpret_cast<const uint4 *>(K + row * DK + EPV * (wave + NW * i));
#pragma unroll
        for (int i = 0; i < NVP; ++i)
            vq[i] = *reinterpret_cast<const uint4 *>(V + row * DV + EPV * (wave + NW * i));
    };
    if constexpr (kPrefetch) load_chunk(0, kp, vp);

    // (the waves exchange only LDS data inside the chunk loop: its barriers
    // leave the global loads of the next chunk in flight)
    for (int ch = 0; ch < NCH; ++ch) {
        const int c0 = ch * kChunk;
        const int nvalid = min(kChunk, T - c0);
        lds_barrier();
        // ---- 1. stage the chunk (zero rows past the stream's end): rows into
        // LDS row-major and transposed; where the registers allow, the pieces
        // were loaded during the previous chunk and the next chunk's are
        // loaded now
        float kmax = 0.0f;
        if constexpr (!kPrefetch) load_chunk(ch, kp, vp);
        if (lane >= nvalid) {
#pragma unroll
            for (int i = 0; i < NKP; ++i) kp[i] = make_uint4(0, 0, 0, 0);
#pragma unroll
            for (int i = 0; i < NVP; ++i) vp[i] = make_uint4(0, 0, 0, 0);
        }
#pragma unroll
        for (int i = 0; i < NKP; ++i) {
            const int r = lane, cv = EPV * (wave + NW * i);
            *reinterpret_cast<uint4 *>(&S.kr[r][cv]) = kp[i];
            const TIO *e = reinterpret_cast<const TIO *>(&kp[i]);
#pragma unroll
            for (int j = 0; j < EPV; ++j) {
                S.kt[cv + j][r] = e[j];
                kmax = fmaxf(kmax, fabsf(to_f(e[j])));
            }
        }
#pragma unroll
        for (int i = 0; i < NVP; ++i) {
            const int r = lane, cv = EPV * (wave + NW * i);
            *reinterpret_cast<uint4 *>(&S.vr[r][cv]) = vp[i];
            const TIO *e = reinterpret_cast<const TIO *>(&vp[i]);
#pragma unroll
            for (int j = 0; j < EPV; ++j) S.vt[cv + j][r] = e[j];
        }
        if constexpr (kPrefetch) {
            if (ch + 1 < NCH) load_chunk(ch + 1, kp, vp);
        }
        // scale of S_pre's fp16 halves and of K's
        float smax = 0.0f;
#pragma unroll
        for (int i = 0; i < IPW; ++i)
#pragma unroll
            for (int j = 0; j < JPW; ++j)
#pragma unroll
                for (int r = 0; r < 4; ++r) smax = fmaxf(smax, fabsf(acc[i][j][r]));
        smax = wave_max(smax);
        kmax = wave_max(kmax);
        if (lane == 0) {
            S.red[wave] = smax;
            S.kred[wave] = kmax;
        }
        lds_barrier();
        float smx = 0.0f, kmx = 0.0f;
#pragma unroll
        for (int w = 0; w < NW; ++w) {
            smx = fmaxf(smx, S.red[w]);
            kmx = fmaxf(kmx, S.kred[w]);
        }
        const int es = f16_exponent(smx);
        const int ek = f16_exponent(kmx);
        const bool pre_live = a < c0;   // the current state began before this chunk

        // ---- 2. u_t = v_t^T S_pre k_t (wave w: its d_v tiles, every token)
        if (pre_live) {
            // (with the d_v split every wave reads every token's K: converted
            // to fp16 once, by all threads; with the d_k split each wave
            // converts its own columns in registers below)
            constexpr bool kShared = !kF32 && JW == 1;
            if constexpr (kShared) {
                for (int idx = tid; idx < kChunk * DK / 8; idx += kSsThreads) {
                    const int r = idx / (DK / 8), cv = (idx % (DK / 8)) * 8;
                    const uint4 x = *reinterpret_cast<const uint4 *>(&S.kr[r][cv]);
                    const TIO *e = reinterpret_cast<const TIO *>(&x);
                    f16x8 h;
#pragma unroll
                    for (int j = 0; j < 8; ++j) h[j] = static_cast<_Float16>(ldexpf(to_f(e[j]), -ek));
                    *reinterpret_cast<f16x8 *>(&S.kh[r][cv]) = h;
                }
                lds_barrier();
            }
            // per d_v tile of the wave: Y = S K^T over the wave's d_k tiles
            // (16x16x16 products: the accumulator tile is the first operand as
            // it stands, K's four columns of the tile the second), then the
            // dot product with v_t of the tile's rows
            typedef _Float16 f16x4 __attribute__((ext_vector_type(4)));
            // K of token 16 tt + lr at columns 16 jt + 4 lg + r of the wave's
            // d_k tiles (fp16 halves for fp32 io), the same for every d_v tile
            f16x4 khf[JPW][4], klf[JPW][4];
#pragma unroll
            for (int j = 0; j < JPW; ++j)
#pragma unroll
                for (int tt = 0; tt < 4; ++tt) {
                    const int jt = jw + JW * j;
                    if constexpr (kShared) {
                        khf[j][tt] = *reinterpret_cast<const f16x4 *>(&S.kh[16 * tt + lr][16 * jt + 4 * lg]);
                        klf[j][tt] = khf[j][tt];
                    } else {
                        TIO kv[4];
                        __builtin_memcpy(kv, &S.kr[16 * tt + lr][16 * jt + 4 * lg], sizeof(kv));
#pragma unroll
                        for (int r = 0; r < 4; ++r) {
                            _Float16 h, l;
                            split16(to_f(kv[r]), ek, h, l);
                            khf[j][tt][r] = h; klf[j][tt][r] = l;
                        }
                    }
                }
            float xacc[4] = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
            for (int i = 0; i < IPW; ++i) {
                const int it = iw + IW * i;
                floatx4 Y[4];
#pragma unroll
                for (int tt = 0; tt < 4; ++tt) Y[tt] = floatx4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int j = 0; j < JPW; ++j) {
                    f16x4 sh, sl;
#pragma unroll
                    for (int r = 0; r < 4; ++r) {
                        _Float16 h, l;
                        split16(acc[i][j][r], es, h, l);
                        sh[r] = h; sl[r] = l;
                    }
#pragma unroll
                    for (int tt = 0; tt < 4; ++tt) {
                        Y[tt] = __builtin_amdgcn_mfma_f32_16x16x16f16(sh, khf[j][tt], Y[tt], 0, 0, 0);
                        Y[tt] = __builtin_amdgcn_mfma_f32_16x16x16f16(sl, khf[j][tt], Y[tt], 0, 0, 0);
                        if constexpr (kF32) Y[tt] = __builtin_amdgcn_mfma_f32_16x16x16f16(sh, klf[j][tt], Y[tt], 0, 0, 0);
                    }
                }
                // Y[tt] holds (S K^T) at rows 16 it + 4 lg + r, token 16 tt + lr
#pragma unroll
                for (int tt = 0; tt < 4; ++tt) {
                    TIO vv[4];
                    __builtin_memcpy(vv, &S.vr[16 * tt + lr][16 * it + 4 * lg], sizeof(vv));
#pragma unroll
                    for (int r = 0; r < 4; ++r) xacc[tt] += to_f(vv[r]) * Y[tt][r];
                }
                // (one d_v tile at a time: the next tile's loads are not
                // hoisted over this one, which would keep them all live)
                asm volatile("" ::: "memory");
            }
#pragma unroll
            for (int tt = 0; tt < 4; ++tt) {
                float x = xacc[tt];
                x += __shfl_xor(x, 16);
                x += __shfl_xor(x, 32);
                if (lg == 0) S.upart[wave][16 * tt + lr] = ldexpf(x, es + ek);
            }
        } else {
            S.upart[wave][lane] = 0.0f;
        }
        // ---- 3. Gram products H = (V V^T) o (K K^T), lower-triangle tiles
        for (int tile = wave; tile < 10; tile += NW) {
            int tt = 0, st = tile;
            while (st > tt) { st -= tt + 1; ++tt; }   // tile -> (tt, st), st <= tt
            floatx4 gk = floatx4{0.f, 0.f, 0.f, 0.f}, gv = gk;
#pragma unroll
            for (int ks = 0; ks < DK / 32; ++ks) {
                Frag<TIO> x, y;
                load_frag(x, &S.kr[16 * tt + lr][32 * ks + 8 * lg]);
                load_frag(y, &S.kr[16 * st + lr][32 * ks + 8 * lg]);
                mma32(gk, x, y);
            }
#pragma unroll
            for (int ks = 0; ks < DV / 32; ++ks) {
                Frag<TIO> x, y;
                load_frag(x, &S.vr[16 * tt + lr][32 * ks + 8 * lg]);
                load_frag(y, &S.vr[16 * st + lr][32 * ks + 8 * lg]);
                mma32(gv, x, y);
            }
#pragma unroll
            for (int r = 0; r < 4; ++r) S.H[16 * tt + 4 * lg + r][16 * st + lr] = gk[r] * gv[r];
        }
        lds_barrier();
        // ---- row sums of H in fp64 below the diagonal: NW threads per row t
        // (adjacent lanes of a wave), a segment of 64 / NW columns each
        {
            constexpr int SEG = kChunk / NW;
            const int t = tid / NW, g = tid % NW;
            double tot = 0.0;
#pragma unroll
            for (int j = 0; j < SEG; ++j)
                if (SEG * g + j < t) tot += static_cast<double>(S.H[t][SEG * g + j]);
#pragma unroll
            for (int o = 1; o < NW; o <<= 1) tot += __shfl_xor(tot, o, NW);
            if (g == 0) {
                S.rowsum[t] = tot;
                S.nn[t] = S.H[t][t];
            }
        }
        lds_barrier();
        // ---- 4. the scan (wave 0, lane t = token t).  A pass scores every
        // token from pos on against the current state as it stands (the one
        // that began at a), as if none of them restarted it: x_t from the
        // Gram prefix sums (and u_t while the state began before the chunk),
        // |S|_F^2 as F plus the prefix sum of 2 x_j + |v_j|^2 |k_j|^2.  Then
        // the pass's boundaries are taken in order; the tokens before one join
        // the current state, and at the boundary the greedy merge decides: a
        // new state that stays apart restarts the current state at the
        // boundary token, and the next pass scores from the token after it.
        if (wave == 0) {
            const int t = lane;
            const bool valid = t < nvalid;
            const double nn_t = valid ? static_cast<double>(S.nn[t]) : 0.0;
            const double rs_t = valid ? S.rowsum[t] : 0.0;
            double u_t = 0.0;
            if (valid && a < c0) {
#pragma unroll
                for (int w = 0; w < NW; ++w) u_t += static_cast<double>(S.upart[w][t]);
            }
            float sc_fin = 0.0f;            // the token's final score and boundary flag
            bool bnd_fin = false;
            int pos = 0;
            while (pos < nvalid) {
                if (m == 0) {
                    // an empty cache: the token opens the first state
                    if (t == pos) { sc_fin = 2.0f; bnd_fin = true; }
                    if (lane == 0) { I = fixed_point(2.0f); n = 1; }
                    m = 1;
                    F = readlane_any(nn_t, pos);
                    a = c0 + pos;
                    ++pos;
                    continue;
                }
                const int lo = a > c0 ? static_cast<int>(a - c0) : 0;
                const bool live = valid && t >= pos;
                double x = 0.0, d = 0.0;
                if (live) {
                    if (lo == 0) {
                        x = rs_t;
                    } else {
                        // the state began at chunk token lo: the Gram row from lo
                        for (int s2 = lo; s2 < t; ++s2) x += static_cast<double>(S.H[t][s2]);
                    }
                    if (a < c0) x += u_t;
                    d = 2.0 * x + nn_t;
                }
                const double dsum = wave_incl_scan_dpp(d);
                const double dex = lane_up1(dsum);
                const double Fin = F + dsum;    // |S|_F^2 after token t joins
                const double Fx = F + dex;      // before it
                float sc = 0.0f;
                if (live) {
                    if (nn_t == 0.0 || Fx <= 0.0) {
                        sc = 2.0f;
                    } else {
                        const double c = x / sqrt(nn_t * Fx);
                        sc = static_cast<float>(sqrt(fmax(0.0, 2.0 * D * (1.0 - c))) / (sqD + 1e-6));
                    }
                }
                const bool b_t = live && sc >= tau;
                const int64_t qv = live ? fixed_point(sc) : 0;
                uint64_t bm = __ballot(b_t);
                bool restart = false;
                while (!restart) {
                    if (m == C && merge_rule != DLA_MERGE_DENSITY && bm) {
                        // A full cache under the summed key: a boundary b merges
                        // into the newest pair (the current state and b itself)
                        // when that pair's key, I_last + q_b, is below the key of
                        // the pair before it (q_b < I_{m-2}) and below every older
                        // pair's key (their minimum M, which such merges leave
                        // alone), I_last grown by every token from pos to b.  The
                        // run of such boundaries is taken at once, up to the first
                        // boundary whose merge lands elsewhere.
                        const int64_t Iprev = m >= 2 ? readlane_any(I, m - 2) : INT64_MAX;
                        const int64_t Ilast = readlane_any(I, m - 1);
                        // (the neighbour's value is moved by every lane before the
                        // select: a lane-to-lane move reads nothing from a lane
                        // that a branch has switched off)
                        const int64_t I_nx = lane_down1(I);
                        const int64_t M = wave_min_i64(lane + 2 < m ? I + I_nx : INT64_MAX);
                        const int64_t qa = t >= pos ? qv : int64_t{0};
                        const int64_t Qin = wave_incl_scan_dpp(qa);
                        const bool joins_newest = qa < Iprev && Ilast + Qin < M;
                        const uint64_t stop = bm & __ballot(!joins_newest);
                        const int bs = stop ? __builtin_ctzll(stop) : nvalid;
                        if (bs > pos) {
                            const int64_t q_run = readlane_any(Qin, bs - 1);
                            if (lane == m - 1) { I += q_run; n += bs - pos; }
                            if (t >= pos && t < bs) { sc_fin = sc; bnd_fin = b_t; }
                            bm &= ~low_bits(bs);
                            pos = bs;
                        }
                        if (bs >= nvalid) {
                            F = readlane_any(Fin, nvalid - 1);
                            pos = nvalid;
                            break;
                        }
                        // (boundary bs is taken below, one step of the greedy merge)
                    }
                    const int b = bm ? __builtin_ctzll(bm) : nvalid;
                    // tokens pos .. b - 1 join the current state
                    if (b > pos) {
                        const int64_t q_join = wave_sum((t >= pos && t < b) ? qv : int64_t{0});
                        if (lane == m - 1) { I += q_join; n += b - pos; }
                        if (t >= pos && t < b) { sc_fin = sc; bnd_fin = false; }
                    }
                    if (b >= nvalid) {
                        F = readlane_any(Fin, nvalid - 1);
                        pos = nvalid;
                        break;
                    }
                    // the boundary token b
                    if (t == b) { sc_fin = sc; bnd_fin = true; }
                    const int64_t qb = readlane_any(qv, b);
                    bool extend = false;
                    if (m < C) {
                        if (lane == m) { I = qb; n = 1; }
                        ++m;
                    } else {
                        // the greedy merge of the state set (as the greedy scan
                        // kernel decides it): only whether it joins the newest
                        // pair matters here
                        const int64_t I_nx = lane_down1(I);
                        const int32_t n_nx = lane_down1(n);
                        const bool inside = lane + 1 < m;
                        const int64_t pI = inside ? I_nx : qb;
                        const int32_t pn = inside ? n_nx : 1;
                        int istar;
                        if (merge_rule == DLA_MERGE_DENSITY) {
                            istar = wave_argmin_frac(I + pI, static_cast<int64_t>(n) + pn, lane < m);
                        } else {
                            const int64_t key = lane < m ? I + pI : INT64_MAX;
                            const int64_t kmin = wave_min_i64(key);
                            istar = __ffsll(static_cast<unsigned long long>(__ballot(key == kmin))) - 1;
                        }
                        if (lane == istar) { I += pI; n += pn; }
                        else if (lane > istar && lane < m) { I = pI; n = pn; }
                        extend = istar == m - 1;
                    }
                    pos = b + 1;
                    bm &= bm - 1;
                    if (!extend) {
                        // a new current state, of the boundary token alone
                        F = readlane_any(nn_t, b);
                        a = c0 + b;
                        restart = true;
                    }
                    // (joined: the pass's scores of the later tokens stand)
                }
            }
            if (valid) {
                S.s_c[t] = sc_fin;
                S.f_c[t] = static_cast<uint8_t>(bnd_fin);
            }
            tcnt += __popcll(__ballot(valid && bnd_fin));
            tsum += wave_sum(valid ? fixed_point(sc_fin) : int64_t{0});
            if (lane == 0) S.a_s = a;
            // per-tile boundary count and information sum for the compaction
            const int tile = c0 / kScoreTile;
            const bool tile_end = (c0 + nvalid) % kScoreTile == 0 || ch == NCH - 1;
            if (tile_end) {
                if (lane == 0) {
                    tile_cnt[static_cast<size_t>(bh) * NT + tile] = tcnt;
                    tile_sum[static_cast<size_t>(bh) * NT + tile] = tsum;
                }
                tcnt = 0;
                tsum = 0;
            }
        }
        lds_barrier();
        a = S.a_s;
        // chunk outputs
        if (tid < nvalid) {
            const float sc = S.s_c[tid];
            s_out[tok0 + c0 + tid] = sc;
            qs_out[tok0 + c0 + tid] = fixed_point(sc);
            flag_out[tok0 + c0 + tid] = S.f_c[tid];
        }
        // ---- 5. S_pre of the next chunk: the current state's tokens of this
        // chunk added, after clearing when the state began inside it
        if (ch + 1 < NCH) {
            const int lo = a > c0 ? static_cast<int>(a - c0) : 0;
            if (a >= c0) {
#pragma unroll
                for (int i = 0; i < IPW; ++i)
#pragma unroll
                    for (int j = 0; j < JPW; ++j) acc[i][j] = floatx4{0.f, 0.f, 0.f, 0.f};
            }
#pragma unroll
            for (int ks = 0; ks < kChunk / 32; ++ks) {
                if (32 * ks + 32 <= lo) continue;
#pragma unroll
                for (int j = 0; j < JPW; ++j) {
                    Frag<TIO> x;
                    load_frag(x, &S.kt[16 * (jw + JW * j) + lr][32 * ks + 8 * lg]);
                    mask_frag(x, 32 * ks + 8 * lg, lo, kChunk);
#pragma unroll
                    for (int i = 0; i < IPW; ++i) {
                        Frag<TIO> y;
                        load_frag(y, &S.vt[16 * (iw + IW * i) + lr][32 * ks + 8 * lg]);
                        mma32(acc[i][j], x, y);
                    }
                }
            }
        }
    }
}

}  // namespace

template <typename TIO, int DK, int DV>
static hipError_t ss_launch(const PrefillArgs &a, hipStream_t stream)
{
    const int BH = a.g.B * a.g.H, T = a.T;
    const int NT = (T + kScoreTile - 1) / kScoreTile;
    const size_t smem = sizeof(SsSmem<TIO, DK, DV>);
    static bool attr_set = false;   // idempotent; a race only repeats the same call
    if (!attr_set) {
        hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void *>(&k_state_score<TIO, DK, DV>),
                                           hipFuncAttributeMaxDynamicSharedMemorySize, static_cast<int>(smem));
        if (e != hipSuccess) return e;
        attr_set = true;
    }
    hipLaunchKernelGGL((k_state_score<TIO, DK, DV>), dim3(BH), dim3((64 * ss_waves<TIO, DK, DV>())), smem, stream,
                       static_cast<const TIO *>(a.k), static_cast<const TIO *>(a.v), T, a.tau, a.g.C, a.merge_rule,
                       a.states, a.active, a.g.state_bf16, a.meta, a.g.meta_stride, a.ws.s, a.ws.qs, a.ws.flag,
                       a.ws.tile_cnt, a.ws.tile_sum, NT);
    return hipGetLastError();
}

template <typename TIO, int DK>
static hipError_t ss_dv(const PrefillArgs &a, hipStream_t stream)
{
    switch (a.g.dv) {
    case 64: return ss_launch<TIO, DK, 64>(a, stream);
    case 128: return ss_launch<TIO, DK, 128>(a, stream);
    case 256:
        // (d_k = d_v = 256: the current state alone would take every register of the block)
        if constexpr (DK < 256 && sizeof(SsSmem<TIO, DK, 256>) <= 160 * 1024) return ss_launch<TIO, DK, 256>(a, stream);
        return hipErrorInvalidValue;
    default: return hipErrorInvalidValue;
    }
}

hipError_t launch_state_score(const PrefillArgs &a, hipStream_t stream)
{
    if (a.io_bf16) {
        switch (a.g.dk) {
        case 64: return ss_dv<__bf16, 64>(a, stream);
        case 128: return ss_dv<__bf16, 128>(a, stream);
        case 256: return ss_dv<__bf16, 256>(a, stream);
        default: return hipErrorInvalidValue;
        }
    }
    switch (a.g.dk) {
    case 64: return ss_dv<float, 64>(a, stream);
    case 128: return ss_dv<float, 128>(a, stream);
    default: return hipErrorInvalidValue;
    }
}

size_t state_score_smem_bytes(int io_bf16, int dk, int dv)
{
    auto pick = [&](auto tio) -> size_t {
        typedef decltype(tio) TIO;
        if (dk == 64) return dv == 64 ? sizeof(SsSmem<TIO, 64, 64>) : dv == 128 ? sizeof(SsSmem<TIO, 64, 128>)
                                                                                 : sizeof(SsSmem<TIO, 64, 256>);
        if (dk == 128) return dv == 64 ? sizeof(SsSmem<TIO, 128, 64>) : dv == 128 ? sizeof(SsSmem<TIO, 128, 128>)
                                                                                   : sizeof(SsSmem<TIO, 128, 256>);
        return dv == 64 ? sizeof(SsSmem<TIO, 256, 64>) : dv == 128 ? sizeof(SsSmem<TIO, 256, 128>)
                                                                    : sizeof(SsSmem<TIO, 256, 256>);
    };
    return io_bf16 ? pick(__bf16{}) : pick(float{});
}

}  // namespace dla
