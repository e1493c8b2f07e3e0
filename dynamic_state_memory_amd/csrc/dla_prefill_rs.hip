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
//                 the state, in MFMA-fragment order -- the query as fp16
//                 scaled by a power of two, lam transposed, K transposed, and
//                 the intra-chunk slot-weighted causal product
//                 P = (Q K^T) o W, W[t][s] = lam_t[#live chunk starts > s].
//   k_prefill_rs  one block (4 waves) per (stream, d_v slice of DVT columns)
//                 sweeping the stream's chunks in order.  It keeps every
//                 closed state (all but the most recent) of the slice as fp16
//                 MFMA operands in the registers of the wave that owns its
//                 physical slot (slot p -> wave p % 4, register set p / 4),
//                 normalised by a power of two kept in LDS, and the most
//                 recent ("active") state as fp32 MFMA accumulators (d_k rows
//                 32w..32w+31 in wave w) plus an fp16 operand copy.  A chunk
//                 without events touches no state memory: read, P V, then
//                 V_c^T K_c accumulated into the active state's registers.  A
//                 chunk with events flushes the active state to the fp32 cache,
//                 runs the general update there (merges, per-group V_g^T K_g)
//                 and reloads the register copies of the states it changed.
//
// Operand order of the read: the reduction index d_k of a 32-wide step is
// split over lane groups g = lane / 16 as {4g..4g+3, 16+4g..16+4g+3}, the
// order in which a 16x16 accumulator pair holds rows; the query fragments use
// the same order, so the active state goes from accumulator to operand in place.
#include <hip/hip_runtime.h>
#include <stdint.h>

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

// ------------------------------------------------------------ chunk pre-pass

template <int DK>
__global__ __launch_bounds__(256) void k_chunk_prep(
    const __bf16 *__restrict__ Q, const __bf16 *__restrict__ K, const __bf16 *__restrict__ LAM, int T, int C,
    const int2 *__restrict__ events, const int32_t *__restrict__ chunk_ev, _Float16 *__restrict__ q16f,
    int32_t *__restrict__ qexp_out, float *__restrict__ lamT, __bf16 *__restrict__ pwf, __bf16 *__restrict__ ktf)
{
    constexpr int KS = DK / 32;
    __shared__ __align__(16) __bf16 q[kChunk][DK + 8];
    __shared__ __align__(16) __bf16 k[kChunk][DK + 8];
    __shared__ __align__(16) __bf16 pw[kChunk][kChunk + 8];
    __shared__ float lam[kChunk][kPrepCmax + 1];
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
    const int lr = lane & 15, lg = lane >> 4;

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
        lam[r][c] = (c < C && r < nvalid) ? static_cast<float>(LAM[(tok0 + c0 + r) * C + c]) : 0.0f;
    }
    const int e0 = chunk_ev[static_cast<size_t>(bh) * (NCH + 1) + ch];
    const int nev = chunk_ev[static_cast<size_t>(bh) * (NCH + 1) + ch + 1] - e0;
    if (tid < nev) evs[tid] = events[tok0 + e0 + tid];
    qmax = wave_max(qmax);
    if (lane == 0) red[wave] = qmax;
    __syncthreads();
    const int qexp = f16_exponent(fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3])));
    if (tid == 0) qexp_out[cb] = qexp;
    if (tid < kChunk) {
        // bit p: the state opened at chunk position p is live after token tid
        uint64_t m = 0;
        for (int e = 0; e < nev; ++e) {
            const int2 ev = evs[e];
            const int pos = ev.x - c0;
            if (tid >= pos) {
                m |= 1ull << pos;
                if (ev.y >= 64) m &= ~(1ull << (ev.y - 64));
            }
        }
        nm[tid] = m;
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
        reinterpret_cast<f16x8 *>(q16f)[cb * 4 * KS * 64 + f] = h;
    }
    // lam, slot-major
#pragma unroll
    for (int j = 0; j < kPrepCmax / 4; ++j) {
        const int idx = tid + 256 * j;
        lamT[cb * kPrepCmax * kChunk + idx] = lam[idx & (kChunk - 1)][idx / kChunk];
    }
    // K^T fragments: d_k rows of a 16-tile, 8 consecutive tokens per lane
#pragma unroll
    for (int j = 0; j < DK / 32; ++j) {
        const int f = tid + 256 * j;                   // (tile, kk, lane)
        const int l = f & 63, kk = (f >> 6) & 1, tile = f >> 7;
        const int dk = 16 * tile + (l & 15), t0 = 32 * kk + 8 * (l >> 4);
        bf16x8 h;
#pragma unroll
        for (int e = 0; e < 8; ++e) h[e] = k[t0 + e][dk];
        reinterpret_cast<bf16x8 *>(ktf)[cb * (DK / 16) * 2 * 64 + f] = h;
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
                if (s <= t) val = A[r] * lam[t][__popcll(shr64(nm[t], s + 1))];
                pw[t][s] = static_cast<__bf16>(val);
            }
        }
    }
    __syncthreads();
#pragma unroll
    for (int j = 0; j < 2; ++j) {
        const int f = tid + 256 * j;                   // (mt, ks2, lane)
        const int l = f & 63, ks2 = (f >> 6) & 1, mt = f >> 7;
        reinterpret_cast<bf16x8 *>(pwf)[cb * 8 * 64 + f] =
            *reinterpret_cast<const bf16x8 *>(&pw[16 * mt + (l & 15)][32 * ks2 + 8 * (l >> 4)]);
    }
}

// ------------------------------------------------------------ the sweep

template <int DK, int DVT, int CMAX>
struct RsSmem {
    _Float16 qf[kChunk / 16][DK / 32][64][8];   // query fragments of the chunk
    float lamT[CMAX][kChunk];                    // lam of the chunk, slot-major
    __bf16 pwf[kChunk / 16][2][64][8];           // fragments of (Q K^T) o W
    __bf16 ktf[DK / 16][2][64][8];               // fragments of K^T
    __bf16 vt[DVT][kChunk + 8];                  // V slice, transposed
    float W[CMAX][kChunk];      // closed-state read weights, by physical slot
    float wact[kChunk];         // active-state read weight
    float ored[4][kChunk][DVT];
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
    int32_t changed[kMaxC + kChunk + 2];
    int32_t shexp[kMaxC];
    int32_t inv[kMaxC];         // chronological index of the state in each physical slot
    int2 evs[kChunk];           // the chunk's events (at most one per token)
    float red[4];
    int32_t n_merge, n_grp, n_changed, m_new, act_new;
};

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

// One chunk's operands in registers, loaded a chunk ahead of their use.
template <int DK, int DVT, int CMAX>
struct ChunkRegs {
    static constexpr int NQ = kChunk * DK * 2 / 16 / 256;     // 16-byte pieces per thread
    static constexpr int NL = (CMAX * kChunk * 4 / 16 + 255) / 256;
    static constexpr int NP = kChunk * kChunk * 2 / 16 / 256;
    static constexpr int NK = kChunk * DK * 2 / 16 / 256;
    u32x4 q[NQ], l[NL], p[NP], k[NK];
    u32x4 v;                    // 64 rows x DVT bf16 (DVT <= 32)
    int qexp, e0, e1;
};

template <int DK, int DVT, int CMAX>
__device__ __forceinline__ void load_chunk(ChunkRegs<DK, DVT, CMAX> &R, const __bf16 *V, const _Float16 *q16f,
                                           const int32_t *qexp, const float *lamT, const __bf16 *pwf,
                                           const __bf16 *ktf, const int32_t *chunk_ev, int bh, int NCH,
                                           int T, int DV, int dv0, int ch, int tid)
{
    typedef ChunkRegs<DK, DVT, CMAX> R_t;
    const size_t cb = static_cast<size_t>(bh) * NCH + ch;
    const u32x4 *qs = reinterpret_cast<const u32x4 *>(q16f) + cb * (kChunk * DK * 2 / 16);
    const u32x4 *ls = reinterpret_cast<const u32x4 *>(lamT) + cb * (kPrepCmax * kChunk * 4 / 16);
    const u32x4 *ps = reinterpret_cast<const u32x4 *>(pwf) + cb * (kChunk * kChunk * 2 / 16);
    const u32x4 *ks = reinterpret_cast<const u32x4 *>(ktf) + cb * (kChunk * DK * 2 / 16);
#pragma unroll
    for (int j = 0; j < R_t::NQ; ++j) R.q[j] = qs[tid + 256 * j];
#pragma unroll
    for (int j = 0; j < R_t::NL; ++j) {
        const int idx = tid + 256 * j;
        R.l[j] = idx < CMAX * kChunk / 4 ? ls[idx] : u32x4{0u, 0u, 0u, 0u};
    }
#pragma unroll
    for (int j = 0; j < R_t::NP; ++j) R.p[j] = ps[tid + 256 * j];
#pragma unroll
    for (int j = 0; j < R_t::NK; ++j) R.k[j] = ks[tid + 256 * j];
    const int c0 = ch * kChunk;
    const int nvalid = min(kChunk, T - c0);
    const int r = tid & (kChunk - 1), cv = (tid / kChunk) * 8;
    R.v = u32x4{0u, 0u, 0u, 0u};
    if (tid < kChunk * DVT / 8 && r < nvalid)
        R.v = *reinterpret_cast<const u32x4 *>(V + (static_cast<size_t>(bh) * T + c0 + r) * DV + dv0 + cv);
    R.qexp = qexp[cb];
    R.e0 = chunk_ev[static_cast<size_t>(bh) * (NCH + 1) + ch];
    R.e1 = chunk_ev[static_cast<size_t>(bh) * (NCH + 1) + ch + 1];
}

template <int DK, int DVT, int SPW>
__global__ __launch_bounds__(256, 1) void k_prefill_rs(
    const __bf16 *__restrict__ V, __bf16 *__restrict__ O, int T, int C, int DV, int nblk_dv,
    float *__restrict__ states, _Float16 *__restrict__ shadow, const int2 *__restrict__ events,
    const int32_t *__restrict__ chunk_ev, const _Float16 *__restrict__ q16f, const int32_t *__restrict__ qexp_g,
    const float *__restrict__ lamT_g, const __bf16 *__restrict__ pwf_g, const __bf16 *__restrict__ ktf_g,
    uint8_t *__restrict__ meta_base, size_t meta_stride, int32_t *__restrict__ m_t_out)
{
    constexpr int KS = DK / 32;
    constexpr int NTV = DVT / 16;
    constexpr int MT = kChunk / 16;
    constexpr int CMAX = 4 * SPW;
    static_assert(KS <= 4, "the active state gives each wave at most one 32-row block of d_k");
    typedef RsSmem<DK, DVT, CMAX> Smem;
    typedef ChunkRegs<DK, DVT, CMAX> Regs;
    extern __shared__ __align__(16) unsigned char smem_raw[];
    Smem &S = *reinterpret_cast<Smem *>(smem_raw);

    const int nblk = gridDim.x;
    int lin = blockIdx.x;
    if ((nblk & 7) == 0) lin = (blockIdx.x & 7) * (nblk >> 3) + (blockIdx.x >> 3);
    const int bh = lin / nblk_dv;
    const int dv0 = (lin % nblk_dv) * DVT;

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int lr = lane & 15, lg = lane >> 4;
    const int NCH = (T + kChunk - 1) / kChunk;
    const size_t tok0 = static_cast<size_t>(bh) * T;
    const size_t slot_stride = static_cast<size_t>(DV) * DK;
    float *st_base = states + static_cast<size_t>(bh) * C * DV * DK + static_cast<size_t>(dv0) * DK;
    _Float16 *sh_base = shadow + static_cast<size_t>(bh) * C * DV * DK + static_cast<size_t>(dv0) * DK;

    Frag<_Float16> stk[SPW][KS][NTV];
    floatx4 am[NTV][2];
    Frag<_Float16> af[NTV];
#pragma unroll
    for (int r = 0; r < SPW; ++r)
#pragma unroll
        for (int ks = 0; ks < KS; ++ks)
#pragma unroll
            for (int nt = 0; nt < NTV; ++nt) zero_frag(stk[r][ks][nt]);
#pragma unroll
    for (int nt = 0; nt < NTV; ++nt) {
        am[nt][0] = floatx4{0.f, 0.f, 0.f, 0.f};
        am[nt][1] = floatx4{0.f, 0.f, 0.f, 0.f};
        zero_frag(af[nt]);
    }
    int ea = 0;           // exponent of this wave's active-state operand
    int m0 = 0, act = -1; // live states and the active state's slot (uniform)
    uint32_t closed = 0;  // physical slots of the closed states (uniform)
    if (tid < kMaxC) { S.order[tid] = tid; S.shexp[tid] = 0; }

    Regs pre;
    load_chunk(pre, V, q16f, qexp_g, lamT_g, pwf_g, ktf_g, chunk_ev, bh, NCH, T, DV, dv0, 0, tid);
    floatx4 Oprev[NTV];           // the previous chunk's outputs, stored one iteration late
    int prev_c0 = 0, prev_nvalid = 0;
    for (int ch = 0; ch < NCH; ++ch) {
        const int c0 = ch * kChunk;
        const int nvalid = min(kChunk, T - c0);
        const int e0 = pre.e0, nev = pre.e1 - pre.e0;
        const bool has_ev = nev > 0;
        const int qexp = pre.qexp;
        lds_barrier();
        // ---- the chunk's operands into LDS, the next chunk's into registers
#pragma unroll
        for (int j = 0; j < Regs::NQ; ++j) reinterpret_cast<u32x4 *>(&S.qf[0][0][0][0])[tid + 256 * j] = pre.q[j];
#pragma unroll
        for (int j = 0; j < Regs::NL; ++j) {
            const int idx = tid + 256 * j;
            if (idx < CMAX * kChunk / 4) reinterpret_cast<u32x4 *>(&S.lamT[0][0])[idx] = pre.l[j];
        }
#pragma unroll
        for (int j = 0; j < Regs::NP; ++j) reinterpret_cast<u32x4 *>(&S.pwf[0][0][0][0])[tid + 256 * j] = pre.p[j];
#pragma unroll
        for (int j = 0; j < Regs::NK; ++j) reinterpret_cast<u32x4 *>(&S.ktf[0][0][0][0])[tid + 256 * j] = pre.k[j];
        if (tid < kChunk * DVT / 8) {
            const int r = tid & (kChunk - 1), cv = (tid / kChunk) * 8;
            const __bf16 *ve = reinterpret_cast<const __bf16 *>(&pre.v);
#pragma unroll
            for (int e = 0; e < 8; ++e) S.vt[cv + e][r] = ve[e];
        }
        if (tid < nev) S.evs[tid] = events[tok0 + e0 + tid];
        if (ch + 1 < NCH)
            load_chunk(pre, V, q16f, qexp_g, lamT_g, pwf_g, ktf_g, chunk_ev, bh, NCH, T, DV, dv0, ch + 1, tid);
        if (ch > 0) {
#pragma unroll
            for (int nt = 0; nt < NTV; ++nt)
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const int t = 16 * wave + 4 * lg + r;
                    if (t < prev_nvalid)
                        O[(tok0 + prev_c0 + t) * DV + dv0 + 16 * nt + lr] = static_cast<__bf16>(Oprev[nt][r]);
                }
        }
        lds_barrier();
        if (has_ev) {
            // token masks: bit i of om_t = state i of the chunk start live after
            // token t, bit p of nm_t = state opened at chunk position p live
            if (tid < kChunk) {
                uint64_t om = low_bits(m0), nm = 0;
                for (int e = 0; e < nev; ++e) {
                    const int2 ev = S.evs[e];
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
            lds_barrier();
        } else if (m_t_out && dv0 == 0 && tid < nvalid) {
            m_t_out[tok0 + c0 + tid] = m0;
        }
        // read weights of every physical slot (0 unless it holds a closed
        // state) and of the active state, with the operand exponents folded in;
        // without events a closed state's slot is j = m0 - 1 - i for all tokens
#pragma unroll
        for (int j = 0; j < CMAX * kChunk / 256; ++j) {
            const int idx = tid + 256 * j;
            const int p = idx / kChunk, t = idx & (kChunk - 1);
            float w = 0.0f;
            if ((closed >> p) & 1u) {
                const int i = S.inv[p];
                const int slot = has_ev ? __popcll(shr64(S.om[t], i + 1)) + __popcll(S.nm[t]) : m0 - 1 - i;
                w = ldexpf(S.lamT[slot][t], S.shexp[p] + qexp);
            }
            S.W[p][t] = w;
        }
        if (m0 > 0 && tid < kChunk)
            S.wact[tid] = ldexpf(S.lamT[has_ev ? __popcll(S.nm[tid]) : 0][tid], qexp);
        lds_barrier();

        // ---- inter-chunk read: closed states from registers, then the active state
        floatx4 Oi[MT][NTV];
#pragma unroll
        for (int mt = 0; mt < MT; ++mt)
#pragma unroll
            for (int nt = 0; nt < NTV; ++nt) Oi[mt][nt] = floatx4{0.f, 0.f, 0.f, 0.f};
        {
            Frag<_Float16> qf[MT][KS];
#pragma unroll
            for (int mt = 0; mt < MT; ++mt)
#pragma unroll
                for (int ks = 0; ks < KS; ++ks) load_frag(qf[mt][ks], S.qf[mt][ks][lane]);
            // every slot of the wave, live or not: a slot without a closed
            // state has weight 0 and finite (zero or stale) operands
#pragma unroll
            for (int r = 0; r < SPW; ++r) {
                const int p = 4 * r + wave;
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
                        for (int nt = 0; nt < NTV; ++nt) mma32(P[mt][nt], qf[mt][ks], stk[r][ks][nt]);
#pragma unroll
                for (int mt = 0; mt < MT; ++mt) {
                    const float4 w = *reinterpret_cast<const float4 *>(&S.W[p][16 * mt + 4 * lg]);
#pragma unroll
                    for (int nt = 0; nt < NTV; ++nt) {
                        Oi[mt][nt][0] += w.x * P[mt][nt][0];
                        Oi[mt][nt][1] += w.y * P[mt][nt][1];
                        Oi[mt][nt][2] += w.z * P[mt][nt][2];
                        Oi[mt][nt][3] += w.w * P[mt][nt][3];
                    }
                }
            }
            if (act >= 0 && wave < KS) {
                // d_k rows 32w..32w+31 of the active state live in wave w
                const float sc = ldexpf(1.0f, ea);
                const float *wrow = &S.wact[0];
#pragma unroll
                for (int mt = 0; mt < MT; ++mt) {
                    Frag<_Float16> qa;
                    load_frag(qa, S.qf[mt][wave][lane]);
                    const float4 w = *reinterpret_cast<const float4 *>(wrow + 16 * mt + 4 * lg);
#pragma unroll
                    for (int nt = 0; nt < NTV; ++nt) {
                        floatx4 P = floatx4{0.f, 0.f, 0.f, 0.f};
                        mma32(P, qa, af[nt]);
                        Oi[mt][nt][0] += (sc * w.x) * P[0];
                        Oi[mt][nt][1] += (sc * w.y) * P[1];
                        Oi[mt][nt][2] += (sc * w.z) * P[2];
                        Oi[mt][nt][3] += (sc * w.w) * P[3];
                    }
                }
            }
        }
#pragma unroll
        for (int mt = 0; mt < MT; ++mt)
#pragma unroll
            for (int nt = 0; nt < NTV; ++nt)
#pragma unroll
                for (int r = 0; r < 4; ++r) S.ored[wave][16 * mt + 4 * lg + r][16 * nt + lr] = Oi[mt][nt][r];
        lds_barrier();
        // ---- reduce the waves' partial reads, add P V (wave w: rows 16w..16w+15)
        {
            const int w = wave;
#pragma unroll
            for (int nt = 0; nt < NTV; ++nt)
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const int t = 16 * w + 4 * lg + r, col = 16 * nt + lr;
                    Oprev[nt][r] = S.ored[0][t][col] + S.ored[1][t][col] + S.ored[2][t][col] + S.ored[3][t][col];
                }
#pragma unroll
            for (int ks = 0; ks < kChunk / 32; ++ks) {
                if (32 * ks <= 16 * w + 15) {
                    Frag<__bf16> a;
                    load_frag(a, S.pwf[w][ks][lane]);
#pragma unroll
                    for (int nt = 0; nt < NTV; ++nt) {
                        Frag<__bf16> b;
                        load_frag(b, &S.vt[16 * nt + lr][32 * ks + 8 * lg]);
                        mma32(Oprev[nt], a, b);
                    }
                }
            }
            prev_c0 = c0;
            prev_nvalid = nvalid;
        }

        // ---- chunk-end update
        if (!has_ev) {
            // every token of the chunk joins the active state: V_c^T K_c into its registers
            if (wave < KS) {
#pragma unroll
                for (int kk = 0; kk < kChunk / 32; ++kk)
#pragma unroll
                    for (int h = 0; h < 2; ++h) {
                        Frag<__bf16> a;
                        load_frag(a, S.ktf[2 * wave + h][kk][lane]);
#pragma unroll
                        for (int nt = 0; nt < NTV; ++nt) {
                            Frag<__bf16> b;
                            load_frag(b, &S.vt[16 * nt + lr][32 * kk + 8 * lg]);
                            mma32(am[nt][h], a, b);
                        }
                    }
                ea = refresh_active<NTV>(am, af);
            }
            continue;
        }

        // chunk with events: general update in the fp32 cache
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
                } else if (tgt >= 0) {
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
            const int an = mnew > 0 ? S.new_order[mnew - 1] : -1;
            // the previous active state, if it is now closed, needs an operand copy
            if (act >= 0 && m0 > 0 && ((oa >> (m0 - 1)) & 1ull) && act != an) S.changed[nch++] = act;
            S.n_merge = nmg;
            S.n_grp = ng;
            S.n_changed = nch;
            S.m_new = mnew;
            S.act_new = an;
        }
        // flush the active state's accumulators to its fp32 state in the cache
        if (act >= 0 && wave < KS) {
            float *dst = st_base + act * slot_stride;
#pragma unroll
            for (int nt = 0; nt < NTV; ++nt)
#pragma unroll
                for (int h = 0; h < 2; ++h)
                    *reinterpret_cast<float4 *>(dst + (16 * nt + lr) * DK + 32 * wave + 16 * h + 4 * lg) =
                        make_float4(am[nt][h][0], am[nt][h][1], am[nt][h][2], am[nt][h][3]);
        }
        __syncthreads();
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
                        Frag<__bf16> a, b;
                        load_frag(a, &S.vt[16 * mt + lr][base]);
                        mask_frag(a, base, lo, hi);
                        load_frag(b, S.ktf[nt][ks][lane]);
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
        const int an = S.act_new;
        // normalised fp16 copies of the changed closed states
        for (int c = 0; c < S.n_changed; ++c) {
            const int slot = S.changed[c];
            if (slot == an) continue;
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
            _Float16 *dst = sh_base + slot * slot_stride;
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
        __syncthreads();
        // owner waves reload the register copies of the changed closed states
        for (int c = 0; c < S.n_changed; ++c) {
            const int slot = S.changed[c];
            if (slot == an || (slot & 3) != wave) continue;
            const _Float16 *src = sh_base + slot * slot_stride;
#pragma unroll
            for (int r = 0; r < SPW; ++r) {
                if ((slot >> 2) == r) {
#pragma unroll
                    for (int ks = 0; ks < KS; ++ks)
#pragma unroll
                        for (int nt = 0; nt < NTV; ++nt)
                            perm_frag_f16(stk[r][ks][nt], src + (16 * nt + lr) * DK, 32 * ks + 4 * lg);
                }
            }
        }
        // the new active state into the accumulators
        if (an >= 0 && wave < KS) {
            const float *src = st_base + an * slot_stride;
#pragma unroll
            for (int nt = 0; nt < NTV; ++nt)
#pragma unroll
                for (int h = 0; h < 2; ++h) {
                    const float4 a = *reinterpret_cast<const float4 *>(src + (16 * nt + lr) * DK + 32 * wave +
                                                                      16 * h + 4 * lg);
                    am[nt][h] = floatx4{a.x, a.y, a.z, a.w};
                }
            ea = refresh_active<NTV>(am, af);
        }
        const int mnew = S.m_new;
        uint32_t cl = 0;
        for (int i = 0; i + 1 < mnew; ++i) cl |= 1u << S.new_order[i];
        __syncthreads();
        if (tid < kMaxC) S.order[tid] = tid < mnew ? S.new_order[tid] : 0;
        if (tid < mnew) S.inv[S.new_order[tid]] = tid;
        m0 = mnew;
        act = an;
        closed = cl;
    }
#pragma unroll
    for (int nt = 0; nt < NTV; ++nt)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int t = 16 * wave + 4 * lg + r;
            if (t < prev_nvalid)
                O[(tok0 + prev_c0 + t) * DV + dv0 + 16 * nt + lr] = static_cast<__bf16>(Oprev[nt][r]);
        }
    // the active state's accumulators are the last state of the final cache
    if (act >= 0 && wave < KS) {
        float *dst = st_base + act * slot_stride;
#pragma unroll
        for (int nt = 0; nt < NTV; ++nt)
#pragma unroll
            for (int h = 0; h < 2; ++h)
                *reinterpret_cast<float4 *>(dst + (16 * nt + lr) * DK + 32 * wave + 16 * h + 4 * lg) =
                    make_float4(am[nt][h][0], am[nt][h][1], am[nt][h][2], am[nt][h][3]);
    }
    __syncthreads();
    if (dv0 == 0 && tid < kMaxC) {
        uint8_t *order = meta_base + static_cast<size_t>(bh) * meta_stride + kOffOrder;
        order[tid] = static_cast<uint8_t>(tid < m0 ? S.order[tid] : 0xFF);
    }
}

template <int DK, int DVT, int SPW>
static hipError_t launch_rs(const PrefillArgs &a, hipStream_t stream)
{
    const int BH = a.g.B * a.g.H;
    const int nblk_dv = a.g.dv / DVT;
    const size_t smem = sizeof(RsSmem<DK, DVT, 4 * SPW>);
    static bool attr_set = false;
    if (!attr_set) {
        hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void *>(&k_prefill_rs<DK, DVT, SPW>),
                                           hipFuncAttributeMaxDynamicSharedMemorySize, static_cast<int>(smem));
        if (e != hipSuccess) return e;
        attr_set = true;
    }
    const int NCH = (a.T + kChunk - 1) / kChunk;
    hipLaunchKernelGGL((k_chunk_prep<DK>), dim3(NCH, BH), dim3(256), 0, stream,
                       static_cast<const __bf16 *>(a.q), static_cast<const __bf16 *>(a.k),
                       static_cast<const __bf16 *>(a.lam), a.T, a.g.C, a.ws.events, a.ws.chunk_ev,
                       static_cast<_Float16 *>(a.ws.q16f), a.ws.qexp, a.ws.lamT,
                       static_cast<__bf16 *>(a.ws.pwf), static_cast<__bf16 *>(a.ws.ktf));
    hipError_t e0 = hipGetLastError();
    if (e0 != hipSuccess) return e0;
    if (a.ev_before) {
        hipError_t e = hipEventRecord(a.ev_before, stream);
        if (e != hipSuccess) return e;
    }
    hipLaunchKernelGGL((k_prefill_rs<DK, DVT, SPW>), dim3(BH * nblk_dv), dim3(256), smem, stream,
                       static_cast<const __bf16 *>(a.v), static_cast<__bf16 *>(a.o), a.T, a.g.C, a.g.dv,
                       nblk_dv, a.states, static_cast<_Float16 *>(a.ws.shadow), a.ws.events, a.ws.chunk_ev,
                       static_cast<const _Float16 *>(a.ws.q16f), a.ws.qexp, a.ws.lamT,
                       static_cast<const __bf16 *>(a.ws.pwf), static_cast<const __bf16 *>(a.ws.ktf), a.meta,
                       a.g.meta_stride, a.sched.m_t);
    hipError_t e = hipGetLastError();
    if (e == hipSuccess && a.ev_after) e = hipEventRecord(a.ev_after, stream);
    return e;
}

// Register budget: with d_k = 128 and more than 16 states the stack of a
// 32-column slice does not fit beside the working set (the compiler spills),
// so that case always uses 16-column slices.
int prefill_rs_dvt(int dk, int C, int dvt_wanted) { return (dk == 128 && C > 16) ? 16 : dvt_wanted; }

hipError_t launch_prefill_rs(const PrefillArgs &a, hipStream_t stream)
{
    const int C = a.g.C;
    if (a.g.dk == 128) {
        if (C > 16) return launch_rs<128, 16, 8>(a, stream);
        if (a.dvt == 32) return C <= 8 ? launch_rs<128, 32, 2>(a, stream) : launch_rs<128, 32, 4>(a, stream);
        return C <= 8 ? launch_rs<128, 16, 2>(a, stream) : launch_rs<128, 16, 4>(a, stream);
    }
    if (a.dvt == 32)
        return C <= 8 ? launch_rs<64, 32, 2>(a, stream) : C <= 16 ? launch_rs<64, 32, 4>(a, stream)
                                                                 : launch_rs<64, 32, 8>(a, stream);
    return C <= 8 ? launch_rs<64, 16, 2>(a, stream) : C <= 16 ? launch_rs<64, 16, 4>(a, stream)
                                                               : launch_rs<64, 16, 8>(a, stream);
}

size_t prefill_rs_smem_bytes(int dk, int dvt, int C)
{
    const int cmax = C <= 8 ? 8 : (C <= 16 ? 16 : 32);
    size_t b = 0;
    if (dk == 128) {
        if (dvt == 32) b = cmax == 8 ? sizeof(RsSmem<128, 32, 8>) : cmax == 16 ? sizeof(RsSmem<128, 32, 16>) : sizeof(RsSmem<128, 32, 32>);
        else b = cmax == 8 ? sizeof(RsSmem<128, 16, 8>) : cmax == 16 ? sizeof(RsSmem<128, 16, 16>) : sizeof(RsSmem<128, 16, 32>);
    } else {
        if (dvt == 32) b = cmax == 8 ? sizeof(RsSmem<64, 32, 8>) : cmax == 16 ? sizeof(RsSmem<64, 32, 16>) : sizeof(RsSmem<64, 32, 32>);
        else b = cmax == 8 ? sizeof(RsSmem<64, 16, 8>) : cmax == 16 ? sizeof(RsSmem<64, 16, 16>) : sizeof(RsSmem<64, 16, 32>);
    }
    return b;
}

}  // namespace dla
