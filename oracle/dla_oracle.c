/*
 * dla_oracle.c -- plain CPU oracle of the Dynamic Linear Attention (DLA)
 * layer forward pass.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the tests, the smoke check and the CPU
 * baseline leg of the benchmark load this library.  It shares no code,
 * header, table or helper with the GPU library, and the GPU library never
 * calls it.
 *
 * What it computes, one stream (batch, head) at a time, token by token, in
 * the order the method states its steps.  Sources: the reading notes
 * "Dynamic Linear Attention | Chlience Paper Archive", section 5.1 (per-token
 * state, merge-into-current / open-new rule), section 5.2 (capacity-bounded
 * cache, greedy adjacent merge), section 5.3 (bounded read) and section 1
 * (single-state linear attention, whose state already holds token t when o_t
 * is read); and the ai-feeds.com summary "Dynamic Linear Attention", section
 * "方法" (method): the information signal may be the feature change between
 * tokens, two consecutive low-information tokens are merged, and a merged
 * state keeps the original timestamp.
 *
 * Fixed choices taken where the pages leave the step open:
 *   - token information s_t = 1 - cos(k_t, k_{t-1}); s = 1 when there is no
 *     previous key or a key has zero norm; dot product and norms are summed
 *     in double precision and s is rounded once to float;
 *   - token t opens a new state unless s_t < tau and s_{t-1} < tau (float
 *     compares; s == tau counts as high information); an empty cache always
 *     opens a state;
 *   - information sums are kept exactly, as int64 multiples of 2^-32 (each
 *     token adds llrint(s * 2^32));
 *   - right after a state is appended, if the cache holds C+1 states, the
 *     adjacent pair (i, i+1) with the smallest summed information
 *     I_i + I_{i+1} is merged (the earliest pair on ties); the merged state
 *     keeps the start of state i.  With merge_rule = 1 the pair is instead
 *     the one of lowest information density (I_i + I_{i+1}) / (n_i + n_{i+1}),
 *     n the token counts: the criterion written in section 5.2 of the
 *     reading notes; fractions are compared exactly by cross-multiplication,
 *     the earliest pair again winning ties;
 *   - the read uses the cache after the update and any merge:
 *     o_t = sum_j lam[t][j] * S_(m-1-j) q_t, slot j = j-th most recent state;
 *   - the per-token state is v_t k_t^T (S is d_v x d_k, o = S q).
 * States, merges and outputs are double precision.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

typedef struct {
    int32_t BH, T, dk, dv, C;
    float tau;
    const float *q, *k, *v, *lam;   /* [BH][T][dk] [BH][T][dk] [BH][T][dv] [BH][T][C] */
    /* starting cache; init_m == NULL means every stream starts empty */
    const int32_t *init_m;          /* [BH] */
    const double *init_S;           /* [BH][C][dv][dk], oldest state first */
    const int64_t *init_I;          /* [BH][C] */
    const int32_t *init_n;          /* [BH][C] */
    const int64_t *init_start;      /* [BH][C] */
    const int32_t *init_has_prev;   /* [BH] */
    const float *init_s_prev;       /* [BH] */
    const float *init_k_prev;       /* [BH][dk] */
    const int64_t *init_t_seen;     /* [BH] */
    const uint8_t *want_o;          /* [BH][T]; NULL = every output */
    /* outputs, each may be NULL */
    double *o;                      /* [BH][T][dv] */
    float *s_out;                   /* [BH][T] token information */
    uint8_t *b_out;                 /* [BH][T] 1 = token opened a state */
    int32_t *seg_out;               /* [BH][T] states opened in this call so far - 1 */
    int32_t *m_out;                 /* [BH][T] states held after the token */
    int32_t *ev_t, *ev_i, *n_ev;    /* merges: token, index of the earlier state */
    int32_t *fin_m;                 /* [BH] */
    double *fin_S;                  /* [BH][C][dv][dk] */
    int64_t *fin_I;                 /* [BH][C] */
    int32_t *fin_n;                 /* [BH][C] */
    int64_t *fin_start;             /* [BH][C] */
    int32_t *fin_has_prev;          /* [BH] */
    float *fin_s_prev;              /* [BH] */
    float *fin_k_prev;              /* [BH][dk] */
    int64_t *fin_t_seen;            /* [BH] */
    int32_t nthreads;
    int32_t merge_rule;             /* 0: smallest summed information; 1: lowest density */
    int32_t score_rule;             /* 0: cosine of consecutive keys; 1: state information score */
} dlao_args;

/* s_t = 1 - cos(k_t, k_prev), rounded once to float. */
static float token_information(const float *kt, const float *kp, int dk)
{
    double d = 0.0, a = 0.0, b = 0.0;
    for (int i = 0; i < dk; ++i) {
        d += (double)kt[i] * (double)kp[i];
        a += (double)kt[i] * (double)kt[i];
        b += (double)kp[i] * (double)kp[i];
    }
    double ab = a * b;
    if (ab == 0.0) return 1.0f;
    return (float)(1.0 - d / sqrt(ab));
}

/* State Information Score (reading notes, section 5.1): the per-token state
 * a = v_t k_t^T is compared with the current state Sc, the most recent state
 * of the cache after token t-1; both are first divided by their root mean
 * square (RMSNorm with unit gain), and
 *     I_t = ||N(a) - N(Sc)||_F / (||N(Sc)||_F + eps),   eps = 1e-6,
 * rounded once to float.  Without a current state (empty cache), or when a
 * or Sc is the zero matrix (its normalisation is undefined), I_t = 2, the
 * largest value the score takes otherwise. */
static float state_information(const float *vt, const float *kt, const double *Sc, int dv, int dk)
{
    if (!Sc) return 2.0f;
    const double D = (double)dv * (double)dk;
    double a2 = 0.0, c2 = 0.0;
    for (int r = 0; r < dv; ++r)
        for (int c = 0; c < dk; ++c) {
            const double x = (double)vt[r] * (double)kt[c];
            const double y = Sc[(size_t)r * dk + c];
            a2 += x * x;
            c2 += y * y;
        }
    if (a2 == 0.0 || c2 == 0.0) return 2.0f;
    const double ra = sqrt(a2 / D), rc = sqrt(c2 / D);
    double diff = 0.0, nc = 0.0;
    for (int r = 0; r < dv; ++r)
        for (int c = 0; c < dk; ++c) {
            const double na = (double)vt[r] * (double)kt[c] / ra;
            const double ns = Sc[(size_t)r * dk + c] / rc;
            diff += (na - ns) * (na - ns);
            nc += ns * ns;
        }
    return (float)(sqrt(diff) / (sqrt(nc) + 1e-6));
}

static void run_stream(const dlao_args *A, int bh, double *S, int64_t *I,
                       int32_t *n, int64_t *st, float *kprev)
{
    const int T = A->T, dk = A->dk, dv = A->dv, C = A->C;
    const size_t SS = (size_t)dv * dk;
    const float tau = A->tau;
    int m = 0, has_prev = 0, nseg = 0, nev = 0;
    float s_prev = 1.0f;
    int64_t t_seen = 0;

    if (A->init_m) {
        m = A->init_m[bh];
        for (int i = 0; i < m; ++i) {
            memcpy(S + i * SS, A->init_S + ((size_t)bh * C + i) * SS, SS * sizeof(double));
            I[i] = A->init_I[(size_t)bh * C + i];
            n[i] = A->init_n[(size_t)bh * C + i];
            st[i] = A->init_start[(size_t)bh * C + i];
        }
        has_prev = A->init_has_prev[bh];
        s_prev = A->init_s_prev[bh];
        memcpy(kprev, A->init_k_prev + (size_t)bh * dk, dk * sizeof(float));
        t_seen = A->init_t_seen[bh];
    }

    for (int t = 0; t < T; ++t) {
        const size_t row = (size_t)bh * T + t;
        const float *kt = A->k + row * dk;
        const float *qt = A->q + row * dk;
        const float *vt = A->v + row * dv;
        const float *lt = A->lam + row * C;

        /* 1. token information: the cosine score of consecutive keys, or
         * (score_rule 1) the state information score against the current state */
        float s;
        int bnd;
        if (A->score_rule == 1) {
            s = state_information(vt, kt, m > 0 ? S + (size_t)(m - 1) * SS : NULL, dv, dk);
            /* 2'. boundary indicator b_t = [I_t >= tau] (section 5.1) */
            bnd = (m == 0) || (s >= tau);
        } else {
            s = has_prev ? token_information(kt, kprev, dk) : 1.0f;
            /* 2. boundary: open a state unless this and the previous token are both low */
            bnd = (m == 0) || !((s < tau) && (s_prev < tau));
        }
        int64_t qs = llrint(ldexp((double)s, 32));

        if (bnd) {
            /* 3a. the per-token state v k^T becomes a new, most recent state */
            double *Sn = S + (size_t)m * SS;
            for (int r = 0; r < dv; ++r)
                for (int c = 0; c < dk; ++c)
                    Sn[(size_t)r * dk + c] = (double)vt[r] * (double)kt[c];
            I[m] = qs;
            n[m] = 1;
            st[m] = t_seen;
            ++m;
            ++nseg;
            if (m > C) {
                /* 4. capacity merge: the adjacent pair with the smallest summed
                 * information, or (merge_rule 1) the lowest information density
                 * (I_i + I_{i+1}) / (n_i + n_{i+1}); a / b < c / d is decided as
                 * a d < c b in 128-bit integers, so the comparison is exact */
                int best = 0;
                if (A->merge_rule == 1) {
                    __int128 bnum = (__int128)(I[0] + I[1]), bden = (__int128)n[0] + n[1];
                    for (int i = 1; i + 1 < m; ++i) {
                        const __int128 num = (__int128)(I[i] + I[i + 1]), den = (__int128)n[i] + n[i + 1];
                        if (num * bden < bnum * den) { bnum = num; bden = den; best = i; }
                    }
                } else {
                    int64_t bestkey = I[0] + I[1];
                    for (int i = 1; i + 1 < m; ++i) {
                        int64_t key = I[i] + I[i + 1];
                        if (key < bestkey) { bestkey = key; best = i; }
                    }
                }
                double *Sa = S + (size_t)best * SS, *Sb = Sa + SS;
                for (size_t e = 0; e < SS; ++e) Sa[e] += Sb[e];
                I[best] += I[best + 1];
                n[best] += n[best + 1];
                /* st[best] is kept: the merged state keeps the earlier timestamp */
                for (int i = best + 1; i + 1 < m; ++i) {
                    memcpy(S + (size_t)i * SS, S + (size_t)(i + 1) * SS, SS * sizeof(double));
                    I[i] = I[i + 1];
                    n[i] = n[i + 1];
                    st[i] = st[i + 1];
                }
                --m;
                if (A->ev_t) {
                    A->ev_t[(size_t)bh * T + nev] = t;
                    A->ev_i[(size_t)bh * T + nev] = best;
                }
                ++nev;
            }
        } else {
            /* 3b. merge the token into the most recent state */
            double *Sl = S + (size_t)(m - 1) * SS;
            for (int r = 0; r < dv; ++r)
                for (int c = 0; c < dk; ++c)
                    Sl[(size_t)r * dk + c] += (double)vt[r] * (double)kt[c];
            I[m - 1] += qs;
            n[m - 1] += 1;
        }

        /* 5. bounded read over the updated cache, slot 0 = most recent state */
        if (A->o && (!A->want_o || A->want_o[row])) {
            double *ot = A->o + row * dv;
            for (int r = 0; r < dv; ++r) ot[r] = 0.0;
            for (int j = 0; j < m; ++j) {
                const double w = (double)lt[j];
                const double *Sj = S + (size_t)(m - 1 - j) * SS;
                for (int r = 0; r < dv; ++r) {
                    double acc = 0.0;
                    for (int c = 0; c < dk; ++c) acc += Sj[(size_t)r * dk + c] * (double)qt[c];
                    ot[r] += w * acc;
                }
            }
        }
        if (A->s_out) A->s_out[row] = s;
        if (A->b_out) A->b_out[row] = (uint8_t)bnd;
        if (A->seg_out) A->seg_out[row] = nseg - 1;
        if (A->m_out) A->m_out[row] = m;

        s_prev = s;
        memcpy(kprev, kt, dk * sizeof(float));
        has_prev = 1;
        ++t_seen;
    }

    if (A->n_ev) A->n_ev[bh] = nev;
    if (A->fin_m) A->fin_m[bh] = m;
    for (int i = 0; i < C; ++i) {
        if (A->fin_S) {
            double *dst = A->fin_S + ((size_t)bh * C + i) * SS;
            if (i < m) memcpy(dst, S + (size_t)i * SS, SS * sizeof(double));
            else memset(dst, 0, SS * sizeof(double));
        }
        if (A->fin_I) A->fin_I[(size_t)bh * C + i] = i < m ? I[i] : 0;
        if (A->fin_n) A->fin_n[(size_t)bh * C + i] = i < m ? n[i] : 0;
        if (A->fin_start) A->fin_start[(size_t)bh * C + i] = i < m ? st[i] : 0;
    }
    if (A->fin_has_prev) A->fin_has_prev[bh] = has_prev;
    if (A->fin_s_prev) A->fin_s_prev[bh] = s_prev;
    if (A->fin_k_prev) memcpy(A->fin_k_prev + (size_t)bh * dk, kprev, dk * sizeof(float));
    if (A->fin_t_seen) A->fin_t_seen[bh] = t_seen;
}

/* Returns 0 on success, -1 on bad arguments, -2 when out of memory. */
int dlao_run(const dlao_args *A)
{
    if (!A || A->BH < 0 || A->T < 0 || A->dk < 1 || A->dv < 1 || A->C < 1) return -1;
    if (A->T > 0 && (!A->q || !A->k || !A->v || !A->lam)) return -1;
    if (A->init_m && (!A->init_S || !A->init_I || !A->init_n || !A->init_start ||
                      !A->init_has_prev || !A->init_s_prev || !A->init_k_prev ||
                      !A->init_t_seen)) return -1;
    if (A->ev_t && (!A->ev_i || !A->n_ev)) return -1;
    if (A->merge_rule != 0 && A->merge_rule != 1) return -1;
    if (A->score_rule != 0 && A->score_rule != 1) return -1;
    if (A->init_m)
        for (int bh = 0; bh < A->BH; ++bh)
            if (A->init_m[bh] < 0 || A->init_m[bh] > A->C) return -1;

    int err = 0;
    int nt = A->nthreads > 0 ? A->nthreads : 1;
    (void)nt;
#pragma omp parallel num_threads(nt)
    {
        const size_t SS = (size_t)A->dv * A->dk;
        double *S = (double *)malloc((size_t)(A->C + 1) * SS * sizeof(double));
        int64_t *I = (int64_t *)malloc((size_t)(A->C + 1) * sizeof(int64_t));
        int32_t *n = (int32_t *)malloc((size_t)(A->C + 1) * sizeof(int32_t));
        int64_t *st = (int64_t *)malloc((size_t)(A->C + 1) * sizeof(int64_t));
        float *kp = (float *)malloc((size_t)A->dk * sizeof(float));
        int ok = S && I && n && st && kp;
        if (!ok) {
#pragma omp atomic write
            err = -2;
        }
#pragma omp for schedule(dynamic, 1)
        for (int bh = 0; bh < A->BH; ++bh)
            if (ok) run_stream(A, bh, S, I, n, st, kp);
        free(S); free(I); free(n); free(st); free(kp);
    }
    return err;
}

int dlao_abi(void) { return 1; }
