/*
 * oracle.c -- plain, slow, fp64 CPU reference for exact softmax attention.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the test suite, the smoke check and the
 * benchmark's CPU-baseline leg may load this library.  It shares no code,
 * header, table or helper with the GPU library; it includes only libc/libm.
 *
 * What it computes (all in double precision, inputs given as doubles):
 *
 *   O[b,h,i,:] = sum_j w_j * V[b,g,j,:] / sum_j w_j,   w_j = exp(s_j - m),
 *   m = max_j s_j over the visible keys, lse = m + log(sum_j w_j),
 *
 * with s_j = scale * <Q[b,h,i,:], K[b,g,j,:]>, optionally soft-capped as
 * kappa * tanh(s_j / kappa).  Sources:
 *   - "Online Softmax Without the Attention Matrix" (notebook, code cell):
 *     the dense weighted average with the maximum subtracted, and the
 *     streaming recurrence with a running max, denominator and numerator.
 *   - nx_flashattn_scale.nx (direct softmax reference block): one query row
 *     at a time, all its scores materialised, max, exp, sum, weighted V;
 *     scale = 1/sqrt(d).
 *   - oxios_kernel flash_attention.rs, naive_attention and attention: the
 *     same definition for N_q x D queries against N_k keys; no keys gives
 *     an empty result and a zero normaliser leaves the output at zero.
 *   - Transformers & Math, Module 16: section 16.5 (soft-cap
 *     kappa*tanh(z/kappa) applied to z = QK^T/sqrt(d_k)), section 16.3
 *     (sliding window: a query sees only the last W positions), section 16.2 "Measured"
 *     (causal mask by absolute position in the full sequence) and the two
 *     merge equations of section 16.2 for combining per-block (m, l, O).
 *
 * Readings where the pages are silent (documented with the design notes):
 *   - query row i sits at absolute position p = i + (Nk - Nq) (the last
 *     query aligned with the last key); causal keeps j <= p;
 *   - a window W > 0 keeps p - W < j, i.e. exactly W keys including the
 *     query's own position; it is defined only together with causal;
 *   - attention sinks (section 16.6, streaming: the opening tokens are
 *     always kept alongside the sliding window): with sinks = S > 0 the
 *     keys j < S stay visible to a windowed row whatever its window (still
 *     subject to the causal rule j <= p);
 *   - query head h reads key/value head g = h / (H / Hkv);
 *   - a row with no visible key gets O = 0, lse = -inf, m = -inf, l = 0;
 *   - the mask is applied after the cap (masked keys never contribute).
 *
 * Layouts (row-major, contiguous): Q, O [B,H,Nq,d]; K, V [B,Hkv,Nk,d];
 * lse, m, l [B,H,Nq].  A "row" index r = (b*H + h)*Nq + i.
 */
#include <math.h>
#include <pthread.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

typedef struct {
    const double *q, *k, *v;
    double *o, *lse, *m_out, *l_out;
    int64_t B, H, Hkv, Nq, Nk, d;
    double scale;
    int causal;
    const int32_t *head_window; /* [H]; <= 0 means no window for that head */
    double softcap;             /* <= 0 disables the cap */
    int64_t sinks;              /* keys j < sinks ignore the window */
    int64_t key_lo, key_hi;     /* keys outside [key_lo, key_hi) are excluded */
    const int64_t *rows;        /* NULL: all rows; else nrows row indices    */
    int64_t nrows;
    int64_t tile;               /* 0: direct definition; > 0: streaming     */
    int64_t first, last;        /* this worker's slice of [0, nrows)         */
} job_t;

/* Is key j visible from query row i of head h? */
static int visible(const job_t *J, int64_t h, int64_t i, int64_t j)
{
    int64_t p = i + (J->Nk - J->Nq);
    int32_t W = J->head_window ? J->head_window[h] : 0;
    if (j < J->key_lo || j >= J->key_hi) return 0;
    if (J->causal && j > p) return 0;
    if (W > 0 && j <= p - W && j >= J->sinks) return 0;
    return 1;
}

/* Score of query row (b,h,i) against key j, after scale and soft-cap. */
static double score(const job_t *J, int64_t b, int64_t h, int64_t i, int64_t j)
{
    int64_t g = h / (J->H / J->Hkv);
    const double *qr = J->q + ((b * J->H + h) * J->Nq + i) * J->d;
    const double *kr = J->k + ((b * J->Hkv + g) * J->Nk + j) * J->d;
    double s = 0.0;
    for (int64_t c = 0; c < J->d; ++c) s += qr[c] * kr[c];
    s *= J->scale;
    if (J->softcap > 0.0) s = J->softcap * tanh(s / J->softcap);
    return s;
}

static void write_row(const job_t *J, int64_t out, double m, double l, const double *num)
{
    double *orow = J->o ? J->o + out * J->d : NULL;
    if (l > 0.0) {
        if (orow)
            for (int64_t c = 0; c < J->d; ++c) orow[c] = num[c] / l;
        if (J->lse) J->lse[out] = m + log(l);
    } else {
        if (orow)
            for (int64_t c = 0; c < J->d; ++c) orow[c] = 0.0;
        if (J->lse) J->lse[out] = -INFINITY;
        m = -INFINITY;
    }
    if (J->m_out) J->m_out[out] = m;
    if (J->l_out) J->l_out[out] = l;
}

/* Direct definition: materialise the row's scores, take their maximum,
 * exponentiate, sum, and form the weighted average of V. */
static void row_direct(const job_t *J, int64_t r, int64_t out, double *sc, double *num)
{
    int64_t b = r / (J->H * J->Nq), h = (r / J->Nq) % J->H, i = r % J->Nq;
    int64_t g = h / (J->H / J->Hkv);
    double m = -INFINITY, l = 0.0;
    int any = 0;
    for (int64_t j = 0; j < J->Nk; ++j) {
        if (!visible(J, h, i, j)) continue;
        sc[j] = score(J, b, h, i, j);
        if (!any || sc[j] > m) m = sc[j];
        any = 1;
    }
    for (int64_t c = 0; c < J->d; ++c) num[c] = 0.0;
    if (any) {
        for (int64_t j = 0; j < J->Nk; ++j) {
            if (!visible(J, h, i, j)) continue;
            double w = exp(sc[j] - m);
            const double *vr = J->v + ((b * J->Hkv + g) * J->Nk + j) * J->d;
            l += w;
            for (int64_t c = 0; c < J->d; ++c) num[c] += w * vr[c];
        }
    }
    write_row(J, out, m, l, num);
}

/* Streaming recurrence over key tiles of J->tile keys: a running maximum,
 * denominator and numerator; on each tile the old denominator and numerator
 * are multiplied by exp(old_max - new_max), which is taken as 0 while no key
 * has been seen yet (old_max = -inf). */
static void row_stream(const job_t *J, int64_t r, int64_t out, double *sc, double *num)
{
    int64_t b = r / (J->H * J->Nq), h = (r / J->Nq) % J->H, i = r % J->Nq;
    int64_t g = h / (J->H / J->Hkv);
    double run_max = -INFINITY, den = 0.0;
    for (int64_t c = 0; c < J->d; ++c) num[c] = 0.0;
    for (int64_t start = 0; start < J->Nk; start += J->tile) {
        int64_t stop = start + J->tile < J->Nk ? start + J->tile : J->Nk;
        double new_max = run_max;
        int any = 0;
        for (int64_t j = start; j < stop; ++j) {
            if (!visible(J, h, i, j)) continue;
            sc[j] = score(J, b, h, i, j);
            if (sc[j] > new_max) new_max = sc[j];
            any = 1;
        }
        if (!any) continue;
        double corr = (run_max == -INFINITY) ? 0.0 : exp(run_max - new_max);
        den *= corr;
        for (int64_t c = 0; c < J->d; ++c) num[c] *= corr;
        for (int64_t j = start; j < stop; ++j) {
            if (!visible(J, h, i, j)) continue;
            double w = exp(sc[j] - new_max);
            const double *vr = J->v + ((b * J->Hkv + g) * J->Nk + j) * J->d;
            den += w;
            for (int64_t c = 0; c < J->d; ++c) num[c] += w * vr[c];
        }
        run_max = new_max;
    }
    write_row(J, out, run_max, den, num);
}

static void *worker(void *arg)
{
    const job_t *J = (const job_t *)arg;
    double *sc = (double *)malloc((size_t)(J->Nk > 0 ? J->Nk : 1) * sizeof(double));
    double *num = (double *)malloc((size_t)(J->d > 0 ? J->d : 1) * sizeof(double));
    if (!sc || !num) { free(sc); free(num); return (void *)1; }
    for (int64_t n = J->first; n < J->last; ++n) {
        int64_t r = J->rows ? J->rows[n] : n;
        if (J->tile > 0) row_stream(J, r, n, sc, num);
        else row_direct(J, r, n, sc, num);
    }
    free(sc);
    free(num);
    return NULL;
}

/*
 * oracle_attention -- direct (tile == 0) or streaming (tile > 0) attention.
 *
 * q [B,H,Nq,d], k and v [B,Hkv,Nk,d]: caller-owned doubles.
 * head_window: int32[H] or NULL (no window on any head).
 * rows: NULL to compute every row, writing o [B*H*Nq, d] and the per-row
 *       outputs [B*H*Nq]; otherwise nrows row indices, writing o [nrows, d].
 * o, lse, m_out, l_out: any may be NULL.  m_out/l_out receive the row max
 *       and sum exp(s - m) (the (m, l) of the merge equations).
 * sinks: keys j < sinks are exempt from the window (attention sinks).
 * key_lo, key_hi: restrict the keys to [key_lo, key_hi) (one split's chunk).
 * nthreads: worker threads over rows (<= 0: one).
 * Returns 0 on success, -1 on invalid arguments, -2 on allocation failure.
 */
int oracle_attention(const double *q, const double *k, const double *v,
                     double *o, double *lse, double *m_out, double *l_out,
                     int64_t B, int64_t H, int64_t Hkv, int64_t Nq, int64_t Nk, int64_t d,
                     double scale, int causal, const int32_t *head_window, double softcap,
                     int64_t sinks, int64_t key_lo, int64_t key_hi,
                     const int64_t *rows, int64_t nrows, int64_t tile, int nthreads)
{
    if (B < 0 || H < 0 || Hkv <= 0 || Nq < 0 || Nk < 0 || d < 0) return -1;
    if (H % Hkv != 0 || tile < 0 || sinks < 0) return -1;
    if (head_window) {
        for (int64_t h = 0; h < H; ++h)
            if (head_window[h] > 0 && !causal) return -1;
    }
    int64_t total = B * H * Nq;
    if (!rows) nrows = total;
    for (int64_t n = 0; rows && n < nrows; ++n)
        if (rows[n] < 0 || rows[n] >= total) return -1;
    if (nrows == 0) return 0;
    if (nthreads <= 0) nthreads = 1;
    if (nthreads > nrows) nthreads = (int)nrows;

    job_t base;
    memset(&base, 0, sizeof base);
    base.q = q; base.k = k; base.v = v;
    base.o = o; base.lse = lse; base.m_out = m_out; base.l_out = l_out;
    base.B = B; base.H = H; base.Hkv = Hkv; base.Nq = Nq; base.Nk = Nk; base.d = d;
    base.scale = scale; base.causal = causal; base.head_window = head_window;
    base.softcap = softcap;
    base.sinks = sinks;
    base.key_lo = key_lo < 0 ? 0 : key_lo;
    base.key_hi = key_hi > Nk ? Nk : key_hi;
    base.rows = rows; base.nrows = nrows; base.tile = tile;

    job_t *jobs = (job_t *)calloc((size_t)nthreads, sizeof(job_t));
    pthread_t *tids = (pthread_t *)calloc((size_t)nthreads, sizeof(pthread_t));
    if (!jobs || !tids) { free(jobs); free(tids); return -2; }
    int rc = 0;
    for (int t = 0; t < nthreads; ++t) {
        jobs[t] = base;
        jobs[t].first = nrows * t / nthreads;
        jobs[t].last = nrows * (t + 1) / nthreads;
    }
    int started = 0;
    for (int t = 1; t < nthreads; ++t) {
        if (pthread_create(&tids[t], NULL, worker, &jobs[t]) != 0) { rc = -2; break; }
        started = t;
    }
    if (worker(&jobs[0]) != NULL) rc = -2;
    for (int t = 1; t <= started; ++t) {
        void *ret = NULL;
        pthread_join(tids[t], &ret);
        if (ret != NULL) rc = -2;
    }
    free(jobs);
    free(tids);
    return rc;
}

/*
 * oracle_combine -- merge S per-block results of each of R rows.
 *
 * Follows the two merge equations of Transformers & Math section 16.2: with
 * m = max(m1, m2), l = e^(m1-m) l1 + e^(m2-m) l2 and
 * O = (e^(m1-m) l1 / l) O1 + (e^(m2-m) l2 / l) O2, where O_i is block i's own
 * normalised output; further blocks are folded in one at a time against the running
 * result, here in block order s = 0, 1, ..., S-1.  A block with l_s = 0 saw
 * no visible key and carries no weight; it is skipped.
 *
 * o_part [R,S,d], m_part and l_part [R,S]; writes o [R,d] and lse [R]
 * (lse = m + log l; -inf and O = 0 when every block is empty).
 */
int oracle_combine(const double *o_part, const double *m_part, const double *l_part,
                   double *o, double *lse, int64_t R, int64_t S, int64_t d)
{
    if (R < 0 || S < 1 || d < 0) return -1;
    for (int64_t r = 0; r < R; ++r) {
        double m_run = -INFINITY, l_run = 0.0;
        double *orow = o + r * d;
        for (int64_t c = 0; c < d; ++c) orow[c] = 0.0;
        for (int64_t s = 0; s < S; ++s) {
            double ms = m_part[r * S + s], ls = l_part[r * S + s];
            const double *os = o_part + (r * S + s) * d;
            if (!(ls > 0.0)) continue;
            if (l_run == 0.0) {
                m_run = ms;
                l_run = ls;
                for (int64_t c = 0; c < d; ++c) orow[c] = os[c];
                continue;
            }
            double m = m_run > ms ? m_run : ms;
            double w_run = exp(m_run - m) * l_run;
            double w_s = exp(ms - m) * ls;
            double l = w_run + w_s;
            for (int64_t c = 0; c < d; ++c) orow[c] = (w_run / l) * orow[c] + (w_s / l) * os[c];
            m_run = m;
            l_run = l;
        }
        lse[r] = l_run > 0.0 ? m_run + log(l_run) : -INFINITY;
    }
    return 0;
}
