/*
 * mac_oracle.c -- TEST INFRASTRUCTURE ONLY.
 *
 * A plain, slow, obviously-correct CPU reference of the MAC-Attention
 * (Match-Amend-Complete) decode step, written in fp64 from the method's
 * description.  Only the test suite, the smoke check and the benchmark's CPU
 * baseline may load this file's library; the GPU product path never does.  It
 * shares no code, header, table or helper with the GPU library.
 *
 * Sources (page title, then the section on that page):
 *   [MAC] "MAC-Attention: Match-Amend-Complete attention reuse, up to 99% less
 *         KV reading in long-context decoding (MLSys 2026)" -- blog post.
 *   [WIKI] "MAC-Attention: A Match-Amend-Complete Scheme for Fast and Accurate
 *         Attention Computation (MLSys 2026)" -- paper summary, section
 *         "Core method".
 *   [KVC] "Attention Cache and Sequence Parallelism", section "MHA: per-token
 *         K/V" (single-layer decode: append then attend, scale 1/sqrt(d),
 *         repeat_kv for GQA) and section "MHA decode: distributed softmax"
 *         (merging partial (max, sum, output) triples).
 *
 * Conventions (readings of points the pages leave open):
 *   - positions are 0-indexed; the query at position m attends [0, m],
 *     itself included ([KVC] append-then-attend);
 *   - logit scale is 1/sqrt(d) ([KVC]; the formula on [MAC] was lost);
 *   - a summary is kept as (o, lse): o = S/Z the normalised output and
 *     lse = ln Z, which is the pair (S, Z) of [MAC] "Decomposable
 *     representation of attention" in the log form of [MAC] "Complete";
 *   - the empty summary is (o = 0, lse = -inf) and is the identity of merge.
 *
 * Parity pins for every function here live in tests/test_oracle_*.py.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#include <time.h>

#define OR_F32 0
#define OR_BF16 1

/* Read element idx of a K/V/query buffer holding fp32 or bf16 bits. */
static double elem(const void *base, int dtype, long idx)
{
    if (dtype == OR_F32)
        return (double)((const float *)base)[idx];
    uint32_t u = (uint32_t)((const uint16_t *)base)[idx] << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return (double)f;
}

static double round_to_f32(double x) { return (double)(float)x; }

static double now_s(void)
{
    struct timespec ts;
    clock_gettime(CLOCK_MONOTONIC, &ts);
    return ts.tv_sec + 1e-9 * ts.tv_nsec;
}

/*
 * Attention summary of query q over key/value positions [a, e] (clamped to
 * a >= 0).  Written out as the textbook definition ([MAC] "Decomposable
 * representation of attention"; [KVC] "MHA: per-token K/V"):
 *   l_t = scale * <q, K_t>,  M = max_t l_t,  Z = sum_t exp(l_t - M),
 *   o = sum_t exp(l_t - M) V_t / Z,  lse = M + ln Z.
 * K and V point at one KV head's rows; row t starts at element t*row_stride.
 */
void mac_oracle_summary(int d, const double *q, double scale, const void *K,
                        const void *V, int dtype, long row_stride, long a,
                        long e, double *o, double *lse)
{
    if (a < 0)
        a = 0;
    for (int i = 0; i < d; ++i)
        o[i] = 0.0;
    if (a > e) {
        *lse = -INFINITY;
        return;
    }
    long n = e - a + 1;
    double *lg = (double *)malloc((size_t)n * sizeof(double));
    double M = -INFINITY;
    for (long t = a; t <= e; ++t) {
        double s = 0.0;
        for (int i = 0; i < d; ++i)
            s += q[i] * elem(K, dtype, t * row_stride + i);
        s *= scale;
        lg[t - a] = s;
        if (s > M)
            M = s;
    }
    double Z = 0.0;
    for (long t = a; t <= e; ++t) {
        double w = exp(lg[t - a] - M);
        Z += w;
        for (int i = 0; i < d; ++i)
            o[i] += w * elem(V, dtype, t * row_stride + i);
    }
    for (int i = 0; i < d; ++i)
        o[i] /= Z;
    *lse = M + log(Z);
    free(lg);
}

/*
 * Rotary position embedding of one d-vector at position pos ([MAC] "Match
 * (1)": RoPE is a product of independent 2x2 rotations, so pre-RoPE queries
 * are compared and post-RoPE ones attend).  Pair j = (x[2j], x[2j+1]) turns
 * by the angle pos * base^(-2j/d):
 *   y[2j]   = x[2j] cos(a) - x[2j+1] sin(a),
 *   y[2j+1] = x[2j] sin(a) + x[2j+1] cos(a).
 * This is the convention the library's fused KV-RoPE append follows.
 */
void mac_oracle_rope(int d, const double *x, long pos, double base, double *y)
{
    for (int j = 0; j < d / 2; ++j) {
        double a = (double)pos * pow(base, -2.0 * j / d);
        double c = cos(a), sn = sin(a);
        y[2 * j] = x[2 * j] * c - x[2 * j + 1] * sn;
        y[2 * j + 1] = x[2 * j] * sn + x[2 * j + 1] * c;
    }
}

/*
 * Merge of the summaries of two disjoint token sets ([MAC] "Decomposable
 * representation of attention": summaries of disjoint sets add, S = S_a + S_b,
 * Z = Z_a + Z_b; [MAC] "Complete": done in the log domain with a running max;
 * [KVC] "MHA decode: distributed softmax" gives the same combination).
 * Output may alias either input.
 */
void mac_oracle_merge(int d, const double *oa, double la, const double *ob,
                      double lb, double *o, double *lse)
{
    if (la == -INFINITY) {
        for (int i = 0; i < d; ++i)
            o[i] = ob[i];
        *lse = lb;
        return;
    }
    if (lb == -INFINITY) {
        for (int i = 0; i < d; ++i)
            o[i] = oa[i];
        *lse = la;
        return;
    }
    double M = la > lb ? la : lb;
    double l = M + log(exp(la - M) + exp(lb - M));
    double wa = exp(la - l), wb = exp(lb - l);
    for (int i = 0; i < d; ++i)
        o[i] = wa * oa[i] + wb * ob[i];
    *lse = l;
}

/*
 * Log-domain subtraction: the summary of (whole minus part), where part is a
 * subset of whole ([MAC] "Paper version: the K1/K2/K3 micro-pipeline", K3
 * removes the last r tokens' contribution from the merged summary):
 *   Z_rest = Z_whole - Z_part,  S_rest = S_whole - S_part.
 * If nothing is left (Z_rest <= 0 numerically) the result is empty.
 */
void mac_oracle_unmerge(int d, const double *ow, double lw, const double *op,
                        double lp, double *o, double *lse)
{
    if (lp == -INFINITY) {
        for (int i = 0; i < d; ++i)
            o[i] = ow[i];
        *lse = lw;
        return;
    }
    double frac = 1.0 - exp(lp - lw); /* Z_rest / Z_whole */
    if (!(frac > 0.0) || lw == -INFINITY) {
        for (int i = 0; i < d; ++i)
            o[i] = 0.0;
        *lse = -INFINITY;
        return;
    }
    double lr = lw + log(frac);
    double cw = exp(lw - lr), cp = exp(lp - lr);
    for (int i = 0; i < d; ++i)
        o[i] = cw * ow[i] - cp * op[i];
    *lse = lr;
}

/*
 * One (request, query head) stream of MAC decode steps.
 *
 * Ring ([MAC] "Paper version": two rings of capacity K addressed by global
 * length mod K -- the pre-RoPE query ring and the rectified-summary ring):
 * slot k holds pos[k] (-1 = empty), the pre-RoPE query qr[k] exactly as
 * stored (ring dtype = K/V dtype), and the rectified summary (so[k], sl[k])
 * rounded to fp32 as stored.
 *
 * Warm start: prompt positions t in [L-W, L-1] are in the ring before the
 * first decode step, each with summary F(q_t, 0, t-r); these summaries are
 * evaluated lazily, the first time the slot is matched.
 *
 * Decode step at position m = L + s:
 *  Match   ([MAC] "Match (1)/(2)/(3)"): candidates are slots with
 *          pos in [m-K, m-1]; D = sum_i (qt_m,i - qr_k,i)^2 on pre-RoPE
 *          queries (NaN counts as +inf); k* = argmin D, ties to the larger
 *          position; hit iff D(k*) < T2 (the squared threshold).
 *  Complete ([MAC] "Reuse", "Complete"): on a hit with p = pos[k*], the
 *          cached summary C = AS_{0:p-r} is merged with fresh attention of
 *          the post-RoPE query over [p-r+1, m]; on a miss the output is full
 *          attention over [0, m].
 *  Rectify-append ([MAC] "Paper version", K3): the merged summary minus the
 *          last r tokens' contribution gives AS_{0:m-r}; it is written with
 *          qt_m and pos = m into slot m mod K.
 *
 * Attention-sink isolation ([MAC] "Production version: one fused persistent
 * BF16 kernel", its front-sink item): with F = front_sink > 0 the
 * first F positions never enter a reusable summary.  Every ring summary
 * covers [F, t-r] instead of [0, t-r] (warm ones included); a hit adds the
 * sink [0, min(F, m+1)) computed exactly with q_m to the cached summary and
 * the fresh range, which starts at max(F, p-r+1); a miss is full attention
 * as before; the rectified summary is the merged one minus the sink and
 * minus the band, i.e. it covers [F, m-r] (empty when m-r < F).  F = 0 is
 * the plain method.
 *
 * Minimum context ([MAC], same section, its settings block: reuse is off
 * below a minimum context): at a position m < min_context the step looks at
 * no candidate, so it is a miss (exact full attention, dist = +inf), and
 * its rectify-append still fills slot m mod K.  0 never blocks.
 *
 * Ready/epoch gating ([MAC], same section, its graph-safe readiness
 * item): restart[s] != 0 marks a ring that is not ready or was invalidated
 * before step s.  Its contents are dropped (every slot empty), so the step
 * finds no candidate and is exact full attention, and its rectify-append
 * starts the ring anew.  restart may be NULL.
 */
typedef struct {
    int d, ring_k, band_r, dtype;
    long ctx_len;    /* L: first decode position */
    int n_warm;      /* W: warm positions [L-W, L-1] */
    int n_steps;     /* decode steps to run */
    double scale;    /* logit scale, 1/sqrt(d) */
    double thresh2;  /* squared-distance threshold T2 (the fp32 value) */
    double exempt;   /* decision-exemption band on distances (1e-4) */
    long front_sink; /* F: leading positions kept out of every summary */
    long min_context; /* positions below it do not reuse (no candidate) */
} mac_oracle_cfg;

/*
 * Outputs per step s: out[s*d..], lse[s], hit[s], p[s] (-1 on miss), dist[s]
 * = sqrt(D*) (+inf when no candidate), dist2[s] = distance of the best
 * candidate at a different position (+inf if none), exempt[s] = 1 when the
 * decision lies within `exempt` of the threshold or of a tie.
 * Optional final ring state (any may be NULL): ring_pos[K], ring_q[K*d],
 * ring_o[K*d], ring_lse[K]; warm slots never matched are evaluated for it.
 * Returns seconds spent evaluating warm summaries via *warm_seconds.
 */
int mac_oracle_stream(const mac_oracle_cfg *c, const void *K, const void *V,
                      long row_stride, const void *qt_warm,
                      const float *q_warm, const void *qt_dec,
                      const float *q_dec, double *out, double *lse, int *hit,
                      long *p_out, double *dist, double *dist2, int *exempt,
                      long *ring_pos, double *ring_q, double *ring_o,
                      double *ring_lse, double *warm_seconds,
                      const int *restart)
{
    const int d = c->d, Kr = c->ring_k, r = c->band_r;
    long *pos = (long *)malloc(sizeof(long) * Kr);
    int *lazy = (int *)malloc(sizeof(int) * Kr); /* warm index + 1, or 0 */
    double *qr = (double *)malloc(sizeof(double) * Kr * d);
    double *so = (double *)malloc(sizeof(double) * Kr * d);
    double *sl = (double *)malloc(sizeof(double) * Kr);
    double *qv = (double *)malloc(sizeof(double) * d);
    double *qw = (double *)malloc(sizeof(double) * d);
    double *qt = (double *)malloc(sizeof(double) * d);
    double *fo = (double *)malloc(sizeof(double) * d);
    double *mo = (double *)malloc(sizeof(double) * d);
    double *bo = (double *)malloc(sizeof(double) * d);
    double *ro = (double *)malloc(sizeof(double) * d);
    double *ko = (double *)malloc(sizeof(double) * d);
    const long F = c->front_sink;
    double warm_t = 0.0;
    if (!pos || !lazy || !qr || !so || !sl || !qv || !qw || !qt || !fo || !mo ||
        !bo || !ro || !ko)
        return -1;

    for (int k = 0; k < Kr; ++k) {
        pos[k] = -1;
        lazy[k] = 0;
        sl[k] = -INFINITY;
        for (int i = 0; i < d; ++i)
            qr[k * d + i] = so[k * d + i] = 0.0;
    }
    for (int w = 0; w < c->n_warm; ++w) {
        long t = c->ctx_len - c->n_warm + w;
        if (t < 0)
            continue;
        int k = (int)(t % Kr);
        pos[k] = t;
        lazy[k] = w + 1;
        for (int i = 0; i < d; ++i)
            qr[k * d + i] = elem(qt_warm, c->dtype, (long)w * d + i);
    }

#define OR_FILL_WARM(k_)                                                     \
    do {                                                                     \
        if (lazy[k_]) {                                                      \
            double t0_ = now_s();                                            \
            int w_ = lazy[k_] - 1;                                           \
            for (int i = 0; i < d; ++i)                                      \
                qw[i] = (double)q_warm[(long)w_ * d + i];                    \
            double l_;                                                       \
            mac_oracle_summary(d, qw, c->scale, K, V, c->dtype, row_stride, \
                               F, pos[k_] - r, fo, &l_);                     \
            for (int i = 0; i < d; ++i)                                      \
                so[(k_) * d + i] = round_to_f32(fo[i]);                      \
            sl[k_] = round_to_f32(l_);                                       \
            lazy[k_] = 0;                                                    \
            warm_t += now_s() - t0_;                                         \
        }                                                                    \
    } while (0)

    for (int s = 0; s < c->n_steps; ++s) {
        const long m = c->ctx_len + s;
        for (int i = 0; i < d; ++i) {
            qt[i] = elem(qt_dec, c->dtype, (long)s * d + i);
            qv[i] = (double)q_dec[(long)s * d + i];
        }
        if (restart && restart[s]) {
            /* Ring not ready for this step: every slot is dropped. */
            for (int k = 0; k < Kr; ++k) {
                pos[k] = -1;
                lazy[k] = 0;
                sl[k] = -INFINITY;
                for (int i = 0; i < d; ++i)
                    qr[k * d + i] = so[k * d + i] = 0.0;
            }
        }

        /* Match: nearest pre-RoPE query among the last K positions. */
        int kb = -1;
        double Db = INFINITY, D2 = INFINITY;
        long pb = -1;
        for (int k = 0; k < Kr && m >= c->min_context; ++k) {
            if (pos[k] < m - Kr || pos[k] > m - 1)
                continue;
            double D = 0.0;
            for (int i = 0; i < d; ++i) {
                double df = qt[i] - qr[k * d + i];
                D += df * df;
            }
            if (isnan(D))
                D = INFINITY;
            if (kb < 0 || D < Db || (D == Db && pos[k] > pb)) {
                if (kb >= 0)
                    D2 = Db < D2 ? Db : D2;
                kb = k;
                Db = D;
                pb = pos[k];
            } else if (D < D2) {
                D2 = D;
            }
        }
        int h = (kb >= 0) && (Db < c->thresh2);
        double sd = sqrt(Db), sd2 = sqrt(D2), st = sqrt(c->thresh2);
        dist[s] = sd;
        dist2[s] = sd2;
        exempt[s] = (kb >= 0) && (fabs(sd - st) < c->exempt ||
                                  (sd2 - sd) < c->exempt);
        hit[s] = h;
        p_out[s] = h ? pb : -1;

        double ml, kl = -INFINITY;
        if (F > 0) /* the sink [0, min(F, m+1)), exact with q_m */
            mac_oracle_summary(d, qv, c->scale, K, V, c->dtype, row_stride, 0,
                               F - 1 < m ? F - 1 : m, ko, &kl);
        if (h) {
            /* Amend + Complete: cached AS_{F:p-r} (+) fresh [max(F, p-r+1),
             * m] (+) the sink. */
            OR_FILL_WARM(kb);
            double fl;
            mac_oracle_summary(d, qv, c->scale, K, V, c->dtype, row_stride,
                               pb - r + 1 > F ? pb - r + 1 : F, m, fo, &fl);
            mac_oracle_merge(d, so + (long)kb * d, sl[kb], fo, fl, mo, &ml);
            if (F > 0)
                mac_oracle_merge(d, mo, ml, ko, kl, mo, &ml);
        } else {
            /* Miss: full attention over [0, m]. */
            mac_oracle_summary(d, qv, c->scale, K, V, c->dtype, row_stride, 0,
                               m, mo, &ml);
        }
        for (int i = 0; i < d; ++i)
            out[(long)s * d + i] = mo[i];
        lse[s] = ml;

        /* Rectify: merged minus the last r tokens' contribution and minus
         * the sink, leaving [F, m-r]. */
        double rl;
        if (m - r < F) {
            for (int i = 0; i < d; ++i)
                ro[i] = 0.0;
            rl = -INFINITY;
        } else {
            double bl;
            mac_oracle_summary(d, qv, c->scale, K, V, c->dtype, row_stride,
                               m - r + 1, m, bo, &bl);
            mac_oracle_unmerge(d, mo, ml, bo, bl, ro, &rl);
            if (F > 0)
                mac_oracle_unmerge(d, ro, rl, ko, kl, ro, &rl);
        }
        /* Append into slot m mod K (the slot's old entry is overwritten). */
        int ks = (int)(m % Kr);
        pos[ks] = m;
        lazy[ks] = 0;
        for (int i = 0; i < d; ++i) {
            qr[ks * d + i] = qt[i];
            so[ks * d + i] = round_to_f32(ro[i]);
        }
        sl[ks] = round_to_f32(rl);
    }

    for (int k = 0; k < Kr; ++k) {
        if (ring_o || ring_lse)
            OR_FILL_WARM(k);
        if (ring_pos)
            ring_pos[k] = pos[k];
        for (int i = 0; i < d; ++i) {
            if (ring_q)
                ring_q[k * d + i] = qr[k * d + i];
            if (ring_o)
                ring_o[k * d + i] = so[k * d + i];
        }
        if (ring_lse)
            ring_lse[k] = sl[k];
    }
#undef OR_FILL_WARM
    if (warm_seconds)
        *warm_seconds = warm_t;
    free(pos);
    free(lazy);
    free(qr);
    free(so);
    free(sl);
    free(qv);
    free(qw);
    free(qt);
    free(fo);
    free(mo);
    free(bo);
    free(ro);
    free(ko);
    return 0;
}
