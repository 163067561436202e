/*
 * lt_oracle.c -- plain fp64 CPU oracle for the LightTransfer-Test hot path.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the product path may call, link or
 * load this file; only the tests, the smoke check and the CPU-baseline leg of
 * the benchmark do.  It shares no code, header or constant with the HIP
 * library.
 *
 * What it computes (all in IEEE double, sums taken sequentially in key order):
 *   - causal attention with every softmax row materialised, its log-sum-exp
 *     (natural log), and the output P.V;
 *   - the per-row lazy ratio: the softmax mass a query puts on the initial
 *     ("sink") keys plus its recent keys;
 *   - the per-head lazy ratio: the mean of the per-row ratios over the last
 *     W queries;
 *   - streaming attention: the same softmax restricted to the sink + recent
 *     key set, with its own log-sum-exp;
 *   - decode attention: one query that sees every row of a cache.
 *
 * Sources (LightTransfer web pages):
 *   - LightTransfer project page, "Introduction": lazy layers attend mostly
 *     to a few tokens and are converted to streaming attention.
 *   - Chinese write-up (xzbcqc.com), "problem 1 / solution 1": Flash
 *     Attention keeps no attention weights; the LSE it produces serves as
 *     the lazy ratio's denominator, the numerator costs O(1) per query.
 *   - Press-release page (wuwenjie.xyz), "LightTransfer method": the lazy
 *     ratio is the sum of attention weights from the queries to the initial
 *     and the most recent keys.
 * Readings where the pages are silent: softmax scale is a caller argument
 * (1/sqrt(D) by default on the Python side); causal masking is square and
 * aligned at position 0 (key j visible to query i iff j <= i); query head h
 * reads KV head h / (Hq/Hkv); the recent set of query i is the R keys
 * (i-R, i]; the sink set is [0, S); the observed queries are the last W.
 *
 * Layouts: q, out [B,Hq,N,D]; k, v [B,Hkv,N,D]; lse [B,Hq,N]; all contiguous.
 *
 * Parity pins for every function here live in tests/test_oracle_*.py:
 * an mpmath brute force without max-subtraction, torch's fp64
 * scaled_dot_product_attention and logsumexp, closed forms for zero queries,
 * and the invariants listed there.
 */
#include <math.h>
#include <omp.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define LTO_OK 0
#define LTO_BAD_ARG 1
#define LTO_NO_MEM 2

/* Membership of key j (j <= i) in query i's sink + recent set. */
static int in_sink_or_recent(long j, long i, long S, long R) {
    return (j < S) || (j > i - R);
}

/*
 * One query row against keys 0..last (inclusive), materialising the row.
 *   qi [D], k [*, D], v [*, D] (row-major, this head's KV).
 *   i is the query position used for the recent set (i - R, i].
 * Outputs (each may be NULL except scratch):
 *   o [D], lse: full causal softmax over keys 0..last.
 *   lazy: sum of P_j over the sink + recent set.
 *   so [D], slse: streaming attention (softmax restricted to that set).
 * s, p: scratch of length last+1.
 */
static void attn_row(long last, int D, double scale, const double *qi, const double *k,
                     const double *v, long i, long S, long R, double *o, double *lse,
                     double *lazy, double *so, double *slse, double *s, double *p) {
    long j;
    int d;
    /* scores s_j = scale * <q_i, k_j> */
    for (j = 0; j <= last; ++j) {
        double acc = 0.0;
        const double *kj = k + (size_t)j * D;
        for (d = 0; d < D; ++d) acc += qi[d] * kj[d];
        s[j] = scale * acc;
    }
    /* full softmax row: m, LSE = m + ln sum exp(s - m), P_j = exp(s_j - LSE) */
    double m = -INFINITY;
    for (j = 0; j <= last; ++j)
        if (s[j] > m) m = s[j];
    double sum = 0.0;
    for (j = 0; j <= last; ++j) sum += exp(s[j] - m);
    double L = m + log(sum);
    for (j = 0; j <= last; ++j) p[j] = exp(s[j] - L);
    if (lse) *lse = L;
    if (o) {
        for (d = 0; d < D; ++d) o[d] = 0.0;
        for (j = 0; j <= last; ++j) {
            const double *vj = v + (size_t)j * D;
            for (d = 0; d < D; ++d) o[d] += p[j] * vj[d];
        }
    }
    /* lazy ratio of this row: attention mass on the sink + recent keys */
    if (lazy) {
        double r = 0.0;
        for (j = 0; j <= last; ++j)
            if (in_sink_or_recent(j, i, S, R)) r += p[j];
        *lazy = r;
    }
    /* streaming attention: its own softmax over the sink + recent keys */
    if (so || slse) {
        double ms = -INFINITY;
        for (j = 0; j <= last; ++j)
            if (in_sink_or_recent(j, i, S, R) && s[j] > ms) ms = s[j];
        double ss = 0.0;
        for (j = 0; j <= last; ++j)
            if (in_sink_or_recent(j, i, S, R)) ss += exp(s[j] - ms);
        double Ls = ms + log(ss);
        if (slse) *slse = Ls;
        if (so) {
            for (d = 0; d < D; ++d) so[d] = 0.0;
            for (j = 0; j <= last; ++j) {
                if (!in_sink_or_recent(j, i, S, R)) continue;
                double pj = exp(s[j] - Ls);
                const double *vj = v + (size_t)j * D;
                for (d = 0; d < D; ++d) so[d] += pj * vj[d];
            }
        }
    }
}

/*
 * Causal GQA prefill.  Any output pointer may be NULL, except that lazy_ratio
 * needs lazy_rows (the per-head mean is taken over the stored per-row values).
 *   out [B,Hq,N,D], lse [B,Hq,N]            full attention
 *   sout [B,Hq,N,D], slse [B,Hq,N]          streaming attention (S, R)
 *   lazy_rows [B,Hq,W], lazy_ratio [B,Hq]   lazy ratio over the last W queries
 */
int lto_prefill(int B, int N, int Hq, int Hkv, int D, double scale, const double *q,
                const double *k, const double *v, int S, int R, int W, double *out,
                double *lse, double *sout, double *slse, double *lazy_rows,
                double *lazy_ratio) {
    if (B < 1 || N < 1 || Hq < 1 || Hkv < 1 || D < 1 || Hq % Hkv != 0) return LTO_BAD_ARG;
    if (S < 0 || R < 0 || W < 0 || W > N) return LTO_BAD_ARG;
    if (lazy_ratio && !lazy_rows) return LTO_BAD_ARG;
    if (lazy_rows && W < 1) return LTO_BAD_ARG;
    const int G = Hq / Hkv;
    const long BH = (long)B * Hq;
    int err = 0;
#pragma omp parallel
    {
        double *sbuf = (double *)malloc(sizeof(double) * (size_t)N);
        double *pbuf = (double *)malloc(sizeof(double) * (size_t)N);
        if (!sbuf || !pbuf) {
#pragma omp atomic write
            err = 1;
        } else {
#pragma omp for schedule(dynamic, 4) collapse(2)
            for (long bh = 0; bh < BH; ++bh) {
                for (long i = 0; i < N; ++i) {
                    long b = bh / Hq, h = bh % Hq, hk = h / G;
                    const double *qi = q + ((size_t)bh * N + i) * D;
                    const double *kh = k + ((size_t)b * Hkv + hk) * N * D;
                    const double *vh = v + ((size_t)b * Hkv + hk) * N * D;
                    double *o = out ? out + ((size_t)bh * N + i) * D : NULL;
                    double *l = lse ? lse + (size_t)bh * N + i : NULL;
                    double *so = sout ? sout + ((size_t)bh * N + i) * D : NULL;
                    double *sl = slse ? slse + (size_t)bh * N + i : NULL;
                    double *lz = NULL;
                    if (lazy_rows && i >= N - W) lz = lazy_rows + (size_t)bh * W + (i - (N - W));
                    if (!o && !l && !so && !sl && !lz) continue;
                    attn_row(i, D, scale, qi, kh, vh, i, S, R, o, l, lz, so, sl, sbuf, pbuf);
                }
            }
        }
        free(sbuf);
        free(pbuf);
    }
    if (err) return LTO_NO_MEM;
    if (lazy_ratio) {
        /* per-head ratio: mean of the last W per-row ratios, summed in row order */
        for (long bh = 0; bh < BH; ++bh) {
            double acc = 0.0;
            for (int w = 0; w < W; ++w) acc += lazy_rows[(size_t)bh * W + w];
            lazy_ratio[bh] = acc / (double)W;
        }
    }
    return LTO_OK;
}

/*
 * Selected rows of one head, for sampled checks at sizes where the full
 * oracle would take too long.  k, v [nk, D] are the head's KV rows; row r is
 * query position pos[r] with qrows[r*D..]; it sees keys 0..pos[r].
 * Any output may be NULL.  Returns LTO_BAD_ARG if a position is >= nk.
 */
int lto_rows(int nk, int D, double scale, const double *k, const double *v, int nrows,
             const int *pos, const double *qrows, int S, int R, double *out, double *lse,
             double *lazy, double *sout, double *slse) {
    if (nk < 1 || D < 1 || nrows < 0 || S < 0 || R < 0) return LTO_BAD_ARG;
    for (int r = 0; r < nrows; ++r)
        if (pos[r] < 0 || pos[r] >= nk) return LTO_BAD_ARG;
    int err = 0;
#pragma omp parallel
    {
        double *sbuf = (double *)malloc(sizeof(double) * (size_t)nk);
        double *pbuf = (double *)malloc(sizeof(double) * (size_t)nk);
        if (!sbuf || !pbuf) {
#pragma omp atomic write
            err = 1;
        } else {
#pragma omp for schedule(dynamic, 1)
            for (int r = 0; r < nrows; ++r) {
                long i = pos[r];
                attn_row(i, D, scale, qrows + (size_t)r * D, k, v, i, S, R,
                         out ? out + (size_t)r * D : NULL, lse ? lse + r : NULL,
                         lazy ? lazy + r : NULL, sout ? sout + (size_t)r * D : NULL,
                         slse ? slse + r : NULL, sbuf, pbuf);
            }
        }
        free(sbuf);
        free(pbuf);
    }
    return err ? LTO_NO_MEM : LTO_OK;
}

/*
 * Decode: one query per (b, h) against every one of the kv_len cache rows.
 *   q [B,Hq,D]; k, v [B,Hkv,kv_len,D]; out [B,Hq,D]; lse [B,Hq] (may be NULL).
 * The cache includes the current token, so the query sees all rows.
 */
int lto_decode(int B, int Hq, int Hkv, int D, double scale, const double *q, const double *k,
               const double *v, long kv_len, double *out, double *lse) {
    if (B < 1 || Hq < 1 || Hkv < 1 || D < 1 || kv_len < 1 || Hq % Hkv != 0) return LTO_BAD_ARG;
    const int G = Hq / Hkv;
    int err = 0;
#pragma omp parallel
    {
        double *sbuf = (double *)malloc(sizeof(double) * (size_t)kv_len);
        double *pbuf = (double *)malloc(sizeof(double) * (size_t)kv_len);
        if (!sbuf || !pbuf) {
#pragma omp atomic write
            err = 1;
        } else {
#pragma omp for schedule(dynamic, 1)
            for (long bh = 0; bh < (long)B * Hq; ++bh) {
                long b = bh / Hq, h = bh % Hq, hk = h / G;
                const double *kh = k + ((size_t)b * Hkv + hk) * kv_len * D;
                const double *vh = v + ((size_t)b * Hkv + hk) * kv_len * D;
                attn_row(kv_len - 1, D, scale, q + (size_t)bh * D, kh, vh, kv_len - 1, 0, 0,
                         out + (size_t)bh * D, lse ? lse + bh : NULL, NULL, NULL, NULL, sbuf,
                         pbuf);
            }
        }
        free(sbuf);
        free(pbuf);
    }
    return err ? LTO_NO_MEM : LTO_OK;
}

/* Threads an OpenMP region of the oracle uses (reported with its timings). */
int lto_threads(void) { return omp_get_max_threads(); }
