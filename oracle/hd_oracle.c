/*
 * hd_oracle.c -- plain, slow CPU oracle for Stream-Factorized Attention.
 *
 * TEST INFRASTRUCTURE ONLY.  This file is the checker, not the product: only
 * the tests, the smoke check and the benchmark's CPU-baseline leg load it.  It
 * shares no code, header or constant with the HIP library under
 * latent_sequence_length_amd/csrc, and nothing in the product path calls it.
 *
 * Source of every definition below: the WeLM blog post "Hidden Decoding at
 * Scale", section "Method Recap and New Designs":
 *   - subsection "Multi-Stream Expansion and Training Objective", the equation
 *     S_t = E_k(x_i) at physical position t = (i-1)n + k;
 *   - subsection "Stream-Factorized Attention", the index maps
 *     i(t) = ceil(t/n), s(t) = (t-1) mod n + 1, and Figure 2 (masks (a) full
 *     cross-stream causal, (b) local cross-stream sliding window, (c) intra-stream
 *     causal within each stream);
 *   - subsection "Persistent KV and the KV-mirror Saving": one KV cache per
 *     stream is retained, and section "Inference Throughput": the n streams of a
 *     new token are processed together in one pass.
 *
 * Indices here are 0-based: position t = i*n + s with token i in [0,L) and
 * stream s in [0,n).  This is the 1-based t = (i-1)n + k with i <- i+1, k <- s+1.
 *
 * Readings where the pages are silent (each one is a choice, listed with the
 * reasons in the design notes):
 *   - the intra-stream mask includes the diagonal (a query sees its own key);
 *   - a window W counts tokens including self: intra keeps i_q - i_k < W, cross
 *     keeps t_q - t_k < n*W on the expanded sequence; W = 0 means no window;
 *   - the GQA group of query head h is kv head h / (Hq/Hkv);
 *   - layouts: Q/O [B][nL][Hq][d], K/V [B][nL][Hkv][d], cache [B][T_cap][n][Hkv][d].
 *
 * Arithmetic: inputs are float32 or bfloat16 (raw bits, widened exactly to
 * float), every sum and exponential is evaluated in double, keys are visited in
 * ascending position order, and the softmax is the textbook max-shifted one.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define OR_F32 0
#define OR_BF16 1
#define OR_INTRA 0
#define OR_CROSS 1

/* Widen one input element to double.  bfloat16 is the top 16 bits of an IEEE
 * float32, so widening is a 16-bit left shift of the raw bits. */
static double load_elem(const void *base, int dtype, int64_t idx) {
    if (dtype == OR_F32) return (double)((const float *)base)[idx];
    uint32_t bits = ((uint32_t)((const uint16_t *)base)[idx]) << 16;
    float f;
    memcpy(&f, &bits, sizeof f);
    return (double)f;
}

/* ---------------------------------------------------------------------------
 * Multi-stream expansion ("Multi-Stream Expansion and Training Objective",
 * equation S_t = E_k(x_i)): out[b][i*n+s][:] = tables[s][ids[b][i]][:].
 * A raw byte copy of one table row per output row.  Returns -1 (and writes
 * nothing further) if an id lies outside [0,V).
 * ------------------------------------------------------------------------- */
int oracle_expand_embed(const int32_t *ids, int B, int L, int n,
                        const void *const *tables, int64_t V, int64_t row_bytes,
                        void *out) {
    for (int b = 0; b < B; ++b)
        for (int i = 0; i < L; ++i) {
            int64_t id = ids[(int64_t)b * L + i];
            if (id < 0 || id >= V) return -1;
            for (int s = 0; s < n; ++s) {
                const char *src = (const char *)tables[s] + id * row_bytes;
                char *dst = (char *)out + (((int64_t)b * L + i) * n + s) * row_bytes;
                memcpy(dst, src, (size_t)row_bytes);
            }
        }
    return 0;
}

/* ---------------------------------------------------------------------------
 * Visibility predicate of Figure 2 on 0-based expanded positions.
 *   intra (mask c): same stream, earlier-or-equal token, within W tokens.
 *   cross (mask a, or b when W > 0): earlier-or-equal position, within n*W
 *   positions of the expanded sequence.
 * ------------------------------------------------------------------------- */
int oracle_visible(int64_t tq, int64_t tk, int n, int mode, int64_t W) {
    if (mode == OR_INTRA) {
        int64_t iq = tq / n, sq = tq % n, ik = tk / n, sk = tk % n;
        if (sk != sq) return 0;
        if (ik > iq) return 0;
        if (W > 0 && iq - ik >= W) return 0;
        return 1;
    }
    if (tk > tq) return 0;
    if (W > 0 && tq - tk >= (int64_t)n * W) return 0;
    return 1;
}

/* One attention row: softmax over the visible keys of scale * q.k, then the
 * weighted sum of the matching value rows.  kpos(j) lists candidate key
 * positions 0..nk-1 (all positions <= tq); the predicate selects the visible
 * ones.  K/V rows are addressed through krow(j) element offsets. */
static void attend_row(const void *q, int64_t qoff, const void *k, const void *v,
                       const int64_t *krow_off, const int64_t *kpos, int64_t nk,
                       int64_t tq, int n, int mode, int64_t W, int d, int dtype,
                       double scale, double *scores, double *o, double *lse) {
    double m = -INFINITY;
    int64_t nvis = 0;
    for (int64_t j = 0; j < nk; ++j) {
        if (!oracle_visible(tq, kpos[j], n, mode, W)) { scores[j] = NAN; continue; }
        double dot = 0.0;
        for (int c = 0; c < d; ++c)
            dot += load_elem(q, dtype, qoff + c) * load_elem(k, dtype, krow_off[j] + c);
        scores[j] = scale * dot;
        if (scores[j] > m) m = scores[j];
        ++nvis;
    }
    for (int c = 0; c < d; ++c) o[c] = 0.0;
    if (nvis == 0) {           /* cannot happen with the diagonal visible */
        if (lse) *lse = -INFINITY;
        return;
    }
    double l = 0.0;
    for (int64_t j = 0; j < nk; ++j) {
        if (isnan(scores[j])) continue;
        double p = exp(scores[j] - m);
        l += p;
        for (int c = 0; c < d; ++c) o[c] += p * load_elem(v, dtype, krow_off[j] + c);
    }
    for (int c = 0; c < d; ++c) o[c] /= l;
    if (lse) *lse = m + log(l);
}

/* ---------------------------------------------------------------------------
 * Prefill attention for a list of query rows.
 * q [B][n*L][Hq][d], k/v [B][n*L][Hkv][d] (dtype OR_F32 or OR_BF16).
 * rows: flat query-row ids r = (b*n*L + t)*Hq + h.  Outputs o [nrows][d],
 * lse [nrows] (natural log of the softmax denominator incl. the max shift).
 * scale <= 0 selects 1/sqrt(d).  Returns 0, or -1 on bad arguments.
 * ------------------------------------------------------------------------- */
int oracle_sfa_rows(const void *q, const void *k, const void *v, int dtype,
                    int B, int L, int n, int Hq, int Hkv, int d, int mode,
                    int64_t W, double scale, const int64_t *rows, int64_t nrows,
                    double *o, double *lse) {
    if (B < 1 || L < 1 || n < 1 || Hq < 1 || Hkv < 1 || d < 1 || Hq % Hkv) return -1;
    if (W < 0 || (mode != OR_INTRA && mode != OR_CROSS)) return -1;
    if (scale <= 0.0) scale = 1.0 / sqrt((double)d);
    const int64_t nL = (int64_t)n * L;
    const int g = Hq / Hkv;
    int bad = 0;
#pragma omp parallel
    {
        double *scores = (double *)malloc(sizeof(double) * (size_t)nL);
        int64_t *kpos = (int64_t *)malloc(sizeof(int64_t) * (size_t)nL);
        int64_t *koff = (int64_t *)malloc(sizeof(int64_t) * (size_t)nL);
#pragma omp for schedule(dynamic, 16)
        for (int64_t r = 0; r < nrows; ++r) {
            int64_t id = rows[r];
            if (id < 0 || id >= (int64_t)B * nL * Hq) { bad = 1; continue; }
            int64_t h = id % Hq, t = (id / Hq) % nL, b = id / Hq / nL;
            int64_t hk = h / g;
            int64_t nk = t + 1; /* every mask of Figure 2 is causal: t_k <= t_q */
            for (int64_t tk = 0; tk < nk; ++tk) {
                kpos[tk] = tk;
                koff[tk] = ((b * nL + tk) * Hkv + hk) * d;
            }
            attend_row(q, id * d, k, v, koff, kpos, nk, t, n, mode, W, d, dtype,
                       scale, scores, o + r * d, lse ? lse + r : NULL);
        }
        free(scores); free(kpos); free(koff);
    }
    return bad ? -1 : 0;
}

/* All rows: o [B][nL][Hq][d] (double), lse [B][Hq][nL] (double, may be NULL). */
int oracle_sfa_fwd(const void *q, const void *k, const void *v, int dtype,
                   int B, int L, int n, int Hq, int Hkv, int d, int mode,
                   int64_t W, double scale, double *o, double *lse) {
    const int64_t nL = (int64_t)n * L, total = (int64_t)B * nL * Hq;
    int64_t *rows = (int64_t *)malloc(sizeof(int64_t) * (size_t)total);
    double *lrow = lse ? (double *)malloc(sizeof(double) * (size_t)total) : NULL;
    for (int64_t r = 0; r < total; ++r) rows[r] = r;
    int rc = oracle_sfa_rows(q, k, v, dtype, B, L, n, Hq, Hkv, d, mode, W, scale,
                             rows, total, o, lrow);
    if (rc == 0 && lse) {
        for (int64_t r = 0; r < total; ++r) {  /* [b][t][h] -> [b][h][t] */
            int64_t h = r % Hq, t = (r / Hq) % nL, b = r / Hq / nL;
            lse[(b * Hq + h) * nL + t] = lrow[r];
        }
    }
    free(rows); free(lrow);
    return rc;
}

/* ---------------------------------------------------------------------------
 * Final-stream queries of a KV-mirror layer ("Persistent KV and the KV-mirror
 * Saving": a mirrored layer's K/V come from an earlier layer's hidden states,
 * where every stream was processed, and only the last stream, the supervised
 * one, is run through the mirrored layer).  Its queries are the rows of stream
 * n-1: query i sits at expanded position t = i*n + (n-1) and attends over the
 * K/V of all n*L positions under the layer's own mask (intra: stream n-1
 * only; cross: every position up to t), exactly as that row of the full layer.
 *
 * qf [B][L][Hq][d] (final-stream rows only), k/v [B][n*L][Hkv][d].
 * rows: flat ids into qf, r = (b*L + i)*Hq + h.  Outputs o [nrows][d],
 * lse [nrows].  Returns 0, or -1 on bad arguments.
 * ------------------------------------------------------------------------- */
int oracle_sfa_final_rows(const void *qf, const void *k, const void *v, int dtype,
                          int B, int L, int n, int Hq, int Hkv, int d, int mode,
                          int64_t W, double scale, const int64_t *rows, int64_t nrows,
                          double *o, double *lse) {
    if (B < 1 || L < 1 || n < 1 || Hq < 1 || Hkv < 1 || d < 1 || Hq % Hkv) return -1;
    if (W < 0 || (mode != OR_INTRA && mode != OR_CROSS)) return -1;
    if (scale <= 0.0) scale = 1.0 / sqrt((double)d);
    const int64_t nL = (int64_t)n * L;
    const int g = Hq / Hkv;
    int bad = 0;
#pragma omp parallel
    {
        double *scores = (double *)malloc(sizeof(double) * (size_t)nL);
        int64_t *kpos = (int64_t *)malloc(sizeof(int64_t) * (size_t)nL);
        int64_t *koff = (int64_t *)malloc(sizeof(int64_t) * (size_t)nL);
#pragma omp for schedule(dynamic, 16)
        for (int64_t r = 0; r < nrows; ++r) {
            int64_t id = rows[r];
            if (id < 0 || id >= (int64_t)B * L * Hq) { bad = 1; continue; }
            int64_t h = id % Hq, i = (id / Hq) % L, b = id / Hq / L;
            int64_t kvh = h / g;
            int64_t t = i * n + (n - 1);   /* the final stream's expanded position */
            int64_t nk = t + 1;            /* every mask is causal: t_k <= t */
            for (int64_t tk = 0; tk < nk; ++tk) {
                kpos[tk] = tk;
                koff[tk] = ((b * nL + tk) * Hkv + kvh) * d;
            }
            attend_row(qf, id * d, k, v, koff, kpos, nk, t, n, mode, W, d, dtype,
                       scale, scores, o + r * d, lse ? lse + r : NULL);
        }
        free(scores); free(kpos); free(koff);
    }
    return bad ? -1 : 0;
}

/* All final-stream rows: o [B][L][Hq][d] (double), lse [B][Hq][L] (may be NULL). */
int oracle_sfa_final(const void *qf, const void *k, const void *v, int dtype,
                     int B, int L, int n, int Hq, int Hkv, int d, int mode,
                     int64_t W, double scale, double *o, double *lse) {
    const int64_t total = (int64_t)B * L * Hq;
    int64_t *rows = (int64_t *)malloc(sizeof(int64_t) * (size_t)total);
    double *lrow = lse ? (double *)malloc(sizeof(double) * (size_t)total) : NULL;
    for (int64_t r = 0; r < total; ++r) rows[r] = r;
    int rc = oracle_sfa_final_rows(qf, k, v, dtype, B, L, n, Hq, Hkv, d, mode, W, scale,
                                   rows, total, o, lrow);
    if (rc == 0 && lse) {
        for (int64_t r = 0; r < total; ++r) {  /* [b][i][h] -> [b][h][i] */
            int64_t h = r % Hq, i = (r / Hq) % L, b = r / Hq / L;
            lse[(b * Hq + h) * L + i] = lrow[r];
        }
    }
    free(rows); free(lrow);
    return rc;
}

/* ---------------------------------------------------------------------------
 * Decode step over the retained per-stream KV cache ("Persistent KV ...",
 * "Inference Throughput").  For each sequence b with len = cache_len[b] tokens
 * already cached, the new token's n stream keys/values are appended at token
 * len, and the n stream queries sit at expanded positions len*n + s.  Each
 * query attends, under the layer's mask, over K' = cache[0:len] ++ new.
 *
 * q [B][n][Hq][d]; k_new/v_new [B][n][Hkv][d]; caches [B][T_cap][n][Hkv][d];
 * o [B][n][Hq][d] (double).  Requires len < T_cap.  Returns 0 or -1.
 * ------------------------------------------------------------------------- */
int oracle_sfa_decode(const void *q, const void *k_new, const void *v_new,
                      const void *k_cache, const void *v_cache, int dtype,
                      const int32_t *cache_len, int T_cap, int B, int n, int Hq,
                      int Hkv, int d, int mode, int64_t W, double scale, double *o) {
    if (B < 1 || n < 1 || Hq < 1 || Hkv < 1 || d < 1 || Hq % Hkv || T_cap < 1) return -1;
    if (W < 0 || (mode != OR_INTRA && mode != OR_CROSS)) return -1;
    for (int b = 0; b < B; ++b)
        if (cache_len[b] < 0 || cache_len[b] >= T_cap) return -1;
    if (scale <= 0.0) scale = 1.0 / sqrt((double)d);
    const int g = Hq / Hkv;
    const int64_t esz = dtype == OR_F32 ? 4 : 2;
    /* Assemble K' and V' per (b, kv head) as contiguous [(len+1)*n][d] copies,
     * then reuse the prefill row routine on them with Hkv = 1. */
    int bad = 0;
    for (int b = 0; b < B && !bad; ++b) {
        const int64_t len = cache_len[b], npos = (len + 1) * n;
        for (int hk = 0; hk < Hkv; ++hk) {
            char *kk = (char *)malloc((size_t)(npos * d * esz));
            char *vv = (char *)malloc((size_t)(npos * d * esz));
            for (int64_t t = 0; t < npos; ++t) {
                int64_t tok = t / n, s = t % n;
                const char *ks, *vs;
                if (tok < len) {
                    int64_t off = ((((int64_t)b * T_cap + tok) * n + s) * Hkv + hk) * d * esz;
                    ks = (const char *)k_cache + off; vs = (const char *)v_cache + off;
                } else {
                    int64_t off = ((((int64_t)b * n) + s) * Hkv + hk) * d * esz;
                    ks = (const char *)k_new + off; vs = (const char *)v_new + off;
                }
                memcpy(kk + t * d * esz, ks, (size_t)(d * esz));
                memcpy(vv + t * d * esz, vs, (size_t)(d * esz));
            }
            /* Queries of this kv group: heads hk*g .. hk*g+g-1, streams 0..n-1,
             * copied into a [npos][g][d] query array (only the last n rows used). */
            char *qq = (char *)calloc((size_t)(npos * g * d), (size_t)esz);
            for (int s = 0; s < n; ++s)
                for (int hh = 0; hh < g; ++hh) {
                    int64_t src = ((((int64_t)b * n) + s) * Hq + hk * g + hh) * d * esz;
                    int64_t dst = ((len * n + s) * g + hh) * d * esz;
                    memcpy(qq + dst, (const char *)q + src, (size_t)(d * esz));
                }
            int64_t *rows = (int64_t *)malloc(sizeof(int64_t) * (size_t)(n * g));
            double *orow = (double *)malloc(sizeof(double) * (size_t)(n * g * d));
            for (int s = 0; s < n; ++s)
                for (int hh = 0; hh < g; ++hh) rows[s * g + hh] = (len * n + s) * g + hh;
            int rc = oracle_sfa_rows(qq, kk, vv, dtype, 1, (int)(len + 1), n, g, 1, d,
                                     mode, W, scale, rows, (int64_t)n * g, orow, NULL);
            if (rc) bad = 1;
            for (int s = 0; s < n && !rc; ++s)
                for (int hh = 0; hh < g; ++hh)
                    memcpy(o + ((((int64_t)b * n) + s) * Hq + hk * g + hh) * d,
                           orow + ((int64_t)s * g + hh) * d, sizeof(double) * (size_t)d);
            free(kk); free(vv); free(qq); free(rows); free(orow);
            if (bad) break;
        }
    }
    return bad ? -1 : 0;
}

/* Decode append: cache[b][cache_len[b]][s][h][:] = new[b][s][h][:], bytewise. */
int oracle_decode_append(const void *x_new, void *cache, const int32_t *cache_len,
                         int T_cap, int B, int n, int Hkv, int d, int64_t elem_bytes) {
    const int64_t row = (int64_t)n * Hkv * d * elem_bytes;
    for (int b = 0; b < B; ++b) {
        if (cache_len[b] < 0 || cache_len[b] >= T_cap) return -1;
        memcpy((char *)cache + ((int64_t)b * T_cap + cache_len[b]) * row,
               (const char *)x_new + (int64_t)b * row, (size_t)row);
    }
    return 0;
}

/* ---------------------------------------------------------------------------
 * Backward of the prefill attention: the gradient of the scalar
 * sum_{b,t,h,c} dO[b][t][h][c] * O[b][t][h][c] with respect to Q, K and V,
 * written out from the definition of O above by the chain rule.  For a query
 * row (b, t, h) with visible keys j (Figure 2's mask), softmax weights
 * p_j = exp(scale * q.k_j - lse) and D = dO . O:
 *   dP_j  = dO . v_j
 *   dS_j  = p_j * (dP_j - D)                 (softmax Jacobian applied to dP)
 *   dQ   += scale * sum_j dS_j k_j
 *   dK_j += scale * dS_j q         (summed over the query heads of the group)
 *   dV_j += p_j dO                 (summed over the query heads of the group)
 * The pages define the forward only; this derivative is the textbook one of
 * that forward (nothing is approximated).
 *
 * lse and Drow ([B][Hq][nL], double) are the forward's softmax normaliser and
 * dO . O of every query row (from oracle_sfa_fwd).  qrows selects flat query
 * rows (b*nL + t)*Hq + h for dq [nq][d]; krows selects flat key rows
 * (b*nL + t)*Hkv + hk for dk, dv [nk][d].  Keys and queries are visited in
 * ascending position order; every sum is in double.  Returns 0 or -1.
 * ------------------------------------------------------------------------- */
int oracle_sfa_bwd_rows(const void *q, const void *k, const void *v, const void *dout, int dtype,
                        int B, int L, int n, int Hq, int Hkv, int d, int mode, int64_t W,
                        double scale, const double *lse, const double *Drow,
                        const int64_t *qrows, int64_t nq, double *dq,
                        const int64_t *krows, int64_t nk, double *dk, double *dv) {
    if (B < 1 || L < 1 || n < 1 || Hq < 1 || Hkv < 1 || d < 1 || Hq % Hkv) return -1;
    if (W < 0 || (mode != OR_INTRA && mode != OR_CROSS)) return -1;
    if (scale <= 0.0) scale = 1.0 / sqrt((double)d);
    const int64_t nL = (int64_t)n * L;
    const int g = Hq / Hkv;
    int bad = 0;
    /* dQ rows */
#pragma omp parallel for schedule(dynamic, 8)
    for (int64_t r = 0; r < nq; ++r) {
        int64_t id = qrows[r];
        if (id < 0 || id >= (int64_t)B * nL * Hq) { bad = 1; continue; }
        int64_t h = id % Hq, t = (id / Hq) % nL, b = id / Hq / nL, hk = h / g;
        double lse_t = lse[(b * Hq + h) * nL + t], D_t = Drow[(b * Hq + h) * nL + t];
        double *out = dq + r * d;
        for (int c = 0; c < d; ++c) out[c] = 0.0;
        for (int64_t tk = 0; tk <= t; ++tk) {
            if (!oracle_visible(t, tk, n, mode, W)) continue;
            int64_t koff = ((b * nL + tk) * Hkv + hk) * d;
            double s = 0.0, dp = 0.0;
            for (int c = 0; c < d; ++c) {
                s += load_elem(q, dtype, id * d + c) * load_elem(k, dtype, koff + c);
                dp += load_elem(dout, dtype, id * d + c) * load_elem(v, dtype, koff + c);
            }
            double p = exp(scale * s - lse_t);
            double ds = p * (dp - D_t);
            for (int c = 0; c < d; ++c) out[c] += scale * ds * load_elem(k, dtype, koff + c);
        }
    }
    /* dK, dV rows */
#pragma omp parallel for schedule(dynamic, 8)
    for (int64_t r = 0; r < nk; ++r) {
        int64_t id = krows[r];
        if (id < 0 || id >= (int64_t)B * nL * Hkv) { bad = 1; continue; }
        int64_t hk = id % Hkv, tk = (id / Hkv) % nL, b = id / Hkv / nL;
        double *gk = dk + r * d, *gv = dv + r * d;
        for (int c = 0; c < d; ++c) gk[c] = gv[c] = 0.0;
        for (int hh = 0; hh < g; ++hh) {
            int64_t h = hk * g + hh;
            for (int64_t t = tk; t < nL; ++t) {
                if (!oracle_visible(t, tk, n, mode, W)) continue;
                int64_t qoff = ((b * nL + t) * Hq + h) * d;
                double lse_t = lse[(b * Hq + h) * nL + t], D_t = Drow[(b * Hq + h) * nL + t];
                double s = 0.0, dp = 0.0;
                for (int c = 0; c < d; ++c) {
                    s += load_elem(q, dtype, qoff + c) * load_elem(k, dtype, id * d + c);
                    dp += load_elem(dout, dtype, qoff + c) * load_elem(v, dtype, id * d + c);
                }
                double p = exp(scale * s - lse_t);
                double ds = p * (dp - D_t);
                for (int c = 0; c < d; ++c) {
                    gk[c] += scale * ds * load_elem(q, dtype, qoff + c);
                    gv[c] += p * load_elem(dout, dtype, qoff + c);
                }
            }
        }
    }
    return bad ? -1 : 0;
}

/* ---------------------------------------------------------------------------
 * Backward of the final-stream queries (oracle_sfa_final): the gradient of
 * sum dOf * Of with respect to qf, k and v.  The same chain rule as above,
 * with the query rows restricted to the final stream: query i sits at
 * t = i*n + (n-1); a key row receives gradient only from the final-stream
 * queries that see it (every expanded position's K/V, of every stream, can).
 *
 * lse and Drow are [B][Hq][L] (double) for the final rows.  qrows index qf
 * ((b*L + i)*Hq + h) for dq [nq][d]; krows index k ((b*nL + t)*Hkv + hk) for
 * dk, dv [nk][d].  Returns 0 or -1.
 * ------------------------------------------------------------------------- */
int oracle_sfa_final_bwd_rows(const void *qf, const void *k, const void *v, const void *doutf, int dtype,
                              int B, int L, int n, int Hq, int Hkv, int d, int mode, int64_t W,
                              double scale, const double *lse, const double *Drow,
                              const int64_t *qrows, int64_t nq, double *dq,
                              const int64_t *krows, int64_t nk, double *dk, double *dv) {
    if (B < 1 || L < 1 || n < 1 || Hq < 1 || Hkv < 1 || d < 1 || Hq % Hkv) return -1;
    if (W < 0 || (mode != OR_INTRA && mode != OR_CROSS)) return -1;
    if (scale <= 0.0) scale = 1.0 / sqrt((double)d);
    const int64_t nL = (int64_t)n * L;
    const int g = Hq / Hkv;
    int bad = 0;
    /* dq of final-stream rows */
#pragma omp parallel for schedule(dynamic, 8)
    for (int64_t r = 0; r < nq; ++r) {
        int64_t id = qrows[r];
        if (id < 0 || id >= (int64_t)B * L * Hq) { bad = 1; continue; }
        int64_t h = id % Hq, i = (id / Hq) % L, b = id / Hq / L, kvh = h / g;
        int64_t tq = i * n + (n - 1);
        double lse_i = lse[(b * Hq + h) * L + i], D_i = Drow[(b * Hq + h) * L + i];
        double *gq = dq + r * d;
        for (int c = 0; c < d; ++c) gq[c] = 0.0;
        for (int64_t tk = 0; tk <= tq; ++tk) {
            if (!oracle_visible(tq, tk, n, mode, W)) continue;
            int64_t koff = ((b * nL + tk) * Hkv + kvh) * d;
            double s = 0.0, dp = 0.0;
            for (int c = 0; c < d; ++c) {
                s += load_elem(qf, dtype, id * d + c) * load_elem(k, dtype, koff + c);
                dp += load_elem(doutf, dtype, id * d + c) * load_elem(v, dtype, koff + c);
            }
            double p = exp(scale * s - lse_i);
            double ds = p * (dp - D_i);
            for (int c = 0; c < d; ++c) gq[c] += scale * ds * load_elem(k, dtype, koff + c);
        }
    }
    /* dk, dv of every key row, from the final-stream queries that see it */
#pragma omp parallel for schedule(dynamic, 8)
    for (int64_t r = 0; r < nk; ++r) {
        int64_t id = krows[r];
        if (id < 0 || id >= (int64_t)B * nL * Hkv) { bad = 1; continue; }
        int64_t kvh = id % Hkv, tk = (id / Hkv) % nL, b = id / Hkv / nL;
        double *gk = dk + r * d, *gv = dv + r * d;
        for (int c = 0; c < d; ++c) gk[c] = gv[c] = 0.0;
        for (int hh = 0; hh < g; ++hh) {
            int64_t h = kvh * g + hh;
            for (int64_t i = 0; i < L; ++i) {
                int64_t tq = i * n + (n - 1);
                if (tq < tk || !oracle_visible(tq, tk, n, mode, W)) continue;
                int64_t qoff = ((b * L + i) * Hq + h) * d;
                double lse_i = lse[(b * Hq + h) * L + i], D_i = Drow[(b * Hq + h) * L + i];
                double s = 0.0, dp = 0.0;
                for (int c = 0; c < d; ++c) {
                    s += load_elem(qf, dtype, qoff + c) * load_elem(k, dtype, id * d + c);
                    dp += load_elem(doutf, dtype, qoff + c) * load_elem(v, dtype, id * d + c);
                }
                double p = exp(scale * s - lse_i);
                double ds = p * (dp - D_i);
                for (int c = 0; c < d; ++c) {
                    gk[c] += scale * ds * load_elem(qf, dtype, qoff + c);
                    gv[c] += p * load_elem(doutf, dtype, qoff + c);
                }
            }
        }
    }
    return bad ? -1 : 0;
}

/* ---------------------------------------------------------------------------
 * Rotary position embedding at the expanded positions.  "Hidden Decoding at
 * Scale", "Multi-Stream Expansion and Training Objective": the expanded
 * sequence S_1 .. S_nL is fed to the Transformer with contiguous RoPE
 * positions, so the position of S_t is t (the expanded index), not the token
 * index i(t).  The pages do not restate RoPE itself; the reading taken is the
 * common "rotate half" form: with h = d/2 and frequency
 * f_c = theta^(-2c/d) for c in [0, h),
 *   out[c]     = x[c]     cos(t f_c) - x[c + h] sin(t f_c)
 *   out[c + h] = x[c + h] cos(t f_c) + x[c]     sin(t f_c)
 * x [B][T][H][d] (float32 or bf16 bits); out [B][T][H][d] double.  The
 * position of row (b, t) is t*t_mul + t_add + pos_mul * pos_base[b]
 * (pos_base may be NULL): a prefill passes NULL with t_mul = 1, t_add = 0; the
 * final-stream rows of a KV-mirror layer (row i is expanded position
 * i*n + n-1) pass t_mul = n, t_add = n-1; a decode step passes the cached
 * token counts with pos_mul = n, so stream s of the new token sits at
 * len*n + s (t_add = n-1 for the final stream's row alone).
 * Returns 0 or -1.
 * ------------------------------------------------------------------------- */
int oracle_rope(const void *x, int dtype, int B, int T, int H, int d, const int32_t *pos_base,
                int64_t pos_mul, int64_t t_mul, int64_t t_add, double theta, double *out) {
    if (B < 1 || T < 1 || H < 1 || d < 2 || d % 2 || theta <= 0.0 || pos_mul < 0 || t_mul < 0 || t_add < 0)
        return -1;
    const int h = d / 2;
    for (int64_t b = 0; b < B; ++b)
        for (int64_t t = 0; t < T; ++t) {
            const double pos = (double)(t * t_mul + t_add) +
                               (pos_base ? (double)pos_mul * (double)pos_base[b] : 0.0);
            for (int64_t hh = 0; hh < H; ++hh) {
                const int64_t row = ((b * T + t) * H + hh) * d;
                for (int c = 0; c < h; ++c) {
                    const double f = pow(theta, -2.0 * c / d);
                    const double a = pos * f, co = cos(a), si = sin(a);
                    const double x0 = load_elem(x, dtype, row + c), x1 = load_elem(x, dtype, row + c + h);
                    out[row + c] = x0 * co - x1 * si;
                    out[row + c + h] = x1 * co + x0 * si;
                }
            }
        }
    return 0;
}
