/*
 * oracle.c — CPU fp64 reference for one context-parallel rank's exact
 * attention. TEST INFRASTRUCTURE ONLY (see oracle.h): the product library never
 * links or calls it, and it shares no code with the GPU path.
 *
 * What it computes is the plain definition of causal softmax attention by
 * global token position. The blockwise method on the FCP page
 * ("从固定环到自由拓扑：FCP到底在解决什么", §3.3) is stated there to reach
 * exactly this result for any order of KV blocks, and §4.2 of the same page asks
 * that the sharded forward be validated against single-card full attention;
 * so the reference is full attention itself, not the blockwise algorithm.
 */
#include "oracle.h"

#include <math.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

/* ---- positions --------------------------------------------------------- */

/* One sequence [base, base+len) split for rank `rank` of `cp`.
 * CONTIGUOUS: the rank's slice [rank*len/cp, (rank+1)*len/cp) — the PCP page,
 *   §3.5 (split by equal contiguous slices, positions stay global).
 * ZIGZAG: 2*cp equal chunks; the rank owns chunk `rank` and chunk
 *   2*cp-1-rank, in ascending order — the zig-zag page, §4.2 (every GPU gets a
 *   mix of early and late tokens; the chunked reading is the one under which
 *   that balance is exact).
 * STRIPED: tokens t with t mod cp == rank — the literal example on the same
 *   page (GPU 0 holds 0,4,8,…; GPU 1 holds 1,5,9,… for four GPUs). */
static int64_t split_one(int64_t base, int64_t len, int32_t cp, int32_t rank, int32_t layout,
                         int32_t *out_pos, int32_t *out_start) {
    int64_t n = 0;
    if (layout == ORACLE_CONTIGUOUS) {
        if (len % cp) return -1;
        int64_t per = len / cp;
        for (int64_t t = 0; t < per; ++t) out_pos[n++] = (int32_t)(base + rank * per + t);
    } else if (layout == ORACLE_ZIGZAG) {
        if (len % (2 * cp)) return -1;
        int64_t c = len / (2 * cp);
        int64_t first = rank, second = 2 * cp - 1 - rank;
        for (int64_t t = 0; t < c; ++t) out_pos[n++] = (int32_t)(base + first * c + t);
        for (int64_t t = 0; t < c; ++t) out_pos[n++] = (int32_t)(base + second * c + t);
    } else if (layout == ORACLE_STRIPED) {
        if (len % cp) return -1;
        for (int64_t t = rank; t < len; t += cp) out_pos[n++] = (int32_t)(base + t);
    } else {
        return -1;
    }
    if (out_start)
        for (int64_t t = 0; t < n; ++t) out_start[t] = (int32_t)base;
    return n;
}

int64_t oracle_local_positions(int64_t S, int32_t cp, int32_t rank, int32_t layout,
                               const int64_t *doc_lens, int32_t n_docs,
                               int32_t *out_pos, int32_t *out_start) {
    if (cp < 1 || rank < 0 || rank >= cp || S < 0) return -1;
    if (!doc_lens) return split_one(0, S, cp, rank, layout, out_pos, out_start);
    int64_t base = 0, n = 0;
    for (int32_t t = 0; t < n_docs; ++t) {
        int64_t m = split_one(base, doc_lens[t], cp, rank, layout, out_pos + n,
                              out_start ? out_start + n : NULL);
        if (m < 0) return -1;
        n += m;
        base += doc_lens[t];
    }
    if (base != S) return -1;
    return n;
}

/* ---- input widening ---------------------------------------------------- */

/* bf16 is the top half of an IEEE float32, so widening is exact. */
static double load_value(const void *base, int32_t in_dtype, int64_t idx) {
    if (in_dtype == ORACLE_IN_F32) return (double)((const float *)base)[idx];
    uint32_t bits = (uint32_t)((const uint16_t *)base)[idx] << 16;
    float f;
    memcpy(&f, &bits, sizeof f);
    return (double)f;
}

static int key_visible(int32_t causal, int32_t qp, const int32_t *q_start, int64_t i, int32_t kp) {
    if (!causal) return 1;
    if (kp > qp) return 0;                       /* only earlier (or the same) tokens */
    if (q_start && kp < q_start[i]) return 0;    /* other documents are invisible */
    return 1;
}

/* Scores s_j = scale * <q_i,h , k_j,g> for every key; non-visible keys get
 * -inf. Returns the number of visible keys and writes their maximum to *m. */
static int64_t score_row(const void *q, const void *k, int32_t in_dtype,
                         int64_t lk, int32_t hq, int32_t hkv, int32_t d,
                         const int32_t *q_pos, const int32_t *q_start, const int32_t *k_pos,
                         int32_t causal, double scale, int64_t i, int32_t h,
                         double *qrow, double *s, double *m) {
    int32_t group = hq / hkv;
    int32_t g = h / group;   /* consecutive query heads share one KV head */
    for (int32_t t = 0; t < d; ++t) qrow[t] = load_value(q, in_dtype, (i * hq + h) * (int64_t)d + t);
    int64_t count = 0;
    double mx = -INFINITY;
    for (int64_t j = 0; j < lk; ++j) {
        if (!key_visible(causal, q_pos ? q_pos[i] : 0, q_start, i, k_pos ? k_pos[j] : 0)) {
            s[j] = -INFINITY;
            continue;
        }
        double acc = 0.0;
        for (int32_t t = 0; t < d; ++t)
            acc += qrow[t] * load_value(k, in_dtype, (j * hkv + g) * (int64_t)d + t);
        s[j] = scale * acc;
        if (s[j] > mx) mx = s[j];
        ++count;
    }
    *m = mx;
    return count;
}

int oracle_attention(const void *q, const void *k, const void *v, int32_t in_dtype,
                     int64_t lq, int64_t lk, int32_t hq, int32_t hkv, int32_t d,
                     const int32_t *q_pos, const int32_t *q_start, const int32_t *k_pos,
                     int32_t causal, double scale,
                     const int64_t *rows, const int32_t *heads, int64_t n_pairs,
                     double *o, double *lse, int64_t *n_visible, int32_t n_threads) {
    if (!q || !k || !v || !o || !lse || hq < 1 || hkv < 1 || hq % hkv || d < 1 || lq < 0 || lk < 0)
        return -1;
    if (causal && (!q_pos || !k_pos)) return -1;
    if ((rows == NULL) != (heads == NULL)) return -1;
    if (!rows) n_pairs = lq * hq;
#ifdef _OPENMP
    if (n_threads > 0) omp_set_num_threads(n_threads);
#else
    (void)n_threads;
#endif
    int failed = 0;
#pragma omp parallel
    {
        double *s = (double *)malloc(sizeof(double) * (size_t)(lk > 0 ? lk : 1));
        double *qrow = (double *)malloc(sizeof(double) * (size_t)d);
        if (!s || !qrow) {
#pragma omp atomic write
            failed = 1;
        }
#pragma omp for schedule(dynamic, 4)
        for (int64_t n = 0; n < n_pairs; ++n) {
            if (!s || !qrow) continue;
            int64_t i = rows ? rows[n] : n / hq;
            int32_t h = heads ? heads[n] : (int32_t)(n % hq);
            double *on = o + n * d;
            if (i < 0 || i >= lq || h < 0 || h >= hq) {
#pragma omp atomic write
                failed = 1;
                continue;
            }
            /* pass 1: scores and their maximum */
            double m;
            int64_t count = score_row(q, k, in_dtype, lk, hq, hkv, d, q_pos, q_start, k_pos,
                                      causal, scale, i, h, qrow, s, &m);
            if (n_visible) n_visible[n] = count;
            for (int32_t t = 0; t < d; ++t) on[t] = 0.0;
            if (count == 0) {            /* no key: empty sum */
                lse[n] = -INFINITY;
                continue;
            }
            /* pass 2: normaliser l = sum_j exp(s_j - m) */
            double l = 0.0;
            for (int64_t j = 0; j < lk; ++j)
                if (s[j] != -INFINITY) l += exp(s[j] - m);
            /* pass 3: O = sum_j exp(s_j - m) v_j / l */
            int32_t g = h / (hq / hkv);
            for (int64_t j = 0; j < lk; ++j) {
                if (s[j] == -INFINITY) continue;
                double w = exp(s[j] - m);
                for (int32_t t = 0; t < d; ++t)
                    on[t] += w * load_value(v, in_dtype, (j * hkv + g) * (int64_t)d + t);
            }
            for (int32_t t = 0; t < d; ++t) on[t] /= l;
            lse[n] = m + log(l);
        }
        free(s);
        free(qrow);
    }
    return failed ? -1 : 0;
}

int64_t oracle_softmax_row(const void *q, const void *k, int32_t in_dtype,
                           int64_t lq, int64_t lk, int32_t hq, int32_t hkv, int32_t d,
                           const int32_t *q_pos, const int32_t *q_start, const int32_t *k_pos,
                           int32_t causal, double scale, int64_t row, int32_t head, double *p) {
    if (!q || !k || !p || row < 0 || row >= lq || head < 0 || head >= hq || hq % hkv) return -1;
    double *qrow = (double *)malloc(sizeof(double) * (size_t)d);
    if (!qrow) return -1;
    double m;
    int64_t count = score_row(q, k, in_dtype, lk, hq, hkv, d, q_pos, q_start, k_pos,
                              causal, scale, row, head, qrow, p, &m);
    free(qrow);
    if (count == 0) {
        for (int64_t j = 0; j < lk; ++j) p[j] = 0.0;
        return 0;
    }
    double l = 0.0;
    for (int64_t j = 0; j < lk; ++j)
        if (p[j] != -INFINITY) l += exp(p[j] - m);
    for (int64_t j = 0; j < lk; ++j) p[j] = (p[j] == -INFINITY) ? 0.0 : exp(p[j] - m) / l;
    return count;
}

/* ---- merge of two partial results ------------------------------------- */

/* Two partials over disjoint key sets combine exactly: each partial's
 * normaliser is e^LSE, so the union's normaliser is their sum, and each
 * partial's output is weighted by its share of it. This is the same identity
 * as the global max / global sum normaliser on the PCP page (§4.2), applied to
 * two shards at a time; the FCP page (§3.3) relies on it to accept blocks in
 * any order. */
void oracle_merge(int64_t n_rows, int32_t d,
                  const double *o_a, const double *lse_a,
                  const double *o_b, const double *lse_b,
                  double *o_out, double *lse_out) {
    for (int64_t n = 0; n < n_rows; ++n) {
        double la = lse_a[n], lb = lse_b[n];
        double wa, wb, L;
        if (la == -INFINITY && lb == -INFINITY) {
            wa = 0.0;
            wb = 0.0;
            L = -INFINITY;
        } else {
            double mx = la > lb ? la : lb;
            L = mx + log(exp(la - mx) + exp(lb - mx));
            wa = exp(la - L);
            wb = exp(lb - L);
        }
        for (int32_t t = 0; t < d; ++t)
            o_out[n * d + t] = wa * o_a[n * d + t] + wb * o_b[n * d + t];
        lse_out[n] = L;
    }
}

/* ---- gradients of the attention above --------------------------------- */

/* The backward pass that training-time context parallelism runs after the
 * forward (PCP page §2.3: the backward exchanges the same blocks again; Halo
 * page, Ulysses section: heads stay independent). For a loss with gradient dO
 * with respect to O, everything follows from the definition
 *     O_i = sum_j P_ij v_j,  P_ij = exp(s_ij) / sum_j' exp(s_ij'),  s_ij = scale <q_i, k_j>
 * over the keys visible to row i:
 *     dV_j  = sum_i P_ij dO_i
 *     dP_ij = <dO_i, v_j>
 *     dS_ij = P_ij (dP_ij - D_i),  D_i = sum_j P_ij dP_ij = <dO_i, O_i>
 *     dQ_i  = scale sum_j dS_ij k_j,   dK_j = scale sum_i dS_ij q_i
 * where the sums for dK and dV also run over every query head that reads the
 * key's KV head. A row with no visible key contributes nothing.
 *
 * Pass 1 (per (row, head) pair): scores, max, normaliser, O_i, D_i, dQ_i.
 * Pass 2 (per (key, KV head)): dK_j and dV_j from every visible (row, head),
 * with P recomputed from the row's normaliser. */
int oracle_attention_grad(const void *q, const void *k, const void *v, int32_t in_dtype,
                          int64_t lq, int64_t lk, int32_t hq, int32_t hkv, int32_t d,
                          const int32_t *q_pos, const int32_t *q_start, const int32_t *k_pos,
                          int32_t causal, double scale, const double *dout,
                          const int64_t *rows, const int32_t *heads, int64_t n_pairs,
                          double *dq, double *dk, double *dv, double *delta, int32_t n_threads) {
    if (!q || !k || !v || !dout || hq < 1 || hkv < 1 || hq % hkv || d < 1 || lq < 0 || lk < 0) return -1;
    if (causal && (!q_pos || !k_pos)) return -1;
    if ((rows == NULL) != (heads == NULL)) return -1;
    if (rows && (dk || dv)) return -1;          /* key gradients need every row */
    if (!rows) n_pairs = lq * hq;
#ifdef _OPENMP
    if (n_threads > 0) omp_set_num_threads(n_threads);
#else
    (void)n_threads;
#endif
    /* per pair: ln of the normaliser (m + ln l) and D, kept for pass 2 */
    double *lse = (double *)malloc(sizeof(double) * (size_t)(n_pairs > 0 ? n_pairs : 1));
    double *dd = (double *)malloc(sizeof(double) * (size_t)(n_pairs > 0 ? n_pairs : 1));
    if (!lse || !dd) {
        free(lse);
        free(dd);
        return -1;
    }
    int failed = 0;
#pragma omp parallel
    {
        double *s = (double *)malloc(sizeof(double) * (size_t)(lk > 0 ? lk : 1));
        double *qrow = (double *)malloc(sizeof(double) * (size_t)d);
        double *orow = (double *)malloc(sizeof(double) * (size_t)d);
        if (!s || !qrow || !orow) {
#pragma omp atomic write
            failed = 1;
        }
#pragma omp for schedule(dynamic, 4)
        for (int64_t n = 0; n < n_pairs; ++n) {
            if (!s || !qrow || !orow) continue;
            int64_t i = rows ? rows[n] : n / hq;
            int32_t h = heads ? heads[n] : (int32_t)(n % hq);
            if (i < 0 || i >= lq || h < 0 || h >= hq) {
#pragma omp atomic write
                failed = 1;
                continue;
            }
            int32_t g = h / (hq / hkv);
            const double *dorow = dout + (i * hq + h) * (int64_t)d;
            double m;
            int64_t count = score_row(q, k, in_dtype, lk, hq, hkv, d, q_pos, q_start, k_pos,
                                      causal, scale, i, h, qrow, s, &m);
            if (dq)
                for (int32_t t = 0; t < d; ++t) dq[n * d + t] = 0.0;
            if (count == 0) {            /* sees nothing: no gradient flows through this row */
                lse[n] = -INFINITY;
                dd[n] = 0.0;
                if (delta) delta[n] = 0.0;
                continue;
            }
            double z = 0.0;              /* the row's normaliser, relative to its max */
            for (int64_t j = 0; j < lk; ++j)
                if (s[j] != -INFINITY) z += exp(s[j] - m);
            /* O_i and D_i = <dO_i, O_i> */
            for (int32_t t = 0; t < d; ++t) orow[t] = 0.0;
            for (int64_t j = 0; j < lk; ++j) {
                if (s[j] == -INFINITY) continue;
                double p = exp(s[j] - m) / z;
                int64_t kv = (j * hkv + g) * (int64_t)d;   /* row j of KV head g */
                for (int32_t t = 0; t < d; ++t) orow[t] += p * load_value(v, in_dtype, kv + t);
            }
            double di = 0.0;
            for (int32_t t = 0; t < d; ++t) di += dorow[t] * orow[t];
            lse[n] = m + log(z);
            dd[n] = di;
            if (delta) delta[n] = di;
            if (!dq) continue;
            /* dQ_i = scale sum_j P_ij (<dO_i, v_j> - D_i) k_j */
            for (int64_t j = 0; j < lk; ++j) {
                if (s[j] == -INFINITY) continue;
                double p = exp(s[j] - m) / z;
                int64_t kv = (j * hkv + g) * (int64_t)d;
                double dp = 0.0;
                for (int32_t t = 0; t < d; ++t) dp += dorow[t] * load_value(v, in_dtype, kv + t);
                double ds = p * (dp - di);
                for (int32_t t = 0; t < d; ++t) dq[n * d + t] += scale * ds * load_value(k, in_dtype, kv + t);
            }
        }
        free(s);
        free(qrow);
        free(orow);
    }
    if (!failed && (dk || dv)) {
        int32_t group = hq / hkv;
#pragma omp parallel for schedule(dynamic, 4)
        for (int64_t jg = 0; jg < lk * hkv; ++jg) {
            int64_t j = jg / hkv;
            int32_t g = (int32_t)(jg % hkv);
            double *dkj = dk ? dk + jg * d : NULL;
            double *dvj = dv ? dv + jg * d : NULL;
            for (int32_t t = 0; t < d; ++t) {
                if (dkj) dkj[t] = 0.0;
                if (dvj) dvj[t] = 0.0;
            }
            for (int32_t h = g * group; h < (g + 1) * group; ++h) {
                for (int64_t i = 0; i < lq; ++i) {
                    if (!key_visible(causal, q_pos ? q_pos[i] : 0, q_start, i, k_pos ? k_pos[j] : 0)) continue;
                    int64_t n = i * hq + h;
                    if (lse[n] == -INFINITY) continue;
                    double acc = 0.0, dp = 0.0;
                    const double *dorow = dout + n * (int64_t)d;
                    for (int32_t t = 0; t < d; ++t) {
                        acc += load_value(q, in_dtype, n * (int64_t)d + t) * load_value(k, in_dtype, jg * d + t);
                        dp += dorow[t] * load_value(v, in_dtype, jg * d + t);
                    }
                    double p = exp(scale * acc - lse[n]);
                    double ds = p * (dp - dd[n]);
                    for (int32_t t = 0; t < d; ++t) {
                        if (dkj) dkj[t] += scale * ds * load_value(q, in_dtype, n * (int64_t)d + t);
                        if (dvj) dvj[t] += p * dorow[t];
                    }
                }
            }
        }
    }
    free(lse);
    free(dd);
    return failed ? -1 : 0;
}
