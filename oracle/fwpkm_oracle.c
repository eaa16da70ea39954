/*
 * fwpkm_oracle.c -- plain fp64 CPU oracle of the FwPKM layer's hot path.
 *
 * TEST INFRASTRUCTURE ONLY (tests, smoke check, benchmark CPU baseline).
 * Independent of the HIP library: no shared code, headers or tables.
 *
 * Written from "Fast-weight Product Key Memory" (Zhao & Jones, arXiv
 * 2601.00671) as summarised on the pages; each function names the passage it
 * follows.  Steps are taken in the pages' order and notation, with no
 * blocking, pruning or fusion: every sub-key is scored, every pair of the
 * two top-k' lists is scored, every list is fully sorted.
 */
#include "fwpkm_oracle.h"

#include <math.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

/* ------------------------------------------------------------------ */
/* storage conversions (exact in, round-to-nearest-even out)            */
/* ------------------------------------------------------------------ */

static double bf16_bits_to_double(uint16_t h) {
    uint32_t u = (uint32_t)h << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return (double)f;
}

/* Round a double to the nearest bf16 (8 significant bits), ties to even,
 * directly from double (no intermediate float rounding). */
uint16_t fwo_double_to_bf16(double x) {
    if (isnan(x)) return 0x7FC0;
    uint16_t sign = signbit(x) ? 0x8000 : 0;
    double ax = fabs(x);
    if (isinf(ax)) return sign | 0x7F80;
    if (ax == 0.0) return sign;
    int e;
    (void)frexp(ax, &e);          /* ax = m * 2^e, m in [0.5, 1) */
    int qexp = e - 8;             /* quantum of an 8-significant-bit value */
    if (qexp < -133) qexp = -133; /* bf16 subnormal quantum is 2^-133 */
    double r = nearbyint(ldexp(ax, -qexp)); /* default mode: ties to even */
    double y = ldexp(r, qexp);
    if (y > 3.3895313892515355e38) return sign | 0x7F80; /* above max bf16 */
    float f = (float)y; /* exact: y has at most 8 significant bits */
    uint32_t u;
    memcpy(&u, &f, sizeof u);
    return sign | (uint16_t)((u >> 16) & 0x7FFF);
}

static double ld(const void* p, size_t i, int store) {
    if (store == FWO_F32) return (double)((const float*)p)[i];
    return bf16_bits_to_double(((const uint16_t*)p)[i]);
}

static void st(void* p, size_t i, int store, double x) {
    if (store == FWO_F32)
        ((float*)p)[i] = (float)x; /* C conversion rounds to nearest even */
    else
        ((uint16_t*)p)[i] = fwo_double_to_bf16(x);
}

int fwo_num_threads(void) {
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}

void fwo_set_threads(int n) {
#ifdef _OPENMP
    if (n > 0) omp_set_num_threads(n);
#else
    (void)n;
#endif
}

/* ------------------------------------------------------------------ */
/* argument checks                                                      */
/* ------------------------------------------------------------------ */

static int cfg_ok(const fwo_cfg* c) {
    if (!c) return 0;
    if (c->n < 1 || c->heads < 1 || c->d_q < 2 || (c->d_q & 1) || c->d_v < 1) return 0;
    if ((int64_t)c->n * c->n > 2147483647LL) return 0;
    if (c->k_half < 1 || c->k_half > c->n) return 0;
    if (c->k < 1 || (int64_t)c->k > (int64_t)c->k_half * c->k_half) return 0;
    if (c->chunk < 1) return 0;
    if (c->store != FWO_F32 && c->store != FWO_BF16) return 0;
    if (!(c->idw_eps > 0.0)) return 0;
    if (c->score != FWO_SCORE_IDW && c->score != FWO_SCORE_DOT) return 0;
    return 1;
}

/* ------------------------------------------------------------------ */
/* retrieval: product-key search with IDW scores                        */
/* ------------------------------------------------------------------ */

typedef struct {
    double s;   /* score, larger is better */
    int32_t id; /* sub-key index or slot id; lower wins ties */
} scored;

/* order: score descending, then id ascending */
static int cmp_scored(const void* a, const void* b) {
    const scored* x = (const scored*)a;
    const scored* y = (const scored*)b;
    if (x->s > y->s) return -1;
    if (x->s < y->s) return 1;
    return (x->id > y->id) - (x->id < y->id);
}

/* Dot product of a query half and one sub-key (product-key memory's own
 * scoring, paperlayer.ai 2.2; the ablation of A.2 / D.1). */
static double dot_qk(const void* q, size_t qoff, const void* K, size_t koff, int dh, int store) {
    double acc = 0.0;
    for (int u = 0; u < dh; ++u) acc += ld(q, qoff + u, store) * ld(K, koff + u, store);
    return acc;
}

/* Squared Euclidean distance between a query half and one sub-key, taken
 * directly as a sum of squared differences (IDW scoring, paperlayer.ai
 * A.2: Euclidean distance replaces the dot product). */
static double sq_dist(const void* q, size_t qoff, const void* K, size_t koff,
                      int dh, int store) {
    double acc = 0.0;
    for (int u = 0; u < dh; ++u) {
        double diff = ld(q, qoff + u, store) - ld(K, koff + u, store);
        acc += diff * diff;
    }
    return acc;
}

/* Per (token, head) result of the product-key search. */
typedef struct {
    int32_t* slot;  /* [k] */
    double* w;      /* [k] */
    double* P;      /* [k] (eps+d1)(eps+d2); dot scoring: exp(-(s1+s2)) */
    double* d1;     /* [n] half 1, kept for addressing: squared distances (IDW) or dot products */
    double* d2;     /* [n] half 2 */
    uint8_t tie;
} pk_result;

/*
 * Product-key retrieval for one token and one head (pages: rainbus digest
 * "prerequisite knowledge: PKM" and method step 2; paperlayer.ai 2.2, A.2).
 *  1. the query is split into two halves (first d_q/2 dims -> K1);
 *  2. each half is scored against every sub-key of its codebook with
 *     s = -log(eps + ||q_half - K_i||^2);
 *  3. the top-k' of each half are kept (score desc, index asc);
 *  4. every pair (a, b) of the two top-k' lists is scored s1[a] + s2[b] and
 *     given slot id a*n + b;
 *  5. the top-k pairs are kept (score desc, slot asc);
 *  6. the weights are the softmax of the k pair scores.
 * scratch must hold 2*n + k_half*k_half scored entries.
 */
static void pk_search(const fwo_cfg* c, const void* qtok, const void* K1h,
                      const void* K2h, pk_result* R, scored* scratch,
                      double tie_rel) {
    const int n = c->n, dh = c->d_q / 2, kh = c->k_half, k = c->k;
    const double eps = c->idw_eps;
    scored* h1 = scratch;
    scored* h2 = scratch + n;
    scored* pr = scratch + 2 * n;

    const int dot = c->score == FWO_SCORE_DOT;
    for (int i = 0; i < n; ++i) {
        if (dot) {
            R->d1[i] = dot_qk(qtok, 0, K1h, (size_t)i * dh, dh, c->store);
            R->d2[i] = dot_qk(qtok, dh, K2h, (size_t)i * dh, dh, c->store);
        } else {
            R->d1[i] = sq_dist(qtok, 0, K1h, (size_t)i * dh, dh, c->store);
            R->d2[i] = sq_dist(qtok, dh, K2h, (size_t)i * dh, dh, c->store);
        }
        h1[i].s = dot ? R->d1[i] : -log(eps + R->d1[i]);
        h1[i].id = i;
        h2[i].s = dot ? R->d2[i] : -log(eps + R->d2[i]);
        h2[i].id = i;
    }
    qsort(h1, (size_t)n, sizeof(scored), cmp_scored);
    qsort(h2, (size_t)n, sizeof(scored), cmp_scored);

    int m = 0;
    for (int a = 0; a < kh; ++a)
        for (int b = 0; b < kh; ++b) {
            pr[m].s = h1[a].s + h2[b].s;
            pr[m].id = h1[a].id * n + h2[b].id;
            ++m;
        }
    qsort(pr, (size_t)m, sizeof(scored), cmp_scored);

    double smax = pr[0].s, z = 0.0;
    for (int j = 0; j < k; ++j) z += exp(pr[j].s - smax);
    for (int j = 0; j < k; ++j) {
        R->slot[j] = pr[j].id;
        R->w[j] = exp(pr[j].s - smax) / z;
        int i1 = pr[j].id / n, i2 = pr[j].id % n;
        R->P[j] = dot ? exp(-pr[j].s) : (eps + R->d1[i1]) * (eps + R->d2[i2]);
    }

    /* Near-tie flag: a decision whose two alternatives differ by less than
     * tie_rel in relative terms of (eps + d) or of the pair product P. */
    R->tie = 0;
    if (tie_rel > 0.0) {
        /* (a) which k' sub-keys of each half are kept */
        if (dot) {
            /* dot scores: a gap below tie_rel of the scores' size */
            if (kh < n) {
                if (h1[kh - 1].s - h1[kh].s <= tie_rel * (fabs(h1[kh - 1].s) + fabs(h1[kh].s)) ||
                    h2[kh - 1].s - h2[kh].s <= tie_rel * (fabs(h2[kh - 1].s) + fabs(h2[kh].s)))
                    R->tie = 1;
            }
            int last = (k < m) ? k : k - 1;
            for (int j = 0; j < last; ++j)
                if (pr[j].s - pr[j + 1].s <= tie_rel * (fabs(pr[j].s) + fabs(pr[j + 1].s))) R->tie = 1;
        } else {
            if (kh < n) {
                double in1 = eps + R->d1[h1[kh - 1].id], out1 = eps + R->d1[h1[kh].id];
                double in2 = eps + R->d2[h2[kh - 1].id], out2 = eps + R->d2[h2[kh].id];
                if (out1 - in1 <= tie_rel * out1 || out2 - in2 <= tie_rel * out2) R->tie = 1;
            }
            /* (b) which k pairs are kept and (c) their order */
            int last = (k < m) ? k : k - 1;
            for (int j = 0; j < last; ++j) {
                int a1 = pr[j].id / n, a2 = pr[j].id % n;
                int b1 = pr[j + 1].id / n, b2 = pr[j + 1].id % n;
                double pa = (eps + R->d1[a1]) * (eps + R->d2[a2]);
                double pb = (eps + R->d1[b1]) * (eps + R->d2[b2]);
                if (pb - pa <= tie_rel * pb) R->tie = 1;
            }
        }
    }
}

int fwo_pair_p(const fwo_cfg* c, int32_t B, int32_t T, int32_t m,
               const void* q, const void* K1, const void* K2,
               const int32_t* slots, double* P) {
    if (!cfg_ok(c) || B < 0 || T < 0 || m < 1 || !q || !K1 || !K2 || !slots || !P) return -1;
    const int n = c->n, H = c->heads, dq = c->d_q, dh = dq / 2;
    const int64_t N = (int64_t)n * n;
    #pragma omp parallel for collapse(2) schedule(static)
    for (int b = 0; b < B; ++b)
        for (int t = 0; t < T; ++t)
            for (int h = 0; h < H; ++h) {
                size_t qoff = (((size_t)b * T + t) * H + h) * dq;
                size_t koff = ((size_t)b * H + h) * n * dh;
                for (int j = 0; j < m; ++j) {
                    size_t o = (((size_t)b * T + t) * H + h) * m + j;
                    int32_t s = slots[o];
                    if (s < 0 || s >= N) { P[o] = NAN; continue; }
                    int i1 = s / n, i2 = s % n;
                    if (c->score == FWO_SCORE_DOT) {
                        /* exp(-(s1 + s2)): decreasing in the pair score, like the IDW product */
                        P[o] = exp(-(dot_qk(q, qoff, K1, koff + (size_t)i1 * dh, dh, c->store) +
                                     dot_qk(q, qoff + dh, K2, koff + (size_t)i2 * dh, dh, c->store)));
                        continue;
                    }
                    double d1 = 0.0, d2 = 0.0;
                    for (int u = 0; u < dh; ++u) {
                        double x = ld(q, qoff + u, c->store) - ld(K1, koff + (size_t)i1 * dh + u, c->store);
                        double y = ld(q, qoff + dh + u, c->store) - ld(K2, koff + (size_t)i2 * dh + u, c->store);
                        d1 += x * x;
                        d2 += y * y;
                    }
                    P[o] = (c->idw_eps + d1) * (c->idw_eps + d2);
                }
            }
    return 0;
}

/*
 * Retrieval + gated output for tokens [t0, t1) of every sequence
 * (rainbus digest method steps 2-3; paperlayer.ai 3.2):
 *   v_hat_t = (1/H) sum_h sum_{i in I^h_t} s'_{t,i} V_i,
 *   o_t = g_t * v_hat_t + (1 - g_t) * v_t.
 * When dist1/dist2 are given they receive the squared distances
 * [b][t - t0][h][n] for the addressing step.
 */
static void retrieve_range(const fwo_cfg* c, int32_t B, int32_t T, int32_t t0, int32_t t1,
                           const void* q, const void* v, const float* g,
                           const void* K1, const void* K2, const void* V,
                           double* o, double* vhat, int32_t* idx, double* w, double* Pout,
                           uint8_t* tie, double tie_rel, double* dist1, double* dist2) {
    const int n = c->n, H = c->heads, dq = c->d_q, dh = dq / 2, dv = c->d_v;
    const int k = c->k, kh = c->k_half;
    const int64_t N = (int64_t)n * n;
    const int nt = t1 - t0;

    #pragma omp parallel
    {
        scored* scratch = (scored*)malloc(sizeof(scored) * (size_t)(2 * n + kh * kh));
        int32_t* slot = (int32_t*)malloc(sizeof(int32_t) * (size_t)k);
        double* ww = (double*)malloc(sizeof(double) * (size_t)k);
        double* PP = (double*)malloc(sizeof(double) * (size_t)k);
        double* d1 = (double*)malloc(sizeof(double) * (size_t)n);
        double* d2 = (double*)malloc(sizeof(double) * (size_t)n);
        double* acc = (double*)malloc(sizeof(double) * (size_t)dv);
        pk_result R = {slot, ww, PP, d1, d2, 0};

        #pragma omp for collapse(2) schedule(dynamic, 4)
        for (int b = 0; b < B; ++b)
            for (int tt = 0; tt < nt; ++tt) {
                const int t = t0 + tt;
                for (int e = 0; e < dv; ++e) acc[e] = 0.0;
                for (int h = 0; h < H; ++h) {
                    const size_t qoff = (((size_t)b * T + t) * H + h) * dq;
                    const size_t koff = ((size_t)b * H + h) * n * dh;
                    const void* qtok = (const char*)q + qoff * (c->store == FWO_F32 ? 4 : 2);
                    const void* K1h = (const char*)K1 + koff * (c->store == FWO_F32 ? 4 : 2);
                    const void* K2h = (const char*)K2 + koff * (c->store == FWO_F32 ? 4 : 2);
                    pk_search(c, qtok, K1h, K2h, &R, scratch, tie_rel);
                    const size_t ooff = (((size_t)b * T + t) * H + h) * k;
                    for (int j = 0; j < k; ++j) {
                        if (idx) idx[ooff + j] = slot[j];
                        if (w) w[ooff + j] = ww[j];
                        if (Pout) Pout[ooff + j] = PP[j];
                        const size_t voff = ((size_t)b * N + slot[j]) * dv;
                        for (int e = 0; e < dv; ++e) acc[e] += ww[j] * ld(V, voff + e, c->store);
                    }
                    if (tie) tie[((size_t)b * T + t) * H + h] = R.tie;
                    if (dist1) {
                        const size_t doff = (((size_t)b * nt + tt) * H + h) * n;
                        memcpy(dist1 + doff, d1, sizeof(double) * (size_t)n);
                        memcpy(dist2 + doff, d2, sizeof(double) * (size_t)n);
                    }
                }
                const double gt = (double)g[(size_t)b * T + t];
                for (int e = 0; e < dv; ++e) {
                    const double vh = acc[e] / H;
                    const double vt = ld(v, ((size_t)b * T + t) * dv + e, c->store);
                    if (vhat) vhat[((size_t)b * T + t) * dv + e] = vh;
                    o[((size_t)b * T + t) * dv + e] = gt * vh + (1.0 - gt) * vt;
                }
            }
        free(scratch); free(slot); free(ww); free(PP); free(d1); free(d2); free(acc);
    }
}

int fwo_retrieve(const fwo_cfg* c, int32_t B, int32_t T,
                 const void* q, const void* v, const float* g,
                 const void* K1, const void* K2, const void* V,
                 double* o, double* vhat, int32_t* idx, double* w, double* P,
                 uint8_t* tie, double tie_rel) {
    if (!cfg_ok(c) || B < 0 || T < 0) return -1;
    if (B == 0 || T == 0) return 0;
    if (!q || !v || !g || !K1 || !K2 || !V || !o) return -1;
    retrieve_range(c, B, T, 0, T, q, v, g, K1, K2, V, o, vhat, idx, w, P, tie, tie_rel,
                   NULL, NULL);
    return 0;
}

/* ------------------------------------------------------------------ */
/* memorisation: gated lookahead reconstruction, read-count consensus   */
/* ------------------------------------------------------------------ */

/*
 * V step of one chunk for one sequence (rainbus digest method step 4;
 * paperlayer.ai 3.3, A.1, A.3, A.4, A.5):
 *   L_mem = 1/2 sum_t g_t ||y_t - v_hat_t||^2   (sum over tokens and
 *   features, no clipping), y_t = z-scored target;
 *   grad_{V_i} L_mem = sum over reads (t,h,j) of row i of (w/H) g_t (v_hat_t - y_t);
 *   grad_agg V_i = grad_{V_i} L_mem / N_read,i;  V_i <- V_i - lr_v grad_agg V_i.
 * tgt_row(t) gives the raw target of token t (t < n_tgt).
 * G_i and N_read,i sum over the reads whose slot id is i, for the rows
 * i in [0, N): a slot id outside [0, N) is the read of no row, so it adds to
 * no G_i and no N_read,i (every retrieval's ids are in range; a list given
 * from outside may not be).
 */
static void memorise_one(const fwo_cfg* c, int32_t Tc, int32_t n_tgt,
                         const float* g_b, const void* tgt_b, size_t tgt_stride_tok,
                         const int32_t* idx_b, const double* w_b, const double* vhat_b,
                         void* V_b, int32_t* nread_b, int32_t* rowmap, int32_t* touched,
                         double* G, int32_t* cnt) {
    const int H = c->heads, k = c->k, dv = c->d_v;
    (void)Tc;
    double* r = (double*)malloc(sizeof(double) * (size_t)dv);
    double* y = (double*)malloc(sizeof(double) * (size_t)dv);
    int nrows = 0;
    for (int t = 0; t < n_tgt; ++t) {
        for (int e = 0; e < dv; ++e) y[e] = ld(tgt_b, (size_t)t * tgt_stride_tok + e, c->store);
        if (c->znorm) {
            double mean = 0.0, var = 0.0;
            for (int e = 0; e < dv; ++e) mean += y[e];
            mean /= dv;
            for (int e = 0; e < dv; ++e) var += (y[e] - mean) * (y[e] - mean);
            var /= dv;
            const double inv = 1.0 / sqrt(var + c->znorm_eps);
            for (int e = 0; e < dv; ++e) y[e] = (y[e] - mean) * inv;
        }
        /* the gate weights the token's reconstruction error (A.5), unless disabled */
        const double gt = c->gate_weight ? (double)g_b[t] : 1.0;
        for (int e = 0; e < dv; ++e) r[e] = gt * (vhat_b[(size_t)t * dv + e] - y[e]);
        for (int h = 0; h < H; ++h)
            for (int j = 0; j < k; ++j) {
                const size_t ent = ((size_t)t * H + h) * k + j;
                const int32_t s = idx_b[ent];
                if (s < 0 || (int64_t)s >= (int64_t)c->n * c->n) continue;
                int32_t row = rowmap[s];
                if (row < 0) {
                    row = nrows++;
                    rowmap[s] = row;
                    touched[row] = s;
                    cnt[row] = 0;
                    for (int e = 0; e < dv; ++e) G[(size_t)row * dv + e] = 0.0;
                }
                const double a = w_b[ent] / H;
                for (int e = 0; e < dv; ++e) G[(size_t)row * dv + e] += a * r[e];
                cnt[row] += 1;
            }
    }
    for (int row = 0; row < nrows; ++row) {
        const int32_t s = touched[row];
        for (int e = 0; e < dv; ++e) {
            const size_t vi = (size_t)s * dv + e;
            const double old = ld(V_b, vi, c->store);
            st(V_b, vi, c->store, old - c->lr_v * G[(size_t)row * dv + e] / cnt[row]);
        }
        if (nread_b) nread_b[s] = cnt[row];
        rowmap[s] = -1;
    }
    free(r);
    free(y);
}

/* ------------------------------------------------------------------ */
/* addressing: entropy of the chunk's marginal sub-key usage            */
/* ------------------------------------------------------------------ */

/*
 * K step of one codebook (one sequence, head and half) for one chunk
 * (rainbus digest method step 5; paperlayer.ai 3.4):
 *   p_t = softmax(s_t) over all n sub-keys, s_{t,i} = -log(eps + d_{t,i})
 *   (or s_{t,i} = q_t . K_i with dot-product scoring, where dist holds the
 *   dot products and ds/dK_i = q_t);
 *   pbar = (1/Tc) sum_t p_t;  L = -H(pbar) = sum_i pbar_i ln pbar_i.
 * Gradient by the chain rule through the softmax and the IDW score:
 *   dL/ds_{t,i} = (1/Tc) p_{t,i} (ln pbar_i - m_t), m_t = sum_l p_{t,l} ln pbar_l;
 *   ds_{t,i}/dK_i = 2 (q_t - K_i) / (eps + d_{t,i});
 *   K_i <- K_i - lr_k sum_t dL/ds_{t,i} ds_{t,i}/dK_i.
 * dist[t*dist_stride + i] = d_{t,i}; qh(t) is the query half of token t.
 */
static void address_one(const fwo_cfg* c, int32_t Tc, const double* dist, size_t dist_stride,
                        const void* q_b, size_t q_stride_tok, size_t q_off,
                        void* Kh, double* p, double* lp, double* m, int inner) {
    /* inner != 0 spreads each loop below over OpenMP threads: every value is
     * still one thread's sum in the order written, so the result does not
     * depend on the thread count */
    const int n = c->n, dh = c->d_q / 2;
    const double eps = c->idw_eps;
    const int dot = c->score == FWO_SCORE_DOT;
    #pragma omp parallel for schedule(static) if(inner)
    for (int t = 0; t < Tc; ++t) {
        const double* d = dist + (size_t)t * dist_stride;
        double smax = -INFINITY;
        for (int i = 0; i < n; ++i) {
            double s = dot ? d[i] : -log(eps + d[i]);
            if (s > smax) smax = s;
        }
        double z = 0.0;
        for (int i = 0; i < n; ++i) z += exp((dot ? d[i] : -log(eps + d[i])) - smax);
        for (int i = 0; i < n; ++i) p[(size_t)t * n + i] = exp((dot ? d[i] : -log(eps + d[i])) - smax) / z;
    }
    #pragma omp parallel for schedule(static) if(inner)
    for (int i = 0; i < n; ++i) {
        double s = 0.0;
        for (int t = 0; t < Tc; ++t) s += p[(size_t)t * n + i];
        lp[i] = log(s / Tc);
    }
    #pragma omp parallel for schedule(static) if(inner)
    for (int t = 0; t < Tc; ++t) {
        double s = 0.0;
        for (int i = 0; i < n; ++i) s += p[(size_t)t * n + i] * lp[i];
        m[t] = s;
    }
    #pragma omp parallel if(inner)
    {
        double* grad = (double*)malloc(sizeof(double) * (size_t)dh);
        #pragma omp for schedule(static)
        for (int i = 0; i < n; ++i) {
            for (int u = 0; u < dh; ++u) grad[u] = 0.0;
            for (int t = 0; t < Tc; ++t) {
                const double dLds = p[(size_t)t * n + i] * (lp[i] - m[t]) / Tc;
                /* ds/dK_i: 2 (q - K_i) / (eps + d) for IDW, q for the dot product */
                const double scale = dot ? 1.0 : 2.0 / (eps + dist[(size_t)t * dist_stride + i]);
                for (int u = 0; u < dh; ++u) {
                    const double qu = ld(q_b, (size_t)t * q_stride_tok + q_off + u, c->store);
                    const double ku = dot ? 0.0 : ld(Kh, (size_t)i * dh + u, c->store);
                    grad[u] += dLds * scale * (qu - ku);
                }
            }
            for (int u = 0; u < dh; ++u) {
                const size_t ki = (size_t)i * dh + u;
                st(Kh, ki, c->store, ld(Kh, ki, c->store) - c->lr_k * grad[u]);
            }
        }
        free(grad);
    }
}

/* ------------------------------------------------------------------ */
/* one chunk's write, given distances from retrieval                     */
/* ------------------------------------------------------------------ */

typedef struct {
    int32_t* rowmap;  /* [B][N], -1 = not touched */
    int32_t* touched; /* [B][Tc*H*k] */
    int32_t* cnt;     /* [B][Tc*H*k] */
    double* G;        /* [B][Tc*H*k][d_v] */
} mem_ws;

static int mem_ws_alloc(mem_ws* m, const fwo_cfg* c, int32_t B, int32_t Tc) {
    const int64_t N = (int64_t)c->n * c->n;
    const size_t ents = (size_t)Tc * c->heads * c->k;
    m->rowmap = (int32_t*)malloc(sizeof(int32_t) * (size_t)B * (size_t)N);
    m->touched = (int32_t*)malloc(sizeof(int32_t) * (size_t)B * ents);
    m->cnt = (int32_t*)malloc(sizeof(int32_t) * (size_t)B * ents);
    m->G = (double*)malloc(sizeof(double) * (size_t)B * ents * (size_t)c->d_v);
    if (!m->rowmap || !m->touched || !m->cnt || !m->G) return -1;
    for (size_t i = 0; i < (size_t)B * (size_t)N; ++i) m->rowmap[i] = -1;
    return 0;
}

static void mem_ws_free(mem_ws* m) {
    free(m->rowmap); free(m->touched); free(m->cnt); free(m->G);
}

/* Steps 4 and 5 for a chunk of Tc tokens of every sequence.  Both steps use
 * the state the chunk was read with; they write disjoint state. */
static void chunk_write(const fwo_cfg* c, int32_t B, int32_t Tc, int32_t n_tgt,
                        const void* q, size_t q_seq_stride, const float* g, size_t g_seq_stride,
                        const void* tgt, size_t tgt_seq_stride,
                        const int32_t* idx, const double* w, const double* vhat,
                        size_t tok_seq_stride,
                        const double* dist1, const double* dist2,
                        void* K1, void* K2, void* V, int32_t* n_read, mem_ws* mw) {
    const int n = c->n, H = c->heads, dq = c->d_q, dh = dq / 2, dv = c->d_v, k = c->k;
    const int64_t N = (int64_t)n * n;
    const size_t ents = (size_t)Tc * H * k;
    const size_t es = (c->store == FWO_F32) ? 4 : 2;

    #pragma omp parallel for schedule(dynamic, 1)
    for (int b = 0; b < B; ++b) {
        memorise_one(c, Tc, n_tgt, g + (size_t)b * g_seq_stride,
                     (const char*)tgt + (size_t)b * tgt_seq_stride * es, (size_t)dv,
                     idx + (size_t)b * tok_seq_stride * H * k, w + (size_t)b * tok_seq_stride * H * k,
                     vhat + (size_t)b * tok_seq_stride * dv,
                     (char*)V + (size_t)b * (size_t)N * dv * es,
                     n_read ? n_read + (size_t)b * (size_t)N : NULL,
                     mw->rowmap + (size_t)b * (size_t)N, mw->touched + (size_t)b * ents,
                     mw->G + (size_t)b * ents * dv, mw->cnt + (size_t)b * ents);
    }

    if (!c->use_addr) return;
    /* one codebook per thread when there are enough of them; otherwise one
     * codebook at a time with its loops spread over the threads (the same
     * arithmetic either way) */
    const int inner = B * H * 2 < fwo_num_threads();
    #pragma omp parallel if(!inner)
    {
        double* p = (double*)malloc(sizeof(double) * (size_t)Tc * n);
        double* lp = (double*)malloc(sizeof(double) * (size_t)n);
        double* m = (double*)malloc(sizeof(double) * (size_t)Tc);
        #pragma omp for collapse(3) schedule(dynamic, 1)
        for (int b = 0; b < B; ++b)
            for (int h = 0; h < H; ++h)
                for (int half = 0; half < 2; ++half) {
                    const double* dist = (half == 0 ? dist1 : dist2) + (((size_t)b * Tc) * H + h) * n;
                    void* Kh = (char*)(half == 0 ? K1 : K2) + (((size_t)b * H + h) * n * dh) * es;
                    address_one(c, Tc, dist, (size_t)H * n,
                                (const char*)q + (size_t)b * q_seq_stride * es, (size_t)H * dq,
                                (size_t)h * dq + (size_t)half * dh, Kh, p, lp, m, inner);
                }
        free(p); free(lp); free(m);
    }
}

int fwo_chunk_update(const fwo_cfg* c, int32_t B, int32_t Tc, int32_t n_tgt,
                     const void* q, const float* g, const void* tgt,
                     const int32_t* idx, const double* w, const double* vhat,
                     void* K1, void* K2, void* V, int32_t* n_read) {
    if (!cfg_ok(c) || B < 0 || Tc < 0 || n_tgt < 0 || n_tgt > Tc) return -1;
    if (B == 0 || Tc == 0) return 0;
    if (!q || !g || !idx || !w || !vhat || !K1 || !K2 || !V) return -1;
    if (n_tgt > 0 && !tgt) return -1;
    const int n = c->n, H = c->heads, dq = c->d_q, dh = dq / 2;
    const int64_t N = (int64_t)n * n;
    if (n_read) memset(n_read, 0, sizeof(int32_t) * (size_t)B * (size_t)N);

    /* distances (or dot products) with the chunk's (pre-update) keys */
    const int dot = c->score == FWO_SCORE_DOT;
    double* dist1 = (double*)malloc(sizeof(double) * (size_t)B * Tc * H * n);
    double* dist2 = (double*)malloc(sizeof(double) * (size_t)B * Tc * H * n);
    if (!dist1 || !dist2) { free(dist1); free(dist2); return -1; }
    #pragma omp parallel for collapse(3) schedule(static)
    for (int b = 0; b < B; ++b)
        for (int t = 0; t < Tc; ++t)
            for (int h = 0; h < H; ++h) {
                const size_t qoff = (((size_t)b * Tc + t) * H + h) * dq;
                const size_t koff = ((size_t)b * H + h) * n * dh;
                const size_t doff = (((size_t)b * Tc + t) * H + h) * n;
                for (int i = 0; i < n; ++i) {
                    if (dot) {
                        dist1[doff + i] = dot_qk(q, qoff, K1, koff + (size_t)i * dh, dh, c->store);
                        dist2[doff + i] = dot_qk(q, qoff + dh, K2, koff + (size_t)i * dh, dh, c->store);
                    } else {
                        dist1[doff + i] = sq_dist(q, qoff, K1, koff + (size_t)i * dh, dh, c->store);
                        dist2[doff + i] = sq_dist(q, qoff + dh, K2, koff + (size_t)i * dh, dh, c->store);
                    }
                }
            }
    mem_ws mw = {NULL, NULL, NULL, NULL};
    if (mem_ws_alloc(&mw, c, B, Tc) != 0) { mem_ws_free(&mw); free(dist1); free(dist2); return -1; }
    chunk_write(c, B, Tc, n_tgt, q, (size_t)Tc * H * dq, g, (size_t)Tc, tgt, (size_t)n_tgt * c->d_v,
                idx, w, vhat, (size_t)Tc, dist1, dist2, K1, K2, V, n_read, &mw);
    mem_ws_free(&mw);
    free(dist1);
    free(dist2);
    return 0;
}

/* ------------------------------------------------------------------ */
/* whole sequence: causal chunks, repeated passes                        */
/* ------------------------------------------------------------------ */

/*
 * Chunk-causal driver (paperlayer.ai 3 and 3.1: predictions in a chunk use
 * the fast weights left by the previous chunk; the write follows the chunk;
 * rainbus digest / paperlayer.ai 4.3: iterative memorisation re-reads the
 * same input with the state carried over).  Lookahead targets (paperlayer.ai
 * A.1): token t is paired with v_{t+1}; the last token of the input pairs
 * with v_next when given, else it has no target.
 */
int fwo_forward_seq(const fwo_cfg* c, int32_t B, int32_t T, int32_t passes,
                    const void* q, const void* v, const float* g,
                    const void* v_next,
                    void* K1, void* K2, void* V,
                    double* o, double* vhat, int32_t chunk_limit) {
    if (!cfg_ok(c) || B < 0 || T < 0 || passes < 1 || chunk_limit < 0) return -1;
    if (B == 0 || T == 0) return 0;
    if (!q || !v || !g || !K1 || !K2 || !V || !o) return -1;
    const int n = c->n, H = c->heads, dq = c->d_q, dv = c->d_v, k = c->k, C = c->chunk;
    const size_t es = (c->store == FWO_F32) ? 4 : 2;
    const int32_t Cmax = (T < C) ? T : C;

    int32_t* idx = (int32_t*)malloc(sizeof(int32_t) * (size_t)B * Cmax * H * k);
    double* w = (double*)malloc(sizeof(double) * (size_t)B * Cmax * H * k);
    double* vh = (double*)malloc(sizeof(double) * (size_t)B * Cmax * dv);
    double* oc = (double*)malloc(sizeof(double) * (size_t)B * Cmax * dv);
    double* dist1 = (double*)malloc(sizeof(double) * (size_t)B * Cmax * H * n);
    double* dist2 = (double*)malloc(sizeof(double) * (size_t)B * Cmax * H * n);
    /* contiguous per-chunk copies of the inputs of every sequence */
    void* qc = malloc(es * (size_t)B * Cmax * H * dq);
    void* vc = malloc(es * (size_t)B * Cmax * dv);
    void* tg = malloc(es * (size_t)B * Cmax * dv);
    float* gc = (float*)malloc(sizeof(float) * (size_t)B * Cmax);
    mem_ws mw = {NULL, NULL, NULL, NULL};
    int rc = 0;
    if (!idx || !w || !vh || !oc || !dist1 || !dist2 || !qc || !vc || !tg || !gc ||
        mem_ws_alloc(&mw, c, B, Cmax) != 0) {
        rc = -1;
        goto done;
    }

    const int32_t nchunks = (T + C - 1) / C;
    int32_t done_chunks = 0;
    for (int32_t pass = 0; pass < passes; ++pass) {
        for (int32_t ci = 0; ci < nchunks; ++ci) {
            if (chunk_limit > 0 && done_chunks >= chunk_limit) goto done;
            const int32_t t0 = ci * C;
            const int32_t Tc = (T - t0 < C) ? T - t0 : C;
            for (int b = 0; b < B; ++b) {
                memcpy((char*)qc + (size_t)b * Tc * H * dq * es,
                       (const char*)q + ((size_t)b * T + t0) * H * dq * es, (size_t)Tc * H * dq * es);
                memcpy((char*)vc + (size_t)b * Tc * dv * es,
                       (const char*)v + ((size_t)b * T + t0) * dv * es, (size_t)Tc * dv * es);
                memcpy(gc + (size_t)b * Tc, g + (size_t)b * T + t0, sizeof(float) * (size_t)Tc);
            }
            /* step 2-3 with the state left by the previous chunk */
            retrieve_range(c, B, Tc, 0, Tc, qc, vc, gc, K1, K2, V, oc, vh, idx, w, NULL, NULL, 0.0,
                           dist1, dist2);
            for (int b = 0; b < B; ++b)
                for (int32_t t = 0; t < Tc; ++t)
                    for (int e = 0; e < dv; ++e) {
                        const size_t src = ((size_t)b * Tc + t) * dv + e;
                        const size_t dst = ((size_t)b * T + t0 + t) * dv + e;
                        o[dst] = oc[src];
                        if (vhat) vhat[dst] = vh[src];
                    }
            /* targets: tokens with a target come first in the chunk */
            int32_t n_tgt;
            if (!c->lookahead) {
                n_tgt = Tc;
                memcpy(tg, vc, es * (size_t)B * Tc * dv);
            } else {
                const int last_has = (t0 + Tc < T) || (v_next != NULL);
                n_tgt = last_has ? Tc : Tc - 1;
                for (int b = 0; b < B; ++b)
                    for (int32_t t = 0; t < n_tgt; ++t) {
                        const void* src = (t0 + t + 1 < T)
                            ? (const char*)v + ((size_t)b * T + t0 + t + 1) * dv * es
                            : (const char*)v_next + (size_t)b * dv * es;
                        memcpy((char*)tg + ((size_t)b * Tc + t) * dv * es, src, (size_t)dv * es);
                    }
            }
            /* steps 4-5 */
            chunk_write(c, B, Tc, n_tgt, qc, (size_t)Tc * H * dq, gc, (size_t)Tc, tg, (size_t)Tc * dv,
                        idx, w, vh, (size_t)Tc, dist1, dist2, K1, K2, V, NULL, &mw);
            ++done_chunks;
        }
    }
done:
    mem_ws_free(&mw);
    free(idx); free(w); free(vh); free(oc); free(dist1); free(dist2);
    free(qc); free(vc); free(tg); free(gc);
    return rc;
}
