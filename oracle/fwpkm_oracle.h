/*
 * fwpkm_oracle.h -- plain, slow, fp64 CPU oracle of the Fast-weight Product Key
 * Memory (FwPKM) layer's hot path.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the test suite, the smoke check and the
 * benchmark's CPU-baseline leg may load this.  It shares no code, header,
 * table or constant with the HIP library: it is an independent statement of
 * what the layer computes, written from the method's description
 * ("Fast-weight Product Key Memory", Zhao & Jones, arXiv 2601.00671):
 *   - paper.rainbus.top digest, "Method step details": steps 1-5 (input
 *     construction, sparse retrieval, gated residual output, memory update
 *     with read-count aggregation, addressing loss -H(p1)-H(p2));
 *   - paperlayer.ai summary, sections 2.2 (PKM), 3 / 3.1 (chunk causality),
 *     3.3 (read-count consensus), 3.4 (addressing entropy), A.1 (lookahead
 *     targets), A.2 (IDW scoring), A.3 (z-scored targets, no clipping),
 *     A.4 (sum reduction), A.5 (gate-weighted loss).
 *
 * Arithmetic: every input is taken exactly (fp32 or bf16 -> double); all
 * arithmetic is double; fast-weight state is rounded back to its storage
 * type (round-to-nearest-even) after every chunk.
 *
 * Readings where the pages are silent (each one listed in the design notes):
 *   IDW score s = -log(eps + ||q - k||^2) per half; pair score s1 + s2;
 *   slot id = i*n + j; ties -> lower sub-key index / lower slot id; weights
 *   = softmax of the k pair scores; heads share V and v_hat is the head
 *   mean; z-score per token over d_v with population variance; addressing
 *   distribution p_t = softmax(s_t) over all n sub-keys; chunk average over
 *   the chunk's actual token count; plain SGD steps lr_v, lr_k.
 * Variants (paperlayer.ai D, the ablation axes): gate_weight = 0 drops the
 *   gate from the memorisation error (A.5 switched off); score = dot uses
 *   PKM's dot product s = q . k in place of the IDW score for the selection,
 *   the weights and the addressing p, with ds/dk = q in the key step.
 *
 * Parity pins: see tests/test_oracle_pins.py.  The readings listed above
 * that the pages do not fix (IDW form and eps, head mean, z-score axis,
 * addressing p and lr_k) are pinned only to their own definitions: parity
 * with the authors' implementation is unpinned for them.
 */
#ifndef FWPKM_ORACLE_H
#define FWPKM_ORACLE_H
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Storage types for q, v, targets, K1, K2 and V. */
#define FWO_F32 0
#define FWO_BF16 1

typedef struct {
    int32_t n;        /* sub-keys per codebook; N = n*n slots */
    int32_t heads;    /* H */
    int32_t d_q;      /* per-head query dim (even); halves of d_q/2 */
    int32_t d_v;      /* value dim */
    int32_t k_half;   /* k' per half */
    int32_t k;        /* final top-k, k <= k'*k' */
    int32_t chunk;    /* C */
    int32_t store;    /* FWO_F32 / FWO_BF16 */
    double idw_eps;   /* eps in s = -log(eps + d) */
    double lr_v;      /* V step size */
    double lr_k;      /* K1/K2 step size */
    int32_t lookahead;/* 1: target of token t is v_{t+1}; 0: v_t */
    int32_t znorm;    /* 1: z-score each target over d_v */
    double znorm_eps; /* variance epsilon of the z-score */
    int32_t use_addr; /* 1: apply the addressing step to K1, K2 */
    int32_t gate_weight; /* 1: memorisation MSE weighted by the gate g_t; 0: unweighted */
    int32_t score;    /* FWO_SCORE_IDW or FWO_SCORE_DOT */
} fwo_cfg;

/* Sub-key scoring: inverse distance s = -log(eps + ||q - k||^2) (the method),
 * or the plain dot product s = q . k of product-key memory (its ablation). */
#define FWO_SCORE_IDW 0
#define FWO_SCORE_DOT 1

/* Layouts (row-major, all per sequence b of the batch):
 *   q[B][T][H][d_q], v[B][T][d_v], tgt[B][n_tgt][d_v] (store dtype)
 *   g[B][T] float in [0,1] (post-sigmoid gate)
 *   K1, K2[B][H][n][d_q/2], V[B][n*n][d_v]           (store dtype)
 *   o, vhat[B][T][d_v] double
 *   idx[B][T][H][k] int32 slot ids, w[B][T][H][k] double weights,
 *   P[B][T][H][k] double (eps+d1)(eps+d2) of each selected pair,
 *   tie[B][T][H] uint8: 1 when a decision of this (token, head) sits within
 *   relative gap tie_rel of its alternative (see fwo_retrieve).
 * Return 0 on success, -1 on a bad argument.
 */

/* Retrieval of T tokens against frozen state (method step 2 and 3).  Any
 * output pointer except o may be NULL.  tie_rel > 0 enables tie flags. */
int fwo_retrieve(const fwo_cfg* c, int32_t B, int32_t T,
                 const void* q, const void* v, const float* g,
                 const void* K1, const void* K2, const void* V,
                 double* o, double* vhat, int32_t* idx, double* w, double* P,
                 uint8_t* tie, double tie_rel);

/* One chunk's fast-weight write (method steps 4 and 5) given that chunk's
 * retrieval results.  Tokens 0..n_tgt-1 of the chunk have raw targets
 * tgt[b][t] (layout [B][n_tgt][d_v]); the rest have none.  V, K1, K2 are
 * updated in place.
 * n_read[B][n*n] may be NULL; when given it receives the read counts. */
int fwo_chunk_update(const fwo_cfg* c, int32_t B, int32_t Tc, int32_t n_tgt,
                     const void* q, const float* g, const void* tgt,
                     const int32_t* idx, const double* w, const double* vhat,
                     void* K1, void* K2, void* V, int32_t* n_read);

/* Whole sequences, chunk-causal, `passes` times with state carried.
 * v_next[B][d_v] (nullable) is the value after the last token, used as the
 * last token's lookahead target.  o / vhat receive the last pass.
 * chunk_limit > 0 stops after that many chunks of the first pass (a
 * bounded sample for timing); 0 runs everything. */
int fwo_forward_seq(const fwo_cfg* c, int32_t B, int32_t T, int32_t passes,
                    const void* q, const void* v, const float* g,
                    const void* v_next,
                    void* K1, void* K2, void* V,
                    double* o, double* vhat, int32_t chunk_limit);

/* (eps+d1)(eps+d2) in double for arbitrary slots slots[B][T][H][m]
 * against frozen K1, K2 (used to assess near-tie alternatives); with dot
 * scoring exp(-(s1 + s2)), which orders pairs the same way. */
int fwo_pair_p(const fwo_cfg* c, int32_t B, int32_t T, int32_t m,
               const void* q, const void* K1, const void* K2,
               const int32_t* slots, double* P);

/* Exact double -> storage rounding (RNE), exposed for tests. */
uint16_t fwo_double_to_bf16(double x);

/* Number of OpenMP threads the oracle runs with. */
int fwo_num_threads(void);

/* Sets the OpenMP thread count of later calls (n > 0). */
void fwo_set_threads(int n);

#ifdef __cplusplus
}
#endif
#endif
