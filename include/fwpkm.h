/*
 * fwpkm.h -- C ABI of the MI355X (gfx950) hot path of the Fast-weight Product
 * Key Memory (FwPKM) layer.
 *
 * The layer ("Fast-weight Product Key Memory", Zhao & Jones, arXiv 2601.00671)
 * keeps a value matrix V with N = n*n rows and two sub-key codebooks K1, K2
 * of n rows each as fast weights.  Per token it reads V sparsely through a
 * product-key search and, after every chunk of C tokens, writes V and the
 * codebooks by one gradient step on chunk-local losses.
 *
 * Citations name the pages the method is taken from:
 *   [digest]     paper.rainbus.top digest of the paper, "Method step details"
 *                (steps 1-5) and "Prerequisites: product key memory";
 *   [layer]      paperlayer.ai section summary of the paper (v2), by section;
 *   [gist-es]    gist.science/es technical summary, "Memoria esparsa".
 *
 * Conventions for every entry point:
 *   - All tensor pointers are DEVICE pointers (HIP device memory), row-major,
 *     densely packed in the layouts given below.  The caller owns every
 *     buffer; the library never allocates, frees or synchronises.
 *   - `stream` is a hipStream_t (NULL = the default stream).  Work is only
 *     enqueued: outputs are valid once the stream reaches this point.
 *   - "store dtype" is cfg->store: FWPKM_F32 (float) or FWPKM_BF16
 *     (bfloat16 bit patterns, 2 bytes).  Arithmetic is fp32 throughout;
 *     state written back to bf16 is rounded to nearest even.
 *   - Return value: FWPKM_OK or a negative fwpkm_status.  Every argument is
 *     validated before anything is enqueued; on error nothing is enqueued
 *     and fwpkm_last_error() describes the problem.  FWPKM_EHIP means a HIP
 *     launch reported an error; device faults surface at the caller's next
 *     synchronisation on `stream`.
 *   - B == 0 or a token count of 0 is a successful no-op.
 *   - Calls on one stream are ordered; concurrent calls that share state
 *     buffers or a workspace on different streams race.
 *
 * Limits of this GPU path (the method itself allows any size; a call
 * outside them returns FWPKM_EUNSUPPORTED before anything is enqueued):
 *
 *   quantity          method              this GPU path
 *   n (N = n*n)       n >= 1, n*n < 2^31  16 <= n <= 1024, n % 16 == 0
 *   d_q / 2           >= 1                32, 64, 128 or 256
 *   d_v               >= 1                64, 128, 256 or 512
 *   k' (k_half)       1 <= k' <= n        k' <= 64
 *   k                 1 <= k <= k'^2      k <= 64; at most 256 pairs (a+1)(b+1) <= k
 *   heads * k         any                 <= 256
 *   B * tokens * heads * k of one call    < 2^31
 *
 * A caller with another d_q can zero-pad: query halves and sub-keys padded
 * with zeros to the next supported d_q / 2 leave every distance ||q - K||^2
 * and every dot product unchanged, and the key step leaves the padded
 * sub-key columns at zero, so the padded layer computes the same values.
 * Value columns can be padded the same way only with znorm = 0 (the
 * z-score's mean and variance run over all d_v columns).
 *
 * Debug overrides (tests, sweeps and profiling).  Read at every call, and
 * only while the environment variable FWPKM_DEBUG is "1"; none changes a
 * result beyond the order of a float sum, and none is needed in use:
 *   FWPKM_SINGLE_STREAM=1        fwpkm_forward_seq keeps every kernel on the
 *                                caller's stream (the same bits);
 *   FWPKM_SCORE_PATH=sweep|rows  pins the scoring path (the same selection;
 *                                usage statistics summed in another order);
 *   FWPKM_KGRAD_SPLIT=<s>        fixes the key step's token split (at most 8);
 *   FWPKM_DECODE=unfused         decode's selection and value read as two
 *                                launches (the same bits).
 */
#ifndef FWPKM_H
#define FWPKM_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define FWPKM_ABI_VERSION 3

typedef enum { FWPKM_F32 = 0, FWPKM_BF16 = 1 } fwpkm_dtype;

/* Sub-key scoring (fwpkm_cfg.score). */
typedef enum { FWPKM_SCORE_IDW = 0, FWPKM_SCORE_DOT = 1 } fwpkm_score;

typedef enum {
    FWPKM_OK = 0,
    FWPKM_EINVAL = -1,      /* bad shape, value or NULL pointer */
    FWPKM_EUNSUPPORTED = -2,/* valid for the method, outside this GPU path's limits */
    FWPKM_EWORKSPACE = -3,  /* workspace NULL or smaller than fwpkm_workspace_bytes() */
    FWPKM_EHIP = -4         /* a HIP call failed */
} fwpkm_status;

/*
 * Layer configuration.
 *   n        sub-keys per codebook; N = n*n value slots ([digest] prerequisites:
 *            keys factorised into two smaller key matrices; [gist-es]: N ~ 10^6).
 *            GPU limits: 16 <= n <= 1024, n % 16 == 0.
 *   heads    H query heads.  Each head has its own query slice and its own
 *            K1, K2; all heads read and write the one shared V, and the
 *            retrieved value is the mean over heads ([layer] D.1, D.3: more
 *            heads raise slot collisions).
 *   d_q      per-head query dimension; the first d_q/2 dims are scored
 *            against K1, the last d_q/2 against K2 ([digest] prerequisites).
 *            GPU limit: d_q/2 in {32, 64, 128, 256}.
 *   d_v      value dimension.  GPU limit: d_v in {64, 128, 256, 512}.
 *   k_half   k': sub-keys kept per half, 1 <= k' <= min(n, 64).
 *   k        final top-k, 1 <= k <= min(k'*k', 64), and the number of
 *            candidate pairs (a, b) with (a+1)(b+1) <= k must be <= 256
 *            (true for every k <= 59; k = 64 with k' = 64 needs about 300
 *            and is refused with FWPKM_EUNSUPPORTED).  heads * k <= 256.
 *            k <= k' makes the search exact over all N slots.
 *   chunk    C: tokens per fast-weight write (fwpkm_forward_seq only).
 *   store    fwpkm_dtype of q, v, targets, K1, K2, V.
 *   idw_eps  eps of the inverse-distance score s = -log(eps + ||q-k||^2)
 *            ([layer] A.2; the constant is not given on the pages).  > 0.
 *   lr_v     step size of the V write ([digest] step 4 uses 1).
 *   lr_k     step size of the K1/K2 write (not given on the pages).
 *   lookahead 1: token t is paired with v_{t+1} ([layer] A.1, default);
 *            0: with v_t ([digest] step 4 as printed).
 *   znorm    1: z-score each target over d_v ([layer] A.3).
 *   znorm_eps variance epsilon of the z-score.
 *   use_addr 1: apply the addressing step to K1, K2 ([digest] step 5).
 *   gate_weight 1: the memorisation error of token t is weighted by its gate
 *            g_t ([layer] A.5); 0: unweighted (the ablation of [layer] D).
 *   score    FWPKM_SCORE_IDW: s = -log(eps + ||q_half - K_i||^2) ([layer] A.2);
 *            FWPKM_SCORE_DOT: s = q_half . K_i, product-key memory's own
 *            scoring ([layer] 2.2; the ablation of A.2 and D.1).  The score
 *            drives the top-k' and top-k (pair score s1 + s2), the weights
 *            (softmax of the k pair scores) and the addressing distribution
 *            p_t = softmax(s_t); the key step uses ds/dK_i = q_t.
 */
typedef struct {
    int32_t n;
    int32_t heads;
    int32_t d_q;
    int32_t d_v;
    int32_t k_half;
    int32_t k;
    int32_t chunk;
    int32_t store;
    float idw_eps;
    float lr_v;
    float lr_k;
    int32_t lookahead;
    int32_t znorm;
    float znorm_eps;
    int32_t use_addr;
    int32_t gate_weight;
    int32_t score;
} fwpkm_cfg;

/* FWPKM_ABI_VERSION of the loaded library. */
int32_t fwpkm_abi_version(void);

/* Message for the last non-OK status returned on the calling thread
 * (thread-local; "" when none).  Never NULL. */
const char* fwpkm_last_error(void);

/*
 * Workspace size in bytes that makes any of fwpkm_retrieve(B, T),
 * fwpkm_chunk_update(B, Tc <= T) and fwpkm_forward_seq(B, T) valid for this
 * configuration.  Writes *bytes and returns FWPKM_OK, or an error status if
 * cfg, B or T is invalid.  The workspace is caller-owned device memory with
 * at least 256-byte alignment; its contents need no initialisation and are
 * not meaningful after a call.
 */
int fwpkm_workspace_bytes(const fwpkm_cfg* cfg, int32_t B, int32_t T, size_t* bytes);

/*
 * Sparse retrieval and gated output of T tokens against frozen state
 * ([digest] steps 2-3; [layer] 2.2, 3.2, A.2):
 *   per head h: split q into halves, score every sub-key of each half with
 *   s = -log(eps + ||q_half - K_i||^2), keep the top-k' of each half (ties:
 *   lower sub-key index), score the k'*k' pairs s1 + s2 with slot id
 *   i*n + j, keep the top-k pairs (ties: lower slot id) in order of
 *   decreasing score, weights w = softmax of their scores;
 *   vhat_t = (1/H) sum_h sum_j w[h][j] V[idx[h][j]];
 *   o_t = g_t * vhat_t + (1 - g_t) * v_t.
 * Inputs:  q[B][T][H][d_q], v[B][T][d_v], K1, K2[B][H][n][d_q/2],
 *          V[B][n*n][d_v] (store dtype); g[B][T] float, post-sigmoid gate.
 * Outputs: o[B][T][d_v] float (required); vhat[B][T][d_v] float,
 *          idx[B][T][H][k] int32, w[B][T][H][k] float (each nullable).
 * State is not modified.
 */
int fwpkm_retrieve(const fwpkm_cfg* cfg, int32_t B, int32_t T,
                   const void* q, const void* v, const float* g,
                   const void* K1, const void* K2, const void* V,
                   float* o, float* vhat, int32_t* idx, float* w,
                   void* ws, size_t ws_bytes, void* stream);

/*
 * One chunk's fast-weight write, given that chunk's retrieval results
 * ([digest] steps 4-5; [layer] 3.3, 3.4, A.1, A.3-A.5):
 *   memorisation (V): tokens t < n_tgt have raw targets tgt[b][t];
 *     y_t = z-score(tgt_t) if znorm, r_t = g_t (vhat_t - y_t);
 *     G_i = sum over reads (t, h, j) of row i, t < n_tgt, of (w/H) r_t;
 *     N_read,i = number of such reads; rows with N_read,i > 0 get
 *     V_i <- V_i - lr_v G_i / N_read,i; other rows are not touched.
 *     The sum runs in a fixed order (no float atomics): results are
 *     bitwise reproducible.
 *   addressing (K1, K2), if use_addr: over all Tc tokens, per head and
 *     half, p_t = softmax over all n sub-keys of s_t, pbar = mean_t p_t,
 *     one step of lr_k on L = -H(pbar_1) - H(pbar_2).  pbar is summed in
 *     tiles of 64 to 256 tokens picked from B, H, Tc and the device's
 *     compute-unit count, so K is reproducible bit for bit for one shape
 *     on one kind of device, and agrees to rounding across shapes.
 * Inputs:  q[B][Tc][H][d_q], tgt[B][n_tgt][d_v] (store dtype; may be NULL
 *          when n_tgt == 0), g[B][Tc] float, idx[B][Tc][H][k] int32 and
 *          w[B][Tc][H][k] float and vhat[B][Tc][d_v] float as returned by
 *          fwpkm_retrieve for this chunk with this state.
 *          Slot ids must lie in [0, n*n) (checked on the device: an
 *          out-of-range id is skipped, never dereferenced).
 * In/out:  K1, K2, V updated in place.
 * Output:  n_read[B][n*n] int32 (nullable): N_read of every row.
 * 0 <= n_tgt <= Tc.
 */
int fwpkm_chunk_update(const fwpkm_cfg* cfg, int32_t B, int32_t Tc, int32_t n_tgt,
                       const void* q, const float* g, const void* tgt,
                       const int32_t* idx, const float* w, const float* vhat,
                       void* K1, void* K2, void* V, int32_t* n_read,
                       void* ws, size_t ws_bytes, void* stream);

/*
 * Gradient of fwpkm_retrieve's output o with respect to q, v and g, for the
 * upstream gradient dO[B][T][d_v] float, with the slot selection idx and the
 * state (K1, K2, V) those outputs were retrieved with held fixed (the top-k
 * selection is piecewise constant; the fast weights are given, not trained
 * by this gradient).  With G = dO_t, per token:
 *   dg_t = G . (vhat_t - v_t),  dv_t = (1 - g_t) G,
 *   a_j = (g_t/H) G . V[idx_j],  dS_j = w_j (a_j - sum_{l in head} w_l a_l),
 *   dq_half = sum_j dS_j * (-2) (q_half - K_half[sub_j]) / (eps + ||q_half - K_half[sub_j]||^2)
 * (S_j = -log(eps + d1) - log(eps + d2) is the pair score of [layer] A.2,
 * w = softmax(S) over the head's k slots).
 * Inputs:  q, v, g, K1, K2, V as for fwpkm_retrieve; idx[B][T][H][k] int32
 *          and w[B][T][H][k] float as returned by it for this state.
 * Outputs: dq[B][T][H][d_q], dv[B][T][d_v], dg[B][T], all float.
 */
int fwpkm_retrieve_backward(const fwpkm_cfg* cfg, int32_t B, int32_t T,
                            const void* q, const void* v, const float* g,
                            const void* K1, const void* K2, const void* V,
                            const int32_t* idx, const float* w, const float* dO,
                            float* dq, float* dv, float* dg, void* stream);

/*
 * Whole sequences: chunks of C tokens in causal order, each read with the
 * state left by the previous chunk and then written ([layer] 3, 3.1), the
 * whole input repeated `passes` times with state carried (iterative
 * memorisation, [layer] 4.3).  Lookahead targets pair token t with v_{t+1};
 * the last token pairs with v_next when given, else it has no target.
 * Inputs:  q[B][T][H][d_q], v[B][T][d_v], v_next[B][d_v] (nullable)
 *          (store dtype); g[B][T] float.
 * In/out:  K1, K2, V.
 * Outputs: o[B][T][d_v] float (required), vhat[B][T][d_v] float
 *          (nullable), both from the last pass.
 * passes >= 1.
 * Streams: the key path of each chunk (scoring, selection, usage
 * statistics, key step) is enqueued on `stream`, the value path (sort of
 * the reads, then gather and value write as two half-batch launches each)
 * on a value stream.  On the sweep scoring path, a chunk with fewer than
 * 2^19 reads (B * tokens * heads * k) runs its selection and sort on a
 * third, selection stream instead, and when half a batch is under 4
 * sequences its gather and write are one launch each.  The library creates
 * both streams (default priority) and seven events on the first such call
 * per host thread and device of `stream`, on that device, and keeps them
 * until fwpkm_release_streams() on that thread (or the end of the
 * process); events fork them from and join them back to `stream`, so when
 * `stream` reaches the end of this call everything is done.  While kernel
 * timing is on (fwpkm_timing_enable), or under the debug override
 * FWPKM_SINGLE_STREAM, everything stays on `stream`: the same kernels, one
 * at a time, and no stream or event of the library is used.  The results
 * are the same bits either way.
 */
int fwpkm_forward_seq(const fwpkm_cfg* cfg, int32_t B, int32_t T, int32_t passes,
                      const void* q, const void* v, const float* g, const void* v_next,
                      void* K1, void* K2, void* V,
                      float* o, float* vhat,
                      void* ws, size_t ws_bytes, void* stream);

/*
 * fwpkm_forward_seq for callers that cannot allocate device memory (code
 * under HIP graph capture, tight serving loops, hosts that forbid
 * allocation): the same computation, the same arguments without the
 * workspace, the same results bit for bit.  Its scratch is a fixed device
 * array of FWPKM_STATIC_SCRATCH_BYTES inside the library, one per GPU it
 * runs on (the device of `stream`), held until the process ends; the
 * call allocates and frees nothing and creates no stream or event: every
 * kernel runs on `stream`, one at a time (the single-stream schedule).
 * Returns FWPKM_EWORKSPACE, before enqueueing anything, when the call would
 * need more scratch than that (fwpkm_workspace_bytes(cfg, B, min(T, C))
 * bounds what it needs), and FWPKM_EINVAL while kernel timing is on.
 * Every call on one GPU shares that GPU's scratch and leaves its contents
 * behind: calls that overlap on one GPU (on different streams, or from
 * different threads) race; calls ordered on one stream do not.  The scratch
 * needs no initialisation.  Capturing fwpkm calls into a HIP graph is not
 * supported: on the test GPU, replays of a captured call of one chunk
 * reproduced the eager results, replays of a captured call of several
 * chunks did not (the cause is not established); enqueue the calls on a
 * stream.
 */
#define FWPKM_STATIC_SCRATCH_BYTES ((size_t)512 << 20)
int fwpkm_forward_seq_static(const fwpkm_cfg* cfg, int32_t B, int32_t T, int32_t passes,
                             const void* q, const void* v, const float* g, const void* v_next,
                             void* K1, void* K2, void* V,
                             float* o, float* vhat, void* stream);

/*
 * Gradients of fwpkm_forward_seq's output o (of its last pass) with respect to
 * q, v and g, for the upstream gradient dO[B][T][d_v] float, by replay: call
 * it with the state (K1, K2, V) that fwpkm_forward_seq started from.  It runs
 * the same chunks in the same order (one kernel at a time on `stream`), so it
 * rewrites the state exactly as the forward did and, when o is given,
 * reproduces o bit for bit; each chunk of the last pass also gets
 * fwpkm_retrieve_backward's gradient against the state that chunk was read
 * with, before that chunk's write.  The fast-weight writes themselves are not
 * differentiated (each chunk's state is taken as given).
 * Outputs: dq[B][T][H][d_q], dv[B][T][d_v], dg[B][T] float (required);
 *          o[B][T][d_v] float (nullable).
 */
int fwpkm_forward_seq_backward(const fwpkm_cfg* cfg, int32_t B, int32_t T, int32_t passes,
                               const void* q, const void* v, const float* g, const void* v_next,
                               void* K1, void* K2, void* V,
                               const float* dO, float* dq, float* dv, float* dg, float* o,
                               void* ws, size_t ws_bytes, void* stream);

/*
 * fwpkm_forward_seq that also counts row contributions for the addressing
 * metrics ([layer] D.3): usage[B][n*n] int32 (nullable; caller-owned,
 * zero it to start an interval) gets +1 per read (t, h, j) of its row, for
 * every token of every pass.  Everything else is fwpkm_forward_seq.
 */
int fwpkm_forward_seq_usage(const fwpkm_cfg* cfg, int32_t B, int32_t T, int32_t passes,
                            const void* q, const void* v, const float* g, const void* v_next,
                            void* K1, void* K2, void* V,
                            float* o, float* vhat, int32_t* usage,
                            void* ws, size_t ws_bytes, void* stream);

/*
 * Addressing metrics ([layer] D.3) of the row contributions c_i = usage[b][i]
 * counted over an interval of tokens, per sequence b, into metrics[B][4]
 * (double, device):
 *   [0] coverage  = |{i : c_i > 0}| / N            (share of rows read)
 *   [1] collision = sum_{c_i > 1} c_i / sum_i c_i   (share of reads that land
 *                   on a row read more than once in the interval)
 *   [2] KLD       = sum_i u_i ln(u_i N), u_i = c_i / sum_i c_i  (divergence of
 *                   row use from uniform, natural log)
 *   [3] sum_i c_i (reads counted).
 * An interval with no reads gives zeros.  reset != 0 zeroes usage afterwards,
 * starting the next interval.  Fixed reduction order: reproducible.
 * ws: device scratch of at least 2048*B bytes, 256-byte aligned.
 */
int fwpkm_usage_metrics(const fwpkm_cfg* cfg, int32_t B, int32_t* usage, double* metrics, int32_t reset,
                        void* ws, size_t ws_bytes, void* stream);

/*
 * Streaming (inference) mode ([layer] A.1: lookahead pairs are collected
 * until a chunk is full, so a token's prediction never waits for its own
 * target; [layer] E.1: memory state carried across sequence boundaries).
 *
 * B sequences decode in lockstep, T >= 1 new tokens per call.  Each token
 * is read against the state left by the last completed chunk write and
 * joins the pending chunk.  With lookahead, the chunk of C pending tokens
 * is written when the token after it arrives (that token's v is the last
 * target), before that token is read; without lookahead it is written as
 * soon as it is full.  fwpkm_stream_flush ends the sequences: it writes the
 * pending tokens (the last one pairs with v_next, or has no target).  The
 * outputs and the state after every call are those of fwpkm_forward_seq
 * over the same tokens (one pass), whatever the split into calls.
 *
 * state: caller-owned device memory of fwpkm_stream_state_bytes() bytes,
 *   256-byte aligned: the sub-key norms and the pending chunk (q, g,
 *   targets, slot ids, weights and vhat of up to C tokens per sequence).
 *   Needs no initialisation; keep it for the life of the stream.
 * pos: HOST memory, read and updated at enqueue time.  pending = tokens in
 *   the pending chunk (0 to start a stream); norms_valid = 0 makes the next
 *   call recompute the sub-key norms (set it to 0 to start, and whenever
 *   the caller itself changes K1 or K2).
 * ws: at least fwpkm_workspace_bytes(cfg, B, cfg->chunk) bytes.
 * Calls of one stream must be enqueued in order on one HIP stream.  After
 * an FWPKM_EHIP error the stream's state is undefined.
 */
typedef struct {
    int32_t pending;
    int32_t norms_valid;
} fwpkm_stream_pos;

/* Bytes of the streaming state for B sequences. */
int fwpkm_stream_state_bytes(const fwpkm_cfg* cfg, int32_t B, size_t* bytes);

/*
 * T new tokens of B sequences: q[B][T][H][d_q], v[B][T][d_v] (store dtype),
 * g[B][T] float.  Outputs o[B][T][d_v] float (required), vhat[B][T][d_v]
 * float (nullable).  K1, K2, V are updated in place by every chunk write
 * the call triggers.  usage[B][n*n] int32 (nullable) counts the reads of
 * the call's tokens, as in fwpkm_forward_seq_usage.
 */
int fwpkm_stream_step(const fwpkm_cfg* cfg, int32_t B, int32_t T,
                      const void* q, const void* v, const float* g,
                      void* K1, void* K2, void* V,
                      float* o, float* vhat, int32_t* usage,
                      void* state, fwpkm_stream_pos* pos,
                      void* ws, size_t ws_bytes, void* stream);

/*
 * End of the B sequences: writes the pending tokens, if any.  v_next[B][d_v]
 * (store dtype, nullable) is the value after the last token, its lookahead
 * target.  Leaves pos->pending = 0; the state carries into the next
 * sequences.
 */
int fwpkm_stream_flush(const fwpkm_cfg* cfg, int32_t B, const void* v_next,
                       void* K1, void* K2, void* V,
                       void* state, fwpkm_stream_pos* pos,
                       void* ws, size_t ws_bytes, void* stream);

/*
 * Destroys the value and selection streams and events that
 * fwpkm_forward_seq created for the calling host thread (on every device),
 * after waiting for the work enqueued on them; the next multi-stream call
 * on the thread creates new ones.  For hosts that run the layer from
 * short-lived threads.  Returns FWPKM_OK (also when there is nothing to
 * release) or FWPKM_EHIP.
 */
int fwpkm_release_streams(void);

/*
 * Kernel timing (observability; not part of the method).  Kernel families
 * of the entry points above, for fwpkm_timing_read.
 */
typedef enum {
    FWPKM_K_KNORM = 0,          /* sub-key norms at the start of a call            */
    FWPKM_K_SWEEP_SELECT = 1,   /* scoring: top-k' candidate lists (+ usage sums)   */
    FWPKM_K_GATHER = 2,         /* value-row gather, gated output, residual        */
    FWPKM_K_RESID = 3,          /* residual of fwpkm_chunk_update                  */
    FWPKM_K_SORT = 4,           /* radix sort of the read list (all passes)        */
    FWPKM_K_SCATTER = 5,        /* read-count-normalised value-row write           */
    FWPKM_K_PBAR = 6,           /* usage partials from stored scores (row path)    */
    FWPKM_K_SWEEP_STATS = 7,    /* usage sums of fwpkm_chunk_update                */
    FWPKM_K_SWEEP_ROWSTAT = 8,  /* row statistic of the entropy gradient           */
    FWPKM_K_KGRAD = 9,          /* sub-key gradient step                           */
    FWPKM_K_FILL = 10,          /* zero fill of n_read                             */
    FWPKM_K_SELECT = 11,        /* per-half top-k', product top-k, weights         */
    FWPKM_K_QT = 12,            /* transposed query halves (rescoring statistic)   */
    FWPKM_K_PEND = 13,          /* copies into a stream's pending chunk            */
    FWPKM_K_USAGE = 14,         /* row-contribution counts and addressing metrics  */
    FWPKM_K_BACKWARD = 15,      /* gradient of the retrieval output                */
    FWPKM_K_COUNT = 16
} fwpkm_kernel;

/*
 * on != 0: from now on every kernel family launch of the calling process is
 * bracketed by a pair of HIP events recorded on the launch's stream, and the
 * accumulated totals are reset.  on == 0 stops recording (totals are kept).
 * While it is on, fwpkm_forward_seq runs one kernel at a time on the caller's
 * stream, so each recorded duration is that kernel's own.  Recording adds
 * two event records per launch; leave it off when timing a whole call.  Not
 * thread-safe against concurrent entry-point calls.
 */
int fwpkm_timing_enable(int32_t on);

/*
 * Waits for every recorded event, then writes the summed elapsed time in
 * milliseconds and the number of timed launches of family `kernel` since the
 * last fwpkm_timing_enable(1).
 */
int fwpkm_timing_read(int32_t kernel, double* total_ms, int64_t* launches);

#ifdef __cplusplus
}
#endif

#endif /* FWPKM_H */
