/*
 * kvpop.h -- C ABI of libkvpop, the MI355X (gfx950) hot path of KVpop.
 *
 * Method: "KVpop -- Key-Value Cache Compression with Predictive Online
 * Pruning" (arXiv 2607.05061v2), as summarised on paperlayer.ai.  Section
 * names below are that page's.
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 * - Pointers are DEVICE pointers owned by the caller; the library never
 *   allocates, frees, synchronises or keeps a pointer past the call.  Every
 *   call is asynchronous on `stream` (0 = the null stream): buffers must stay
 *   alive until the stream has finished the work.
 * - Layouts are dense and row-major, head-major:
 *     Q   [B][Hq][S][D]   bf16          K, V [B][Hkv][S][D] bf16
 *     LSE [B][Hq][S]      fp32 (natural log)
 *   Query head g reads KV head g / (Hq / Hkv) (grouped-query attention).
 * - bf16 is the raw 16-bit brain-float format; fp32 is IEEE binary32.
 * - Device pointers must be 16-byte aligned (fp32 score/mass/LSE arrays
 *   4-byte aligned).
 * - Errors: all argument checks run on the host before any launch and
 *   return KVPOP_ERR_INVALID_ARGUMENT / KVPOP_ERR_UNSUPPORTED /
 *   KVPOP_ERR_WORKSPACE_TOO_SMALL without touching the GPU.  A failed launch
 *   returns KVPOP_ERR_DEVICE.  Faults during execution surface at the next
 *   stream synchronisation, as for any HIP work.
 * - Calls keep no global state and may be issued concurrently on different
 *   streams with disjoint outputs.
 * - Supported head dims: 64 and 128.  Hq must be a multiple of Hkv and
 *   128 must be a multiple of Hq/Hkv (group sizes 1, 2, 4, ..., 128).
 */
#ifndef KVPOP_H
#define KVPOP_H

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

#define KVPOP_ABI_VERSION 3

typedef enum {
    KVPOP_OK = 0,
    KVPOP_ERR_INVALID_ARGUMENT = 1,
    KVPOP_ERR_UNSUPPORTED = 2,
    KVPOP_ERR_WORKSPACE_TOO_SMALL = 3,
    KVPOP_ERR_DEVICE = 4
} kvpop_status;

/* Aggregation of the per-query-head future mass over a KV-head group
 * (App. B.1: max is the paper's default, a probability-space mean the
 * alternative; SUM is the plain total over the group). */
typedef enum { KVPOP_AGG_SUM = 0, KVPOP_AGG_MEAN = 1, KVPOP_AGG_MAX = 2 } kvpop_agg;

typedef enum { KVPOP_OUT_F32 = 0, KVPOP_OUT_BF16 = 1 } kvpop_out_dtype;

typedef struct {
    int batch;       /* B   */
    int n_q_heads;   /* Hq  */
    int n_kv_heads;  /* Hkv */
    int seq_len;     /* S (for decode: the number of cache slots) */
    int head_dim;    /* D: 64 or 128 */
    float scale;     /* softmax scale; <= 0 selects 1/sqrt(D) */
} kvpop_dims;

/* Workspace sizes (bytes) for the calls that take one. */
#define KVPOP_OP_FUTURE_TARGET 0
#define KVPOP_OP_DECODE 1
#define KVPOP_OP_FWD_LSE 2
#define KVPOP_OP_FWD_LSE_SPARSE 3 /* third argument: the budget */
#define KVPOP_OP_FWD_ATTN 4       /* kvpop_fwd_lse / _sparse with v and o */

int kvpop_abi_version(void);
const char* kvpop_status_string(kvpop_status s);

/*
 * kvpop_fwd_lse -- main causal attention pass: per-query log-normalizers,
 * and optionally the attention output.
 * App. D.1 (dense target identity) and D.4, first step: the main attention
 * pass yields one log-normalizer per query, which the target reuses; the
 * pass itself is the model's causal attention.
 *   LSE[b][g][d] = log sum_{t <= d} exp(scale * Q[b][g][d] . K[b][g/G][t])
 *   O[b][g][d]   = sum_{t <= d} exp(scale * Q[b][g][d] . K[b][g/G][t] - LSE[b][g][d]) V[b][g/G][t]
 * (the diagonal t = d is included, so no row is empty).  No S x S matrix is
 * formed.  q, k, v: bf16 as laid out above; lse: fp32 [B][Hq][S], written
 * in full.  Accumulation is fp32; the probabilities enter the product with V
 * rounded to bf16.
 *   v, o:      nullable together (NULL: log-normalizers only).  o is
 *              [B][Hq][S][D], fp32 or bf16 (round to nearest even) per
 *              o_dtype, 16-byte aligned, written in full.
 *   workspace: kvpop_workspace_bytes(KVPOP_OP_FWD_LSE, dims, 0) bytes without
 *              v (zero for shapes with many row blocks; then it may be NULL;
 *              16-byte aligned; partial (max, sum) pairs when long causal rows
 *              are split to balance the launch), or
 *              kvpop_workspace_bytes(KVPOP_OP_FWD_ATTN, dims, 0) bytes with v
 *              (256-byte aligned; V transposed, 64-key padded).  No
 *              initialisation needed.
 * Errors: INVALID_ARGUMENT for NULL q, k or lse, v without o (or the
 * reverse), misaligned pointers, a bad o_dtype; UNSUPPORTED when one KV
 * head's K or V (S * D * 2 bytes, S rounded up to 64) reaches 2 GiB;
 * WORKSPACE_TOO_SMALL.
 */
kvpop_status kvpop_fwd_lse(const kvpop_dims* dims, const void* q, const void* k, const void* v,
                           float* lse, void* o, kvpop_out_dtype o_dtype, void* workspace,
                           size_t workspace_bytes, hipStream_t stream);

/*
 * kvpop_running_topk -- running top-k retention mask and its cutoffs.
 * App. C.1 (mask definition): at query position d the fixed-budget mask
 * keeps the sinks [0, min(s, d+1)), the protected window (d-w, d] and the
 * k = budget - s - w best tokens of the eligible pool P_d = [s, d-w] (all
 * of P_d while it holds at most k).  App. C.2: the per-query cutoffs of that
 * running top-k.  Sec. 3 (teacher policy) and App. B.3: a per-KV-head decay
 * gamma_h in (0, 1) ranks by the static priority
 *   pi_t = sigma_t + lambda_h * t,  lambda_h = -ln gamma_h,
 * both operations rounded to fp32 (App. F: ranking in fp32); the order is
 * that of kvpop_evict_select (higher first, lower position on ties, NaN
 * last, -0 = +0).
 *   scores:     fp32 [B][Hkv][S] (sigma; positions < s are ignored).
 *   log_decay:  nullable fp32 [Hkv] (lambda_h; NULL = no decay).  Finite
 *               values >= 0 are the intended use; any value still gives a
 *               valid total order on pi.
 *   keep_until: int32 [B][Hkv][S], written in full: key t is retained for
 *               the queries t <= d < keep_until[t] (S: to the end).
 *   cutoff:     nullable int32 [B][Hkv][S]: cutoff[d] = the k-th best token
 *               of P_d (the teacher's cutoff token), -1 while |P_d| < k or
 *               when k = 0.
 *   workspace:  kvpop_running_topk_workspace_bytes(batch, n_kv_heads,
 *               seq_len, n_sink) bytes, 16-byte aligned, no initialisation
 *               needed (sort buffers, the rank structure and the cutoff
 *               ranks of rows past 8192 tokens, which take O(S log S) work
 *               like App. C.2's Fenwick sweep); NULL when that size is 0.
 * Errors: INVALID_ARGUMENT for non-positive sizes, s < 0, w < 0,
 * budget < s + w, a NULL scores or keep_until, misaligned pointers, a
 * missing workspace; WORKSPACE_TOO_SMALL; UNSUPPORTED for seq_len > 2^24.
 * The result is exact (integer outputs, no rounding-order dependence).
 */
size_t kvpop_running_topk_workspace_bytes(int batch, int n_kv_heads, int seq_len, int n_sink);
kvpop_status kvpop_running_topk(int batch, int n_kv_heads, int seq_len, int n_sink, int window,
                                int budget, const float* scores, const float* log_decay,
                                int32_t* keep_until, int32_t* cutoff, void* workspace,
                                size_t workspace_bytes, hipStream_t stream);

/*
 * kvpop_fwd_lse_sparse -- main causal pass with the sparse normalizer (and
 * optionally the sparse attention output).
 * App. D.3: the target may reuse the log-normalizer of the fixed-budget
 * sparse attention instead of the dense one; App. C.1 gives its mask; App. I
 * has that sparse (student) attention supply both output and normalizers:
 *   R_d          = { t <= d : d < keep_until[b][h][t] }
 *   LSE[b][g][d] = log sum_{t in R_d} exp(scale * q_d . k_t)
 *   O[b][g][d]   = sum_{t in R_d} exp(scale * q_d . k_t - LSE[b][g][d]) v_t
 * with keep_until from kvpop_running_topk (h = g / G); keep_until is int32
 * [B][Hkv][S], 4-byte aligned; q, k, v, lse, o and o_dtype as for
 * kvpop_fwd_lse.
 *   budget:    the budget keep_until was made with (> 0), or 0.  Without v
 *              and with a budget the pass first lists, for every block of
 *              P = 128/G query positions, the keys still retained at its
 *              first query (at most budget + P for a running top-k mask) and
 *              attends over those only; a block whose list would exceed that
 *              bound (keep_until made otherwise) walks its whole causal row,
 *              so the result is the same for any keep_until.  With 0, or
 *              with v, every causal key is read and tested.
 *   workspace: with v: kvpop_workspace_bytes(KVPOP_OP_FWD_ATTN, dims, 0)
 *              bytes; without: kvpop_workspace_bytes(KVPOP_OP_FWD_LSE_SPARSE,
 *              dims, budget) bytes; 256-byte aligned with v or a budget (16
 *              otherwise), no initialisation needed; it may be NULL when the
 *              size is zero.
 * A row whose retained set is empty gets LSE = -inf and O = 0 (the mask of
 * kvpop_running_topk always keeps token d itself when w >= 1).  The LSE
 * feeds kvpop_future_attn_target unchanged.
 * Errors: as kvpop_fwd_lse; INVALID_ARGUMENT for a NULL keep_until or a
 * negative budget.
 */
kvpop_status kvpop_fwd_lse_sparse(const kvpop_dims* dims, const void* q, const void* k,
                                  const void* v, const int32_t* keep_until, int budget,
                                  float* lse, void* o, kvpop_out_dtype o_dtype, void* workspace,
                                  size_t workspace_bytes, hipStream_t stream);

/*
 * kvpop_future_attn_target -- transposed future-attention pass.
 * App. D.1-D.2 and D.4: keys take the role of queries; the original
 * log-normalizer is subtracted and queries d < t + w are masked, so for key
 * t and query head g
 *   m_t^(g) = sum_{d = t+w}^{end_t} exp(scale * Q[g][d] . K[h][t] - LSE[g][d])
 * with end_t = S-1 when lookahead < 0, else min(S-1, t+w+lookahead)
 * (App. B.2 finite lookahead).  Keys t >= S - w receive 0.
 * The group of G query heads of KV head h is aggregated (App. B.1) by `agg`;
 * with count_normalize != 0 the result is divided by the number of
 * contributing queries N_t = clip(S - t - w, 0, lookahead + 1) (App. B.2;
 * N_t = 0 gives 0).
 *   lse:            fp32 [B][Hq][S] from kvpop_fwd_lse (natural log).
 *   mass:           fp32 [B][Hkv][S], written in full.
 *   mass_per_qhead: nullable fp32 [B][Hq][S]: the per-query-head m_t^(g)
 *                   (count-normalised when count_normalize != 0).
 *   workspace:      at least kvpop_workspace_bytes(KVPOP_OP_FUTURE_TARGET,
 *                   dims, window) bytes, 256-byte aligned; contents are
 *                   scratch and need no initialisation.
 * The result is deterministic on a given device: partial sums are reduced
 * in a fixed order, and how the work is cut depends only on the shape and
 * the device's count of resident workgroups.
 * Errors: INVALID_ARGUMENT for NULL q, k, lse, mass or workspace, w < 0, a
 * bad agg, misaligned pointers; UNSUPPORTED when one group's Q (G * S * D
 * * 2 bytes) or one group's LSE (S * G * 4 bytes) reaches 2 GiB;
 * WORKSPACE_TOO_SMALL.
 */
kvpop_status kvpop_future_attn_target(const kvpop_dims* dims, const void* q, const void* k,
                                      const float* lse, int window, int lookahead, kvpop_agg agg,
                                      int count_normalize, float* mass, float* mass_per_qhead,
                                      void* workspace, size_t workspace_bytes, hipStream_t stream);

/*
 * kvpop_evict_select -- fixed-budget retention and compaction.
 * Sec. 3 (sinks + protected recent window + per-head top-k long-range
 * tokens; attention over the retained set only), App. C.1 (budget
 * B = s + w + k), App. F (ranking and selection in fp32).
 * Per (b, h) row of S fp32 scores: eligible positions E = [s, S - w);
 * keep the k = budget - s - w best of E, where a higher score ranks first,
 * equal scores rank by lower position, NaN ranks below every number and
 * -0.0 equals +0.0.  Scores at sink and window positions are ignored.
 * Canonical slot layout of slot_pos [B][Hkv][budget] (int32, -1 = empty):
 *   [0, s)        sink p at slot p
 *   [s, s+k)      kept long-range positions, ascending, then -1 padding
 *   [s+k, budget) window ring: position p in [max(S-w, s), S) at slot
 *                 s + k + (p mod w)
 *   slot_score: nullable fp32 [B][Hkv][budget]: scores[slot_pos], -inf when
 *               empty.
 *   k, v:       nullable together: bf16 [B][Hkv][S][head_dim].
 *   k_cache, v_cache: nullable together (must be non-null when k, v are):
 *               bf16 [B][Hkv][budget][head_dim]; row j is a bitwise copy
 *               of row slot_pos[j], zero when empty.
 * The output is bit-exact and deterministic.
 */
kvpop_status kvpop_evict_select(int batch, int n_kv_heads, int seq_len, int head_dim, int n_sink,
                                int window, int budget, const float* scores, const void* k,
                                const void* v, int32_t* slot_pos, float* slot_score, void* k_cache,
                                void* v_cache, hipStream_t stream);

/*
 * kvpop_decode_attend -- one decoding query per head over the bounded cache.
 * Sec. 3 and App. C.1: decoding attends only over the retained entries.
 *   q:        bf16 [B][Hq][D]
 *   k_cache, v_cache: bf16 [B][Hkv][n_slots][D], n_slots = dims->seq_len
 *   slot_pos: int32 [B][Hkv][n_slots]; slots with slot_pos < 0 are skipped
 *   o:        [B][Hq][D], fp32 or bf16 (round to nearest even) per o_dtype
 *   lse:      nullable fp32 [B][Hq], natural log of the softmax denominator
 *   workspace: kvpop_workspace_bytes(KVPOP_OP_DECODE, dims, 0) bytes,
 *   16-byte aligned (zero when B * Hkv rows fill the device without
 *   splitting the slots; then it may be NULL).
 * A head with no valid slot gets o = 0 and lse = -inf.
 */
kvpop_status kvpop_decode_attend(const kvpop_dims* dims, const void* q, const void* k_cache,
                                 const void* v_cache, const int32_t* slot_pos, void* o,
                                 kvpop_out_dtype o_dtype, float* lse, void* workspace,
                                 size_t workspace_bytes, hipStream_t stream);

/*
 * kvpop_decode_attend_noalloc -- kvpop_decode_attend for callers that cannot
 * allocate device memory: code under HIP graph capture, tight serving
 * loops, harnesses that forbid hipMalloc.  Same arguments, result (bit for
 * bit) and errors as kvpop_decode_attend, without the workspace: when the
 * launch splits the slots over several workgroups, their partial states go
 * to a fixed array of KVPOP_DECODE_NOALLOC_SCRATCH_BYTES inside the library
 * (one per device, held until the process ends; its address is looked up
 * on the first call on each device).  The call itself allocates nothing.
 *   Returns KVPOP_ERR_WORKSPACE_TOO_SMALL, before any launch, when the shape
 *   needs more than that (kvpop_workspace_bytes(KVPOP_OP_DECODE, dims, 0) >
 *   KVPOP_DECODE_NOALLOC_SCRATCH_BYTES; never for B * Hkv rows that fill
 *   the device, which need no split).
 * All calls on one device share the array and it keeps the last call's
 * contents: calls that may overlap in time on one device (different
 * streams, or several host threads) race and must be serialised by the
 * caller; calls issued in order on one stream are safe.
 */
#define KVPOP_DECODE_NOALLOC_SCRATCH_BYTES (8u << 20)
kvpop_status kvpop_decode_attend_noalloc(const kvpop_dims* dims, const void* q,
                                         const void* k_cache, const void* v_cache,
                                         const int32_t* slot_pos, void* o,
                                         kvpop_out_dtype o_dtype, float* lse, hipStream_t stream);

/*
 * kvpop_score_mlp -- stateless headwise MLP scorer (App. E.2), on keys:
 *   score = b2[h] + sum_j w2[h][j] * gelu(b1[h][j] + sum_c W1[h][j][c] k[c])
 *   gelu(x) = 0.5 x (1 + erf(x / sqrt 2))
 *   keys: bf16 [B][Hkv][n_tok][D]; w1 fp32 [Hkv][hidden][D]; b1, w2 fp32
 *   [Hkv][hidden]; b2 fp32 [Hkv]; scores fp32 [B][Hkv][n_tok].
 *   1 <= hidden <= 64.  Accumulation is fp32.
 */
kvpop_status kvpop_score_mlp(int batch, int n_kv_heads, int n_tok, int head_dim, int hidden,
                             const void* keys, const float* w1, const float* b1, const float* w2,
                             const float* b2, float* scores, hipStream_t stream);

/*
 * kvpop_cache_step -- one decoding step of the bounded per-head cache.
 * Sec. 3 (a token is scored while in the protected window and judged when it
 * leaves it), App. E.4 (at query q the newly eligible token is u = q - w),
 * App. C.1 (B = s + w + k).  Slot layout as for kvpop_evict_select.
 * For the new token at position pos_q, for every (b, h):
 *  (a) exit: if u = pos_q - w >= s, token u leaves its ring slot.  It takes
 *      the lowest empty long-range slot if there is one; otherwise it
 *      replaces the worst kept token v (lowest score; among equal scores the
 *      highest position; NaN lowest) when it ranks strictly before v, else
 *      it is dropped.
 *  (b) append: pos_q is written to sink slot pos_q when pos_q < s, else to
 *      ring slot s + k + (pos_q mod w), its score set to quiet NaN.
 *  (c) delayed scoring: token r = pos_q - delay (when r >= s) receives its
 *      score in its ring slot: the MLP of kvpop_score_mlp on its cached key
 *      when w1 != NULL, else scores_r[b][h]; with neither, nothing is scored
 *      here (for scorers that score the exiting token themselves before the
 *      step, such as kvpop_mlstm_step).
 *   k_new, v_new: bf16 [B][Hkv][D]; the cache state (k_cache, v_cache bf16
 *   [B][Hkv][budget][D], slot_pos int32 and slot_score fp32
 *   [B][Hkv][budget]) is updated in place.  Requires w >= 1,
 *   0 <= delay < w, and at most one of {w1 (with b1, w2, b2, hidden)} and
 *   scores_r.
 * Bit-exact and deterministic given the same scores.
 */
kvpop_status kvpop_cache_step(int batch, int n_kv_heads, int head_dim, int n_sink, int window,
                              int budget, int delay, int pos_q, const void* k_new,
                              const void* v_new, const float* w1, const float* b1,
                              const float* w2, const float* b2, int hidden,
                              const float* scores_r, void* k_cache, void* v_cache,
                              int32_t* slot_pos, float* slot_score, hipStream_t stream);

/*
 * kvpop_mlstm_step -- one decoding step of the delayed stateful mLSTM scorer.
 * App. A (a running key-value summary and normalizer updated by rank-one
 * outer products), App. E.1 (headwise input x = [k; v]), App. E.3 (mLSTM
 * matrix memory C and normalizer n with scalar input and forget gates from
 * headwise projections, stabilised form, Hedgehog features), App. E.4 (at
 * query q the state has taken tokens through q and the newly eligible
 * token u = q - w is read out).  Per (b, h), with x_q = [k_new; v_new]:
 *   hedgehog(z) = [softmax(z); softmax(-z)]
 *   phi = hedgehog(Wk x_q), val = Wv x_q, ig = wi.x_q + bi,
 *   lf = log sigmoid(wf.x_q + bf), m' = max(lf + m, ig),
 *   C' = e^(lf + m - m') C + e^(ig - m') val phi^T,  n' likewise with phi;
 * then, when slot_score != NULL and u = pos_q - w >= s, with x_u = the
 * cached [K; V] rows of u's ring slot s + k + (u mod w):
 *   r = hedgehog(Wr x_u), h = C' r / max(|n'.r|, e^(-m')),
 *   slot_score[b][h][ring slot of u] = wo.silu(h) + bo.
 * Called before kvpop_cache_step of the same position with no scorer, it
 * gives the exit decision of u the score from the state through pos_q.
 *   w: feat = 32 (P), vdim = 64 (E); Wk, Wr fp32 [Hkv][P][2D], Wv
 *      [Hkv][E][2D], wi, wf [Hkv][2D] (these five 16-byte aligned), bi,
 *      bf, bo [Hkv], wo [Hkv][E].
 *   state: fp32 [B][Hkv][KVPOP_MLSTM_STATE_FLOATS], 16-byte aligned: C
 *      row-major [E][2P], then n [2P], then m, then 3 unused floats.  An
 *      empty state is C = 0, n = 0, m = -inf; it is updated in place.
 *   k_cache, v_cache: bf16 [B][Hkv][budget][D], read only (u's ring slot).
 *   slot_score: nullable fp32 [B][Hkv][budget]; NULL updates the state only.
 * Errors: INVALID_ARGUMENT for non-positive sizes, w < 1, budget < s + w,
 * pos_q < 0, NULL or misaligned pointers; UNSUPPORTED for D not 64 or 128
 * or other feature sizes.  fp32 arithmetic; deterministic.
 */
#define KVPOP_MLSTM_STATE_FLOATS (64 * 64 + 64 + 4)
typedef struct {
    int feat, vdim;
    const float *wk, *wr, *wv, *wi, *bi, *wf, *bf, *wo, *bo;
} kvpop_mlstm_weights;
kvpop_status kvpop_mlstm_step(int batch, int n_kv_heads, int head_dim, int n_sink, int window,
                              int budget, int pos_q, const void* k_new, const void* v_new,
                              const void* k_cache, const void* v_cache,
                              const kvpop_mlstm_weights* w, float* state, float* slot_score,
                              hipStream_t stream);

/*
 * kvpop_decode_step_mlstm -- one decode step with the delayed mLSTM scorer:
 * kvpop_mlstm_step (the new token enters the scorer state, the exiting
 * token u = pos_q - w is scored into its ring slot), then kvpop_cache_step
 * with no scorer of its own (u is kept or dropped on that score, the new
 * token enters), then kvpop_decode_attend over the updated cache.  App. E.3,
 * E.4 and Sec. 3 (the scorer reads out the token leaving the window, which
 * is judged at once), App. C.1 (attention over the retained entries).
 * Same effect, bit for bit, as the three calls with the same arguments
 * (dims->seq_len is the budget); when B * Hkv rows fill the device they run
 * in one launch.  Arguments and errors as for those calls; workspace:
 * kvpop_workspace_bytes(KVPOP_OP_DECODE, dims, 0) bytes.
 */
kvpop_status kvpop_decode_step_mlstm(const kvpop_dims* dims, int n_sink, int window, int pos_q,
                                     const void* k_new, const void* v_new,
                                     const kvpop_mlstm_weights* w, float* state, void* k_cache,
                                     void* v_cache, int32_t* slot_pos, float* slot_score,
                                     const void* q, void* o, kvpop_out_dtype o_dtype, float* lse,
                                     void* workspace, size_t workspace_bytes, hipStream_t stream);

/*
 * kvpop_decode_step -- one bounded-cache decode step, then decode attention
 * over the updated cache.  Sec. 3, App. C.1 and App. E.4: the token leaving
 * the window is kept or dropped, the new token enters its ring slot, the
 * delayed score is taken, and the query attends over the retained entries.
 * Same effect, bit for bit, as kvpop_cache_step(...) followed by
 * kvpop_decode_attend(...) with the same arguments (dims->seq_len is the
 * budget); when B * Hkv rows fill the device the two run in one launch.
 *   workspace: kvpop_workspace_bytes(KVPOP_OP_DECODE, dims, 0) bytes.
 * Errors: the union of the two calls' checks.
 */
kvpop_status kvpop_decode_step(const kvpop_dims* dims, int n_sink, int window, int delay,
                               int pos_q, const void* k_new, const void* v_new, const float* w1,
                               const float* b1, const float* w2, const float* b2, int hidden,
                               const float* scores_r, void* k_cache, void* v_cache,
                               int32_t* slot_pos, float* slot_score, const void* q, void* o,
                               kvpop_out_dtype o_dtype, float* lse, void* workspace,
                               size_t workspace_bytes, hipStream_t stream);

/* Bytes of workspace needed by `op` for these dims (0 if none).  The
 * target and decode sizes depend on the current HIP device (its compute
 * units and the kernels' occupancy): query with the device the call will
 * run on current. */
size_t kvpop_workspace_bytes(int op, const kvpop_dims* dims, int window);

#ifdef __cplusplus
}
#endif

#endif /* KVPOP_H */
