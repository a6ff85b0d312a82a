/*
 * kvpop_oracle.c -- plain CPU oracle for the KVpop hot path.
 *
 * TEST INFRASTRUCTURE ONLY.  Only tests/, __graft_entry__.smoke() and the
 * cpu_baseline leg of bench.py may load this library.  It shares no code,
 * header, table or helper with the HIP library: it is a second, independent
 * statement of what the method computes, written for a reader to check
 * against the pages by eye.  Every floating-point quantity is accumulated in
 * double precision from the exact float values of the (bf16) inputs.  Loops
 * are plain; the only parallelism is a split of independent output rows over
 * POSIX threads, which cannot change any result.
 *
 * Source: "KVpop -- Key-Value Cache Compression with Predictive Online
 * Pruning" (arXiv 2607.05061v2), as summarised on paperlayer.ai.  Sections
 * cited below are that page's.
 */
#include <math.h>
#include <pthread.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define AGG_SUM 0
#define AGG_MEAN 1
#define AGG_MAX 2

/* ------------------------------------------------------------------ */
/* threading: item i is handled by thread (i mod T); no shared writes */
/* ------------------------------------------------------------------ */
typedef void (*item_fn)(void* ctx, long item, double* scratch);

typedef struct {
    item_fn fn;
    void* ctx;
    long n_items;
    int tid, nthreads;
    long scratch_len;
} worker_arg;

static void* worker_main(void* p) {
    worker_arg* a = (worker_arg*)p;
    double* scratch = a->scratch_len > 0 ? (double*)malloc(sizeof(double) * a->scratch_len) : NULL;
    for (long i = a->tid; i < a->n_items; i += a->nthreads) a->fn(a->ctx, i, scratch);
    free(scratch);
    return NULL;
}

static void run_items(item_fn fn, void* ctx, long n_items, int nthreads, long scratch_len) {
    if (nthreads < 1) nthreads = 1;
    if (nthreads > 256) nthreads = 256;
    pthread_t th[256];
    worker_arg args[256];
    for (int t = 0; t < nthreads; ++t) {
        args[t].fn = fn; args[t].ctx = ctx; args[t].n_items = n_items;
        args[t].tid = t; args[t].nthreads = nthreads; args[t].scratch_len = scratch_len;
    }
    for (int t = 1; t < nthreads; ++t) pthread_create(&th[t], NULL, worker_main, &args[t]);
    worker_main(&args[0]);
    for (int t = 1; t < nthreads; ++t) pthread_join(th[t], NULL);
}

/* exact dot product of two float vectors, accumulated in double */
static double dot(const float* a, const float* b, int n) {
    double s = 0.0;
    for (int c = 0; c < n; ++c) s += (double)a[c] * (double)b[c];
    return s;
}

/* ------------------------------------------------------------------ */
/* Dense causal log-normalizer (App. D.1 dense target identity; D.4   */
/* first step: the main pass yields one log-normalizer per query).    */
/*   z[d][t]  = scale * q_d . k_t   for t <= d (diagonal included)     */
/*   LSE_d    = log sum_{t<=d} exp z[d][t]   (natural log)            */
/* Query head g reads KV head g / (Hq/Hkv) (grouped-query sharing).   */
/* ------------------------------------------------------------------ */
typedef struct {
    int B, Hq, Hkv, S, D;
    double scale;
    const float *q, *k;
    const long* rows;
    double* out;
} lse_ctx;

static void lse_item(void* p, long i, double* z) {
    lse_ctx* c = (lse_ctx*)p;
    long r = c->rows ? c->rows[i] : i;
    int d = (int)(r % c->S);
    int g = (int)((r / c->S) % c->Hq);
    int b = (int)(r / ((long)c->S * c->Hq));
    int h = g / (c->Hq / c->Hkv);
    const float* qd = c->q + (((long)b * c->Hq + g) * c->S + d) * c->D;
    const float* kh = c->k + ((long)b * c->Hkv + h) * (long)c->S * c->D;
    double m = -INFINITY;
    for (int t = 0; t <= d; ++t) {
        z[t] = c->scale * dot(qd, kh + (long)t * c->D, c->D);
        if (z[t] > m) m = z[t];
    }
    double sum = 0.0;
    for (int t = 0; t <= d; ++t) sum += exp(z[t] - m);
    c->out[i] = m + log(sum);
}

/* rows: flat indices (b*Hq + g)*S + d, or NULL for all B*Hq*S rows in order */
int oracle_lse(int B, int Hq, int Hkv, int S, int D, double scale,
               const float* q, const float* k, long n_rows, const long* rows,
               double* out, int nthreads) {
    if (B <= 0 || Hq <= 0 || Hkv <= 0 || S <= 0 || D <= 0 || Hq % Hkv) return 1;
    lse_ctx c = {B, Hq, Hkv, S, D, scale, q, k, rows, out};
    run_items(lse_item, &c, n_rows, nthreads, S);
    return 0;
}

/* ------------------------------------------------------------------ */
/* Future-attention mass (App. D.1-D.2, D.4; B.1 aggregation, B.2     */
/* count normalisation and finite lookahead).                          */
/* For key t of KV head h and each query head g of its group:          */
/*   m_t^(g) = sum over d with t+w <= d <= end_t of                    */
/*             exp(scale * q_d^(g) . k_t - LSE_d^(g))                  */
/*   end_t   = S-1 (unbounded lookahead) or min(S-1, t+w+L)            */
/* The token counts as attended only once it has left the window of   */
/* the w most recent tokens, i.e. for queries d >= t + w.              */
/* Aggregate over the group: SUM, MEAN (= SUM / G, a mean of           */
/* probabilities) or MAX.  Count normalisation divides by the number  */
/* of contributing queries N_t = clip(S - t - w, 0, L + 1); N_t = 0    */
/* gives 0.                                                            */
/* ------------------------------------------------------------------ */
typedef struct {
    int B, Hq, Hkv, S, D;
    double scale;
    const float *q, *k;
    const double* lse;
    int window, lookahead, agg, count_normalize;
    const long* cols;
    double *mass, *per_head;
} mass_ctx;

static void mass_item(void* p, long i, double* unused) {
    (void)unused;
    mass_ctx* c = (mass_ctx*)p;
    long col = c->cols ? c->cols[i] : i;
    int t = (int)(col % c->S);
    int h = (int)((col / c->S) % c->Hkv);
    int b = (int)(col / ((long)c->S * c->Hkv));
    int G = c->Hq / c->Hkv;
    const float* kt = c->k + (((long)b * c->Hkv + h) * c->S + t) * c->D;
    long first = (long)t + c->window;
    long last = c->S - 1;
    if (c->lookahead >= 0 && first + c->lookahead < last) last = first + c->lookahead;
    long n_t = last - first + 1;
    if (n_t < 0) n_t = 0;

    double sum = 0.0, mx = 0.0;
    for (int gl = 0; gl < G; ++gl) {
        int g = h * G + gl;
        const float* qg = c->q + ((long)b * c->Hq + g) * (long)c->S * c->D;
        const double* lg = c->lse + ((long)b * c->Hq + g) * (long)c->S;
        double m = 0.0;
        for (long d = first; d <= last; ++d)
            m += exp(c->scale * dot(qg + d * c->D, kt, c->D) - lg[d]);
        if (c->per_head) c->per_head[i * G + gl] = c->count_normalize ? (n_t > 0 ? m / (double)n_t : 0.0) : m;
        sum += m;
        if (gl == 0 || m > mx) mx = m;
    }
    double v = c->agg == AGG_SUM ? sum : c->agg == AGG_MEAN ? sum / G : mx;
    if (c->count_normalize) v = n_t > 0 ? v / (double)n_t : 0.0;
    c->mass[i] = v;
}

/* lse: [B][Hq][S] natural-log normalizers (only rows d >= t+w of the
 * requested columns are read).  cols: flat (b*Hkv + h)*S + t, or NULL for
 * all columns in order.  per_head: nullable [n_cols][G]. */
int oracle_future_mass(int B, int Hq, int Hkv, int S, int D, double scale,
                       const float* q, const float* k, const double* lse,
                       int window, int lookahead, int agg, int count_normalize,
                       long n_cols, const long* cols, double* mass, double* per_head,
                       int nthreads) {
    if (B <= 0 || Hq <= 0 || Hkv <= 0 || S <= 0 || D <= 0 || Hq % Hkv) return 1;
    if (window < 0 || agg < 0 || agg > 2) return 1;
    mass_ctx c = {B, Hq, Hkv, S, D, scale, q, k, lse, window, lookahead, agg,
                  count_normalize, cols, mass, per_head};
    run_items(mass_item, &c, n_cols, nthreads, 0);
    return 0;
}

/* ------------------------------------------------------------------ */
/* Fixed-budget retention (Sec. 3 fixed-budget pruning; App. C.1 mask */
/* definition B = s + w + k; App. F: ranking and selection in fp32).   */
/* Per (b, h) row of S fp32 scores:                                    */
/*   eligible E = [s, S - w); k = budget - s - w                       */
/*   keep the k best of E under the order: higher score first, equal   */
/*   scores broken by the lower position; NaN ranks below every number */
/*   (below -inf) and -0 equals +0.                                    */
/* Slot layout of the bounded cache (budget slots):                    */
/*   [0, s)        sink token p at slot p                              */
/*   [s, s+k)      selected tokens in ascending position, -1 padding   */
/*   [s+k, s+k+w)  window ring: token p at slot s+k+(p mod w)          */
/* Unused slots hold -1.                                               */
/* ------------------------------------------------------------------ */
typedef struct { float score; int pos; } cand;

/* returns 1 if a ranks strictly before b in the retention order */
static int better(float sa, int pa, float sb, int pb) {
    int na = isnan(sa), nb = isnan(sb);
    if (na != nb) return nb;          /* the number beats the NaN */
    if (!na && sa != sb) return sa > sb; /* IEEE compare: -0 == +0 */
    return pa < pb;                   /* tie: lower position first */
}

static int cand_cmp(const void* x, const void* y) {
    const cand* a = (const cand*)x;
    const cand* b = (const cand*)y;
    if (a->pos == b->pos) return 0;
    return better(a->score, a->pos, b->score, b->pos) ? -1 : 1;
}

static int int_cmp(const void* x, const void* y) {
    int a = *(const int*)x, b = *(const int*)y;
    return (a > b) - (a < b);
}

int oracle_select(int B, int Hkv, int S, int n_sink, int window, int budget,
                  const float* scores, int32_t* slot_pos, float* slot_score) {
    if (B <= 0 || Hkv <= 0 || S <= 0 || n_sink < 0 || window < 0) return 1;
    int kk = budget - n_sink - window;
    if (kk < 0) return 1;
    cand* e = (cand*)malloc(sizeof(cand) * (size_t)S);
    int* chosen = (int*)malloc(sizeof(int) * (size_t)(kk > 0 ? kk : 1));
    for (long row = 0; row < (long)B * Hkv; ++row) {
        const float* sc = scores + row * S;
        int32_t* sp = slot_pos + row * budget;
        for (int j = 0; j < budget; ++j) sp[j] = -1;
        for (int p = 0; p < n_sink && p < S; ++p) sp[p] = p;
        int e_lo = n_sink, e_hi = S - window;
        int n_e = 0;
        for (int p = e_lo; p < e_hi; ++p) { e[n_e].score = sc[p]; e[n_e].pos = p; ++n_e; }
        qsort(e, (size_t)n_e, sizeof(cand), cand_cmp);
        int n_keep = n_e < kk ? n_e : kk;
        for (int i = 0; i < n_keep; ++i) chosen[i] = e[i].pos;
        qsort(chosen, (size_t)n_keep, sizeof(int), int_cmp);
        for (int i = 0; i < n_keep; ++i) sp[n_sink + i] = chosen[i];
        int w_lo = S - window > n_sink ? S - window : n_sink;
        for (int p = w_lo; p < S; ++p) sp[n_sink + kk + (p % window)] = p;
        if (slot_score)
            for (int j = 0; j < budget; ++j)
                slot_score[row * budget + j] = sp[j] >= 0 ? sc[sp[j]] : -INFINITY;
    }
    free(e);
    free(chosen);
    return 0;
}

/* ------------------------------------------------------------------ */
/* Attention of one decoding query over the retained cache entries    */
/* only (Sec. 3: attention over the retained set; App. C.1: decoding  */
/* attends directly over the retained cache).                          */
/* Slots with slot_pos < 0 are empty and take no part.                 */
/*   z_j = scale * q . K_c[j];  lse = log sum_j exp z_j                */
/*   o   = sum_j exp(z_j - lse) V_c[j]                                 */
/* With no valid slot: o = 0, lse = -inf.                              */
/* ------------------------------------------------------------------ */
typedef struct {
    int B, Hq, Hkv, n_slots, D;
    double scale;
    const float *q, *kc, *vc;
    const int32_t* slot_pos;
    double *o, *lse;
} dec_ctx;

static void dec_item(void* p, long i, double* z) {
    dec_ctx* c = (dec_ctx*)p;
    int g = (int)(i % c->Hq);
    int b = (int)(i / c->Hq);
    int h = g / (c->Hq / c->Hkv);
    const float* qg = c->q + i * c->D;
    long base = ((long)b * c->Hkv + h) * c->n_slots;
    double m = -INFINITY;
    for (int j = 0; j < c->n_slots; ++j) {
        if (c->slot_pos[base + j] < 0) continue;
        z[j] = c->scale * dot(qg, c->kc + (base + j) * c->D, c->D);
        if (z[j] > m) m = z[j];
    }
    double* o = c->o + i * c->D;
    for (int e = 0; e < c->D; ++e) o[e] = 0.0;
    if (m == -INFINITY) { c->lse[i] = -INFINITY; return; }
    double l = 0.0;
    for (int j = 0; j < c->n_slots; ++j) {
        if (c->slot_pos[base + j] < 0) continue;
        double wj = exp(z[j] - m);
        l += wj;
        const float* v = c->vc + (base + j) * c->D;
        for (int e = 0; e < c->D; ++e) o[e] += wj * (double)v[e];
    }
    for (int e = 0; e < c->D; ++e) o[e] /= l;
    c->lse[i] = m + log(l);
}

int oracle_decode_attend(int B, int Hq, int Hkv, int n_slots, int D, double scale,
                         const float* q, const float* kc, const float* vc,
                         const int32_t* slot_pos, double* o, double* lse, int nthreads) {
    if (B <= 0 || Hq <= 0 || Hkv <= 0 || n_slots <= 0 || D <= 0 || Hq % Hkv) return 1;
    dec_ctx c = {B, Hq, Hkv, n_slots, D, scale, q, kc, vc, slot_pos, o, lse};
    run_items(dec_item, &c, (long)B * Hq, nthreads, n_slots);
    return 0;
}

/* ------------------------------------------------------------------ */
/* Stateless headwise MLP scorer (App. E.2), here on the key alone:   */
/*   sigma = b2 + sum_j w2[j] * gelu(b1[j] + sum_c W1[j][c] k[c])      */
/*   gelu(x) = x * Phi(x) = 0.5 x (1 + erf(x / sqrt 2))                */
/* Weights per KV head: W1 [hidden][D], b1 [hidden], w2 [hidden], b2.  */
/* ------------------------------------------------------------------ */
static double gelu(double x) { return 0.5 * x * (1.0 + erf(x / sqrt(2.0))); }

int oracle_mlp_score(int B, int Hkv, int n_tok, int D, int hidden, const float* keys,
                     const float* w1, const float* b1, const float* w2, const float* b2,
                     double* out) {
    if (B <= 0 || Hkv <= 0 || n_tok < 0 || D <= 0 || hidden <= 0) return 1;
    for (int b = 0; b < B; ++b)
        for (int h = 0; h < Hkv; ++h)
            for (int t = 0; t < n_tok; ++t) {
                const float* kt = keys + (((long)b * Hkv + h) * n_tok + t) * D;
                double s = (double)b2[h];
                for (int j = 0; j < hidden; ++j) {
                    const float* wj = w1 + ((long)h * hidden + j) * D;
                    double a = (double)b1[h * hidden + j] + dot(wj, kt, D);
                    s += (double)w2[h * hidden + j] * gelu(a);
                }
                out[((long)b * Hkv + h) * n_tok + t] = s;
            }
    return 0;
}

/* ------------------------------------------------------------------ */
/* One decoding step of the bounded cache for every (b, h)             */
/* (Sec. 3 fixed-budget pruning and stateful scoring: a token is       */
/* scored while in the protected window and judged when it leaves it;  */
/* App. E.4: at query q the newly eligible token is u = q - w;         */
/* App. C.1: B = s + w + k).  Slot layout as in oracle_select.          */
/* Order of the step at new position q:                                 */
/*  (a) exit: if u = q - w >= s, token u leaves the ring slot           */
/*      s+k+(u mod w).  If a long-range slot is empty (slot_pos = -1)   */
/*      u moves to the lowest such slot; otherwise the worst kept token */
/*      v (lowest score, ties -> highest position, NaN lowest) is       */
/*      replaced by u iff u ranks strictly before v (u is the newest,   */
/*      so equal scores keep v); else u is dropped.                     */
/*  (b) append: q goes to sink slot q if q < s, else to ring slot       */
/*      s+k+(q mod w) with its score marked unscored (quiet NaN).        */
/*  (c) delayed score: token r = q - delay (r >= s) receives score      */
/*      scores_r[b][h] in its ring slot.                                */
/* k_new/v_new and the caches hold raw bf16 bit patterns.               */
/* ------------------------------------------------------------------ */
int oracle_cache_step(int B, int Hkv, int D, int n_sink, int window, int budget,
                      int delay, int pos_q, const uint16_t* k_new, const uint16_t* v_new,
                      const float* scores_r, uint16_t* kc, uint16_t* vc,
                      int32_t* slot_pos, float* slot_score) {
    int kk = budget - n_sink - window;
    if (B <= 0 || Hkv <= 0 || D <= 0 || n_sink < 0 || window < 1 || kk < 0) return 1;
    if (delay < 0 || delay >= window || pos_q < 0) return 1;
    const uint32_t qnan_bits = 0x7fc00000u;
    float qnan;
    memcpy(&qnan, &qnan_bits, 4);
    for (long row = 0; row < (long)B * Hkv; ++row) {
        int32_t* sp = slot_pos + row * budget;
        float* ss = slot_score + row * budget;
        uint16_t* kr = kc + row * (long)budget * D;
        uint16_t* vr = vc + row * (long)budget * D;
        int q = pos_q;
        int u = q - window;
        if (u >= n_sink) {
            int ring = n_sink + kk + (u % window);
            int dst = -1;
            for (int j = n_sink; j < n_sink + kk; ++j)
                if (sp[j] < 0) { dst = j; break; }
            if (dst < 0 && kk > 0) {
                int v = n_sink;
                for (int j = n_sink + 1; j < n_sink + kk; ++j)
                    if (better(ss[v], sp[v], ss[j], sp[j])) v = j; /* j is worse than v */
                if (better(ss[ring], sp[ring], ss[v], sp[v])) dst = v;
            }
            if (dst >= 0) {
                sp[dst] = sp[ring];
                ss[dst] = ss[ring];
                memcpy(kr + (long)dst * D, kr + (long)ring * D, sizeof(uint16_t) * D);
                memcpy(vr + (long)dst * D, vr + (long)ring * D, sizeof(uint16_t) * D);
            }
        }
        int slot = q < n_sink ? q : n_sink + kk + (q % window);
        sp[slot] = q;
        ss[slot] = qnan;
        memcpy(kr + (long)slot * D, k_new + row * D, sizeof(uint16_t) * D);
        memcpy(vr + (long)slot * D, v_new + row * D, sizeof(uint16_t) * D);
        int r = q - delay;
        if (r >= n_sink) ss[n_sink + kk + (r % window)] = scores_r[row];
    }
    return 0;
}

/* ------------------------------------------------------------------ */
/* Running top-k retention mask (App. C.1 mask definition, App. C.2    */
/* Fenwick-tree cutoffs; Sec. 3 teacher policy with per-head decay;    */
/* App. B.3 temporal decay as static priorities; App. F fp32 ranking). */
/* Per (b, h) row, at query position d:                                */
/*   eligible pool  P_d = { t : s <= t <= d - w }                      */
/*   selected       Sel_d = the k best of P_d (all of P_d if |P_d|<=k) */
/*   retained       R_d = sinks [0, min(s, d+1)) U window (d-w, d]     */
/*                        U Sel_d,   k = budget - s - w                */
/* Ranking uses the static priority pi_t = sigma_t + lambda_h * t,     */
/* both operations rounded to fp32 (lambda_h = -ln gamma_h >= 0; the  */
/* decayed score sigma_t + (d - t) ln gamma_h orders keys the same way */
/* at every d), under the retention order of oracle_select.            */
/* Outputs per (b, h, position):                                       */
/*   cutoff[d]     = the k-th best token of P_d (the teacher's cutoff  */
/*                   token), or -1 while |P_d| < k or when k = 0       */
/*   keep_until[t] = first query d >= t with t not in R_d, or S:       */
/*                   t is retained exactly for queries t <= d < keep_until[t] */
/* Cutoffs follow App. C.2: tokens enter a Fenwick tree over their     */
/* ranks as they leave the window, and the k-th smallest rank present  */
/* is found by a descent of the tree.                                  */
/* ------------------------------------------------------------------ */
static float priority(float sigma, float lambda, int t) {
    float age = lambda * (float)t;   /* rounded to fp32 */
    float pi = sigma + age;          /* rounded to fp32 */
    return pi;
}

static int kth_in_fenwick(const int* tree, int n, int kth) {
    /* smallest index i (0-based) with prefix count(0..i) >= kth */
    int pos = 0, logn = 1;
    while ((logn << 1) <= n) logn <<= 1;
    for (int step = logn; step > 0; step >>= 1) {
        if (pos + step <= n && tree[pos + step] < kth) {
            pos += step;
            kth -= tree[pos];
        }
    }
    return pos; /* 1-based pos+1 holds it, i.e. 0-based index pos */
}

int oracle_running_topk(int B, int Hkv, int S, int n_sink, int window, int budget,
                        const float* scores, const float* log_decay,
                        int32_t* keep_until, int32_t* cutoff) {
    if (B <= 0 || Hkv <= 0 || S <= 0 || n_sink < 0 || window < 0) return 1;
    int kk = budget - n_sink - window;
    if (kk < 0) return 1;
    cand* e = (cand*)malloc(sizeof(cand) * (size_t)S);
    int* rank = (int*)malloc(sizeof(int) * (size_t)S);
    int* tok_of_rank = (int*)malloc(sizeof(int) * (size_t)S);
    int* tree = (int*)malloc(sizeof(int) * (size_t)(S + 1));
    int* cutrank = (int*)malloc(sizeof(int) * (size_t)S);
    for (long row = 0; row < (long)B * Hkv; ++row) {
        int h = (int)(row % Hkv);
        float lam = log_decay ? log_decay[h] : 0.0f;
        const float* sc = scores + row * S;
        int32_t* until = keep_until + row * S;
        int32_t* cut = cutoff ? cutoff + row * S : NULL;
        /* ranks of every token that can become eligible: [s, S) */
        int n_e = 0;
        for (int p = n_sink; p < S; ++p) {
            e[n_e].score = priority(sc[p], lam, p);
            e[n_e].pos = p;
            ++n_e;
        }
        qsort(e, (size_t)n_e, sizeof(cand), cand_cmp);
        for (int r = 0; r < n_e; ++r) { rank[e[r].pos] = r; tok_of_rank[r] = e[r].pos; }
        /* running cutoffs: token d - w enters the pool at query d */
        for (int i = 0; i <= n_e; ++i) tree[i] = 0;
        int count = 0;
        for (int d = 0; d < S; ++d) {
            int u = d - window;
            if (u >= n_sink) {
                for (int i = rank[u] + 1; i <= n_e; i += i & (-i)) tree[i] += 1;
                ++count;
            }
            if (kk > 0 && count >= kk) cutrank[d] = kth_in_fenwick(tree, n_e, kk);
            else cutrank[d] = -1;
            if (cut) cut[d] = cutrank[d] >= 0 ? tok_of_rank[cutrank[d]] : -1;
        }
        /* keep_until: sinks stay; a long-range token is kept from t + w on
         * while it is selected, and selection ends for good once k better
         * tokens have entered the pool (cutoff ranks only decrease) */
        for (int t = 0; t < S; ++t) {
            if (t < n_sink) { until[t] = S; continue; }
            long first = (long)t + window;
            if (first >= S) { until[t] = S; continue; }
            /* selected(d) for d >= first: pool not yet over k, or rank <= cutoff rank */
            long lo = first, hi = S; /* find first d in [first, S) not selected */
            while (lo < hi) {
                long mid = (lo + hi) / 2;
                int pool = (int)(mid - window - n_sink + 1);
                int sel = kk > 0 && (pool <= kk || rank[t] <= cutrank[mid]);
                if (sel) lo = mid + 1;
                else hi = mid;
            }
            until[t] = (int32_t)lo;
        }
    }
    free(e);
    free(rank);
    free(tok_of_rank);
    free(tree);
    free(cutrank);
    return 0;
}

/* ------------------------------------------------------------------ */
/* Sparse log-normalizer (App. D.3: the target may reuse the           */
/* normalizer of the fixed-budget sparse attention instead of the      */
/* dense one; App. C.1 retained set R_d as above):                     */
/*   LSE_d = log sum_{t in R_d} exp(scale * q_d . k_t)                 */
/* R_d is built for each requested query row straight from its         */
/* definition: the pool P_d is sorted in the retention order of the    */
/* priorities and its first k entries are kept.                        */
/* ------------------------------------------------------------------ */
typedef struct {
    int B, Hq, Hkv, S, D;
    double scale;
    const float *q, *k, *scores, *log_decay;
    int n_sink, window, kk;
    const long* rows;
    double* out;
} slse_ctx;

static void slse_item(void* p, long i, double* z) {
    slse_ctx* c = (slse_ctx*)p;
    long r = c->rows ? c->rows[i] : i;
    int d = (int)(r % c->S);
    int g = (int)((r / c->S) % c->Hq);
    int b = (int)(r / ((long)c->S * c->Hq));
    int h = g / (c->Hq / c->Hkv);
    const float* sc = c->scores + ((long)b * c->Hkv + h) * c->S;
    float lam = c->log_decay ? c->log_decay[h] : 0.0f;
    /* scratch: z[0..S) logits, then membership flags and the pool */
    char* keep = (char*)(z + c->S);
    cand* pool = (cand*)(keep + c->S + 8 - (c->S % 8));
    for (int t = 0; t <= d; ++t) keep[t] = 0;
    for (int t = 0; t <= d && t < c->n_sink; ++t) keep[t] = 1;          /* sinks */
    for (int t = d - c->window + 1; t <= d; ++t) if (t >= 0) keep[t] = 1; /* window */
    int n_pool = 0;
    for (int t = c->n_sink; t <= d - c->window; ++t) {
        pool[n_pool].score = priority(sc[t], lam, t);
        pool[n_pool].pos = t;
        ++n_pool;
    }
    qsort(pool, (size_t)n_pool, sizeof(cand), cand_cmp);
    for (int j = 0; j < n_pool && j < c->kk; ++j) keep[pool[j].pos] = 1;
    const float* qd = c->q + (((long)b * c->Hq + g) * c->S + d) * c->D;
    const float* kh = c->k + ((long)b * c->Hkv + h) * (long)c->S * c->D;
    double m = -INFINITY;
    for (int t = 0; t <= d; ++t) {
        if (!keep[t]) continue;
        z[t] = c->scale * dot(qd, kh + (long)t * c->D, c->D);
        if (z[t] > m) m = z[t];
    }
    if (m == -INFINITY) { c->out[i] = -INFINITY; return; }
    double sum = 0.0;
    for (int t = 0; t <= d; ++t) if (keep[t]) sum += exp(z[t] - m);
    c->out[i] = m + log(sum);
}

int oracle_lse_sparse(int B, int Hq, int Hkv, int S, int D, double scale,
                      const float* q, const float* k, const float* scores, const float* log_decay,
                      int n_sink, int window, int budget, long n_rows, const long* rows,
                      double* out, int nthreads) {
    if (B <= 0 || Hq <= 0 || Hkv <= 0 || S <= 0 || D <= 0 || Hq % Hkv) return 1;
    if (n_sink < 0 || window < 0 || budget - n_sink - window < 0) return 1;
    slse_ctx c = {B, Hq, Hkv, S, D, scale, q, k, scores, log_decay, n_sink, window,
                  budget - n_sink - window, rows, out};
    /* doubles: S logits + S flag bytes + S pool entries (8 bytes each) + slack */
    run_items(slse_item, &c, n_rows, nthreads, 2L * S + S / 8 + 4);
    return 0;
}

/* ------------------------------------------------------------------ */
/* Attention output of the main pass (App. D.4, first step: the main   */
/* attention pass of the model, whose per-query normalizers the target */
/* reuses; App. I: the sparse student attention, over the fixed-budget */
/* mask of App. C.1, supplies the normalizers in the paper's default). */
/* For query row d of head g (KV head h = g / G):                      */
/*   R_d    = [0, d] (dense causal) or, given scores, the retained set */
/*            of the running top-k mask built as for oracle_lse_sparse */
/*   p_dt   = exp(scale * q_d . k_t - LSE_d),  t in R_d                */
/*   LSE_d  = log sum_{t in R_d} exp(scale * q_d . k_t)                */
/*   O_d[c] = sum_{t in R_d} p_dt v_t[c]                               */
/*   A_d[c] = sum_{t in R_d} p_dt |v_t[c]|   (the scale of O_d[c]'s    */
/*            sensitivity to a relative change of each p_dt)           */
/* An empty R_d gives LSE = -inf and O = A = 0.                        */
/* ------------------------------------------------------------------ */
typedef struct {
    int B, Hq, Hkv, S, D;
    double scale;
    const float *q, *k, *v, *scores, *log_decay;
    int n_sink, window, kk;
    const long* rows;
    double *lse, *o, *o_abs;
} attn_ctx;

static void attn_item(void* p, long i, double* z) {
    attn_ctx* c = (attn_ctx*)p;
    long r = c->rows ? c->rows[i] : i;
    int d = (int)(r % c->S);
    int g = (int)((r / c->S) % c->Hq);
    int b = (int)(r / ((long)c->S * c->Hq));
    int h = g / (c->Hq / c->Hkv);
    char* keep = (char*)(z + c->S);
    cand* pool = (cand*)(keep + c->S + 8 - (c->S % 8));
    for (int t = 0; t <= d; ++t) keep[t] = c->scores ? 0 : 1;
    if (c->scores) {  /* sinks, window and the k best of the pool P_d = [s, d-w] */
        const float* sc = c->scores + ((long)b * c->Hkv + h) * c->S;
        float lam = c->log_decay ? c->log_decay[h] : 0.0f;
        for (int t = 0; t <= d && t < c->n_sink; ++t) keep[t] = 1;
        for (int t = d - c->window + 1; t <= d; ++t) if (t >= 0) keep[t] = 1;
        int n_pool = 0;
        for (int t = c->n_sink; t <= d - c->window; ++t) {
            pool[n_pool].score = priority(sc[t], lam, t);
            pool[n_pool].pos = t;
            ++n_pool;
        }
        qsort(pool, (size_t)n_pool, sizeof(cand), cand_cmp);
        for (int j = 0; j < n_pool && j < c->kk; ++j) keep[pool[j].pos] = 1;
    }
    const float* qd = c->q + (((long)b * c->Hq + g) * c->S + d) * c->D;
    const float* kh = c->k + ((long)b * c->Hkv + h) * (long)c->S * c->D;
    const float* vh = c->v + ((long)b * c->Hkv + h) * (long)c->S * c->D;
    double* o = c->o + i * c->D;
    double* a = c->o_abs ? c->o_abs + i * c->D : NULL;
    for (int e = 0; e < c->D; ++e) { o[e] = 0.0; if (a) a[e] = 0.0; }
    double m = -INFINITY;
    for (int t = 0; t <= d; ++t) {
        if (!keep[t]) continue;
        z[t] = c->scale * dot(qd, kh + (long)t * c->D, c->D);
        if (z[t] > m) m = z[t];
    }
    if (m == -INFINITY) { c->lse[i] = -INFINITY; return; }
    double sum = 0.0;
    for (int t = 0; t <= d; ++t) if (keep[t]) sum += exp(z[t] - m);
    double lse = m + log(sum);
    c->lse[i] = lse;
    for (int t = 0; t <= d; ++t) {
        if (!keep[t]) continue;
        double pt = exp(z[t] - lse);
        const float* vt = vh + (long)t * c->D;
        for (int e = 0; e < c->D; ++e) {
            o[e] += pt * (double)vt[e];
            if (a) a[e] += pt * fabs((double)vt[e]);
        }
    }
}

/* scores == NULL: dense causal rows; otherwise the running top-k mask    */
/* with sinks, window, budget and the nullable per-head log_decay.        */
/* rows: flat indices (b*Hq + g)*S + d, or NULL for all rows in order;    */
/* lse [n_rows], o and o_abs [n_rows][D] (o_abs nullable).                */
int oracle_attn_out(int B, int Hq, int Hkv, int S, int D, double scale,
                    const float* q, const float* k, const float* v, const float* scores,
                    const float* log_decay, int n_sink, int window, int budget,
                    long n_rows, const long* rows, double* lse, double* o, double* o_abs,
                    int nthreads) {
    if (B <= 0 || Hq <= 0 || Hkv <= 0 || S <= 0 || D <= 0 || Hq % Hkv) return 1;
    if (scores && (n_sink < 0 || window < 0 || budget - n_sink - window < 0)) return 1;
    attn_ctx c = {B, Hq, Hkv, S, D, scale, q, k, v, scores, log_decay, n_sink, window,
                  budget - n_sink - window, rows, lse, o, o_abs};
    /* doubles: S logits + S flag bytes + S pool entries (8 bytes each) + slack */
    run_items(attn_item, &c, n_rows, nthreads, 2L * S + S / 8 + 4);
    return 0;
}

/* ------------------------------------------------------------------ */
/* Delayed stateful mLSTM scorer (App. A linear-attention background;  */
/* App. E.1 headwise input x = [k; v]; App. E.3 matrix memory C, norm- */
/* alizer n, scalar input/forget gates from headwise projections, the  */
/* stabilised mLSTM form, Hedgehog features; App. E.4 delayed readout  */
/* of u = q - w from the state through q, SiLU readout with a bias).   */
/* Per KV head h and token t, x_t = [k_t; v_t] (2D values):            */
/*   hedgehog(z) = [softmax(z); softmax(-z)]         (2P features)     */
/*   phi_t  = hedgehog(Wk x_t),  val_t = Wv x_t      (E values)        */
/*   ig_t   = wi.x_t + bi,   lf_t = log sigmoid(wf.x_t + bf)          */
/*   m_t    = max(lf_t + m_{t-1}, ig_t)              (m_{-1} = -inf)   */
/*   C_t    = exp(lf_t + m_{t-1} - m_t) C_{t-1} + exp(ig_t - m_t) val_t phi_t^T */
/*   n_t    = exp(lf_t + m_{t-1} - m_t) n_{t-1} + exp(ig_t - m_t) phi_t */
/* After token q has entered, token u = q - w is read out:             */
/*   r = hedgehog(Wr x_u),  h = C_q r / max(|n_q . r|, exp(-m_q))      */
/*   sigma_u = wo . silu(h) + bo,   silu(a) = a / (1 + exp(-a))        */
/* Weights per head: Wk, Wr [P][2D], Wv [E][2D], wi, wf [2D], bi, bf,  */
/* wo [E], bo.  scores[u] is NaN for tokens never read out (u + w      */
/* beyond the last token).  state_out: nullable [B][Hkv][E*2P+2P+1],   */
/* the final (C row-major [E][2P], n, m).                              */
/* ------------------------------------------------------------------ */
static void hedgehog(const double* z, int P, double* phi) {
    double mx = -INFINITY, mn = INFINITY;
    for (int j = 0; j < P; ++j) { if (z[j] > mx) mx = z[j]; if (z[j] < mn) mn = z[j]; }
    double sp = 0.0, sn = 0.0;
    for (int j = 0; j < P; ++j) { sp += exp(z[j] - mx); sn += exp(mn - z[j]); }
    for (int j = 0; j < P; ++j) { phi[j] = exp(z[j] - mx) / sp; phi[P + j] = exp(mn - z[j]) / sn; }
}

static double log_sigmoid(double a) {
    /* log(1 / (1 + exp(-a))), evaluated without overflow */
    return a >= 0 ? -log1p(exp(-a)) : a - log1p(exp(a));
}

int oracle_mlstm_scores(int B, int Hkv, int n_tok, int D, int P, int E, int window,
                        const float* keys, const float* values,
                        const float* wk, const float* wr, const float* wv,
                        const float* wi, const float* bi, const float* wf, const float* bf,
                        const float* wo, const float* bo, double* scores, double* state_out) {
    if (B <= 0 || Hkv <= 0 || n_tok < 0 || D <= 0 || P <= 0 || E <= 0 || window < 0) return 1;
    const int X = 2 * D, F = 2 * P;
    double* x = (double*)malloc(sizeof(double) * (size_t)X * (n_tok > 0 ? n_tok : 1));
    double* C = (double*)malloc(sizeof(double) * (size_t)E * F);
    double* nrm = (double*)malloc(sizeof(double) * F);
    double* z = (double*)malloc(sizeof(double) * P);
    double* phi = (double*)malloc(sizeof(double) * F);
    double* val = (double*)malloc(sizeof(double) * E);
    double* r = (double*)malloc(sizeof(double) * F);
    for (int b = 0; b < B; ++b)
        for (int h = 0; h < Hkv; ++h) {
            long row = (long)b * Hkv + h;
            for (int t = 0; t < n_tok; ++t) {
                const float* kt = keys + (row * n_tok + t) * D;
                const float* vt = values + (row * n_tok + t) * D;
                for (int c = 0; c < D; ++c) { x[(long)t * X + c] = kt[c]; x[(long)t * X + D + c] = vt[c]; }
            }
            for (int i = 0; i < E * F; ++i) C[i] = 0.0;
            for (int j = 0; j < F; ++j) nrm[j] = 0.0;
            double m = -INFINITY;
            for (int t = 0; t < n_tok; ++t) scores[row * n_tok + t] = NAN;
            for (int q = 0; q < n_tok; ++q) {
                const double* xq = x + (long)q * X;
                /* projections of the entering token */
                for (int j = 0; j < P; ++j) {
                    double s = 0.0;
                    for (int c = 0; c < X; ++c) s += (double)wk[((long)h * P + j) * X + c] * xq[c];
                    z[j] = s;
                }
                hedgehog(z, P, phi);
                for (int e = 0; e < E; ++e) {
                    double s = 0.0;
                    for (int c = 0; c < X; ++c) s += (double)wv[((long)h * E + e) * X + c] * xq[c];
                    val[e] = s;
                }
                double ig = bi[h], fg = bf[h];
                for (int c = 0; c < X; ++c) {
                    ig += (double)wi[(long)h * X + c] * xq[c];
                    fg += (double)wf[(long)h * X + c] * xq[c];
                }
                double lf = log_sigmoid(fg);
                double m_new = lf + m > ig ? lf + m : ig;
                double fs = exp(lf + m - m_new); /* 0 for the first token */
                double is = exp(ig - m_new);
                for (int e = 0; e < E; ++e)
                    for (int j = 0; j < F; ++j) C[e * F + j] = fs * C[e * F + j] + is * val[e] * phi[j];
                for (int j = 0; j < F; ++j) nrm[j] = fs * nrm[j] + is * phi[j];
                m = m_new;
                /* delayed readout of u = q - w */
                int u = q - window;
                if (u < 0) continue;
                const double* xu = x + (long)u * X;
                for (int j = 0; j < P; ++j) {
                    double s = 0.0;
                    for (int c = 0; c < X; ++c) s += (double)wr[((long)h * P + j) * X + c] * xu[c];
                    z[j] = s;
                }
                hedgehog(z, P, r);
                double nr = 0.0;
                for (int j = 0; j < F; ++j) nr += nrm[j] * r[j];
                double den = fabs(nr) > exp(-m) ? fabs(nr) : exp(-m);
                double sc = bo[h];
                for (int e = 0; e < E; ++e) {
                    double a = 0.0;
                    for (int j = 0; j < F; ++j) a += C[e * F + j] * r[j];
                    a /= den;
                    sc += (double)wo[(long)h * E + e] * (a / (1.0 + exp(-a)));
                }
                scores[row * n_tok + u] = sc;
            }
            if (state_out) {
                double* so = state_out + row * ((long)E * F + F + 1);
                for (int i = 0; i < E * F; ++i) so[i] = C[i];
                for (int j = 0; j < F; ++j) so[E * F + j] = nrm[j];
                so[E * F + F] = m;
            }
        }
    free(x); free(C); free(nrm); free(z); free(phi); free(val); free(r);
    return 0;
}
