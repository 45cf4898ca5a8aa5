/*
 * fa_oracle.c -- the CPU reference for exact softmax attention with a
 * log-sum-exp side output and its gradient. TEST INFRASTRUCTURE ONLY: it is
 * called by the test suite, by the package's smoke check and by the bench's
 * CPU-baseline leg, never by the op itself. It shares no code, header or
 * constant with the HIP library.
 *
 * What it computes (plain definition, float64 throughout, every score row
 * materialised, no tiling, no online softmax):
 *
 *   S_ij   = cap(scale * <q_i, k_g(h),j>) + M_ij    or -inf where masked / causal
 *   cap(x) = x, or c tanh(x / c) with a logit softcap c > 0 (a score modifier of
 *            llama.cpp pull request 57's list; the cap bounds the product, and the
 *            mask and ALiBi terms are added after it)
 *   m_i    = max(max_j S_ij, sink_h)            (sink_h = -inf without sinks)
 *   row fully masked (m_i = -inf):  O_i = 0, LSE_i = 0, P_i. = 0
 *   otherwise: LSE_i = m_i + ln (sum_j exp(S_ij - m_i) + exp(sink_h - m_i)),
 *              P_ij = exp(S_ij - LSE_i),  O_i = sum_j P_ij v_j
 *   (with ALiBi slopes a_h, S_ij also gets -a_h |j - (q_offset + i)|: a linear
 *   penalty on the distance between key and query positions, llama.cpp pull
 *   request 57's score modifiers; under a causal mask it is a_h (j - q_offset - i))
 *   (an attention sink is one more logit per head in the softmax's denominator,
 *   with no value row: llama.cpp pull request 57, the list of score modifiers
 *   whose flash backward was missing; its own gradient is formed from LSE and
 *   Delta by the Python wrapper)
 *   Delta_i = <dO_i, O_i>
 *   dP_ij   = <dO_i, v_j>,   dS_ij = P_ij (dP_ij - Delta_i) cap'(scale <q_i, k_j>)
 *             (cap' = 1, or 1 - tanh^2 under a softcap)
 *   dQ_i    = scale * sum_j dS_ij k_j
 *   dK_j    = scale * sum_{h in group} sum_i dS_ij q_i
 *   dV_j    =         sum_{h in group} sum_i P_ij dO_i
 *   dM_ij   = P_ij (dP_ij - Delta_i)   (the gradient of the additive term M_ij, which
 *             enters S after the cap: a learnable KQ bias, another modifier on the pull
 *             request's list; 0 where the entry is hidden)
 *
 * Sources on the pages:
 *   - fully masked query rows give O = 0 and LSE = 0, where a plain softmax
 *     would give NaN: "Flash Attn Training" skill page, section 6, trap 9;
 *   - the forward emits O and the LSE, the LSE part receives no gradient:
 *     same page, section 6, trap 3 (packed O|LSE output, zero-scaled slot);
 *   - the backward goes LSE, then D, then the gradients, with the GQA
 *     group-sum: llama.cpp pull request 57, commit 86c140d (tiled
 *     FLASH_ATTN_EXT backward);
 *   - native GQA: query head h reads KV head floor(h / G), G = Hq / Hkv
 *     (skill page, section 6, trap 5; contiguous head groups).
 *
 * Causal convention: query row i sits at key position q_offset + i and sees
 * keys j <= q_offset + i.
 *
 * Layouts: contiguous [B, Hq, Sq, D] for Q, dO, O, dQ; [B, Hkv, Sk, D] for K, V,
 * dK, dV; [B, Hq, Sq] for LSE and Delta; the optional additive mask is
 * [mask_b, mask heads, Sq, Sk] with mask_b = 1 (shared by the batch) or B and mask
 * heads 1 (shared by the heads) or Hq (a per-head score bias).
 */
#include <math.h>
#include <pthread.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#include <unistd.h>

typedef struct {
    int32_t B, Hq, Hkv, Sq, Sk, D;
    int32_t causal;
    int32_t mask_b; /* 0 = no mask, 1 = shared by the batch, B = one per sample */
    int64_t q_offset;
    double scale;
    const double *sinks; /* [Hq] logits, NULL = none */
    const double *alibi; /* [Hq] slopes, NULL = none */
    int32_t mask_h;      /* heads of the mask: 0 or 1 = one mask for every head, Hq = one per head */
    double softcap;      /* logit softcap c, 0 = none */
} ora_problem;

typedef struct {
    const ora_problem *p;
    const double *Q, *K, *V, *M, *dO;
} ora_inputs;

/* ------------------------------------------------------------------------- */
/* element access                                                             */
/* ------------------------------------------------------------------------- */
static const double *q_row(const ora_inputs *in, int b, int h, int i) {
    const ora_problem *p = in->p;
    return in->Q + (((int64_t)b * p->Hq + h) * p->Sq + i) * p->D;
}
static const double *do_row(const ora_inputs *in, int b, int h, int i) {
    const ora_problem *p = in->p;
    return in->dO + (((int64_t)b * p->Hq + h) * p->Sq + i) * p->D;
}
static const double *k_row(const ora_inputs *in, int b, int g, int j) {
    const ora_problem *p = in->p;
    return in->K + (((int64_t)b * p->Hkv + g) * p->Sk + j) * p->D;
}
static const double *v_row(const ora_inputs *in, int b, int g, int j) {
    const ora_problem *p = in->p;
    return in->V + (((int64_t)b * p->Hkv + g) * p->Sk + j) * p->D;
}
static int kv_head(const ora_problem *p, int h) { return h / (p->Hq / p->Hkv); }

static double dot(const double *a, const double *b, int n) {
    double s = 0.0;
    for (int d = 0; d < n; ++d) s += a[d] * b[d];
    return s;
}

/* The mask entry of (b, h, i, j): [mask_b][mask heads][Sq][Sk], a dimension of size 1
 * shared by every batch entry or head. */
static double mask_at(const ora_inputs *in, int b, int h, int i, int j) {
    const ora_problem *p = in->p;
    const int mb = p->mask_b == 1 ? 0 : b;
    const int hm = p->mask_h > 1 ? p->mask_h : 1, mh = p->mask_h > 1 ? h : 0;
    return in->M[(((int64_t)mb * hm + mh) * p->Sq + i) * p->Sk + j];
}

/* Is score (b, h, i, j) visible at all (neither causal- nor mask-excluded)? */
static int visible(const ora_inputs *in, int b, int h, int i, int j) {
    const ora_problem *p = in->p;
    if (p->causal && (int64_t)j > p->q_offset + i) return 0;
    if (p->mask_b) {
        double mv = mask_at(in, b, h, i, j);
        if (isinf(mv) && mv < 0) return 0;
    }
    return 1;
}

/* S_ij for query head h (step 1 of the definition). If dcap is not NULL it receives
 * cap' at the scaled product, the factor dS_ij carries back to the product. */
static double score_d(const ora_inputs *in, int b, int h, int i, int j, double *dcap) {
    const ora_problem *p = in->p;
    if (dcap) *dcap = 1.0;
    if (!visible(in, b, h, i, j)) return -INFINITY;
    double mv = 0.0;
    if (p->mask_b) mv = mask_at(in, b, h, i, j);
    if (p->alibi) mv -= p->alibi[h] * fabs((double)j - (double)(p->q_offset + i));
    int g = kv_head(p, h);
    double x = p->scale * dot(q_row(in, b, h, i), k_row(in, b, g, j), p->D);
    if (p->softcap > 0.0) {
        const double t = tanh(x / p->softcap);
        x = p->softcap * t;
        if (dcap) *dcap = 1.0 - t * t;
    }
    return x + mv;
}
static double score(const ora_inputs *in, int b, int h, int i, int j) { return score_d(in, b, h, i, j, NULL); }

/* Steps 1-4 for one query row: materialise the row of scores, then LSE, O and
 * Delta (Delta only if dO is given). srow is caller scratch of Sk doubles. */
static void row_forward(const ora_inputs *in, int b, int h, int i, double *srow, double *O_out,
                        double *lse_out, double *delta_out) {
    const ora_problem *p = in->p;
    const int D = p->D, Sk = p->Sk, g = kv_head(p, h);
    const double sink = p->sinks ? p->sinks[h] : -INFINITY;
    double m = sink;
    for (int j = 0; j < Sk; ++j) {
        srow[j] = score(in, b, h, i, j);
        if (srow[j] > m) m = srow[j];
    }
    for (int d = 0; d < D; ++d) O_out[d] = 0.0;
    if (m == -INFINITY) { /* fully masked row */
        *lse_out = 0.0;
        if (delta_out) *delta_out = 0.0;
        return;
    }
    double l = exp(sink - m);
    for (int j = 0; j < Sk; ++j) l += exp(srow[j] - m);
    const double lse = m + log(l);
    for (int j = 0; j < Sk; ++j) {
        if (srow[j] == -INFINITY) continue;
        const double pij = exp(srow[j] - lse);
        const double *vj = v_row(in, b, g, j);
        for (int d = 0; d < D; ++d) O_out[d] += pij * vj[d];
    }
    *lse_out = lse;
    if (delta_out) *delta_out = dot(do_row(in, b, h, i), O_out, D);
}

/* Steps 5-6 for one query row: dQ_i, given the row's LSE and Delta. */
static void row_dq(const ora_inputs *in, int b, int h, int i, double lse, double delta, double *dq_out) {
    const ora_problem *p = in->p;
    const int D = p->D, Sk = p->Sk, g = kv_head(p, h);
    for (int d = 0; d < D; ++d) dq_out[d] = 0.0;
    const double *doi = do_row(in, b, h, i);
    for (int j = 0; j < Sk; ++j) {
        double dcap;
        const double s = score_d(in, b, h, i, j, &dcap);
        if (s == -INFINITY) continue;
        const double pij = exp(s - lse);
        const double dpij = dot(doi, v_row(in, b, g, j), D);
        const double dsij = pij * (dpij - delta) * dcap;
        const double *kj = k_row(in, b, g, j);
        for (int d = 0; d < D; ++d) dq_out[d] += p->scale * dsij * kj[d];
    }
}

/* Step 7 for one key column (b, g, j): dK_j and dV_j summed over the group's
 * query heads and all query rows, given every row's LSE and Delta. */
static void col_dkdv(const ora_inputs *in, int b, int g, int j, const double *LSE, const double *Delta,
                     double *dk_out, double *dv_out) {
    const ora_problem *p = in->p;
    const int D = p->D, G = p->Hq / p->Hkv;
    for (int d = 0; d < D; ++d) dk_out[d] = dv_out[d] = 0.0;
    const double *vj = v_row(in, b, g, j);
    for (int h = g * G; h < (g + 1) * G; ++h) {
        for (int i = 0; i < p->Sq; ++i) {
            double dcap;
            const double s = score_d(in, b, h, i, j, &dcap);
            if (s == -INFINITY) continue;
            const int64_t r = ((int64_t)b * p->Hq + h) * p->Sq + i;
            const double pij = exp(s - LSE[r]);
            const double *doi = do_row(in, b, h, i);
            const double dsij = pij * (dot(doi, vj, D) - Delta[r]) * dcap;
            const double *qi = q_row(in, b, h, i);
            for (int d = 0; d < D; ++d) {
                dk_out[d] += p->scale * dsij * qi[d];
                dv_out[d] += pij * doi[d];
            }
        }
    }
}

/* ------------------------------------------------------------------------- */
/* a minimal thread pool: run fn(ctx, idx) for idx in [0, n)                   */
/* ------------------------------------------------------------------------- */
typedef void (*item_fn)(void *ctx, int64_t idx, double *scratch);
typedef struct {
    item_fn fn;
    void *ctx;
    int64_t n;
    int64_t next;
    pthread_mutex_t lock;
    int scratch_len;
} pool_job;

static void *pool_worker(void *arg) {
    pool_job *job = (pool_job *)arg;
    double *scratch = (double *)malloc(sizeof(double) * (size_t)(job->scratch_len > 0 ? job->scratch_len : 1));
    for (;;) {
        pthread_mutex_lock(&job->lock);
        int64_t idx = job->next++;
        pthread_mutex_unlock(&job->lock);
        if (idx >= job->n) break;
        job->fn(job->ctx, idx, scratch);
    }
    free(scratch);
    return NULL;
}

static int run_parallel(item_fn fn, void *ctx, int64_t n, int scratch_len, int nthreads) {
    if (nthreads <= 0) nthreads = (int)sysconf(_SC_NPROCESSORS_ONLN);
    if (nthreads < 1) nthreads = 1;
    if (nthreads > 256) nthreads = 256;
    pool_job job;
    job.fn = fn;
    job.ctx = ctx;
    job.n = n;
    job.next = 0;
    job.scratch_len = scratch_len;
    pthread_mutex_init(&job.lock, NULL);
    pthread_t th[256];
    int started = 0;
    for (int t = 0; t < nthreads; ++t) {
        if (pthread_create(&th[t], NULL, pool_worker, &job) != 0) break;
        ++started;
    }
    if (started == 0) pool_worker(&job);
    for (int t = 0; t < started; ++t) pthread_join(th[t], NULL);
    pthread_mutex_destroy(&job.lock);
    return 0;
}

static int check_problem(const ora_problem *p) {
    if (p->B <= 0 || p->Hq <= 0 || p->Hkv <= 0 || p->Sq <= 0 || p->Sk <= 0 || p->D <= 0) return 1;
    if (p->Hq % p->Hkv) return 2;
    if (p->mask_b != 0 && p->mask_b != 1 && p->mask_b != p->B) return 3;
    if (p->mask_h < 0 || (p->mask_h > 1 && p->mask_h != p->Hq)) return 4;
    if (!(p->softcap >= 0.0) || isinf(p->softcap)) return 5;
    return 0;
}

/* ------------------------------------------------------------------------- */
/* exported entry points                                                      */
/* ------------------------------------------------------------------------- */
typedef struct {
    ora_inputs in;
    double *O, *LSE, *Delta, *dQ;
    const int64_t *rows; /* NULL = every row in order */
    double *dK, *dV;
    const int64_t *cols; /* NULL = every column in order */
} ora_job;

static void fwd_item(void *vctx, int64_t idx, double *srow) {
    ora_job *c = (ora_job *)vctx;
    const ora_problem *p = c->in.p;
    const int64_t r = c->rows ? c->rows[idx] : idx;
    const int i = (int)(r % p->Sq);
    const int h = (int)((r / p->Sq) % p->Hq);
    const int b = (int)(r / ((int64_t)p->Sq * p->Hq));
    double delta = 0.0, lse = 0.0;
    row_forward(&c->in, b, h, i, srow, c->O + idx * p->D, &lse, c->in.dO ? &delta : NULL);
    c->LSE[idx] = lse;
    if (c->Delta) c->Delta[idx] = delta;
    if (c->dQ) row_dq(&c->in, b, h, i, lse, delta, c->dQ + idx * p->D);
}

/* O and LSE for every query row. */
int ora_forward(const ora_problem *p, const double *Q, const double *K, const double *V, const double *M,
                double *O, double *LSE, int nthreads) {
    int e = check_problem(p);
    if (e) return e;
    ora_job c;
    memset(&c, 0, sizeof c);
    c.in.p = p; c.in.Q = Q; c.in.K = K; c.in.V = V; c.in.M = M; c.in.dO = NULL;
    c.O = O; c.LSE = LSE;
    return run_parallel(fwd_item, &c, (int64_t)p->B * p->Hq * p->Sq, p->Sk, nthreads);
}

static void col_item(void *vctx, int64_t idx, double *unused) {
    (void)unused;
    ora_job *c = (ora_job *)vctx;
    const ora_problem *p = c->in.p;
    const int64_t r = c->cols ? c->cols[idx] : idx;
    const int j = (int)(r % p->Sk);
    const int g = (int)((r / p->Sk) % p->Hkv);
    const int b = (int)(r / ((int64_t)p->Sk * p->Hkv));
    col_dkdv(&c->in, b, g, j, c->LSE, c->Delta, c->dK + idx * p->D, c->dV + idx * p->D);
}

/* The whole forward and backward: O, LSE, Delta, dQ for every row, then dK, dV
 * for every key column. */
int ora_backward(const ora_problem *p, const double *Q, const double *K, const double *V, const double *M,
                 const double *dO, double *O, double *LSE, double *Delta, double *dQ, double *dK, double *dV,
                 int nthreads) {
    int e = check_problem(p);
    if (e) return e;
    ora_job c;
    memset(&c, 0, sizeof c);
    c.in.p = p; c.in.Q = Q; c.in.K = K; c.in.V = V; c.in.M = M; c.in.dO = dO;
    c.O = O; c.LSE = LSE; c.Delta = Delta; c.dQ = dQ; c.dK = dK; c.dV = dV;
    run_parallel(fwd_item, &c, (int64_t)p->B * p->Hq * p->Sq, p->Sk, nthreads);
    return run_parallel(col_item, &c, (int64_t)p->B * p->Hkv * p->Sk, 1, nthreads);
}

/* Selected query rows only: rows[n] = (b * Hq + h) * Sq + i. Outputs are packed
 * per selected row: O [n, D], LSE [n], Delta [n], dQ [n, D]. */
int ora_rows(const ora_problem *p, const double *Q, const double *K, const double *V, const double *M,
             const double *dO, int64_t n, const int64_t *rows, double *O, double *LSE, double *Delta,
             double *dQ, int nthreads) {
    int e = check_problem(p);
    if (e) return e;
    ora_job c;
    memset(&c, 0, sizeof c);
    c.in.p = p; c.in.Q = Q; c.in.K = K; c.in.V = V; c.in.M = M; c.in.dO = dO;
    c.O = O; c.LSE = LSE; c.Delta = Delta; c.dQ = dQ; c.rows = rows;
    return run_parallel(fwd_item, &c, n, p->Sk, nthreads);
}

typedef struct {
    ora_inputs in;
    const int64_t *need; /* rows whose LSE / Delta some selected column needs */
    double *LSE, *Delta; /* full-size [B, Hq, Sq] arrays, filled at need[] */
} need_job;

static void need_item(void *vctx, int64_t idx, double *scratch) {
    need_job *c = (need_job *)vctx;
    const ora_problem *p = c->in.p;
    const int64_t r = c->need[idx];
    const int i = (int)(r % p->Sq);
    const int h = (int)((r / p->Sq) % p->Hq);
    const int b = (int)(r / ((int64_t)p->Sq * p->Hq));
    /* scratch holds the score row (Sk) followed by the output row (D) */
    row_forward(&c->in, b, h, i, scratch, scratch + p->Sk, &c->LSE[r], &c->Delta[r]);
}

/* Selected key columns only: cols[n] = (b * Hkv + g) * Sk + j. Outputs dK [n, D]
 * and dV [n, D]. Computes LSE and Delta for exactly the rows that can see one of
 * the selected columns, then sums each column over the group. */
int ora_cols(const ora_problem *p, const double *Q, const double *K, const double *V, const double *M,
             const double *dO, int64_t n, const int64_t *cols, double *dK, double *dV, int nthreads) {
    int e = check_problem(p);
    if (e) return e;
    const int64_t nrows = (int64_t)p->B * p->Hq * p->Sq;
    const int G = p->Hq / p->Hkv;
    unsigned char *flag = (unsigned char *)calloc((size_t)nrows, 1);
    double *LSE = (double *)calloc((size_t)nrows, sizeof(double));
    double *Delta = (double *)calloc((size_t)nrows, sizeof(double));
    int64_t *need = (int64_t *)malloc(sizeof(int64_t) * (size_t)(nrows > 0 ? nrows : 1));
    if (!flag || !LSE || !Delta || !need) {
        free(flag); free(LSE); free(Delta); free(need);
        return 9;
    }
    ora_inputs in;
    in.p = p; in.Q = Q; in.K = K; in.V = V; in.M = M; in.dO = dO;
    for (int64_t c = 0; c < n; ++c) {
        const int j = (int)(cols[c] % p->Sk);
        const int g = (int)((cols[c] / p->Sk) % p->Hkv);
        const int b = (int)(cols[c] / ((int64_t)p->Sk * p->Hkv));
        for (int i = 0; i < p->Sq; ++i)
            for (int h = g * G; h < (g + 1) * G; ++h)
                if (visible(&in, b, h, i, j)) flag[((int64_t)b * p->Hq + h) * p->Sq + i] = 1;
    }
    int64_t nn = 0;
    for (int64_t r = 0; r < nrows; ++r)
        if (flag[r]) need[nn++] = r;
    need_job nj;
    nj.in = in; nj.need = need; nj.LSE = LSE; nj.Delta = Delta;
    run_parallel(need_item, &nj, nn, p->Sk + p->D, nthreads);
    ora_job c;
    memset(&c, 0, sizeof c);
    c.in = in; c.LSE = LSE; c.Delta = Delta; c.dK = dK; c.dV = dV; c.cols = cols;
    run_parallel(col_item, &c, n, 1, nthreads);
    free(flag); free(LSE); free(Delta); free(need);
    return 0;
}

typedef struct {
    ora_inputs in;
    double *dM; /* [B, Hq, Sq, Sk] */
} bias_job;

static void bias_item(void *vctx, int64_t idx, double *scratch) {
    bias_job *c = (bias_job *)vctx;
    const ora_problem *p = c->in.p;
    const int i = (int)(idx % p->Sq);
    const int h = (int)((idx / p->Sq) % p->Hq);
    const int b = (int)(idx / ((int64_t)p->Sq * p->Hq));
    const int g = kv_head(p, h);
    /* scratch holds the score row (Sk) followed by the output row (D) */
    double lse = 0.0, delta = 0.0;
    row_forward(&c->in, b, h, i, scratch, scratch + p->Sk, &lse, &delta);
    double *out = c->dM + idx * p->Sk;
    const double *doi = do_row(&c->in, b, h, i);
    for (int j = 0; j < p->Sk; ++j) {
        const double s = score(&c->in, b, h, i, j);
        if (s == -INFINITY) {
            out[j] = 0.0;
            continue;
        }
        const double pij = exp(s - lse);
        out[j] = pij * (dot(doi, v_row(&c->in, b, g, j), p->D) - delta);
    }
}

/* The gradient of every additive score term, dM [B, Hq, Sq, Sk] = P (dP - Delta) per
 * entry (no cap' factor: the term is added after the cap). The Python wrapper sums it
 * over the mask's broadcast dimensions. */
int ora_score_grad(const ora_problem *p, const double *Q, const double *K, const double *V, const double *M,
                   const double *dO, double *dM, int nthreads) {
    int e = check_problem(p);
    if (e) return e;
    bias_job c;
    memset(&c, 0, sizeof c);
    c.in.p = p; c.in.Q = Q; c.in.K = K; c.in.V = V; c.in.M = M; c.in.dO = dO;
    c.dM = dM;
    return run_parallel(bias_item, &c, (int64_t)p->B * p->Hq * p->Sq, p->Sk + p->D, nthreads);
}
