/*
 * ORACLE -- test infrastructure only.  Plain, slow CPU causal grouped-query
 * attention used to check the HIP path.  Only the tests, the smoke check and
 * the bench's CPU-baseline leg may load it; the library never does.  It shares
 * no code, header or constant with the HIP sources.
 *
 * What it computes (the plain definition of the operator the KernelBraid /
 * AReaL-TIK README builds its kernels around):
 *   - "Features": BF16 causal attention over contiguous [batch, heads,
 *     sequence, head_dim] tensors, 32 query heads and 8 KV heads.
 *   - "Usage": unified_prefill(q, k, v, H_Q, H_KV) is the causal
 *     full-sequence forward; unified_decode(q[:, :, -1:], k, v, H_Q, H_KV)
 *     is the last query token attending to the whole KV context, and equals
 *     the last prefill row.  The output has the shape of the query.
 *   - "Method": a partitioned forward runs a chunk of query rows against
 *     the cached keys.
 * Readings where the pages are silent (each listed in the design notes):
 *   - query row r of a call with q_len rows over kv_len cached keys sits at
 *     absolute position pos = kv_len - q_len + r and sees keys 0..pos
 *     (bottom-right causal; it is the only alignment under which decode of
 *     the last token equals the last prefill row);
 *   - query head h reads KV head h / (Hq / Hkv) (contiguous groups);
 *   - scores are scale * <q, k>, scale given by the caller (1/sqrt(D) in the
 *     workloads); softmax in REAL precision from the bf16 inputs widened
 *     exactly; the output is left unrounded.
 *
 * Per row:   s_j = scale * sum_d q[d] k_j[d]            (j = 0..pos)
 *            m   = max_j s_j,  e_j = exp(s_j - m),  l = sum_j e_j
 *            o[d] = (sum_j e_j v_j[d]) / l,   lse = m + log(l)
 * Subtracting m changes nothing mathematically; it only keeps exp finite.
 *
 * Gradients (the pages cover the forward only and say that training forward
 * and backward still run, README "Background"; the backward is the
 * derivative of the operator above, written out; full causal sequences,
 * q_len == kv_len):  with P_ij = e_j / l of row i and an upstream gradient
 * dO,
 *            dV_j  = sum_i P_ij dO_i
 *            dP_ij = <dO_i, v_j>,   D_i = <dO_i, o_i> = sum_j P_ij dP_ij
 *            dS_ij = P_ij (dP_ij - D_i)
 *            dQ_i  = scale sum_j dS_ij k_j,   dK_j = scale sum_i dS_ij q_i
 * with dK, dV summed over the query heads that share a KV head.
 *
 * Build: gcc -std=c11 -O2 -ffp-contract=off -DKBO_REAL=double|float.
 * The exported names carry the precision suffix (_f64 or _f32).
 */
#include <math.h>
#include <pthread.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#ifndef KBO_REAL
#define KBO_REAL double
#endif
#ifndef KBO_SUFFIX
#define KBO_SUFFIX _f64
#endif
#define KBO_CAT2(a, b) a##b
#define KBO_CAT(a, b) KBO_CAT2(a, b)
#define KBO_NAME(n) KBO_CAT(n, KBO_SUFFIX)

typedef KBO_REAL real;

static real kbo_exp(real x) { return (sizeof(real) == sizeof(float)) ? (real)expf((float)x) : (real)exp((double)x); }
static real kbo_log(real x) { return (sizeof(real) == sizeof(float)) ? (real)logf((float)x) : (real)log((double)x); }

/* bf16 bit pattern -> value: the 16 bits are the upper half of an fp32. */
static real widen(uint16_t b) {
    uint32_t u = (uint32_t)b << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return (real)f;
}

typedef struct {
    const uint16_t *q, *k, *v;
    int64_t batch, n_q_heads, n_kv_heads, q_len, kv_len, kv_capacity, head_dim;
    real scale;
} problem_t;

/* One output row (b, h, r).  s must hold pos+1 values; w (optional) receives
 * the normalised weights e_j / l.  out receives head_dim values. */
static void attention_row(const problem_t* p, int64_t b, int64_t h, int64_t r, real* s, real* out,
                          double* w, real* lse) {
    const int64_t D = p->head_dim;
    const int64_t pos = p->kv_len - p->q_len + r;
    const int64_t g = h / (p->n_q_heads / p->n_kv_heads);
    const uint16_t* qrow = p->q + ((b * p->n_q_heads + h) * p->q_len + r) * D;
    const uint16_t* kbase = p->k + (b * p->n_kv_heads + g) * p->kv_capacity * D;
    const uint16_t* vbase = p->v + (b * p->n_kv_heads + g) * p->kv_capacity * D;

    for (int64_t j = 0; j <= pos; ++j) {
        real dot = 0;
        for (int64_t d = 0; d < D; ++d) dot += widen(qrow[d]) * widen(kbase[j * D + d]);
        s[j] = p->scale * dot;
    }
    real m = s[0];
    for (int64_t j = 1; j <= pos; ++j)
        if (s[j] > m) m = s[j];
    real l = 0;
    for (int64_t j = 0; j <= pos; ++j) {
        s[j] = kbo_exp(s[j] - m);
        l += s[j];
    }
    for (int64_t d = 0; d < D; ++d) out[d] = 0;
    for (int64_t j = 0; j <= pos; ++j)
        for (int64_t d = 0; d < D; ++d) out[d] += s[j] * widen(vbase[j * D + d]);
    for (int64_t d = 0; d < D; ++d) out[d] /= l;
    if (lse) *lse = m + kbo_log(l);
    if (w)
        for (int64_t j = 0; j <= pos; ++j) w[j] = (double)(s[j] / l);
}

typedef struct {
    const problem_t* p;
    const int64_t* rows; /* flat row ids into [batch, n_q_heads, q_len], or NULL = identity */
    int64_t begin, end;
    double* out;
    double* lse; /* optional: receives each row's log-sum-exp */
    int status;
} job_t;

static void* worker(void* arg) {
    job_t* jb = (job_t*)arg;
    const problem_t* p = jb->p;
    real* s = (real*)malloc(sizeof(real) * (size_t)(p->kv_len > 0 ? p->kv_len : 1));
    real* o = (real*)malloc(sizeof(real) * (size_t)p->head_dim);
    if (!s || !o) {
        jb->status = -3;
        free(s);
        free(o);
        return NULL;
    }
    real lse = 0;
    for (int64_t i = jb->begin; i < jb->end; ++i) {
        const int64_t flat = jb->rows ? jb->rows[i] : i;
        const int64_t r = flat % p->q_len;
        const int64_t h = (flat / p->q_len) % p->n_q_heads;
        const int64_t b = flat / (p->q_len * p->n_q_heads);
        attention_row(p, b, h, r, s, o, NULL, jb->lse ? &lse : NULL);
        if (jb->lse) jb->lse[i] = (double)lse;
        for (int64_t d = 0; d < p->head_dim; ++d) jb->out[i * p->head_dim + d] = (double)o[d];
    }
    free(s);
    free(o);
    return NULL;
}

static int check_problem(const problem_t* p) {
    if (!p->q || !p->k || !p->v) return -1;
    if (p->batch < 1 || p->n_q_heads < 1 || p->n_kv_heads < 1 || p->head_dim < 1) return -1;
    if (p->n_q_heads % p->n_kv_heads) return -1;
    if (p->q_len < 1 || p->q_len > p->kv_len || p->kv_len > p->kv_capacity) return -1;
    return 0;
}

/*
 * q [batch, n_q_heads, q_len, head_dim], k/v [batch, n_kv_heads, kv_capacity,
 * head_dim], all bf16 bit patterns.  Computes the rows listed in `rows` (flat
 * ids b*n_q_heads*q_len + h*q_len + r) or every row when rows == NULL
 * (n_rows is then ignored).  out receives n_rows x head_dim doubles and lse
 * (when not NULL) the n_rows log-sum-exps log(sum_j exp(s_j)).
 * Returns 0, or -1 for a malformed problem, -2 for a thread failure, -3 when
 * out of memory.
 */
int KBO_NAME(kbo_attention)(const uint16_t* q, const uint16_t* k, const uint16_t* v, int64_t batch,
                            int64_t n_q_heads, int64_t n_kv_heads, int64_t q_len, int64_t kv_len,
                            int64_t kv_capacity, int64_t head_dim, double scale, const int64_t* rows,
                            int64_t n_rows, double* out, double* lse, int n_threads) {
    problem_t p = {q, k, v, batch, n_q_heads, n_kv_heads, q_len, kv_len, kv_capacity, head_dim, (real)scale};
    if (check_problem(&p) || !out) return -1;
    const int64_t total = batch * n_q_heads * q_len;
    if (!rows) n_rows = total;
    for (int64_t i = 0; rows && i < n_rows; ++i)
        if (rows[i] < 0 || rows[i] >= total) return -1;
    if (n_threads < 1) n_threads = 1;
    if (n_threads > 256) n_threads = 256;
    if (n_threads > n_rows) n_threads = (int)(n_rows > 0 ? n_rows : 1);
    pthread_t tid[256];
    job_t jobs[256];
    for (int t = 0; t < n_threads; ++t) {
        jobs[t] = (job_t){&p, rows, n_rows * t / n_threads, n_rows * (t + 1) / n_threads, out, lse, 0};
    }
    int rc = 0;
    int started = 1;
    for (int t = 1; t < n_threads; ++t, ++started)
        if (pthread_create(&tid[t], NULL, worker, &jobs[t]) != 0) {
            rc = -2;
            break;
        }
    worker(&jobs[0]);
    for (int t = 1; t < started; ++t) pthread_join(tid[t], NULL);
    for (int t = 0; t < n_threads && !rc; ++t) rc = jobs[t].status;
    return rc;
}

/* The normalised softmax weights of one row (flat id as above): w[0..pos]. */
int KBO_NAME(kbo_weights)(const uint16_t* q, const uint16_t* k, const uint16_t* v, int64_t batch,
                          int64_t n_q_heads, int64_t n_kv_heads, int64_t q_len, int64_t kv_len,
                          int64_t kv_capacity, int64_t head_dim, double scale, int64_t row, double* w) {
    problem_t p = {q, k, v, batch, n_q_heads, n_kv_heads, q_len, kv_len, kv_capacity, head_dim, (real)scale};
    if (check_problem(&p) || !w || row < 0 || row >= batch * n_q_heads * q_len) return -1;
    real* s = (real*)malloc(sizeof(real) * (size_t)kv_len);
    real* o = (real*)malloc(sizeof(real) * (size_t)head_dim);
    if (!s || !o) {
        free(s);
        free(o);
        return -3;
    }
    const int64_t r = row % q_len;
    const int64_t h = (row / q_len) % n_q_heads;
    const int64_t b = row / (q_len * n_q_heads);
    attention_row(&p, b, h, r, s, o, w, NULL);
    free(s);
    free(o);
    return 0;
}

/* ------------------------------------------------------------------------
 * Backward of full causal sequences (q_len == kv_len == kv_capacity == S).
 * dout is the upstream gradient dO, bf16 bits shaped like q.  The error
 * budgets are sums of absolute values, in the same loops, that bound how far
 * a computation in fp32 with bf16-rounded operands may land from the exact
 * gradient (each weighted sum term carries at most a few bf16 roundings):
 *   eq_id = scale sum_j (|dS_ij| + P_ij A_i) |k_jd|
 *   ek_jd = scale sum_i (|dS_ij| + P_ij A_i) |q_id|
 *   ev_jd = sum_i P_ij |dO_id|
 * with A_i = sum_j P_ij sum_d |dO_id| |v_jd| (the size of D_i's terms).
 * ------------------------------------------------------------------------ */

/* P (into w), dS (into ds) and A_i of row i of head h, sequence b. */
static real row_grad(const problem_t* p, const uint16_t* dout, int64_t b, int64_t h, int64_t i, real* s,
                     real* o, double* w, real* ds, int want_budget) {
    const int64_t D = p->head_dim, S = p->kv_len;
    const int64_t g = h / (p->n_q_heads / p->n_kv_heads);
    const uint16_t* vrows = p->v + (b * p->n_kv_heads + g) * S * D;
    const uint16_t* dorow = dout + ((b * p->n_q_heads + h) * S + i) * D;
    attention_row(p, b, h, i, s, o, w, NULL);
    real Di = 0;
    for (int64_t d = 0; d < D; ++d) Di += widen(dorow[d]) * o[d];
    real Ai = 0;
    for (int64_t j = 0; j <= i; ++j) {
        real dp = 0, mag = 0;
        for (int64_t d = 0; d < D; ++d) {
            dp += widen(dorow[d]) * widen(vrows[j * D + d]);
            if (want_budget) mag += fabs((double)widen(dorow[d])) * fabs((double)widen(vrows[j * D + d]));
        }
        ds[j] = (real)w[j] * (dp - Di);
        Ai += (real)w[j] * mag;
    }
    return Ai;
}

typedef struct {
    const problem_t* p;
    const uint16_t* dout;
    int64_t row_from;
    int64_t begin, end; /* (b, g) pairs, or flat rows for the dq-rows form */
    const int64_t* rows;
    double *dq, *dk, *dv, *eq, *ek, *ev;
    int status;
} bjob_t;

static void* bwd_worker(void* arg) {
    bjob_t* jb = (bjob_t*)arg;
    const problem_t* p = jb->p;
    const int64_t D = p->head_dim, S = p->kv_len, Hq = p->n_q_heads, Hkv = p->n_kv_heads;
    const int64_t hpg = Hq / Hkv;
    const int budget = jb->eq || jb->ek || jb->ev;
    real* s = (real*)malloc(sizeof(real) * (size_t)S);
    real* o = (real*)malloc(sizeof(real) * (size_t)D);
    real* ds = (real*)malloc(sizeof(real) * (size_t)S);
    double* w = (double*)malloc(sizeof(double) * (size_t)S);
    if (!s || !o || !ds || !w) {
        jb->status = -3;
        free(s);
        free(o);
        free(ds);
        free(w);
        return NULL;
    }
    for (int64_t x = jb->begin; x < jb->end; ++x) {
        int64_t b, g, h_first, h_end, i_first, i_end;
        if (jb->rows) { /* one listed row: dq only */
            const int64_t flat = jb->rows[x];
            b = flat / (Hq * S);
            h_first = (flat / S) % Hq;
            h_end = h_first + 1;
            i_first = flat % S;
            i_end = i_first + 1;
            g = h_first / hpg;
        } else { /* one (b, g) pair: every head of the group, rows row_from.. */
            b = x / Hkv;
            g = x % Hkv;
            h_first = g * hpg;
            h_end = h_first + hpg;
            i_first = jb->row_from;
            i_end = S;
        }
        const uint16_t* krows = p->k + (b * Hkv + g) * S * D;
        double* dkb = jb->dk ? jb->dk + (b * Hkv + g) * S * D : NULL;
        double* dvb = jb->dv ? jb->dv + (b * Hkv + g) * S * D : NULL;
        double* ekb = jb->ek ? jb->ek + (b * Hkv + g) * S * D : NULL;
        double* evb = jb->ev ? jb->ev + (b * Hkv + g) * S * D : NULL;
        for (int64_t h = h_first; h < h_end; ++h) {
            for (int64_t i = i_first; i < i_end; ++i) {
                const real Ai = row_grad(p, jb->dout, b, h, i, s, o, w, ds, budget);
                const uint16_t* qrow = p->q + ((b * Hq + h) * S + i) * D;
                const uint16_t* dorow = jb->dout + ((b * Hq + h) * S + i) * D;
                const int64_t out_row = jb->rows ? x : (b * Hq + h) * S + i;
                if (jb->dq) {
                    double* dqr = jb->dq + out_row * D;
                    double* eqr = jb->eq ? jb->eq + out_row * D : NULL;
                    for (int64_t d = 0; d < D; ++d) {
                        real acc = 0, bud = 0;
                        for (int64_t j = 0; j <= i; ++j) {
                            acc += ds[j] * widen(krows[j * D + d]);
                            if (eqr) bud += (fabs((double)ds[j]) + w[j] * Ai) * fabs((double)widen(krows[j * D + d]));
                        }
                        dqr[d] = (double)(p->scale * acc);
                        if (eqr) eqr[d] = (double)(p->scale * bud);
                    }
                }
                if (jb->rows) continue;
                for (int64_t j = 0; j <= i; ++j) {
                    for (int64_t d = 0; d < D; ++d) {
                        const real qd = widen(qrow[d]), dod = widen(dorow[d]);
                        if (dkb) dkb[j * D + d] += (double)(p->scale * ds[j] * qd);
                        if (dvb) dvb[j * D + d] += (double)((real)w[j] * dod);
                        if (ekb) ekb[j * D + d] += (double)p->scale * (fabs((double)ds[j]) + w[j] * Ai) * fabs((double)qd);
                        if (evb) evb[j * D + d] += w[j] * fabs((double)dod);
                    }
                }
            }
        }
    }
    free(s);
    free(o);
    free(ds);
    free(w);
    return NULL;
}

static int run_bwd(bjob_t* proto, int64_t n_items, int n_threads) {
    if (n_threads < 1) n_threads = 1;
    if (n_threads > 256) n_threads = 256;
    if (n_threads > n_items) n_threads = (int)(n_items > 0 ? n_items : 1);
    pthread_t tid[256];
    bjob_t jobs[256];
    for (int t = 0; t < n_threads; ++t) {
        jobs[t] = *proto;
        jobs[t].begin = n_items * t / n_threads;
        jobs[t].end = n_items * (t + 1) / n_threads;
        jobs[t].status = 0;
    }
    int rc = 0, started = 1;
    for (int t = 1; t < n_threads; ++t, ++started)
        if (pthread_create(&tid[t], NULL, bwd_worker, &jobs[t]) != 0) {
            rc = -2;
            break;
        }
    bwd_worker(&jobs[0]);
    for (int t = 1; t < started; ++t) pthread_join(tid[t], NULL);
    for (int t = 0; t < n_threads && !rc; ++t) rc = jobs[t].status;
    return rc;
}

/*
 * Gradients of full causal sequences: q, dout [batch, n_q_heads, S, D] and
 * k, v [batch, n_kv_heads, S, D] as bf16 bits.  Rows below row_from are
 * skipped: dq is then written for rows >= row_from only, and dk, dv hold the
 * exact gradient for keys >= row_from (earlier rows never see those keys).
 * dq [batch, n_q_heads, S, D] and dk, dv [batch, n_kv_heads, S, D] doubles
 * (dk, dv, ek, ev must start at zero); any of dq, dk, dv and the budgets
 * eq, ek, ev may be NULL.  Returns 0 or a negative code as above.
 */
int KBO_NAME(kbo_backward)(const uint16_t* q, const uint16_t* k, const uint16_t* v, const uint16_t* dout,
                           int64_t batch, int64_t n_q_heads, int64_t n_kv_heads, int64_t seq_len,
                           int64_t head_dim, double scale, int64_t row_from, double* dq, double* dk, double* dv,
                           double* eq, double* ek, double* ev, int n_threads) {
    problem_t p = {q, k, v, batch, n_q_heads, n_kv_heads, seq_len, seq_len, seq_len, head_dim, (real)scale};
    if (check_problem(&p) || !dout || row_from < 0 || row_from >= seq_len) return -1;
    bjob_t proto = {&p, dout, row_from, 0, 0, NULL, dq, dk, dv, eq, ek, ev, 0};
    return run_bwd(&proto, batch * n_kv_heads, n_threads);
}

/* dq (and its budget eq, optional) of the listed flat rows b*Hq*S + h*S + i
 * only: dq, eq receive n_rows x head_dim doubles. */
int KBO_NAME(kbo_backward_dq_rows)(const uint16_t* q, const uint16_t* k, const uint16_t* v, const uint16_t* dout,
                                   int64_t batch, int64_t n_q_heads, int64_t n_kv_heads, int64_t seq_len,
                                   int64_t head_dim, double scale, const int64_t* rows, int64_t n_rows, double* dq,
                                   double* eq, int n_threads) {
    problem_t p = {q, k, v, batch, n_q_heads, n_kv_heads, seq_len, seq_len, seq_len, head_dim, (real)scale};
    if (check_problem(&p) || !dout || !rows || !dq || n_rows < 1) return -1;
    for (int64_t i = 0; i < n_rows; ++i)
        if (rows[i] < 0 || rows[i] >= batch * n_q_heads * seq_len) return -1;
    bjob_t proto = {&p, dout, 0, 0, 0, rows, dq, NULL, NULL, eq, NULL, NULL, 0};
    return run_bwd(&proto, n_rows, n_threads);
}
