/*
 * fp64 CPU oracle for scaled dot-product attention (forward).
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the product path may link, load or
 * call this file: only the test suite, the smoke check and the benchmark's
 * CPU-baseline leg use it.  It shares no code, header or constant with the
 * GPU library.
 *
 * What it computes (the plain, non-online definition):
 *   VeriTile, "FlashAttention1.NaiveRefinement", section "Naive FA reference":
 *   `fa1NaiveReference4D` = `attentionReal4D`, i.e. softmax(Q K^T * scale) V
 *   for every (batch, head) slice, output indexed like Q; and
 *   `fa1NaiveCausalReference4D` = `attentionReal4DCausal`, its causal form.
 *   The same page's refinement theorems state that the tiled FA-1 kernels
 *   (non-causal and causal, with S_q / S_k boundaries and a head-dim tail)
 *   equal these references exactly in real arithmetic, so the oracle is the
 *   reference itself, evaluated in double precision.
 *
 * Order of operations per query row, as the reductions are chained on
 *   tiny.accy.kernel.library.attention (the `reductions` list of the
 *   scaled-dot-product specialization, and the test helper `expectedOutput`):
 *     1. score_dot       s_j = scale * sum_d Q[i,d] K[j,d]   (dot first, then scale)
 *     2. score_max       m   = max_j s_j, starting from -infinity
 *     3. score_exp_sum   l   = sum_j exp(s_j - m)
 *     4. weighted_sum    O[i,e] = sum_j (exp(s_j - m) / l) * V[j,e]
 *                        (the weight is formed first, then multiplied)
 *   plus LSE[i] = m + ln(l)  (natural log of the sum of exp of scaled scores).
 *   The key width D_qk may differ from the value width D_v (equation
 *   "bqh,bkh,bkv->bqv" on the same page).
 *
 * Readings where the pages are silent (each listed in the design notes):
 *   - causal: key j is visible to query i iff j <= i (top-left alignment);
 *     rows i >= S_k therefore see every key;
 *   - masked keys are simply left out of every sum (exact);
 *   - LSE uses the natural logarithm of the scaled scores.
 *
 * The extended entry point (attn_ref_ext_f64) restricts each row to one
 * contiguous key range, which covers the page-2 variants:
 *   - a key range [kv_begin, kv_end): one chunk of a split key sequence
 *     (the continuation case of attention_fwd_triton3, whose partial
 *     results merge into the full one);
 *   - a signed causal offset: key j visible iff j <= i + causal_offset
 *     (attention_llama's start_position shifts the diagonal; S_k - S_q
 *     aligns it to the bottom-right corner);
 *   - a window W > 0: only keys j > i + causal_offset - W (the sliding
 *     window of attention_fwd_triton3 case 1, read as the W keys ending at
 *     the diagonal).
 *   A row that sees no key gets O = 0 and LSE = -infinity (the neutral
 *   element of the merge).
 *   It also takes grouped K/V heads: K and V hold H_kv heads (H a multiple
 *   of H_kv) and query head h reads K/V head h / (H / H_kv), the key
 *   address of attention_score on the same page (program p of batch p / H
 *   reads K head (p mod H) / (H / H_KV)); H_kv = H is the plain layout.
 *
 * attn_ref_scaled_f64 is the base-2 attention with per-block Q and K scales
 * of attention_forward_triton on the same page (`attentionRealBase2PerKeyScale`
 * over `keyScale` built from Q_scale, one value per BLOCK_M query rows, and
 * K_scale, one per BLOCK_N keys):
 *     s_ij = Q_scale[b,h,i / q_block] * K_scale[b,h,j / k_block] * (Q_i . K_j)
 *     O_i  = sum_j 2^(s_ij) V_j / sum_j 2^(s_ij),   LSE_i = ln sum_j 2^(s_ij).
 *   2^x = exp(x ln 2), so this is the plain definition with the score
 *   multiplied by ln 2 * Q_scale * K_scale (the definition's body is not
 *   printed; this is the reading the name and the scale layout support).
 *
 * Layout: contiguous row-major Q[B,H,S_q,D_qk], K[B,H,S_k,D_qk],
 * V[B,H,S_k,D_v], O[B,H,S_q,D_v], LSE[B,H,S_q] (all double).
 * With a row list, only those query rows are computed and O / LSE are
 * packed as [B,H,n_rows,D_v] / [B,H,n_rows].
 */
#include <math.h>
#include <pthread.h>
#include <stdint.h>
#include <stdlib.h>

typedef struct {
    const double *Q, *K, *V;
    double *O, *LSE, *P;
    int64_t B, H, H_kv, S_q, S_k, D_qk, D_v;
    double scale;
    int causal;
    int64_t coff, window, kv_begin, kv_end;   /* key range of every row, see above */
    const double *q_scale, *k_scale;          /* per-block scales, or NULL */
    int64_t q_block, k_block;
    const int64_t *rows;
    int64_t n_rows;          /* rows computed per slice */
    int64_t first, last;     /* work items [first, last) over slices*n_rows */
    int status;
} oracle_job;

/* One query row of one (batch, head) slice. */
static void oracle_row(const oracle_job *jb, int64_t slice, int64_t out_row,
                       int64_t i, double *s, double *w, double *acc)
{
    const double *q = jb->Q + (slice * jb->S_q + i) * jb->D_qk;
    /* K/V head of this query head: H / H_kv consecutive query heads share one */
    const int64_t kv_slice = (slice / jb->H) * jb->H_kv + (slice % jb->H) / (jb->H / jb->H_kv);
    const double *k = jb->K + kv_slice * jb->S_k * jb->D_qk;
    const double *v = jb->V + kv_slice * jb->S_k * jb->D_v;

    /* visible keys j in [lo, hi): the key range, then j <= i + coff when
       causal, then j > i + coff - window when windowed */
    int64_t lo = jb->kv_begin, hi = jb->kv_end;
    if (jb->causal && i + jb->coff + 1 < hi)
        hi = i + jb->coff + 1;
    if (jb->window > 0 && i + jb->coff - jb->window + 1 > lo)
        lo = i + jb->coff - jb->window + 1;

    double *o = jb->O + (slice * jb->n_rows + out_row) * jb->D_v;
    if (hi <= lo) {
        /* no visible key: the merge's neutral element */
        for (int64_t e = 0; e < jb->D_v; ++e)
            o[e] = 0.0;
        if (jb->LSE)
            jb->LSE[slice * jb->n_rows + out_row] = -INFINITY;
        if (jb->P) {
            double *p = jb->P + (slice * jb->n_rows + out_row) * jb->S_k;
            for (int64_t j = 0; j < jb->S_k; ++j)
                p[j] = 0.0;
        }
        return;
    }

    /* 1. score_dot, then the scale */
    for (int64_t j = lo; j < hi; ++j) {
        double dot = 0.0;
        for (int64_t d = 0; d < jb->D_qk; ++d)
            dot += q[d] * k[j * jb->D_qk + d];
        s[j] = jb->scale * dot;
        if (jb->q_scale)   /* the query block's and the key block's scales */
            s[j] *= jb->q_scale[slice * ((jb->S_q + jb->q_block - 1) / jb->q_block) +
                                i / jb->q_block] *
                    jb->k_scale[slice * ((jb->S_k + jb->k_block - 1) / jb->k_block) +
                                j / jb->k_block];
    }
    /* 2. score_max, seeded with -infinity */
    double m = -INFINITY;
    for (int64_t j = lo; j < hi; ++j)
        if (s[j] > m)
            m = s[j];
    /* 3. score_exp_sum: the shifted exponentials summed */
    double l = 0.0;
    for (int64_t j = lo; j < hi; ++j)
        l += exp(s[j] - m);
    /* 4. weighted_sum: weight = exp(s_j - m) / l, then weight * V[j, e] */
    for (int64_t j = lo; j < hi; ++j)
        w[j] = exp(s[j] - m) / l;
    for (int64_t e = 0; e < jb->D_v; ++e)
        acc[e] = 0.0;
    for (int64_t j = lo; j < hi; ++j)
        for (int64_t e = 0; e < jb->D_v; ++e)
            acc[e] += w[j] * v[j * jb->D_v + e];

    for (int64_t e = 0; e < jb->D_v; ++e)
        o[e] = acc[e];
    if (jb->LSE)
        jb->LSE[slice * jb->n_rows + out_row] = m + log(l);
    if (jb->P) {
        double *p = jb->P + (slice * jb->n_rows + out_row) * jb->S_k;
        for (int64_t j = 0; j < jb->S_k; ++j)
            p[j] = (j >= lo && j < hi) ? w[j] : 0.0;
    }
}

static void *oracle_worker(void *arg)
{
    oracle_job *jb = (oracle_job *)arg;
    double *s = (double *)malloc(sizeof(double) * (size_t)jb->S_k);
    double *w = (double *)malloc(sizeof(double) * (size_t)jb->S_k);
    double *acc = (double *)malloc(sizeof(double) * (size_t)jb->D_v);
    if (!s || !w || !acc) {
        jb->status = 3;
    } else {
        for (int64_t it = jb->first; it < jb->last; ++it) {
            int64_t slice = it / jb->n_rows;
            int64_t r = it % jb->n_rows;
            int64_t i = jb->rows ? jb->rows[r] : r;
            oracle_row(jb, slice, r, i, s, w, acc);
        }
    }
    free(s);
    free(w);
    free(acc);
    return NULL;
}

/* Validate the row list, then split the B*H*n_rows rows over threads. */
static int run_jobs(const oracle_job *proto, int nthreads)
{
    int64_t n_rows = proto->n_rows;
    if (proto->rows) {
        if (n_rows < 1)
            return 1;
        for (int64_t r = 0; r < n_rows; ++r)
            if (proto->rows[r] < 0 || proto->rows[r] >= proto->S_q)
                return 1;
    } else {
        n_rows = proto->S_q;
    }
    int64_t total = proto->B * proto->H * n_rows;
    if (nthreads < 1)
        nthreads = 1;
    if ((int64_t)nthreads > total)
        nthreads = (int)total;

    oracle_job *jobs = (oracle_job *)calloc((size_t)nthreads, sizeof(oracle_job));
    pthread_t *tids = (pthread_t *)calloc((size_t)nthreads, sizeof(pthread_t));
    if (!jobs || !tids) {
        free(jobs);
        free(tids);
        return 3;
    }
    int rc = 0, started = 0;
    for (int t = 0; t < nthreads; ++t) {
        oracle_job *jb = &jobs[t];
        *jb = *proto;
        jb->n_rows = n_rows;
        jb->first = total * t / nthreads;
        jb->last = total * (t + 1) / nthreads;
        jb->status = 0;
    }
    for (int t = 1; t < nthreads; ++t) {
        if (pthread_create(&tids[t], NULL, oracle_worker, &jobs[t]) != 0) {
            rc = 2;
            break;
        }
        started = t;
    }
    if (rc == 0)
        oracle_worker(&jobs[0]);
    for (int t = 1; t <= started; ++t)
        pthread_join(tids[t], NULL);
    for (int t = 0; t < nthreads && rc == 0; ++t)
        if (jobs[t].status)
            rc = jobs[t].status;
    free(jobs);
    free(tids);
    return rc;
}

/*
 * attn_ref_ext_f64: the definition above with each row's keys restricted to
 * [max(kv_begin, i + causal_offset - window + 1) (window > 0 only),
 *  min(kv_end, i + causal_offset + 1) (causal only)).
 * Requires 0 <= kv_begin <= kv_end <= S_k, window >= 0 and H_kv >= 1
 * dividing H; K is [B,H_kv,S_k,D_qk] and V [B,H_kv,S_k,D_v].
 *
 * Returns 0 on success, 1 for a bad argument (null pointer, a dimension
 * below 1, a row index outside [0, S_q), a key range outside [0, S_k]),
 * 2 if a thread could not be started, 3 if a work buffer could not be
 * allocated.  P, when not NULL, receives the softmax weights
 * [B,H,rows,S_k] (0 where a key is masked); LSE may be NULL.
 */
int attn_ref_ext_f64(const double *Q, const double *K, const double *V,
                     double *O, double *LSE, double *P,
                     int64_t B, int64_t H, int64_t H_kv, int64_t S_q, int64_t S_k,
                     int64_t D_qk, int64_t D_v, double scale, int causal,
                     int64_t causal_offset, int64_t window, int64_t kv_begin,
                     int64_t kv_end, const int64_t *rows, int64_t n_rows, int nthreads)
{
    if (!Q || !K || !V || !O)
        return 1;
    if (B < 1 || H < 1 || S_q < 1 || S_k < 1 || D_qk < 1 || D_v < 1)
        return 1;
    if (kv_begin < 0 || kv_end < kv_begin || kv_end > S_k || window < 0)
        return 1;
    if (H_kv < 1 || H % H_kv != 0)
        return 1;
    oracle_job proto = {0};
    proto.Q = Q; proto.K = K; proto.V = V;
    proto.O = O; proto.LSE = LSE; proto.P = P;
    proto.B = B; proto.H = H; proto.H_kv = H_kv; proto.S_q = S_q; proto.S_k = S_k;
    proto.D_qk = D_qk; proto.D_v = D_v;
    proto.scale = scale; proto.causal = causal;
    proto.coff = causal_offset; proto.window = window;
    proto.kv_begin = kv_begin; proto.kv_end = kv_end;
    proto.rows = rows; proto.n_rows = n_rows;
    return run_jobs(&proto, nthreads);
}

/*
 * attn_ref_scaled_f64: base-2 attention with per-block scales (see the top
 * of this file).  Q_scale is [B,H,ceil(S_q/q_block)], K_scale
 * [B,H,ceil(S_k/k_block)]; causal is top-left as in attn_ref_f64.  Same
 * return codes as attn_ref_ext_f64.
 */
int attn_ref_scaled_f64(const double *Q, const double *K, const double *V,
                        double *O, double *LSE, double *P,
                        const double *Q_scale, const double *K_scale,
                        int64_t B, int64_t H, int64_t S_q, int64_t S_k,
                        int64_t D_qk, int64_t D_v, int64_t q_block, int64_t k_block,
                        int causal, const int64_t *rows, int64_t n_rows, int nthreads)
{
    if (!Q || !K || !V || !O || !Q_scale || !K_scale)
        return 1;
    if (B < 1 || H < 1 || S_q < 1 || S_k < 1 || D_qk < 1 || D_v < 1 || q_block < 1 ||
        k_block < 1)
        return 1;
    oracle_job proto = {0};
    proto.Q = Q; proto.K = K; proto.V = V;
    proto.O = O; proto.LSE = LSE; proto.P = P;
    proto.B = B; proto.H = H; proto.H_kv = H; proto.S_q = S_q; proto.S_k = S_k;
    proto.D_qk = D_qk; proto.D_v = D_v;
    proto.scale = log(2.0);   /* 2^x = e^(x ln 2) */
    proto.causal = causal;
    proto.coff = 0; proto.window = 0; proto.kv_begin = 0; proto.kv_end = S_k;
    proto.q_scale = Q_scale; proto.k_scale = K_scale;
    proto.q_block = q_block; proto.k_block = k_block;
    proto.rows = rows; proto.n_rows = n_rows;
    return run_jobs(&proto, nthreads);
}

/* The plain definition over every key (top-left causal when `causal`). */
int attn_ref_f64(const double *Q, const double *K, const double *V,
                 double *O, double *LSE, double *P,
                 int64_t B, int64_t H, int64_t S_q, int64_t S_k,
                 int64_t D_qk, int64_t D_v, double scale, int causal,
                 const int64_t *rows, int64_t n_rows, int nthreads)
{
    return attn_ref_ext_f64(Q, K, V, O, LSE, P, B, H, H, S_q, S_k, D_qk, D_v, scale, causal,
                            0, 0, 0, S_k, rows, n_rows, nthreads);
}
