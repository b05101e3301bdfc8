/*
 * fa_oracle.c -- plain, slow, fp64 CPU oracle for the attention forward pass.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing on the product path may link, load or
 * call this file; only the test suite, the smoke check and the CPU-baseline
 * leg of the benchmark do.  It shares no code, header, table or constant with
 * the HIP library.
 *
 * What it computes is the plain three-step definition of attention, with no
 * tiling, no online rescaling and no reordering beyond what the definition
 * states:
 *
 *   Page "使用 TileLang 在 AMD GPU 上快速开发高性能 Flash Attention"
 *   (Fast Flash Attention on AMD GPUs with TileLang), section
 *   "核心公式与计算流程" (core formulas): scores = Q K^T scaled by 1/sqrt(d),
 *   an optional lower-triangular causal mask, a softmax over keys, and the
 *   weighted sum of V.  The formula images are lost from that page; the same
 *   steps are spelled out in its section "参考实现（PyTorch 版本）"
 *   (reference implementation): check head counts, repeat K/V heads by the
 *   group count, Q K^T, divide by sqrt(dim), lower-triangular mask, softmax,
 *   multiply by V.
 *
 *   Mask rule (same page, section "K/V Tile 遍历与核心计算"): a key j is kept
 *   for query i iff i >= j.  With a query sequence shorter than the key
 *   sequence (queries that follow past_len earlier positions, e.g. a prefill
 *   after a cached prefix), query row i sits at position i + past_len and
 *   keeps key j iff i + past_len >= j: page "TileLang性能分析报告：H100上
 *   FlashAttention吞吐量达1.2PFlops", section "因果掩码优化" (causal mask
 *   optimisation).  A row that keeps no key at all (possible only when
 *   i + past_len < 0, or with no keys) has output 0 -- what the division
 *   guard of the first page's section "最终输出写回与Q tile 迭代" produces from
 *   an all-zero accumulator -- and log-sum-exp ln(0) = -inf.
 *
 *   Grouped-query heads (same page, section "初始化与Kernel 入口" and the K/V
 *   loads of "K/V Tile 遍历与核心计算"): head_kv = heads / groups and query
 *   head h reads K/V head floor(h / groups).
 *
 *   Log-sum-exp: the natural log of the softmax denominator of the scaled,
 *   masked scores of a row, i.e. LSE_i = m_i + ln(sum_j exp(s_ij - m_i)).
 *   The page "TileLang 与机器学习训练：反向传播算子优化案例" (backward-pass
 *   case), section on the main backward kernel, consumes it as "lse".
 *
 * Layouts (all contiguous, row-major; Lq query rows, Lk key rows):
 *   q, o : [B][Lq][H][D]          (BSHD)
 *   k, v : [B][Lk][Hkv][D]
 *   lse  : [B][H][Lq]
 * q/k/v are IEEE binary16 bit patterns, decoded exactly to double.
 * o and lse are written in double.
 *
 * Floating point: every score is a sum over d in ascending order of exact
 * fp16*fp16 products, in double; exp/log are the C library's double routines.
 * Compiled without -ffast-math so the summation order is the one written.
 *
 * Backward pass (fa_oracle_bwd, fa_oracle_bwd_kv): the gradients of the
 * scalar sum_{b,i,h,d} O[b,i,h,d] * dO[b,i,h,d] with respect to Q, K and V,
 * for equal query and key lengths, or (fa_oracle_bwd_kv) for different
 * lengths with the forward's position offset and mask.  Page "TileLang 与机器学习训练：反向传播算子优化
 * 案例", section "算子拆分与流水线设计", splits the computation into a
 * preprocess computing Delta from O and dO and a main kernel producing dQ,
 * dK and dV from Q, K, V, dO, lse and Delta; the section "反向传播算子的性能
 * 挑战" names its parts: the input gradients and the softmax-derivative
 * adjustment.  Written out by the chain rule through the softmax, per row i
 * of head h (K/V head hk, visible keys j):
 *   P_ij  = softmax_j(s_ij)                  (the forward's probabilities)
 *   dP_ij = sum_d dO[i,d] * V[j,d]
 *   Delta_i = sum_j P_ij * dP_ij             (= sum_d O[i,d] * dO[i,d])
 *   dS_ij = P_ij * (dP_ij - Delta_i)         (softmax derivative)
 *   dQ[i,:]  = scale * sum_j dS_ij * K[j,:]
 *   dK[j,:] += scale * dS_ij * Q[i,:]        (summed over i and over the
 *   dV[j,:] += P_ij * dO[i,:]                  query heads of the group)
 * dO is an input in binary16 bits like Q, K, V; the gradients are written
 * in double.
 *
 * FP8 inputs (fa_oracle_fwd_fp8, fa_oracle_rows_fp8): the same forward on
 * E4M3-coded Q, K, V with one descale factor per tensor, plus an optional
 * per-element error bound for implementations that round the probabilities
 * before the weighted sum; the section at the end of this file says which
 * passage it follows.
 */
#include <math.h>
#include <pthread.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#include <unistd.h>

/* Exact decode of an IEEE 754 binary16 bit pattern to double.
 * binary16: 1 sign bit, 5 exponent bits (bias 15), 10 fraction bits.
 * exponent 0  -> subnormal: (-1)^s * 2^-14 * (frac / 1024)
 * exponent 31 -> inf (frac == 0) or NaN
 * otherwise   -> (-1)^s * 2^(e-15) * (1 + frac / 1024)                    */
double fa_oracle_half_to_double(uint16_t h)
{
    int sign = (h >> 15) & 1;
    int e = (h >> 10) & 0x1f;
    int frac = h & 0x3ff;
    double mag;
    if (e == 0) {
        mag = ldexp((double)frac, -24); /* 2^-14 * frac / 2^10 */
    } else if (e == 31) {
        mag = frac == 0 ? INFINITY : NAN;
    } else {
        mag = ldexp(1.0 + (double)frac / 1024.0, e - 15);
    }
    return sign ? -mag : mag;
}

/* Decoded value of every binary16 bit pattern, filled once from the decoder
 * above, so the inner loops do a lookup instead of re-decoding. */
static double g_half[65536];
static pthread_once_t g_half_once = PTHREAD_ONCE_INIT;

static void fill_half_table(void)
{
    for (uint32_t b = 0; b < 65536u; ++b) g_half[b] = fa_oracle_half_to_double((uint16_t)b);
}

static double h2d(uint16_t h) { return g_half[h]; }

typedef struct {
    const uint16_t *q, *k, *v;
    int B, Lq, Lk, H, Hkv, D, causal, past_len;
    double scale;
} problem_t;

static size_t q_index(const problem_t *p, int b, int i, int h, int d)
{
    return (((size_t)b * p->Lq + i) * p->H + h) * p->D + d;
}

static size_t kv_index(const problem_t *p, int b, int j, int hk, int d)
{
    return (((size_t)b * p->Lk + j) * p->Hkv + hk) * p->D + d;
}

/* Number of keys query i may attend to; the kept keys are always 0..n-1.
 * Without the mask: all Lk keys.  Under the causal mask: keys j with
 * i + past_len >= j, clipped to [0, Lk]. */
static int visible_keys(const problem_t *p, int i)
{
    if (!p->causal) return p->Lk;
    long n = (long)i + p->past_len + 1;
    return n < 0 ? 0 : (n > p->Lk ? p->Lk : (int)n);
}

/* One output row, straight from the definition.
 *   s_j  = scale * sum_d Q[b,i,h,d] * K[b,j,hk,d]        for visible j
 *   m    = max_j s_j
 *   w_j  = exp(s_j - m),   Z = sum_j w_j
 *   O_d  = sum_j (w_j / Z) * V[b,j,hk,d]
 *   LSE  = m + ln Z
 * `s` is caller-provided scratch of at least Lk doubles; on return it holds
 * the probabilities w_j / Z of the visible keys (used by the P export).
 * A row with no visible key: O = 0, LSE = -inf. */
static void attention_row(const problem_t *p, int b, int h, int i,
                          double *s, double *o_row, double *lse_out)
{
    int groups = p->H / p->Hkv;
    int hk = h / groups;
    int n = visible_keys(p, i);
    if (n == 0) {
        for (int d = 0; d < p->D; ++d) o_row[d] = 0.0;
        *lse_out = -INFINITY;
        return;
    }

    /* step 1: scaled scores */
    for (int j = 0; j < n; ++j) {
        double dot = 0.0;
        for (int d = 0; d < p->D; ++d)
            dot += h2d(p->q[q_index(p, b, i, h, d)]) * h2d(p->k[kv_index(p, b, j, hk, d)]);
        s[j] = p->scale * dot;
    }

    /* step 2: softmax over the visible keys */
    double m = -INFINITY;
    for (int j = 0; j < n; ++j)
        if (s[j] > m) m = s[j];
    double z = 0.0;
    for (int j = 0; j < n; ++j) {
        s[j] = exp(s[j] - m);
        z += s[j];
    }
    for (int j = 0; j < n; ++j)
        s[j] = s[j] / z;

    /* step 3: weighted sum of V */
    for (int d = 0; d < p->D; ++d) {
        double acc = 0.0;
        for (int j = 0; j < n; ++j)
            acc += s[j] * h2d(p->v[kv_index(p, b, j, hk, d)]);
        o_row[d] = acc;
    }
    *lse_out = m + log(z);
}

/* ---------------------------------------------------------------- threads */

typedef struct {
    const problem_t *p;
    /* full mode */
    double *o, *lse;
    /* rows mode */
    const int64_t *rows; /* triples (b, h, i) */
    double *o_rows, *lse_rows;
    long n_items;
    long next;
    pthread_mutex_t lock;
} job_t;

enum { ROW_CHUNK = 64 };

static long take_item(job_t *job)
{
    pthread_mutex_lock(&job->lock);
    long it = job->next < job->n_items ? job->next++ : -1;
    pthread_mutex_unlock(&job->lock);
    return it;
}

static void *full_worker(void *arg)
{
    job_t *job = (job_t *)arg;
    const problem_t *p = job->p;
    double *s = (double *)malloc(sizeof(double) * (size_t)(p->Lk > 0 ? p->Lk : 1));
    long chunks = (p->Lq + ROW_CHUNK - 1) / ROW_CHUNK;
    long it;
    while ((it = take_item(job)) >= 0) {
        long bh = it / chunks, c = it % chunks;
        int b = (int)(bh / p->H), h = (int)(bh % p->H);
        int i_end = (int)((c + 1) * ROW_CHUNK < p->Lq ? (c + 1) * ROW_CHUNK : p->Lq);
        for (int i = (int)(c * ROW_CHUNK); i < i_end; ++i)
            attention_row(p, b, h, i, s, job->o + q_index(p, b, i, h, 0),
                          job->lse + ((size_t)b * p->H + h) * p->Lq + i);
    }
    free(s);
    return NULL;
}

static void *rows_worker(void *arg)
{
    job_t *job = (job_t *)arg;
    const problem_t *p = job->p;
    double *s = (double *)malloc(sizeof(double) * (size_t)(p->Lk > 0 ? p->Lk : 1));
    long it;
    while ((it = take_item(job)) >= 0) {
        const int64_t *r = job->rows + 3 * it;
        attention_row(p, (int)r[0], (int)r[1], (int)r[2], s,
                      job->o_rows + (size_t)it * p->D, job->lse_rows + it);
    }
    free(s);
    return NULL;
}

static int resolve_threads(int nthreads)
{
    if (nthreads > 0) return nthreads;
    long n = sysconf(_SC_NPROCESSORS_ONLN);
    return n > 0 ? (int)n : 1;
}

static void run_pool(job_t *job, void *(*fn)(void *), int nthreads)
{
    int n = resolve_threads(nthreads);
    if (n > job->n_items) n = (int)(job->n_items > 0 ? job->n_items : 1);
    pthread_t *tid = (pthread_t *)malloc(sizeof(pthread_t) * (size_t)n);
    pthread_mutex_init(&job->lock, NULL);
    job->next = 0;
    for (int t = 0; t < n; ++t) pthread_create(&tid[t], NULL, fn, job);
    for (int t = 0; t < n; ++t) pthread_join(tid[t], NULL);
    pthread_mutex_destroy(&job->lock);
    free(tid);
}

/* Returns 0 on success, -1 on invalid arguments (the oracle checks only what
 * it needs to stay in bounds: H divisible by Hkv, non-negative sizes). */
static int check_problem(int B, int Lq, int Lk, int H, int Hkv, int D)
{
    pthread_once(&g_half_once, fill_half_table);
    if (B < 0 || Lq < 0 || Lk < 0 || H <= 0 || Hkv <= 0 || D <= 0) return -1;
    if (H % Hkv != 0) return -1;
    return 0;
}

/* Whole forward with Lq query rows and Lk key rows; query row i sits at
 * position i + past_len under the causal mask (past_len is ignored without
 * it).  o [B][Lq][H][D], lse [B][H][Lq] (lse may be NULL).  Work is split
 * over (b, h, 64-row chunk) among `nthreads` POSIX threads (0 = all online
 * cores); each row is computed independently, so the thread count never
 * changes a result. */
int fa_oracle_fwd_kv(const uint16_t *q, const uint16_t *k, const uint16_t *v,
                     double *o, double *lse, int B, int Lq, int Lk, int H, int Hkv, int D,
                     int causal, int past_len, double scale, int nthreads)
{
    if (check_problem(B, Lq, Lk, H, Hkv, D)) return -1;
    problem_t p = {q, k, v, B, Lq, Lk, H, Hkv, D, causal ? 1 : 0, past_len, scale};
    double *lse_buf = lse;
    if (!lse_buf) lse_buf = (double *)malloc(sizeof(double) * ((size_t)B * H * Lq + 1));
    job_t job;
    memset(&job, 0, sizeof(job));
    job.p = &p;
    job.o = o;
    job.lse = lse_buf;
    job.n_items = (long)B * H * ((Lq + ROW_CHUNK - 1) / ROW_CHUNK);
    if (job.n_items > 0) run_pool(&job, full_worker, nthreads);
    if (!lse) free(lse_buf);
    return 0;
}

/* Whole forward with one sequence length L for queries and keys (the
 * i >= j mask): o [B][L][H][D], lse [B][H][L] (lse may be NULL). */
int fa_oracle_fwd(const uint16_t *q, const uint16_t *k, const uint16_t *v,
                  double *o, double *lse, int B, int L, int H, int Hkv, int D,
                  int causal, double scale, int nthreads)
{
    return fa_oracle_fwd_kv(q, k, v, o, lse, B, L, L, H, Hkv, D, causal, 0, scale, nthreads);
}

/* Selected rows only: rows holds n_rows triples (b, h, i); o_rows is
 * [n_rows][D], lse_rows is [n_rows].  Same arithmetic as the whole forward,
 * so a sampled row equals the corresponding full-forward row bit for bit. */
int fa_oracle_rows_kv(const uint16_t *q, const uint16_t *k, const uint16_t *v,
                      int B, int Lq, int Lk, int H, int Hkv, int D, int causal, int past_len,
                      double scale, const int64_t *rows, long n_rows, double *o_rows,
                      double *lse_rows, int nthreads)
{
    if (check_problem(B, Lq, Lk, H, Hkv, D)) return -1;
    for (long r = 0; r < n_rows; ++r) {
        const int64_t *t = rows + 3 * r;
        if (t[0] < 0 || t[0] >= B || t[1] < 0 || t[1] >= H || t[2] < 0 || t[2] >= Lq)
            return -1;
    }
    problem_t p = {q, k, v, B, Lq, Lk, H, Hkv, D, causal ? 1 : 0, past_len, scale};
    job_t job;
    memset(&job, 0, sizeof(job));
    job.p = &p;
    job.rows = rows;
    job.o_rows = o_rows;
    job.lse_rows = lse_rows;
    job.n_items = n_rows;
    if (n_rows > 0) run_pool(&job, rows_worker, nthreads);
    return 0;
}

int fa_oracle_rows(const uint16_t *q, const uint16_t *k, const uint16_t *v,
                   int B, int L, int H, int Hkv, int D, int causal, double scale,
                   const int64_t *rows, long n_rows, double *o_rows,
                   double *lse_rows, int nthreads)
{
    return fa_oracle_rows_kv(q, k, v, B, L, L, H, Hkv, D, causal, 0, scale, rows, n_rows, o_rows,
                             lse_rows, nthreads);
}

/* Softmax probabilities of one row: probs[j] for j < Lk, zero for masked keys
 * (all zero for a row with no visible key).  Exposed so tests can check that
 * each row of the softmax sums to one. */
int fa_oracle_row_probs_kv(const uint16_t *q, const uint16_t *k, const uint16_t *v,
                           int B, int Lq, int Lk, int H, int Hkv, int D, int causal, int past_len,
                           double scale, int b, int h, int i, double *probs)
{
    if (check_problem(B, Lq, Lk, H, Hkv, D)) return -1;
    if (b < 0 || b >= B || h < 0 || h >= H || i < 0 || i >= Lq) return -1;
    problem_t p = {q, k, v, B, Lq, Lk, H, Hkv, D, causal ? 1 : 0, past_len, scale};
    double *s = (double *)malloc(sizeof(double) * (size_t)(Lk > 0 ? Lk : 1));
    double *o_row = (double *)malloc(sizeof(double) * (size_t)D);
    double lse;
    attention_row(&p, b, h, i, s, o_row, &lse);
    int n = visible_keys(&p, i);
    for (int j = 0; j < Lk; ++j) probs[j] = j < n ? s[j] : 0.0;
    free(s);
    free(o_row);
    return 0;
}

int fa_oracle_row_probs(const uint16_t *q, const uint16_t *k, const uint16_t *v,
                        int B, int L, int H, int Hkv, int D, int causal,
                        double scale, int b, int h, int i, double *probs)
{
    return fa_oracle_row_probs_kv(q, k, v, B, L, L, H, Hkv, D, causal, 0, scale, b, h, i, probs);
}

/* ---------------------------------------------------------------- backward */

typedef struct {
    const problem_t *p;
    const uint16_t *dout;
    double *dq, *dk, *dv;
    long n_items; /* B * Hkv */
    long next;
    pthread_mutex_t lock;
} bwd_job_t;

static long bwd_take(bwd_job_t *job)
{
    pthread_mutex_lock(&job->lock);
    long it = job->next < job->n_items ? job->next++ : -1;
    pthread_mutex_unlock(&job->lock);
    return it;
}

/* All gradients that involve K/V head hk of batch b: dQ of the query heads
 * of its group, and dK, dV of hk (accumulated over those heads' rows in
 * ascending head, then row, order -- one thread owns them, so the result
 * does not depend on the thread count). */
static void bwd_group(const problem_t *p, const uint16_t *dout, int b, int hk, double *dq,
                      double *dk, double *dv, double *prob, double *dprob, double *o_row)
{
    const int groups = p->H / p->Hkv;
    for (int j = 0; j < p->Lk; ++j)
        for (int d = 0; d < p->D; ++d) {
            dk[kv_index(p, b, j, hk, d)] = 0.0;
            dv[kv_index(p, b, j, hk, d)] = 0.0;
        }
    for (int h = hk * groups; h < (hk + 1) * groups; ++h) {
        for (int i = 0; i < p->Lq; ++i) {
            double lse;
            /* the forward's probabilities of row i (prob[j], j < n) */
            attention_row(p, b, h, i, prob, o_row, &lse);
            const int n = visible_keys(p, i);
            /* dP_ij and Delta_i */
            double delta = 0.0;
            for (int j = 0; j < n; ++j) {
                double acc = 0.0;
                for (int d = 0; d < p->D; ++d)
                    acc += h2d(dout[q_index(p, b, i, h, d)]) * h2d(p->v[kv_index(p, b, j, hk, d)]);
                dprob[j] = acc;
                delta += prob[j] * acc;
            }
            /* dS_ij = P_ij (dP_ij - Delta_i), kept in dprob */
            for (int j = 0; j < n; ++j) dprob[j] = prob[j] * (dprob[j] - delta);
            for (int d = 0; d < p->D; ++d) {
                double acc = 0.0;
                for (int j = 0; j < n; ++j) acc += dprob[j] * h2d(p->k[kv_index(p, b, j, hk, d)]);
                dq[q_index(p, b, i, h, d)] = p->scale * acc;
            }
            for (int j = 0; j < n; ++j)
                for (int d = 0; d < p->D; ++d) {
                    dk[kv_index(p, b, j, hk, d)] += p->scale * dprob[j] * h2d(p->q[q_index(p, b, i, h, d)]);
                    dv[kv_index(p, b, j, hk, d)] += prob[j] * h2d(dout[q_index(p, b, i, h, d)]);
                }
        }
    }
}

static void *bwd_worker(void *arg)
{
    bwd_job_t *job = (bwd_job_t *)arg;
    const problem_t *p = job->p;
    size_t n = (size_t)(p->Lk > 0 ? p->Lk : 1);
    double *prob = (double *)malloc(sizeof(double) * n);
    double *dprob = (double *)malloc(sizeof(double) * n);
    double *o_row = (double *)malloc(sizeof(double) * (size_t)p->D);
    long it;
    while ((it = bwd_take(job)) >= 0)
        bwd_group(p, job->dout, (int)(it / p->Hkv), (int)(it % p->Hkv), job->dq, job->dk, job->dv,
                  prob, dprob, o_row);
    free(prob);
    free(dprob);
    free(o_row);
    return NULL;
}

/* Gradients of sum(O * dO) for queries and keys of different lengths:
 * query row i sits at position i + past_len and, under the causal mask,
 * keeps key j iff i + past_len >= j (past_len is ignored without the mask),
 * as in fa_oracle_fwd_kv; a row that keeps no key has output 0 and
 * contributes nothing.  dq [B][Lq][H][D], dk and dv [B][Lk][Hkv][D], all
 * double.  q, k, v, dout are binary16 bits in the forward's layouts (dout
 * like q).  Work is split over (b, K/V head) among `nthreads` threads (0 =
 * all online cores); returns 0, or -1 on invalid sizes. */
int fa_oracle_bwd_kv(const uint16_t *q, const uint16_t *k, const uint16_t *v, const uint16_t *dout,
                     double *dq, double *dk, double *dv, int B, int Lq, int Lk, int H, int Hkv, int D,
                     int causal, int past_len, double scale, int nthreads)
{
    if (check_problem(B, Lq, Lk, H, Hkv, D)) return -1;
    problem_t p = {q, k, v, B, Lq, Lk, H, Hkv, D, causal ? 1 : 0, causal ? past_len : 0, scale};
    bwd_job_t job;
    memset(&job, 0, sizeof(job));
    job.p = &p;
    job.dout = dout;
    job.dq = dq;
    job.dk = dk;
    job.dv = dv;
    job.n_items = (long)B * Hkv;
    if (job.n_items <= 0) return 0;
    int nt = resolve_threads(nthreads);
    if (nt > job.n_items) nt = (int)job.n_items;
    pthread_t *tid = (pthread_t *)malloc(sizeof(pthread_t) * (size_t)nt);
    pthread_mutex_init(&job.lock, NULL);
    for (int t = 0; t < nt; ++t) pthread_create(&tid[t], NULL, bwd_worker, &job);
    for (int t = 0; t < nt; ++t) pthread_join(tid[t], NULL);
    pthread_mutex_destroy(&job.lock);
    free(tid);
    return 0;
}

/* The same with sequence length L for queries and keys (mask i >= j when
 * causal): dq [B][L][H][D], dk and dv [B][L][Hkv][D]. */
int fa_oracle_bwd(const uint16_t *q, const uint16_t *k, const uint16_t *v, const uint16_t *dout,
                  double *dq, double *dk, double *dv, int B, int L, int H, int Hkv, int D,
                  int causal, double scale, int nthreads)
{
    return fa_oracle_bwd_kv(q, k, v, dout, dq, dk, dv, B, L, L, H, Hkv, D, causal, 0, scale, nthreads);
}

/* ---------------------------------------------------------------- fp8 */

/* Forward with 8-bit floating-point inputs.  Page "TileLang性能分析报告：H100上
 * FlashAttention吞吐量达1.2PFlops", section "生产环境部署建议", item 1, names
 * FP8 mixed precision for this kernel and gives no further detail.  Read
 * here as: Q, K, V are stored as OCP FP8 E4M3 codes, each tensor with one
 * descale factor, so the value of a stored code c of Q is q_descale * e4m3(c)
 * (likewise K, V); attention is then the plain definition above on those
 * values.  O and the log-sum-exp are written in double.
 *
 * E4M3 (the OCP 8-bit format "E4M3", also called e4m3fn): 1 sign bit,
 * 4 exponent bits with bias 7, 3 fraction bits; no infinities.
 *   exponent 0                 -> (-1)^s * 2^-6 * (frac / 8)   (subnormal)
 *   exponent 15, fraction 7    -> NaN
 *   otherwise                  -> (-1)^s * 2^(e-7) * (1 + frac / 8)
 * The largest finite magnitude is 448.                                    */
double fa_oracle_e4m3_to_double(uint8_t c)
{
    int sign = (c >> 7) & 1;
    int e = (c >> 3) & 0xf;
    int frac = c & 7;
    double mag;
    if (e == 0)
        mag = ldexp((double)frac, -9); /* 2^-6 * frac / 2^3 */
    else if (e == 15 && frac == 7)
        mag = NAN;
    else
        mag = ldexp(1.0 + (double)frac / 8.0, e - 7);
    return sign ? -mag : mag;
}

typedef struct {
    const uint8_t *q, *k, *v;
    int B, Lq, Lk, H, Hkv, D, causal, past_len;
    double scale, qd, kd, vd; /* score scale; the three descales */
    /* rounding model of the probabilities for the error bound (see
     * fp8_row): relative error above `floor`, absolute error below it */
    double b_rel, b_floor, b_abs;
} problem8_t;

static double g_e4m3[256];
static pthread_once_t g_e4m3_once = PTHREAD_ONCE_INIT;

static void fill_e4m3_table(void)
{
    for (int c = 0; c < 256; ++c) g_e4m3[c] = fa_oracle_e4m3_to_double((uint8_t)c);
}

static size_t q8_index(const problem8_t *p, int b, int i, int h, int d)
{
    return (((size_t)b * p->Lq + i) * p->H + h) * p->D + d;
}

static size_t kv8_index(const problem8_t *p, int b, int j, int hk, int d)
{
    return (((size_t)b * p->Lk + j) * p->Hkv + hk) * p->D + d;
}

static int visible_keys8(const problem8_t *p, int i)
{
    if (!p->causal) return p->Lk;
    long n = (long)i + p->past_len + 1;
    return n < 0 ? 0 : (n > p->Lk ? p->Lk : (int)n);
}

/* One output row on the decoded values (the same three steps as
 * attention_row):
 *   s_j = scale * sum_d (qd * Q[i,d]) * (kd * K[j,d])
 *   w_j = exp(s_j - max s),  Z = sum_j w_j
 *   O_d = sum_j (w_j / Z) * (vd * V[j,d]),   LSE = max s + ln Z
 * and, when bound_row is given, for every d
 *   bound_d = sum_j e_j * |vd * V[j,d]| / Z,
 *   e_j = b_rel * w_j            if w_j >= b_floor
 *         min(w_j, b_abs)        otherwise,
 * the largest change of O_d when every weight w_j (the maximum's weight is 1)
 * is replaced by a rounded value within e_j of it while the denominator Z
 * stays exact.  It is the error model of an implementation that rounds the
 * probabilities to a format with relative precision b_rel down to b_floor
 * and a fixed spacing below it.  A row with no visible key: O = 0,
 * LSE = -inf, bound 0. */
static void fp8_row(const problem8_t *p, int b, int h, int i, double *s, double *o_row,
                    double *lse_out, double *bound_row)
{
    int groups = p->H / p->Hkv;
    int hk = h / groups;
    int n = visible_keys8(p, i);
    if (n == 0) {
        for (int d = 0; d < p->D; ++d) {
            o_row[d] = 0.0;
            if (bound_row) bound_row[d] = 0.0;
        }
        *lse_out = -INFINITY;
        return;
    }
    for (int j = 0; j < n; ++j) {
        double dot = 0.0;
        for (int d = 0; d < p->D; ++d)
            dot += (p->qd * g_e4m3[p->q[q8_index(p, b, i, h, d)]]) *
                   (p->kd * g_e4m3[p->k[kv8_index(p, b, j, hk, d)]]);
        s[j] = p->scale * dot;
    }
    double m = -INFINITY;
    for (int j = 0; j < n; ++j)
        if (s[j] > m) m = s[j];
    double z = 0.0;
    for (int j = 0; j < n; ++j) {
        s[j] = exp(s[j] - m);
        z += s[j];
    }
    for (int d = 0; d < p->D; ++d) {
        double acc = 0.0, err = 0.0;
        for (int j = 0; j < n; ++j) {
            double val = p->vd * g_e4m3[p->v[kv8_index(p, b, j, hk, d)]];
            acc += s[j] * val;
            if (bound_row) {
                double e = s[j] >= p->b_floor ? p->b_rel * s[j] : (s[j] < p->b_abs ? s[j] : p->b_abs);
                err += e * fabs(val);
            }
        }
        o_row[d] = acc / z;
        if (bound_row) bound_row[d] = err / z;
    }
    *lse_out = m + log(z);
}

typedef struct {
    const problem8_t *p;
    double *o, *lse, *bound;                 /* full mode */
    const int64_t *rows;                     /* rows mode: triples (b, h, i) */
    double *o_rows, *lse_rows, *bound_rows;
    long n_items, next;
    int rows_mode;
    pthread_mutex_t lock;
} job8_t;

static void *fp8_worker(void *arg)
{
    job8_t *job = (job8_t *)arg;
    const problem8_t *p = job->p;
    double *s = (double *)malloc(sizeof(double) * (size_t)(p->Lk > 0 ? p->Lk : 1));
    long chunks = (p->Lq + ROW_CHUNK - 1) / ROW_CHUNK;
    for (;;) {
        pthread_mutex_lock(&job->lock);
        long it = job->next < job->n_items ? job->next++ : -1;
        pthread_mutex_unlock(&job->lock);
        if (it < 0) break;
        if (job->rows_mode) {
            const int64_t *r = job->rows + 3 * it;
            fp8_row(p, (int)r[0], (int)r[1], (int)r[2], s, job->o_rows + (size_t)it * p->D,
                    job->lse_rows + it, job->bound_rows ? job->bound_rows + (size_t)it * p->D : NULL);
        } else {
            long bh = it / chunks, c = it % chunks;
            int b = (int)(bh / p->H), h = (int)(bh % p->H);
            int i_end = (int)((c + 1) * ROW_CHUNK < p->Lq ? (c + 1) * ROW_CHUNK : p->Lq);
            for (int i = (int)(c * ROW_CHUNK); i < i_end; ++i)
                fp8_row(p, b, h, i, s, job->o + q8_index(p, b, i, h, 0),
                        job->lse + ((size_t)b * p->H + h) * p->Lq + i,
                        job->bound ? job->bound + q8_index(p, b, i, h, 0) : NULL);
        }
    }
    free(s);
    return NULL;
}

static void run_pool8(job8_t *job, int nthreads)
{
    int n = resolve_threads(nthreads);
    if (n > job->n_items) n = (int)(job->n_items > 0 ? job->n_items : 1);
    pthread_t *tid = (pthread_t *)malloc(sizeof(pthread_t) * (size_t)n);
    pthread_mutex_init(&job->lock, NULL);
    job->next = 0;
    for (int t = 0; t < n; ++t) pthread_create(&tid[t], NULL, fp8_worker, job);
    for (int t = 0; t < n; ++t) pthread_join(tid[t], NULL);
    pthread_mutex_destroy(&job->lock);
    free(tid);
}

static int check_problem8(int B, int Lq, int Lk, int H, int Hkv, int D)
{
    pthread_once(&g_e4m3_once, fill_e4m3_table);
    if (B < 0 || Lq < 0 || Lk < 0 || H <= 0 || Hkv <= 0 || D <= 0) return -1;
    if (H % Hkv != 0) return -1;
    return 0;
}

/* Whole fp8 forward: q [B][Lq][H][D], k, v [B][Lk][Hkv][D] E4M3 codes;
 * o [B][Lq][H][D] and bound (same shape, may be NULL) and lse [B][H][Lq]
 * (may be NULL) in double.  Mask and past_len as fa_oracle_fwd_kv. */
int fa_oracle_fwd_fp8(const uint8_t *q, const uint8_t *k, const uint8_t *v, double *o,
                      double *lse, double *bound, int B, int Lq, int Lk, int H, int Hkv, int D,
                      int causal, int past_len, double scale, double q_descale, double k_descale,
                      double v_descale, double b_rel, double b_floor, double b_abs, int nthreads)
{
    if (check_problem8(B, Lq, Lk, H, Hkv, D)) return -1;
    problem8_t p = {q, k, v, B, Lq, Lk, H, Hkv, D, causal ? 1 : 0, past_len, scale,
                    q_descale, k_descale, v_descale, b_rel, b_floor, b_abs};
    double *lse_buf = lse;
    if (!lse_buf) lse_buf = (double *)malloc(sizeof(double) * ((size_t)B * H * Lq + 1));
    job8_t job;
    memset(&job, 0, sizeof(job));
    job.p = &p;
    job.o = o;
    job.lse = lse_buf;
    job.bound = bound;
    job.n_items = (long)B * H * ((Lq + ROW_CHUNK - 1) / ROW_CHUNK);
    if (job.n_items > 0) run_pool8(&job, nthreads);
    if (!lse) free(lse_buf);
    return 0;
}

/* Selected rows of the fp8 forward: rows holds n_rows triples (b, h, i);
 * o_rows and bound_rows (may be NULL) are [n_rows][D], lse_rows [n_rows]. */
int fa_oracle_rows_fp8(const uint8_t *q, const uint8_t *k, const uint8_t *v, int B, int Lq,
                       int Lk, int H, int Hkv, int D, int causal, int past_len, double scale,
                       double q_descale, double k_descale, double v_descale, double b_rel,
                       double b_floor, double b_abs, const int64_t *rows, long n_rows,
                       double *o_rows, double *lse_rows, double *bound_rows, int nthreads)
{
    if (check_problem8(B, Lq, Lk, H, Hkv, D)) return -1;
    for (long r = 0; r < n_rows; ++r) {
        const int64_t *t = rows + 3 * r;
        if (t[0] < 0 || t[0] >= B || t[1] < 0 || t[1] >= H || t[2] < 0 || t[2] >= Lq)
            return -1;
    }
    problem8_t p = {q, k, v, B, Lq, Lk, H, Hkv, D, causal ? 1 : 0, past_len, scale,
                    q_descale, k_descale, v_descale, b_rel, b_floor, b_abs};
    job8_t job;
    memset(&job, 0, sizeof(job));
    job.p = &p;
    job.rows_mode = 1;
    job.rows = rows;
    job.o_rows = o_rows;
    job.lse_rows = lse_rows;
    job.bound_rows = bound_rows;
    job.n_items = n_rows;
    if (n_rows > 0) run_pool8(&job, nthreads);
    return 0;
}
