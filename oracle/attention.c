/*
 * oracle/attention.c -- fp64 CPU reference for the FlashAttention-2 forward.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the product path may call, link or load
 * this file: only the tests, the smoke check and the benchmark's CPU-baseline leg
 * use it.  It shares no code, header or table with the HIP kernels.
 *
 * What it computes is the plain definition of attention, not the tiled method:
 * FlashAttention is exact (it reaches the three-step result, up to summation
 * order), so the reference is that result written out in double precision.
 *
 *   Sources (the four web pages this project is built from):
 *   - Ringi, "Lecture 25: why attention need not store the intermediate matrix"
 *     section 1.1 (S = QK^T, P = softmax(S), O = PV) and section 2.1 (safe softmax:
 *     m = max x, l = sum e^{x-m}, p = e^{x-m}/l).
 *   - AIInfraGuide 6.2 "FlashAttention V2 explained", section 5.1 (the causal mask
 *     adds -inf before the softmax) and the forward pseudocode of section 6
 *     (the saved statistic is L = m + log l).
 *   - LLM Infra Atlas "FA2: parallelism and work partitioning", section 4 (the
 *     causal key bound is offset by seqlen_k - seqlen_q, i.e. bottom-right
 *     alignment when Nq != Nk).
 *   - KingOfEgg, "Flash Attention (4): v2.1 forward vs official source", section 3.5
 *     (lse = row_max * scale + log(sum); an empty row normalises to O = 0).
 *
 * For one (b, h, query i) and a key range [kb, ke):
 *   visible  V_i = { j : kb <= j < ke, j < Nk, and (not causal or j <= i + Nk - Nq) }
 *   s_ij     = sigma * sum_t q[i,t] k[j,t]         (sigma = the float scale, widened)
 *   m_i      = max_{j in V_i} s_ij
 *   l_i      = sum_{j in V_i} exp(s_ij - m_i)
 *   O_i      = sum_{j in V_i} exp(s_ij - m_i) v_j / l_i
 *   LSE_i    = m_i + ln l_i                         (natural log, scaled-score units)
 *   V_i empty: O_i = 0 and LSE_i = -inf.
 *
 * Inputs are raw 16-bit patterns (IEEE binary16 or bfloat16) decoded here exactly.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#include <pthread.h>

#define ORACLE_F16 0
#define ORACLE_BF16 1

/* IEEE 754 binary16: 1 sign bit, 5 exponent bits (bias 15), 10 fraction bits. */
double oracle_decode_f16(uint16_t h) {
    int sign = (h >> 15) & 1;
    int expo = (h >> 10) & 0x1f;
    int frac = h & 0x3ff;
    double mag;
    if (expo == 0) {
        mag = ldexp((double)frac, -24);               /* subnormal: frac * 2^-24 */
    } else if (expo == 31) {
        mag = frac ? NAN : INFINITY;
    } else {
        mag = ldexp((double)(1024 + frac), expo - 25); /* (1 + frac/2^10) * 2^(e-15) */
    }
    return sign ? -mag : mag;
}

/* bfloat16: 1 sign bit, 8 exponent bits (bias 127), 7 fraction bits. */
double oracle_decode_bf16(uint16_t b) {
    int sign = (b >> 15) & 1;
    int expo = (b >> 7) & 0xff;
    int frac = b & 0x7f;
    double mag;
    if (expo == 0) {
        mag = ldexp((double)frac, -133);              /* subnormal: frac * 2^-133 */
    } else if (expo == 255) {
        mag = frac ? NAN : INFINITY;
    } else {
        mag = ldexp((double)(128 + frac), expo - 134); /* (1 + frac/2^7) * 2^(e-127) */
    }
    return sign ? -mag : mag;
}

/* Every 16-bit pattern decoded once by the functions above, so that the inner
 * products below read a table instead of re-decoding: the values are the same
 * doubles either way. */
static double f16_values[65536], bf16_values[65536];
static pthread_once_t values_once = PTHREAD_ONCE_INIT;

static void fill_values(void) {
    for (uint32_t x = 0; x < 65536; ++x) {
        f16_values[x] = oracle_decode_f16((uint16_t)x);
        bf16_values[x] = oracle_decode_bf16((uint16_t)x);
    }
}

/* called by every entry point that decodes, before any worker starts */
static void ensure_values(void) { pthread_once(&values_once, fill_values); }

static double decode(uint16_t x, int dtype) {
    return dtype == ORACLE_BF16 ? bf16_values[x] : f16_values[x];
}

typedef struct {
    const uint16_t *q, *k, *v;
    int dtype, B, H, Nq, Nk, d, causal;
    double sigma;
    int key_begin, key_end;
    const int64_t *rows;      /* flat (b*H + h)*Nq + i indices (varlen: token*H + h), or NULL */
    int64_t nrows;
    double *o, *lse;          /* o: [nrows, d], lse: [nrows] */
    int64_t first, last;      /* this worker's slice of [0, nrows) */
    /* packed variable-length layout (varlen != 0) */
    int varlen, H_kv, total_q, max_k;
    const int32_t *cu_q, *cu_k;
} job_t;

/*
 * One query row against keys lo <= j < hi, written straight from the definition
 * above.  qp is the query row; kp and vp point at key 0 of the row's key/value
 * sequence, whose rows are kstride elements apart.
 */
static void row_core(const uint16_t *qp, const uint16_t *kp, const uint16_t *vp, size_t kstride,
                     int d, int lo, int hi, int dtype, double sigma,
                     double *o_row, double *lse_out, double *qrow, double *s) {
    for (int t = 0; t < d; ++t) o_row[t] = 0.0;
    if (hi <= lo) { *lse_out = -INFINITY; return; }

    for (int t = 0; t < d; ++t) qrow[t] = decode(qp[t], dtype);

    /* scores of the visible keys and their maximum */
    double m = -INFINITY;
    for (int j = lo; j < hi; ++j) {
        double acc = 0.0;
        const uint16_t *kj = kp + (size_t)j * kstride;
        for (int t = 0; t < d; ++t) acc += qrow[t] * decode(kj[t], dtype);
        s[j - lo] = sigma * acc;
        if (s[j - lo] > m) m = s[j - lo];
    }
    /* softmax denominator and weighted sum of V */
    double l = 0.0;
    for (int j = lo; j < hi; ++j) {
        double p = exp(s[j - lo] - m);
        l += p;
        const uint16_t *vj = vp + (size_t)j * kstride;
        for (int t = 0; t < d; ++t) o_row[t] += p * decode(vj[t], dtype);
    }
    for (int t = 0; t < d; ++t) o_row[t] /= l;
    *lse_out = m + log(l);
}

/* Last visible key + 1 for query i of a sequence of Nq queries and Nk keys. */
static int causal_end(int i, int Nq, int Nk, int lo, int hi) {
    int64_t lim = (int64_t)i + (Nk - Nq) + 1;              /* keys j <= i + Nk - Nq */
    if (lim < hi) hi = lim < lo ? lo : (int)lim;
    return hi;
}

/* One row of the [B, H, N, d] layout. */
static void one_row(const job_t *jb, int64_t flat, double *o_row, double *lse_out,
                    double *qrow, double *s) {
    const int d = jb->d, Nq = jb->Nq, Nk = jb->Nk;
    const int64_t bh = flat / Nq;
    const int i = (int)(flat % Nq);
    const uint16_t *qp = jb->q + ((size_t)bh * Nq + i) * d;
    const uint16_t *kp = jb->k + (size_t)bh * Nk * d;
    const uint16_t *vp = jb->v + (size_t)bh * Nk * d;

    int lo = jb->key_begin < 0 ? 0 : jb->key_begin;
    int hi = jb->key_end > Nk ? Nk : jb->key_end;
    if (jb->causal) hi = causal_end(i, Nq, Nk, lo, hi);
    row_core(qp, kp, vp, (size_t)d, d, lo, hi, jb->dtype, jb->sigma, o_row, lse_out, qrow, s);
}

/*
 * One row of the packed variable-length layout with grouped K/V heads
 * (KingOfEgg, "Flash Attention (4)", section 5: K/V indexed by head group and
 * sequences delimited by cumulative offsets cu_seqlens; Ringi, "Lecture 25",
 * section 7: packing without padding).  q: [total_q, H, d]; k, v: [total_k,
 * H_kv, d].  Sequence b owns query tokens [cu_q[b], cu_q[b+1]) and key tokens
 * [cu_k[b], cu_k[b+1]); query head h reads K/V head h / (H / H_kv).  Within a
 * sequence the definition above applies with its own Nq and Nk.
 */
static void varlen_row(const job_t *jb, int64_t flat, double *o_row, double *lse_out,
                       double *qrow, double *s) {
    const int d = jb->d, H = jb->H, H_kv = jb->H_kv;
    const int64_t token = flat / H;
    const int h = (int)(flat % H);
    int b = 0;
    while (b + 1 < jb->B && jb->cu_q[b + 1] <= token) ++b;  /* sequence holding the token */
    const int i = (int)(token - jb->cu_q[b]);
    const int Nq = jb->cu_q[b + 1] - jb->cu_q[b];
    const int Nk = jb->cu_k[b + 1] - jb->cu_k[b];
    const int g = h / (H / H_kv);
    const uint16_t *qp = jb->q + ((size_t)token * H + h) * d;
    const uint16_t *kp = jb->k + ((size_t)jb->cu_k[b] * H_kv + g) * d;
    const uint16_t *vp = jb->v + ((size_t)jb->cu_k[b] * H_kv + g) * d;
    int hi = Nk;
    if (jb->causal) hi = causal_end(i, Nq, Nk, 0, hi);
    row_core(qp, kp, vp, (size_t)H_kv * d, d, 0, hi, jb->dtype, jb->sigma, o_row, lse_out, qrow, s);
}

static void *worker(void *arg) {
    job_t *jb = (job_t *)arg;
    const int max_k = jb->varlen ? jb->max_k : jb->Nk;
    double *qrow = (double *)malloc(sizeof(double) * (size_t)jb->d);
    double *s = (double *)malloc(sizeof(double) * (size_t)(max_k > 0 ? max_k : 1));
    if (!qrow || !s) { free(qrow); free(s); return (void *)1; }
    for (int64_t r = jb->first; r < jb->last; ++r) {
        int64_t flat = jb->rows ? jb->rows[r] : r;
        if (jb->varlen)
            varlen_row(jb, flat, jb->o + r * jb->d, jb->lse + r, qrow, s);
        else
            one_row(jb, flat, jb->o + r * jb->d, jb->lse + r, qrow, s);
    }
    free(qrow);
    free(s);
    return NULL;
}

static int run_jobs(const job_t *base, int nthreads);

/*
 * Attention rows of [B, H, Nq, d] queries against [B, H, Nk, d] keys/values,
 * restricted to keys in [key_begin, key_end).  rows == NULL means every row in
 * flat order (nrows must then be B*H*Nq).  Returns 0, or -1 on a bad argument,
 * -2 on allocation or thread failure.
 */
int oracle_attention_rows(const uint16_t *q, const uint16_t *k, const uint16_t *v, int dtype,
                          int B, int H, int Nq, int Nk, int d, int causal, float scale,
                          int key_begin, int key_end, const int64_t *rows, int64_t nrows,
                          double *o, double *lse, int nthreads) {
    if (!q || !k || !v || !o || !lse) return -1;
    if (B <= 0 || H <= 0 || Nq <= 0 || Nk <= 0 || d <= 0 || nrows < 0) return -1;
    if (dtype != ORACLE_F16 && dtype != ORACLE_BF16) return -1;
    ensure_values();
    const int64_t total = (int64_t)B * H * Nq;
    if (!rows && nrows != total) return -1;
    if (rows)
        for (int64_t r = 0; r < nrows; ++r)
            if (rows[r] < 0 || rows[r] >= total) return -1;
    job_t base = {q, k, v, dtype, B, H, Nq, Nk, d, causal, (double)scale,
                  key_begin, key_end, rows, nrows, o, lse, 0, 0, 0, H, 0, 0, NULL, NULL};
    return run_jobs(&base, nthreads);
}

/*
 * Attention rows of the packed layout (see varlen_row): rows == NULL means every
 * (token, head) in flat order token*H + h (nrows must then be total_q*H); o is
 * [nrows, d], lse [nrows].  cu_q and cu_k are host arrays of B+1 non-decreasing
 * offsets starting at 0.  Returns 0, or -1 on a bad argument, -2 on allocation
 * or thread failure.
 */
int oracle_attention_varlen(const uint16_t *q, const uint16_t *k, const uint16_t *v, int dtype,
                            int B, int H, int H_kv, int d, const int32_t *cu_q, const int32_t *cu_k,
                            int causal, float scale, const int64_t *rows, int64_t nrows,
                            double *o, double *lse, int nthreads) {
    if (!q || !k || !v || !o || !lse || !cu_q || !cu_k) return -1;
    if (B <= 0 || H <= 0 || H_kv <= 0 || H % H_kv != 0 || d <= 0 || nrows < 0) return -1;
    if (dtype != ORACLE_F16 && dtype != ORACLE_BF16) return -1;
    ensure_values();
    if (cu_q[0] != 0 || cu_k[0] != 0) return -1;
    int max_k = 0;
    for (int b = 0; b < B; ++b) {
        if (cu_q[b + 1] < cu_q[b] || cu_k[b + 1] < cu_k[b]) return -1;
        if (cu_k[b + 1] - cu_k[b] > max_k) max_k = cu_k[b + 1] - cu_k[b];
    }
    const int64_t total = (int64_t)cu_q[B] * H;
    if (!rows && nrows != total) return -1;
    if (rows)
        for (int64_t r = 0; r < nrows; ++r)
            if (rows[r] < 0 || rows[r] >= total) return -1;
    job_t base = {q, k, v, dtype, B, H, 0, 0, d, causal, (double)scale,
                  0, 0, rows, nrows, o, lse, 0, 0, 1, H_kv, cu_q[B], max_k, cu_q, cu_k};
    return run_jobs(&base, nthreads);
}

/* Split rows [0, base->nrows) over nthreads workers and run them. */
static int run_jobs(const job_t *basep, int nthreads) {
    const job_t base = *basep;
    const int64_t nrows = base.nrows;
    if (nthreads < 1) nthreads = 1;
    if (nthreads > 256) nthreads = 256;
    if ((int64_t)nthreads > nrows) nthreads = nrows > 0 ? (int)nrows : 1;
    job_t jobs[256];
    pthread_t tid[256];
    int started[256];
    int rc = 0;
    for (int w = 0; w < nthreads; ++w) {
        jobs[w] = base;
        jobs[w].first = nrows * w / nthreads;
        jobs[w].last = nrows * (w + 1) / nthreads;
        started[w] = pthread_create(&tid[w], NULL, worker, &jobs[w]) == 0;
        if (!started[w]) worker(&jobs[w]);   /* run inline if a thread cannot start */
    }
    for (int w = 0; w < nthreads; ++w) {
        void *ret = NULL;
        if (started[w]) pthread_join(tid[w], &ret);
        if (ret) rc = -2;
    }
    return rc;
}

/*
 * Merge of per-split partial results (split-KV decode).  The pages give only
 * "each split emits a partial (O, LSE), a combine kernel merges them" (LLM Infra
 * Atlas, "FA2: parallelism", section 2) together with the merge identity of the
 * online softmax (Ringi, Lecture 25, section 2.2):
 *   l_new = l_prev * e^{m_prev - m_new} + l_cur * e^{m_cur - m_new}.
 * With normalised partials O_s and LSE_s = m_s + ln l_s this reads
 *   M = max_s LSE_s;  w_s = e^{LSE_s - M} (0 when LSE_s = -inf);
 *   O = sum_s w_s O_s / sum_s w_s;  LSE = M + ln sum_s w_s  (-inf if every split is empty).
 * o_part: [S, R, d], lse_part: [S, R]; outputs o: [R, d], lse: [R].
 */
int oracle_combine(const double *o_part, const double *lse_part, int S, int64_t R, int d,
                   double *o, double *lse) {
    if (!o_part || !lse_part || !o || !lse || S <= 0 || R < 0 || d <= 0) return -1;
    for (int64_t r = 0; r < R; ++r) {
        double M = -INFINITY;
        for (int s = 0; s < S; ++s)
            if (lse_part[(size_t)s * R + r] > M) M = lse_part[(size_t)s * R + r];
        double *orow = o + r * d;
        for (int t = 0; t < d; ++t) orow[t] = 0.0;
        if (M == -INFINITY) { lse[r] = -INFINITY; continue; }
        double wsum = 0.0;
        for (int s = 0; s < S; ++s) {
            double ls = lse_part[(size_t)s * R + r];
            if (ls == -INFINITY) continue;
            double w = exp(ls - M);
            wsum += w;
            const double *op = o_part + ((size_t)s * R + r) * d;
            for (int t = 0; t < d; ++t) orow[t] += w * op[t];
        }
        for (int t = 0; t < d; ++t) orow[t] /= wsum;
        lse[r] = M + log(wsum);
    }
    return 0;
}

/*
 * Backward pass (gradients of a loss with upstream gradient dO = dL/dO), from
 * the chain rule as Ringi, "Lecture 25", section 3.3 states it for P =
 * softmax(S):
 *   dV = P^T dO;   dP = dO V^T;   dS = P o (dP - rowsum(dP o P));
 *   dQ = dS K;     dK = dS^T Q
 * with the scores here S = sigma * Q K^T, so the chain rule adds sigma to dQ and
 * dK (dS is the gradient with respect to the scaled scores).  Masked keys have
 * P = 0 and so contribute nothing; a row that sees no key has P = 0 throughout.
 * The statistics of the query rows that the requested gradients read are
 * computed first (m, l and D_i = rowsum(dP o P)): each requested query row, and
 * for a head with requested key rows every query row that sees one of them
 * (causal: rows i >= j_min - (Nk - Nq); otherwise all rows); then
 *   dq_i = sigma * sum_j dS_ij k_j                 for the requested query rows,
 *   dv_j = sum_i P_ij dO_i,  dk_j = sigma * sum_i dS_ij q_i   for the requested key rows.
 * Layouts [B, H, N, d]; q_rows are flat (b*H + h)*Nq + i, k_rows (b*H + h)*Nk + j;
 * NULL means all.  Outputs: dq [n_q, d], dk and dv [n_k, d].
 */
typedef struct {
    const uint16_t *q, *k, *v, *dout;
    int dtype, H, Nq, Nk, d, causal;
    double sigma;
    double *m, *l, *D;          /* per query row of the needed heads */
    int64_t *head_slot;         /* (b*H + h) -> slot in m/l/D, or -1 */
    const int64_t *q_rows, *k_rows;
    int64_t n_q, n_k;
    double *dq, *dk, *dv;
    int64_t first, last;        /* worker's slice: phase 0 rows of needed heads, 1 q rows, 2 k rows */
    int phase;
    const int64_t *stat_rows;   /* phase 0: flat query rows needing statistics */
    int failed;                 /* set by a worker that could not allocate */
} bjob_t;

static int row_visible_end(int i, int Nq, int Nk, int causal) {
    int hi = Nk;
    if (causal) hi = causal_end(i, Nq, Nk, 0, hi);
    return hi;
}

/* dO_i . v_j and sigma * q_i . k_j in double */
static double dot_rows(const uint16_t *a, const uint16_t *b, int d, int dtype) {
    double acc = 0.0;
    for (int t = 0; t < d; ++t) acc += decode(a[t], dtype) * decode(b[t], dtype);
    return acc;
}

/* s: scratch of Nk doubles for the row's scaled scores */
static void bwd_stats(const bjob_t *jb, int64_t flat, double *s) {
    const int d = jb->d, Nq = jb->Nq, Nk = jb->Nk;
    const int64_t bh = flat / Nq;
    const int i = (int)(flat % Nq);
    const int64_t slot = jb->head_slot[bh] * Nq + i;
    const uint16_t *qi = jb->q + ((size_t)bh * Nq + i) * d;
    const uint16_t *gi = jb->dout + ((size_t)bh * Nq + i) * d;
    const uint16_t *kp = jb->k + (size_t)bh * Nk * d;
    const uint16_t *vp = jb->v + (size_t)bh * Nk * d;
    const int hi = row_visible_end(i, Nq, Nk, jb->causal);
    double m = -INFINITY;
    for (int j = 0; j < hi; ++j) {
        s[j] = jb->sigma * dot_rows(qi, kp + (size_t)j * d, d, jb->dtype);
        if (s[j] > m) m = s[j];
    }
    double l = 0.0;
    for (int j = 0; j < hi; ++j) l += exp(s[j] - m);
    double D = 0.0;                                           /* rowsum(dP o P) */
    for (int j = 0; j < hi; ++j) {
        double p = exp(s[j] - m) / l;
        D += p * dot_rows(gi, vp + (size_t)j * d, d, jb->dtype);
    }
    jb->m[slot] = m;
    jb->l[slot] = l;
    jb->D[slot] = hi > 0 ? D : 0.0;
}

static void bwd_q_row(const bjob_t *jb, int64_t flat, double *dq) {
    const int d = jb->d, Nq = jb->Nq, Nk = jb->Nk;
    const int64_t bh = flat / Nq;
    const int i = (int)(flat % Nq);
    const int64_t slot = jb->head_slot[bh] * Nq + i;
    const uint16_t *qi = jb->q + ((size_t)bh * Nq + i) * d;
    const uint16_t *gi = jb->dout + ((size_t)bh * Nq + i) * d;
    const uint16_t *kp = jb->k + (size_t)bh * Nk * d;
    const uint16_t *vp = jb->v + (size_t)bh * Nk * d;
    const int hi = row_visible_end(i, Nq, Nk, jb->causal);
    for (int t = 0; t < d; ++t) dq[t] = 0.0;
    for (int j = 0; j < hi; ++j) {
        const uint16_t *kj = kp + (size_t)j * d;
        double p = exp(jb->sigma * dot_rows(qi, kj, d, jb->dtype) - jb->m[slot]) / jb->l[slot];
        double ds = p * (dot_rows(gi, vp + (size_t)j * d, d, jb->dtype) - jb->D[slot]);
        for (int t = 0; t < d; ++t) dq[t] += jb->sigma * ds * decode(kj[t], jb->dtype);
    }
}

static void bwd_k_row(const bjob_t *jb, int64_t flat, double *dk, double *dv) {
    const int d = jb->d, Nq = jb->Nq, Nk = jb->Nk;
    const int64_t bh = flat / Nk;
    const int j = (int)(flat % Nk);
    const uint16_t *kj = jb->k + ((size_t)bh * Nk + j) * d;
    const uint16_t *vj = jb->v + ((size_t)bh * Nk + j) * d;
    for (int t = 0; t < d; ++t) dk[t] = dv[t] = 0.0;
    for (int i = 0; i < Nq; ++i) {
        if (j >= row_visible_end(i, Nq, Nk, jb->causal)) continue;   /* key j masked for query i */
        const int64_t slot = jb->head_slot[bh] * Nq + i;
        const uint16_t *qi = jb->q + ((size_t)bh * Nq + i) * d;
        const uint16_t *gi = jb->dout + ((size_t)bh * Nq + i) * d;
        double p = exp(jb->sigma * dot_rows(qi, kj, d, jb->dtype) - jb->m[slot]) / jb->l[slot];
        double ds = p * (dot_rows(gi, vj, d, jb->dtype) - jb->D[slot]);
        for (int t = 0; t < d; ++t) {
            dv[t] += p * decode(gi[t], jb->dtype);
            dk[t] += jb->sigma * ds * decode(qi[t], jb->dtype);
        }
    }
}

static void *bwd_worker(void *arg) {
    bjob_t *jb = (bjob_t *)arg;
    double *s = NULL;
    if (jb->phase == 0 && jb->last > jb->first) {
        s = (double *)malloc(sizeof(double) * (size_t)jb->Nk);
        if (!s) { jb->failed = 1; return NULL; }
    }
    for (int64_t r = jb->first; r < jb->last; ++r) {
        if (jb->phase == 0) bwd_stats(jb, jb->stat_rows[r], s);
        else if (jb->phase == 1) bwd_q_row(jb, jb->q_rows ? jb->q_rows[r] : r, jb->dq + r * jb->d);
        else bwd_k_row(jb, jb->k_rows ? jb->k_rows[r] : r, jb->dk + r * jb->d, jb->dv + r * jb->d);
    }
    free(s);
    return NULL;
}

/* Returns 0, or -2 if a worker could not allocate its scratch. */
static int bwd_run(const bjob_t *base, int phase, int64_t n, int nthreads) {
    if (nthreads < 1) nthreads = 1;
    if (nthreads > 256) nthreads = 256;
    if ((int64_t)nthreads > n) nthreads = n > 0 ? (int)n : 1;
    bjob_t jobs[256];
    pthread_t tid[256];
    int started[256];
    for (int w = 0; w < nthreads; ++w) {
        jobs[w] = *base;
        jobs[w].phase = phase;
        jobs[w].first = n * w / nthreads;
        jobs[w].last = n * (w + 1) / nthreads;
        started[w] = pthread_create(&tid[w], NULL, bwd_worker, &jobs[w]) == 0;
        if (!started[w]) bwd_worker(&jobs[w]);
    }
    int rc = 0;
    for (int w = 0; w < nthreads; ++w) {
        if (started[w]) pthread_join(tid[w], NULL);
        if (jobs[w].failed) rc = -2;
    }
    return rc;
}

int oracle_attention_bwd(const uint16_t *q, const uint16_t *k, const uint16_t *v, const uint16_t *dout,
                         int dtype, int B, int H, int Nq, int Nk, int d, int causal, float scale,
                         const int64_t *q_rows, int64_t n_q, const int64_t *k_rows, int64_t n_k,
                         double *dq, double *dk, double *dv, int nthreads) {
    if (!q || !k || !v || !dout || !dq || !dk || !dv) return -1;
    if (B <= 0 || H <= 0 || Nq <= 0 || Nk <= 0 || d <= 0 || n_q < 0 || n_k < 0) return -1;
    if (dtype != ORACLE_F16 && dtype != ORACLE_BF16) return -1;
    ensure_values();
    const int64_t BH = (int64_t)B * H;
    if (!q_rows && n_q != BH * Nq) return -1;
    if (!k_rows && n_k != BH * Nk) return -1;
    for (int64_t r = 0; q_rows && r < n_q; ++r)
        if (q_rows[r] < 0 || q_rows[r] >= BH * Nq) return -1;
    for (int64_t r = 0; k_rows && r < n_k; ++r)
        if (k_rows[r] < 0 || k_rows[r] >= BH * Nk) return -1;
    /* heads whose row statistics are needed */
    int64_t *slot = (int64_t *)malloc(sizeof(int64_t) * (size_t)BH);
    if (!slot) return -2;
    for (int64_t h = 0; h < BH; ++h) slot[h] = -1;
    int64_t nheads = 0;
    for (int64_t r = 0; r < n_q; ++r) {
        int64_t h = (q_rows ? q_rows[r] : r) / Nq;
        if (slot[h] < 0) slot[h] = nheads++;
    }
    for (int64_t r = 0; r < n_k; ++r) {
        int64_t h = (k_rows ? k_rows[r] : r) / Nk;
        if (slot[h] < 0) slot[h] = nheads++;
    }
    const int64_t nslots = nheads * Nq;
    double *m = (double *)malloc(sizeof(double) * (size_t)(nslots > 0 ? nslots : 1));
    double *l = (double *)malloc(sizeof(double) * (size_t)(nslots > 0 ? nslots : 1));
    double *D = (double *)malloc(sizeof(double) * (size_t)(nslots > 0 ? nslots : 1));
    int64_t *srows = (int64_t *)malloc(sizeof(int64_t) * (size_t)(nslots > 0 ? nslots : 1));
    char *need = (char *)calloc((size_t)(nslots > 0 ? nslots : 1), 1);
    if (!m || !l || !D || !srows || !need) {
        free(slot); free(m); free(l); free(D); free(srows); free(need);
        return -2;
    }
    /* rows whose statistics a requested gradient reads: the requested query rows,
     * and every query row that sees a requested key (key j is seen by query i
     * iff j < row_visible_end(i), i.e. causal: i >= j - (Nk - Nq)) */
    for (int64_t r = 0; r < n_q; ++r) {
        const int64_t f = q_rows ? q_rows[r] : r;
        need[slot[f / Nq] * Nq + f % Nq] = 1;
    }
    int *first = (int *)malloc(sizeof(int) * (size_t)(nheads > 0 ? nheads : 1));   /* per slot */
    if (!first) {
        free(slot); free(m); free(l); free(D); free(srows); free(need);
        return -2;
    }
    for (int64_t h = 0; h < nheads; ++h) first[h] = Nq;
    for (int64_t r = 0; r < n_k; ++r) {
        const int64_t f = k_rows ? k_rows[r] : r;
        const int j = (int)(f % Nk);
        int lo = causal ? j - (Nk - Nq) : 0;
        if (lo < 0) lo = 0;
        if (lo < first[slot[f / Nk]]) first[slot[f / Nk]] = lo;
    }
    for (int64_t h = 0; h < nheads; ++h)
        for (int i = first[h]; i < Nq; ++i) need[h * Nq + i] = 1;
    free(first);
    int64_t nstat = 0;
    for (int64_t h = 0; h < BH; ++h)
        if (slot[h] >= 0)
            for (int i = 0; i < Nq; ++i) {
                const int64_t sl = slot[h] * Nq + i;
                m[sl] = l[sl] = D[sl] = NAN;          /* never read unless computed */
                if (need[sl]) srows[nstat++] = h * Nq + i;
            }
    free(need);
    bjob_t base = {q, k, v, dout, dtype, H, Nq, Nk, d, causal, (double)scale, m, l, D, slot,
                   q_rows, k_rows, n_q, n_k, dq, dk, dv, 0, 0, 0, srows, 0};
    int rc = bwd_run(&base, 0, nstat, nthreads);
    if (rc == 0) rc = bwd_run(&base, 1, n_q, nthreads);
    if (rc == 0) rc = bwd_run(&base, 2, n_k, nthreads);
    free(slot); free(m); free(l); free(D); free(srows);
    return rc;
}
