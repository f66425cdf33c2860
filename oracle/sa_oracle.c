/*
 * sa_oracle.c -- the reference oracle for causal streaming attention.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the product path may link, load or
 * call this file: only the tests, the smoke check and the CPU-baseline leg
 * of the benchmark use it.  It shares no code, header or constant with the
 * HIP library.
 *
 * What it computes is the plain definition of the attention the streaming
 * kernels reach up to rounding, written out in binary64 with one
 * materialised score row at a time:
 *
 *   StreamingAttentionSM86 page, banner "Causal attention as a streaming
 *   normalised sum": scores in base-2 units t = S * scale / ln 2, the
 *   probabilities 2^(t - m) / l, the output O = P V and the base-2
 *   log-sum-exp L = m + log2 l.  The oracle takes the exact binary64
 *   value of scale / ln 2; the kernels take the binary32 nearest one.
 *
 *   StreamingAttentionSM86 page, banner "The backward pass, deterministic
 *   and in two launches": dP = dO V^T, D = rowsum(dO * O),
 *   dS = P * (dP - D), dQ = s dS K, dK = s dS^T Q, dV = P^T dO.
 *
 *   Variable-length gist page (self_attn_fwd): a query or key at or past
 *   the sequence's length is masked; a row with no admitted key gets
 *   O = 0.  Its L is -inf (log2 of an empty sum), and its D, dQ and the
 *   gradients it would send to keys are 0.
 *
 * Grouped query attention: query head h reads K/V head h / (heads / kvHeads)
 * (contiguous groups, the page's grid y / grid z head selection).  dK and dV
 * are the gradients with respect to the K and V^T inputs, i.e. summed over
 * the query heads of the group.
 *
 * Layouts (element offsets; the inputs are binary64 arrays, normally the
 * exact values of the fp16 inputs the kernels receive):
 *   Q, dO [B][H][T][64];  K [B][KV][T][64];  Vt [B][KV][64][T];
 *   seqlens int32[B] or NULL (every sequence has length T).
 * Outputs are binary64, one 64-wide row per requested row or column.
 *
 * Every loop runs over the definition's index in its natural order; OpenMP
 * only distributes independent rows or columns.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

#define HD 64 /* head width */

typedef struct {
    int B, T, H, KV, causal;
    const int32_t* seqlens;
    double s;        /* natural score scale */
    double c;        /* s / ln 2, exact in binary64 arithmetic */
    const double *Q, *K, *Vt, *dO;
} problem;

static int seq_len(const problem* p, int b) {
    if (!p->seqlens) return p->T;
    int n = p->seqlens[b];
    return n < 0 ? 0 : (n > p->T ? p->T : n);
}

/* Key j is admitted for query i of sequence b. */
static int admitted(const problem* p, int len, int i, int j) {
    if (i >= len || j >= len) return 0;
    if (p->causal && j > i) return 0;
    return 1;
}

static double q_at(const problem* p, int b, int h, int i, int d) {
    return p->Q[(((int64_t)b * p->H + h) * p->T + i) * HD + d];
}
static double do_at(const problem* p, int b, int h, int i, int d) {
    return p->dO[(((int64_t)b * p->H + h) * p->T + i) * HD + d];
}
static double k_at(const problem* p, int b, int kv, int j, int d) {
    return p->K[(((int64_t)b * p->KV + kv) * p->T + j) * HD + d];
}
/* V[j][d] is stored transposed: Vt[b][kv][d][j]. */
static double v_at(const problem* p, int b, int kv, int j, int d) {
    return p->Vt[(((int64_t)b * p->KV + kv) * HD + d) * p->T + j];
}

/* Base-2 score t_ij = (sum_d Q_id K_jd) * s / ln 2. */
static double score2(const problem* p, int b, int h, int kv, int i, int j) {
    double acc = 0.0;
    for (int d = 0; d < HD; ++d) acc += q_at(p, b, h, i, d) * k_at(p, b, kv, j, d);
    return acc * p->c;
}

/*
 * One query row: fills t[0..T) (only admitted entries are meaningful), and
 * returns through *m, *l, the row maximum and sum of 2^(t - m) over the
 * admitted keys.  Returns the number of admitted keys.
 */
static int row_scores(const problem* p, int b, int h, int i, double* t, double* m, double* l) {
    int kv = h / (p->H / p->KV), len = seq_len(p, b), n = 0;
    double mx = -INFINITY;
    for (int j = 0; j < p->T; ++j) {
        if (!admitted(p, len, i, j)) continue;
        t[j] = score2(p, b, h, kv, i, j);
        if (t[j] > mx) mx = t[j];
        ++n;
    }
    double sum = 0.0;
    for (int j = 0; j < p->T; ++j)
        if (admitted(p, len, i, j)) sum += exp2(t[j] - mx);
    *m = mx;
    *l = sum;
    return n;
}

/* O_i = sum_j P_ij V_j with P_ij = 2^(t_ij - m) / l; L_i = m + log2 l. */
static void row_forward(const problem* p, int b, int h, int i, double* t, double* O, double* L) {
    int kv = h / (p->H / p->KV), len = seq_len(p, b);
    double m, l;
    for (int d = 0; d < HD; ++d) O[d] = 0.0;
    if (row_scores(p, b, h, i, t, &m, &l) == 0) {
        *L = -INFINITY;
        return;
    }
    for (int j = 0; j < p->T; ++j) {
        if (!admitted(p, len, i, j)) continue;
        double P = exp2(t[j] - m) / l;
        for (int d = 0; d < HD; ++d) O[d] += P * v_at(p, b, kv, j, d);
    }
    *L = m + log2(l);
}

static problem make_problem(const double* Q, const double* K, const double* Vt, const double* dO,
                            int B, int T, int H, int KV, int causal, const int32_t* seqlens, double s) {
    problem p;
    p.B = B; p.T = T; p.H = H; p.KV = KV; p.causal = causal; p.seqlens = seqlens;
    p.s = s; p.c = s / log(2.0);
    p.Q = Q; p.K = K; p.Vt = Vt; p.dO = dO;
    return p;
}

static int bad_shape(int B, int T, int H, int KV) {
    return B < 1 || T < 1 || H < 1 || KV < 1 || H % KV != 0;
}

/*
 * Forward for a list of rows, row id = (b * H + h) * T + i.
 * O: [nrows][64], L: [nrows].  Returns 0, or -1 on a bad shape or row id.
 */
int oracle_forward_rows(const double* Q, const double* K, const double* Vt,
                        int B, int T, int H, int KV, int causal, const int32_t* seqlens, double s,
                        const int64_t* rows, int64_t nrows, double* O, double* L) {
    if (bad_shape(B, T, H, KV)) return -1;
    int64_t total = (int64_t)B * H * T;
    for (int64_t r = 0; r < nrows; ++r)
        if (rows[r] < 0 || rows[r] >= total) return -1;
    problem p = make_problem(Q, K, Vt, NULL, B, T, H, KV, causal, seqlens, s);
    #pragma omp parallel
    {
        double* t = (double*)malloc(sizeof(double) * T);
        #pragma omp for schedule(dynamic, 4)
        for (int64_t r = 0; r < nrows; ++r) {
            int64_t id = rows[r];
            int i = (int)(id % T), h = (int)((id / T) % H), b = (int)(id / ((int64_t)T * H));
            row_forward(&p, b, h, i, t, O + r * HD, L + r);
        }
        free(t);
    }
    return 0;
}

/*
 * Row terms and query gradient for a list of rows (ids as above):
 *   D_i  = sum_d dO_id O_id                      (O the oracle's own output)
 *   dP_ij = sum_d dO_id V_jd,   dS_ij = P_ij (dP_ij - D_i)
 *   dQ_i = s sum_j dS_ij K_j
 * D: [nrows], dQ: [nrows][64].  O and L are also returned if non-NULL.
 */
int oracle_backward_rows(const double* Q, const double* K, const double* Vt, const double* dO,
                         int B, int T, int H, int KV, int causal, const int32_t* seqlens, double s,
                         const int64_t* rows, int64_t nrows, double* D, double* dQ,
                         double* O_out, double* L_out) {
    if (bad_shape(B, T, H, KV)) return -1;
    int64_t total = (int64_t)B * H * T;
    for (int64_t r = 0; r < nrows; ++r)
        if (rows[r] < 0 || rows[r] >= total) return -1;
    problem p = make_problem(Q, K, Vt, dO, B, T, H, KV, causal, seqlens, s);
    #pragma omp parallel
    {
        double* t = (double*)malloc(sizeof(double) * T);
        #pragma omp for schedule(dynamic, 4)
        for (int64_t r = 0; r < nrows; ++r) {
            int64_t id = rows[r];
            int i = (int)(id % T), h = (int)((id / T) % H), b = (int)(id / ((int64_t)T * H));
            int kv = h / (H / KV), len = seq_len(&p, b);
            double O[HD], L;
            row_forward(&p, b, h, i, t, O, &L);
            if (O_out) memcpy(O_out + r * HD, O, sizeof O);
            if (L_out) L_out[r] = L;
            double Di = 0.0;
            for (int d = 0; d < HD; ++d) Di += do_at(&p, b, h, i, d) * O[d];
            double* g = dQ + r * HD;
            for (int d = 0; d < HD; ++d) g[d] = 0.0;
            D[r] = Di;                      /* O = 0 on a row with no admitted key */
            if (L == -INFINITY) continue;   /* ... and nothing flows from it */
            for (int j = 0; j < T; ++j) {
                if (!admitted(&p, len, i, j)) continue;
                double P = exp2(t[j] - L);
                double dP = 0.0;
                for (int d = 0; d < HD; ++d) dP += do_at(&p, b, h, i, d) * v_at(&p, b, kv, j, d);
                double dS = P * (dP - Di);
                for (int d = 0; d < HD; ++d) g[d] += dS * k_at(&p, b, kv, j, d);
            }
            for (int d = 0; d < HD; ++d) g[d] *= s;
        }
        free(t);
    }
    return 0;
}

/*
 * Key/value gradients for a list of key columns, column id = (b * KV + kv) * T + j:
 *   dK_j = s sum_{h in group(kv)} sum_i dS_ij Q_i
 *   dV_j =   sum_{h in group(kv)} sum_i P_ij dO_i
 * with P_ij = 2^(t_ij - L_i) and D_i from the oracle's own forward rows.
 * dK, dV: [ncols][64].
 */
int oracle_backward_cols(const double* Q, const double* K, const double* Vt, const double* dO,
                         int B, int T, int H, int KV, int causal, const int32_t* seqlens, double s,
                         const int64_t* cols, int64_t ncols, double* dK, double* dV) {
    if (bad_shape(B, T, H, KV)) return -1;
    int G = H / KV;
    int64_t total = (int64_t)B * KV * T;
    for (int64_t r = 0; r < ncols; ++r)
        if (cols[r] < 0 || cols[r] >= total) return -1;
    problem p = make_problem(Q, K, Vt, dO, B, T, H, KV, causal, seqlens, s);

    /* Which query rows are needed: for each (b, kv) group, rows from the
     * smallest requested key (causal) or from 0, for all G heads. */
    int64_t ngroups = (int64_t)B * KV;
    int* first = (int*)malloc(sizeof(int) * ngroups);
    for (int64_t g = 0; g < ngroups; ++g) first[g] = T;
    for (int64_t r = 0; r < ncols; ++r) {
        int64_t g = cols[r] / T;
        int j = (int)(cols[r] % T);
        int lo = causal ? j : 0;
        if (lo < first[g]) first[g] = lo;
    }
    double* Lrow = (double*)malloc(sizeof(double) * (size_t)B * H * T);
    double* Drow = (double*)malloc(sizeof(double) * (size_t)B * H * T);
    int64_t nrowtasks = (int64_t)B * H * T;
    #pragma omp parallel
    {
        double* t = (double*)malloc(sizeof(double) * T);
        #pragma omp for schedule(dynamic, 8)
        for (int64_t id = 0; id < nrowtasks; ++id) {
            int i = (int)(id % T), h = (int)((id / T) % H), b = (int)(id / ((int64_t)T * H));
            int64_t g = (int64_t)b * KV + h / G;
            if (i < first[g]) continue;
            double O[HD], L, Di = 0.0;
            row_forward(&p, b, h, i, t, O, &L);
            for (int d = 0; d < HD; ++d) Di += do_at(&p, b, h, i, d) * O[d];
            Lrow[id] = L;
            Drow[id] = Di;
        }
        free(t);
    }

    #pragma omp parallel for schedule(dynamic, 1)
    for (int64_t r = 0; r < ncols; ++r) {
        int64_t g = cols[r] / T;
        int j = (int)(cols[r] % T), kv = (int)(g % KV), b = (int)(g / KV), len = seq_len(&p, b);
        double gk[HD], gv[HD];
        for (int d = 0; d < HD; ++d) gk[d] = gv[d] = 0.0;
        for (int hh = 0; hh < G; ++hh) {
            int h = kv * G + hh;
            for (int i = 0; i < T; ++i) {
                if (!admitted(&p, len, i, j)) continue;
                int64_t id = ((int64_t)b * H + h) * T + i;
                double L = Lrow[id], Di = Drow[id];
                double P = exp2(score2(&p, b, h, kv, i, j) - L);
                double dP = 0.0;
                for (int d = 0; d < HD; ++d) dP += do_at(&p, b, h, i, d) * v_at(&p, b, kv, j, d);
                double dS = P * (dP - Di);
                for (int d = 0; d < HD; ++d) {
                    gk[d] += dS * q_at(&p, b, h, i, d);
                    gv[d] += P * do_at(&p, b, h, i, d);
                }
            }
        }
        for (int d = 0; d < HD; ++d) {
            dK[r * HD + d] = s * gk[d];
            dV[r * HD + d] = gv[d];
        }
    }
    free(Lrow);
    free(Drow);
    free(first);
    return 0;
}

/* Number of OpenMP threads the oracle runs on (1 without OpenMP). */
int oracle_threads(void) {
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}
