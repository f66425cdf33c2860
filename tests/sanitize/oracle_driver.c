/*
 * Drives the binary64 oracle (oracle/sa_oracle.c) on small problems so that a
 * build with AddressSanitizer and UndefinedBehaviorSanitizer walks every path
 * of it: causal and full masks, grouped heads, sequence lengths of 0, partial
 * and full, every row and column, bad row/column ids.  It also checks, in
 * binary64, invariants the definition fixes: the backward's O and L equal the
 * forward's, padded rows and keys are exact zeros, sum_j dK_j = 0 and
 * sum_j dV_j = the group's sum of admitted dO rows per sequence.
 * Test infrastructure: built and run by tests/test_sanitizers.py only.
 */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

int oracle_forward_rows(const double* Q, const double* K, const double* Vt, int B, int T, int H, int KV, int causal,
                        const int32_t* seqlens, double s, const int64_t* rows, int64_t nrows, double* O, double* L);
int oracle_backward_rows(const double* Q, const double* K, const double* Vt, const double* dO, int B, int T, int H,
                         int KV, int causal, const int32_t* seqlens, double s, const int64_t* rows, int64_t nrows,
                         double* D, double* dQ, double* O_out, double* L_out);
int oracle_backward_cols(const double* Q, const double* K, const double* Vt, const double* dO, int B, int T, int H,
                         int KV, int causal, const int32_t* seqlens, double s, const int64_t* cols, int64_t ncols,
                         double* dK, double* dV);

static int fails = 0;
#define EXPECT(c) do { if (!(c)) { printf("FAILED: %s (line %d)\n", #c, __LINE__); ++fails; } } while (0)

static uint64_t rng_state = 88172645463325252ull;
static double gauss(void) {  /* sum of four uniforms, centred: a cheap bell shape */
    double u = 0.0;
    for (int i = 0; i < 4; ++i) {
        rng_state ^= rng_state << 13; rng_state ^= rng_state >> 7; rng_state ^= rng_state << 17;
        u += (double)(rng_state >> 11) / 9007199254740992.0;
    }
    return (u - 2.0) * 1.7;
}

static double* randn(size_t n) {
    double* a = malloc(n * sizeof(double));
    for (size_t i = 0; i < n; ++i) a[i] = gauss();
    return a;
}

static void run(int B, int T, int H, int KV, int causal, const int32_t* lens) {
    const double s = 0.125;
    double *Q = randn((size_t)B * H * T * 64), *K = randn((size_t)B * KV * T * 64);
    double *Vt = randn((size_t)B * KV * 64 * T), *dO = randn((size_t)B * H * T * 64);
    int64_t nr = (int64_t)B * H * T, nc = (int64_t)B * KV * T;
    int64_t* rows = malloc(nr * sizeof(int64_t));
    int64_t* cols = malloc(nc * sizeof(int64_t));
    for (int64_t i = 0; i < nr; ++i) rows[i] = i;
    for (int64_t i = 0; i < nc; ++i) cols[i] = i;
    double *O = malloc(nr * 64 * sizeof(double)), *L = malloc(nr * sizeof(double));
    double *O2 = malloc(nr * 64 * sizeof(double)), *L2 = malloc(nr * sizeof(double));
    double *D = malloc(nr * sizeof(double)), *dQ = malloc(nr * 64 * sizeof(double));
    double *dK = malloc(nc * 64 * sizeof(double)), *dV = malloc(nc * 64 * sizeof(double));
    EXPECT(oracle_forward_rows(Q, K, Vt, B, T, H, KV, causal, lens, s, rows, nr, O, L) == 0);
    EXPECT(oracle_backward_rows(Q, K, Vt, dO, B, T, H, KV, causal, lens, s, rows, nr, D, dQ, O2, L2) == 0);
    EXPECT(oracle_backward_cols(Q, K, Vt, dO, B, T, H, KV, causal, lens, s, cols, nc, dK, dV) == 0);
    EXPECT(memcmp(O, O2, nr * 64 * sizeof(double)) == 0);
    for (int64_t i = 0; i < nr; ++i) EXPECT(L[i] == L2[i] || (isinf(L[i]) && isinf(L2[i])));
    int G = H / KV;
    for (int b = 0; b < B; ++b) {
        int n = lens ? (lens[b] < 0 ? 0 : (lens[b] > T ? T : lens[b])) : T;
        for (int h = 0; h < H; ++h)
            for (int i = n; i < T; ++i) {
                int64_t r = ((int64_t)b * H + h) * T + i;
                EXPECT(isinf(L[r]) && L[r] < 0 && D[r] == 0.0);
                for (int d = 0; d < 64; ++d) EXPECT(O[r * 64 + d] == 0.0 && dQ[r * 64 + d] == 0.0);
            }
        for (int kv = 0; kv < KV; ++kv) {
            for (int d = 0; d < 64; ++d) {
                double sk = 0.0, nk = 0.0, sv = 0.0, want = 0.0;
                for (int j = 0; j < T; ++j) {
                    int64_t c = ((int64_t)b * KV + kv) * T + j;
                    if (j >= n) EXPECT(dK[c * 64 + d] == 0.0 && dV[c * 64 + d] == 0.0);
                    sk += dK[c * 64 + d];
                    nk += fabs(dK[c * 64 + d]);
                    sv += dV[c * 64 + d];
                }
                for (int g = 0; g < G; ++g)
                    for (int i = 0; i < n; ++i) want += dO[((((int64_t)b * H + kv * G + g) * T) + i) * 64 + d];
                EXPECT(fabs(sk) <= 1e-9 * (1.0 + nk));
                EXPECT(fabs(sv - want) <= 1e-9 * (1.0 + fabs(want)));
            }
        }
    }
    int64_t bad = nr;
    EXPECT(oracle_forward_rows(Q, K, Vt, B, T, H, KV, causal, lens, s, &bad, 1, O, L) == -1);
    bad = -1;
    EXPECT(oracle_backward_cols(Q, K, Vt, dO, B, T, H, KV, causal, lens, s, &bad, 1, dK, dV) == -1);
    EXPECT(oracle_forward_rows(Q, K, Vt, B, T, 3, 2, causal, lens, s, rows, 1, O, L) == -1);   /* 3 % 2 != 0 */
    free(Q); free(K); free(Vt); free(dO); free(rows); free(cols); free(O); free(L); free(O2); free(L2);
    free(D); free(dQ); free(dK); free(dV);
}

int main(void) {
    run(1, 64, 2, 1, 1, NULL);
    run(2, 96, 4, 2, 1, NULL);
    run(1, 80, 2, 2, 0, NULL);
    const int32_t lens3[3] = {0, 17, 70};
    run(3, 70, 2, 1, 0, lens3);
    const int32_t lens2[2] = {33, 90};
    run(2, 64, 4, 2, 1, lens2);   /* lengths past T are clamped to T */
    printf("%s\n", fails ? "oracle-sanitize: failures" : "oracle-sanitize: ok");
    return fails != 0;
}
