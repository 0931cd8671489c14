/* Drives the C oracle (oracle/cpu/oracle_cpu.c) on a small case so that a
 * build with AddressSanitizer and UndefinedBehaviorSanitizer checks its memory
 * accesses and arithmetic; built without OpenMP (serial loops).  Exit 0 means
 * both entry points ran and rejected invalid shapes; a sanitizer report aborts. */
#include <stdio.h>
#include <stdlib.h>

int oracle_eqR_decode(int B, int Hv, int Hk, int P, int N, int steps,
                      const float* alpha, const float* k, const float* v, const float* q,
                      double* S, double* o, int nthreads);
int oracle_split_read_bound(int B, int Hv, int Hk, int P, int N, int steps, int L,
                            const float* alpha, const float* k, const float* v, const float* q,
                            const double* S0, double* A, double* Z, int nthreads);

static unsigned lcg = 12345u;
static float uni(void) { lcg = lcg * 1664525u + 1013904223u; return (float)((lcg >> 8) & 0xffff) / 65536.0f - 0.5f; }

int main(void) {
    const int B = 2, Hv = 4, Hk = 2, P = 8, N = 16, steps = 21, L = 5;
    const size_t na = (size_t)steps * B * Hv, nk = (size_t)steps * B * Hk * N, nv = (size_t)steps * B * Hv * P;
    float* alpha = malloc(na * sizeof(float));
    float* k = malloc(nk * sizeof(float));
    float* q = malloc(nk * sizeof(float));
    float* v = malloc(nv * sizeof(float));
    double* S = calloc((size_t)B * Hv * P * N, sizeof(double));
    double* S0 = calloc((size_t)B * Hv * P * N, sizeof(double));
    double* o = malloc(nv * sizeof(double));
    double* A = malloc(nv * sizeof(double));
    double* Z = malloc(nv * sizeof(double));
    if (!alpha || !k || !q || !v || !S || !S0 || !o || !A || !Z) return 2;
    for (size_t i = 0; i < na; ++i) alpha[i] = 0.75f + 0.5f * uni();
    for (size_t i = 0; i < nk; ++i) { k[i] = uni(); q[i] = uni(); }
    for (size_t i = 0; i < nv; ++i) v[i] = uni();
    for (size_t i = 0; i < (size_t)B * Hv * P * N; ++i) S0[i] = 0.1 * uni();
    int rc = oracle_eqR_decode(B, Hv, Hk, P, N, steps, alpha, k, v, q, S, o, 1);
    rc |= oracle_split_read_bound(B, Hv, Hk, P, N, steps, L, alpha, k, v, q, S0, A, Z, 1);
    /* invalid shapes are rejected before any access */
    if (oracle_eqR_decode(B, 3, 2, P, N, steps, alpha, k, v, q, S, o, 1) != -1) rc |= 4;
    if (oracle_split_read_bound(B, Hv, Hk, P, N, steps, 0, alpha, k, v, q, S0, A, Z, 1) != -1) rc |= 8;
    double sum = 0.0;
    for (size_t i = 0; i < nv; ++i) sum += o[i] + A[i] + Z[i];
    printf("rc %d checksum %.6e\n", rc, sum);
    free(alpha); free(k); free(q); free(v); free(S); free(S0); free(o); free(A); free(Z);
    return rc == 0 ? 0 : 1;
}
