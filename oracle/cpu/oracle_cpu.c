/* Plain fp64 stepper of the scalar-decay recurrence -- TEST INFRASTRUCTURE ONLY.
 *
 * Used by the tests for sizes where numpy would be slow, and timed by the
 * benchmark as the CPU baseline.  It is a correctness oracle, not a tuned CPU
 * implementation.  Nothing in the GPU library links or includes this file.
 *
 * Recurrence ([ru] = aikraft.ru article "ReplaySSM: Революция в декодировании
 * гибридных моделей", section 01):
 *     S_t = a_t S_{t-1} + v_t k_t^T,    o_t = S_t q_t
 * for every (sequence b, value head h); value head h reads key/query head
 * h / (Hv / Hk) (a key group shares k and q; aikraft/cheesepanini pages,
 * method points).  Each step first updates the whole P x N state, then forms the
 * output from the updated state; the independent (b, h) pairs run in parallel.
 *
 * Layouts (row-major, last index fastest):
 *   alpha [steps][B][Hv] f32,  k, q [steps][B][Hk][N] f32,  v [steps][B][Hv][P] f32
 *   S     [B][Hv][P][N] f64 (in: initial state, out: final state)
 *   o     [steps][B][Hv][P] f64 (may be NULL)
 * Returns 0, or -1 on bad sizes.
 */
#include <math.h>
#include <stddef.h>
#include <stdint.h>
#include <stdlib.h>
#ifdef _OPENMP
#include <omp.h>
#endif

int oracle_eqR_decode(int B, int Hv, int Hk, int P, int N, int steps,
                      const float* alpha, const float* k, const float* v, const float* q,
                      double* S, double* o, int nthreads)
{
    if (B < 0 || Hv <= 0 || Hk <= 0 || P <= 0 || N <= 0 || steps < 0 || Hv % Hk != 0)
        return -1;
    const int group = Hv / Hk;
    const long pairs = (long)B * Hv;
#ifdef _OPENMP
    if (nthreads > 0) omp_set_num_threads(nthreads);
#pragma omp parallel for schedule(static)
#endif
    for (long pair = 0; pair < pairs; ++pair) {
        const long b = pair / Hv;
        const long h = pair % Hv;
        const long kh = h / group;
        double* St = S + pair * (long)P * N;
        for (int t = 0; t < steps; ++t) {
            const double a = (double)alpha[((long)t * B + b) * Hv + h];
            const float* kt = k + (((long)t * B + b) * Hk + kh) * N;
            const float* qt = q + (((long)t * B + b) * Hk + kh) * N;
            const float* vt = v + (((long)t * B + b) * Hv + h) * P;
            /* state update */
            for (int p = 0; p < P; ++p) {
                const double vp = (double)vt[p];
                double* row = St + (long)p * N;
                for (int n = 0; n < N; ++n)
                    row[n] = a * row[n] + vp * (double)kt[n];
            }
            /* output from the updated state */
            if (o) {
                double* ot = o + (((long)t * B + b) * Hv + h) * P;
                for (int p = 0; p < P; ++p) {
                    const double* row = St + (long)p * N;
                    double acc = 0.0;
                    for (int n = 0; n < N; ++n)
                        acc += row[n] * (double)qt[n];
                    ot[p] = acc;
                }
            }
        }
    }
    return 0;
}

int oracle_threads(void)
{
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}

/* Rounding-error bound of the split-precision read path -- TEST INFRASTRUCTURE.
 *
 * With a read copy R of the checkpoint ([ru] §06), a non-flush output differs
 * from the recurrence only by g_{1:h} (R - S_ckpt) q, where S_ckpt is the state
 * at the last flush (every L steps, flush on the step that fills the window).
 * Each copy entry obeys |R - S| <= u_rel |S| + u_abs amax_row(S); hence
 *     |o_t - o_t^exact|_p <= g_{1:h} ( u_rel (|S_ckpt| |q_t|)_p + u_abs amax_p sum_n |q_t,n| ).
 * This routine steps the recurrence in fp64 and writes, for every step and
 * output element, the two sums  A = g (|S_ckpt| |q|)_p  and  Z = g amax_p sum|q|
 * (zero on flush steps, whose outputs come from the high-precision fold).
 * Layouts as in oracle_eqR_decode; A, Z: [steps][B][Hv][P] f64.
 */
int oracle_split_read_bound(int B, int Hv, int Hk, int P, int N, int steps, int L,
                            const float* alpha, const float* k, const float* v, const float* q,
                            const double* S0, double* A, double* Z, int nthreads)
{
    if (B < 0 || Hv <= 0 || Hk <= 0 || P <= 0 || N <= 0 || steps < 0 || L <= 0 || Hv % Hk != 0)
        return -1;
    const int group = Hv / Hk;
    const long pairs = (long)B * Hv;
#ifdef _OPENMP
    if (nthreads > 0) omp_set_num_threads(nthreads);
#pragma omp parallel for schedule(static)
#endif
    for (long pair = 0; pair < pairs; ++pair) {
        const long b = pair / Hv;
        const long h = pair % Hv;
        const long kh = h / group;
        double* S = (double*)malloc(sizeof(double) * (size_t)P * N);
        double* C = (double*)malloc(sizeof(double) * (size_t)P * N);   /* checkpoint */
        for (long i = 0; i < (long)P * N; ++i) S[i] = C[i] = S0 ? S0[pair * (long)P * N + i] : 0.0;
        double gam = 1.0;
        int since = 0;
        for (int t = 0; t < steps; ++t) {
            const double a = (double)alpha[((long)t * B + b) * Hv + h];
            const float* kt = k + (((long)t * B + b) * Hk + kh) * N;
            const float* qt = q + (((long)t * B + b) * Hk + kh) * N;
            const float* vt = v + (((long)t * B + b) * Hv + h) * P;
            for (int p = 0; p < P; ++p)
                for (int n = 0; n < N; ++n)
                    S[(long)p * N + n] = a * S[(long)p * N + n] + (double)vt[p] * (double)kt[n];
            gam *= a;
            since += 1;
            double* At = A + (((long)t * B + b) * Hv + h) * P;
            double* Zt = Z + (((long)t * B + b) * Hv + h) * P;
            if (since == L) {                      /* flush step: new checkpoint */
                for (long i = 0; i < (long)P * N; ++i) C[i] = S[i];
                for (int p = 0; p < P; ++p) At[p] = Zt[p] = 0.0;
                gam = 1.0;
                since = 0;
                continue;
            }
            double qsum = 0.0;
            for (int n = 0; n < N; ++n) qsum += fabs((double)qt[n]);
            for (int p = 0; p < P; ++p) {
                const double* row = C + (long)p * N;
                double acc = 0.0, amax = 0.0;
                for (int n = 0; n < N; ++n) {
                    acc += fabs(row[n]) * fabs((double)qt[n]);
                    if (fabs(row[n]) > amax) amax = fabs(row[n]);
                }
                At[p] = gam * acc;
                Zt[p] = gam * amax * qsum;
            }
        }
        free(S);
        free(C);
    }
    return 0;
}
