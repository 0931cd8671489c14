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
#include <stddef.h>
#include <stdint.h>
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
