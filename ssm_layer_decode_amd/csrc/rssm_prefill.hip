// rssm_prefill.hip -- prefill of a prompt into the checkpoint and the record
// buffer, for gfx950.
//
// Citation keys: [zh] ai.cheesepanini.fun card "ReplaySSM——重新思考混合模型解码的
// 状态存储" (method points: the unrolled output O = S_ckpt Q D + V (W ⊙ K^T Q)
// is the chunkwise form prefill kernels use); [ru] aikraft.ru "ReplaySSM:
// Революция в декодировании гибридных моделей" (§03: checkpoint + window of
// records).
//
// Prefill leaves the state that decoding the prompt token by token would:
// outputs o_t = S_t q_t for every prompt token, the checkpoint advanced to the
// last complete window, the buffer holding the records after it.  One
// 256-thread workgroup per (sequence, tile) processes the tile's heads in
// turn.  A head's P x N state stays in registers for the whole prompt (lane
// gl of a row group of N/4 lanes holds 4 entries of each of its NP rows), so
// HBM sees the checkpoint once each way plus the prompt's records.  The
// prompt is cut into chunks of at most 16 queries that never cross a window
// boundary; per chunk (records 0..m-1 of the current window in LDS, the chunk
// being the last n of them):
//   scores  s[j][i] = k_j . q_i
//   outputs O[i] = g_{1:r+1} S q_i + sum_{j<=r} g_{j+1:r+1} s[j][i] v_j,  r = m - n + i
//   fold    when the window is complete: S <- g_{1:L} S + sum_j g_{j+1:L} v_j k_j^T
#include "rssm_replay.h"
#include "rssm_launch.h"
#include "rssm_dispatch.h"

namespace rssm {

constexpr int kPrefillTT = 16;     // queries per chunk

template <int N, int IN, int CK, int NP>
__global__ __launch_bounds__(RSSM_THREADS) void rssm_prefill_kernel(StepArgs A) {
    extern __shared__ __attribute__((aligned(16))) float lds[];
    constexpr int R4 = N / 4, RPP4 = RSSM_THREADS / R4, TT = kPrefillTT;
    const int tid = threadIdx.x, rg = tid / R4, gl = tid % R4;
    const Ctx c = ctx_of(A);
    const int L = A.L, P = A.P, T = A.T, C = A.C, Hv = A.Hv, Hk = A.Hk;
    const int LS = (L + 3) & ~3;
    const int h0 = A.count[c.cidx];
    if (h0 < 0 || h0 >= L) {
        if (tid == 0) atomicOr(A.err, 1);
        return;
    }
    // LDS: window keys [L][N] | values [L][P] | decays [LS] | chunk queries [TT][N] |
    //      scores [L][TT] | S q [TT][P] | G [4]
    float* kw = lds;
    float* vw = kw + L * N;
    float* aw = vw + L * P;
    float* qc = aw + LS;
    float* sc = qc + TT * N;
    float* yc = sc + L * TT;
    float* Gl = yc + TT * P;
    const int folds = (h0 + T) / L;
    const int hend = (h0 + T) % L;
    constexpr int ESZ = InVec4<IN>::ESZ;
    const uint32_t sr_key = fold_key<CK>(A, c.cidx);     // one rounding per prefill that folds

    for (int vh = 0; vh < A.hvpt; ++vh) {
        const long seqhv = c.seqhv + vh;
        const int kh = (c.vh0 + vh) / A.g;
        char* ck = reinterpret_cast<char*>(A.ckpt) + seqhv * P * ck_row_bytes(CK, N);
        const char* kin = reinterpret_cast<const char*>(A.k) + ((long)c.b * T * Hk + kh) * N * ESZ;
        const char* vin = reinterpret_cast<const char*>(A.v) + ((long)c.b * T * Hv + c.vh0 + vh) * P * ESZ;
        const float* ain = A.alpha + (long)c.b * T * Hv + c.vh0 + vh;
        char* kbt = reinterpret_cast<char*>(A.kbuf) + ((long)c.b * Hk + kh) * C * N * ESZ;
        char* vbt = reinterpret_cast<char*>(A.vbuf) + seqhv * C * P * ESZ;
        float* abt = A.abuf + seqhv * C;

        // the head's state in registers
        u32x4 S0[NP];
        load_ck_rows<N, CK, NP>(S0, ck, 0, P, rg, gl);
        f32x4 S[NP];
#pragma unroll
        for (int u = 0; u < NP; ++u) S[u] = ck_values<CK>(S0[u]);
        // records already buffered: window slots [0, h0)
        for (int e = tid; e < h0 * R4; e += RSSM_THREADS)
            InVec4<IN>::load_ptr(kbt + e * 4 * ESZ, kw + 4 * e);
        for (int e = tid; e < h0 * (P / 4); e += RSSM_THREADS)
            InVec4<IN>::load_ptr(vbt + e * 4 * ESZ, vw + 4 * e);
        for (int e = tid; e < h0; e += RSSM_THREADS) aw[e] = abt[e];

        int hw = h0, t0 = 0;
        while (t0 < T) {
            const int n = min(TT, min(L - hw, T - t0));
            const int m = hw + n;
            // stage the chunk: queries, and keys, values, decays at window slots [hw, m)
            for (int e = tid; e < n * R4; e += RSSM_THREADS) {
                const int i = e / R4, c4 = e - i * R4;
                const long off = ((long)(t0 + i) * Hk * N + c4 * 4) * ESZ;
                float x[4];
                InVec4<IN>::load_ptr(reinterpret_cast<const char*>(A.q) + ((long)c.b * T * Hk + kh) * N * ESZ + off, x);
                *reinterpret_cast<f32x4*>(qc + i * N + c4 * 4) = f32x4{x[0], x[1], x[2], x[3]};
                InVec4<IN>::load_ptr(kin + off, x);
                *reinterpret_cast<f32x4*>(kw + (hw + i) * N + c4 * 4) = f32x4{x[0], x[1], x[2], x[3]};
            }
            for (int e = tid; e < n * (P / 4); e += RSSM_THREADS) {
                const int i = e / (P / 4), p4 = e - i * (P / 4);
                float x[4];
                InVec4<IN>::load_ptr(vin + ((long)(t0 + i) * Hv * P + p4 * 4) * ESZ, x);
                *reinterpret_cast<f32x4*>(vw + (hw + i) * P + p4 * 4) = f32x4{x[0], x[1], x[2], x[3]};
            }
            for (int e = tid; e < n; e += RSSM_THREADS) aw[hw + e] = ain[(long)(t0 + e) * Hv];
            lds_barrier();
            // scores s[j][i] (all j < m; the causal ones are used)
            scores_from_lds<N, TT>(kw, L, qc, TT, sc, LS, 1, m, n);
            // S q_i for the chunk's queries
#pragma unroll
            for (int u = 0; u < NP; ++u) {
                float part[TT];
#pragma unroll
                for (int i = 0; i < TT; ++i) {
                    const f32x4 qv = *reinterpret_cast<const f32x4*>(qc + (i < n ? i : 0) * N + gl * 4);
                    part[i] = S[u].x * qv.x + S[u].y * qv.y + S[u].z * qv.z + S[u].w * qv.w;
                }
                group_transpose_reduce<TT, R4>(part, gl);
                const int row = u * RPP4 + rg;
                if (row < P) {
                    if constexpr (TT >= R4) {
#pragma unroll
                        for (int k2 = 0; k2 < TT / R4; ++k2) {
                            const int i = gl * (TT / R4) + k2;
                            if (i < n) yc[i * P + row] = part[k2];
                        }
                    } else {
                        if (gl % (R4 / TT) == 0) {
                            const int i = gl / (R4 / TT);
                            if (i < n) yc[i * P + row] = part[0];
                        }
                    }
                }
            }
            lds_barrier();
            // outputs of the chunk's tokens
            for (int item = tid; item < n * P; item += RSSM_THREADS) {
                const int i = item / P, row = item - i * P, r = hw + i;
                float g = 1.f, acc = 0.f;
                for (int j = r; j >= 0; --j) {
                    acc = fmaf(g * sc[j * TT + i], vw[j * P + row], acc);
                    g *= aw[j];
                }
                A.o[(((long)c.b * T + t0 + i) * Hv + c.vh0 + vh) * P + row] = fmaf(g, yc[i * P + row], acc);
            }
            t0 += n;
            hw = m;
            if (hw == L) {
                // fold the complete window into the state
                lds_barrier();
                make_weights(vw, aw, Gl, 1, P, L, LS, L);
                lds_barrier();
                const float G = Gl[0];
#pragma unroll
                for (int u = 0; u < NP; ++u) S[u] = S[u] * G;
#pragma unroll 1
                for (int j = 0; j < L; ++j) {
                    const f32x4 kj = *reinterpret_cast<const f32x4*>(kw + j * N + gl * 4);
#pragma unroll
                    for (int u = 0; u < NP; ++u) {
                        const int row = u * RPP4 + rg;
                        const float wv = row < P ? vw[j * P + row] : 0.f;
                        S[u].x = fmaf(wv, kj.x, S[u].x);
                        S[u].y = fmaf(wv, kj.y, S[u].y);
                        S[u].z = fmaf(wv, kj.z, S[u].z);
                        S[u].w = fmaf(wv, kj.w, S[u].w);
                    }
                }
                hw = 0;
            }
            lds_barrier();
        }
        // the records after the last window boundary go to the buffer (the
        // ones this prefill added: slots [h0, hend) without a fold, else
        // [0, hend)).  Keys are appended by rssm_prefill_keys_kernel after this
        // kernel: other tiles of a key group may still read slots [0, h0).
        const int first = folds ? 0 : h0;
        for (int e = first * (P / 4) + tid; e < hend * (P / 4); e += RSSM_THREADS)
            InVec4<IN>::store_ptr(vbt + e * 4 * ESZ, vw + 4 * e);
        for (int e = first + tid; e < hend; e += RSSM_THREADS) abt[e] = aw[e];
        if (folds) {
            const long g_tile = seqhv * P * N;
#pragma unroll
            for (int u = 0; u < NP; ++u) {
                const int row = u * RPP4 + rg;
                const float sig = ck_row_scale<N, CK>(S[u]);    // every lane of the row group
                if (row < P) store_ck4<N, CK>(ck, row, gl, S[u], sr_key, g_tile + (long)row * N + gl * 4, sig);
            }
        }
        lds_barrier();
    }
    if (tid == 0) A.count[c.cidx] = hend;
    if (folds) fold_done<CK>(A, c.cidx);
}

// Value of x in lane (lane + K) of the same 16-lane row, or 1 where that
// lane lies past the row's end (a DPP row shift whose out-of-row lanes keep
// the old value).
template <int K>
__device__ __forceinline__ float row_next_or_one(float x) {
    return __int_as_float(__builtin_amdgcn_update_dpp(__float_as_int(1.0f), __float_as_int(x), 0x100 + K, 0xF, 0xF, false));
}

// ------------------------------------------------------------------------
// The same prefill on the matrix cores, for a window of 16 records and P, N
// multiples of 16 (fp32 MFMA 16x16x4: lane l supplies A[l%16][l/16] and
// B[l/16][l%16] and holds D[4(l/16)+r][l%16], r = 0..3).  Each head's state
// is kept transposed, S^T[n][p], in 16x16 accumulator blocks (nb, pb); wave w
// owns the p blocks pb = w, w+4, .. and all n blocks.  Per chunk of n <= 16
// queries (records 0..m-1 of the window in LDS, the chunk the last n):
//   Y^T = Q^T S^T     (t x p; the n sum runs over n = 16 nb + 4 (l/16) + r so
//                      that the state's own accumulator registers are the B
//                      operand)
//   s   = K Q^T       (16 records x 16 queries; the n sum split over the
//                      waves by 16-column group, partial blocks added in M)
//   M[t][j] = g_{j+1:r_t+1} s[j][t] for j <= r_t = m-n+t, else 0;  D_t = g_{1:r_t+1}
//   O^T = D Y^T + M V
//   fold, once the window is full: S^T <- g_{1:16} S^T + K^T W,  W[j] = g_{j+1:16} v_j
//                      (the weights g_{j+1:16} scale the B operand as it is read)
// ------------------------------------------------------------------------
// One p block per wave (P <= 64) fits 4 waves per SIMD and two p blocks 3
// (the compiler's defaults stop at 3 and 1; at 3 waves the two-block kernel
// spills a few registers outside the chunk loop, and runs 10-13 % faster than
// at 2); the chunk's loads are then all issued before their LDS stores, one
// memory round trip per chunk.  Two p blocks per wave stage fp32 inputs that
// way too, with the next chunk's loads in flight (a few registers then spill
// inside the chunk loop, and it still runs 8-11 % faster than loading item by
// item); four p blocks load fp32 inputs item by item.  Rows in LDS are padded (q: N + 4,
// k: N + 16, v: 64 NPB + 16, s and M: 17 floats) so the rows an MFMA operand
// read touches fall in different banks.
template <int N, int IN, int CK, int NPB>
__global__ __launch_bounds__(RSSM_THREADS) __attribute__((amdgpu_waves_per_eu(NPB == 1 ? 4 : NPB == 2 ? 3 : 1, 8)))
void rssm_prefill_mfma_kernel(StepArgs A) {
    extern __shared__ __attribute__((aligned(16))) float lds[];
    constexpr int NNB = N / 16, WIN = 16, ESZ = InVec4<IN>::ESZ;
    constexpr bool BATCH = NPB <= 2 || IN == IN_BF16;
    constexpr bool PIPE = BATCH && NPB >= 2;     // registers allow the next chunk in flight
    const int tid = threadIdx.x, wave = tid / 64, l = tid % 64, lr = l % 16, lq = l / 16;
    const Ctx c = ctx_of(A);
    const int P = A.P, T = A.T, C = A.C, Hv = A.Hv, Hk = A.Hk, NPBALL = P / 16;
    const int h0 = A.count[c.cidx];
    if (h0 < 0 || h0 >= WIN) {
        if (tid == 0) atomicOr(A.err, 1);
        return;
    }
    // LDS: chunk queries [16][N+4] | window keys [16][N+16] | window values [16][64 NPB+16] |
    //      decays [16] | score partials s_w[j][t] [4][16][17] | M[t][j] [16][17] | D [16] |
    //      fold weights [16] | G [4]
    // Padded row strides spread an operand read's lanes over the banks: rows
    // of q and k read 16 at a time as 16-byte pieces (scores, Y: 4 floats of
    // pad), and the fold and outputs read k and v down a column, lanes l / 16
    // on 4 rows (a stride of 16 mod 64 floats puts those rows 16 banks
    // apart).  Value rows take the largest P of the tile class (P <= 64 NPB).
    constexpr int QS = N + 4, KS = N + 16, VS = 64 * NPB + 16, MS = WIN + 1;
    float* qc = lds;
    float* kw = qc + WIN * QS;
    float* vw = kw + WIN * KS;
    float* aw = vw + WIN * VS;
    float* sl = aw + WIN;
    float* Ml = sl + 4 * WIN * MS;
    float* Dl = Ml + WIN * MS;
    float* Wl = Dl + WIN;
    float* Gl = Wl + WIN;
    const int total = WIN * QS + WIN * KS + WIN * VS + WIN + 5 * WIN * MS + 2 * WIN + 4;
    for (int e = tid; e < total; e += RSSM_THREADS) lds[e] = 0.f;     // unused rows stay finite
    lds_barrier();
    const int folds = (h0 + T) / WIN, hend = (h0 + T) % WIN;
    const uint32_t sr_key = fold_key<CK>(A, c.cidx);     // one rounding per prefill that folds

    for (int vh = 0; vh < A.hvpt; ++vh) {
        const long seqhv = c.seqhv + vh;
        const int kh = (c.vh0 + vh) / A.g;
        char* ck = reinterpret_cast<char*>(A.ckpt) + seqhv * P * ck_row_bytes(CK, N);
        const char* qin = reinterpret_cast<const char*>(A.q) + ((long)c.b * T * Hk + kh) * N * ESZ;
        const char* kin = reinterpret_cast<const char*>(A.k) + ((long)c.b * T * Hk + kh) * N * ESZ;
        const char* vin = reinterpret_cast<const char*>(A.v) + ((long)c.b * T * Hv + c.vh0 + vh) * P * ESZ;
        const float* ain = A.alpha + (long)c.b * T * Hv + c.vh0 + vh;
        const char* kbt = reinterpret_cast<const char*>(A.kbuf) + ((long)c.b * Hk + kh) * C * N * ESZ;
        char* vbt = reinterpret_cast<char*>(A.vbuf) + seqhv * C * P * ESZ;
        float* abt = A.abuf + seqhv * C;

        // this lane's outputs: tokens t0 + 4 lq + r of the chunk, value rows 16 pb + lr
        const long HvP = (long)Hv * P;
        float* const oh = A.o + ((long)c.b * T * Hv + c.vh0 + vh) * P + 4 * lq * HvP + lr;
        // S^T blocks: st[ib][nb][r] = S[16 pb + lr][16 nb + 4 lq + r], pb = wave + 4 ib
        f32x4 st[NPB][NNB];
#pragma unroll
        for (int ib = 0; ib < NPB; ++ib) {
            const int pb = wave + 4 * ib;
#pragma unroll
            for (int nb = 0; nb < NNB; ++nb) {
                st[ib][nb] = f32x4{0.f, 0.f, 0.f, 0.f};
                if (pb < NPBALL) {
                    u32x4 w[1];
                    load_ck_rows<N, CK, 1>(w, ck + (long)(16 * pb + lr) * ck_row_bytes(CK, N), 0, 1, 0, 4 * nb + lq);
                    st[ib][nb] = ck_values<CK>(w[0]);
                }
            }
        }
        for (int e = tid; e < h0 * (N / 4); e += RSSM_THREADS)
            InVec4<IN>::load_ptr(kbt + e * 4 * ESZ, kw + (e / (N / 4)) * KS + (e % (N / 4)) * 4);
        for (int e = tid; e < h0 * (P / 4); e += RSSM_THREADS)
            InVec4<IN>::load_ptr(vbt + e * 4 * ESZ, vw + (e / (P / 4)) * VS + (e % (P / 4)) * 4);
        for (int e = tid; e < h0; e += RSSM_THREADS) aw[e] = abt[e];

        int hw = h0, t0 = 0;
        // BATCH: every load of a chunk is issued before its LDS stores; PIPE: they
        // are issued while the previous chunk's outputs and fold run
        constexpr int UQ = (WIN * (N / 4) + RSSM_THREADS - 1) / RSSM_THREADS;
        constexpr int UV = (WIN * 16 * NPB + RSSM_THREADS - 1) / RSSM_THREADS;   // P <= 64 NPB
        using Raw = typename InVec4<IN>::Raw;
        Raw rq[BATCH ? UQ : 1], rk[BATCH ? UQ : 1], rv[BATCH ? UV : 1];
        float a_in = 0.f;
        // item e of a chunk is token e / (N/4) (values: e / (P/4)) and its
        // 16-byte column; the byte offsets from the chunk's first token are
        // the same for every chunk, so the loop adds only the chunk's base
        const long qtok = (long)Hk * N * ESZ, vtok = (long)Hv * P * ESZ;    // bytes per token
        long offq[BATCH ? UQ : 1], offv[BATCH ? UV : 1];
        int iv[BATCH ? UV : 1], pv[BATCH ? UV : 1];
        if constexpr (BATCH) {
#pragma unroll
            for (int u = 0; u < UQ; ++u) {
                const int e = tid + u * RSSM_THREADS, i = e / (N / 4);
                offq[u] = i * qtok + (e - i * (N / 4)) * 4 * ESZ;
            }
#pragma unroll
            for (int u = 0; u < UV; ++u) {
                const int e = tid + u * RSSM_THREADS;
                iv[u] = e / (P / 4);
                pv[u] = e - iv[u] * (P / 4);
                offv[u] = iv[u] * vtok + pv[u] * 4 * ESZ;
            }
        }
        // items past the chunk's end re-read its last item
        auto issue = [&](int ti, int ni) {
            const int nq = ni * (N / 4), nv = ni * (P / 4);
            const char* qb = qin + ti * qtok;
            const char* kb = kin + ti * qtok;
            const char* vb = vin + ti * vtok;
            const long lastq = (ni - 1) * qtok + (N - 4) * ESZ, lastv = (ni - 1) * vtok + (P - 4) * ESZ;
#pragma unroll
            for (int u = 0; u < UQ; ++u) {
                const long off = tid + u * RSSM_THREADS < nq ? offq[u] : lastq;
                rq[u] = InVec4<IN>::load_raw(qb + off);
                rk[u] = InVec4<IN>::load_raw(kb + off);
            }
#pragma unroll
            for (int u = 0; u < UV; ++u)
                rv[u] = InVec4<IN>::load_raw(vb + (tid + u * RSSM_THREADS < nv ? offv[u] : lastv));
            a_in = ain[(long)(ti + min(tid, ni - 1)) * Hv];
        };
        if constexpr (PIPE) issue(0, min(WIN - hw, T));
        while (t0 < T) {
            const int n = min(WIN - hw, T - t0);
            const int m = hw + n;
            if constexpr (BATCH) {
                if constexpr (!PIPE) issue(t0, n);
                const int nq = n * (N / 4), nv = n * (P / 4);
#pragma unroll
                for (int u = 0; u < UQ; ++u) {
                    const int e = tid + u * RSSM_THREADS;
                    if (e < nq) {
                        const int i = e / (N / 4), c4 = e - i * (N / 4);
                        *reinterpret_cast<f32x4*>(qc + i * QS + c4 * 4) = InVec4<IN>::unpack(rq[u]);
                        *reinterpret_cast<f32x4*>(kw + (hw + i) * KS + c4 * 4) = InVec4<IN>::unpack(rk[u]);
                    }
                }
#pragma unroll
                for (int u = 0; u < UV; ++u) {
                    if (tid + u * RSSM_THREADS < nv)
                        *reinterpret_cast<f32x4*>(vw + (hw + iv[u]) * VS + pv[u] * 4) = InVec4<IN>::unpack(rv[u]);
                }
                if (tid < n) aw[hw + tid] = a_in;
            } else {
                for (int e = tid; e < n * (N / 4); e += RSSM_THREADS) {
                    const int i = e / (N / 4), c4 = e - i * (N / 4);
                    const long off = ((long)(t0 + i) * Hk * N + c4 * 4) * ESZ;
                    InVec4<IN>::load_ptr(qin + off, qc + i * QS + c4 * 4);
                    InVec4<IN>::load_ptr(kin + off, kw + (hw + i) * KS + c4 * 4);
                }
                for (int e = tid; e < n * (P / 4); e += RSSM_THREADS) {
                    const int i = e / (P / 4), p4 = e - i * (P / 4);
                    InVec4<IN>::load_ptr(vin + ((long)(t0 + i) * Hv * P + p4 * 4) * ESZ, vw + (hw + i) * VS + p4 * 4);
                }
                for (int e = tid; e < n; e += RSSM_THREADS) aw[hw + e] = ain[(long)(t0 + e) * Hv];
            }
            lds_barrier();
            // scores, the n sum split over the waves by 16-column group (wave w takes
            // groups w, w + 4, ..): acc[r] = s_w[j = 4 lq + r][t = lr]; the four
            // partial blocks are added where M is formed
            {
                f32x4 acc = {0.f, 0.f, 0.f, 0.f};
                for (int nb = wave; nb < NNB; nb += 4) {
                    const f32x4 ka = *reinterpret_cast<const f32x4*>(kw + lr * KS + 16 * nb + 4 * lq);
                    const f32x4 qb = *reinterpret_cast<const f32x4*>(qc + lr * QS + 16 * nb + 4 * lq);
                    acc = __builtin_amdgcn_mfma_f32_16x16x4f32(ka.x, qb.x, acc, 0, 0, 0);
                    acc = __builtin_amdgcn_mfma_f32_16x16x4f32(ka.y, qb.y, acc, 0, 0, 0);
                    acc = __builtin_amdgcn_mfma_f32_16x16x4f32(ka.z, qb.z, acc, 0, 0, 0);
                    acc = __builtin_amdgcn_mfma_f32_16x16x4f32(ka.w, qb.w, acc, 0, 0, 0);
                }
                float* sw = sl + wave * WIN * MS;
                sw[(4 * lq + 0) * MS + lr] = acc.x;
                sw[(4 * lq + 1) * MS + lr] = acc.y;
                sw[(4 * lq + 2) * MS + lr] = acc.z;
                sw[(4 * lq + 3) * MS + lr] = acc.w;
            }
            // Y^T blocks: y[ib][r] = Y^T[t = 4 lq + r][p = 16 pb + lr]
            // one p block per wave: the n sum in two independent chains (even and odd n blocks)
            constexpr int YC = NPB == 1 ? 2 : 1;
            f32x4 y[NPB], y2[NPB];
#pragma unroll
            for (int ib = 0; ib < NPB; ++ib) y[ib] = y2[ib] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int nb = 0; nb < NNB; ++nb) {
                const f32x4 qa = *reinterpret_cast<const f32x4*>(qc + lr * QS + 16 * nb + 4 * lq);
#pragma unroll
                for (int ib = 0; ib < NPB; ++ib) {
                    f32x4& acc = (YC == 2 && (nb & 1)) ? y2[ib] : y[ib];
                    acc = __builtin_amdgcn_mfma_f32_16x16x4f32(qa.x, st[ib][nb].x, acc, 0, 0, 0);
                    acc = __builtin_amdgcn_mfma_f32_16x16x4f32(qa.y, st[ib][nb].y, acc, 0, 0, 0);
                    acc = __builtin_amdgcn_mfma_f32_16x16x4f32(qa.z, st[ib][nb].z, acc, 0, 0, 0);
                    acc = __builtin_amdgcn_mfma_f32_16x16x4f32(qa.w, st[ib][nb].w, acc, 0, 0, 0);
                }
            }
            if constexpr (YC == 2) {
#pragma unroll
                for (int ib = 0; ib < NPB; ++ib) y[ib] = y[ib] + y2[ib];
            }
            lds_barrier();
            // decay-weighted scores M[t][j] and D[t] (rows t >= n are not used).
            // Thread (t, j) is lane j of a 16-lane row; with y_i = a_i for i <= r
            // (else 1) a suffix product over the row gives z_j = prod_{i >= j} y_i,
            // so record j's weight prod_{j < i <= r} a_i is z_{j+1} and
            // D_t = prod_{i <= r} a_i is z_0.  The last row (r = 15) gives the
            // fold's record weights prod_{i > j} a_i and G = prod_i a_i.
            {
                const int t = tid / WIN, j = tid % WIN;
                const int r = min(hw + t, WIN - 1);
                float z = j <= r ? aw[j] : 1.f;
                z *= row_next_or_one<1>(z);
                z *= row_next_or_one<2>(z);
                z *= row_next_or_one<4>(z);
                z *= row_next_or_one<8>(z);
                const float g = row_next_or_one<1>(z);
                const int sj = j * MS + t;
                const float sv = (sl[sj] + sl[WIN * MS + sj]) + (sl[2 * WIN * MS + sj] + sl[3 * WIN * MS + sj]);
                Ml[t * MS + j] = j <= r ? g * sv : 0.f;
                if (j == 0) Dl[t] = z;
                if (t == WIN - 1 && hw + n == WIN) {
                    Wl[j] = g;
                    if (j == 0) Gl[0] = z;
                }
            }
            lds_barrier();
            if constexpr (PIPE) {
                // the next chunk's loads, in flight during the outputs and the fold
                const int tn = t0 + n, hn = (m == WIN) ? 0 : m;
                if (tn < T) issue(tn, min(WIN - hn, T - tn));
            }
            // outputs O^T = D Y^T + M V
#pragma unroll
            for (int ib = 0; ib < NPB; ++ib) {
                const int pb = wave + 4 * ib;
                if (pb >= NPBALL) continue;
                f32x4 o = y[ib];
                o.x *= Dl[4 * lq + 0];
                o.y *= Dl[4 * lq + 1];
                o.z *= Dl[4 * lq + 2];
                o.w *= Dl[4 * lq + 3];
#pragma unroll
                for (int s4 = 0; s4 < WIN / 4; ++s4) {
                    const float a = Ml[lr * MS + 4 * s4 + lq];
                    const float b = vw[(4 * s4 + lq) * VS + 16 * pb + lr];
                    o = __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, o, 0, 0, 0);
                }
                const float ov[4] = {o.x, o.y, o.z, o.w};
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const int t = 4 * lq + r;
                    if (t < n) oh[(t0 + r) * HvP + 16 * pb] = ov[r];
                }
            }
            t0 += n;
            hw = m;
            if (hw == WIN) {
                const float G = Gl[0];
#pragma unroll
                for (int ib = 0; ib < NPB; ++ib)
#pragma unroll
                    for (int nb = 0; nb < NNB; ++nb) st[ib][nb] = st[ib][nb] * G;
#pragma unroll
                for (int s4 = 0; s4 < WIN / 4; ++s4) {
                    float bw[NPB];
#pragma unroll
                    for (int ib = 0; ib < NPB; ++ib) {
                        const int pb = wave + 4 * ib;
                        bw[ib] = pb < NPBALL ? vw[(4 * s4 + lq) * VS + 16 * pb + lr] * Wl[4 * s4 + lq] : 0.f;
                    }
#pragma unroll
                    for (int nb = 0; nb < NNB; ++nb) {
                        const float a = kw[(4 * s4 + lq) * KS + 16 * nb + lr];
#pragma unroll
                        for (int ib = 0; ib < NPB; ++ib)
                            st[ib][nb] = __builtin_amdgcn_mfma_f32_16x16x4f32(a, bw[ib], st[ib][nb], 0, 0, 0);
                    }
                }
                hw = 0;
            }
            lds_barrier();
        }
        const int first = folds ? 0 : h0;
        for (int e = first * (P / 4) + tid; e < hend * (P / 4); e += RSSM_THREADS)
            InVec4<IN>::store_ptr(vbt + e * 4 * ESZ, vw + (e / (P / 4)) * VS + (e % (P / 4)) * 4);
        for (int e = first + tid; e < hend; e += RSSM_THREADS) abt[e] = aw[e];
        if (folds) {
#pragma unroll
            for (int ib = 0; ib < NPB; ++ib) {
                const int pb = wave + 4 * ib;
                if (pb >= NPBALL) continue;
                const int row = 16 * pb + lr;
                // fp8: the row's scale from its N entries, held by lanes lr, lr + 16,
                // lr + 32 and lr + 48 (4 per n block each)
                float sig = 1.0f;
                if constexpr (CK == CK_FP8) {
                    float m = 0.0f;
#pragma unroll
                    for (int nb = 0; nb < NNB; ++nb)
                        m = fmaxf(m, fmaxf(fmaxf(fabsf(st[ib][nb].x), fabsf(st[ib][nb].y)),
                                           fmaxf(fabsf(st[ib][nb].z), fabsf(st[ib][nb].w))));
                    m = fmaxf(m, xor_lane<16>(m));
                    m = fmaxf(m, xor_lane<32>(m));
                    sig = fp8_row_scale_of(m);
                }
#pragma unroll
                for (int nb = 0; nb < NNB; ++nb)
                    store_ck4<N, CK>(ck, row, 4 * nb + lq, st[ib][nb], sr_key,
                                     (seqhv * P + row) * (long)N + 16 * nb + 4 * lq, sig);
            }
        }
        lds_barrier();
    }
    if (tid == 0) A.count[c.cidx] = hend;
    if (folds) fold_done<CK>(A, c.cidx);
}

// Key records of the prompt's last partial window into the buffer: slot j of
// [max(0, hend - T), hend) takes prompt token T - hend + j, hend being the
// record count the prefill left.  Grid: B x Hk workgroups.
template <int IN>
__global__ __launch_bounds__(RSSM_THREADS) void rssm_prefill_keys_kernel(StepArgs A, int N) {
    constexpr int ESZ = InVec4<IN>::ESZ;
    const int b = blockIdx.x / A.Hk, kh = blockIdx.x - b * A.Hk;
    const int tile = (kh * A.g) / A.hvpt;
    const int hend = A.count[(long)b * A.tiles + tile], T = A.T;
    if (hend < 0 || hend >= A.L) return;           // flagged by the prefill kernel
    const int lo = hend > T ? hend - T : 0, R4 = N / 4;
    char* kbt = reinterpret_cast<char*>(A.kbuf) + ((long)b * A.Hk + kh) * A.C * N * ESZ;
    const char* kin = reinterpret_cast<const char*>(A.k);
    for (int e = lo * R4 + threadIdx.x; e < hend * R4; e += RSSM_THREADS) {
        const int j = e / R4, c4 = e - j * R4;
        float x[4];
        InVec4<IN>::load_ptr(kin + ((((long)b * T + (T - hend + j)) * A.Hk + kh) * N + c4 * 4) * ESZ, x);
        InVec4<IN>::store_ptr(kbt + ((long)j * N + c4 * 4) * ESZ, x);
    }
}

// Launch of the matrix-core kernel.  The host takes it only with NPB (N / 16)
// <= 16 (the state blocks one wave holds), so the other combinations are not
// instantiated.
template <int N, int IN, int CK, int NPB>
hipError_t launch_prefill_mfma(const StepArgs& A, int grid, size_t lds, hipStream_t s) {
    if constexpr (NPB * (N / 16) <= 16) {
        hipLaunchKernelGGL((rssm_prefill_mfma_kernel<N, IN, CK, NPB>), dim3(grid), dim3(RSSM_THREADS), lds, s, A);
        return hipSuccess;
    } else {
        return hipErrorInvalidValue;
    }
}

// Rows per thread per head: the smallest of 2, 4, 8, 16 with NP * (1024 / N) >= P.
// np > 0: the VALU kernel with np rows per thread per head; np < 0: the
// matrix-core kernel with -np p blocks per wave.
hipError_t launch_prefill(const StepArgs& A, int N, int in_dtype, int ck, int np, int grid, size_t lds,
                          hipStream_t s) {
#define RSSM_PF(NPV)                                                                                   \
    RSSM_DISPATCH_N(N, RSSM_DISPATCH_IN(in_dtype, RSSM_DISPATCH_CK(ck,                                 \
        hipLaunchKernelGGL((rssm_prefill_kernel<NN, II, CKK, NPV>), dim3(grid), dim3(RSSM_THREADS), lds, s, A))))
#define RSSM_PFM(NPB)                                                                                  \
    RSSM_DISPATCH_N(N, RSSM_DISPATCH_IN(in_dtype, RSSM_DISPATCH_CK(ck, {                               \
        const hipError_t r = launch_prefill_mfma<NN, II, CKK, NPB>(A, grid, lds, s);                   \
        if (r != hipSuccess) return r; })))
    switch (np) {
        case 2: RSSM_PF(2); break;
        case 4: RSSM_PF(4); break;
        case 8: RSSM_PF(8); break;
        case 16: RSSM_PF(16); break;
        case -1: RSSM_PFM(1); break;
        case -2: RSSM_PFM(2); break;
        case -4: RSSM_PFM(4); break;
        default: return hipErrorInvalidValue;
    }
#undef RSSM_PF
#undef RSSM_PFM
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    switch (in_dtype) {
        case IN_F32: hipLaunchKernelGGL((rssm_prefill_keys_kernel<IN_F32>), dim3(A.B * A.Hk), dim3(RSSM_THREADS), 0, s, A, N); break;
        case IN_BF16: hipLaunchKernelGGL((rssm_prefill_keys_kernel<IN_BF16>), dim3(A.B * A.Hk), dim3(RSSM_THREADS), 0, s, A, N); break;
        default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

}  // namespace rssm
