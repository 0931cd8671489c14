// rssm_verify.hip -- output-only speculative verification for gfx950.
//
// Citation keys: [ru] aikraft.ru "ReplaySSM: Революция в декодировании
// гибридных моделей" (§05); [zh] ai.cheesepanini.fun card "ReplaySSM——重新思考
// 混合模型解码的状态存储" (method points: O = S_ckpt Q D + V (W ⊙ K^T Q), the
// checkpoint used once for all T queries, K^T Q shared inside a key group).
//
// The read format RC is the checkpoint's own (RC_NONE fp32, RC_F16 fp16) or
// that of its read copy.  Two variants with the same results: rssm_verify1_kernel for tiles inside one
// key group (queries in registers, scores formed straight from the key loads)
// and rssm_verify_kernel for tiles of several whole key groups (queries, keys
// and scores in LDS).
#include "rssm_replay.h"
#include "rssm_launch.h"
#include "rssm_dispatch.h"

namespace rssm {

// ------------------------------------------------------------------------
// Tiles inside one key group (fp32, bf16 and fp8 reads; MXFP4 copies, with 32
// entries per lane, go through rssm_verify_kernel).
// LDS (sized for C records; staged records use stride nrec = h + T):
//   v [hvpt][nrec][P] | a [hvpt][nrec] | s [C][TT] | y [TT][rows]
// ------------------------------------------------------------------------
// VCAP: the buffer capacity C the key passes are sized for (24 or 40 records).
template <int N, int IN, int RC, int TT, int VCAP>
__global__ __launch_bounds__(RSSM_THREADS) void rssm_verify1_kernel(StepArgs A) {
    extern __shared__ __attribute__((aligned(16))) float lds[];
    constexpr int R4 = N / 4, RPP4 = RSSM_THREADS / R4;
    constexpr int EPL = Ck<RC>::EPL, RR = N / EPL, RPP = RSSM_THREADS / RR;
    constexpr int UV = (RC == RC_NONE) ? 2 : 1;
    const int tid = threadIdx.x;
    if (blockIdx.x == 0 && tid == 0 && A.work) A.work[0] = 0;     // the commit that follows starts an empty list
    const Ctx t = ctx_of(A);
    const int h = A.count[(long)t.b * A.ctiles + t.vh0 / A.chvpt];   // all copies of a row are equal
    const int T = A.T;
    if (h < 0 || h >= A.L) {
        if (tid == 0) atomicOr(A.err, 1);
        return;
    }
    const int nrec = h + T;
    if (nrec > A.C) {
        if (tid == 0) atomicOr(A.err, 4);
        return;
    }
    const int P = A.P, C = A.C, hvpt = A.hvpt, rows = t.rows;
    const int CS = (C + 3) & ~3;
    const long seqhv = t.seqhv;
    // LDS regions (sized for C records and TT queries)
    float* v_l = lds;
    float* a_l = v_l + hvpt * C * P;
    float* sc_l = a_l + hvpt * CS;
    float* y_l = sc_l + C * TT;

    // the checkpoint itself (fp32 or fp16), or its read copy
    const char* rd = (RC == RC_NONE || RC == RC_F16)
        ? reinterpret_cast<const char*>(A.ckpt) + seqhv * P * copy_row_bytes(RC, N)
        : reinterpret_cast<const char*>(A.rcopy) + seqhv * P * copy_row_bytes(RC, N);
    const int rg = tid / RR, gl = tid % RR;
    u32x4 w[UV];
    load_rows<N, RC, UV>(w, rd, 0, rows, rg, gl);
    // queries: draft t's query at q[b][t][kh].  Every load is unconditional
    // (no branch for the compiler to wait in): slots t >= T re-read draft T-1,
    // and what they produce (scores, y) is never read.
    const long qstride = (long)A.Hk * N;                        // between drafts
    const long q0 = (long)t.b * T * qstride + (long)t.kh0 * N;  // draft 0 of this key head
    float qs[TT][EPL];
#pragma unroll
    for (int tq = 0; tq < TT; ++tq) load_in<IN, EPL>(A.q, q0 + min(tq, T - 1) * qstride + gl * EPL, qs[tq]);
    // value and decay regions (loaded together with the keys below)
    const auto rv = v_region<IN, true>(A, t, v_l, nrec, h, T, true);
    const auto ra = a_region<true>(A, t, a_l, nrec, h, T, true);
    Batch4<IN, 2> bv;
    BatchA<1> ba;
    // scores sc[j][t] = k_j . q_t for all records (committed + drafts)
    {
        const int rg4 = tid / R4, gl4 = tid % R4;
        // for the fp32 read format the score lanes hold the same q slices as
        // the checkpoint lanes, so they are reused instead of reloaded
        float q4b[RC == RC_NONE ? 1 : TT][4];
        auto q4 = [&](int tq) -> const float* {
            if constexpr (RC == RC_NONE) return qs[tq];
            else return q4b[tq];
        };
        if constexpr (RC != RC_NONE) {
#pragma unroll
            for (int tq = 0; tq < TT; ++tq)
                InVec4<IN>::load(A.q, q0 + min(tq, T - 1) * qstride + gl4 * 4, q4b[tq]);
        }
        // all key loads first (fixed pass count, unconditional: slots past
        // nrec re-read the last draft's key, and their scores are not stored),
        // then the reductions
        constexpr int VP = (VCAP + RPP4 - 1) / RPP4;        // capacity C <= VCAP records
        float kv[VP][4];
#pragma unroll
        for (int ps = 0; ps < VP; ++ps) {
            const int j = ps * RPP4 + rg4;
            if (j < h)
                InVec4<IN>::load(A.kbuf, (((long)t.b * A.Hk + t.kh0) * C + j) * N + gl4 * 4, kv[ps]);
            else                                            // k has the layout of q
                InVec4<IN>::load(A.k, q0 + min(j - h, T - 1) * qstride + gl4 * 4, kv[ps]);
        }
        // value and decay loads, before anything waits for the keys
        bv.load(rv);
        ba.load(ra);
        // append the drafts' keys (the tile that owns the key group)
        if (t.kwriter) {
#pragma unroll
            for (int ps = 0; ps < VP; ++ps) {
                const int j = ps * RPP4 + rg4;
                if (j >= h && j < nrec)
                    InVec4<IN>::store(A.kbuf, (((long)t.b * A.Hk + t.kh0) * C + j) * N + gl4 * 4, kv[ps]);
            }
        }
#pragma unroll
        for (int ps = 0; ps < VP; ++ps) {
            if (ps * RPP4 >= nrec) break;                  // uniform over the workgroup
            const int j = ps * RPP4 + rg4;
            float sp[TT];
#pragma unroll
            for (int tq = 0; tq < TT; ++tq)
                sp[tq] = kv[ps][0] * q4(tq)[0] + kv[ps][1] * q4(tq)[1] + kv[ps][2] * q4(tq)[2] + kv[ps][3] * q4(tq)[3];
            group_transpose_reduce<TT, R4>(sp, gl4);
            if constexpr (TT >= R4) {
#pragma unroll
                for (int i = 0; i < TT / R4; ++i) {
                    const int tq = gl4 * (TT / R4) + i;
                    if (j < nrec) sc_l[j * TT + tq] = sp[i];
                }
            } else {
                if (gl4 % (R4 / TT) == 0 && j < nrec) sc_l[j * TT + gl4 / (R4 / TT)] = sp[0];
            }
        }
    }
    // value records and decays: committed from the buffer, drafts appended
    bv.store(rv);
    ba.store(ra);
    stage_rest<IN, 2>(rv);
    stage_rest_a<1>(ra);
    lds_barrier();
    // S_ckpt q_t for all t, each checkpoint row read once
    {
        const float* sc = (RC == RC_FP8) ? A.rscale + seqhv * P : nullptr;
        const int nchunks = (rows + UV * RPP - 1) / (UV * RPP);
        for (int c = 0; c < nchunks; ++c) {
            u32x4 nx[UV];
            const bool more = (c + 1 < nchunks);
            if (more) load_rows<N, RC, UV>(nx, rd, c + 1, rows, rg, gl);
            float part[UV * TT];
#pragma unroll
            for (int u = 0; u < UV; ++u) {
                float x[EPL];
                Ck<RC>::decode(w[u], x);
#pragma unroll
                for (int tq = 0; tq < TT; ++tq) {
                    float s = 0.f;
#pragma unroll
                    for (int i = 0; i < EPL; ++i) s = fmaf(x[i], qs[tq][i], s);
                    part[u * TT + tq] = s;
                }
            }
            constexpr int UT = UV * TT;
            group_transpose_reduce<UT, RR>(part, gl);
            auto put = [&](int idx, float val) {
                const int u = idx / TT, tq = idx - u * TT;
                const int row = (c * UV + u) * RPP + rg;
                if (row < rows) {
                    if constexpr (RC == RC_FP8) val *= sc[row];
                    y_l[tq * rows + row] = val;
                }
            };
            if constexpr (UT >= RR) {
#pragma unroll
                for (int i = 0; i < UT / RR; ++i) put(gl * (UT / RR) + i, part[i]);
            } else {
                if (gl % (RR / UT) == 0) put(gl / (RR / UT), part[0]);
            }
            if (more) {
#pragma unroll
                for (int u = 0; u < UV; ++u) w[u] = nx[u];
            }
        }
    }
    lds_barrier();
    // O[t][row] = D_t y_t[row] + sum_{j<=h+t} W[j][t] sc[j][t] v_j[row]
    for (int item = tid; item < rows * T; item += RSSM_THREADS) {
        const int tq = item / rows, row = item - tq * rows;
        const int vh = row / P, p = row - vh * P;
        float c = 1.f, acc = 0.f;
        for (int j = h + tq; j >= 0; --j) {
            acc = fmaf(c * sc_l[j * TT + tq], v_l[(vh * nrec + j) * P + p], acc);
            c *= a_l[vh * nrec + j];
        }
        // o [B][T][Hv][P]
        A.o[(((long)t.b * T + tq) * A.Hv + t.vh0) * P + row] = fmaf(c, y_l[tq * rows + row], acc);
    }
}

// ------------------------------------------------------------------------
// Tiles of several key groups.  Output-only verification of T drafts ([zh] method points, eq. for O with D
// and W; [ru] §05): drafts are appended after the h committed records; the
// checkpoint is read once and dotted with all T queries.
// Reading of D and W (not defined on the pages): D_t = g_{1:h+t},
// W[j][t] = g_{j+1:h+t} for j <= h+t, else 0.
// LDS (sized for TT queries and C records; staged with T and nrec = h + T):
//      q [kgpt][T][N] | k [kgpt][nrec][N] | v [hvpt][nrec][P] | a [hvpt][nrec] |
//      s [kgpt][CS][TT] | y [TT][rows]
// ------------------------------------------------------------------------
template <int N, int IN, int RC, int TT>
__global__ __launch_bounds__(RSSM_THREADS) void rssm_verify_kernel(StepArgs A) {
    extern __shared__ __attribute__((aligned(16))) float lds[];
    constexpr int EPL = Ck<RC>::EPL, RR = N / EPL;
    constexpr int UV = (RC == RC_NONE) ? 2 : 1;
    const int tid = threadIdx.x;
    if (blockIdx.x == 0 && tid == 0 && A.work) A.work[0] = 0;     // the commit that follows starts an empty list
    const Ctx c = ctx_of(A);
    const int h = A.count[(long)c.b * A.ctiles + c.vh0 / A.chvpt];   // all copies of a row are equal
    const int T = A.T;
    if (h < 0 || h >= A.L) {
        if (tid == 0) atomicOr(A.err, 1);
        return;
    }
    const int nrec = h + T;
    if (nrec > A.C) {
        if (tid == 0) atomicOr(A.err, 4);
        return;
    }
    const int P = A.P, C = A.C, CS = (C + 3) & ~3, rows = c.rows;
    float* q_l = lds;
    float* k_l = q_l + c.kgpt * TT * N;
    float* v_l = k_l + c.kgpt * C * N;
    float* a_l = v_l + A.hvpt * C * P;
    float* s_l = a_l + A.hvpt * CS;
    float* y_l = s_l + c.kgpt * CS * TT;

    const char* rd = (RC == RC_NONE || RC == RC_F16)
        ? reinterpret_cast<const char*>(A.ckpt) + c.seqhv * P * copy_row_bytes(RC, N)
        : reinterpret_cast<const char*>(A.rcopy) + c.seqhv * P * copy_row_bytes(RC, N);
    const void* sc = (RC == RC_FP8 || RC == RC_MXFP4)
        ? reinterpret_cast<const char*>(A.rscale) + c.seqhv * P * scale_row_bytes(RC, N) : nullptr;
    u32x4 w[UV];
    int ex[UV];
    load_rows<N, RC, UV>(w, rd, 0, rows, tid / RR, tid % RR);
    load_block_exp<N, RC, UV>(ex, reinterpret_cast<const uint8_t*>(sc), 0, rows, tid / RR, tid % RR);
    stage_qkva<IN, 1, 4, 2>(q_region<N, IN>(A, c, q_l, T),
                            k_region<N, IN, true>(A, c, k_l, nrec, h, T, true),
                            v_region<IN, true>(A, c, v_l, nrec, h, T, true),
                            a_region<true>(A, c, a_l, nrec, h, T, true));
    lds_barrier();
    scores_from_lds<N, TT>(k_l, nrec, q_l, T, s_l, CS, c.kgpt, nrec, T);
    matvec_rows<N, RC, UV, TT>(w, ex, rd, A, c, q_l, T, y_l, rows, sc);
    lds_barrier();
    // O[t][row] = D_t y_t[row] + sum_{j<=h+t} W[j][t] s[j][t] v_j[row]
    for (int item = tid; item < rows * T; item += RSSM_THREADS) {
        const int t = item / rows, row = item - t * rows;
        const int vh = row / P, p = row - vh * P;
        const float* s = s_l + kg_of_head(A, c.kgpt, vh) * CS * TT;
        float g = 1.f, acc = 0.f;
        for (int j = h + t; j >= 0; --j) {
            acc = fmaf(g * s[j * TT + t], v_l[(vh * nrec + j) * P + p], acc);
            g *= a_l[vh * nrec + j];
        }
        // o [B][T][Hv][P]
        A.o[(((long)c.b * T + t) * A.Hv + c.vh0) * P + row] = fmaf(g, y_l[t * rows + row], acc);
    }
}


hipError_t launch_verify(const StepArgs& A, int N, int in_dtype, int rc, int tt, bool multi, int grid,
                         size_t lds, hipStream_t s) {
#define RSSM_V(TTV)                                                                                 \
    if (multi) {                                                                                    \
        RSSM_DISPATCH_N(N, RSSM_DISPATCH_IN(in_dtype, RSSM_DISPATCH_RD(rc,                          \
            hipLaunchKernelGGL((rssm_verify_kernel<NN, II, RCC, TTV>), dim3(grid), dim3(RSSM_THREADS),  \
                               lds, s, A))));                                                       \
    } else if (A.C <= 24) {                                                                         \
        RSSM_DISPATCH_N(N, RSSM_DISPATCH_IN(in_dtype, RSSM_DISPATCH_RD3(rc,                         \
            hipLaunchKernelGGL((rssm_verify1_kernel<NN, II, RCC, TTV, 24>), dim3(grid),             \
                               dim3(RSSM_THREADS), lds, s, A))));                                   \
    } else {                                                                                        \
        RSSM_DISPATCH_N(N, RSSM_DISPATCH_IN(in_dtype, RSSM_DISPATCH_RD3(rc,                         \
            hipLaunchKernelGGL((rssm_verify1_kernel<NN, II, RCC, TTV, 40>), dim3(grid),             \
                               dim3(RSSM_THREADS), lds, s, A))));                                   \
    }
    switch (tt) {
        case 1: RSSM_V(1); break;
        case 2: RSSM_V(2); break;
        case 4: RSSM_V(4); break;
        case 8: RSSM_V(8); break;
        default: return hipErrorInvalidValue;
    }
#undef RSSM_V
    return hipGetLastError();
}

}  // namespace rssm
