// rssm_kernels.hip -- ReplaySSM decode, fold, verify and copy kernels for gfx950.
//
// Citation keys: [ru] aikraft.ru "ReplaySSM: Революция в декодировании
// гибридных моделей" (§01-§07); [ar] sitech.ge "NVIDIA و Dao AI Lab يقدّمان
// ReplaySSM ..."; [zh] ai.cheesepanini.fun card "ReplaySSM——重新思考混合模型
// 解码的状态存储".
//
// The state of one (sequence, value head) is an fp32 checkpoint S_ckpt (P x N)
// plus the records (a_j, k_j, v_j) appended since it was written
// ([ru] §03; [zh] method points).  With g_{a:b} = prod_{i=a..b} a_i:
//   replay output     o = g_{1:h} S_ckpt q + sum_{j<=h} g_{j+1:h} v_j (k_j . q)
//                     (unrolled window of [ru] §03, rank-1 output of [ru] §05)
//   fold              S_ckpt <- g_{1:h} S_ckpt + sum_{j<=h} g_{j+1:h} v_j k_j^T
//   T-query verify    O[t] = g_{1:h+t} S_ckpt q_t + sum_{j<=h+t} g_{j+1:h+t} v_j (k_j . q_t)
//                     (output-only chunk of [zh] method points: the checkpoint
//                     is read once for all T queries, scores k^T q are shared by
//                     the value heads of a key group)
//
// All kernels: one 256-thread workgroup per (sequence, tile); a tile is `hvpt`
// value heads of one key group, so its scores are computed once and shared
// through LDS.  The per-tile copy count[b][tile] of the record pointer is read
// at the start and rewritten at the end by that workgroup only, so no kernel
// needs synchronisation between workgroups.  Records are staged in LDS; the
// checkpoint streams through registers in 16-byte loads, issued before the
// record staging so that they are in flight while the small work runs.
#include "rssm_stream.h"

namespace rssm {

// Fold the nrec records staged in LDS into the tile's checkpoint:
//   S <- G[vh] S + sum_j w[vh][j][p] k_j        (w = g_{j+1:h} v_j, precomputed)
// Chunk 0 of the fp32 rows is already loaded in S0.  Writes the checkpoint (and
// the read copy); with OUT also writes y[row] = S_new[row] . q.
template <int N, int RC, int UF, bool OUT>
__device__ __forceinline__ void fold_tile(u32x4 (&S0)[UF], float* ck_tile, void* rcopy_tile,
                                          float* rscale_tile, int rows, int P, int L, int nrec,
                                          const float* k_l, const float* w_l, const float* G_l,
                                          const float* q4, float* y) {
    constexpr int R4 = N / 4;
    constexpr int RPP4 = RSSM_THREADS / R4;
    const int tid = threadIdx.x, rg = tid / R4, gl = tid % R4;
    const int nchunks = (rows + UF * RPP4 - 1) / (UF * RPP4);
    const char* base = reinterpret_cast<const char*>(ck_tile);
    for (int c = 0; c < nchunks; ++c) {
        if (c > 0) load_rows<N, RC_NONE, UF>(S0, base, c, rows, rg, gl);
        f32x4 S[UF];
        int woff[UF];
#pragma unroll
        for (int u = 0; u < UF; ++u) {
            const int row = (c * UF + u) * RPP4 + rg;
            const int r = row < rows ? row : 0;
            const int vh = r / P;
            woff[u] = vh * L * P + (r - vh * P);
            S[u] = f32x4{__uint_as_float(S0[u].x), __uint_as_float(S0[u].y),
                         __uint_as_float(S0[u].z), __uint_as_float(S0[u].w)} * G_l[vh];
        }
#pragma unroll 1
        for (int j = 0; j < nrec; ++j) {
            const f32x4 kj = *reinterpret_cast<const f32x4*>(k_l + j * N + gl * 4);
#pragma unroll
            for (int u = 0; u < UF; ++u) {
                const float wv = w_l[woff[u] + j * P];
                S[u].x = fmaf(wv, kj.x, S[u].x);
                S[u].y = fmaf(wv, kj.y, S[u].y);
                S[u].z = fmaf(wv, kj.z, S[u].z);
                S[u].w = fmaf(wv, kj.w, S[u].w);
            }
        }
        float part[UF];
#pragma unroll
        for (int u = 0; u < UF; ++u) {
            const int row = (c * UF + u) * RPP4 + rg;
            if (row < rows) {
                st16(reinterpret_cast<char*>(ck_tile) + (long)row * N * 4 + gl * 16,
                     u32x4{__float_as_uint(S[u].x), __float_as_uint(S[u].y),
                           __float_as_uint(S[u].z), __float_as_uint(S[u].w)});
            }
            if constexpr (RC != RC_NONE) {
                store_copy<N, RC>(S[u], rcopy_tile, rscale_tile, row, gl, row < rows);
            }
            if constexpr (OUT) part[u] = S[u].x * q4[0] + S[u].y * q4[1] + S[u].z * q4[2] + S[u].w * q4[3];
        }
        if constexpr (OUT) {
            group_transpose_reduce<UF, R4>(part, gl);
            put_rows<N, RC_NONE, UF>(part, y, c, rows, rg, gl, nullptr);
        }
    }
}

// LDS layout shared by decode and fold: k_l [L][N], v_l [hvpt][L][P],
// a_l [hvpt][LS], s_l [LS], y_l [rows], G_l [hvpt] (floats; LS = L rounded to 4).
struct Lds {
    float *k, *v, *a, *s, *y, *G;
};
__device__ __forceinline__ Lds carve(float* lds, int N, int L, int hvpt, int P) {
    const int LS = (L + 3) & ~3;
    Lds d;
    d.k = lds;
    d.v = d.k + L * N;
    d.a = d.v + hvpt * L * P;
    d.s = d.a + hvpt * LS;
    d.y = d.s + LS;
    d.G = d.y + ((hvpt * P + 3) & ~3);
    return d;
}

// Stage value records j < nrec into v_l[vh][j][p] (fp32): slot j < h_buf from the
// buffer, later ones from `src` (the step's inputs, record j - h_buf, stride
// src_rec elements between records); when `append` also store those raw into
// the buffer at slot j.
template <int IN, bool WITH_INPUT>
__device__ __forceinline__ void stage_v(const StepArgs& A, const Tile& t, float* v_l, int nrec,
                                        int h_buf, const void* src, long src_b, long src_rec,
                                        bool append) {
    const int P = A.P, P4 = P / 4, L = A.L;
    const int total = A.hvpt * nrec * P4;
#pragma unroll 1
    for (int e = threadIdx.x; e < total; e += RSSM_THREADS) {
        const int vh = e / (nrec * P4);
        const int r = e - vh * nrec * P4;
        const int j = r / P4, p4 = r - j * P4;
        const long vrow = (long)t.b * A.Hv + t.vh0 + vh;
        float x[4];
        if (!WITH_INPUT || j < h_buf) {
            InVec4<IN>::load(A.vbuf, (vrow * A.C + j) * P + p4 * 4, x);
        } else {
            const long sidx = src_b + (long)(j - h_buf) * src_rec + (long)(t.vh0 + vh) * P + p4 * 4;
            InVec4<IN>::load(src, sidx, x);
            if (append) copy_vec4<IN>(A.vbuf, (vrow * A.C + j) * P + p4 * 4, src, sidx);
        }
        *reinterpret_cast<f32x4*>(v_l + (vh * L + j) * P + p4 * 4) = f32x4{x[0], x[1], x[2], x[3]};
    }
}

// Stage decays j < nrec into a_l[vh][j]; same sourcing rules as stage_v.
template <bool WITH_INPUT>
__device__ __forceinline__ void stage_a(const StepArgs& A, const Tile& t, float* a_l, int nrec,
                                        int h_buf, const float* src, long src_b, long src_rec,
                                        bool append) {
    const int LS = (A.L + 3) & ~3;
    const int total = A.hvpt * nrec;
#pragma unroll 1
    for (int e = threadIdx.x; e < total; e += RSSM_THREADS) {
        const int vh = e / nrec, j = e - vh * nrec;
        const long arow = (long)t.b * A.Hv + t.vh0 + vh;
        float a;
        if (!WITH_INPUT || j < h_buf) {
            a = A.abuf[arow * A.C + j];
        } else {
            a = src[src_b + (long)(j - h_buf) * src_rec + t.vh0 + vh];
            if (append) A.abuf[arow * A.C + j] = a;
        }
        a_l[vh * LS + j] = a;
    }
}

// w[vh][j][p] <- g_{j+1:nrec} v[vh][j][p] in place, and G[vh] = g_{1:nrec}.
__device__ __forceinline__ void make_weights(const Lds& d, int hvpt, int P, int L, int nrec) {
    const int LS = (L + 3) & ~3;
    for (int row = threadIdx.x; row < hvpt * P; row += RSSM_THREADS) {
        const int vh = row / P, p = row - vh * P;
        float c = 1.0f;
        for (int j = nrec - 1; j >= 0; --j) {
            float* wp = d.v + (vh * L + j) * P + p;
            *wp = c * *wp;
            c *= d.a[vh * LS + j];
        }
        if (p == 0) d.G[vh] = c;
    }
}

// ------------------------------------------------------------------------
// Decode step: append + replay output, or fold on the step that fills the
// window ([ru] §03 non-flush and flush steps; [ar] "how ReplaySSM works").
// ------------------------------------------------------------------------
template <int N, int IN, int RC>
__global__ __launch_bounds__(RSSM_THREADS) void rssm_decode_kernel(StepArgs A) {
    extern __shared__ __attribute__((aligned(16))) float lds[];
    constexpr int R4 = N / 4, RPP4 = RSSM_THREADS / R4;
    constexpr int EPL = Ck<RC>::EPL, RR = N / EPL;
    constexpr int UM = ReadU<RC>::U, UF = 4;
    constexpr int SP = (32 + RPP4 - 1) / RPP4;    // score passes for up to 32 records

    const int tid = threadIdx.x;
    const Tile t = tile_of(A);
    const int h = A.count[t.cidx];
    if (h < 0 || h >= A.L) {
        if (tid == 0) atomicOr(A.err, 1);
        return;
    }
    const int P = A.P, L = A.L, hvpt = A.hvpt, rows = hvpt * P;
    const int nrec = h + 1;
    const bool flush = (nrec == L);
    const long seqhv = (long)t.b * A.Hv + t.vh0;
    float* ck_tile = A.ckpt + seqhv * P * N;
    const Lds d = carve(lds, N, L, hvpt, P);
    const long qoff = ((long)t.b * A.Hk + t.kh) * N;
    const int rg4 = tid / R4, gl4 = tid % R4;

    if (!flush) {
        // ---- non-flush: read checkpoint (or its copy), replay the records ----
        const char* rd = (RC == RC_NONE)
            ? reinterpret_cast<const char*>(ck_tile)
            : reinterpret_cast<const char*>(A.rcopy) + seqhv * P * N * Ck<RC>::ESZ;
        const int rg = tid / RR, gl = tid % RR;
        u32x4 w[UM];
        load_rows<N, RC, UM>(w, rd, 0, rows, rg, gl);
        float qs[EPL];
        load_in<IN, EPL>(A.q, qoff + gl * EPL, qs);
        float q4[4];
        InVec4<IN>::load(A.q, qoff + gl4 * 4, q4);
        // key records -> scores s_j = k_j . q (current record from the inputs)
        float sp[SP];
#pragma unroll
        for (int ps = 0; ps < SP; ++ps) {
            const int j = ps * RPP4 + rg4;
            float kv[4] = {0.f, 0.f, 0.f, 0.f};
            if (j < h) {
                InVec4<IN>::load(A.kbuf, (((long)t.b * A.Hk + t.kh) * A.C + j) * N + gl4 * 4, kv);
            } else if (j == h) {
                InVec4<IN>::load(A.k, qoff + gl4 * 4, kv);
                if (t.kwriter)
                    copy_vec4<IN>(A.kbuf, (((long)t.b * A.Hk + t.kh) * A.C + j) * N + gl4 * 4, A.k,
                                  qoff + gl4 * 4);
            }
            sp[ps] = kv[0] * q4[0] + kv[1] * q4[1] + kv[2] * q4[2] + kv[3] * q4[3];
        }
        stage_v<IN, true>(A, t, d.v, nrec, h, A.v, (long)t.b * A.Hv * P, 0, true);
        stage_a<true>(A, t, d.a, nrec, h, A.alpha, (long)t.b * A.Hv, 0, true);
        group_transpose_reduce<SP, R4>(sp, gl4);
        if (gl4 % (R4 / SP) == 0) {
            const int j = (gl4 / (R4 / SP)) * RPP4 + rg4;
            if (j < nrec) d.s[j] = sp[0];
        }
        lds_barrier();
        const float* sc = (RC == RC_FP8) ? A.rscale + seqhv * P : nullptr;
        matvec_tile<N, RC, UM>(w, rd, rows, qs, d.y, sc);
        // replay vector r = sum_j g_{j+1:h+1} s_j v_j and G = g_{1:h+1}
        const int LS = (L + 3) & ~3;
        float r[4], G[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int row = tid + i * RSSM_THREADS;
            r[i] = 0.f; G[i] = 1.f;
            if (row < rows) {
                const int vh = row / P, p = row - vh * P;
                float c = 1.f, acc = 0.f;
                for (int j = nrec - 1; j >= 0; --j) {
                    acc = fmaf(c * d.s[j], d.v[(vh * L + j) * P + p], acc);
                    c *= d.a[vh * LS + j];
                }
                r[i] = acc; G[i] = c;
            }
        }
        lds_barrier();
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int row = tid + i * RSSM_THREADS;
            if (row < rows) A.o[seqhv * P + row] = fmaf(G[i], d.y[row], r[i]);
        }
        if (tid == 0) A.count[t.cidx] = nrec;
    } else {
        // ---- flush: fold the L records, write checkpoint (+copy) once ----
        u32x4 S0[UF];
        load_rows<N, RC_NONE, UF>(S0, reinterpret_cast<const char*>(ck_tile), 0, rows, rg4, gl4);
        float q4[4];
        InVec4<IN>::load(A.q, qoff + gl4 * 4, q4);
#pragma unroll 1
        for (int e = tid; e < nrec * R4; e += RSSM_THREADS) {
            const int j = e / R4, c4 = e - j * R4;
            float kv[4];
            if (j < h) InVec4<IN>::load(A.kbuf, (((long)t.b * A.Hk + t.kh) * A.C + j) * N + c4 * 4, kv);
            else InVec4<IN>::load(A.k, qoff + c4 * 4, kv);
            *reinterpret_cast<f32x4*>(d.k + j * N + c4 * 4) = f32x4{kv[0], kv[1], kv[2], kv[3]};
        }
        stage_v<IN, true>(A, t, d.v, nrec, h, A.v, (long)t.b * A.Hv * P, 0, false);
        stage_a<true>(A, t, d.a, nrec, h, A.alpha, (long)t.b * A.Hv, 0, false);
        lds_barrier();
        make_weights(d, hvpt, P, L, nrec);
        lds_barrier();
        void* rc_tile = (RC == RC_NONE) ? nullptr
            : reinterpret_cast<char*>(A.rcopy) + seqhv * P * N * Ck<RC>::ESZ;
        float* rs_tile = (RC == RC_FP8) ? A.rscale + seqhv * P : nullptr;
        fold_tile<N, RC, UF, true>(S0, ck_tile, rc_tile, rs_tile, rows, P, L, nrec, d.k, d.v, d.G, q4, d.y);
        lds_barrier();
        for (int row = tid; row < rows; row += RSSM_THREADS) A.o[seqhv * P + row] = d.y[row];
        if (tid == 0) A.count[t.cidx] = 0;
    }
}

// ------------------------------------------------------------------------
// Standalone fold: explicit flush (fold h > 0 records) or commit (advance
// the pointer by accepted[b]; fold every committed record once it reaches L)
// ([ru] §03 flush; [ru] §05 commit by pointer advance; [zh] method points).
// ------------------------------------------------------------------------
template <int N, int IN, int RC>
__global__ __launch_bounds__(RSSM_THREADS) void rssm_fold_kernel(StepArgs A) {
    extern __shared__ __attribute__((aligned(16))) float lds[];
    constexpr int R4 = N / 4, RPP4 = RSSM_THREADS / R4, UF = 4;
    const int tid = threadIdx.x;
    const Tile t = tile_of(A);
    const int h = A.count[t.cidx];
    const int Lc = A.C;    // staging capacity (records)
    if (h < 0 || h >= A.L) {
        if (tid == 0) atomicOr(A.err, 1);
        return;
    }
    int nrec = h;
    if (A.mode == FOLD_COMMIT) {
        const int acc = A.accepted[t.b];
        if (acc < 0 || acc > A.T) {
            if (tid == 0) atomicOr(A.err, 2);
            return;
        }
        nrec = h + acc;
        if (nrec > A.C) {
            if (tid == 0) atomicOr(A.err, 4);
            return;
        }
        if (nrec < A.L) {
            if (tid == 0) A.count[t.cidx] = nrec;
            return;
        }
    } else if (nrec == 0) {
        return;
    }
    const int P = A.P, hvpt = A.hvpt, rows = hvpt * P;
    const long seqhv = (long)t.b * A.Hv + t.vh0;
    float* ck_tile = A.ckpt + seqhv * P * N;
    const Lds d = carve(lds, N, Lc, hvpt, P);
    const int rg4 = tid / R4, gl4 = tid % R4;
    u32x4 S0[UF];
    load_rows<N, RC_NONE, UF>(S0, reinterpret_cast<const char*>(ck_tile), 0, rows, rg4, gl4);
    for (int j = rg4; j < nrec; j += RPP4) {
        float kv[4];
        InVec4<IN>::load(A.kbuf, (((long)t.b * A.Hk + t.kh) * A.C + j) * N + gl4 * 4, kv);
        *reinterpret_cast<f32x4*>(d.k + j * N + gl4 * 4) = f32x4{kv[0], kv[1], kv[2], kv[3]};
    }
    // stage with capacity C so that up to L-1+T committed records fit
    StepArgs B = A;
    B.L = Lc;
    stage_v<IN, false>(B, t, d.v, nrec, nrec, nullptr, 0, 0, false);
    stage_a<false>(B, t, d.a, nrec, nrec, nullptr, 0, 0, false);
    lds_barrier();
    make_weights(d, hvpt, P, Lc, nrec);
    lds_barrier();
    void* rc_tile = (RC == RC_NONE) ? nullptr
        : reinterpret_cast<char*>(A.rcopy) + seqhv * P * N * Ck<RC>::ESZ;
    float* rs_tile = (RC == RC_FP8) ? A.rscale + seqhv * P : nullptr;
    fold_tile<N, RC, UF, false>(S0, ck_tile, rc_tile, rs_tile, rows, P, Lc, nrec, d.k, d.v, d.G, nullptr, nullptr);
    if (tid == 0) A.count[t.cidx] = 0;
}

// ------------------------------------------------------------------------
// Output-only verification of T drafts ([zh] method points, eq. for O with D
// and W; [ru] §05): drafts are appended after the h committed records; the
// checkpoint is read once and dotted with all T queries.
// Reading of D and W (not defined on the pages): D_t = g_{1:h+t},
// W[j][t] = g_{j+1:h+t} for j <= h+t, else 0.
// ------------------------------------------------------------------------
template <int N, int IN, int RC, int TT>
__global__ __launch_bounds__(RSSM_THREADS) void rssm_verify_kernel(StepArgs A) {
    extern __shared__ __attribute__((aligned(16))) float lds[];
    constexpr int R4 = N / 4, RPP4 = RSSM_THREADS / R4;
    constexpr int EPL = Ck<RC>::EPL, RR = N / EPL, RPP = RSSM_THREADS / RR;
    constexpr int UV = (RC == RC_NONE) ? 2 : 1;
    const int tid = threadIdx.x;
    const Tile t = tile_of(A);
    const int h = A.count[t.cidx];
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
    const int P = A.P, C = A.C, hvpt = A.hvpt, rows = hvpt * P;
    const int CS = (C + 3) & ~3;
    const long seqhv = (long)t.b * A.Hv + t.vh0;
    // LDS: v_l [hvpt][C][P], a_l [hvpt][CS], sc_l [C][TT], y_l [TT][rows]
    float* v_l = lds;
    float* a_l = v_l + hvpt * C * P;
    float* sc_l = a_l + hvpt * CS;
    float* y_l = sc_l + C * TT;

    const char* rd = (RC == RC_NONE)
        ? reinterpret_cast<const char*>(A.ckpt + seqhv * P * N)
        : reinterpret_cast<const char*>(A.rcopy) + seqhv * P * N * Ck<RC>::ESZ;
    const int rg = tid / RR, gl = tid % RR;
    u32x4 w[UV];
    load_rows<N, RC, UV>(w, rd, 0, rows, rg, gl);
    // queries: draft t's query at q[b][t][kh]
    const long qstride = (long)A.Hk * N;                        // between drafts
    const long q0 = (long)t.b * T * qstride + (long)t.kh * N;  // draft 0 of this key head
    float qs[TT][EPL];
#pragma unroll
    for (int tq = 0; tq < TT; ++tq) {
        if (tq < T) load_in<IN, EPL>(A.q, q0 + tq * qstride + gl * EPL, qs[tq]);
        else {
#pragma unroll
            for (int i = 0; i < EPL; ++i) qs[tq][i] = 0.f;
        }
    }
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
            for (int tq = 0; tq < TT; ++tq) {
                if (tq < T) InVec4<IN>::load(A.q, q0 + tq * qstride + gl4 * 4, q4b[tq]);
                else { q4b[tq][0] = q4b[tq][1] = q4b[tq][2] = q4b[tq][3] = 0.f; }
            }
        }
        // all key loads first (predicated, fixed pass count), then the reductions
        constexpr int VP = (40 + RPP4 - 1) / RPP4;          // capacity C <= 40 records
        float kv[VP][4];
#pragma unroll
        for (int ps = 0; ps < VP; ++ps) {
            const int j = ps * RPP4 + rg4;
            kv[ps][0] = kv[ps][1] = kv[ps][2] = kv[ps][3] = 0.f;
            if (j < h) {
                InVec4<IN>::load(A.kbuf, (((long)t.b * A.Hk + t.kh) * C + j) * N + gl4 * 4, kv[ps]);
            } else if (j < nrec) {
                const long src = q0 + (j - h) * qstride + gl4 * 4;   // k has the layout of q
                InVec4<IN>::load(A.k, src, kv[ps]);
                if (t.kwriter)
                    copy_vec4<IN>(A.kbuf, (((long)t.b * A.Hk + t.kh) * C + j) * N + gl4 * 4, A.k, src);
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
    {
        StepArgs B = A;
        B.L = C;
        stage_v<IN, true>(B, t, v_l, nrec, h, A.v, (long)t.b * T * A.Hv * P, (long)A.Hv * P, true);
        stage_a<true>(B, t, a_l, nrec, h, A.alpha, (long)t.b * T * A.Hv, A.Hv, true);
    }
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
            acc = fmaf(c * sc_l[j * TT + tq], v_l[(vh * C + j) * P + p], acc);
            c *= a_l[vh * CS + j];
        }
        // o [B][T][Hv][P]
        A.o[(((long)t.b * T + tq) * A.Hv + t.vh0) * P + row] = fmaf(c, y_l[tq * rows + row], acc);
    }
}

// ------------------------------------------------------------------------
// Read copy refresh: R = Q(S_ckpt) for every row ([ru] §06: the copy is
// derived from the high-precision checkpoint, never the other way round).
// ------------------------------------------------------------------------
template <int N, int RC>
__global__ __launch_bounds__(RSSM_THREADS) void rssm_refresh_kernel(StepArgs A) {
    constexpr int R4 = N / 4, RPP4 = RSSM_THREADS / R4;
    const Tile t = tile_of(A);
    const int rows = A.hvpt * A.P;
    const long seqhv = (long)t.b * A.Hv + t.vh0;
    const float* ck = A.ckpt + seqhv * A.P * N;
    void* rc = reinterpret_cast<char*>(A.rcopy) + seqhv * A.P * N * Ck<RC>::ESZ;
    float* rs = (RC == RC_FP8) ? A.rscale + seqhv * A.P : nullptr;
    const int rg4 = threadIdx.x / R4, gl4 = threadIdx.x % R4;
    for (int row0 = 0; row0 < rows; row0 += RPP4) {
        const int row = row0 + rg4;
        f32x4 s = {0.f, 0.f, 0.f, 0.f};
        if (row < rows) s = *reinterpret_cast<const f32x4*>(ck + (long)row * N + gl4 * 4);
        store_copy<N, RC>(s, rc, rs, row, gl4, row < rows);
    }
}

// ------------------------------------------------------------------------
// Reset listed sequences: zero checkpoint and copy, scale 1, pointer 0.
// Grid: (ids or B) x tiles workgroups.
// ------------------------------------------------------------------------
template <int RC>
__global__ __launch_bounds__(RSSM_THREADS) void rssm_reset_kernel(StepArgs A, int N) {
    const int n_ids = A.mode;
    const int i = blockIdx.x / A.tiles, tile = blockIdx.x % A.tiles;
    int b = i;
    if (A.seq_ids) {
        b = A.seq_ids[i];
        if (b < 0 || b >= A.B) {
            if (threadIdx.x == 0 && tile == 0) atomicOr(A.err, 1);
            return;
        }
    }
    (void)n_ids;
    const int rows = A.hvpt * A.P;
    const long seqhv = (long)b * A.Hv + tile * A.hvpt;
    f32x4* ck = reinterpret_cast<f32x4*>(A.ckpt + seqhv * A.P * N);
    const int n4 = rows * N / 4;
    for (int e = threadIdx.x; e < n4; e += RSSM_THREADS) ck[e] = f32x4{0.f, 0.f, 0.f, 0.f};
    if constexpr (RC != RC_NONE) {
        uint8_t* rc = reinterpret_cast<uint8_t*>(A.rcopy) + seqhv * A.P * N * Ck<RC>::ESZ;
        const int nb = rows * N * Ck<RC>::ESZ / 4;
        for (int e = threadIdx.x; e < nb; e += RSSM_THREADS) reinterpret_cast<uint32_t*>(rc)[e] = 0u;
    }
    if constexpr (RC == RC_FP8) {
        for (int e = threadIdx.x; e < rows; e += RSSM_THREADS) A.rscale[seqhv * A.P + e] = 1.0f;
    }
    if (threadIdx.x == 0) A.count[(long)b * A.tiles + tile] = 0;
}

}  // namespace rssm

// ------------------------------------------------------------------------
// Host-side launchers (template dispatch on key dim, input dtype, copy
// format and draft capacity).
// ------------------------------------------------------------------------
#include "rssm_launch.h"

namespace rssm {

#define RSSM_DISPATCH_N(N_, ...)                                      \
    switch (N_) {                                                     \
        case 16: { constexpr int NN = 16; __VA_ARGS__; } break;       \
        case 32: { constexpr int NN = 32; __VA_ARGS__; } break;       \
        case 64: { constexpr int NN = 64; __VA_ARGS__; } break;       \
        case 128: { constexpr int NN = 128; __VA_ARGS__; } break;     \
        case 256: { constexpr int NN = 256; __VA_ARGS__; } break;     \
        default: return hipErrorInvalidValue;                         \
    }
#define RSSM_DISPATCH_IN(I_, ...)                                     \
    switch (I_) {                                                     \
        case IN_F32: { constexpr int II = IN_F32; __VA_ARGS__; } break;   \
        case IN_BF16: { constexpr int II = IN_BF16; __VA_ARGS__; } break; \
        default: return hipErrorInvalidValue;                         \
    }
#define RSSM_DISPATCH_RC(R_, ...)                                     \
    switch (R_) {                                                     \
        case RC_NONE: { constexpr int RCC = RC_NONE; __VA_ARGS__; } break; \
        case RC_BF16: { constexpr int RCC = RC_BF16; __VA_ARGS__; } break; \
        case RC_FP8: { constexpr int RCC = RC_FP8; __VA_ARGS__; } break;   \
        default: return hipErrorInvalidValue;                         \
    }

hipError_t launch_decode(const StepArgs& A, int N, int in_dtype, int rc, int grid, size_t lds,
                         hipStream_t s) {
    RSSM_DISPATCH_N(N, RSSM_DISPATCH_IN(in_dtype, RSSM_DISPATCH_RC(rc,
        hipLaunchKernelGGL((rssm_decode_kernel<NN, II, RCC>), dim3(grid), dim3(RSSM_THREADS), lds, s, A))));
    return hipGetLastError();
}

hipError_t launch_fold(const StepArgs& A, int N, int in_dtype, int rc, int grid, size_t lds,
                       hipStream_t s) {
    RSSM_DISPATCH_N(N, RSSM_DISPATCH_IN(in_dtype, RSSM_DISPATCH_RC(rc,
        hipLaunchKernelGGL((rssm_fold_kernel<NN, II, RCC>), dim3(grid), dim3(RSSM_THREADS), lds, s, A))));
    return hipGetLastError();
}

hipError_t launch_verify(const StepArgs& A, int N, int in_dtype, int rc, int tt, int grid,
                         size_t lds, hipStream_t s) {
#define RSSM_V(TTV)                                                                            \
    RSSM_DISPATCH_N(N, RSSM_DISPATCH_IN(in_dtype, RSSM_DISPATCH_RC(rc,                         \
        hipLaunchKernelGGL((rssm_verify_kernel<NN, II, RCC, TTV>), dim3(grid), dim3(RSSM_THREADS), \
                           lds, s, A))))
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

hipError_t launch_refresh(const StepArgs& A, int N, int rc, int grid, hipStream_t s) {
    RSSM_DISPATCH_N(N, switch (rc) {
        case RC_BF16: hipLaunchKernelGGL((rssm_refresh_kernel<NN, RC_BF16>), dim3(grid), dim3(RSSM_THREADS), 0, s, A); break;
        case RC_FP8: hipLaunchKernelGGL((rssm_refresh_kernel<NN, RC_FP8>), dim3(grid), dim3(RSSM_THREADS), 0, s, A); break;
        default: return hipErrorInvalidValue;
    });
    return hipGetLastError();
}

hipError_t launch_reset(const StepArgs& A, int N, int rc, int grid, hipStream_t s) {
    RSSM_DISPATCH_RC(rc,
        hipLaunchKernelGGL((rssm_reset_kernel<RCC>), dim3(grid), dim3(RSSM_THREADS), 0, s, A, N));
    return hipGetLastError();
}

}  // namespace rssm
