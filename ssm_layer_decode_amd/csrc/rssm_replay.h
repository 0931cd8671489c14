// rssm_replay.h -- device building blocks of the ReplaySSM kernels: tile
// context, LDS staging of records and queries, scores, checkpoint matvecs and
// the fold.  See rssm_kernels.hip for the method and the work decomposition.
#pragma once
#include "rssm_stream.h"

namespace rssm {

// ------------------------------------------------------------------------
// Tile context
// ------------------------------------------------------------------------
struct Ctx {
    int b, vh0, kh0, kgpt, rows, cidx;
    long seqhv;          // b * Hv + vh0
    bool kwriter;        // stores the key records of its key group(s)
};

__device__ __forceinline__ Ctx ctx_of(const StepArgs& A) {
    Ctx c;
    c.cidx = blockIdx.x;
    c.b = c.cidx / A.tiles;
    const int tile = c.cidx - c.b * A.tiles;
    c.vh0 = tile * A.hvpt;
    c.kh0 = c.vh0 / A.g;
    c.kgpt = A.hvpt >= A.g ? A.hvpt / A.g : 1;
    c.rows = A.hvpt * A.P;
    c.seqhv = (long)c.b * A.Hv + c.vh0;
    c.kwriter = (c.vh0 % A.g) == 0;
    return c;
}

// Key group (within the tile) of local value head i.
__device__ __forceinline__ int kg_of_head(const StepArgs& A, int kgpt, int i) {
    return kgpt > 1 ? i / A.g : 0;
}

// ------------------------------------------------------------------------
// Staging into LDS.  Items are groups of 4 consecutive input elements; up to
// UNR loads per thread are issued before their LDS stores.
// ------------------------------------------------------------------------
template <int IN, int UNR, class Src, class Dst>
__device__ __forceinline__ void stage4(int n, Src src, Dst dst) {
    for (int base = threadIdx.x; base < n; base += UNR * RSSM_THREADS) {
        float x[UNR][4];
#pragma unroll
        for (int i = 0; i < UNR; ++i) {
            const int e = base + i * RSSM_THREADS;
            if (e < n) {
                const void* p;
                long idx;
                src(e, p, idx);
                InVec4<IN>::load(p, idx, x[i]);
            }
        }
#pragma unroll
        for (int i = 0; i < UNR; ++i) {
            const int e = base + i * RSSM_THREADS;
            if (e < n) *reinterpret_cast<f32x4*>(dst(e)) = f32x4{x[i][0], x[i][1], x[i][2], x[i][3]};
        }
    }
}

// Query slices q_l[kg][t][N] (t stride TS) of the tile's key groups for T
// queries; q is [B][T][Hk][N] (decode: T = 1).
template <int N, int IN>
__device__ __forceinline__ void stage_q(const StepArgs& A, const Ctx& c, float* q_l, int T, int TS) {
    constexpr int R4 = N / 4;
    const int per = T * R4;
    stage4<IN, 1>(c.kgpt * per,
        [&](int e, const void*& p, long& idx) {
            const int kg = e / per, r = e - kg * per, t = r / R4, c4 = r - t * R4;
            p = A.q;
            idx = (((long)c.b * T + t) * A.Hk + c.kh0 + kg) * N + c4 * 4;
        },
        [&](int e) {
            const int kg = e / per, r = e - kg * per, t = r / R4, c4 = r - t * R4;
            return q_l + (kg * TS + t) * N + c4 * 4;
        });
}

// Key records j < nrec of the tile's key groups into k_l[kg][LK][N]: slots below
// h_buf from the buffer, later ones from the step's inputs k[B][T][Hk][N]
// (record j - h_buf), appended raw to the buffer when `append` and this tile
// owns the key group.
template <int N, int IN, bool WITH_INPUT>
__device__ __forceinline__ void stage_k(const StepArgs& A, const Ctx& c, float* k_l, int LK, int nrec,
                                        int h_buf, int T, bool append) {
    constexpr int R4 = N / 4;
    const int per = nrec * R4;
    stage4<IN, 2>(c.kgpt * per,
        [&](int e, const void*& p, long& idx) {
            const int kg = e / per, r = e - kg * per, j = r / R4, c4 = r - j * R4;
            const long kh = c.kh0 + kg;
            const long bidx = (((long)c.b * A.Hk + kh) * A.C + j) * N + c4 * 4;
            if (!WITH_INPUT || j < h_buf) {
                p = A.kbuf;
                idx = bidx;
            } else {
                p = A.k;
                idx = (((long)c.b * T + (j - h_buf)) * A.Hk + kh) * N + c4 * 4;
                if (append && c.kwriter) copy_vec4<IN>(A.kbuf, bidx, A.k, idx);
            }
        },
        [&](int e) {
            const int kg = e / per, r = e - kg * per, j = r / R4, c4 = r - j * R4;
            return k_l + (kg * LK + j) * N + c4 * 4;
        });
}

// Value records j < nrec into v_l[vh][LV][P]; inputs v[B][T][Hv][P].
template <int IN, bool WITH_INPUT>
__device__ __forceinline__ void stage_v(const StepArgs& A, const Ctx& c, float* v_l, int LV, int nrec,
                                        int h_buf, int T, bool append) {
    const int P = A.P, P4 = P / 4, per = nrec * P4;
    stage4<IN, 2>(A.hvpt * per,
        [&](int e, const void*& p, long& idx) {
            const int vh = e / per, r = e - vh * per, j = r / P4, p4 = r - j * P4;
            const long bidx = ((c.seqhv + vh) * A.C + j) * P + p4 * 4;
            if (!WITH_INPUT || j < h_buf) {
                p = A.vbuf;
                idx = bidx;
            } else {
                p = A.v;
                idx = (((long)c.b * T + (j - h_buf)) * A.Hv + c.vh0 + vh) * P + p4 * 4;
                if (append) copy_vec4<IN>(A.vbuf, bidx, A.v, idx);
            }
        },
        [&](int e) {
            const int vh = e / per, r = e - vh * per, j = r / P4, p4 = r - j * P4;
            return v_l + (vh * LV + j) * P + p4 * 4;
        });
}

// Decays j < nrec into a_l[vh][AS]; inputs alpha[B][T][Hv].
template <bool WITH_INPUT>
__device__ __forceinline__ void stage_a(const StepArgs& A, const Ctx& c, float* a_l, int AS, int nrec,
                                        int h_buf, int T, bool append) {
    const int total = A.hvpt * nrec;
    for (int e = threadIdx.x; e < total; e += RSSM_THREADS) {
        const int vh = e / nrec, j = e - vh * nrec;
        const long arow = c.seqhv + vh;
        float a;
        if (!WITH_INPUT || j < h_buf) {
            a = A.abuf[arow * A.C + j];
        } else {
            a = A.alpha[((long)c.b * T + (j - h_buf)) * A.Hv + c.vh0 + vh];
            if (append) A.abuf[arow * A.C + j] = a;
        }
        a_l[vh * AS + j] = a;
    }
}

// w[vh][j][p] <- g_{j+1:nrec} v[vh][j][p] in place, and G[vh] = g_{1:nrec}.
__device__ __forceinline__ void make_weights(float* v_l, const float* a_l, float* G_l, int hvpt, int P,
                                             int LV, int AS, int nrec) {
    for (int row = threadIdx.x; row < hvpt * P; row += RSSM_THREADS) {
        const int vh = row / P, p = row - vh * P;
        float c = 1.0f;
        for (int j = nrec - 1; j >= 0; --j) {
            float* wp = v_l + (vh * LV + j) * P + p;
            *wp = c * *wp;
            c *= a_l[vh * AS + j];
        }
        if (p == 0) G_l[vh] = c;
    }
}

// Scores s[kg][j][t] = k_j . q_t for the tile's key groups, from LDS.  Row
// groups of R4 lanes take one record each; the TT query partials are reduced
// together.  Layout: s_l[(kg * LS + j) * TT + t].
template <int N, int TT>
__device__ __forceinline__ void scores_from_lds(const float* k_l, int LK, const float* q_l, int TS,
                                                float* s_l, int LS, int kgpt, int nrec, int T) {
    constexpr int R4 = N / 4, RPP4 = RSSM_THREADS / R4;
    const int tid = threadIdx.x, rg = tid / R4, gl = tid % R4;
    const int total = kgpt * nrec;
    for (int j0 = 0; j0 < total; j0 += RPP4) {              // uniform trip count
        const int jj = j0 + rg;
        const int kg = jj < total ? jj / nrec : 0;
        const int j = jj < total ? jj - kg * nrec : 0;
        const f32x4 kv = *reinterpret_cast<const f32x4*>(k_l + (kg * LK + j) * N + gl * 4);
        float sp[TT];
#pragma unroll
        for (int t = 0; t < TT; ++t) {
            const f32x4 qv = *reinterpret_cast<const f32x4*>(q_l + (kg * TS + t) * N + gl * 4);
            sp[t] = kv.x * qv.x + kv.y * qv.y + kv.z * qv.z + kv.w * qv.w;
        }
        group_transpose_reduce<TT, R4>(sp, gl);
        if (jj < total) {
            if constexpr (TT >= R4) {
#pragma unroll
                for (int i = 0; i < TT / R4; ++i) {
                    const int t = gl * (TT / R4) + i;
                    if (t < T) s_l[(kg * LS + j) * TT + t] = sp[i];
                }
            } else {
                if (gl % (R4 / TT) == 0) {
                    const int t = gl / (R4 / TT);
                    if (t < T) s_l[(kg * LS + j) * TT + t] = sp[0];
                }
            }
        }
    }
}

// y[t * ys + row] = sum_n M[row][n] q_t[n] for all rows of the tile (M in read
// format RC), the q slice of each row's key group read from LDS.  Chunk 0 is
// already loaded in w (and its MXFP4 block exponents in ex); the next chunk is
// prefetched while one is reduced.  scale_tile: fp32 row scales (fp8) or E8M0
// block exponents (MXFP4) of the tile.
template <int N, int RC, int U, int TT>
__device__ __forceinline__ void matvec_rows(u32x4 (&w)[U], int (&ex)[U], const char* base, const StepArgs& A,
                                            const Ctx& c, const float* q_l, int TS, float* y, int ys,
                                            const void* scale_tile) {
    constexpr int EPL = Ck<RC>::EPL, R = N / EPL, RPP = RSSM_THREADS / R;
    const int tid = threadIdx.x, rg = tid / R, gl = tid % R;
    const int rows = c.rows, P = A.P;
    const int nchunks = (rows + U * RPP - 1) / (U * RPP);
    for (int ch = 0; ch < nchunks; ++ch) {
        u32x4 nx[U];
        int nex[U];
        const bool more = (ch + 1 < nchunks);
        if (more) {
            load_rows<N, RC, U>(nx, base, ch + 1, rows, rg, gl);
            load_block_exp<N, RC, U>(nex, reinterpret_cast<const uint8_t*>(scale_tile), ch + 1, rows, rg, gl);
        }
        float part[U * TT];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int row = (ch * U + u) * RPP + rg;
            const int kg = kg_of_head(A, c.kgpt, (row < rows ? row : 0) / P);
            float x[EPL];
            Ck<RC>::decode(w[u], x);
#pragma unroll
            for (int t = 0; t < TT; ++t) {
                const float* qp = q_l + (kg * TS + t) * N + gl * EPL;
                float s = 0.f;
#pragma unroll
                for (int i = 0; i < EPL; i += 4) {
                    const f32x4 qv = *reinterpret_cast<const f32x4*>(qp + i);
                    s = fmaf(x[i], qv.x, s);
                    s = fmaf(x[i + 1], qv.y, s);
                    s = fmaf(x[i + 2], qv.z, s);
                    s = fmaf(x[i + 3], qv.w, s);
                }
                part[u * TT + t] = block_scaled<RC>(s, ex[u]);
            }
        }
        constexpr int UT = U * TT;
        group_transpose_reduce<UT, R>(part, gl);
        auto put = [&](int idx, float val) {
            const int u = idx / TT, t = idx - u * TT;
            const int row = (ch * U + u) * RPP + rg;
            if (row < rows) {
                if constexpr (RC == RC_FP8) val *= reinterpret_cast<const float*>(scale_tile)[row];
                y[t * ys + row] = val;
            }
        };
        if constexpr (UT >= R) {
#pragma unroll
            for (int i = 0; i < UT / R; ++i) put(gl * (UT / R) + i, part[i]);
        } else {
            if (gl % (R / UT) == 0) put(gl / (R / UT), part[0]);
        }
        if (more) {
#pragma unroll
            for (int u = 0; u < U; ++u) {
                w[u] = nx[u];
                if constexpr (RC == RC_MXFP4) ex[u] = nex[u];
            }
        }
    }
}

// Fold the nrec records staged in LDS into the tile's checkpoint:
//   S <- G[vh] S + sum_j w[vh][j][p] k_{kg(vh), j}     (w = g_{j+1:h} v_j)
// Chunk 0 of the fp32 rows is already loaded in S0.  Writes the checkpoint (and
// the read copy); with OUT also writes y[row] = S_new[row] . q_{kg(row)}.
// MULTI: the tile spans several key groups (each row picks its group's keys).
template <int N, int RC, int UF, bool OUT, bool MULTI>
__device__ __forceinline__ void fold_rows(u32x4 (&S0)[UF], float* ck_tile, void* rcopy_tile,
                                          void* rscale_tile, const StepArgs& A, const Ctx& c, int LV,
                                          int LK, int nrec, const float* k_l, const float* w_l,
                                          const float* G_l, const float* q_l, float* y) {
    constexpr int R4 = N / 4, RPP4 = RSSM_THREADS / R4;
    const int tid = threadIdx.x, rg = tid / R4, gl = tid % R4;
    const int rows = c.rows, P = A.P;
    const int nchunks = (rows + UF * RPP4 - 1) / (UF * RPP4);
    const char* base = reinterpret_cast<const char*>(ck_tile);
    for (int ch = 0; ch < nchunks; ++ch) {
        if (ch > 0) load_rows<N, RC_NONE, UF>(S0, base, ch, rows, rg, gl);
        f32x4 S[UF];
        int woff[UF], kgu[UF];
#pragma unroll
        for (int u = 0; u < UF; ++u) {
            const int row = (ch * UF + u) * RPP4 + rg;
            const int r = row < rows ? row : 0;
            const int vh = r / P;
            woff[u] = vh * LV * P + (r - vh * P);
            kgu[u] = MULTI ? kg_of_head(A, c.kgpt, vh) : 0;
            S[u] = f32x4{__uint_as_float(S0[u].x), __uint_as_float(S0[u].y),
                         __uint_as_float(S0[u].z), __uint_as_float(S0[u].w)} * G_l[vh];
        }
#pragma unroll 1
        for (int j = 0; j < nrec; ++j) {
            const f32x4 kj0 = *reinterpret_cast<const f32x4*>(k_l + j * N + gl * 4);
#pragma unroll
            for (int u = 0; u < UF; ++u) {
                const f32x4 kj = MULTI ? *reinterpret_cast<const f32x4*>(k_l + (kgu[u] * LK + j) * N + gl * 4) : kj0;
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
            const int row = (ch * UF + u) * RPP4 + rg;
            if (row < rows) {
                st16(reinterpret_cast<char*>(ck_tile) + (long)row * N * 4 + gl * 16,
                     u32x4{__float_as_uint(S[u].x), __float_as_uint(S[u].y),
                           __float_as_uint(S[u].z), __float_as_uint(S[u].w)});
            }
            if constexpr (RC != RC_NONE) store_copy<N, RC>(S[u], rcopy_tile, rscale_tile, row, gl, row < rows);
            if constexpr (OUT) {
                const f32x4 qv = *reinterpret_cast<const f32x4*>(q_l + kgu[u] * N + gl * 4);
                part[u] = S[u].x * qv.x + S[u].y * qv.y + S[u].z * qv.z + S[u].w * qv.w;
            }
        }
        if constexpr (OUT) {
            group_transpose_reduce<UF, R4>(part, gl);
            put_rows<N, RC_NONE, UF>(part, y, ch, rows, rg, gl, nullptr);
        }
    }
}

// y[row] = sum_n M[row][n] q[n] for all rows of a tile inside one key group,
// the lane's q slice held in registers; chunk 0 already loaded in w (and its
// MXFP4 block exponents in ex).  scale_tile as for matvec_rows.
template <int N, int RC, int U>
__device__ __forceinline__ void matvec_tile(u32x4 (&w)[U], int (&ex)[U], const char* base, int rows,
                                            const float (&qs)[Ck<RC>::EPL], float* y,
                                            const void* scale_tile) {
    constexpr int EPL = Ck<RC>::EPL;
    constexpr int R = N / EPL;
    constexpr int RPP = RSSM_THREADS / R;
    const int tid = threadIdx.x, rg = tid / R, gl = tid % R;
    const int nchunks = (rows + U * RPP - 1) / (U * RPP);
    for (int c = 0; c < nchunks; ++c) {
        u32x4 nx[U];
        int nex[U];
        const bool more = (c + 1 < nchunks);
        if (more) {
            load_rows<N, RC, U>(nx, base, c + 1, rows, rg, gl);
            load_block_exp<N, RC, U>(nex, reinterpret_cast<const uint8_t*>(scale_tile), c + 1, rows, rg, gl);
        }
        float part[U];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            float x[EPL];
            Ck<RC>::decode(w[u], x);
            float s = 0.f;
#pragma unroll
            for (int i = 0; i < EPL; ++i) s = fmaf(x[i], qs[i], s);
            part[u] = block_scaled<RC>(s, ex[u]);
        }
        group_transpose_reduce<U, R>(part, gl);
        put_rows<N, RC, U>(part, y, c, rows, rg, gl, reinterpret_cast<const float*>(scale_tile));
        if (more) {
#pragma unroll
            for (int u = 0; u < U; ++u) {
                w[u] = nx[u];
                if constexpr (RC == RC_MXFP4) ex[u] = nex[u];
            }
        }
    }
}

// LDS layout of decode and fold (floats; L = record stride, LS = L rounded to 4):
//   q [kgpt][N] | k [kgpt][L][N] | v [hvpt][L][P] | a [hvpt][LS] | s [kgpt][LS] | y [rows4] | G [hvpt]
struct Lds {
    float *q, *k, *v, *a, *s, *y, *G;
};
__device__ __forceinline__ Lds carve(float* lds, int N, int L, int kgpt, int hvpt, int P) {
    const int LS = (L + 3) & ~3;
    Lds d;
    d.q = lds;
    d.k = d.q + kgpt * N;
    d.v = d.k + kgpt * L * N;
    d.a = d.v + hvpt * L * P;
    d.s = d.a + hvpt * LS;
    d.y = d.s + kgpt * LS;
    d.G = d.y + ((hvpt * P + 3) & ~3);
    return d;
}

}  // namespace rssm
