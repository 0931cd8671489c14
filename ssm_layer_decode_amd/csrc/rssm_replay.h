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

__device__ __forceinline__ Ctx ctx_of(const StepArgs& A, int cidx) {
    Ctx c;
    c.cidx = cidx;
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

// The tile of a one-workgroup-per-tile launch.
__device__ __forceinline__ Ctx ctx_of(const StepArgs& A) { return ctx_of(A, blockIdx.x); }

// fp16 checkpoint: the stochastic-rounding key of the fold tile `cidx` is
// about to store (its epoch = the folds it stored before), and the epoch
// advance once the fold is written.  Every thread reads the same word; one
// writes it back after the stores.  Each tile's count is read and rewritten
// only by the workgroup that folds it, so no launch waits on another
// workgroup, and a launch replayed from a captured graph draws new numbers.
template <int CK>
__device__ __forceinline__ uint32_t fold_key(const StepArgs& A, int cidx) {
    if constexpr (CK != CK_F32) return sr_fold_key(A.sr_seed, A.folds[cidx]);
    else return 0u;
}
template <int CK>
__device__ __forceinline__ void fold_done(const StepArgs& A, int cidx) {
    if constexpr (CK != CK_F32) {
        if (threadIdx.x == 0) A.folds[cidx] += 1u;
    }
}

// Key group (within the tile) of local value head i.
__device__ __forceinline__ int kg_of_head(const StepArgs& A, int kgpt, int i) {
    return kgpt > 1 ? i / A.g : 0;
}

// ------------------------------------------------------------------------
// Staging into LDS.  A region is n items laid out contiguously in LDS: item e
// (4 consecutive input elements, or one fp32 decay) goes to dst + 4e (dst + e
// for decays), so each head's (or key group's) records sit back to back with
// stride nrec.  src(e, ao) returns the item's global address and sets ao to
// the byte offset from `abase` where the item is appended to the record
// buffer, or kNoApp.  A batch holds UNR items per thread: load() only issues
// global loads, store() writes LDS and the appends, so a kernel can issue the
// loads of all its regions (and its first state rows) before any of them is
// waited for -- the memory counter completes in order, so a store placed
// between loads would wait for every earlier load.  Items beyond
// UNR * RSSM_THREADS take further rounds (stage_rest).
// ------------------------------------------------------------------------
constexpr uint32_t kNoApp = 0xffffffffu;

template <class Src>
struct Region {
    int n;
    float* dst;
    char* abase;
    Src src;
};
template <class Src>
__device__ __forceinline__ Region<Src> region(int n, float* dst, char* abase, Src s) {
    return Region<Src>{n, dst, abase, s};
}

template <int IN, int UNR>
struct Batch4 {
    typename InVec4<IN>::Raw x[UNR];     // loaded bits, unpacked at the LDS store
    uint32_t ao[UNR];
    template <class R>
    __device__ __forceinline__ void load(const R& r, int first = 0) {
#pragma unroll
        for (int i = 0; i < UNR; ++i) {
            const int e = first + threadIdx.x + i * RSSM_THREADS;
            ao[i] = kNoApp;
            if (e < r.n) x[i] = InVec4<IN>::load_raw(r.src(e, ao[i]));
        }
    }
    template <class R>
    __device__ __forceinline__ void store(const R& r, int first = 0) const {
#pragma unroll
        for (int i = 0; i < UNR; ++i) {
            const int e = first + threadIdx.x + i * RSSM_THREADS;
            if (e < r.n) {
                *reinterpret_cast<f32x4*>(r.dst + 4 * e) = InVec4<IN>::unpack(x[i]);
                if (ao[i] != kNoApp) InVec4<IN>::store_raw(r.abase + ao[i], x[i]);
            }
        }
    }
};

template <int UNR>
struct BatchA {
    float x[UNR];
    uint32_t ao[UNR];
    template <class R>
    __device__ __forceinline__ void load(const R& r, int first = 0) {
#pragma unroll
        for (int i = 0; i < UNR; ++i) {
            const int e = first + threadIdx.x + i * RSSM_THREADS;
            ao[i] = kNoApp;
            if (e < r.n) x[i] = *reinterpret_cast<const float*>(r.src(e, ao[i]));
        }
    }
    template <class R>
    __device__ __forceinline__ void store(const R& r, int first = 0) const {
#pragma unroll
        for (int i = 0; i < UNR; ++i) {
            const int e = first + threadIdx.x + i * RSSM_THREADS;
            if (e < r.n) {
                r.dst[e] = x[i];
                if (ao[i] != kNoApp) *reinterpret_cast<float*>(r.abase + ao[i]) = x[i];
            }
        }
    }
};

// Remaining rounds of a region after its first UNR * RSSM_THREADS items.
template <int IN, int UNR, class R>
__device__ __forceinline__ void stage_rest(const R& r) {
    for (int first = UNR * RSSM_THREADS; first < r.n; first += UNR * RSSM_THREADS) {
        Batch4<IN, UNR> b;
        b.load(r, first);
        b.store(r, first);
    }
}
template <int UNR, class R>
__device__ __forceinline__ void stage_rest_a(const R& r) {
    for (int first = UNR * RSSM_THREADS; first < r.n; first += UNR * RSSM_THREADS) {
        BatchA<UNR> b;
        b.load(r, first);
        b.store(r, first);
    }
}

// Query slices of the tile's key groups for T queries: LDS q_l[kg][T][N];
// q is [B][T][Hk][N] (decode: T = 1).
template <int N, int IN>
__device__ __forceinline__ auto q_region(const StepArgs& A, const Ctx& c, float* q_l, int T) {
    constexpr int R4 = N / 4, ESZ = InVec4<IN>::ESZ;
    const int per = T * R4, Hk = A.Hk;
    const char* qt = reinterpret_cast<const char*>(A.q) + ((long)c.b * T * Hk + c.kh0) * N * ESZ;
    return region(c.kgpt * per, q_l, nullptr, [=](int e, uint32_t&) {
        const int kg = (T == 1) ? e / R4 : e / per;
        const int r = e - kg * per, t = r / R4, c4 = r - t * R4;
        return qt + (uint32_t)(((t * Hk + kg) * N + c4 * 4) * ESZ);
    });
}

// Key records j < nrec of the tile's key groups: LDS k_l[kg][nrec][N].
// Records below h_buf come from the buffer [B][Hk][C][N]; later ones from the
// step's inputs k[B][T][Hk][N] (record j - h_buf), appended to the buffer when
// `append` and this tile owns the key group.
template <int N, int IN, bool WITH_INPUT>
__device__ __forceinline__ auto k_region(const StepArgs& A, const Ctx& c, float* k_l, int nrec, int h_buf,
                                         int T, bool append) {
    constexpr int R4 = N / 4, ESZ = InVec4<IN>::ESZ;
    const int per = nrec * R4, C = A.C, Hk = A.Hk, hb4 = h_buf * R4;
    char* kbt = reinterpret_cast<char*>(A.kbuf) + ((long)c.b * Hk + c.kh0) * C * N * ESZ;
    const char* kin = reinterpret_cast<const char*>(A.k) + ((long)c.b * T * Hk + c.kh0) * N * ESZ;
    const bool app = append && c.kwriter;
    return region(c.kgpt * per, k_l, kbt, [=](int e, uint32_t& ao) -> const char* {
        const int kg = e / per, ep = e - kg * per;
        const uint32_t boff = (uint32_t)((kg * C * N + ep * 4) * ESZ);
        if (!WITH_INPUT || ep < hb4) return kbt + boff;
        const int r = ep - hb4, t = r / R4, c4 = r - t * R4;
        if (app) ao = boff;
        return kin + (uint32_t)(((t * Hk + kg) * N + c4 * 4) * ESZ);
    });
}

// Value records j < nrec: LDS v_l[vh][nrec][P]; buffer [B][Hv][C][P], inputs
// v[B][T][Hv][P].
template <int IN, bool WITH_INPUT>
__device__ __forceinline__ auto v_region(const StepArgs& A, const Ctx& c, float* v_l, int nrec, int h_buf,
                                         int T, bool append) {
    constexpr int ESZ = InVec4<IN>::ESZ;
    const int P = A.P, P4 = P / 4, per = nrec * P4, C = A.C, Hv = A.Hv, hb4 = h_buf * P4;
    char* vbt = reinterpret_cast<char*>(A.vbuf) + c.seqhv * C * P * ESZ;
    const char* vin = reinterpret_cast<const char*>(A.v) + ((long)c.b * T * Hv + c.vh0) * P * ESZ;
    return region(A.hvpt * per, v_l, vbt, [=](int e, uint32_t& ao) -> const char* {
        const int vh = e / per, ep = e - vh * per;
        const uint32_t boff = (uint32_t)((vh * C * P + ep * 4) * ESZ);
        if (!WITH_INPUT || ep < hb4) return vbt + boff;
        const int r = ep - hb4, t = (T == 1) ? 0 : r / P4, p4 = r - t * P4;
        if (append) ao = boff;
        return vin + (uint32_t)(((t * Hv + vh) * P + p4 * 4) * ESZ);
    });
}

// Decays j < nrec: LDS a_l[vh][nrec]; buffer [B][Hv][C], inputs alpha[B][T][Hv].
template <bool WITH_INPUT>
__device__ __forceinline__ auto a_region(const StepArgs& A, const Ctx& c, float* a_l, int nrec, int h_buf,
                                         int T, bool append) {
    const int C = A.C, Hv = A.Hv;
    char* abt = reinterpret_cast<char*>(A.abuf) + c.seqhv * C * 4;
    const char* ain = reinterpret_cast<const char*>(A.alpha) + ((long)c.b * T * Hv + c.vh0) * 4;
    return region(A.hvpt * nrec, a_l, abt, [=](int e, uint32_t& ao) -> const char* {
        const int vh = e / nrec, j = e - vh * nrec;
        const uint32_t boff = (uint32_t)((vh * C + j) * 4);
        if (!WITH_INPUT || j < h_buf) return abt + boff;
        if (append) ao = boff;
        return ain + (uint32_t)(((j - h_buf) * Hv + vh) * 4);
    });
}

// Stage q, keys, values and decays of a tile with all first-round loads
// issued together (UQ, UK, UV items of 4 per thread; one decay per thread).
template <int IN, int UQ, int UK, int UV, class RQ, class RK, class RV, class RA>
__device__ __forceinline__ void stage_qkva(const RQ& rq, const RK& rk, const RV& rv, const RA& ra) {
    Batch4<IN, UQ> bq;
    Batch4<IN, UK> bk;
    Batch4<IN, UV> bv;
    BatchA<1> ba;
    bq.load(rq);
    bk.load(rk);
    bv.load(rv);
    ba.load(ra);
    bq.store(rq);
    bk.store(rk);
    bv.store(rv);
    ba.store(ra);
    stage_rest<IN, UQ>(rq);
    stage_rest<IN, UK>(rk);
    stage_rest<IN, UV>(rv);
    stage_rest_a<1>(ra);
}

// Keys, values and decays (folds, which need no query).
template <int IN, int UK, int UV, class RK, class RV, class RA>
__device__ __forceinline__ void stage_kva(const RK& rk, const RV& rv, const RA& ra) {
    Batch4<IN, UK> bk;
    Batch4<IN, UV> bv;
    BatchA<1> ba;
    bk.load(rk);
    bv.load(rv);
    ba.load(ra);
    bk.store(rk);
    bv.store(rv);
    ba.store(ra);
    stage_rest<IN, UK>(rk);
    stage_rest<IN, UV>(rv);
    stage_rest_a<1>(ra);
}

// Values and decays only (tiles whose scores come straight from key loads).
template <int IN, int UV, class RV, class RA>
__device__ __forceinline__ void stage_va(const RV& rv, const RA& ra) {
    Batch4<IN, UV> bv;
    BatchA<1> ba;
    bv.load(rv);
    ba.load(ra);
    bv.store(rv);
    ba.store(ra);
    stage_rest<IN, UV>(rv);
    stage_rest_a<1>(ra);
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
// in fp32.  Chunk 0 of the checkpoint rows (format CK) is already loaded in
// S0.  Writes the checkpoint (fp16: stochastically rounded with the fold's
// key sr_key) and the read copy, both from the fp32 result; with OUT also writes
// y[row] = S_new[row] . q_{kg(row)}.  MULTI: the tile spans several key
// groups (each row picks its group's keys).
template <int N, int RC, int UF, bool OUT, bool MULTI, int CK>
__device__ __forceinline__ void fold_rows(u32x4 (&S0)[UF], char* ck_tile, void* rcopy_tile,
                                          void* rscale_tile, const StepArgs& A, const Ctx& c, int LV,
                                          int LK, int nrec, const float* k_l, const float* w_l,
                                          const float* G_l, const float* q_l, float* y, uint32_t sr_key) {
    constexpr int R4 = N / 4, RPP4 = RSSM_THREADS / R4;
    const int tid = threadIdx.x, rg = tid / R4, gl = tid % R4;
    const int rows = c.rows, P = A.P;
    const int nchunks = (rows + UF * RPP4 - 1) / (UF * RPP4);
    const long g_tile = c.seqhv * P * N;          // flat index of the tile's first entry
    for (int ch = 0; ch < nchunks; ++ch) {
        if (ch > 0) load_ck_rows<N, CK, UF>(S0, ck_tile, ch, rows, rg, gl);
        f32x4 S[UF];
        int woff[UF], kgu[UF];
#pragma unroll
        for (int u = 0; u < UF; ++u) {
            const int row = (ch * UF + u) * RPP4 + rg;
            const int r = row < rows ? row : 0;
            const int vh = r / P;
            woff[u] = vh * LV * P + (r - vh * P);
            kgu[u] = MULTI ? kg_of_head(A, c.kgpt, vh) : 0;
            S[u] = ck_values<CK>(S0[u]) * G_l[vh];
        }
        // Rows of one chunk usually share a key group (a head's P rows span
        // whole chunks); then each record's key slice is read from LDS once
        // for all UF rows, else once per row.  The test is uniform over the
        // workgroup (it depends on the chunk only).
        const int r_first = ch * UF * RPP4, r_last = min(rows, (ch + 1) * UF * RPP4) - 1;
        const int kg_chunk = MULTI ? kg_of_head(A, c.kgpt, r_first / P) : 0;
        const bool one_group = !MULTI || kg_chunk == kg_of_head(A, c.kgpt, r_last / P);
        if (one_group) {
            const float* kbase = k_l + kg_chunk * LK * N + gl * 4;
#pragma unroll 1
            for (int j = 0; j < nrec; ++j) {
                const f32x4 kj = *reinterpret_cast<const f32x4*>(kbase + j * N);
#pragma unroll
                for (int u = 0; u < UF; ++u) {
                    const float wv = w_l[woff[u] + j * P];
                    S[u].x = fmaf(wv, kj.x, S[u].x);
                    S[u].y = fmaf(wv, kj.y, S[u].y);
                    S[u].z = fmaf(wv, kj.z, S[u].z);
                    S[u].w = fmaf(wv, kj.w, S[u].w);
                }
            }
        } else {
            // a group boundary inside the chunk: one record loop per row
#pragma unroll
            for (int u = 0; u < UF; ++u) {
                const float* kbase = k_l + kgu[u] * LK * N + gl * 4;
#pragma unroll 1
                for (int j = 0; j < nrec; ++j) {
                    const f32x4 kj = *reinterpret_cast<const f32x4*>(kbase + j * N);
                    const float wv = w_l[woff[u] + j * P];
                    S[u].x = fmaf(wv, kj.x, S[u].x);
                    S[u].y = fmaf(wv, kj.y, S[u].y);
                    S[u].z = fmaf(wv, kj.z, S[u].z);
                    S[u].w = fmaf(wv, kj.w, S[u].w);
                }
            }
        }
        float part[UF];
#pragma unroll
        for (int u = 0; u < UF; ++u) {
            const int row = (ch * UF + u) * RPP4 + rg;
            const float sig = ck_row_scale<N, CK>(S[u]);        // every lane of the row group
            if (row < rows) store_ck4<N, CK>(ck_tile, row, gl, S[u], sr_key, g_tile + (long)row * N + gl * 4, sig);
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

// LDS layout of decode and fold (floats; regions sized for L records, LS = L
// rounded to 4; the staged records use stride nrec <= L):
//   q [kgpt][N] | k [kgpt][nrec][N] | v [hvpt][nrec][P] | a [hvpt][nrec] | s [kgpt][LS] | y [rows4] | G [hvpt]
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
