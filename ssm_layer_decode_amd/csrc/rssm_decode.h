// rssm_decode.h -- the flush step of a decode launch, shared by the decode
// kernels: on the step whose append fills the window ([ru] §03 flush step;
// [ar] "how ReplaySSM works") the tile folds its L records into the
// checkpoint,
//     S_ckpt <- g_{1:L} S_ckpt + sum_j g_{j+1:L} v_j k_j^T,
// writes it (and its read copy) once, outputs S_new q from the fp32 fold and
// empties its buffer.  The current record is read from the step's inputs (it
// is never appended: the buffer empties).
#pragma once
#include "rssm_replay.h"

namespace rssm {

// The fold of the heads of c with the stochastic-rounding key `key`: stage
// their records, fold, store the checkpoint (and copy), output S_new q.
// UF: checkpoint rows per thread in flight during the fold.
template <int N, int IN, int RC, bool MULTI, int CK, int UF>
__device__ __forceinline__ void flush_fold(const StepArgs& A, const Ctx& c, float* lds, int h, uint32_t key) {
    constexpr int R4 = N / 4;
    const int tid = threadIdx.x, P = A.P, L = A.L, nrec = h + 1;
    char* ck_tile = reinterpret_cast<char*>(A.ckpt) + c.seqhv * P * ck_row_bytes(CK, N);
    const Lds d = carve(lds, N, L, c.kgpt, A.hvpt, P);
    u32x4 S0[UF];
    load_ck_rows<N, CK, UF>(S0, ck_tile, 0, c.rows, tid / R4, tid % R4);
    stage_qkva<IN, 1, 4, 2>(q_region<N, IN>(A, c, d.q, 1),
                            k_region<N, IN, true>(A, c, d.k, nrec, h, 1, false),
                            v_region<IN, true>(A, c, d.v, nrec, h, 1, false),
                            a_region<true>(A, c, d.a, nrec, h, 1, false));
    lds_barrier();
    make_weights(d.v, d.a, d.G, A.hvpt, P, nrec, nrec, nrec);
    lds_barrier();
    void* rc_tile = (RC == RC_NONE) ? nullptr
        : reinterpret_cast<char*>(A.rcopy) + c.seqhv * P * copy_row_bytes(RC, N);
    void* rs_tile = reinterpret_cast<char*>(A.rscale) + c.seqhv * P * scale_row_bytes(RC, N);
    fold_rows<N, RC, UF, true, MULTI, CK>(S0, ck_tile, rc_tile, rs_tile, A, c, nrec, nrec, nrec, d.k, d.v, d.G, d.q,
                                          d.y, key);
    lds_barrier();
    for (int row = tid; row < c.rows; row += RSSM_THREADS) A.o[c.seqhv * P + row] = d.y[row];
}

// The flush of the whole tile at once (shared memory for the tile's records).
template <int N, int IN, int RC, bool MULTI, int CK, int UF = 4>
__device__ __forceinline__ void decode_flush(const StepArgs& A, const Ctx& c, float* lds, int h) {
    flush_fold<N, IN, RC, MULTI, CK, UF>(A, c, lds, h, fold_key<CK>(A, c.cidx));
    if (threadIdx.x == 0) A.count[c.cidx] = 0;
    fold_done<CK>(A, c.cidx);
}

// The same flush one value head at a time for tiles of HV (1 or 2) heads, so
// the shared memory holds one head's records only (a launch sized for that
// keeps more workgroups resident).  Every head rounds with the tile's key; a
// head's staging starts after the previous head's fold has passed its last
// barrier, and the previous head's outputs are read from y before the next
// fold writes y (behind the next head's first barrier).  The heads are two
// calls, not a loop: in a loop the compiler keeps the body's address
// arithmetic live across iterations (about 40 more VGPRs).
template <int N, int IN, int RC, int CK, int UF, int HV>
__device__ __forceinline__ void decode_flush_by_head(const StepArgs& A, const Ctx& c, float* lds, int h) {
    static_assert(HV == 1 || HV == 2, "tiles of one or two heads");
    StepArgs A1 = A;
    A1.hvpt = 1;
    const uint32_t key = fold_key<CK>(A, c.cidx);
    auto head = [&](int i) {
        Ctx ci = c;
        ci.vh0 = c.vh0 + i;
        ci.kh0 = ci.vh0 / A.g;
        ci.kgpt = 1;
        ci.rows = A.P;
        ci.seqhv = c.seqhv + i;
        ci.kwriter = (ci.vh0 % A.g) == 0;
        flush_fold<N, IN, RC, false, CK, UF>(A1, ci, lds, h, key);
    };
    head(0);
    if constexpr (HV == 2) head(1);
    if (threadIdx.x == 0) A.count[c.cidx] = 0;
    fold_done<CK>(A, c.cidx);
}

}  // namespace rssm
