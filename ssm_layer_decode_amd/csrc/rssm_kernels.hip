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
// Decode, flush, refresh and reset: one 256-thread workgroup per (sequence,
// tile).  Commit: one thread per tile advances the pointers and lists the
// tiles that fold, then a fixed grid of workgroups folds the listed tiles.  A
// tile is `hvpt` consecutive value heads: either part of one key group (hvpt
// divides the group size g) or `kgpt` whole key groups (hvpt = kgpt * g).
// Records, queries and scores live in LDS; a key group's scores are computed
// once and shared by its value heads.  The checkpoint streams through
// registers in 16-byte loads issued before the record staging, so they are in
// flight while the small work runs.  The per-tile copy count[b][tile] of the
// record pointer is read and rewritten by the one workgroup (or thread) that
// owns the tile in a launch, so no kernel waits on another workgroup.
#include "replayssm.h"
#include "rssm_decode.h"

namespace rssm {

// ------------------------------------------------------------------------
// Decode step: append + replay output, or fold on the step that fills the
// window ([ru] §03 non-flush and flush steps; [ar] "how ReplaySSM works").
// ------------------------------------------------------------------------
template <int N, int IN, int RC, bool MULTI, int CK>
__global__ __launch_bounds__(RSSM_THREADS) void rssm_decode_kernel(StepArgs A) {
    extern __shared__ __attribute__((aligned(16))) float lds[];
    // non-flush steps read the copy, or without one the checkpoint in its own format
    constexpr int RD = (RC == RC_NONE) ? ck_read_format(CK) : RC;
    constexpr int R4 = N / 4;
    constexpr int EPL = Ck<RD>::EPL, RR = N / EPL;
    constexpr int UM = ReadU<RD>::U, UF = 4;

    const int tid = threadIdx.x;
    const Ctx c = ctx_of(A);
    const int h = A.count[c.cidx];
    if (h < 0 || h >= A.L) {
        if (tid == 0) atomicOr(A.err, 1);
        return;
    }
    const int P = A.P, L = A.L, LS = (L + 3) & ~3;
    const int nrec = h + 1;
    const bool flush = (nrec == L);
    char* ck_tile = reinterpret_cast<char*>(A.ckpt) + c.seqhv * P * ck_row_bytes(CK, N);
    const Lds d = carve(lds, N, L, c.kgpt, A.hvpt, P);

    if (!flush) {
        // ---- non-flush: read checkpoint (or its copy), replay the records ----
        const char* rd = (RC == RC_NONE)
            ? ck_tile
            : reinterpret_cast<const char*>(A.rcopy) + c.seqhv * P * copy_row_bytes(RC, N);
        const void* sc = (RD == RC_FP8 || RD == RC_MXFP4)
            ? reinterpret_cast<const char*>(A.rscale) + c.seqhv * P * scale_row_bytes(RD, N) : nullptr;
        const int rg = tid / RR, gl = tid % RR;
        u32x4 w[UM];
        int ex[UM];
        load_rows<N, RD, UM>(w, rd, 0, c.rows, rg, gl);
        load_block_exp<N, RD, UM>(ex, reinterpret_cast<const uint8_t*>(sc), 0, c.rows, rg, gl);
        if constexpr (!MULTI) {
            // One key group: q slices stay in registers and the scores are
            // formed straight from the key loads, before the first barrier.
            constexpr int RPP4 = RSSM_THREADS / R4;
            constexpr int SP = (32 + RPP4 - 1) / RPP4;    // up to 32 records
            const int rg4 = tid / R4, gl4 = tid % R4;
            const long qoff = ((long)c.b * A.Hk + c.kh0) * N;
            float qs[EPL];
            if constexpr (RD == RC_NONE) load_in<IN, EPL>(A.q, qoff + gl * EPL, qs);
            float q4b[RD == RC_NONE ? 1 : 4];
            if constexpr (RD != RC_NONE) InVec4<IN>::load(A.q, qoff + gl4 * 4, q4b);
            const float* q4 = (RD == RC_NONE) ? qs : q4b;
            // key loads of the score passes (record h, the current one, from the
            // input). Every lane issues exactly one load per pass, lanes past h
            // re-reading the current key (a cache hit) and zeroing it after: a
            // load under a branch makes the compiler wait there for every load in
            // flight, the state rows included.
            constexpr int KSZ = InVec4<IN>::ESZ;
            const char* kb = reinterpret_cast<const char*>(A.kbuf) + ((((long)c.b * A.Hk + c.kh0) * A.C) * N + gl4 * 4) * KSZ;
            const char* kin = reinterpret_cast<const char*>(A.k) + (qoff + gl4 * 4) * KSZ;
            float kv[SP][4];
#pragma unroll
            for (int ps = 0; ps < SP; ++ps) {
                const int j = ps * RPP4 + rg4;
                InVec4<IN>::load_ptr((j < h) ? kb + (long)j * N * KSZ : kin, kv[ps]);
            }
            // value and decay loads, then (copy formats) this lane's q slice
            // for the matvec, so it is not live next to the key values
            const auto rv = v_region<IN, true>(A, c, d.v, nrec, h, 1, true);
            const auto ra = a_region<true>(A, c, d.a, nrec, h, 1, true);
            Batch4<IN, 2> bv;
            BatchA<1> ba;
            bv.load(rv);
            ba.load(ra);
            if constexpr (RD != RC_NONE) load_in<IN, EPL>(A.q, qoff + gl * EPL, qs);
            // append the current key (the tile that owns the key group)
            float sp[SP];
#pragma unroll
            for (int ps = 0; ps < SP; ++ps) {
                const int j = ps * RPP4 + rg4;
                if (j == h && c.kwriter)
                    InVec4<IN>::store(A.kbuf, (((long)c.b * A.Hk + c.kh0) * A.C + j) * N + gl4 * 4, kv[ps]);
                sp[ps] = (j <= h) ? kv[ps][0] * q4[0] + kv[ps][1] * q4[1] + kv[ps][2] * q4[2] + kv[ps][3] * q4[3] : 0.f;
            }
            group_transpose_reduce<SP, R4>(sp, gl4);
            if (gl4 % (R4 / SP) == 0) {
                const int j = (gl4 / (R4 / SP)) * RPP4 + rg4;
                if (j < nrec) d.s[j] = sp[0];
            }
            bv.store(rv);
            ba.store(ra);
            stage_rest<IN, 2>(rv);
            stage_rest_a<1>(ra);
            lds_barrier();
            matvec_tile<N, RD, UM>(w, ex, rd, c.rows, qs, d.y, sc);
        } else {
            // Several key groups: queries and keys staged in LDS, scores and the
            // per-row q slices read from there.
            stage_qkva<IN, 1, 4, 2>(q_region<N, IN>(A, c, d.q, 1),
                                    k_region<N, IN, true>(A, c, d.k, nrec, h, 1, true),
                                    v_region<IN, true>(A, c, d.v, nrec, h, 1, true),
                                    a_region<true>(A, c, d.a, nrec, h, 1, true));
            lds_barrier();
            scores_from_lds<N, 1>(d.k, nrec, d.q, 1, d.s, LS, c.kgpt, nrec, 1);
            matvec_rows<N, RD, UM, 1>(w, ex, rd, A, c, d.q, 1, d.y, 0, sc);
        }
        lds_barrier();
        // o = G y + r,  r = sum_j g_{j+1:h+1} s_j v_j,  G = g_{1:h+1}
        for (int row = tid; row < c.rows; row += RSSM_THREADS) {
            const int vh = row / P, p = row - vh * P;
            const float* s = d.s + kg_of_head(A, c.kgpt, vh) * LS;
            float g = 1.f, acc = 0.f;
            for (int j = nrec - 1; j >= 0; --j) {
                acc = fmaf(g * s[j], d.v[(vh * nrec + j) * P + p], acc);
                g *= d.a[vh * nrec + j];
            }
            A.o[c.seqhv * P + row] = fmaf(g, d.y[row], acc);
        }
        if (tid == 0) A.count[c.cidx] = nrec;
    } else {
        decode_flush<N, IN, RC, MULTI, CK>(A, c, lds, h);
    }
}

// ------------------------------------------------------------------------
// Standalone folds ([ru] §03 flush; [ru] §05 commit by pointer advance;
// [zh] method points): fold the nrec records of tile c into its checkpoint
// (and copy), write it once and set the tile's pointer to 0.
// ------------------------------------------------------------------------
template <int N, int IN, int RC, bool MULTI, int CK>
__device__ __forceinline__ void fold_tile(const StepArgs& A, const Ctx& c, float* lds, int nrec) {
    constexpr int R4 = N / 4, UF = 4;
    const int tid = threadIdx.x, P = A.P, C = A.C;
    char* ck_tile = reinterpret_cast<char*>(A.ckpt) + c.seqhv * P * ck_row_bytes(CK, N);
    const Lds d = carve(lds, N, C, c.kgpt, A.hvpt, P);
    u32x4 S0[UF];
    load_ck_rows<N, CK, UF>(S0, ck_tile, 0, c.rows, tid / R4, tid % R4);
    stage_kva<IN, 4, 2>(k_region<N, IN, false>(A, c, d.k, nrec, nrec, 1, false),
                        v_region<IN, false>(A, c, d.v, nrec, nrec, 1, false),
                        a_region<false>(A, c, d.a, nrec, nrec, 1, false));
    lds_barrier();
    make_weights(d.v, d.a, d.G, A.hvpt, P, nrec, nrec, nrec);
    lds_barrier();
    void* rc_tile = (RC == RC_NONE) ? nullptr
        : reinterpret_cast<char*>(A.rcopy) + c.seqhv * P * copy_row_bytes(RC, N);
    void* rs_tile = reinterpret_cast<char*>(A.rscale) + c.seqhv * P * scale_row_bytes(RC, N);
    const uint32_t key = fold_key<CK>(A, c.cidx);
    fold_rows<N, RC, UF, false, MULTI, CK>(S0, ck_tile, rc_tile, rs_tile, A, c, nrec, nrec, nrec, d.k, d.v, d.G, nullptr,
                                           nullptr, key);
    if (tid == 0) A.count[c.cidx] = 0;
    fold_done<CK>(A, c.cidx);
}

// Explicit flush: every tile with h > 0 records folds them.
template <int N, int IN, int RC, bool MULTI, int CK>
__global__ __launch_bounds__(RSSM_THREADS) void rssm_fold_kernel(StepArgs A) {
    extern __shared__ __attribute__((aligned(16))) float lds[];
    const Ctx c = ctx_of(A);
    const int h = A.count[c.cidx];
    if (h < 0 || h >= A.L) {
        if (threadIdx.x == 0) atomicOr(A.err, 1);
        return;
    }
    if (h > 0) fold_tile<N, IN, RC, MULTI, CK>(A, c, lds, h);
}

// Commit, first kernel: one thread per tile advances its pointer by
// accepted[b]; a tile whose committed records reach L keeps its pointer and is
// appended to the list of tiles to fold.  One atomic per workgroup reserves
// the list slots in work[0], which the verify this commit completes has set
// to 0 (a commit always follows a verify in stream order, also when both are
// replayed from a captured graph).  Invalid pointers or accepted lengths set
// the error word and leave the tile as it was.
__global__ __launch_bounds__(RSSM_THREADS) void rssm_commit_plan_kernel(StepArgs A) {
    __shared__ int wave_n[RSSM_THREADS / 64];
    __shared__ int base;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int ntile = A.B * A.tiles;
    const int i = blockIdx.x * RSSM_THREADS + tid;
    bool fold = false;
    if (i < ntile) {
        const int h = A.count[i];
        const int acc = A.accepted[i / A.tiles];
        const int nrec = h + acc;
        if (h < 0 || h >= A.L) {
            atomicOr(A.err, 1);
        } else if (acc < 0 || acc > A.T) {
            atomicOr(A.err, 2);
        } else if (nrec > A.C) {
            atomicOr(A.err, 4);
        } else if (nrec < A.L) {
            A.count[i] = nrec;
        } else {
            fold = true;
        }
    }
    const uint64_t m = __ballot(fold);
    if (lane == 0) wave_n[wave] = __popcll(m);
    __syncthreads();
    if (tid == 0) {
        int tot = 0;
        for (int w = 0; w < RSSM_THREADS / 64; ++w) tot += wave_n[w];
        base = tot ? atomicAdd(A.work, tot) : 0;
    }
    __syncthreads();
    if (fold) {
        int pos = base;
        for (int w = 0; w < wave; ++w) pos += wave_n[w];
        pos += __popcll(m & ((1ull << lane) - 1ull));
        if (pos < ntile) A.work[2 + pos] = i;             // always, from a zeroed work buffer
    }
}

// Commit, second kernel: a fixed grid walks the list of tiles to fold (none:
// every workgroup exits at once).  Each listed tile folds all h + accepted[b]
// committed records.
template <int N, int IN, int RC, bool MULTI, int CK>
__global__ __launch_bounds__(RSSM_THREADS) void rssm_commit_fold_kernel(StepArgs A) {
    extern __shared__ __attribute__((aligned(16))) float lds[];
    const int ntile = A.B * A.tiles;
    const int n = min(A.work[0], ntile);
    for (int j = blockIdx.x; j < n; j += gridDim.x) {
        const int cidx = A.work[2 + j];
        if (cidx < 0 || cidx >= ntile) continue;
        const Ctx c = ctx_of(A, cidx);
        const int nrec = A.count[cidx] + A.accepted[c.b];
        fold_tile<N, IN, RC, MULTI, CK>(A, c, lds, nrec);
        __syncthreads();                                  // the next tile reuses LDS
    }
}

// ------------------------------------------------------------------------
// Read copy refresh: R = Q(S_ckpt) for every row ([ru] §06: the copy is
// derived from the high-precision checkpoint, never the other way round).
// ------------------------------------------------------------------------
template <int N, int RC, int CK>
__global__ __launch_bounds__(RSSM_THREADS) void rssm_refresh_kernel(StepArgs A) {
    constexpr int R4 = N / 4, RPP4 = RSSM_THREADS / R4;
    const Ctx c = ctx_of(A);
    const char* ck = reinterpret_cast<const char*>(A.ckpt) + c.seqhv * A.P * ck_row_bytes(CK, N);
    void* rc = reinterpret_cast<char*>(A.rcopy) + c.seqhv * A.P * copy_row_bytes(RC, N);
    void* rs = reinterpret_cast<char*>(A.rscale) + c.seqhv * A.P * scale_row_bytes(RC, N);
    const int rg4 = threadIdx.x / R4, gl4 = threadIdx.x % R4;
    for (int row0 = 0; row0 < c.rows; row0 += RPP4) {
        u32x4 w[1];
        load_ck_rows<N, CK, 1>(w, ck, row0 / RPP4, c.rows, rg4, gl4);
        const int row = row0 + rg4;
        store_copy<N, RC>(ck_values<CK>(w[0]), rc, rs, row, gl4, row < c.rows);
    }
}

// ------------------------------------------------------------------------
// Reset listed sequences: zero checkpoint and copy, pointer 0; fp8 row
// scales 1, MXFP4 block exponents 0 (the encoding of an all-zero block).
// Grid: (ids or B) x tiles workgroups.
// ------------------------------------------------------------------------
template <int RC, int CK>
__global__ __launch_bounds__(RSSM_THREADS) void rssm_reset_kernel(StepArgs A, int N) {
    const int i = blockIdx.x / A.tiles, tile = blockIdx.x % A.tiles;
    int b = i;
    if (A.seq_ids) {
        b = A.seq_ids[i];
        if (b < 0 || b >= A.B) {
            if (threadIdx.x == 0 && tile == 0) atomicOr(A.err, 1);
            return;
        }
    }
    const int rows = A.hvpt * A.P;
    const long seqhv = (long)b * A.Hv + tile * A.hvpt;
    // checkpoint bytes rows * N * (4 or 2): a multiple of 16 since P and N are multiples of 4
    u32x4* ck = reinterpret_cast<u32x4*>(reinterpret_cast<char*>(A.ckpt) + seqhv * A.P * ck_row_bytes(CK, N));
    const int n16 = (int)(rows * ck_row_bytes(CK, N) / 16);
    for (int e = threadIdx.x; e < n16; e += RSSM_THREADS) ck[e] = u32x4{0u, 0u, 0u, 0u};
    if constexpr (RC != RC_NONE) {
        uint8_t* rc = reinterpret_cast<uint8_t*>(A.rcopy) + seqhv * A.P * copy_row_bytes(RC, N);
        const int nb = (int)(rows * copy_row_bytes(RC, N) / 4);
        for (int e = threadIdx.x; e < nb; e += RSSM_THREADS) reinterpret_cast<uint32_t*>(rc)[e] = 0u;
    }
    if constexpr (RC == RC_FP8) {
        for (int e = threadIdx.x; e < rows; e += RSSM_THREADS) A.rscale[seqhv * A.P + e] = 1.0f;
    }
    if constexpr (RC == RC_MXFP4) {
        // rows * N/32 bytes: a multiple of 4 since P is
        uint8_t* sb = reinterpret_cast<uint8_t*>(A.rscale) + seqhv * A.P * scale_row_bytes(RC, N);
        const int nb = (int)(rows * scale_row_bytes(RC, N) / 4);
        for (int e = threadIdx.x; e < nb; e += RSSM_THREADS) reinterpret_cast<uint32_t*>(sb)[e] = 0u;
    }
    if (threadIdx.x == 0) A.count[(long)b * A.tiles + tile] = 0;
}

// ------------------------------------------------------------------------
// Commit without a caller work area: the list count and the list of tiles to
// fold live in a library-owned device array, one per GPU (each device holds
// its own copy of this file-scope array until the process ends).  Every call
// on a device shares it, so calls that overlap on one GPU race; each call
// clears the count before planning, and the fold kernel reads only the
// entries this call's plan kernel wrote.
// ------------------------------------------------------------------------
constexpr int kStaticWorkWords = 2 + RSSM_STATIC_COMMIT_MAX_TILES;
static __device__ __align__(256) int32_t scratch[kStaticWorkWords];

__global__ __launch_bounds__(64) void rssm_clear_list_kernel(int32_t* work) {
    if (threadIdx.x == 0) work[0] = 0;
}

}  // namespace rssm

// ------------------------------------------------------------------------
// Host-side launchers (template dispatch on key dim, input dtype, copy
// format and draft capacity).
// ------------------------------------------------------------------------
#include <mutex>
#include "rssm_launch.h"
#include "rssm_dispatch.h"

namespace rssm {

hipError_t launch_decode(const StepArgs& A, int N, int in_dtype, int rc, bool multi, int ck, int grid,
                         size_t lds, hipStream_t s) {
    if (multi) {
        RSSM_DISPATCH_N(N, RSSM_DISPATCH_IN(in_dtype, RSSM_DISPATCH_RC(rc, RSSM_DISPATCH_CK_RC(ck,
            hipLaunchKernelGGL((rssm_decode_kernel<NN, II, RCC, true, CKK>), dim3(grid), dim3(RSSM_THREADS), lds, s, A)))));
    } else {
        RSSM_DISPATCH_N(N, RSSM_DISPATCH_IN(in_dtype, RSSM_DISPATCH_RC(rc, RSSM_DISPATCH_CK_RC(ck,
            hipLaunchKernelGGL((rssm_decode_kernel<NN, II, RCC, false, CKK>), dim3(grid), dim3(RSSM_THREADS), lds, s, A)))));
    }
    return hipGetLastError();
}

hipError_t launch_fold(const StepArgs& A, int N, int in_dtype, int rc, bool multi, int ck, int grid,
                       size_t lds, hipStream_t s) {
    if (multi) {
        RSSM_DISPATCH_N(N, RSSM_DISPATCH_IN(in_dtype, RSSM_DISPATCH_RC(rc, RSSM_DISPATCH_CK_RC(ck,
            hipLaunchKernelGGL((rssm_fold_kernel<NN, II, RCC, true, CKK>), dim3(grid), dim3(RSSM_THREADS), lds, s, A)))));
    } else {
        RSSM_DISPATCH_N(N, RSSM_DISPATCH_IN(in_dtype, RSSM_DISPATCH_RC(rc, RSSM_DISPATCH_CK_RC(ck,
            hipLaunchKernelGGL((rssm_fold_kernel<NN, II, RCC, false, CKK>), dim3(grid), dim3(RSSM_THREADS), lds, s, A)))));
    }
    return hipGetLastError();
}

hipError_t launch_commit(const StepArgs& A, int N, int in_dtype, int rc, bool multi, int ck, int fold_grid,
                         size_t lds, hipStream_t s) {
    const int ntile = A.B * A.tiles;
    hipLaunchKernelGGL(rssm_commit_plan_kernel, dim3((ntile + RSSM_THREADS - 1) / RSSM_THREADS),
                       dim3(RSSM_THREADS), 0, s, A);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    if (multi) {
        RSSM_DISPATCH_N(N, RSSM_DISPATCH_IN(in_dtype, RSSM_DISPATCH_RC(rc, RSSM_DISPATCH_CK_RC(ck,
            hipLaunchKernelGGL((rssm_commit_fold_kernel<NN, II, RCC, true, CKK>), dim3(fold_grid), dim3(RSSM_THREADS), lds, s, A)))));
    } else {
        RSSM_DISPATCH_N(N, RSSM_DISPATCH_IN(in_dtype, RSSM_DISPATCH_RC(rc, RSSM_DISPATCH_CK_RC(ck,
            hipLaunchKernelGGL((rssm_commit_fold_kernel<NN, II, RCC, false, CKK>), dim3(fold_grid), dim3(RSSM_THREADS), lds, s, A)))));
    }
    return hipGetLastError();
}

namespace {
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
int32_t* g_scratch[kMaxDevices] = {};     // device address of `scratch` per device, set on first use
}  // namespace

// Device address of the current device's `scratch` array, looked up once per
// device (the host-side name is only a stand-in, never a device address).
hipError_t static_work(int32_t** out) {
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch[dev]) {
        void* p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return e;
        g_scratch[dev] = static_cast<int32_t*>(p);
    }
    *out = g_scratch[dev];
    return hipSuccess;
}

hipError_t launch_commit_static(const StepArgs& A, int N, int in_dtype, int rc, bool multi, int ck, int fold_grid,
                                size_t lds, hipStream_t s) {
    if ((long)A.B * A.tiles > RSSM_STATIC_COMMIT_MAX_TILES) return hipErrorInvalidValue;
    int32_t* work = nullptr;
    hipError_t e = static_work(&work);
    if (e != hipSuccess) return e;
    StepArgs B = A;
    B.work = work;
    hipLaunchKernelGGL(rssm_clear_list_kernel, dim3(1), dim3(64), 0, s, work);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
    return launch_commit(B, N, in_dtype, rc, multi, ck, fold_grid, lds, s);
}

hipError_t launch_refresh(const StepArgs& A, int N, int rc, int ck, int grid, hipStream_t s) {
    if (rc == RC_NONE) return hipErrorInvalidValue;
    RSSM_DISPATCH_N(N, RSSM_DISPATCH_RC(rc, RSSM_DISPATCH_CK_RC(ck,
        hipLaunchKernelGGL((rssm_refresh_kernel<NN, RCC, CKK>), dim3(grid), dim3(RSSM_THREADS), 0, s, A))));
    return hipGetLastError();
}

hipError_t launch_reset(const StepArgs& A, int N, int rc, int ck, int grid, hipStream_t s) {
    switch (rc) {
        case RC_NONE: RSSM_DISPATCH_CK(ck, hipLaunchKernelGGL((rssm_reset_kernel<RC_NONE, CKK>), dim3(grid), dim3(RSSM_THREADS), 0, s, A, N)); break;
        case RC_BF16: RSSM_DISPATCH_CK(ck, hipLaunchKernelGGL((rssm_reset_kernel<RC_BF16, CKK>), dim3(grid), dim3(RSSM_THREADS), 0, s, A, N)); break;
        case RC_FP8: RSSM_DISPATCH_CK(ck, hipLaunchKernelGGL((rssm_reset_kernel<RC_FP8, CKK>), dim3(grid), dim3(RSSM_THREADS), 0, s, A, N)); break;
        case RC_MXFP4: RSSM_DISPATCH_CK(ck, hipLaunchKernelGGL((rssm_reset_kernel<RC_MXFP4, CKK>), dim3(grid), dim3(RSSM_THREADS), 0, s, A, N)); break;
        default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

}  // namespace rssm
