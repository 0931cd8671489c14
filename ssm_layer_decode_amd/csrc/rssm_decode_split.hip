// rssm_decode_split.hip -- decode step for layers whose non-flush steps read a
// low-precision copy of the checkpoint (MXFP4, or fp8 for heads of at most 64
// rows), on tiles of two value heads; the checkpoint is fp32 or fp16.  The
// device code handles any read format narrower than fp32; the launcher
// instantiates the two it is chosen for.
//
// Citation keys: [ru] aikraft.ru "ReplaySSM: Революция в декодировании
// гибридных моделей" (§03 non-flush step, §06 split precision); [zh]
// ai.cheesepanini.fun card "ReplaySSM——重新思考混合模型解码的状态存储" (method
// points: unrolled window, scores shared by a key group).
//
// A non-flush step outputs, per value head ([ru] §03; eq.U applied to q):
//     o = g_{1:h+1} (R q) + sum_{j<=h+1} g_{j+1:h+1} v_j (k_j . q)
// with R the read data (the copy written at the last fold, [ru] §06) and
// appends the current record.  With a narrow read format a head's rows are a
// few KiB, so the work per head is small next to its fixed costs.  Here a
// 256-thread workgroup holds HV = 256 / NT heads and each head is handled by
// its own NT threads (whole waves, so a head's indices and decays are
// wave-uniform and its decays come through scalar loads): the scores come
// straight from the key loads, each output row's values v_j[p] sit in the
// registers of the thread that owns row p, and the workgroup meets at two LDS
// barriers only.  Every global load is issued before the first use of any
// (the memory counter completes in order).  The flush step folds the tile one
// head at a time (decode_flush_by_head), so the launch's shared memory is the
// larger of the non-flush staging and one head's records, not the whole
// tile's: at the Mamba-2 shape that keeps 8 workgroups per CU resident
// instead of 6, which the non-flush steps need to hide their load latency.
#include "rssm_decode.h"
#include "rssm_launch.h"
#include "rssm_dispatch.h"

namespace rssm {

// Windows up to this many records (the values a thread holds per row).
constexpr int kSplitWindow = 16;

// fp8 row scales of the U rows load_rows streams (rows past the head re-read
// the last row's).
template <int N, int RC, int U, int TH>
__device__ __forceinline__ void load_row_scales(float (&s)[U], const float* sc, int chunk, int rows, int rg) {
    if constexpr (RC == RC_FP8) {
        constexpr int RPP = TH / (N / Ck<RC>::EPL);
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int row = (chunk * U + u) * RPP + rg;
            s[u] = sc[row < rows ? row : rows - 1];
        }
    }
}

// y[row] = R[row] . q for the `rows` rows of one head, TH threads, read format
// RC; chunk 0 (rows, MXFP4 exponents, fp8 scales) is already loaded.  q comes
// from LDS (q_l, the head's N entries), each group of 4 entries read once for
// all U rows of the chunk.
template <int N, int RC, int U, int TH>
__device__ __forceinline__ void matvec_split(u32x4 (&w)[U], int (&ex)[U], float (&rs)[U], const char* base,
                                             const uint8_t* exp_head, const float* scale_head, int rows,
                                             const float* q_l, float* y, int rg, int gl) {
    constexpr int EPL = Ck<RC>::EPL, R = N / EPL, RPP = TH / R;
    const int nchunks = (rows + U * RPP - 1) / (U * RPP);
    const float* qp = q_l + gl * EPL;
    for (int ch = 0; ch < nchunks; ++ch) {
        u32x4 nx[U];
        int nex[U] = {};
        float nrs[U] = {};
        const bool more = ch + 1 < nchunks;
        if (more) {
            load_rows<N, RC, U, TH>(nx, base, ch + 1, rows, rg, gl);
            load_block_exp<N, RC, U, TH>(nex, exp_head, ch + 1, rows, rg, gl);
            load_row_scales<N, RC, U, TH>(nrs, scale_head, ch + 1, rows, rg);
        }
        float part[U];
#pragma unroll
        for (int u = 0; u < U; ++u) part[u] = 0.f;
        // 16 bytes of a row hold EPL entries: 4 words of EPL / 4 entries each
#pragma unroll
        for (int wi = 0; wi < 4; ++wi) {
            constexpr int EW = EPL / 4;                       // entries per 32-bit word
            float qv[EW];
            if constexpr (EW == 2) {
                const f32x2 t = *reinterpret_cast<const f32x2*>(qp + EW * wi);
                qv[0] = t.x; qv[1] = t.y;
            } else {
#pragma unroll
                for (int i = 0; i < EW; i += 4) {
                    const f32x4 t = *reinterpret_cast<const f32x4*>(qp + EW * wi + i);
                    qv[i] = t.x; qv[i + 1] = t.y; qv[i + 2] = t.z; qv[i + 3] = t.w;
                }
            }
#pragma unroll
            for (int u = 0; u < U; ++u) {
                const uint32_t word = wi == 0 ? w[u].x : wi == 1 ? w[u].y : wi == 2 ? w[u].z : w[u].w;
                float x[EPL];
                Ck<RC>::decode(u32x4{word, word, word, word}, x);     // entries of this word: x[0 .. EW)
                float s = part[u];
#pragma unroll
                for (int i = 0; i < EW; ++i) s = fmaf(x[i], qv[i], s);
                part[u] = s;
            }
        }
#pragma unroll
        for (int u = 0; u < U; ++u) {
            part[u] = block_scaled<RC>(part[u], ex[u]);
            if constexpr (RC == RC_FP8) part[u] *= rs[u];
        }
        group_transpose_reduce<U, R>(part, gl);
        put_rows<N, RC, U, false, TH>(part, y, ch, rows, rg, gl, nullptr);
        if (more) {
#pragma unroll
            for (int u = 0; u < U; ++u) {
                w[u] = nx[u];
                ex[u] = nex[u];
                rs[u] = nrs[u];
            }
        }
    }
}

// Non-flush step of tile c (h records buffered, h + 1 < L <= kSplitWindow).
// rbase: the read data (copy, or the fp16 checkpoint) of the whole layer.
// VU: 16-byte value items per thread, kSplitWindow * P / (4 NT) rounded up.
template <int N, int IN, int RD, int NT, int VU>
__device__ __forceinline__ void nonflush_split(const StepArgs& A, const Ctx& c, float* lds, int h, const char* rbase) {
    constexpr int HV = RSSM_THREADS / NT;
    constexpr int R4 = N / 4, RPP4 = NT / R4, SP = (kSplitWindow + RPP4 - 1) / RPP4;
    constexpr int EPL = Ck<RD>::EPL, RR = N / EPL, UM = ReadU<RD>::U;
    constexpr int ESZ = InVec4<IN>::ESZ;
    static_assert(NT % 64 == 0 && RPP4 >= 1 && SP <= R4, "split tile shape");
    static_assert(VU >= 1, "value items");   // VU * NT >= kSplitWindow * P / 4: chosen by the launcher
    const int tid = threadIdx.x;
    const int sub = __builtin_amdgcn_readfirstlane(tid / NT);       // the wave's head within the tile
    const int st = tid - sub * NT;
    const int P = A.P, C = A.C, Hk = A.Hk, nrec = h + 1;
    const int vh = c.vh0 + sub, kh = vh / A.g;
    const bool kwriter = vh == kh * A.g;                           // first head of its key group
    const long seqhv = c.seqhv + sub;
    const long kq = ((long)c.b * Hk + kh) * N;                     // the head's k / q rows
    const int L = A.L;
    float* q_l = lds;                                               // [HV][N]
    float* s_l = q_l + HV * N;                                      // [HV][kSplitWindow]
    float* a_l = s_l + HV * kSplitWindow;                           // [HV][kSplitWindow]
    float* y_l = a_l + HV * kSplitWindow;                           // [HV][P]
    float* v_l = y_l + HV * P;                                      // [HV][L][P]

    // ---- global loads ----
    const char* rd = rbase + seqhv * P * copy_row_bytes(RD, N);
    const uint8_t* exh = reinterpret_cast<const uint8_t*>(A.rscale) + seqhv * P * scale_row_bytes(RD, N);
    const float* sch = A.rscale + seqhv * P;
    const int rg = st / RR, gl = st % RR;
    u32x4 w[UM];
    int ex[UM] = {};
    float rs[UM] = {};
    load_rows<N, RD, UM, NT>(w, rd, 0, P, rg, gl);
    load_block_exp<N, RD, UM, NT>(ex, exh, 0, P, rg, gl);
    load_row_scales<N, RD, UM, NT>(rs, sch, 0, P, rg);
    // keys of records j = ps * RPP4 + rg4 (j >= h: the current key, a cache hit, dropped below j > h)
    const int rg4 = st / R4, gl4 = st % R4;
    const char* kb = reinterpret_cast<const char*>(A.kbuf) + (((long)c.b * Hk + kh) * C * N + gl4 * 4) * ESZ;
    const char* kin = reinterpret_cast<const char*>(A.k) + (kq + gl4 * 4) * ESZ;
    float kv[SP][4];
#pragma unroll
    for (int ps = 0; ps < SP; ++ps) {
        const int j = ps * RPP4 + rg4;
        InVec4<IN>::load_ptr(j < h ? kb + (long)j * N * ESZ : kin, kv[ps]);
    }
    float q4[4];
    InVec4<IN>::load(A.q, kq + gl4 * 4, q4);
    // the head's value records j <= h, 4 entries per item: slots 0..h-1 of the
    // buffer are contiguous (item e at entry 4e), slot h is the current input;
    // items past the head's re-read its last one
    const int nv = nrec * (P / 4), hv4 = h * (P / 4);
    char* vbh = reinterpret_cast<char*>(A.vbuf) + seqhv * C * P * ESZ;
    const char* vinh = reinterpret_cast<const char*>(A.v) + seqhv * P * ESZ;
    typename InVec4<IN>::Raw vr[VU];
#pragma unroll
    for (int i = 0; i < VU; ++i) {
        const int e0 = st + i * NT, e = e0 < nv ? e0 : nv - 1;
        vr[i] = InVec4<IN>::load_raw(e < hv4 ? vbh + (long)e * 4 * ESZ : vinh + (long)(e - hv4) * 4 * ESZ);
    }
    // decays: thread st of the head loads a_st (st < h from the buffer, else
    // the current one), passed on through LDS like the scores
    float* ab = A.abuf + seqhv * C;
    const float a_mine = *(st < h ? ab + st : A.alpha + seqhv);

    // ---- appends of the current record (slot h), q to LDS, scores ----
    if (rg4 == 0) *reinterpret_cast<f32x4*>(q_l + sub * N + gl4 * 4) = f32x4{q4[0], q4[1], q4[2], q4[3]};
    float sp[SP];
#pragma unroll
    for (int ps = 0; ps < SP; ++ps) {
        const int j = ps * RPP4 + rg4;
        if (j == h && kwriter)
            InVec4<IN>::store(A.kbuf, ((long)c.b * Hk + kh) * C * N + (long)j * N + gl4 * 4, kv[ps]);
        sp[ps] = (j <= h) ? kv[ps][0] * q4[0] + kv[ps][1] * q4[1] + kv[ps][2] * q4[2] + kv[ps][3] * q4[3] : 0.f;
    }
    // values into LDS; the current record's items are appended to slot h (entry 4e of the head)
#pragma unroll
    for (int i = 0; i < VU; ++i) {
        const int e = st + i * NT;
        if (e < nv) {
            *reinterpret_cast<f32x4*>(v_l + sub * L * P + 4 * e) = InVec4<IN>::unpack(vr[i]);
            if (e >= hv4) InVec4<IN>::store_raw(vbh + (long)e * 4 * ESZ, vr[i]);
        }
    }
    if (st < nrec) a_l[sub * kSplitWindow + st] = a_mine;
    if (st == h) ab[h] = a_mine;                                    // append the current decay
    group_transpose_reduce<SP, R4>(sp, gl4);
    if (gl4 % (R4 / SP) == 0) {
        const int j = (gl4 / (R4 / SP)) * RPP4 + rg4;
        if (j < nrec) s_l[sub * kSplitWindow + j] = sp[0];
    }
    lds_barrier();

    // ---- replay for row p = st < P (a whole wave skips it when P <= 64):
    //      acc = sum_j g_{j+1:h+1} s_j v_j[p], G = g_{1:h+1} ----
    float acc = 0.f, g = 1.f;
    if (st < P) {
        const float* vp = v_l + sub * L * P + st;
#pragma unroll
        for (int j = kSplitWindow - 1; j >= 0; --j) {
            if (j <= h) {
                acc = fmaf(g * s_l[sub * kSplitWindow + j], vp[j * P], acc);
                g *= a_l[sub * kSplitWindow + j];
            }
        }
    }
    // ---- y = R q over the head's rows ----
    matvec_split<N, RD, UM, NT>(w, ex, rs, rd, exh, sch, P, q_l + sub * N, y_l + sub * P, rg, gl);
    lds_barrier();
    if (st < P) A.o[seqhv * P + st] = fmaf(g, y_l[sub * P + st], acc);
    if (tid == 0) A.count[c.cidx] = nrec;
}

// Occupancy: the non-flush steps hide their load latency with resident
// waves, so the register budget is capped for 8 waves per SIMD (6 for heads
// of more than 64 rows, whose value items need more registers; 7 spilled).
// Uncapped, the compiler's 106 SGPRs allowed 7 and 5 waves: capped, non-flush
// steps measured 3-5 % faster and flush steps about 3 % slower.
template <int N, int IN, int RC, int CK, int NT, int VU>
__global__ __launch_bounds__(RSSM_THREADS) __attribute__((amdgpu_waves_per_eu(VU == 2 ? 8 : 6)))
void rssm_decode_split_kernel(StepArgs A) {
    extern __shared__ __attribute__((aligned(16))) float lds[];
    constexpr int RD = (RC == RC_NONE) ? ck_read_format(CK) : RC;
    static_assert(RD != RC_NONE, "the split path reads a copy or an fp16 checkpoint");
    const Ctx c = ctx_of(A);
    const int h = A.count[c.cidx];
    if (h < 0 || h >= A.L) {
        if (threadIdx.x == 0) atomicOr(A.err, 1);
        return;
    }
    if (h + 1 < A.L) {
        const char* base = (RC == RC_NONE) ? reinterpret_cast<const char*>(A.ckpt)
                                           : reinterpret_cast<const char*>(A.rcopy);
        nonflush_split<N, IN, RD, NT, VU>(A, c, lds, h, base);
    } else {
        decode_flush_by_head<N, IN, RC, CK, 2, RSSM_THREADS / NT>(A, c, lds, h);
    }
}

// Key dims 64 and 128, fp8 or MXFP4 copies, two heads of 128 threads per tile;
// value items per thread for rows per head up to 64 (2) or 128 (4).
hipError_t launch_decode_split(const StepArgs& A, int N, int in_dtype, int rc, int ck, int grid, size_t lds,
                               hipStream_t s) {
#define RSSM_SPLIT(NN, II, RCC, CKK)                                                                      \
    if (A.P <= 64)                                                                                        \
        hipLaunchKernelGGL((rssm_decode_split_kernel<NN, II, RCC, CKK, 128, 2>), dim3(grid),              \
                           dim3(RSSM_THREADS), lds, s, A);                                                \
    else                                                                                                  \
        hipLaunchKernelGGL((rssm_decode_split_kernel<NN, II, RCC, CKK, 128, 4>), dim3(grid),              \
                           dim3(RSSM_THREADS), lds, s, A)
#define RSSM_SPLIT_RC(NN, II)                                                                             \
    switch (rc) {                                                                                         \
        case RC_FP8: RSSM_DISPATCH_CK(ck, RSSM_SPLIT(NN, II, RC_FP8, CKK)); break;                        \
        case RC_MXFP4: RSSM_DISPATCH_CK(ck, RSSM_SPLIT(NN, II, RC_MXFP4, CKK)); break;                    \
        default: return hipErrorInvalidValue;                                                             \
    }
    switch (N) {
        case 64: RSSM_DISPATCH_IN(in_dtype, RSSM_SPLIT_RC(64, II)); break;
        case 128: RSSM_DISPATCH_IN(in_dtype, RSSM_SPLIT_RC(128, II)); break;
        default: return hipErrorInvalidValue;
    }
#undef RSSM_SPLIT_RC
#undef RSSM_SPLIT
    return hipGetLastError();
}

}  // namespace rssm
