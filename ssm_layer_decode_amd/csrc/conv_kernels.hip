// conv_kernels.hip -- in-run GPU baselines for gfx950: conventional fused decode
// and snapshot speculative verification.
//
// Citation keys: [ru] aikraft.ru "ReplaySSM: Революция в декодировании
// гибридных моделей" (§01-§07).
//
// Conventional decode ([ru] §01): every step loads the whole state, applies
// the decay and the rank-1 update S <- a S + v k^T, forms o = S q, and stores
// the state back, so each token moves the state twice.  With a quantised state
// format the state is re-quantised after every step and the rounding re-enters
// the next update ([ru] §02, problem 3).
//
// Snapshot verification ([ru] §02 problem 2 and §05): one state read, then one
// full state snapshot written per draft so that any accepted prefix can be
// restored; commit selects the snapshot by moving a ring index.
//
// Same decomposition as the ReplaySSM kernels: one 256-thread workgroup per
// (sequence, tile of hvpt value heads of one key group), state rows split over
// R lanes with 16-byte loads.
#include "rssm_stream.h"
#include "rssm_launch.h"

namespace rssm {

// Store one row slice held by a lane (EPL values, 16 bytes) in state format
// fp32 or bf16 (round to nearest even).  fp8 rows are stored inline by the
// kernel because their scale needs the whole row group.
template <int N, int SF>
__device__ __forceinline__ void store_state_row(const float* x, char* rowp, int gl) {
    if constexpr (SF == RC_NONE) {
        st16(rowp + gl * 16, u32x4{__float_as_uint(x[0]), __float_as_uint(x[1]),
                                   __float_as_uint(x[2]), __float_as_uint(x[3])});
    } else if constexpr (SF == RC_BF16) {
        uint32_t w[4];
#pragma unroll
        for (int i = 0; i < 4; ++i)
            w[i] = f32_to_bf16_bits(x[2 * i]) | (f32_to_bf16_bits(x[2 * i + 1]) << 16);
        st16(rowp + gl * 16, u32x4{w[0], w[1], w[2], w[3]});
    }
}

template <int N, int IN, int SF>
__global__ __launch_bounds__(RSSM_THREADS) void conv_decode_kernel(ConvArgs A) {
    extern __shared__ __attribute__((aligned(16))) float lds[];
    constexpr int EPL = Ck<SF>::EPL, ESZ = Ck<SF>::ESZ, R = N / EPL, RPP = RSSM_THREADS / R;
    constexpr int U = (SF == RC_NONE) ? 4 : (SF == RC_BF16 ? 2 : 1);
    const int tid = threadIdx.x;
    const Tile t = tile_of(A);
    const int P = A.P, rows = A.hvpt * P;
    const long seqhv = (long)t.b * A.Hv + t.vh0;
    char* st = reinterpret_cast<char*>(A.state) + seqhv * P * N * ESZ;
    float* scale = (SF == RC_FP8) ? A.rscale + seqhv * P : nullptr;
    const int rg = tid / R, gl = tid % R;
    // LDS: v_l [rows], a_l [hvpt], y_l [rows]
    float* v_l = lds;
    float* a_l = v_l + rows;
    float* y_l = a_l + ((A.hvpt + 3) & ~3);

    u32x4 w[U];
    load_rows<N, SF, U>(w, st, 0, rows, rg, gl);
    const long qoff = ((long)t.b * A.Hk + t.kh) * N + gl * EPL;
    float kk[EPL], qq[EPL];
    load_in<IN, EPL>(A.k, qoff, kk);
    load_in<IN, EPL>(A.q, qoff, qq);
    for (int row = tid; row < rows; row += RSSM_THREADS)
        v_l[row] = load_scalar<IN>(A.v, seqhv * P + row);
    if (tid < A.hvpt) a_l[tid] = A.alpha[seqhv + tid];
    lds_barrier();

    const int nchunks = (rows + U * RPP - 1) / (U * RPP);
    for (int c = 0; c < nchunks; ++c) {
        u32x4 nx[U];
        const bool more = (c + 1 < nchunks);
        if (more) load_rows<N, SF, U>(nx, st, c + 1, rows, rg, gl);
        float part[U];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int row = (c * U + u) * RPP + rg;
            const bool valid = row < rows;
            const int r = valid ? row : 0;
            float x[EPL];
            Ck<SF>::decode(w[u], x);
            float sc_old = 1.f;
            if constexpr (SF == RC_FP8) sc_old = valid ? scale[r] : 1.f;
            const float a = a_l[r / P], vv = v_l[r];
            float s = 0.f;
#pragma unroll
            for (int i = 0; i < EPL; ++i) {
                x[i] = fmaf(a, x[i] * sc_old, vv * kk[i]);
                s = fmaf(x[i], qq[i], s);
            }
            part[u] = s;
            if constexpr (SF == RC_FP8) {
                // the row max needs every lane of the row group
                float m = 0.f;
#pragma unroll
                for (int i = 0; i < EPL; ++i) m = fmaxf(m, fabsf(x[i]));
                m = group_max<R>(m);
                if (valid) {
                    float sc = m / 448.0f;
                    if (!(sc > 0.0f)) sc = 1.0f;
                    uint32_t q4[4];
#pragma unroll
                    for (int i = 0; i < 4; ++i)
                        q4[i] = pack4_e4m3(x[4 * i] / sc, x[4 * i + 1] / sc, x[4 * i + 2] / sc,
                                           x[4 * i + 3] / sc);
                    st16(st + (long)row * N * ESZ + gl * 16, u32x4{q4[0], q4[1], q4[2], q4[3]});
                    if (gl == 0) scale[row] = sc;
                }
            } else {
                if (valid) store_state_row<N, SF>(x, st + (long)row * N * ESZ, gl);
            }
        }
        group_transpose_reduce<U, R>(part, gl);
        put_rows<N, SF, U, false>(part, y_l, c, rows, rg, gl, nullptr);
        if (more) {
#pragma unroll
            for (int u = 0; u < U; ++u) w[u] = nx[u];
        }
    }
    lds_barrier();
    for (int row = tid; row < rows; row += RSSM_THREADS) A.o[seqhv * P + row] = y_l[row];
}

// Snapshot verify: T drafts through the recurrence from ring slot cur[b];
// state after draft t stored in slot (cur[b] + t) mod ring.
template <int N, int IN, int TT>
__global__ __launch_bounds__(RSSM_THREADS) void conv_verify_kernel(ConvArgs A) {
    extern __shared__ __attribute__((aligned(16))) float lds[];
    constexpr int R = N / 4, RPP = RSSM_THREADS / R, U = 2;
    const int tid = threadIdx.x;
    const Tile t = tile_of(A);
    const int P = A.P, rows = A.hvpt * P, T = A.T, ring = A.ring;
    const int cur = A.cur[t.b];
    if (cur < 0 || cur >= ring) {
        if (tid == 0) atomicOr(A.err, 1);
        return;
    }
    const long slot_stride = (long)A.Hv * P * N;                  // floats per ring slot
    float* seq = reinterpret_cast<float*>(A.state) + (long)t.b * ring * slot_stride;
    const long tile_off = (long)t.vh0 * P * N;
    const int rg = tid / R, gl = tid % R;
    // LDS: v_l [TT][rows], a_l [TT][hvpt], y_l [TT][rows]
    float* v_l = lds;
    float* a_l = v_l + TT * rows;
    float* y_l = a_l + TT * ((A.hvpt + 3) & ~3);
    const int HS = (A.hvpt + 3) & ~3;

    u32x4 w[U];
    load_rows<N, RC_NONE, U>(w, reinterpret_cast<const char*>(seq + cur * slot_stride + tile_off), 0,
                             rows, rg, gl);
    const long dstride = (long)A.Hk * N;                          // between drafts in k/q
    const long k0 = (long)t.b * T * dstride + (long)t.kh * N + gl * 4;
    float kk[TT][4], qq[TT][4];
#pragma unroll
    for (int d = 0; d < TT; ++d) {
        if (d < T) {
            InVec4<IN>::load(A.k, k0 + d * dstride, kk[d]);
            InVec4<IN>::load(A.q, k0 + d * dstride, qq[d]);
        } else {
#pragma unroll
            for (int i = 0; i < 4; ++i) kk[d][i] = qq[d][i] = 0.f;
        }
    }
    for (int e = tid; e < T * rows; e += RSSM_THREADS) {
        const int d = e / rows, row = e - d * rows;
        v_l[d * rows + row] = load_scalar<IN>(A.v, ((long)t.b * T + d) * A.Hv * P + (long)t.vh0 * P + row);
    }
    for (int e = tid; e < T * A.hvpt; e += RSSM_THREADS) {
        const int d = e / A.hvpt, vh = e - d * A.hvpt;
        a_l[d * HS + vh] = A.alpha[((long)t.b * T + d) * A.Hv + t.vh0 + vh];
    }
    lds_barrier();
    const int nchunks = (rows + U * RPP - 1) / (U * RPP);
    for (int c = 0; c < nchunks; ++c) {
        u32x4 nx[U];
        const bool more = (c + 1 < nchunks);
        if (more)
            load_rows<N, RC_NONE, U>(nx, reinterpret_cast<const char*>(seq + cur * slot_stride + tile_off),
                                     c + 1, rows, rg, gl);
        float part[U * TT];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int row = (c * U + u) * RPP + rg;
            const bool valid = row < rows;
            const int r = valid ? row : 0;
            f32x4 s = {__uint_as_float(w[u].x), __uint_as_float(w[u].y), __uint_as_float(w[u].z),
                       __uint_as_float(w[u].w)};
#pragma unroll
            for (int d = 0; d < TT; ++d) {
                part[u * TT + d] = 0.f;
                if (d < T) {
                    const float a = a_l[d * HS + r / P], vv = v_l[d * rows + r];
                    s.x = fmaf(a, s.x, vv * kk[d][0]);
                    s.y = fmaf(a, s.y, vv * kk[d][1]);
                    s.z = fmaf(a, s.z, vv * kk[d][2]);
                    s.w = fmaf(a, s.w, vv * kk[d][3]);
                    part[u * TT + d] = s.x * qq[d][0] + s.y * qq[d][1] + s.z * qq[d][2] + s.w * qq[d][3];
                    if (valid) {
                        const int slot = (cur + 1 + d) % ring;
                        st16(reinterpret_cast<char*>(seq + slot * slot_stride + tile_off) + (long)row * N * 4 + gl * 16,
                             u32x4{__float_as_uint(s.x), __float_as_uint(s.y), __float_as_uint(s.z),
                                   __float_as_uint(s.w)});
                    }
                }
            }
        }
        constexpr int UT = U * TT;
        group_transpose_reduce<UT, R>(part, gl);
        auto put = [&](int idx, float val) {
            const int u = idx / TT, d = idx - u * TT;
            const int row = (c * U + u) * RPP + rg;
            if (row < rows) y_l[d * rows + row] = val;
        };
        if constexpr (UT >= R) {
#pragma unroll
            for (int i = 0; i < UT / R; ++i) put(gl * (UT / R) + i, part[i]);
        } else {
            if (gl % (R / UT) == 0) put(gl / (R / UT), part[0]);
        }
        if (more) {
#pragma unroll
            for (int u = 0; u < U; ++u) w[u] = nx[u];
        }
    }
    lds_barrier();
    for (int e = tid; e < T * rows; e += RSSM_THREADS) {
        const int d = e / rows, row = e - d * rows;
        A.o[(((long)t.b * T + d) * A.Hv + t.vh0) * P + row] = y_l[d * rows + row];
    }
}

__global__ void conv_commit_kernel(ConvArgs A) {
    const int b = blockIdx.x * blockDim.x + threadIdx.x;
    if (b >= A.B) return;
    const int a = A.accepted[b];
    if (a < 0 || a > A.T) {
        atomicOr(A.err, 2);
        return;
    }
    A.cur_rw[b] = (A.cur_rw[b] + a) % A.ring;
}

#define CONV_DISPATCH_N(N_, ...)                                      \
    switch (N_) {                                                     \
        case 16: { constexpr int NN = 16; __VA_ARGS__; } break;       \
        case 32: { constexpr int NN = 32; __VA_ARGS__; } break;       \
        case 64: { constexpr int NN = 64; __VA_ARGS__; } break;       \
        case 128: { constexpr int NN = 128; __VA_ARGS__; } break;     \
        case 256: { constexpr int NN = 256; __VA_ARGS__; } break;     \
        default: return hipErrorInvalidValue;                         \
    }
#define CONV_DISPATCH_IN(I_, ...)                                     \
    switch (I_) {                                                     \
        case IN_F32: { constexpr int II = IN_F32; __VA_ARGS__; } break;   \
        case IN_BF16: { constexpr int II = IN_BF16; __VA_ARGS__; } break; \
        default: return hipErrorInvalidValue;                         \
    }

hipError_t launch_conv_decode(const ConvArgs& A, int N, int in_dtype, int sf, int grid, size_t lds,
                              hipStream_t s) {
    CONV_DISPATCH_N(N, CONV_DISPATCH_IN(in_dtype, switch (sf) {
        case RC_NONE: hipLaunchKernelGGL((conv_decode_kernel<NN, II, RC_NONE>), dim3(grid), dim3(RSSM_THREADS), lds, s, A); break;
        case RC_BF16: hipLaunchKernelGGL((conv_decode_kernel<NN, II, RC_BF16>), dim3(grid), dim3(RSSM_THREADS), lds, s, A); break;
        case RC_FP8: hipLaunchKernelGGL((conv_decode_kernel<NN, II, RC_FP8>), dim3(grid), dim3(RSSM_THREADS), lds, s, A); break;
        default: return hipErrorInvalidValue;
    }));
    return hipGetLastError();
}

hipError_t launch_conv_verify(const ConvArgs& A, int N, int in_dtype, int tt, int grid, size_t lds,
                              hipStream_t s) {
    CONV_DISPATCH_N(N, CONV_DISPATCH_IN(in_dtype, switch (tt) {
        case 1: hipLaunchKernelGGL((conv_verify_kernel<NN, II, 1>), dim3(grid), dim3(RSSM_THREADS), lds, s, A); break;
        case 2: hipLaunchKernelGGL((conv_verify_kernel<NN, II, 2>), dim3(grid), dim3(RSSM_THREADS), lds, s, A); break;
        case 4: hipLaunchKernelGGL((conv_verify_kernel<NN, II, 4>), dim3(grid), dim3(RSSM_THREADS), lds, s, A); break;
        case 8: hipLaunchKernelGGL((conv_verify_kernel<NN, II, 8>), dim3(grid), dim3(RSSM_THREADS), lds, s, A); break;
        default: return hipErrorInvalidValue;
    }));
    return hipGetLastError();
}

hipError_t launch_conv_commit(const ConvArgs& A, hipStream_t s) {
    hipLaunchKernelGGL(conv_commit_kernel, dim3((A.B + 255) / 256), dim3(256), 0, s, A);
    return hipGetLastError();
}

}  // namespace rssm
