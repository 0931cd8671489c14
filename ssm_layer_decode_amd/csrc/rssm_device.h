// rssm_device.h -- device helpers shared by the ReplaySSM kernels (gfx950).
//
// Work decomposition used by every kernel: one 256-thread workgroup per
// (sequence, tile), a tile being `hvpt` consecutive value heads of one key
// group.  A state row (the N key-dim entries that one output element dots with
// q) is split across R = N / EPL lanes, each lane holding EPL consecutive
// elements in one 16-byte load; RPP = 256 / R rows are in flight per pass.
// A thread accumulates U rows' partial dot products and the R lanes of a row
// group are combined with a transposing butterfly (group_transpose_reduce),
// which halves the number of live values at each exchange.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#define RSSM_THREADS 256

typedef float    f32x4 __attribute__((ext_vector_type(4)));
typedef float    f32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

namespace rssm {

enum { IN_F32 = 0, IN_BF16 = 1 };
// Read formats of the state rows a matvec streams: the fp32 checkpoint, a
// read copy (bf16, fp8, MXFP4), or an fp16 checkpoint (RC_F16, internal).
enum { RC_NONE = 0, RC_BF16 = 1, RC_FP8 = 2, RC_MXFP4 = 3, RC_F16 = 4 };
// Storage of the recurrent checkpoint: fp32, fp16 with stochastic rounding,
// or row-scaled e4m3 with stochastic rounding (read through a copy only).
enum { CK_F32 = 0, CK_F16 = 1, CK_FP8 = 2 };

// ------------------------------------------------------------- conversions
__device__ __forceinline__ float bf16_to_f32(uint32_t bits16) {
    return __uint_as_float(bits16 << 16);
}

// Round to nearest even; NaN stays NaN (quiet).
__device__ __forceinline__ uint32_t f32_to_bf16_bits(float f) {
    uint32_t u = __float_as_uint(f);
    if ((u & 0x7fffffffu) > 0x7f800000u) return (u >> 16) | 0x40u;
    u += 0x7fffu + ((u >> 16) & 1u);
    return u >> 16;
}

// OCP e4m3fn (gfx950's native fp8): hardware convert, round to nearest even.
// Inputs are pre-scaled into [-448, 448] (plus at most one rounding step of
// the scale division), so no value can reach the overflow threshold 464.
__device__ __forceinline__ uint32_t pack4_e4m3(float a, float b, float c, float d) {
    int w = __builtin_amdgcn_cvt_pk_fp8_f32(a, b, 0, false);
    w = __builtin_amdgcn_cvt_pk_fp8_f32(c, d, w, true);
    return (uint32_t)w;
}

__device__ __forceinline__ void unpack4_e4m3(uint32_t w, float* out) {
    f32x2 lo = __builtin_amdgcn_cvt_pk_f32_fp8((int)w, false);
    f32x2 hi = __builtin_amdgcn_cvt_pk_f32_fp8((int)w, true);
    out[0] = lo.x; out[1] = lo.y; out[2] = hi.x; out[3] = hi.y;
}

// ------------------------------------------------------------- loads
template <int IN>
struct InVec4;   // 4 consecutive k/q/v elements of the input dtype

template <>
struct InVec4<IN_F32> {
    static constexpr int ESZ = 4;
    // raw bits of 4 elements: loaded, stored back and unpacked separately, so
    // a conditional load needs no arithmetic on its result under the branch
    using Raw = u32x4;
    static __device__ __forceinline__ Raw load_raw(const char* p) { return *reinterpret_cast<const u32x4*>(p); }
    static __device__ __forceinline__ void store_raw(char* p, const Raw& r) { *reinterpret_cast<u32x4*>(p) = r; }
    static __device__ __forceinline__ f32x4 unpack(const Raw& r) {
        return f32x4{__uint_as_float(r.x), __uint_as_float(r.y), __uint_as_float(r.z), __uint_as_float(r.w)};
    }
    static __device__ __forceinline__ void load_ptr(const char* p, float* out) {
        f32x4 v = *reinterpret_cast<const f32x4*>(p);
        out[0] = v.x; out[1] = v.y; out[2] = v.z; out[3] = v.w;
    }
    static __device__ __forceinline__ void store_ptr(char* p, const float* in) {
        *reinterpret_cast<f32x4*>(p) = f32x4{in[0], in[1], in[2], in[3]};
    }
    static __device__ __forceinline__ void load(const void* base, long idx, float* out) {
        f32x4 v = *reinterpret_cast<const f32x4*>(reinterpret_cast<const float*>(base) + idx);
        out[0] = v.x; out[1] = v.y; out[2] = v.z; out[3] = v.w;
    }
    static __device__ __forceinline__ void store(void* base, long idx, const float* in) {
        f32x4 v = {in[0], in[1], in[2], in[3]};
        *reinterpret_cast<f32x4*>(reinterpret_cast<float*>(base) + idx) = v;
    }
};

template <>
struct InVec4<IN_BF16> {
    static constexpr int ESZ = 2;
    using Raw = u32x2;
    static __device__ __forceinline__ Raw load_raw(const char* p) { return *reinterpret_cast<const u32x2*>(p); }
    static __device__ __forceinline__ void store_raw(char* p, const Raw& r) { *reinterpret_cast<u32x2*>(p) = r; }
    static __device__ __forceinline__ f32x4 unpack(const Raw& r) {
        return f32x4{__uint_as_float(r.x << 16), __uint_as_float(r.x & 0xffff0000u),
                     __uint_as_float(r.y << 16), __uint_as_float(r.y & 0xffff0000u)};
    }
    static __device__ __forceinline__ void load_ptr(const char* p, float* out) {
        u32x2 v = *reinterpret_cast<const u32x2*>(p);
        out[0] = __uint_as_float(v.x << 16);
        out[1] = __uint_as_float(v.x & 0xffff0000u);
        out[2] = __uint_as_float(v.y << 16);
        out[3] = __uint_as_float(v.y & 0xffff0000u);
    }
    // Stores values that were loaded from bf16 (low 16 bits zero): the
    // original bits move back unchanged.
    static __device__ __forceinline__ void store_ptr(char* p, const float* in) {
        const uint32_t lo = (__float_as_uint(in[0]) >> 16) | (__float_as_uint(in[1]) & 0xffff0000u);
        const uint32_t hi = (__float_as_uint(in[2]) >> 16) | (__float_as_uint(in[3]) & 0xffff0000u);
        *reinterpret_cast<u32x2*>(p) = u32x2{lo, hi};
    }
    static __device__ __forceinline__ void load(const void* base, long idx, float* out) {
        u32x2 v = *reinterpret_cast<const u32x2*>(reinterpret_cast<const uint16_t*>(base) + idx);
        out[0] = __uint_as_float(v.x << 16);
        out[1] = __uint_as_float(v.x & 0xffff0000u);
        out[2] = __uint_as_float(v.y << 16);
        out[3] = __uint_as_float(v.y & 0xffff0000u);
    }
    // Store values that were loaded from bf16 (the low 16 bits of each are
    // zero), so this moves the original bits back unchanged.
    static __device__ __forceinline__ void store(void* base, long idx, const float* in) {
        const uint32_t lo = (__float_as_uint(in[0]) >> 16) | (__float_as_uint(in[1]) & 0xffff0000u);
        const uint32_t hi = (__float_as_uint(in[2]) >> 16) | (__float_as_uint(in[3]) & 0xffff0000u);
        *reinterpret_cast<u32x2*>(reinterpret_cast<uint16_t*>(base) + idx) = u32x2{lo, hi};
    }
};

template <int IN>
__device__ __forceinline__ float load_scalar(const void* base, long idx) {
    if constexpr (IN == IN_F32) return reinterpret_cast<const float*>(base)[idx];
    else return bf16_to_f32(reinterpret_cast<const uint16_t*>(base)[idx]);
}

// ------------------------------------------------------------- cross-lane
// Value of `x` held by lane (lane ^ M).  M < 64.
template <int M>
__device__ __forceinline__ float xor_lane(float x) {
    if constexpr (M == 1) {
        return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), 0xB1, 0xF, 0xF, false));
    } else if constexpr (M == 2) {
        return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), 0x4E, 0xF, 0xF, false));
    } else if constexpr (M <= 16) {
        // ds_swizzle bit mode: and_mask 0x1f, or_mask 0, xor_mask M
        return __int_as_float(__builtin_amdgcn_ds_swizzle(__float_as_int(x), 0x1F | (M << 10)));
    } else {
        return __shfl_xor(x, M, 64);
    }
}

// Sum each of the U values over the R consecutive lanes of a row group
// (lane index in group = `gl`).  Afterwards, for U >= R lane gl holds in
// v[0 .. U/R) the totals of values [gl*U/R, (gl+1)*U/R); for U < R it holds in
// v[0] the total of value gl / (R/U) (R/U lanes agree).
template <int U, int R, int M = R / 2, int CNT = U>
__device__ __forceinline__ void group_transpose_reduce(float (&v)[U], int gl) {
    if constexpr (M >= 1) {
        if constexpr (CNT > 1) {
            constexpr int H = CNT / 2;
            const bool upper = (gl & M) != 0;
#pragma unroll
            for (int i = 0; i < H; ++i) {
                const float send = upper ? v[i] : v[H + i];
                const float keep = upper ? v[H + i] : v[i];
                v[i] = keep + xor_lane<M>(send);
            }
            group_transpose_reduce<U, R, M / 2, H>(v, gl);
        } else {
            v[0] += xor_lane<M>(v[0]);
            group_transpose_reduce<U, R, M / 2, 1>(v, gl);
        }
    }
}

// Max over the R lanes of a row group (all lanes get the result).
template <int R, int M = R / 2>
__device__ __forceinline__ float group_max(float x) {
    if constexpr (M >= 1) {
        x = fmaxf(x, xor_lane<M>(x));
        return group_max<R, M / 2>(x);
    } else {
        return x;
    }
}

// Sum over the R lanes of a row group (all lanes get the result).
template <int R, int M = R / 2>
__device__ __forceinline__ float group_sum(float x) {
    if constexpr (M >= 1) {
        x += xor_lane<M>(x);
        return group_sum<R, M / 2>(x);
    } else {
        return x;
    }
}

// Barrier for LDS traffic only: waits for this wave's LDS operations, then
// joins the workgroup barrier.  Outstanding global loads stay in flight
// (a full __syncthreads would drain them too).
__device__ __forceinline__ void lds_barrier() {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

}  // namespace rssm
