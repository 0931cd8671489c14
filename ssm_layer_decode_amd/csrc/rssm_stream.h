// rssm_stream.h -- row streaming helpers shared by the ReplaySSM kernels and
// the conventional baselines: 16-byte-per-lane row loads in each storage
// format, reduced-row placement, and read-copy quantisation of fp32 rows.
#pragma once
#include "rssm_device.h"
#include "rssm_args.h"

namespace rssm {

// ------------------------------------------------------------------------
// Checkpoint read formats (16 bytes per lane per row).
// ------------------------------------------------------------------------
template <int RC> struct Ck;
template <> struct Ck<RC_NONE> {
    static constexpr int EPL = 4, ESZ = 4;
    static __device__ __forceinline__ void decode(const u32x4& w, float* x) {
        x[0] = __uint_as_float(w.x); x[1] = __uint_as_float(w.y);
        x[2] = __uint_as_float(w.z); x[3] = __uint_as_float(w.w);
    }
};
template <> struct Ck<RC_BF16> {
    static constexpr int EPL = 8, ESZ = 2;
    static __device__ __forceinline__ void decode(const u32x4& w, float* x) {
        const uint32_t u[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            x[2 * i] = __uint_as_float(u[i] << 16);
            x[2 * i + 1] = __uint_as_float(u[i] & 0xffff0000u);
        }
    }
};
template <> struct Ck<RC_FP8> {
    static constexpr int EPL = 16, ESZ = 1;
    static __device__ __forceinline__ void decode(const u32x4& w, float* x) {
        unpack4_e4m3(w.x, x); unpack4_e4m3(w.y, x + 4);
        unpack4_e4m3(w.z, x + 8); unpack4_e4m3(w.w, x + 12);
    }
};

template <> struct Ck<RC_F16> {
    static constexpr int EPL = 8;
    static __device__ __forceinline__ void decode(const u32x4& w, float* x) {
        const uint32_t u[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            x[2 * i] = (float)__builtin_bit_cast(_Float16, (uint16_t)(u[i] & 0xffffu));
            x[2 * i + 1] = (float)__builtin_bit_cast(_Float16, (uint16_t)(u[i] >> 16));
        }
    }
};

// MXFP4 (OCP microscaling): 32 E2M1 codes per 16 bytes, entry n of a row in
// byte n/2, low nibble first; one E8M0 exponent byte per block of 32 entries
// in a separate [rows][N/32] array.  A lane's 16 bytes are exactly one block,
// so the block scale is applied to the lane's partial dot product.
template <int SEL>
__device__ __forceinline__ void unpack2_e2m1(uint32_t w, float* x) {
    const f32x2 r = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, 1.0f, SEL);
    x[0] = r.x;
    x[1] = r.y;
}
__device__ __forceinline__ void unpack8_e2m1(uint32_t w, float* x) {
    unpack2_e2m1<0>(w, x); unpack2_e2m1<1>(w, x + 2);
    unpack2_e2m1<2>(w, x + 4); unpack2_e2m1<3>(w, x + 6);
}
template <> struct Ck<RC_MXFP4> {
    static constexpr int EPL = 32;
    static __device__ __forceinline__ void decode(const u32x4& w, float* x) {
        unpack8_e2m1(w.x, x); unpack8_e2m1(w.y, x + 8);
        unpack8_e2m1(w.z, x + 16); unpack8_e2m1(w.w, x + 24);
    }
};

// Bytes of one state row in read format RC (host and device).
__host__ __device__ constexpr long copy_row_bytes(int rc, int N) {
    return rc == RC_NONE ? 4L * N : (rc == RC_BF16 || rc == RC_F16) ? 2L * N : rc == RC_FP8 ? (long)N : (long)N / 2;
}
// Bytes of one checkpoint row, and the read format of the checkpoint itself.
// An fp8 row is N e4m3 codes and a 16-byte trailer whose first 4 bytes hold
// the row's fp32 scale; an fp8 checkpoint is always read through a copy.
__host__ __device__ constexpr long ck_row_bytes(int ck, int N) {
    return ck == CK_F16 ? 2L * N : ck == CK_FP8 ? (long)N + 16 : 4L * N;
}
__host__ __device__ constexpr int ck_read_format(int ck) { return ck == CK_F16 ? RC_F16 : RC_NONE; }
// Bytes of one state row's scales: fp32 per row (fp8), one E8M0 byte per 32
// entries (MXFP4), none otherwise.
__host__ __device__ constexpr long scale_row_bytes(int rc, int N) {
    return rc == RC_FP8 ? 4L : rc == RC_MXFP4 ? (long)N / 32 : 0L;
}

// Rows per thread per chunk when streaming the read format.
template <int RC> struct ReadU { static constexpr int U = 4; };
template <> struct ReadU<RC_BF16> { static constexpr int U = 4; };
template <> struct ReadU<RC_FP8> { static constexpr int U = 2; };
template <> struct ReadU<RC_MXFP4> { static constexpr int U = 2; };
template <> struct ReadU<RC_F16> { static constexpr int U = 4; };

__device__ __forceinline__ u32x4 ld16(const void* p) {
    return __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
}
__device__ __forceinline__ void st16(void* p, const u32x4& v) {
    __builtin_nontemporal_store(v, reinterpret_cast<u32x4*>(p));
}

// Load `cnt` input elements (cnt = 4 or a multiple of 4) of the input dtype.
template <int IN, int CNT>
__device__ __forceinline__ void load_in(const void* base, long idx, float* out) {
#pragma unroll
    for (int i = 0; i < CNT; i += 4) InVec4<IN>::load(base, idx + i, out + i);
}

// Tile geometry of the baseline kernels (tiles inside one key group).
struct Tile {
    int b, tile, vh0, kh, cidx;
    bool kwriter;
};
template <class Args>
__device__ __forceinline__ Tile tile_of(const Args& A) {
    Tile t;
    const int lin = blockIdx.x;
    t.b = lin / A.tiles;
    t.tile = lin - t.b * A.tiles;
    t.vh0 = t.tile * A.hvpt;
    t.kh = t.vh0 / A.g;
    t.kwriter = (t.vh0 % A.g) == 0;
    t.cidx = lin;
    return t;
}

// Stream U rows of a row-major [rows][N] matrix in format RC: lane `gl` of row
// group `rg` loads 16 bytes of row (c*U + u)*RPP + rg, RPP = TH / R rows per
// pass for TH threads.  A row past the tile re-reads row rows-1 and every
// caller discards its result: an unconditional load leaves the compiler no
// branch to wait inside.
template <int N, int RC, int U, int TH = RSSM_THREADS>
__device__ __forceinline__ void load_rows(u32x4 (&w)[U], const char* base, int chunk, int rows,
                                          int rg, int gl) {
    constexpr int R = N / Ck<RC>::EPL;
    constexpr int RPP = TH / R;
    constexpr int ROWB = R * 16;
#pragma unroll
    for (int u = 0; u < U; ++u) {
        const int row = (chunk * U + u) * RPP + rg;
        w[u] = ld16(base + (long)(row < rows ? row : rows - 1) * ROWB + gl * 16);
    }
}

// MXFP4 only: the E8M0 exponent byte of the block lane `gl` holds, for the
// same U rows as load_rows (rows past the tile re-read row rows-1).
template <int N, int RC, int U, int TH = RSSM_THREADS>
__device__ __forceinline__ void load_block_exp(int (&e)[U], const uint8_t* sb, int chunk, int rows,
                                               int rg, int gl) {
    if constexpr (RC == RC_MXFP4) {
        constexpr int R = N / 32, RPP = TH / R;
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int row = (chunk * U + u) * RPP + rg;
            e[u] = (int)sb[(long)(row < rows ? row : rows - 1) * R + gl];
        }
    }
}

// Apply lane gl's MXFP4 block scale 2^(E - 127) to its partial dot product.
template <int RC>
__device__ __forceinline__ float block_scaled(float s, int e) {
    if constexpr (RC == RC_MXFP4) return __builtin_amdgcn_ldexpf(s, e - 127);
    else return s;
}

// E2M1 code (4 bits) of a value already divided by its block scale: round to
// nearest, ties to the even code, saturate at 6; the sign bit is taken from
// `sgn` (the unscaled value), so a negative value that rounds to 0 gives -0.
// The magnitude code counts the rounding thresholds at or below |y|.
__device__ __forceinline__ uint32_t e2m1_code(float y, float sgn) {
    const float a = fabsf(y);
    const uint32_t m = (uint32_t)(a > 0.25f) + (uint32_t)(a >= 0.75f) + (uint32_t)(a > 1.25f) +
                       (uint32_t)(a >= 1.75f) + (uint32_t)(a > 2.5f) + (uint32_t)(a >= 3.5f) +
                       (uint32_t)(a > 5.0f);
    return m | ((__float_as_uint(sgn) >> 28) & 8u);
}

// ------------------------------------------------------------------------
// Checkpoint rows in folds: lane gl4 of a row group of R4 = N/4 lanes holds
// entries [4 gl4, 4 gl4 + 4) of its row, in any storage format (16 bytes of
// fp32; 8 bytes of fp16 kept in .x/.y; 4 e4m3 codes in .x and the row's
// scale in .y).
// ------------------------------------------------------------------------
template <int N, int CK, int U>
__device__ __forceinline__ void load_ck_rows(u32x4 (&w)[U], const char* tile, int chunk, int rows, int rg,
                                             int gl) {
    constexpr int RPP4 = RSSM_THREADS / (N / 4);
#pragma unroll
    for (int u = 0; u < U; ++u) {
        const long r = (chunk * U + u) * RPP4 + rg;
        const long rr = r < rows ? r : rows - 1;                     // as load_rows: past the tile, row rows-1
        const long e = rr * N + gl * 4;
        if constexpr (CK == CK_F32) {
            w[u] = ld16(tile + e * 4);
        } else if constexpr (CK == CK_F16) {
            const u32x2 h = __builtin_nontemporal_load(reinterpret_cast<const u32x2*>(tile + e * 2));
            w[u] = u32x4{h.x, h.y, 0u, 0u};
        } else {
            const char* row = tile + rr * (N + 16);
            w[u] = u32x4{__builtin_nontemporal_load(reinterpret_cast<const uint32_t*>(row + gl * 4)),
                         *reinterpret_cast<const uint32_t*>(row + N), 0u, 0u};
        }
    }
}

template <int CK>
__device__ __forceinline__ f32x4 ck_values(const u32x4& w) {
    if constexpr (CK == CK_F32) {
        return f32x4{__uint_as_float(w.x), __uint_as_float(w.y), __uint_as_float(w.z), __uint_as_float(w.w)};
    } else if constexpr (CK == CK_FP8) {
        float x[4];
        unpack4_e4m3(w.x, x);
        const float sc = __uint_as_float(w.y);
        return f32x4{x[0] * sc, x[1] * sc, x[2] * sc, x[3] * sc};
    } else {
        return f32x4{(float)__builtin_bit_cast(_Float16, (uint16_t)(w.x & 0xffffu)),
                     (float)__builtin_bit_cast(_Float16, (uint16_t)(w.x >> 16)),
                     (float)__builtin_bit_cast(_Float16, (uint16_t)(w.y & 0xffffu)),
                     (float)__builtin_bit_cast(_Float16, (uint16_t)(w.y >> 16))};
    }
}

// pcg_hash of Jarzynski and Olano ("Hash Functions for GPU Rendering", JCGT
// 2020): one LCG step, then PCG's RXS-M-XS output permutation, on 32 bits.
__host__ __device__ constexpr uint32_t pcg_hash(uint32_t x) {
    const uint32_t state = x * 747796405u + 2891336453u;
    const uint32_t word = ((state >> ((state >> 28u) + 4u)) ^ state) * 277803737u;
    return (word >> 22u) ^ word;
}

// Stochastic-rounding key of one fold: pcg_hash chained over the layer seed
// s and the epoch E (the number of folds the tile stored before this one),
// key = h(lo(s) ^ h(hi(s) ^ h(lo(E) ^ h(hi(E))))).
__host__ __device__ constexpr uint32_t sr_fold_key(uint64_t seed, uint64_t epoch) {
    return pcg_hash((uint32_t)seed ^
                    pcg_hash((uint32_t)(seed >> 32) ^ pcg_hash((uint32_t)epoch ^ pcg_hash((uint32_t)(epoch >> 32)))));
}

// fp16 bits of x rounded stochastically with the 16-bit draw u: up to the
// next fp16 step iff u / 2^16 is below the dropped fraction p of the step at
// |x| (steps 2^(e-10), e = max(floor(log2|x|), -14)); finite values saturate
// at 65504; the sign of x kept; infinities stay infinite and NaN stays NaN
// (quiet).  Every step is exact in fp32.
__device__ __forceinline__ uint32_t f16_stochastic(float x, uint32_t u) {
    const uint32_t b = __float_as_uint(x) & 0x7fffffffu;
    const uint32_t E = b >> 23;
    const uint32_t sgn = (__float_as_uint(x) >> 16) & 0x8000u;
    if (E == 255u) return (b > 0x7f800000u ? 0x7e00u : 0x7c00u) | sgn;
    float r;
    if (E >= 113u && E <= 142u) {
        // fp16 normal range, 2^-14 <= |x| < 2^16: the step drops the low 13 of
        // the 23 fraction bits, p = low13 / 2^13, and u / 2^16 < p exactly
        // when (u >> 3) < low13; a carry into the exponent is the next binade.
        const uint32_t up = ((u >> 3) < (b & 0x1fffu)) ? 0x2000u : 0u;
        r = fminf(__uint_as_float((b & ~0x1fffu) + up), 65504.0f);
    } else {
        const float a = __uint_as_float(b);
        int e = (a > 0.0f) ? __builtin_amdgcn_frexp_expf(a) - 1 : -14;
        e = e < -14 ? -14 : e;
        const float m = __builtin_amdgcn_ldexpf(a, 10 - e);          // a / q, exact
        const float f = floorf(m);
        const float p = m - f;
        const float up = ((float)u * (1.0f / 65536.0f) < p) ? 1.0f : 0.0f;
        r = fminf(__builtin_amdgcn_ldexpf(f + up, e - 10), 65504.0f);
    }
    const uint32_t h = __builtin_bit_cast(uint16_t, (_Float16)r);   // exact: r is an fp16 value
    return h | sgn;
}

// The fp8 checkpoint's row scale from the row's largest magnitude (see
// ck_row_scale).
__device__ __forceinline__ float fp8_row_scale_of(float amax) {
    if (!(amax > 0.0f)) return 1.0f;
    if (amax > 3.4028235e38f) return __builtin_inff();
    const int E = __builtin_amdgcn_frexp_expf(amax) - 1;                      // amax = m 2^E, m in [1, 2)
    const float m = __builtin_amdgcn_ldexpf(amax, -E);
    int s = E - 8 + (m > 1.75f ? 1 : 0);
    s = s < -126 ? -126 : (s > 127 ? 127 : s);
    return __builtin_amdgcn_ldexpf(1.0f, s);
}

// e4m3fn code of y (a value already divided by its row scale) rounded
// stochastically with the 16-bit draw u: up to the next e4m3 step iff
// u / 2^16 is below the dropped fraction p of the step at |y| (steps
// 2^(e-3), e = max(floor(log2|y|), -6)); saturating at 448, the sign of y
// kept.  e4m3fn has no infinity: a non-finite y gives the NaN code 0x7f.
// Every step is exact in fp32, and the rounded value converts exactly.
__device__ __forceinline__ uint32_t f8_stochastic(float y, uint32_t u) {
    const uint32_t b = __float_as_uint(y) & 0x7fffffffu;
    const uint32_t E = b >> 23;
    float r;
    if (E >= 121u && E <= 135u) {
        // e4m3 normal range, 2^-6 <= |y| < 2^9: the step drops the low 20 of
        // the 23 fraction bits, p = low20 / 2^20, and u / 2^16 < p exactly
        // when (u << 4) < low20; a carry into the exponent is the next binade.
        const uint32_t up = ((u << 4) < (b & 0xfffffu)) ? 0x100000u : 0u;
        r = fminf(__uint_as_float((b & ~0xfffffu) + up), 448.0f);
    } else if (E < 121u) {
        // below 2^-6 the step stays 2^-9
        const float m = __builtin_amdgcn_ldexpf(__uint_as_float(b), 9);      // |y| / 2^-9, exact
        const float f = floorf(m);
        const float up = ((float)u * (1.0f / 65536.0f) < m - f) ? 1.0f : 0.0f;
        r = __builtin_amdgcn_ldexpf(f + up, -9);
    } else if (E < 255u) {
        r = 448.0f;                                                           // beyond 2^9: saturate
    } else {
        return 0x7fu;                                                         // inf or NaN
    }
    r = copysignf(r, y);
    return (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(r, r, 0, false) & 0xffu;
}

// Scale of an fp8 checkpoint row held 4 entries per lane by the R4 = N/4
// lanes of a row group: 2^s, the smallest power of two with amax <= 448 2^s
// (amax = m 2^E, m in [1, 2): s = E - 8, plus 1 if m > 1.75; s in
// [-126, 127]); 1 for a row with no nonzero entry (NaN entries are ignored
// by the max), +inf for a row with an infinite entry; 1 for the other
// formats.  Every lane of the group takes part.
template <int N, int CK>
__device__ __forceinline__ float ck_row_scale(const f32x4& s) {
    if constexpr (CK == CK_FP8) {
        float m = fmaxf(fmaxf(fabsf(s.x), fabsf(s.y)), fmaxf(fabsf(s.z), fabsf(s.w)));
        m = group_max<N / 4>(m);
        return fp8_row_scale_of(m);
    } else {
        return 1.0f;
    }
}

// Store 4 entries of a checkpoint row.  fp16 and fp8: stochastic rounding
// with the draws of flat entry index g0 .. g0 + 3 (g0 a multiple of 4, so two
// hashes: pair (g0 >> 1) and the next; low half of a hash for the even
// entry); fp8 codes of y = x / sig, sig the row's power-of-two scale
// (ck_row_scale), which the row's lane 0 (gl == 0) stores in the trailer.
template <int N, int CK>
__device__ __forceinline__ void store_ck4(char* tile, int row, int gl, const f32x4& s, uint32_t key, long g0,
                                          float sig) {
    if constexpr (CK == CK_F32) {
        st16(tile + ((long)row * N + gl * 4) * 4,
             u32x4{__float_as_uint(s.x), __float_as_uint(s.y), __float_as_uint(s.z), __float_as_uint(s.w)});
    } else if constexpr (CK == CK_F16) {
        const uint32_t pair = (uint32_t)(g0 >> 1);
        const uint32_t w0 = pcg_hash(key ^ pair), w1 = pcg_hash(key ^ (pair + 1u));
        const uint32_t h0 = f16_stochastic(s.x, w0 & 0xffffu), h1 = f16_stochastic(s.y, w0 >> 16);
        const uint32_t h2 = f16_stochastic(s.z, w1 & 0xffffu), h3 = f16_stochastic(s.w, w1 >> 16);
        __builtin_nontemporal_store(u32x2{h0 | (h1 << 16), h2 | (h3 << 16)},
                                    reinterpret_cast<u32x2*>(tile + ((long)row * N + gl * 4) * 2));
    } else {
        // y = x / sig: sig is a power of two, so a multiplication by its exact
        // reciprocal (an infinite sig: finite entries give +-0, others NaN)
        const bool inf_row = sig > 3.4028235e38f;
        const float inv = inf_row ? 0.0f : __builtin_amdgcn_ldexpf(1.0f, 1 - __builtin_amdgcn_frexp_expf(sig));
        const auto y = [&](float x) { return inf_row ? x / sig : x * inv; };
        const uint32_t pair = (uint32_t)(g0 >> 1);
        const uint32_t w0 = pcg_hash(key ^ pair), w1 = pcg_hash(key ^ (pair + 1u));
        const uint32_t c0 = f8_stochastic(y(s.x), w0 & 0xffffu), c1 = f8_stochastic(y(s.y), w0 >> 16);
        const uint32_t c2 = f8_stochastic(y(s.z), w1 & 0xffffu), c3 = f8_stochastic(y(s.w), w1 >> 16);
        char* rowp = tile + (long)row * (N + 16);
        __builtin_nontemporal_store(c0 | (c1 << 8) | (c2 << 16) | (c3 << 24),
                                    reinterpret_cast<uint32_t*>(rowp + gl * 4));
        if (gl == 0) *reinterpret_cast<float*>(rowp + N) = sig;
    }
}

// Store the U reduced dot products of a chunk into y[row] (times the row
// scale for fp8).  Layout of the reduced values: see group_transpose_reduce.
template <int N, int RC, int U, bool SCALED = (RC == RC_FP8), int TH = RSSM_THREADS>
__device__ __forceinline__ void put_rows(float (&v)[U], float* y, int chunk, int rows, int rg,
                                         int gl, const float* scale_tile) {
    constexpr int R = N / Ck<RC>::EPL;
    constexpr int RPP = TH / R;
    if constexpr (U >= R) {
#pragma unroll
        for (int i = 0; i < U / R; ++i) {
            const int u = gl * (U / R) + i;
            const int row = (chunk * U + u) * RPP + rg;
            if (row < rows) {
                float val = v[i];
                if constexpr (SCALED) val *= scale_tile[row];
                y[row] = val;
            }
        }
    } else {
        if (gl % (R / U) == 0) {
            const int u = gl / (R / U);
            const int row = (chunk * U + u) * RPP + rg;
            if (row < rows) {
                float val = v[0];
                if constexpr (SCALED) val *= scale_tile[row];
                y[row] = val;
            }
        }
    }
}

// Write the read copy of one fp32 row slice (4 values in lane gl4 of a row
// group of R4 lanes).  bf16: round to nearest even.  fp8: per-row scale
// amax/448 (1 for an all-zero row), codes = e4m3(x / scale).  MXFP4: per block
// of 32 entries (8 lanes) exponent e = floor(log2 amax) - 2 clamped to
// [-127, 127] (-127 for an all-zero block), codes = e2m1(x * 2^-e).
template <int N, int RC>
__device__ __forceinline__ void store_copy(const f32x4& s, void* rcopy_tile, void* rscale_tile,
                                           int row, int gl4, bool valid) {
    constexpr int R4 = N / 4;
    if constexpr (RC == RC_BF16) {
        if (!valid) return;
        const uint32_t lo = f32_to_bf16_bits(s.x) | (f32_to_bf16_bits(s.y) << 16);
        const uint32_t hi = f32_to_bf16_bits(s.z) | (f32_to_bf16_bits(s.w) << 16);
        *reinterpret_cast<u32x2*>(reinterpret_cast<uint16_t*>(rcopy_tile) + (long)row * N + gl4 * 4) =
            u32x2{lo, hi};
    } else if constexpr (RC == RC_FP8) {
        // all lanes of the row group join the max; only valid rows store
        float m = fmaxf(fmaxf(fabsf(s.x), fabsf(s.y)), fmaxf(fabsf(s.z), fabsf(s.w)));
        m = group_max<R4>(m);
        if (!valid) return;
        float sc = m / 448.0f;
        if (!(sc > 0.0f)) sc = 1.0f;
        const uint32_t code = pack4_e4m3(s.x / sc, s.y / sc, s.z / sc, s.w / sc);
        *reinterpret_cast<uint32_t*>(reinterpret_cast<uint8_t*>(rcopy_tile) + (long)row * N + gl4 * 4) = code;
        if (gl4 == 0) reinterpret_cast<float*>(rscale_tile)[row] = sc;
    } else if constexpr (RC == RC_MXFP4) {
        float m = fmaxf(fmaxf(fabsf(s.x), fabsf(s.y)), fmaxf(fabsf(s.z), fabsf(s.w)));
        m = group_max<8>(m);                                 // the 8 lanes of this block
        if (!valid) return;
        // frexp: m = f 2^x with f in [0.5, 1), so floor(log2 m) = x - 1
        int e = (m > 0.0f) ? __builtin_amdgcn_frexp_expf(m) - 1 - 2 : -127;
        e = e < -127 ? -127 : (e > 127 ? 127 : e);
        uint32_t codes;
        if (e > -127) {
            // gfx950 conversion of x / 2^e (2^e a normal float here): round to
            // nearest even, saturating, sign kept -- the encoding above
            const float sc = __builtin_amdgcn_ldexpf(1.0f, e);
            codes = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(0u, s.x, s.y, sc, 0);
            codes = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(codes, s.z, s.w, sc, 1);
        } else {
            codes = e2m1_code(__builtin_amdgcn_ldexpf(s.x, -e), s.x) | (e2m1_code(__builtin_amdgcn_ldexpf(s.y, -e), s.y) << 4) |
                    (e2m1_code(__builtin_amdgcn_ldexpf(s.z, -e), s.z) << 8) | (e2m1_code(__builtin_amdgcn_ldexpf(s.w, -e), s.w) << 12);
        }
        *reinterpret_cast<uint16_t*>(reinterpret_cast<uint8_t*>(rcopy_tile) + (long)row * (N / 2) + gl4 * 2) =
            (uint16_t)codes;
        if (gl4 % 8 == 0)
            reinterpret_cast<uint8_t*>(rscale_tile)[(long)row * (N / 32) + gl4 / 8] = (uint8_t)(e + 127);
    }
}

}  // namespace rssm
