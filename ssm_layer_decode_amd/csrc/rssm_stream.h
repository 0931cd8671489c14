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

// Rows per thread per chunk when streaming the read format.
template <int RC> struct ReadU { static constexpr int U = 4; };
template <> struct ReadU<RC_BF16> { static constexpr int U = 4; };
template <> struct ReadU<RC_FP8> { static constexpr int U = 2; };

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
// group `rg` loads 16 bytes of row (c*U + u)*RPP + rg.
template <int N, int RC, int U>
__device__ __forceinline__ void load_rows(u32x4 (&w)[U], const char* base, int chunk, int rows,
                                          int rg, int gl) {
    constexpr int R = N / Ck<RC>::EPL;
    constexpr int RPP = RSSM_THREADS / R;
    constexpr int ROWB = N * Ck<RC>::ESZ;
#pragma unroll
    for (int u = 0; u < U; ++u) {
        const int row = (chunk * U + u) * RPP + rg;
        if (row < rows) w[u] = ld16(base + (long)row * ROWB + gl * 16);
        else w[u] = u32x4{0u, 0u, 0u, 0u};
    }
}

// Store the U reduced dot products of a chunk into y[row] (times the row
// scale for fp8).  Layout of the reduced values: see group_transpose_reduce.
template <int N, int RC, int U, bool SCALED = (RC == RC_FP8)>
__device__ __forceinline__ void put_rows(float (&v)[U], float* y, int chunk, int rows, int rg,
                                         int gl, const float* scale_tile) {
    constexpr int R = N / Ck<RC>::EPL;
    constexpr int RPP = RSSM_THREADS / R;
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
// amax/448 (1 for an all-zero row), codes = e4m3(x / scale).
template <int N, int RC>
__device__ __forceinline__ void store_copy(const f32x4& s, void* rcopy_tile, float* rscale_tile,
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
        if (gl4 == 0) rscale_tile[row] = sc;
    }
}

}  // namespace rssm
