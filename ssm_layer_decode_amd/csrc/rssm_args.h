// rssm_args.h -- kernel argument blocks shared by the host launcher and the
// kernels.  Plain data, passed by value as the kernel's single argument.
#pragma once
#include <stdint.h>

namespace rssm {

struct StepArgs {
    // caller-owned buffers of a handle
    float*   ckpt;      // [B][Hv][P][N] fp32, or fp16 bits (fp16 checkpoint)
    void*    rcopy;     // read copy (bf16 / e4m3 / E2M1 codes), or null
    float*   rscale;    // fp8 row scales or MXFP4 E8M0 bytes, or null
    void*    kbuf;      // [B][Hk][C][N] in_dtype
    void*    vbuf;      // [B][Hv][C][P] in_dtype
    float*   abuf;      // [B][Hv][C]
    int32_t* count;     // [B][tiles]
    int32_t* err;       // [1]
    int32_t* work;      // commit: [0] listed tiles (cleared by verify), [1] unused, [2..] tile list
    uint32_t* folds;    // [B][tiles] folds stored per tile (fp16 checkpoint's rounding epoch), or null
    // per-call inputs / outputs
    const float*   alpha;     // decode [B][Hv]; verify [B][T][Hv]
    const void*    k;         // decode [B][Hk][N]; verify [B][T][Hk][N]
    const void*    v;         // decode [B][Hv][P]; verify [B][T][Hv][P]
    const void*    q;         // as k
    float*         o;         // decode [B][Hv][P]; verify [B][T][Hv][P]
    const int32_t* accepted;  // commit [B]
    const int32_t* seq_ids;   // reset (null = all)
    // sizes
    int B, Hv, Hk, P, L, C, g, hvpt, tiles;
    int ctiles, chvpt;  // the tiling of the pointer copies count[B][ctiles] (decode's tile)
    int T;          // verify/commit: drafts of the pending verify
    int mode;       // reset: number of ids
    uint64_t sr_seed; // fp16 checkpoint: seed of the stochastic rounding
};

struct ConvArgs {
    void*          state;     // [B][Hv][P][N] (fp32 / bf16 / e4m3)  or snapshot ring
    float*         rscale;    // [B][Hv][P] (fp8 state), or null
    const int32_t* cur;       // snapshot ring index [B]
    int32_t*       cur_rw;    // commit
    const int32_t* accepted;
    int32_t*       err;
    const float*   alpha;
    const void*    k;
    const void*    v;
    const void*    q;
    float*         o;
    int B, Hv, Hk, P, g, hvpt, tiles, T, ring;
};

}  // namespace rssm
