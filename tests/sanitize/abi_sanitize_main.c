/* Drives the host side of the C ABI (include/replayssm.h) with no GPU: size
 * queries over many shapes (valid and invalid), handle creation and
 * destruction with aligned host addresses standing in for device buffers, and
 * calls that every entry point rejects before any HIP call.  Built with
 * AddressSanitizer and UBSan on the host pass only, so out-of-bounds accesses,
 * leaks of handles and undefined arithmetic in the host code abort the run. */
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "replayssm.h"
#include "rssm_probes.h"

static int fails = 0;
#define EXPECT(cond) do { if (!(cond)) { printf("FAIL line %d: %s\n", __LINE__, #cond); ++fails; } } while (0)

static rssm_config cfg_of(int B, int Hv, int Hk, int P, int N, int L, int T, int in, int rc, int hvpt, int ck) {
    rssm_config c;
    memset(&c, 0, sizeof c);
    c.batch = B; c.n_vheads = Hv; c.n_kheads = Hk; c.dim_v = P; c.dim_k = N; c.window = L;
    c.max_draft = T; c.in_dtype = in; c.read_copy = rc; c.heads_per_tile = hvpt; c.ckpt_fmt = ck; c.sr_seed = 7;
    return c;
}

int main(void) {
    EXPECT(replayssm_version() != NULL && strlen(replayssm_version()) > 0);
    /* size queries over a grid of shapes; sizes must be positive where required */
    const int Ns[] = {16, 32, 64, 128, 256, 48};
    const int Ps[] = {4, 16, 64, 128, 256, 6};
    int ok = 0, rejected = 0;
    for (int in = 0; in < 2; ++in)
        for (int rc = 0; rc < 4; ++rc)
            for (int ck = 0; ck < 3; ++ck)
                for (int ni = 0; ni < 6; ++ni)
                    for (int pi = 0; pi < 6; ++pi)
                        for (int g = 1; g <= 4; g *= 2) {
                            rssm_config c = cfg_of(3, 4 * g, 4, Ps[pi], Ns[ni], 16, 4, in, rc, 0, ck);
                            size_t sz[RSSM_NUM_BUFS];
                            int32_t tiles = -1;
                            rssm_status s = replayssm_query_sizes(&c, sz, &tiles);
                            if (s == RSSM_OK) {
                                ++ok;
                                EXPECT(tiles > 0 && sz[RSSM_BUF_CKPT] > 0 && sz[RSSM_BUF_COUNT] > 0);
                                /* fp8 checkpoint: rows of N + 16 bytes and a fold-epoch word per tile */
                                if (ck == RSSM_CKPT_FP8_SR)
                                    EXPECT(rc != RSSM_READ_NONE &&
                                           sz[RSSM_BUF_CKPT] == (size_t)3 * c.n_vheads * c.dim_v * (c.dim_k + 16) &&
                                           sz[RSSM_BUF_FOLDS] == (size_t)3 * tiles * 4);
                            } else {
                                ++rejected;
                            }
                        }
    EXPECT(ok > 0 && rejected > 0);
    rssm_config bad = cfg_of(0, 4, 4, 16, 16, 16, 0, 0, 0, 0, 0);
    size_t sz[RSSM_NUM_BUFS];
    EXPECT(replayssm_query_sizes(&bad, sz, NULL) != RSSM_OK);
    EXPECT(replayssm_query_sizes(NULL, sz, NULL) == RSSM_EINVAL);

    /* create / destroy with aligned host stand-ins; misaligned pointers rejected */
    unsigned char* mem = aligned_alloc(64, 1 << 16);
    if (!mem) return 2;
    for (int round = 0; round < 50; ++round) {
        rssm_config c = cfg_of(2, 2, 2, 16, 16, 16, 4, 0, round % 2 ? RSSM_READ_FP8_ROW : RSSM_READ_NONE, 0, 0);
        rssm_buffers b;
        b.ckpt = mem; b.read_copy = mem + 1024; b.row_scale = mem + 2048; b.kbuf = mem + 3072;
        b.vbuf = mem + 4096; b.abuf = (float*)(mem + 5120); b.count = (int32_t*)(mem + 6144);
        b.err = (int32_t*)(mem + 7168); b.work = (int32_t*)(mem + 8192); b.folds = NULL;
        if (c.read_copy == RSSM_READ_NONE) { b.read_copy = NULL; b.row_scale = NULL; }
        replayssm_t h = NULL;
        EXPECT(replayssm_create(&c, &b, &h) == RSSM_OK && h != NULL);
        /* rejected before any HIP call */
        EXPECT(replayssm_decode_step(h, NULL, mem, mem, mem, (float*)mem, NULL) == RSSM_EINVAL);
        EXPECT(replayssm_decode_step(h, (const float*)(mem + 4), mem, mem, mem, (float*)mem, NULL) == RSSM_EINVAL);
        EXPECT(replayssm_spec_verify(h, 0, (const float*)mem, mem, mem, mem, (float*)mem, NULL) == RSSM_EINVAL);
        EXPECT(replayssm_spec_verify(h, 5, (const float*)mem, mem, mem, mem, (float*)mem, NULL) == RSSM_EINVAL);
        EXPECT(replayssm_commit(h, (const int32_t*)mem, NULL) == RSSM_ESTATE);
        EXPECT(replayssm_commit(h, NULL, NULL) == RSSM_EINVAL);
        EXPECT(replayssm_commit_static(h, (const int32_t*)mem, NULL) == RSSM_ESTATE);
        EXPECT(replayssm_commit_static(h, (const int32_t*)(mem + 4), NULL) == RSSM_EINVAL);
        EXPECT(replayssm_prefill(h, 0, (const float*)mem, mem, mem, mem, (float*)mem, NULL) == RSSM_EINVAL);
        EXPECT(replayssm_read_error(h, NULL, 0, NULL) == RSSM_EINVAL);
        EXPECT(replayssm_destroy(h) == RSSM_OK);
        b.kbuf = mem + 3072 + 4;
        h = (replayssm_t)1;
        EXPECT(replayssm_create(&c, &b, &h) == RSSM_EINVAL && h == NULL);
        /* an fp16 checkpoint needs the fold-epoch buffer, 16-byte aligned */
        b.kbuf = mem + 3072;
        c.ckpt_fmt = RSSM_CKPT_F16_SR;
        EXPECT(replayssm_create(&c, &b, &h) == RSSM_EINVAL && h == NULL);
        b.folds = (uint32_t*)(mem + 9216 + 4);
        EXPECT(replayssm_create(&c, &b, &h) == RSSM_EINVAL && h == NULL);
        b.folds = (uint32_t*)(mem + 9216);
        EXPECT(replayssm_create(&c, &b, &h) == RSSM_OK && h != NULL);
        EXPECT(replayssm_destroy(h) == RSSM_OK);
    }
    EXPECT(replayssm_destroy(NULL) == RSSM_EINVAL);
    /* baselines and probes: argument checks only */
    rssm_config c = cfg_of(2, 2, 2, 16, 16, 16, 4, 0, 0, 0, 0);
    EXPECT(convssm_decode_step(&c, NULL, NULL, 0, (const float*)mem, mem, mem, mem, (float*)mem, NULL) == RSSM_EINVAL);
    EXPECT(convssm_commit(&c, (int32_t*)mem, (const int32_t*)mem, 0, (int32_t*)mem, NULL) == RSSM_EINVAL);
    EXPECT(rssm_probe_copy(mem, mem, 17, NULL) == RSSM_EINVAL);
    EXPECT(rssm_probe_read_chunked(mem, 32768 + 16, mem, 0, (float*)mem, NULL) == RSSM_EINVAL);
    free(mem);
    printf("fails %d, shapes accepted %d rejected %d\n", fails, ok, rejected);
    return fails == 0 ? 0 : 1;
}
