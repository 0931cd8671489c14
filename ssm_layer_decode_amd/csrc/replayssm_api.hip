// replayssm_api.hip -- the C ABI declared in include/replayssm.h: argument
// validation (always before any HIP call), tiling and LDS sizing, the host
// state machine of verify -> commit, and kernel launches on the caller's stream.
#include <hip/hip_runtime.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#include "replayssm.h"
#include "rssm_args.h"
#include "rssm_launch.h"
#include "rssm_stream.h"

using namespace rssm;

struct replayssm {
    rssm_config cfg;
    rssm_buffers buf;
    int hvpt, tiles, C;
    int vhvpt;         // value heads per verify workgroup
    int pending_T;     // -1: no verify pending
};

static_assert(RSSM_READ_NONE == RC_NONE && RSSM_READ_BF16 == RC_BF16 && RSSM_READ_FP8_ROW == RC_FP8 &&
                  RSSM_READ_MXFP4 == RC_MXFP4, "read-copy codes of the ABI and the kernels differ");

namespace {

constexpr size_t kMaxLds = 64 * 1024;

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

bool key_dim_ok(int n) { return n == 16 || n == 32 || n == 64 || n == 128 || n == 256; }

int round4(int x) { return (x + 3) & ~3; }

int group_of(const rssm_config* c) { return c->n_vheads / c->n_kheads; }

int ck_of(const rssm_config* c) {
    return c->ckpt_fmt == RSSM_CKPT_F16_SR ? CK_F16 : c->ckpt_fmt == RSSM_CKPT_FP8_SR ? CK_FP8 : CK_F32;
}

// Default value heads per workgroup inside one key group: the largest divisor
// of the group size whose tile has at most 128 state rows (256-row tiles halve
// the workgroups and measured equal or slower for fp32 and bf16 reads; the
// copy widening below restores them where the reads are narrower).
int default_hvpt(const rssm_config* c) {
    const int g = group_of(c);
    int best = 1;
    for (int d = 1; d <= g; ++d)
        if (g % d == 0 && d * c->dim_v <= 128) best = d;
    return best;
}

// A tile is part of one key group (hvpt divides g) or whole key groups
// (g divides hvpt, hvpt divides Hv).
bool tile_ok(const rssm_config* c, int hvpt) {
    const int g = group_of(c);
    if (hvpt < 1 || hvpt * c->dim_v > 1024) return false;
    return (g % hvpt == 0) || (hvpt % g == 0 && c->n_vheads % hvpt == 0);
}

int kgpt_of(const rssm_config* c, int hvpt) { return hvpt >= group_of(c) ? hvpt / group_of(c) : 1; }

size_t decode_lds_w(const rssm_config* c, int hvpt, int L) {
    const int N = c->dim_k, P = c->dim_v, kg = kgpt_of(c, hvpt);
    return (size_t)(kg * N + kg * L * N + hvpt * L * P + hvpt * round4(L) + kg * round4(L) +
                    round4(hvpt * P) + hvpt) * 4;
}

size_t decode_lds(const rssm_config* c, int hvpt) { return decode_lds_w(c, hvpt, c->window); }

size_t fold_lds(const rssm_config* c, int hvpt) { return decode_lds_w(c, hvpt, c->window + c->max_draft); }

int verify_tt(int T) { return T <= 1 ? 1 : T <= 2 ? 2 : T <= 4 ? 4 : 8; }

// Format non-flush steps and verify read: the copy, or the checkpoint's own.
int read_fmt(const rssm_config* c) {
    return c->read_copy != RSSM_READ_NONE ? c->read_copy : ck_read_format(ck_of(c));
}

size_t verify_lds_reg(const rssm_config* c, int hvpt, int tt) {
    const int C = c->window + c->max_draft, P = c->dim_v, rows = hvpt * P;
    return (size_t)(hvpt * C * P + hvpt * round4(C) + C * tt + tt * rows) * 4;
}

size_t verify_lds_staged(const rssm_config* c, int hvpt, int tt) {
    const int C = c->window + c->max_draft, N = c->dim_k, P = c->dim_v, rows = hvpt * P;
    const int kg = kgpt_of(c, hvpt), CS = round4(C);
    return (size_t)(kg * tt * N + kg * C * N + hvpt * C * P + hvpt * CS + kg * CS * tt + tt * rows) * 4;
}

// Verify kernel.  Tiles of several key groups and MXFP4 reads (32 entries per
// lane) stage the queries in LDS.  Inside one key group the queries can stay in
// registers, TT x (entries per lane) floats: with fp32 inputs and a bf16, fp16
// or fp8 read, 16 or more of those cost more occupancy than the LDS re-reads
// (measured 5-46 % slower), so such tiles stage too where the staged regions
// fit; bf16 inputs, and fp32 reads of fp32 inputs, measured faster in registers.
bool verify_staged(const rssm_config* c, int hvpt, int tt) {
    if (hvpt > group_of(c) || c->read_copy == RSSM_READ_MXFP4) return true;
    const int rd = read_fmt(c);
    if (c->in_dtype != RSSM_F32 || rd == RC_NONE) return false;
    const int epl = rd == RC_FP8 ? 16 : 8;
    return tt * epl >= 16 && verify_lds_staged(c, hvpt, tt) <= kMaxLds;
}

size_t verify_lds(const rssm_config* c, int hvpt, int tt) {
    return verify_staged(c, hvpt, tt) ? verify_lds_staged(c, hvpt, tt) : verify_lds_reg(c, hvpt, tt);
}

// Tiles of more than one key group take the staged-query kernel variants.
bool multi_of(const rssm_config* c, int hvpt) { return hvpt > group_of(c); }

// Decode of two-head tiles whose non-flush steps read an MXFP4 copy, or an
// fp8 copy of heads of at most 64 rows: each head on 128 threads of its own
// (rssm_decode_split.hip).  Windows up to 16 records, key dims 64 and 128, at
// most 128 rows per head.  Measured against the tile-wide decode on two-head
// tiles, bf16 copies gained 3 % and an fp16 checkpoint read directly lost 8 %
// at the Mamba-2 shape; both keep the tile-wide decode, as do fp8 copies of
// 128-row heads (28 -> 30 us per step at 64 heads of P = N = 128).
bool split_ok(const rssm_config* c, int hvpt) {
    const bool fmt = c->read_copy == RSSM_READ_MXFP4 || (c->read_copy == RSSM_READ_FP8_ROW && c->dim_v <= 64);
    return fmt && hvpt == 2 && c->window <= 16 && (c->dim_k == 64 || c->dim_k == 128) && c->dim_v <= 128;
}

// Shared memory of that path's non-flush steps:
// q [2][N] | scores [2][16] | decays [2][16] | outputs [2][P] | values [2][L][P].
size_t split_lds(const rssm_config* c) {
    return (size_t)(2 * c->dim_k + 4 * 16 + 2 * c->dim_v + 2 * c->window * c->dim_v) * 4;
}

size_t conv_lds(int hvpt, int P) { return (size_t)(2 * hvpt * P + round4(hvpt)) * 4; }

size_t conv_verify_lds(int hvpt, int P, int tt) { return (size_t)tt * (2 * hvpt * P + round4(hvpt)) * 4; }

// Shape checks shared by every entry point.  Returns RSSM_OK or an error.
rssm_status check_shape(const rssm_config* c, bool need_window) {
    if (!c) return RSSM_EINVAL;
    if (c->batch < 1 || c->n_vheads < 1 || c->n_kheads < 1 || c->n_vheads % c->n_kheads != 0)
        return RSSM_EINVAL;
    if (c->dim_v < 4 || c->dim_v > 256 || c->dim_v % 4 != 0) return RSSM_EINVAL;
    if (c->dim_k < 1) return RSSM_EINVAL;
    if (!key_dim_ok(c->dim_k)) return RSSM_EUNSUPPORTED;
    if (c->in_dtype != RSSM_F32 && c->in_dtype != RSSM_BF16) return RSSM_EINVAL;
    if (need_window) {
        if (c->window < 1 || c->window > 32) return RSSM_EINVAL;
        if (c->max_draft < 0 || c->max_draft > 8) return RSSM_EINVAL;
        if (c->read_copy < RSSM_READ_NONE || c->read_copy > RSSM_READ_MXFP4) return RSSM_EINVAL;
        if (c->read_copy == RSSM_READ_MXFP4 && c->dim_k < 32) return RSSM_EUNSUPPORTED;
        if (c->ckpt_fmt != RSSM_CKPT_F32 && c->ckpt_fmt != RSSM_CKPT_F16_SR && c->ckpt_fmt != RSSM_CKPT_FP8_SR)
            return RSSM_EINVAL;
        // an fp8 checkpoint is read through a copy only
        if (c->ckpt_fmt == RSSM_CKPT_FP8_SR && c->read_copy == RSSM_READ_NONE) return RSSM_EUNSUPPORTED;
        // stochastic rounding hashes entry pairs with 32-bit indices
        if (c->ckpt_fmt != RSSM_CKPT_F32 &&
            (double)c->batch * c->n_vheads * c->dim_v * c->dim_k >= 8589934592.0)
            return RSSM_EUNSUPPORTED;
    }
    if (c->heads_per_tile < 0) return RSSM_EINVAL;
    if (c->heads_per_tile > 0 && !tile_ok(c, c->heads_per_tile)) return RSSM_EINVAL;
    if ((long)c->batch * (c->n_vheads) > (1L << 30)) return RSSM_EINVAL;
    return RSSM_OK;
}

// Value heads per tile.  Default: the in-group tile above; when non-flush
// steps read fewer than 4 bytes per state entry (a read copy, or an fp16
// checkpoint without one) a tile of less than 32 KiB of such data is
// widened by whole tiles while its decode LDS stays within 28 KiB and it has at
// most 256 rows -- small tiles leave too little of the copy in flight per
// workgroup, large LDS footprints cut the workgroups per CU.  Only MXFP4 reads
// (4 KiB per 64-row head) widen past one key group: for bf16, fp16 and fp8 the
// one-group tile, whose scores come straight from the key loads, measured
// faster than a tile of two groups staging keys and queries in LDS.
// (The verify tile: decode's own split preference below does not apply.)
int verify_hvpt_of(const rssm_config* c) {
    if (c->heads_per_tile > 0) return c->heads_per_tile;
    int hv = default_hvpt(c);
    const int rd = read_fmt(c);
    if (rd == RC_NONE) return hv;
    const size_t rowb = (size_t)copy_row_bytes(rd, c->dim_k);
    while ((size_t)hv * c->dim_v * rowb < 32 * 1024) {
        const int next = 2 * hv;
        if (!tile_ok(c, next) || c->n_vheads % next != 0 || next * c->dim_v > 256 ||
            decode_lds(c, next) > 28 * 1024)
            break;
        if (rd != RC_MXFP4 && group_of(c) % next != 0) break;       // stays inside one key group
        hv = next;
    }
    return hv;
}

// Decode tile (and the tile of the per-tile pointer copies, flush and commit):
// the verify tile, except that MXFP4 copies, and fp8 copies of heads of at most
// 64 rows, take two-head tiles on the split decode where it applies (window
// averages at the Mamba-2 shape measured 114 -> 97 us for MXFP4 and 127 -> 117
// us for fp8; 29 -> 25 us for MXFP4 at 64 heads of P = N = 128, where fp8
// measured 28 -> 30 us and keeps its one-head tile).  Verification keeps its
// own tile: with two-head fp8 tiles it measured 10-20 % slower (the pointer
// copies of a sequence are all equal, so a verify tile reads any of them).
int hvpt_of(const rssm_config* c) {
    if (c->heads_per_tile > 0) return c->heads_per_tile;
    if (split_ok(c, 2) && tile_ok(c, 2) && c->n_vheads % 2 == 0 && decode_lds(c, 2) <= kMaxLds &&
        fold_lds(c, 2) <= kMaxLds)
        return 2;
    return verify_hvpt_of(c);
}

StepArgs base_args(const replayssm* h) {
    StepArgs a;
    memset(&a, 0, sizeof(a));
    a.ckpt = static_cast<float*>(h->buf.ckpt);
    a.rcopy = h->buf.read_copy;
    a.rscale = static_cast<float*>(h->buf.row_scale);
    a.kbuf = h->buf.kbuf;
    a.vbuf = h->buf.vbuf;
    a.abuf = h->buf.abuf;
    a.count = h->buf.count;
    a.err = h->buf.err;
    a.work = h->buf.work;
    a.folds = h->buf.folds;
    a.sr_seed = h->cfg.sr_seed;
    a.B = h->cfg.batch;
    a.Hv = h->cfg.n_vheads;
    a.Hk = h->cfg.n_kheads;
    a.P = h->cfg.dim_v;
    a.L = h->cfg.window;
    a.C = h->C;
    a.g = h->cfg.n_vheads / h->cfg.n_kheads;
    a.hvpt = h->hvpt;
    a.tiles = h->tiles;
    a.ctiles = h->tiles;
    a.chvpt = h->hvpt;
    return a;
}

rssm_status hip_status(hipError_t e) { return e == hipSuccess ? RSSM_OK : RSSM_EHIP; }

}  // namespace

extern "C" {

const char* replayssm_version(void) { return "replayssm-gfx950 " RSSM_ABI_VERSION; }

rssm_status replayssm_query_sizes(const rssm_config* cfg, size_t sizes[RSSM_NUM_BUFS], int32_t* tiles) {
    if (!sizes) return RSSM_EINVAL;
    const rssm_status s = check_shape(cfg, true);
    if (s != RSSM_OK) return s;
    const int hvpt = hvpt_of(cfg);
    if (decode_lds(cfg, hvpt) > kMaxLds || fold_lds(cfg, hvpt) > kMaxLds) return RSSM_EUNSUPPORTED;
    // a layer that speculates must also be able to verify max_draft drafts
    if (cfg->max_draft > 0 && verify_lds(cfg, verify_hvpt_of(cfg), verify_tt(cfg->max_draft)) > kMaxLds)
        return RSSM_EUNSUPPORTED;
    const size_t B = cfg->batch, Hv = cfg->n_vheads, Hk = cfg->n_kheads, P = cfg->dim_v, N = cfg->dim_k;
    const size_t C = cfg->window + cfg->max_draft;
    const size_t e = cfg->in_dtype == RSSM_BF16 ? 2 : 4;
    const int nt = cfg->n_vheads / hvpt;
    sizes[RSSM_BUF_CKPT] = B * Hv * P * (size_t)ck_row_bytes(ck_of(cfg), cfg->dim_k);
    sizes[RSSM_BUF_READ_COPY] = cfg->read_copy == RSSM_READ_NONE ? 0
                              : B * Hv * P * (size_t)copy_row_bytes(cfg->read_copy, cfg->dim_k);
    sizes[RSSM_BUF_ROW_SCALE] = B * Hv * P * (size_t)scale_row_bytes(cfg->read_copy, cfg->dim_k);
    sizes[RSSM_BUF_KBUF] = B * Hk * C * N * e;
    sizes[RSSM_BUF_VBUF] = B * Hv * C * P * e;
    sizes[RSSM_BUF_ABUF] = B * Hv * C * 4;
    sizes[RSSM_BUF_COUNT] = B * (size_t)nt * 4;
    sizes[RSSM_BUF_ERR] = 4;
    sizes[RSSM_BUF_WORK] = ((2 + B * (size_t)nt) * 4 + 15) / 16 * 16;
    sizes[RSSM_BUF_FOLDS] = cfg->ckpt_fmt != RSSM_CKPT_F32 ? B * (size_t)nt * 4 : 0;
    if (tiles) *tiles = nt;
    return RSSM_OK;
}

rssm_status replayssm_create(const rssm_config* cfg, const rssm_buffers* bufs, replayssm_t* out) {
    if (!out) return RSSM_EINVAL;
    *out = nullptr;
    size_t sizes[RSSM_NUM_BUFS];
    int32_t nt = 0;
    const rssm_status s = replayssm_query_sizes(cfg, sizes, &nt);
    if (s != RSSM_OK) return s;
    if (!bufs) return RSSM_EINVAL;
    const void* req[] = {bufs->ckpt, bufs->kbuf, bufs->vbuf, bufs->abuf, bufs->count, bufs->err};
    for (const void* p : req)
        if (!p || !aligned16(p)) return RSSM_EINVAL;
    if (bufs->work && !aligned16(bufs->work)) return RSSM_EINVAL;    // NULL: static commits only
    if (cfg->read_copy != RSSM_READ_NONE && (!bufs->read_copy || !aligned16(bufs->read_copy)))
        return RSSM_EINVAL;
    if ((cfg->read_copy == RSSM_READ_FP8_ROW || cfg->read_copy == RSSM_READ_MXFP4) &&
        (!bufs->row_scale || !aligned16(bufs->row_scale)))
        return RSSM_EINVAL;
    if (cfg->ckpt_fmt != RSSM_CKPT_F32 && (!bufs->folds || !aligned16(bufs->folds))) return RSSM_EINVAL;
    replayssm* h = static_cast<replayssm*>(calloc(1, sizeof(replayssm)));
    if (!h) return RSSM_EINVAL;
    h->cfg = *cfg;
    h->buf = *bufs;
    h->hvpt = hvpt_of(cfg);
    h->vhvpt = verify_hvpt_of(cfg);
    h->tiles = nt;
    h->C = cfg->window + cfg->max_draft;
    h->pending_T = -1;
    *out = h;
    return RSSM_OK;
}

rssm_status replayssm_destroy(replayssm_t h) {
    if (!h) return RSSM_EINVAL;
    free(h);
    return RSSM_OK;
}

rssm_status replayssm_reset(replayssm_t h, const int32_t* seq_ids, int32_t n, void* stream) {
    if (!h) return RSSM_EINVAL;
    if (h->pending_T >= 0) return RSSM_ESTATE;
    if (seq_ids && n < 0) return RSSM_EINVAL;
    const int count = seq_ids ? n : h->cfg.batch;
    if (count == 0) return RSSM_OK;
    StepArgs a = base_args(h);
    a.seq_ids = seq_ids;
    a.mode = count;
    const int rc = h->cfg.read_copy;
    return hip_status(launch_reset(a, h->cfg.dim_k, rc, ck_of(&h->cfg), count * h->tiles, (hipStream_t)stream));
}

rssm_status replayssm_refresh_read_copy(replayssm_t h, void* stream) {
    if (!h) return RSSM_EINVAL;
    if (h->cfg.read_copy == RSSM_READ_NONE) return RSSM_OK;
    StepArgs a = base_args(h);
    return hip_status(launch_refresh(a, h->cfg.dim_k, h->cfg.read_copy, ck_of(&h->cfg), h->cfg.batch * h->tiles,
                                     (hipStream_t)stream));
}

rssm_status replayssm_decode_step(replayssm_t h, const float* alpha, const void* k, const void* v,
                                  const void* q, float* o, void* stream) {
    if (!h) return RSSM_EINVAL;
    const void* req[] = {alpha, k, v, q, o};
    for (const void* p : req)
        if (!p || !aligned16(p)) return RSSM_EINVAL;
    if (h->pending_T >= 0) return RSSM_ESTATE;
    StepArgs a = base_args(h);
    a.alpha = alpha;
    a.k = k;
    a.v = v;
    a.q = q;
    a.o = o;
    const rssm_config* c = &h->cfg;
    const int grid = c->batch * h->tiles;
    if (split_ok(c, h->hvpt)) {
        // flush folds one head at a time: one head's records, or the non-flush staging
        const size_t lds = decode_lds(c, 1) > split_lds(c) ? decode_lds(c, 1) : split_lds(c);
        return hip_status(launch_decode_split(a, c->dim_k, c->in_dtype, c->read_copy, ck_of(c), grid, lds,
                                              (hipStream_t)stream));
    }
    return hip_status(launch_decode(a, c->dim_k, c->in_dtype, c->read_copy, multi_of(c, h->hvpt), ck_of(c), grid,
                                    decode_lds(c, h->hvpt), (hipStream_t)stream));
}

rssm_status replayssm_flush(replayssm_t h, void* stream) {
    if (!h) return RSSM_EINVAL;
    if (h->pending_T >= 0) return RSSM_ESTATE;
    StepArgs a = base_args(h);
    const rssm_status s = hip_status(launch_fold(a, h->cfg.dim_k, h->cfg.in_dtype, h->cfg.read_copy,
                                                 multi_of(&h->cfg, h->hvpt), ck_of(&h->cfg), h->cfg.batch * h->tiles,
                                                 fold_lds(&h->cfg, h->hvpt), (hipStream_t)stream));
    return s;
}

rssm_status replayssm_spec_verify(replayssm_t h, int32_t T, const float* alpha, const void* k,
                                  const void* v, const void* q, float* o, void* stream) {
    if (!h) return RSSM_EINVAL;
    if (T < 1 || T > h->cfg.max_draft) return RSSM_EINVAL;
    const void* req[] = {alpha, k, v, q, o};
    for (const void* p : req)
        if (!p || !aligned16(p)) return RSSM_EINVAL;
    if (h->pending_T >= 0) return RSSM_ESTATE;
    const int tt = verify_tt(T);
    const int vhv = h->vhvpt;
    const size_t lds = verify_lds(&h->cfg, vhv, tt);
    if (lds > kMaxLds) return RSSM_EUNSUPPORTED;
    StepArgs a = base_args(h);
    a.hvpt = vhv;                                       // verify's own tile; pointer copies by decode tile
    a.tiles = h->cfg.n_vheads / vhv;
    a.alpha = alpha;
    a.k = k;
    a.v = v;
    a.q = q;
    a.o = o;
    a.T = T;
    const rssm_status s = hip_status(launch_verify(a, h->cfg.dim_k, h->cfg.in_dtype, read_fmt(&h->cfg), tt,
                                                   verify_staged(&h->cfg, vhv, tt),
                                                   h->cfg.batch * a.tiles, lds, (hipStream_t)stream));
    if (s == RSSM_OK) h->pending_T = T;
    return s;
}

rssm_status replayssm_prefill(replayssm_t h, int32_t T, const float* alpha, const void* k, const void* v,
                             const void* q, float* o, void* stream) {
    if (!h) return RSSM_EINVAL;
    if (T < 1) return RSSM_EINVAL;
    const void* req[] = {alpha, k, v, q, o};
    for (const void* p : req)
        if (!p || !aligned16(p)) return RSSM_EINVAL;
    if (h->pending_T >= 0) return RSSM_ESTATE;
    const rssm_config* c = &h->cfg;
    const int N = c->dim_k, P = c->dim_v, L = c->window, LS = round4(L);
    // matrix-core kernel: a 16-record window, P and N multiples of 16, at most
    // 16 state blocks of 16 x 16 per wave (ceil(P / 64) p blocks x N / 16 n blocks)
    const int npb = P <= 64 ? 1 : P <= 128 ? 2 : 4;
    int np;
    size_t lds;
    if (L == 16 && P % 16 == 0 && N % 16 == 0 && npb * (N / 16) <= 16) {
        np = -npb;
        lds = (size_t)(16 * (N + 4) + 16 * (N + 16) + 16 * (64 * npb + 16) + 16 + 5 * 16 * 17 + 2 * 16 + 4) * 4;
    } else {
        const int rows_per_pass = 1024 / N;             // RSSM_THREADS / (N / 4)
        np = 2;
        while (np * rows_per_pass < P && np < 16) np *= 2;
        if (np * rows_per_pass < P) return RSSM_EUNSUPPORTED;
        lds = (size_t)(L * N + L * P + LS + 16 * N + L * 16 + 16 * P + 4) * 4;
    }
    if (lds > kMaxLds) return RSSM_EUNSUPPORTED;
    StepArgs a = base_args(h);
    a.alpha = alpha;
    a.k = k;
    a.v = v;
    a.q = q;
    a.o = o;
    a.T = T;
    rssm_status s = hip_status(launch_prefill(a, N, c->in_dtype, ck_of(c), np, c->batch * h->tiles, lds,
                                              (hipStream_t)stream));
    if (s == RSSM_OK && c->read_copy != RSSM_READ_NONE)
        s = hip_status(launch_refresh(base_args(h), N, c->read_copy, ck_of(c), c->batch * h->tiles, (hipStream_t)stream));
    return s;
}

// Commit's launch set-up, shared by both entry points: the fold kernel's
// fixed grid walks the list, 64 workgroups per CU -- more than are resident
// at once, so many folds keep every CU busy (a grid of 8 per CU measured 2 %
// slower at 8 drafts) and none cost one wave of exits.
static rssm_status commit_with(replayssm_t h, const int32_t* accepted, void* stream, bool static_work) {
    StepArgs a = base_args(h);
    a.accepted = accepted;
    a.T = h->pending_T;
    const int ntile = h->cfg.batch * h->tiles;
    const int fold_grid = ntile < 16384 ? ntile : 16384;
    const hipError_t e = static_work
        ? launch_commit_static(a, h->cfg.dim_k, h->cfg.in_dtype, h->cfg.read_copy, multi_of(&h->cfg, h->hvpt),
                               ck_of(&h->cfg), fold_grid, fold_lds(&h->cfg, h->hvpt), (hipStream_t)stream)
        : launch_commit(a, h->cfg.dim_k, h->cfg.in_dtype, h->cfg.read_copy, multi_of(&h->cfg, h->hvpt),
                        ck_of(&h->cfg), fold_grid, fold_lds(&h->cfg, h->hvpt), (hipStream_t)stream);
    const rssm_status s = hip_status(e);
    if (s == RSSM_OK) h->pending_T = -1;
    return s;
}

rssm_status replayssm_commit(replayssm_t h, const int32_t* accepted, void* stream) {
    if (!h) return RSSM_EINVAL;
    if (!accepted || !aligned16(accepted)) return RSSM_EINVAL;
    if (!h->buf.work) return RSSM_EINVAL;                 // created for static commits only
    if (h->pending_T < 0) return RSSM_ESTATE;
    return commit_with(h, accepted, stream, false);
}

rssm_status replayssm_commit_static(replayssm_t h, const int32_t* accepted, void* stream) {
    if (!h) return RSSM_EINVAL;
    if (!accepted || !aligned16(accepted)) return RSSM_EINVAL;
    if ((long)h->cfg.batch * h->tiles > RSSM_STATIC_COMMIT_MAX_TILES) return RSSM_EUNSUPPORTED;
    if (h->pending_T < 0) return RSSM_ESTATE;
    return commit_with(h, accepted, stream, true);
}

rssm_status replayssm_read_error(replayssm_t h, int32_t* host_err, int32_t clear, void* stream) {
    if (!h || !host_err) return RSSM_EINVAL;
    hipStream_t s = (hipStream_t)stream;
    if (hipMemcpyAsync(host_err, h->buf.err, sizeof(int32_t), hipMemcpyDeviceToHost, s) != hipSuccess)
        return RSSM_EHIP;
    if (hipStreamSynchronize(s) != hipSuccess) return RSSM_EHIP;
    if (clear) {
        static const int32_t zero = 0;
        if (hipMemcpyAsync(h->buf.err, &zero, sizeof(int32_t), hipMemcpyHostToDevice, s) != hipSuccess)
            return RSSM_EHIP;
        if (hipStreamSynchronize(s) != hipSuccess) return RSSM_EHIP;
    }
    return RSSM_OK;
}

// ------------------------------------------------------------------ baselines
// Baseline tiles stay inside one key group: the configured tile when it is a
// divisor of the group size, else the default.
static int conv_hvpt(const rssm_config* c) {
    const int g = group_of(c);
    return (c->heads_per_tile > 0 && g % c->heads_per_tile == 0) ? c->heads_per_tile : default_hvpt(c);
}

static ConvArgs conv_args(const rssm_config* c, int hvpt) {
    ConvArgs a;
    memset(&a, 0, sizeof(a));
    a.B = c->batch;
    a.Hv = c->n_vheads;
    a.Hk = c->n_kheads;
    a.P = c->dim_v;
    a.g = c->n_vheads / c->n_kheads;
    a.hvpt = hvpt;
    a.tiles = c->n_vheads / hvpt;
    return a;
}

rssm_status convssm_decode_step(const rssm_config* cfg, void* state, float* row_scale, int32_t state_fmt,
                                const float* alpha, const void* k, const void* v, const void* q, float* o,
                                void* stream) {
    const rssm_status s = check_shape(cfg, false);
    if (s != RSSM_OK) return s;
    if (state_fmt < RSSM_STATE_F32 || state_fmt > RSSM_STATE_FP8_ROW) return RSSM_EINVAL;
    const void* req[] = {state, alpha, k, v, q, o};
    for (const void* p : req)
        if (!p || !aligned16(p)) return RSSM_EINVAL;
    if (state_fmt == RSSM_STATE_FP8_ROW && (!row_scale || !aligned16(row_scale))) return RSSM_EINVAL;
    const int hvpt = conv_hvpt(cfg);
    const size_t lds = conv_lds(hvpt, cfg->dim_v);
    if (lds > kMaxLds) return RSSM_EUNSUPPORTED;
    ConvArgs a = conv_args(cfg, hvpt);
    a.state = state;
    a.rscale = row_scale;
    a.alpha = alpha;
    a.k = k;
    a.v = v;
    a.q = q;
    a.o = o;
    return hip_status(launch_conv_decode(a, cfg->dim_k, cfg->in_dtype, state_fmt, cfg->batch * a.tiles, lds,
                                         (hipStream_t)stream));
}

rssm_status convssm_spec_verify(const rssm_config* cfg, float* states, const int32_t* cur, int32_t T,
                                const float* alpha, const void* k, const void* v, const void* q, float* o,
                                void* stream) {
    const rssm_status s = check_shape(cfg, false);
    if (s != RSSM_OK) return s;
    if (cfg->max_draft < 1 || cfg->max_draft > 8 || T < 1 || T > cfg->max_draft) return RSSM_EINVAL;
    const void* req[] = {states, cur, alpha, k, v, q, o};
    for (const void* p : req)
        if (!p || !aligned16(p)) return RSSM_EINVAL;
    const int hvpt = conv_hvpt(cfg);
    const int tt = verify_tt(T);
    const size_t lds = conv_verify_lds(hvpt, cfg->dim_v, tt);
    if (lds > kMaxLds) return RSSM_EUNSUPPORTED;
    ConvArgs a = conv_args(cfg, hvpt);
    a.state = states;
    a.cur = cur;
    a.T = T;
    a.ring = cfg->max_draft + 1;
    a.alpha = alpha;
    a.k = k;
    a.v = v;
    a.q = q;
    a.o = o;
    return hip_status(launch_conv_verify(a, cfg->dim_k, cfg->in_dtype, tt, cfg->batch * a.tiles, lds,
                                         (hipStream_t)stream));
}

rssm_status convssm_commit(const rssm_config* cfg, int32_t* cur, const int32_t* accepted, int32_t T,
                           int32_t* err, void* stream) {
    const rssm_status s = check_shape(cfg, false);
    if (s != RSSM_OK) return s;
    if (cfg->max_draft < 1 || T < 1 || T > cfg->max_draft) return RSSM_EINVAL;
    const void* req[] = {cur, accepted, err};
    for (const void* p : req)
        if (!p || !aligned16(p)) return RSSM_EINVAL;
    ConvArgs a = conv_args(cfg, conv_hvpt(cfg));
    a.cur_rw = cur;
    a.accepted = accepted;
    a.err = err;
    a.T = T;
    a.ring = cfg->max_draft + 1;
    return hip_status(launch_conv_commit(a, (hipStream_t)stream));
}

}  // extern "C"
