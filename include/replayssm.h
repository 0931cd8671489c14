/* replayssm.h -- C ABI of the ReplaySSM decode hot path for MI355X (gfx950).
 *
 * One scalar-decay SSM layer, decoded token by token:
 *     S_t = a_t S_{t-1} + v_t k_t^T,   o_t = S_t q_t                       (eq.R)
 * S is P x N per (sequence, value head): P = value dim (rows), N = key dim
 * (columns, contiguous).  The state is held as a high-precision checkpoint
 * plus a buffer of the last input records (a_j, k_j, v_j), and outputs are
 * formed by replay from the checkpoint and the buffer:
 *     o = g_{1:h} S_ckpt q + sum_j g_{j+1:h} v_j (k_j . q)                  (eq.U, eq.O1)
 * with g_{a:b} the product of the decays a_a..a_b (empty product 1).
 *
 * Citation keys (web pages describing the method):
 *   [ru] aikraft.ru "ReplaySSM: Революция в декодировании гибридных моделей", §01-§07
 *   [ar] sitech.ge "NVIDIA و Dao AI Lab يقدّمان ReplaySSM لتسريع فك ترميز النماذج الهجينة"
 *   [zh] ai.cheesepanini.fun card "ReplaySSM——重新思考混合模型解码的状态存储"
 *
 * Conventions for every call
 *   - Pointers marked (device) are HIP device pointers; all others are host.
 *     Every device array is contiguous, row-major, last index fastest, and its
 *     base must be 16-byte aligned.  Violations return RSSM_EINVAL before any
 *     HIP call.
 *   - The caller owns all device memory (typically torch tensors) and keeps it
 *     alive until replayssm_destroy.  The library never allocates device memory.
 *   - Calls are asynchronous on `stream` (a hipStream_t passed as void*; NULL =
 *     the null stream) and return a host-side status.  Only replayssm_read_error
 *     synchronises.  A handle is not thread-safe.
 *   - alpha, the checkpoint, the outputs and the row scales are fp32; k, q, v
 *     are fp32 or bf16 (rssm_config.in_dtype).  Value head h uses key/query head
 *     h / (n_vheads / n_kheads): the value heads of a key group share k and q
 *     and therefore the scores k^T q ([zh] method points).
 *   - Errors the device detects (a pointer outside 0..L-1 at decode, an
 *     accepted length outside 0..T, a buffer overflow) leave the affected tile
 *     untouched and OR a RSSM_DEVERR_* bit into the error word; read it with
 *     replayssm_read_error.  No exception crosses this ABI.
 */
#ifndef REPLAYSSM_H
#define REPLAYSSM_H

#include <stddef.h>
#include <stdint.h>

#if defined(__GNUC__) || defined(__clang__)
#define RSSM_API __attribute__((visibility("default")))
#else
#define RSSM_API
#endif

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    RSSM_OK = 0,
    RSSM_EINVAL = 1,        /* bad argument: null/misaligned pointer, bad size */
    RSSM_EUNSUPPORTED = 2,  /* valid but not built (e.g. key dim not in {16,32,64,128,256}) */
    RSSM_ESTATE = 3,        /* call not allowed now (decode/flush while a verify is pending,
                               commit without a verify) */
    RSSM_EHIP = 4           /* a HIP launch or copy failed */
} rssm_status;

typedef enum { RSSM_F32 = 0, RSSM_BF16 = 1 } rssm_dtype;

/* Low-precision read copy of the checkpoint ([ru] §06; [ar] "limiting
 * quantization error"): written next to the fp32 checkpoint at every fold,
 * read only by non-flush outputs and verification, never by the recurrence. */
typedef enum {
    RSSM_READ_NONE = 0,     /* outputs read the fp32 checkpoint                     */
    RSSM_READ_BF16 = 1,     /* bf16 copy, round to nearest even                     */
    RSSM_READ_FP8_ROW = 2,  /* OCP e4m3fn codes + fp32 scale per state row:
                               scale = amax(row)/448 (1 for an all-zero row),
                               code = e4m3_rne_saturating(x / scale)                 */
    RSSM_READ_MXFP4 = 3     /* OCP MXFP4 (needs N >= 32): each block of 32
                               consecutive entries of a row shares X = 2^e,
                               e = floor(log2 amax(block)) - 2 clamped to
                               [-127, 127] (-127 for an all-zero block), stored
                               as the E8M0 byte e + 127; entries are E2M1 codes
                               of x / X, round to nearest even, saturating at 6,
                               two per byte (entry n in byte n/2, low nibble
                               first).  Stands in for the pages' NVFP4 copy.     */
} rssm_read_copy;

/* Storage of the recurrent checkpoint ([ru] §06, last paragraph: an FP16
 * recurrent checkpoint with stochastic rounding stays close to FP32). */
typedef enum {
    RSSM_CKPT_F32 = 0,      /* fp32 checkpoint                                      */
    RSSM_CKPT_F16_SR = 1    /* fp16 checkpoint; every fold computes in fp32 and
                               stores each entry x rounded stochastically:
                               a = |x|, e = max(floor(log2 a), -14), q = 2^(e-10),
                               m = a/q, f = floor(m), p = m - f; the result is
                               (f+1)q if u/2^16 < p else fq, at most 65504, with
                               the sign of x (an infinity stays infinite, NaN
                               stays NaN).  u is 16 bits of pcg_hash (Jarzynski
                               and Olano, JCGT 2020), h: entry g (flat index in
                               [B][Hv][P][N]) takes the low (g even) or high half of
                               h(key ^ (g >> 1)), with key = h(lo(s) ^ h(hi(s) ^
                               h(lo(E) ^ h(hi(E))))) for the layer seed s and the
                               fold epoch E of the entry's tile: the number of
                               folds that tile stored before, kept on the device
                               in the `folds` buffer and advanced by every call
                               that writes the checkpoint (decode's flush steps,
                               flush, commit, prefill; reset leaves it).  So a
                               call replayed from a captured HIP graph draws new
                               numbers at every fold.  The read copy and
                               flush-step outputs come from the unrounded fp32
                               fold.  Needs B*Hv*P*N < 2^33.                       */,
    RSSM_CKPT_FP8_SR = 2    /* fp8 checkpoint ([ar] section on limiting
                               quantization error: low-precision reads with an
                               FP16 or FP8 recurrence); needs a read copy
                               (non-flush steps and verify read the copy).
                               Each row is N OCP e4m3fn codes followed by a
                               16-byte trailer whose first 4 bytes hold the row's
                               fp32 scale sig = 2^s, the smallest power of two
                               with amax <= 448 sig (amax = m 2^E, m in [1, 2):
                               s = E - 8, plus 1 if m > 1.75; s in [-126, 127];
                               sig = 1 for a row with no nonzero entry, NaN
                               entries ignored by the max), so a row takes
                               N + 16 bytes and x / sig is exact.  Every fold
                               computes in fp32 from code * sig and stores entry
                               x as the code of y = x / sig rounded
                               stochastically: a = |y|, e = max(floor(log2 a),
                               -6), q = 2^(e-3), m = a/q, f = floor(m), p = m -
                               f; (f+1)q if u/2^16 < p else fq, at most 448,
                               with the sign of y; u, the key and the fold
                               epochs as for RSSM_CKPT_F16_SR.  e4m3fn has no
                               infinity: a non-finite y stores the NaN code 0x7f
                               (an infinite entry makes its row's scale infinite,
                               and the row then reads as NaN).  Needs
                               B*Hv*P*N < 2^33.                                    */
} rssm_ckpt_fmt;

/* Device error word bits. */
#define RSSM_DEVERR_POINTER  1   /* buffered-record count outside its valid range */
#define RSSM_DEVERR_ACCEPT   2   /* accepted[b] outside 0..T                      */
#define RSSM_DEVERR_OVERFLOW 4   /* h_b + T exceeds the buffer capacity           */

typedef struct {
    int32_t batch;          /* B                                                  */
    int32_t n_vheads;       /* Hv                                                 */
    int32_t n_kheads;       /* Hk, divides Hv                                     */
    int32_t dim_v;          /* P, 4..256, a multiple of 4                         */
    int32_t dim_k;          /* N, one of 16, 32, 64, 128, 256                     */
    int32_t window;         /* L, 1..32: records buffered before a flush          */
    int32_t max_draft;      /* T_max, 0..8: drafts per verify (0 = no verify)     */
    int32_t in_dtype;       /* rssm_dtype of k, q, v                              */
    int32_t read_copy;      /* rssm_read_copy                                     */
    int32_t heads_per_tile; /* value heads per workgroup (a tile); either a
                               divisor of the group size g = Hv/Hk, or a multiple
                               of g that divides Hv (the tile then holds whole
                               key groups).  The tile's rows, heads_per_tile*P,
                               may not exceed 1024, and its shared-memory
                               footprint in decode, fold and (max_draft > 0)
                               verify of max_draft drafts must fit 64 KiB
                               (else RSSM_EUNSUPPORTED when sizes are
                               queried).  0 = library default: one
                               key group's share (at most 128 rows); with a
                               read copy or fp16 checkpoint doubled while the
                               tile's read data stays under 32 KiB, its rows
                               within 256, its LDS under 28 KiB and (except
                               for MXFP4) the tile inside one key group.      */
    int32_t ckpt_fmt;       /* rssm_ckpt_fmt                                      */
    uint64_t sr_seed;       /* seed of an fp16 or fp8 checkpoint's stochastic
                               rounding                                           */
} rssm_config;

/* Indices into the sizes array of replayssm_query_sizes. */
enum {
    RSSM_BUF_CKPT = 0,      /* checkpoint [B][Hv][P][N], fp32 or fp16, or fp8 rows of
                               N + 16 bytes [B][Hv][P][N + 16] (ckpt_fmt)             */
    RSSM_BUF_READ_COPY,     /* bf16 [B][Hv][P][N], e4m3 codes [B][Hv][P][N] or E2M1
                               code pairs [B][Hv][P][N/2] bytes; 0 if none          */
    RSSM_BUF_ROW_SCALE,     /* fp32 [B][Hv][P] (fp8 copy), E8M0 bytes [B][Hv][P][N/32]
                               (MXFP4 copy); else 0                                 */
    RSSM_BUF_KBUF,          /* key records   [B][Hk][C][N] in in_dtype, C = L + T_max   */
    RSSM_BUF_VBUF,          /* value records [B][Hv][C][P] in in_dtype                  */
    RSSM_BUF_ABUF,          /* decays        [B][Hv][C] fp32                            */
    RSSM_BUF_COUNT,         /* int32 [B][tiles]: records since the checkpoint, h_b,
                               one copy per workgroup tile (all copies of a row equal) */
    RSSM_BUF_ERR,           /* int32 [1] device error word                              */
    RSSM_BUF_WORK,          /* int32 [2 + B * tiles] commit work: list count, one
                               unused word, list of tiles to fold; every verify
                               clears the count for the commit that follows   */
    RSSM_BUF_FOLDS,         /* uint32 [B][tiles] fold epochs of the fp16 checkpoint's
                               stochastic rounding (RSSM_CKPT_F16_SR or
                               RSSM_CKPT_FP8_SR; else 0) */
    RSSM_NUM_BUFS
};

typedef struct {
    void*    ckpt;          /* fp32 or fp16 entries (ckpt_fmt)                        */
    void*    read_copy;
    void*    row_scale;     /* fp32 row scales (fp8) or E8M0 block exponents (MXFP4) */
    void*    kbuf;
    void*    vbuf;
    float*   abuf;
    int32_t* count;
    int32_t* err;
    int32_t* work;          /* commit work area (RSSM_BUF_WORK), or NULL when the caller
                               commits only with replayssm_commit_static        */
    uint32_t* folds;        /* fold epochs (RSSM_BUF_FOLDS): needed with an fp16
                               checkpoint, ignored (may be NULL) otherwise       */
} rssm_buffers;

typedef struct replayssm* replayssm_t;

/* Library version string (static storage): "replayssm-gfx950 <RSSM_ABI_VERSION>".
 * ABI 0.2: rssm_buffers gained `work` (RSSM_BUF_WORK).  ABI 0.3: rssm_buffers
 * gained `folds` (RSSM_BUF_FOLDS), the fp16 checkpoint's rounding epochs moved
 * from a host launch count to the device, and replayssm_launch_count is gone.
 * ABI 0.4: the HBM probes (rssm_probe_*) moved to librssm_probes.so
 * (rssm_probes.h); this library no longer exports them.
 * A caller built against another version's header must not be linked with
 * this library. */
#define RSSM_ABI_VERSION "0.4"
RSSM_API const char* replayssm_version(void);

/* Byte size of each caller-owned device buffer for `cfg` (host only; no HIP
 * call).  sizes[RSSM_BUF_*]; `tiles` (may be NULL) receives the number of
 * workgroup tiles per sequence, the second dimension of the count array.
 * The buffers must be zero-filled before first use (empty buffer, zero
 * checkpoint), or set up by the caller and then replayssm_refresh_read_copy. */
RSSM_API rssm_status replayssm_query_sizes(const rssm_config* cfg, size_t sizes[RSSM_NUM_BUFS],
                                  int32_t* tiles);

/* Validate cfg and buffers and make a handle that keeps the raw pointers
 * (host allocation only).  *out is NULL on failure. */
RSSM_API rssm_status replayssm_create(const rssm_config* cfg, const rssm_buffers* bufs, replayssm_t* out);
RSSM_API rssm_status replayssm_destroy(replayssm_t h);

/* Start new sequences: zero the checkpoint and the read copy (fp8 row scales
 * 1, MXFP4 block exponents those of an all-zero block), and set
 * the record count to 0 for the sequences listed in seq_ids (device int32[n];
 * NULL = all B sequences).  Ids outside 0..B-1 are ignored and flagged with
 * RSSM_DEVERR_POINTER.  Not allowed while a verify is pending. */
RSSM_API rssm_status replayssm_reset(replayssm_t h, const int32_t* seq_ids, int32_t n, void* stream);

/* Re-derive the read copy from the fp32 checkpoint for every sequence (after
 * the caller wrote a checkpoint, e.g. from prefill).  No-op without a copy. */
RSSM_API rssm_status replayssm_refresh_read_copy(replayssm_t h, void* stream);

/* One decode step for all B sequences ([ru] §03; [ar] "how ReplaySSM works";
 * [zh] method points).  With h_b records buffered, the step appends the
 * current record (alpha, k, v) as record h_b + 1 and outputs
 *     o = g_{1:h+1} S_ckpt q + sum_{j<=h+1} g_{j+1:h+1} v_j (k_j . q)
 * reading the checkpoint (or its read copy) and writing no state.  When the
 * append fills the window (h_b + 1 == L) the same call instead folds the L
 * records into the checkpoint,
 *     S_ckpt <- g_{1:L} S_ckpt + sum_j g_{j+1:L} v_j k_j^T,
 * writes it (and its read copy) once, outputs S_ckpt q from the folded fp32
 * state, and empties the buffer.
 *   alpha (device) [B][Hv] fp32;  k, q (device) [B][Hk][N];  v (device) [B][Hv][P]
 *   o (device, written) [B][Hv][P] fp32
 * RSSM_ESTATE while a verify is pending. */
RSSM_API rssm_status replayssm_decode_step(replayssm_t h, const float* alpha, const void* k,
                                  const void* v, const void* q, float* o, void* stream);

/* Fold every non-empty buffer into its checkpoint (write once, empty the
 * buffer) so that the checkpoint equals the current state S_t: the flush of
 * [ru] §03 (the buffered records folded into the high-precision checkpoint,
 * which is then written once) and [ar] "how ReplaySSM works", called here on
 * demand instead of when the window fills.  Sequences with an empty buffer
 * are untouched.  RSSM_ESTATE while a verify is pending. */
RSSM_API rssm_status replayssm_flush(replayssm_t h, void* stream);

/* Speculative verification of T drafts, output only ([ru] §05; [ar] rollback
 * section; [zh] method points, eq.OT).  Appends the T draft records after the
 * h_b committed ones (slots h_b..h_b+T-1) and outputs, for draft t = 1..T,
 *     O[t] = g_{1:h+t} S_ckpt q_t + sum_{j<=h+t} g_{j+1:h+t} v_j (k_j . q_t)
 * reading each checkpoint row once for all T queries; no state is written and
 * the pointer does not move.  1 <= T <= max_draft.
 *   alpha (device) [B][T][Hv];  k, q (device) [B][T][Hk][N];  v (device) [B][T][Hv][P]
 *   o (device, written) [B][T][Hv][P] fp32
 * Leaves the handle with a pending verify of T; RSSM_ESTATE if one is pending. */
RSSM_API rssm_status replayssm_spec_verify(replayssm_t h, int32_t T, const float* alpha, const void* k,
                                  const void* v, const void* q, float* o, void* stream);

/* Commit the accepted prefix of the pending verify by advancing the pointer:
 * h_b += accepted[b] (0..T); drafts past it are ignored and later overwritten,
 * and no state snapshot is saved or restored ([ru] §05; [zh] method points).
 * If h_b reaches L or more, all h_b committed records are folded into the
 * checkpoint at once and the buffer is emptied.  Two launches: one thread per
 * tile advances the pointers and lists the tiles that fold (in the work
 * buffer, whose count the pending verify cleared), then a fixed grid folds
 * the listed tiles only.
 *   accepted (device) int32 [B].  RSSM_ESTATE without a pending verify. */
RSSM_API rssm_status replayssm_commit(replayssm_t h, const int32_t* accepted, void* stream);

/* replayssm_commit for callers that cannot allocate device memory (code under
 * HIP graph capture, tight serving loops, harnesses that forbid allocation):
 * the same pointer advance and folds, results identical to replayssm_commit,
 * with the list of tiles to fold kept in a device array the library owns
 * instead of the handle's work buffer (which may then be NULL at create).  The
 * array holds RSSM_STATIC_COMMIT_MAX_TILES tiles (batch * tiles per sequence,
 * 1 MiB); larger layers get RSSM_EUNSUPPORTED before any HIP call.  Each GPU
 * has one such array, set up on the first call made with that device current
 * (`stream` must belong to the current device), kept until the process ends
 * and shared by every handle: it keeps the last call's contents (each call
 * clears its list count first), and calls that overlap on one GPU -- on
 * different streams, or from different threads -- race.  Allocates nothing
 * and calls no allocating routine; three launches (clear the count, plan,
 * fold).  Same states and errors as replayssm_commit. */
#define RSSM_STATIC_COMMIT_MAX_TILES 262144
RSSM_API rssm_status replayssm_commit_static(replayssm_t h, const int32_t* accepted, void* stream);

/* Prefill T >= 1 prompt tokens ([zh] method points: the unrolled window is
 * the chunkwise form prefill kernels use).  Leaves the state that T decode
 * steps would leave: o holds every token's output, the checkpoint advances to
 * the last complete window (computed in fp32 throughout; an fp16 or fp8
 * checkpoint is rounded once, as one fold), the buffer holds the
 * records after it and the count becomes (h_b + T) mod L.  With a read copy,
 * the copy is then refreshed from the stored checkpoint.  Same inputs and
 * layouts as replayssm_spec_verify: alpha [B][T][Hv], k and q [B][T][Hk][N],
 * v [B][T][Hv][P], o [B][T][Hv][P] fp32.  One workgroup per tile keeps each
 * head's state in registers for the whole prompt.  RSSM_EUNSUPPORTED when a
 * head has more than 16 * 1024 / N rows or the chunk buffers exceed 64 KiB of
 * LDS; RSSM_ESTATE while a verify is pending. */
RSSM_API rssm_status replayssm_prefill(replayssm_t h, int32_t T, const float* alpha, const void* k,
                                       const void* v, const void* q, float* o, void* stream);

/* Copy the device error word to *host_err (synchronises `stream`).  If clear
 * is nonzero the word is reset to 0 afterwards. */
RSSM_API rssm_status replayssm_read_error(replayssm_t h, int32_t* host_err, int32_t clear, void* stream);

/* ---------------------------------------------------------------------------
 * In-run baselines (same conventions; cfg->window/max_draft/read_copy ignored
 * unless stated).
 * ------------------------------------------------------------------------- */

/* State formats of the conventional decode. */
typedef enum {
    RSSM_STATE_F32 = 0,     /* fp32 state, read and written every step             */
    RSSM_STATE_BF16 = 1,    /* state stored as bf16 every step (quantised recurrence) */
    RSSM_STATE_FP8_ROW = 2  /* state stored as e4m3 codes + fp32 row scales          */
} rssm_state_fmt;

/* Conventional fused decode ([ru] §01): each step reads the whole state,
 * decays it, adds v k^T, outputs S q, and writes the state back.
 *   state (device) [B][Hv][P][N] in state_fmt (fp32, bf16 or e4m3 codes);
 *   row_scale (device) [B][Hv][P] fp32 for RSSM_STATE_FP8_ROW, else NULL.
 * For the quantised formats the update and the output are computed in fp32
 * from the dequantised state, then the new state is re-quantised: the rounding
 * feeds the next step ([ru] §02 problem 3). */
RSSM_API rssm_status convssm_decode_step(const rssm_config* cfg, void* state, float* row_scale,
                                int32_t state_fmt, const float* alpha, const void* k,
                                const void* v, const void* q, float* o, void* stream);

/* Snapshot speculative verify ([ru] §02 problem 2, §05): from the state in
 * ring slot cur[b], run T drafts through the recurrence, output each draft's
 * S q_t, and store the state after draft t in slot (cur[b] + t) mod (T_max+1):
 * one state read and T state writes.
 *   states (device) fp32 [B][T_max+1][Hv][P][N];  cur (device) int32 [B];
 *   alpha, k, v, q, o as in replayssm_spec_verify. */
RSSM_API rssm_status convssm_spec_verify(const rssm_config* cfg, float* states, const int32_t* cur,
                                int32_t T, const float* alpha, const void* k, const void* v,
                                const void* q, float* o, void* stream);

/* Snapshot commit: cur[b] <- (cur[b] + accepted[b]) mod (T_max+1); accepted
 * outside 0..T sets RSSM_DEVERR_ACCEPT in err (device int32[1]) and leaves
 * cur[b] unchanged. */
RSSM_API rssm_status convssm_commit(const rssm_config* cfg, int32_t* cur, const int32_t* accepted,
                           int32_t T, int32_t* err, void* stream);

#ifdef __cplusplus
}
#endif
#endif /* REPLAYSSM_H */
