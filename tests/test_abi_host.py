"""C ABI checks that need no GPU: the library loads, exports every function
include/replayssm.h declares, sizes buffers as documented, and rejects misuse
before any HIP call."""
import ctypes
import os
import re

import pytest

from ssm_layer_decode_amd import _lib
from ssm_layer_decode_amd import bytes_model as bm
from ssm_layer_decode_amd import workloads as W
from ssm_layer_decode_amd.replayssm import LayerConfig, replayssm_query_sizes

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "replayssm.h")

pytestmark = pytest.mark.skipif(not os.path.exists(_lib.LIB_PATH), reason="library not built")


def declared_functions(header=HEADER):
    text = open(header).read()
    return sorted(set(re.findall(r"RSSM_API\s+[\w\s\*]+?\b(\w+)\s*\(", text)))


def _dynamic_symbols(path):
    """Names the shared library exports (nm -D, defined text symbols)."""
    import subprocess
    out = subprocess.run(["nm", "-D", "--defined-only", path], capture_output=True, text=True, check=True).stdout
    return {line.split()[-1] for line in out.splitlines() if len(line.split()) == 3 and line.split()[1] == "T"}


def test_every_declared_symbol_is_exported():
    lib = _lib.load()
    names = declared_functions()
    assert len(names) >= 16
    for n in names:
        assert hasattr(lib, n), n
    assert sorted(names) == sorted(_lib.EXPORTED)


def test_probes_live_in_their_own_library():
    """The HBM probes are declared in rssm_probes.h and exported by
    librssm_probes.so only; the product library exports exactly its header's
    functions."""
    probe_header = os.path.join(os.path.dirname(HEADER), "rssm_probes.h")
    names = declared_functions(probe_header)
    assert sorted(names) == sorted(_lib.PROBE_EXPORTED)
    probes = _lib.load_probes()
    for n in names:
        assert hasattr(probes, n), n
    product = {s for s in _dynamic_symbols(_lib.LIB_PATH) if s.startswith(("replayssm_", "convssm_", "rssm_"))}
    assert product == set(_lib.EXPORTED)
    probe_syms = {s for s in _dynamic_symbols(_lib.PROBE_LIB_PATH) if s.startswith(("replayssm_", "convssm_", "rssm_"))}
    assert probe_syms == set(_lib.PROBE_EXPORTED)


def test_version():
    """The library's ABI version is the header's and the binding's."""
    import re
    got = _lib.load().replayssm_version().decode()
    hdr = open(os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "include",
                            "replayssm.h")).read()
    m = re.search(r'#define RSSM_ABI_VERSION "([^"]+)"', hdr)
    assert m and got == "replayssm-gfx950 " + m.group(1) == "replayssm-gfx950 " + _lib.ABI_VERSION


@pytest.mark.parametrize("shape", [W.TINY, W.MAMBA2, W.GDN, W.SPEC, W.LONG])
def test_buffer_sizes_match_layout(shape):
    cfg = LayerConfig.of(shape)
    sizes, tiles = replayssm_query_sizes(cfg)
    B, Hv, Hk, P, N = shape.batch, shape.n_vheads, shape.n_kheads, shape.dim_v, shape.dim_k
    C = shape.window + shape.max_draft
    e = 2 if shape.in_dtype == "bf16" else 4
    assert sizes[_lib.RSSM_BUF_CKPT] == B * bm.state_bytes(bm.Dims.of(shape))
    assert sizes[_lib.RSSM_BUF_KBUF] == B * Hk * C * N * e
    assert sizes[_lib.RSSM_BUF_VBUF] == B * Hv * C * P * e
    assert sizes[_lib.RSSM_BUF_ABUF] == B * Hv * C * 4
    assert sizes[_lib.RSSM_BUF_COUNT] == B * tiles * 4
    assert sizes[_lib.RSSM_BUF_WORK] == -(-(2 + B * tiles) * 4 // 16) * 16
    assert Hv % tiles == 0 and (Hv // tiles) * P <= 256
    assert sizes[_lib.RSSM_BUF_READ_COPY] == 0 and sizes[_lib.RSSM_BUF_ROW_SCALE] == 0


def test_read_copy_sizes():
    s_bf, _ = replayssm_query_sizes(LayerConfig.of(W.LONG, read_copy="bf16"))
    s_f8, _ = replayssm_query_sizes(LayerConfig.of(W.LONG, read_copy="fp8"))
    n = 64 * 64 * 128 * 128
    assert s_bf[_lib.RSSM_BUF_READ_COPY] == 2 * n and s_bf[_lib.RSSM_BUF_ROW_SCALE] == 0
    assert s_f8[_lib.RSSM_BUF_READ_COPY] == n and s_f8[_lib.RSSM_BUF_ROW_SCALE] == 64 * 64 * 128 * 4
    s_f4, _ = replayssm_query_sizes(LayerConfig.of(W.LONG, read_copy="mxfp4"))
    assert s_f4[_lib.RSSM_BUF_READ_COPY] == n // 2            # two E2M1 codes per byte
    assert s_f4[_lib.RSSM_BUF_ROW_SCALE] == n // 32           # one E8M0 byte per 32 entries


def test_mxfp4_needs_blocks_of_32():
    cfg = LayerConfig.of(W.with_(W.TINY, read_copy="mxfp4"))     # dim_k 16
    with pytest.raises(_lib.RssmError) as ei:
        replayssm_query_sizes(cfg)
    assert ei.value.status == _lib.RSSM_EUNSUPPORTED
    sizes, _ = replayssm_query_sizes(LayerConfig(**{**cfg.__dict__, "dim_k": 32}))
    assert sizes[_lib.RSSM_BUF_ROW_SCALE] == 2 * 2 * 16 * 1


@pytest.mark.parametrize("bad,status", [
    (dict(n_kheads=3), _lib.RSSM_EINVAL),          # does not divide Hv
    (dict(dim_k=48), _lib.RSSM_EUNSUPPORTED),      # key dim not built
    (dict(dim_v=6), _lib.RSSM_EINVAL),             # not a multiple of 4
    (dict(window=0), _lib.RSSM_EINVAL),
    (dict(window=33), _lib.RSSM_EINVAL),
    (dict(max_draft=9), _lib.RSSM_EINVAL),
    (dict(heads_per_tile=3), _lib.RSSM_EINVAL),    # neither divides nor is a multiple of the group
    (dict(batch=0), _lib.RSSM_EINVAL),
])
def test_bad_configs_rejected(bad, status):
    cfg = LayerConfig.of(W.with_(W.TINY, n_vheads=4, n_kheads=2, max_draft=2), **{})
    d = dict(cfg.__dict__)
    d.update(bad)
    with pytest.raises(_lib.RssmError) as ei:
        replayssm_query_sizes(LayerConfig(**d))
    assert ei.value.status == status


class _FakeBufs:
    """Aligned host addresses standing in for device buffers: create() only
    stores pointers, and every call below is rejected before any HIP call."""

    def __init__(self, nbytes=1 << 16):
        self.mem = ctypes.create_string_buffer(nbytes + 64)
        base = ctypes.addressof(self.mem)
        self.base = (base + 15) & ~15

    def ptr(self, off=0):
        return self.base + off


def _create(cfg: LayerConfig, fake: _FakeBufs, misalign=None):
    lib = _lib.load()
    vals = []
    for i, n in enumerate(_lib.BUFFER_NAMES):
        p = fake.ptr(1024 * i)
        if n == misalign:
            p += 4
        if n in ("read_copy", "row_scale") and cfg.read_copy == "none":
            p = None
        if n == "folds" and (cfg.ckpt == "f32" or misalign == "no folds"):
            p = None
        if n == "work" and misalign == "no work":
            p = None
        vals.append(p)
    b = _lib.RssmBuffers(*vals)
    c = cfg.c()
    h = ctypes.c_void_p()
    st = lib.replayssm_create(ctypes.byref(c), ctypes.byref(b), ctypes.byref(h))
    return st, h


def test_create_validates_pointers():
    fake = _FakeBufs()
    cfg = LayerConfig.of(W.with_(W.TINY, max_draft=4))
    st, h = _create(cfg, fake)
    assert st == _lib.RSSM_OK and h.value
    assert _lib.load().replayssm_destroy(h) == _lib.RSSM_OK
    for n in ("kbuf", "work"):
        st, h = _create(cfg, fake, misalign=n)
        assert st == _lib.RSSM_EINVAL and not h.value
    # an fp16 checkpoint needs its fold-epoch buffer (aligned); others ignore it
    cfg16 = LayerConfig.of(W.with_(W.TINY, max_draft=4), ckpt="f16sr")
    st, h = _create(cfg16, fake)
    assert st == _lib.RSSM_OK and h.value
    assert _lib.load().replayssm_destroy(h) == _lib.RSSM_OK
    for bad in ("folds", "no folds"):
        st, h = _create(cfg16, fake, misalign=bad)
        assert st == _lib.RSSM_EINVAL and not h.value
    cfg8 = LayerConfig.of(W.with_(W.TINY, read_copy="fp8"))
    lib = _lib.load()
    b = _lib.RssmBuffers(fake.ptr(0), fake.ptr(1024), None, fake.ptr(2048), fake.ptr(3072),
                         fake.ptr(4096), fake.ptr(5120), fake.ptr(6144), fake.ptr(7168))
    c = cfg8.c()
    h = ctypes.c_void_p()
    assert lib.replayssm_create(ctypes.byref(c), ctypes.byref(b), ctypes.byref(h)) == _lib.RSSM_EINVAL


def test_calls_rejected_before_any_hip_call():
    lib = _lib.load()
    fake = _FakeBufs()
    cfg = LayerConfig.of(W.with_(W.TINY, max_draft=4))
    st, h = _create(cfg, fake)
    assert st == _lib.RSSM_OK
    p = fake.ptr
    # null / misaligned step pointers
    assert lib.replayssm_decode_step(h, None, p(0), p(0), p(0), p(0), None) == _lib.RSSM_EINVAL
    assert lib.replayssm_decode_step(h, p(4), p(0), p(0), p(0), p(0), None) == _lib.RSSM_EINVAL
    # verify with T out of range
    assert lib.replayssm_spec_verify(h, 0, p(0), p(0), p(0), p(0), p(0), None) == _lib.RSSM_EINVAL
    assert lib.replayssm_spec_verify(h, 5, p(0), p(0), p(0), p(0), p(0), None) == _lib.RSSM_EINVAL
    # commit without a pending verify
    assert lib.replayssm_commit(h, p(0), None) == _lib.RSSM_ESTATE
    assert lib.replayssm_commit(h, None, None) == _lib.RSSM_EINVAL
    assert lib.replayssm_read_error(h, None, 0, None) == _lib.RSSM_EINVAL
    assert lib.replayssm_destroy(None) == _lib.RSSM_EINVAL
    lib.replayssm_destroy(h)


def test_baseline_entry_points_validate():
    lib = _lib.load()
    fake = _FakeBufs()
    cfg = LayerConfig.of(W.with_(W.TINY, max_draft=4)).c()
    p = fake.ptr
    assert lib.convssm_decode_step(ctypes.byref(cfg), None, None, 0, p(0), p(0), p(0), p(0), p(0), None) == _lib.RSSM_EINVAL
    assert lib.convssm_decode_step(ctypes.byref(cfg), p(0), None, 2, p(0), p(0), p(0), p(0), p(0), None) == _lib.RSSM_EINVAL
    assert lib.convssm_decode_step(ctypes.byref(cfg), p(0), None, 7, p(0), p(0), p(0), p(0), p(0), None) == _lib.RSSM_EINVAL
    assert lib.convssm_spec_verify(ctypes.byref(cfg), p(0), p(0), 5, p(0), p(0), p(0), p(0), p(0), None) == _lib.RSSM_EINVAL
    assert lib.convssm_commit(ctypes.byref(cfg), p(0), p(0), 0, p(0), None) == _lib.RSSM_EINVAL


def test_probe_entry_points_validate():
    lib = _lib.load_probes()
    fake = _FakeBufs()
    p = fake.ptr
    assert lib.rssm_probe_copy(p(0), p(0), 17, None) == _lib.RSSM_EINVAL
    assert lib.rssm_probe_read(None, 16, p(0), None) == _lib.RSSM_EINVAL
    # chunked probe: whole 32 KiB chunks, writes a multiple of 16 up to 4 KiB, dst when writing
    assert lib.rssm_probe_read_chunked(p(16), 32768 + 16, p(16), 0, p(16), None) == _lib.RSSM_EINVAL
    assert lib.rssm_probe_read_chunked(p(16), 0, p(16), 0, p(16), None) == _lib.RSSM_EINVAL
    assert lib.rssm_probe_read_chunked(p(16), 32768, p(16), 24, p(16), None) == _lib.RSSM_EINVAL
    assert lib.rssm_probe_read_chunked(p(16), 32768, p(16), 8192, p(16), None) == _lib.RSSM_EINVAL
    assert lib.rssm_probe_read_chunked(p(16), 32768, None, 1024, p(16), None) == _lib.RSSM_EINVAL
    assert lib.rssm_probe_read_chunked(None, 32768, None, 0, p(16), None) == _lib.RSSM_EINVAL


def test_tiles_of_whole_key_groups_accepted():
    base = LayerConfig.of(W.with_(W.TINY, n_vheads=8, n_kheads=4))      # group of 2
    for hvpt, ok in ((1, True), (2, True), (4, True), (8, True), (3, False), (6, False)):
        cfg = LayerConfig(**{**base.__dict__, "heads_per_tile": hvpt})
        if ok:
            sizes, tiles = replayssm_query_sizes(cfg)
            assert tiles == 8 // hvpt
        else:
            with pytest.raises(_lib.RssmError):
                replayssm_query_sizes(cfg)


def test_shared_memory_limits_rejected():
    """Largest dims, window and drafts together exceed a workgroup's 64 KiB of
    shared memory: refused when the sizes are queried, before any buffer."""
    big = W.Shape(batch=2, n_vheads=2, n_kheads=2, dim_v=256, dim_k=256, window=32, max_draft=8)
    with pytest.raises(_lib.RssmError) as e:
        replayssm_query_sizes(LayerConfig.of(big))
    assert e.value.status == _lib.RSSM_EUNSUPPORTED
    replayssm_query_sizes(LayerConfig.of(W.with_(big, window=16)))       # fits
    # a tile of three key groups stages 4 drafts' queries and keys for verify: too large
    multi = W.Shape(batch=2, n_vheads=3, n_kheads=3, dim_v=44, dim_k=256, window=13, max_draft=4)
    with pytest.raises(_lib.RssmError) as e:
        replayssm_query_sizes(LayerConfig.of(multi, heads_per_tile=3))
    assert e.value.status == _lib.RSSM_EUNSUPPORTED
    replayssm_query_sizes(LayerConfig.of(multi, heads_per_tile=1))        # in registers: fits
    replayssm_query_sizes(LayerConfig.of(W.with_(multi, max_draft=0), heads_per_tile=3))


def test_default_tile_rule():
    """Default tile: one key group's share of at most 128 rows; MXFP4 copies,
    and fp8 copies of heads of at most 64 rows, take tiles of two heads where
    the split decode applies (windows up to 16, key dims 64 or 128, at most 128
    rows per head); otherwise doubled
    while a tile's narrow read data (copy or fp16 checkpoint) is under 32 KiB,
    its rows stay within 256, its decode LDS within 28 KiB and, except for
    MXFP4, it stays inside one key group."""
    shared = W.with_(W.MAMBA2, n_kheads=1)                          # g = 128, P = 64
    cases = [
        (W.MAMBA2, "none", "f32", 1),          # g = 1
        (W.MAMBA2, "fp8", "f32", 2),           # split decode: two heads of 128 threads each
        (W.MAMBA2, "bf16", "f32", 1),
        (W.MAMBA2, "none", "f16sr", 1),
        (W.MAMBA2, "mxfp4", "f32", 2),         # split decode
        (W.with_(W.MAMBA2, window=32), "mxfp4", "f32", 1),   # window beyond the split decode: LDS caps it at 1
        (W.with_(W.MAMBA2, window=32), "fp8", "f32", 1),
        (W.with_(W.MAMBA2, dim_k=256), "fp8", "f32", 1),    # key dim beyond the split decode, in-group widening
        (W.GDN, "none", "f32", 1),             # g = 4, P = 128: 128-row cap
        (W.GDN, "fp8", "f32", 2),              # 16 KiB -> 32 KiB (tile-wide decode: 128-row heads)
        (W.LONG, "fp8", "f32", 1),             # 128-row heads of one key group each
        (W.LONG, "mxfp4", "f32", 2),           # split decode
        (W.GDN, "bf16", "f32", 1),             # already 32 KiB
        (W.GDN, "none", "f16sr", 1),           # fp16 rows of 128 heads: 32 KiB
        (shared, "none", "f32", 2),
        (shared, "fp8", "f32", 2),
        (shared, "bf16", "f32", 2),
    ]
    for shape, rc, ck, hvpt in cases:
        _, tiles = replayssm_query_sizes(LayerConfig.of(shape, read_copy=rc, ckpt=ck))
        assert tiles == shape.n_vheads // hvpt, (shape, rc, ck, tiles)


def test_f16_checkpoint_sizes():
    s32, _ = replayssm_query_sizes(LayerConfig.of(W.MAMBA2))
    s16, t16 = replayssm_query_sizes(LayerConfig.of(W.MAMBA2, ckpt="f16sr"))
    assert s16[_lib.RSSM_BUF_CKPT] * 2 == s32[_lib.RSSM_BUF_CKPT]
    assert s32[_lib.RSSM_BUF_FOLDS] == 0 and s16[_lib.RSSM_BUF_FOLDS] == W.MAMBA2.batch * t16 * 4
    assert all(s16[i] == s32[i] for i in range(1, _lib.RSSM_NUM_BUFS)
               if i not in (_lib.RSSM_BUF_COUNT, _lib.RSSM_BUF_FOLDS))
    bad = LayerConfig(**{**LayerConfig.of(W.TINY).__dict__, "ckpt": "f32"}).c()
    bad.ckpt_fmt = 7
    sizes = (ctypes.c_size_t * _lib.RSSM_NUM_BUFS)()
    assert _lib.load().replayssm_query_sizes(ctypes.byref(bad), sizes, None) == _lib.RSSM_EINVAL


def test_static_commit_host_checks():
    """replayssm_commit_static: a handle may be created without a commit work
    area (then replayssm_commit refuses it); layers of more tiles than the
    library's array holds are refused before any HIP call, as are commits
    without a pending verify; the header's limit is the binding's."""
    lib = _lib.load()
    fake = _FakeBufs()
    hdr = open(HEADER).read()
    m = re.search(r"#define RSSM_STATIC_COMMIT_MAX_TILES (\d+)", hdr)
    assert m and int(m.group(1)) == _lib.RSSM_STATIC_COMMIT_MAX_TILES
    cfg = LayerConfig.of(W.with_(W.TINY, max_draft=4))
    st, h = _create(cfg, fake, misalign="no work")
    assert st == _lib.RSSM_OK and h.value
    p = fake.ptr
    assert lib.replayssm_commit(h, p(0), None) == _lib.RSSM_EINVAL          # no work area
    assert lib.replayssm_commit_static(h, p(0), None) == _lib.RSSM_ESTATE   # no pending verify
    assert lib.replayssm_commit_static(h, None, None) == _lib.RSSM_EINVAL
    assert lib.replayssm_commit_static(h, p(4), None) == _lib.RSSM_EINVAL
    assert lib.replayssm_commit_static(None, p(0), None) == _lib.RSSM_EINVAL
    lib.replayssm_destroy(h)
    # 2049 sequences x 128 one-head tiles = 262272 tiles > 262144
    big = LayerConfig.of(W.with_(W.MAMBA2, batch=2049, max_draft=4))
    _, tiles = replayssm_query_sizes(big)
    assert 2049 * tiles > _lib.RSSM_STATIC_COMMIT_MAX_TILES
    st, h = _create(big, fake)
    assert st == _lib.RSSM_OK
    assert lib.replayssm_commit_static(h, p(0), None) == _lib.RSSM_EUNSUPPORTED
    lib.replayssm_destroy(h)


def test_fp8_checkpoint_sizes_and_validation():
    """An fp8 checkpoint needs a read copy (RSSM_EUNSUPPORTED without one);
    its rows take N + 16 bytes (codes and a scale trailer); it needs the
    fold-epoch buffer, one word per tile, like the fp16 checkpoint."""
    from ssm_layer_decode_amd.replayssm import replayssm_query_sizes
    with pytest.raises(_lib.RssmError) as e:
        replayssm_query_sizes(LayerConfig.of(W.TINY, ckpt="fp8sr"))
    assert e.value.status == _lib.RSSM_EUNSUPPORTED
    for copy in ("bf16", "fp8", "mxfp4"):
        sh = W.with_(W.MAMBA2, batch=4)
        sizes, tiles = replayssm_query_sizes(LayerConfig.of(sh, read_copy=copy, ckpt="fp8sr"))
        B, Hv, P, N = sh.batch, sh.n_vheads, sh.dim_v, sh.dim_k
        assert sizes[_lib.RSSM_BUF_CKPT] == B * Hv * P * (N + 16)
        assert sizes[_lib.RSSM_BUF_FOLDS] == B * tiles * 4
        ref, ref_tiles = replayssm_query_sizes(LayerConfig.of(sh, read_copy=copy))
        assert ref_tiles == tiles and sizes[_lib.RSSM_BUF_READ_COPY] == ref[_lib.RSSM_BUF_READ_COPY]
    fake = _FakeBufs()
    cfg = LayerConfig.of(W.with_(W.TINY, max_draft=4, dim_k=32), read_copy="mxfp4", ckpt="fp8sr")
    st, h = _create(cfg, fake)
    assert st == _lib.RSSM_OK and h.value
    assert _lib.load().replayssm_destroy(h) == _lib.RSSM_OK
    for bad in ("folds", "no folds"):
        st, h = _create(cfg, fake, misalign=bad)
        assert st == _lib.RSSM_EINVAL and not h.value

