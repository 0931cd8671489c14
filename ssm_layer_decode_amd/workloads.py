"""Seeded synthetic workloads for the ReplaySSM decode path.

This module only draws random inputs (alpha, k, v, q, draft records, accepted
prefix lengths, initial states).  It holds none of the method's arithmetic, so
both the HIP path (through the binding) and the fp64 oracle can consume the
same values without sharing any computation.

Shapes follow the decode-step signature of the library:
  alpha [B][Hv] fp32,  k, q [B][Hk][N],  v [B][Hv][P]   (fp32 or bf16 storage)
Draft records for speculative verification add a T axis after B.

Two generator back-ends are provided:
  * ``numpy`` -- ``Generator(PCG64(SeedSequence([seed, tag, step])))``; any step
    can be regenerated alone.  Used for sizes the oracle checks element by
    element.
  * ``torch`` on a device -- a ``torch.Generator`` seeded from the same
    (seed, tag, step) triple.  Used for the full serving shapes, where drawing
    gigabytes on the host would dominate the run.  Host copies of sampled
    slices feed the oracle, so both sides still see identical values.

Input distributions (the pages give none; these are the workload recipes):
  * ``mamba2``: alpha = exp(-softplus(x)) = sigmoid(-x), x ~ N(0,1), clamped to
    [0.8, 1); k, q, v ~ N(0, std = 1/sqrt(N)).
  * ``gdn``: alpha = sigmoid(y), y ~ N(2,1); k, q are N(0,1) vectors scaled to
    unit L2 norm; v ~ N(0,1).
  * ``uniform``: alpha ~ U(0.5, 1); k, q, v ~ N(0, 1/sqrt(N)) -- spreads the
    decays so ordering mistakes cannot hide behind equal alphas.
  * ``integer``: alpha = 1; k, q, v integers in [-4, 4] (fp32 arithmetic on these
    stays exact for the sizes used in tests).
bf16 storage rounds the fp64 draws to bf16 (round to nearest even) once; the
fp32 values handed to the oracle are the exact up-conversions of those bf16
values.
"""
from __future__ import annotations

import dataclasses
import hashlib
import math

import numpy as np

# Tags keep independent streams for the different kinds of draws.
TAG_DECODE = 0
TAG_DRAFT = 1
TAG_ACCEPT = 2
TAG_STATE0 = 3
TAG_PROJ = 4


@dataclasses.dataclass(frozen=True)
class Shape:
    batch: int
    n_vheads: int
    n_kheads: int
    dim_v: int      # P, value dim (rows of the state)
    dim_k: int      # N, key dim (columns of the state)
    window: int     # L
    max_draft: int = 0
    in_dtype: str = "f32"        # "f32" | "bf16" storage of k, q, v
    dist: str = "mamba2"         # see module docstring
    read_copy: str = "none"      # "none" | "bf16" | "fp8" | "mxfp4"
    ckpt: str = "f32"            # "f32" | "f16sr"

    @property
    def group(self) -> int:
        assert self.n_vheads % self.n_kheads == 0
        return self.n_vheads // self.n_kheads


def _seed_words(seed: int, tag: int, step: int) -> list[int]:
    return [int(seed), int(tag), int(step)]


def _rng(seed: int, tag: int, step: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence(_seed_words(seed, tag, step))))


def _torch_seed(seed: int, tag: int, step: int) -> int:
    h = hashlib.blake2b(f"{seed}/{tag}/{step}".encode(), digest_size=8).digest()
    return int.from_bytes(h, "little") & ((1 << 62) - 1)


def bf16_round_np(x: np.ndarray) -> np.ndarray:
    """Round fp64/fp32 values to bf16 (nearest, ties to even) and return them
    as float32 (exactly representable).  Input generation only."""
    import torch
    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32))
    return t.to(torch.bfloat16).to(torch.float32).numpy()


# --------------------------------------------------------------------------
# numpy back-end
# --------------------------------------------------------------------------
def _draw_np(rng: np.random.Generator, sh: Shape, lead: tuple):
    B, Hv, Hk, P, N = sh.batch, sh.n_vheads, sh.n_kheads, sh.dim_v, sh.dim_k
    if sh.dist == "mamba2":
        x = rng.standard_normal(lead + (Hv,))
        a = 1.0 / (1.0 + np.exp(x))              # exp(-softplus(x)) = sigmoid(-x)
        a = np.maximum(a, 0.8)
        s = 1.0 / math.sqrt(N)
        k = rng.normal(0.0, s, lead + (Hk, N))
        v = rng.normal(0.0, s, lead + (Hv, P))
        q = rng.normal(0.0, s, lead + (Hk, N))
    elif sh.dist == "gdn":
        y = rng.normal(2.0, 1.0, lead + (Hv,))
        a = 1.0 / (1.0 + np.exp(-y))
        k = rng.standard_normal(lead + (Hk, N))
        k /= np.linalg.norm(k, axis=-1, keepdims=True)
        v = rng.standard_normal(lead + (Hv, P))
        q = rng.standard_normal(lead + (Hk, N))
        q /= np.linalg.norm(q, axis=-1, keepdims=True)
    elif sh.dist == "uniform":
        a = rng.uniform(0.5, 1.0, lead + (Hv,))
        s = 1.0 / math.sqrt(N)
        k = rng.normal(0.0, s, lead + (Hk, N))
        v = rng.normal(0.0, s, lead + (Hv, P))
        q = rng.normal(0.0, s, lead + (Hk, N))
    elif sh.dist == "integer":
        a = np.ones(lead + (Hv,))
        k = rng.integers(-4, 5, lead + (Hk, N)).astype(np.float64)
        v = rng.integers(-4, 5, lead + (Hv, P)).astype(np.float64)
        q = rng.integers(-4, 5, lead + (Hk, N)).astype(np.float64)
    else:
        raise ValueError(f"unknown dist {sh.dist}")
    a = a.astype(np.float32)
    if sh.in_dtype == "bf16":
        k, v, q = bf16_round_np(k), bf16_round_np(v), bf16_round_np(q)
    else:
        k, v, q = k.astype(np.float32), v.astype(np.float32), q.astype(np.float32)
    return a, k, v, q


def decode_inputs_np(sh: Shape, seed: int, step: int):
    """One decode step's inputs: alpha [B][Hv], k [B][Hk][N], v [B][Hv][P],
    q [B][Hk][N], all float32 arrays (bf16-representable when in_dtype=bf16)."""
    return _draw_np(_rng(seed, TAG_DECODE, step), sh, (sh.batch,))


def decode_inputs_np_steps(sh: Shape, seed: int, steps: int):
    """All inputs of ``steps`` decode steps drawn at once in float32 (one
    generator; for bounded CPU timing samples): alpha [steps][B][Hv],
    k, q [steps][B][Hk][N], v [steps][B][Hv][P]."""
    rng = _rng(seed, TAG_DECODE, 2_000_000)
    lead = (steps, sh.batch)
    B, Hv, Hk, P, N = sh.batch, sh.n_vheads, sh.n_kheads, sh.dim_v, sh.dim_k
    f = np.float32
    if sh.dist != "mamba2" or sh.in_dtype != "f32":
        return _draw_np(rng, sh, lead)
    x = rng.standard_normal(lead + (Hv,), dtype=f)
    a = np.maximum(1.0 / (1.0 + np.exp(x)), f(0.8)).astype(f)
    s = f(1.0 / math.sqrt(N))
    k = rng.standard_normal(lead + (Hk, N), dtype=f) * s
    v = rng.standard_normal(lead + (Hv, P), dtype=f) * s
    q = rng.standard_normal(lead + (Hk, N), dtype=f) * s
    return a, k, v, q


def draft_inputs_np(sh: Shape, seed: int, rnd: int, T: int):
    """T draft records for one verify round: alpha [B][T][Hv], k [B][T][Hk][N],
    v [B][T][Hv][P], q [B][T][Hk][N]."""
    return _draw_np(_rng(seed, TAG_DRAFT, rnd), sh, (sh.batch, T))


def accepted_np(batch: int, T: int, seed: int, rnd: int) -> np.ndarray:
    """Accepted-prefix lengths, uniform in {0..T}, int32 [B]."""
    return _rng(seed, TAG_ACCEPT, rnd).integers(0, T + 1, batch).astype(np.int32)


def initial_state_np(sh: Shape, seed: int, std: float = 0.1) -> np.ndarray:
    """Initial fp32 state [B][Hv][P][N] ~ N(0, std^2)."""
    rng = _rng(seed, TAG_STATE0, 0)
    return rng.normal(0.0, std, (sh.batch, sh.n_vheads, sh.dim_v, sh.dim_k)).astype(np.float32)


# --------------------------------------------------------------------------
# torch (device) back-end, for the serving shapes
# --------------------------------------------------------------------------
def _draw_torch(gen, sh: Shape, lead: tuple, device):
    import torch
    B, Hv, Hk, P, N = sh.batch, sh.n_vheads, sh.n_kheads, sh.dim_v, sh.dim_k
    f32 = torch.float32
    if sh.dist == "mamba2":
        x = torch.randn(lead + (Hv,), generator=gen, device=device, dtype=f32)
        a = torch.sigmoid(-x).clamp_min(0.8)
        s = 1.0 / math.sqrt(N)
        k = torch.randn(lead + (Hk, N), generator=gen, device=device, dtype=f32) * s
        v = torch.randn(lead + (Hv, P), generator=gen, device=device, dtype=f32) * s
        q = torch.randn(lead + (Hk, N), generator=gen, device=device, dtype=f32) * s
    elif sh.dist == "gdn":
        y = torch.randn(lead + (Hv,), generator=gen, device=device, dtype=f32) + 2.0
        a = torch.sigmoid(y)
        k = torch.randn(lead + (Hk, N), generator=gen, device=device, dtype=f32)
        k = k / k.norm(dim=-1, keepdim=True)
        v = torch.randn(lead + (Hv, P), generator=gen, device=device, dtype=f32)
        q = torch.randn(lead + (Hk, N), generator=gen, device=device, dtype=f32)
        q = q / q.norm(dim=-1, keepdim=True)
    elif sh.dist == "uniform":
        a = torch.rand(lead + (Hv,), generator=gen, device=device, dtype=f32) * 0.5 + 0.5
        s = 1.0 / math.sqrt(N)
        k = torch.randn(lead + (Hk, N), generator=gen, device=device, dtype=f32) * s
        v = torch.randn(lead + (Hv, P), generator=gen, device=device, dtype=f32) * s
        q = torch.randn(lead + (Hk, N), generator=gen, device=device, dtype=f32) * s
    elif sh.dist == "integer":
        a = torch.ones(lead + (Hv,), device=device, dtype=f32)
        k = torch.randint(-4, 5, lead + (Hk, N), generator=gen, device=device).to(f32)
        v = torch.randint(-4, 5, lead + (Hv, P), generator=gen, device=device).to(f32)
        q = torch.randint(-4, 5, lead + (Hk, N), generator=gen, device=device).to(f32)
    else:
        raise ValueError(f"unknown dist {sh.dist}")
    if sh.in_dtype == "bf16":
        k, v, q = k.to(torch.bfloat16), v.to(torch.bfloat16), q.to(torch.bfloat16)
    return a.contiguous(), k.contiguous(), v.contiguous(), q.contiguous()


def _gen(device, seed, tag, step):
    import torch
    g = torch.Generator(device=device)
    g.manual_seed(_torch_seed(seed, tag, step))
    return g


def decode_inputs_torch(sh: Shape, seed: int, step: int, device="cuda"):
    """Device tensors for one decode step (k, v, q in the storage dtype)."""
    return _draw_torch(_gen(device, seed, TAG_DECODE, step), sh, (sh.batch,), device)


def decode_inputs_torch_steps(sh: Shape, seed: int, steps: int, device="cuda", first: int = 0):
    """All inputs of ``steps`` decode steps at once, on the device:
    alpha [steps][B][Hv], k, q [steps][B][Hk][N], v [steps][B][Hv][P].
    (Drawn from one generator seeded by ``first``; for staging benchmark runs.)"""
    return _draw_torch(_gen(device, seed, TAG_DECODE, 1_000_000 + first), sh, (steps, sh.batch), device)


def draft_inputs_torch(sh: Shape, seed: int, rnd: int, T: int, device="cuda"):
    return _draw_torch(_gen(device, seed, TAG_DRAFT, rnd), sh, (sh.batch, T), device)


def accepted_torch(batch: int, T: int, seed: int, rnd: int, device="cuda"):
    import torch
    g = _gen(device, seed, TAG_ACCEPT, rnd)
    return torch.randint(0, T + 1, (batch,), generator=g, device=device, dtype=torch.int32)


def initial_state_torch(sh: Shape, seed: int, std: float = 0.1, device="cuda"):
    import torch
    g = _gen(device, seed, TAG_STATE0, 0)
    return torch.randn((sh.batch, sh.n_vheads, sh.dim_v, sh.dim_k), generator=g,
                       device=device, dtype=torch.float32) * std


def projection_np(dim: int, vocab: int, seed: int = 2) -> np.ndarray:
    """Random N(0,1) projection [dim][vocab] used to turn outputs into logits."""
    return _rng(seed, TAG_PROJ, 0).standard_normal((dim, vocab))


# --------------------------------------------------------------------------
# The workloads the library is measured and checked on
# --------------------------------------------------------------------------
TINY = Shape(batch=2, n_vheads=2, n_kheads=2, dim_v=16, dim_k=16, window=16, dist="mamba2")
TINY_STEPS = 64

MAMBA2 = Shape(batch=256, n_vheads=128, n_kheads=128, dim_v=64, dim_k=128, window=16, dist="mamba2")
MAMBA2_STEPS = 256
MAMBA2_BATCH_SWEEP = (1, 32, 128, 256, 512)

GDN = Shape(batch=256, n_vheads=64, n_kheads=16, dim_v=128, dim_k=128, window=16,
            in_dtype="bf16", dist="gdn")
GDN_STEPS = 512

SPEC = Shape(batch=512, n_vheads=128, n_kheads=128, dim_v=64, dim_k=128, window=16,
             max_draft=4, dist="mamba2")
SPEC_T = 4

LONG = Shape(batch=64, n_vheads=64, n_kheads=64, dim_v=128, dim_k=128, window=16, dist="gdn")
LONG_STEPS = 4096
LONG_VOCAB = 512


def with_(sh: Shape, **kw) -> Shape:
    return dataclasses.replace(sh, **kw)
