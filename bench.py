#!/usr/bin/env python3
"""ReplaySSM decode benchmark on one MI355X.

A "step" is one decode step of one SSM layer for the whole batch: every
sequence appends its record and produces its output, and on every L-th step the
buffered records are folded into the checkpoint (flush cost included, as in the
kernel numbers the pages report).  Inputs for all steps are drawn on the device
before timing; the timed region launches only the decode kernel, back to back
on torch's current stream, bracketed by HIP events on that stream.

Default workload: Mamba-2-style layer at serving shape -- batch 256, 128 heads,
P = 64, N = 128 (4 MiB fp32 state per sequence), L = 16, fp32 inputs.

Printed: one JSON line with the contract fields plus
  roofline      achieved algorithmic GB/s of the decode kernel vs 8 TB/s,
  cpu_baseline  the fp64 C oracle timed on this host's cores on a bounded sample,
  extras        the conventional fused decode on the same inputs (in-run GPU
                baseline), HBM copy/read probes, per-launch flush/non-flush times,
                and the decode with 4 independent layers rotated, so that the
                re-read records come from HBM rather than the on-die cache.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "SSM decode tokens/s at batch 256, L=16 + achieved HBM GB/s vs peak"
HBM_PEAK_GBS = 8000.0


# Sources the decode and conventional-decode kernels (and their launch set-up) are built
# from; the prefill, verify and probe kernels are left out so that a change there does not
# retire the decode traffic counters.
DECODE_SOURCES = ("conv_kernels.hip", "replayssm_api.hip", "rssm_decode_split.hip", "rssm_kernels.hip")


def kernel_source_sha() -> str:
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "ssm_layer_decode_amd", "csrc")
    for name in sorted(os.listdir(csrc)):
        if name.endswith(".h") or name in DECODE_SOURCES:
            h.update(name.encode())
            h.update(open(os.path.join(csrc, name), "rb").read())
    return h.hexdigest()[:16]


def workload_shape(name: str, batch=None):
    from ssm_layer_decode_amd import workloads as W
    if name == "mamba2":
        sh, steps = W.MAMBA2, W.MAMBA2_STEPS
    elif name == "mamba2-shared-k":
        sh, steps = W.with_(W.MAMBA2, n_kheads=1), W.MAMBA2_STEPS
    elif name == "gdn":
        sh, steps = W.GDN, W.GDN_STEPS
    elif name == "long-bf16":
        sh, steps = W.with_(W.LONG, read_copy="bf16"), 256
    elif name == "long-fp8":
        sh, steps = W.with_(W.LONG, read_copy="fp8"), 256
    elif name == "long-mxfp4":
        sh, steps = W.with_(W.LONG, read_copy="mxfp4"), 256
    elif name in ("gdn-bf16", "gdn-fp8", "gdn-mxfp4"):
        sh, steps = W.with_(W.GDN, read_copy=name.split("-")[1]), W.GDN_STEPS
    elif name in ("mamba2-bf16", "mamba2-fp8", "mamba2-mxfp4"):
        sh, steps = W.with_(W.MAMBA2, read_copy=name.split("-")[1]), W.MAMBA2_STEPS
    elif name in ("mamba2-f16sr", "mamba2-f16sr-fp8", "mamba2-f16sr-mxfp4"):
        rc = name.split("-")[2] if name.count("-") == 2 else "none"
        sh, steps = W.with_(W.MAMBA2, ckpt="f16sr", read_copy=rc), W.MAMBA2_STEPS
    elif name in ("mamba2-fp8sr-bf16", "mamba2-fp8sr-fp8", "mamba2-fp8sr-mxfp4"):
        sh, steps = W.with_(W.MAMBA2, ckpt="fp8sr", read_copy=name.split("-")[2]), W.MAMBA2_STEPS
    else:
        raise SystemExit(f"unknown workload {name}")
    if batch is not None:
        sh = W.with_(sh, batch=batch)
    return sh, steps


def describe(sh) -> str:
    return (f"B={sh.batch} Hv={sh.n_vheads} Hk={sh.n_kheads} P={sh.dim_v} N={sh.dim_k} "
            f"L={sh.window} in={sh.in_dtype} read_copy={sh.read_copy} ckpt={sh.ckpt}")


def time_loop(fn, n, stream):
    import torch
    start = torch.cuda.Event(enable_timing=True)
    end = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    start.record(stream)
    for i in range(n):
        fn(i)
    end.record(stream)
    torch.cuda.synchronize()
    return start.elapsed_time(end) / 1e3


def per_launch_times(fn, n, stream):
    """Per-launch durations from events recorded between launches (separate pass)."""
    import torch
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(n + 1)]
    torch.cuda.synchronize()
    ev[0].record(stream)
    for i in range(n):
        fn(i)
        ev[i + 1].record(stream)
    torch.cuda.synchronize()
    return [ev[i].elapsed_time(ev[i + 1]) / 1e3 for i in range(n)]


def window_positions(h0: int, n: int, L: int):
    """Window position (records buffered before the step, 0..L-1) of each of n
    consecutive decode launches of a layer that holds h0 records when the
    first of them starts; the launch at position L - 1 is the flush step."""
    return [(h0 + i) % L for i in range(n)]


def split_launch_times(times, h0: int, L: int):
    """Per-launch durations of consecutive decode steps starting at window
    position h0 -> (non-flush durations, flush durations, mean duration per
    window position).  The last is None unless every position was timed."""
    pos = window_positions(h0, len(times), L)
    nonflush = [x for x, p in zip(times, pos) if p != L - 1]
    flush = [x for x, p in zip(times, pos) if p == L - 1]
    per_pos = None
    if len(set(pos)) == L:
        per_pos = [sum(x for x, p in zip(times, pos) if p == j) / pos.count(j) for j in range(L)]
    return nonflush, flush, per_pos


def over_peak(obj, path="", peak=HBM_PEAK_GBS):
    """Paths of every numeric field named *GBps* in a nested dict whose value
    exceeds the HBM peak (a labelling or byte-model mistake: no kernel here
    moves more than the peak from HBM)."""
    bad = []
    if isinstance(obj, dict):
        for k, v in obj.items():
            p = f"{path}.{k}" if path else k
            if isinstance(v, (int, float)) and "GBps" in k and v > peak:
                bad.append(p)
            else:
                bad += over_peak(v, p, peak)
    return bad


def hbm_probes(dev, stream, nbytes=2 << 30, reps=10):
    """Practical ceilings on this device: a streaming copy and read (grid-stride),
    and a read of one 32 KiB chunk per workgroup without and with 1 KiB of plain
    stores per chunk (about a decode step's mix: appended record + output per
    32 KiB head of state)."""
    import torch
    from ssm_layer_decode_amd.probes import rssm_probe_copy, rssm_probe_read, rssm_probe_read_chunked
    src = torch.empty(nbytes // 4, dtype=torch.float32, device=dev).uniform_()
    dst = torch.empty_like(src)
    sink = torch.zeros(4, dtype=torch.float32, device=dev)
    rssm_probe_copy(dst, src)
    rssm_probe_read(src, sink)
    t_copy = time_loop(lambda i: rssm_probe_copy(dst, src), reps, stream)
    t_read = time_loop(lambda i: rssm_probe_read(src, sink), reps, stream)
    out = {"copy_GBps": 2 * nbytes * reps / t_copy / 1e9, "read_GBps": nbytes * reps / t_read / 1e9,
           "bytes": nbytes}
    for wb, key in ((0, "read_chunk32k_GBps"), (1024, "read_chunk32k_write1k_GBps")):
        rssm_probe_read_chunked(src, dst, wb, sink)
        t = time_loop(lambda i: rssm_probe_read_chunked(src, dst, wb, sink), reps, stream)
        out[key] = nbytes * reps / t / 1e9
    del src, dst
    return out


def cpu_baseline(sh, target_s: float, steps_max: int):
    """fp64 C oracle on a bounded sample of the same workload (fewer sequences,
    same per-sequence shape and distributions)."""
    import numpy as np
    from oracle import cpu_c
    from ssm_layer_decode_amd import workloads as W

    def run(nb, ns, nthreads):
        shs = W.with_(sh, batch=nb, read_copy="none")
        a, k, v, q = W.decode_inputs_np_steps(shs, 11, ns)
        S0 = np.zeros((nb, sh.n_vheads, sh.dim_v, sh.dim_k))
        t0 = time.perf_counter()
        cpu_c.decode(S0, a, k, v, q, want_outputs=True, nthreads=nthreads)
        return time.perf_counter() - t0

    cpu_c.build()
    threads = cpu_c.threads()
    nb = max(1, min(threads, sh.batch))
    run(nb, 8, threads)                               # warm-up (thread pool, page faults)
    per_token = run(nb, 16, threads) / (nb * 16)      # calibration
    tokens = max(nb * 16, int(target_s / per_token))
    ns2 = min(steps_max, max(16, tokens // nb))
    nb2 = max(1, min(sh.batch, (tokens // ns2) // nb * nb or nb))
    t2 = run(nb2, ns2, threads)
    # the same stepper on one core, on a sample of about 2 s
    per1 = run(1, 16, 1) / 16
    ns1 = min(steps_max, max(16, int(2.0 / per1)))
    nb1 = max(1, min(sh.batch, int(2.0 / per1) // ns1))
    t1 = run(nb1, ns1, 1)
    return ({"value": nb2 * ns2 / t2, "unit": "tokens/s", "cores": threads, "kind": "oracle",
             "sample": f"{nb2} sequences x {ns2} decode steps of the same layer shape "
                       f"({sh.n_vheads} heads, P={sh.dim_v}, N={sh.dim_k}), plain fp64 C stepper, "
                       f"{t2:.1f} s"},
            {"value": nb1 * ns1 / t1, "unit": "tokens/s", "cores": 1, "kind": "oracle",
             "sample": f"{nb1} sequences x {ns1} decode steps, {t1:.2f} s"})


def load_traffic(sha: str, workload: str, bytes_per_launch: float):
    path = os.path.join(ROOT, "profiles", f"rssm_decode_{workload}_traffic.json")
    if not os.path.exists(path):
        return None
    d = json.load(open(path))
    if d.get("kernel_src_sha") != sha:
        return None                                   # kernel changed since the counters were taken
    return d.get("hbm_bytes_per_launch")


# --------------------------------------------------------------------------
# Secondary measurements (``--suite``): one JSON line each
# --------------------------------------------------------------------------
def _decode_rate(sh, K, Wm, dev, stream, hvpt=0, layers=1, conv=False):
    """tokens/s of one layer's decode step (timed over K steps after Wm warm-up);
    `layers` independent layers are stepped round-robin so that their
    checkpoints do not stay resident in the 256 MB last-level cache."""
    import torch
    from ssm_layer_decode_amd import bytes_model as bm
    from ssm_layer_decode_amd import workloads as W
    from ssm_layer_decode_amd.replayssm import LayerConfig, ReplaySSM, convssm_decode_step
    a, k, v, q = W.decode_inputs_torch_steps(sh, 0, Wm + K, device=dev)
    o = torch.empty((sh.batch, sh.n_vheads, sh.dim_v), dtype=torch.float32, device=dev)
    cfg = LayerConfig.of(sh, heads_per_tile=hvpt)
    if conv:
        states = [torch.zeros((sh.batch, sh.n_vheads, sh.dim_v, sh.dim_k), device=dev) for _ in range(layers)]
        fn = lambda i: [convssm_decode_step(cfg, st, None, "f32", a[i], k[i], v[i], q[i], o) for st in states]
        per_tok = bm.conv_bytes_per_token(bm.Dims.of(sh))
    else:
        ls = [ReplaySSM(cfg, device=dev) for _ in range(layers)]
        fn = lambda i: [l.decode_step(a[i], k[i], v[i], q[i], o) for l in ls]
        per_tok = bm.replay_bytes_per_token(bm.Dims.of(sh))
    for i in range(Wm):
        fn(i)
    t = time_loop(lambda i: fn(Wm + i), K, stream)
    return sh.batch * K * layers / t, per_tok * sh.batch * K * layers / t / 1e9, t / (K * layers) * 1e6


def suite_decode(dev, stream, emit):
    from ssm_layer_decode_amd import workloads as W
    shared = W.with_(W.MAMBA2, n_kheads=1)
    cases = [("gdn", W.GDN, 0), ("gdn-hvpt2", W.GDN, 2), ("mamba2-shared-k", shared, 0),
             ("mamba2-shared-k-hvpt4", shared, 4)]
    for name, sh, hvpt in cases:
        r, g, us = _decode_rate(sh, 128, 16, dev, stream, hvpt=hvpt)
        rc, gc, usc = _decode_rate(sh, 128, 16, dev, stream, hvpt=hvpt, conv=True)
        emit({"suite": "decode", "case": name, "workload": describe(sh), "tokens_per_s": r, "GBps": g,
              "us_per_step": us, "conventional_tokens_per_s": rc, "conventional_GBps": gc, "speedup": r / rc})
    # windows with a key per head (the serving shape) and with keys shared by groups of 16 heads:
    # the best L moves with the record size (the byte model's minimum is near sqrt(2 S / record))
    from ssm_layer_decode_amd import bytes_model as bm
    for hk in (128, 8):
        for L in (4, 8, 16, 32):
            sh = W.with_(W.MAMBA2, window=L, n_kheads=hk)
            r, g, us = _decode_rate(sh, 4 * max(L, 16), 16 if L <= 16 else 32, dev, stream)
            emit({"suite": "window", "L": L, "key_heads": hk, "workload": describe(sh), "tokens_per_s": r,
                  "GBps": g, "us_per_step": us, "bytes_per_token": bm.replay_bytes_per_token(bm.Dims.of(sh))})
    for B in W.MAMBA2_BATCH_SWEEP:
        sh = W.with_(W.MAMBA2, batch=B)
        layers = max(1, -(-(1 << 30) // (B * 4 * (1 << 20))))
        K = 64 if B >= 128 else 32
        r, g, us = _decode_rate(sh, K, 16, dev, stream, layers=layers)
        rc, gc, usc = _decode_rate(sh, K, 16, dev, stream, layers=layers, conv=True)
        emit({"suite": "batch", "B": B, "layers_rotated": layers, "tokens_per_s": r, "GBps": g,
              "us_per_layer_step": us, "conventional_tokens_per_s": rc, "conventional_us_per_layer_step": usc,
              "speedup": r / rc})


def suite_spec(dev, stream, emit, rounds=32):
    """Speculative verify + commit at batch 512 (ReplaySSM output-only verify vs
    snapshot verify), for T = 1, 2, 4, 8, and a plain decode step for scale."""
    import torch
    from ssm_layer_decode_amd import bytes_model as bm
    from ssm_layer_decode_amd import workloads as W
    from ssm_layer_decode_amd.replayssm import (LayerConfig, ReplaySSM, convssm_commit,
                                                convssm_decode_step, convssm_spec_verify)
    base = W.SPEC
    # a standard decode step at the same batch (conventional and ReplaySSM)
    r_std, _, us_std = _decode_rate(W.with_(base, max_draft=0), 64, 16, dev, stream, conv=True)
    r_rep, _, us_rep = _decode_rate(W.with_(base, max_draft=0), 64, 16, dev, stream)
    for T in (1, 2, 4, 8):
        sh = W.with_(base, max_draft=T)
        cfg = LayerConfig.of(sh)
        nd = 8                                              # distinct draft sets, cycled
        drafts = [W.draft_inputs_torch(sh, 0, r, T, device=dev) for r in range(nd)]
        accs = [W.accepted_torch(sh.batch, T, 1, r, device=dev) for r in range(rounds)]
        layer = ReplaySSM(cfg, device=dev)
        layer.ckpt.copy_(W.initial_state_torch(sh, 1, device=dev))
        o = torch.empty((sh.batch, T, sh.n_vheads, sh.dim_v), device=dev)

        def rep(i):
            layer.spec_verify(*drafts[i % nd], o)
            layer.commit(accs[i])
        # warm-up: the first launch of a kernel loads its code object
        for i in range(2):
            layer.spec_verify(*drafts[i % nd], o)
            layer.commit(torch.zeros_like(accs[0]))
        t_rep = time_loop(rep, rounds, stream)
        # verify-only latency
        def rep_v(i):
            layer.spec_verify(*drafts[i % nd], o)
            layer.commit(torch.zeros_like(accs[0]))
        t_rep_v = time_loop(rep_v, rounds, stream)
        del layer
        ring = T + 1
        snaps = torch.zeros((sh.batch, ring, sh.n_vheads, sh.dim_v, sh.dim_k), device=dev)
        cur = torch.zeros(sh.batch, dtype=torch.int32, device=dev)
        err = torch.zeros(4, dtype=torch.int32, device=dev)

        def snap(i):
            convssm_spec_verify(cfg, snaps, cur, T, *drafts[i % nd], o)
            convssm_commit(cfg, cur, accs[i], T, err)
        for i in range(2):
            snap(i)
        cur.zero_()
        t_snap = time_loop(snap, rounds, stream)
        del snaps
        torch.cuda.empty_cache()
        committed = float(sum(int(a.sum()) for a in accs))
        d = bm.Dims.of(sh)
        emit({"suite": "spec", "T": T, "batch": sh.batch,
              "replay_us_per_round": t_rep / rounds * 1e6, "snapshot_us_per_round": t_snap / rounds * 1e6,
              "replay_verify_only_us": t_rep_v / rounds * 1e6,
              "replay_verified_tokens_per_s": sh.batch * T * rounds / t_rep,
              "snapshot_verified_tokens_per_s": sh.batch * T * rounds / t_snap,
              "replay_committed_tokens_per_s": committed / t_rep,
              "snapshot_committed_tokens_per_s": committed / t_snap,
              "speedup": t_snap / t_rep,
              "replay_verify_over_conv_decode_step": (t_rep_v / rounds * 1e6) / us_std,
              "snapshot_round_over_conv_decode_step": (t_snap / rounds * 1e6) / us_std,
              "conv_decode_step_us": us_std, "replay_decode_step_us": us_rep,
              "snapshot_bytes_per_round_per_seq": bm.snapshot_verify_bytes(d, T),
              "replay_verify_bytes_per_round_per_seq_h7": bm.replay_verify_bytes(d, 7, T)})


def suite_verify_h7(dev, stream, emit, reps=16):
    """Verify alone at batch 512 with every sequence holding h = 7 committed
    records (the window's mean), so each launch's algorithmic bytes are exact:
    T = 1, 2, 4, 8, each verify followed by a commit of nothing."""
    import torch
    from ssm_layer_decode_amd import bytes_model as bm
    from ssm_layer_decode_amd import workloads as W
    from ssm_layer_decode_amd.replayssm import LayerConfig, ReplaySSM
    h = 7
    for T in (1, 2, 4, 8):
        sh = W.with_(W.SPEC, max_draft=T)
        layer = ReplaySSM(LayerConfig.of(sh), device=dev)
        layer.ckpt.copy_(W.initial_state_torch(sh, 1, device=dev))
        for t in range(h):
            layer.decode_step(*W.decode_inputs_torch(sh, 2, t, device=dev))
        drafts = [W.draft_inputs_torch(sh, 3, r, T, device=dev) for r in range(4)]
        zero = torch.zeros(sh.batch, dtype=torch.int32, device=dev)
        o = torch.empty((sh.batch, T, sh.n_vheads, sh.dim_v), device=dev)
        for i in range(2):
            layer.spec_verify(*drafts[i % 4], o)
            layer.commit(zero)
        ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(reps)]
        for i in range(reps):
            ev[i][0].record(stream)
            layer.spec_verify(*drafts[i % 4], o)
            ev[i][1].record(stream)
            layer.commit(zero)
        torch.cuda.synchronize()
        assert layer.read_error() == 0 and int(layer.count[0, 0]) == h
        us = sum(a.elapsed_time(b) for a, b in ev) / reps * 1e3
        by = sh.batch * bm.replay_verify_bytes(bm.Dims.of(sh), h, T)
        emit({"suite": "verify_h7", "T": T, "batch": sh.batch, "h": h, "verify_us": us,
              "algorithmic_bytes_per_launch": by, "GBps": by / us / 1e3})
        del layer, drafts, o
        torch.cuda.empty_cache()


def suite_ceiling(dev, stream, emit, nbytes=2 << 30, reps=10):
    """The device's read ceiling as a function of the write share: the
    chunked-read probe (one 32 KiB chunk per workgroup, non-temporal loads)
    with 0 to 4 KiB of plain stores per chunk.  A kernel whose traffic mixes
    reads and writes in some proportion is measured against the ceiling at
    that proportion (decode: appended records + outputs; verify: the drafts'
    records + T outputs)."""
    import torch
    from ssm_layer_decode_amd.probes import rssm_probe_read_chunked
    src = torch.empty(nbytes // 4, dtype=torch.float32, device=dev).uniform_()
    dst = torch.empty(nbytes // 32768 * 4096 // 4, dtype=torch.float32, device=dev)
    sink = torch.zeros(4, dtype=torch.float32, device=dev)
    for wb in (0, 256, 512, 1024, 1536, 2048, 2816, 3584, 4096):
        rssm_probe_read_chunked(src, dst, wb, sink)
        t = time_loop(lambda i: rssm_probe_read_chunked(src, dst, wb, sink), reps, stream)
        moved = nbytes + nbytes // 32768 * wb
        emit({"suite": "ceiling", "write_bytes_per_32KiB": wb, "write_share": wb / (32768 + wb),
              "read_GBps": nbytes * reps / t / 1e9, "total_GBps": moved * reps / t / 1e9})
    del src, dst


def suite_graph(dev, stream, emit):
    """Decode steps of independent layers (Mamba-2 shape) launched one by one
    vs captured once in a HIP graph and replayed, at small batches where a
    step is launch-bound.  Both modes time one whole window per layer from an
    empty buffer (window positions 0..L-1, one flush), so they run the same
    steps."""
    import torch
    from ssm_layer_decode_amd import workloads as W
    from ssm_layer_decode_amd.replayssm import LayerConfig, ReplaySSM
    for B, layers in ((1, 64), (4, 32), (32, 8)):
        sh = W.with_(W.MAMBA2, batch=B)
        reps = sh.window
        ls = [ReplaySSM(LayerConfig.of(sh), device=dev) for _ in range(layers)]
        x = W.decode_inputs_torch(sh, 0, 0, device=dev)
        o = torch.empty((B, sh.n_vheads, sh.dim_v), device=dev)
        for layer in ls:                              # first launches (code loading)
            layer.decode_step(*x, o)
            layer.reset()
        t_eager = time_loop(lambda i: [layer.decode_step(*x, o) for layer in ls], reps, stream)
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            for layer in ls:
                layer.decode_step(*x, o)
        g.replay()
        for layer in ls:
            layer.reset()
        t_graph = time_loop(lambda i: g.replay(), reps, stream)
        emit({"suite": "graph", "B": B, "layers": layers,
              "eager_us_per_layer_step": t_eager / (reps * layers) * 1e6,
              "graph_us_per_layer_step": t_graph / (reps * layers) * 1e6})
        del ls, g, x, o
        torch.cuda.empty_cache()


def suite_spec_copies(dev, stream, emit, rounds=32):
    """Speculative verify + commit at batch 512 when verification reads a
    low-precision copy of the checkpoint or an fp16 checkpoint (T = 4, 8)."""
    import torch
    from ssm_layer_decode_amd import workloads as W
    from ssm_layer_decode_amd.replayssm import LayerConfig, ReplaySSM
    for ck, rc in (("f32", "none"), ("f32", "bf16"), ("f32", "fp8"), ("f32", "mxfp4"), ("f16sr", "none"),
                   ("fp8sr", "mxfp4")):
        for T in (4, 8):
            sh = W.with_(W.SPEC, max_draft=T)
            layer = ReplaySSM(LayerConfig.of(sh, read_copy=rc, ckpt=ck), device=dev)
            if ck != "fp8sr":                       # an fp8 checkpoint starts empty (zero codes and scales)
                S0 = W.initial_state_torch(sh, 1, device=dev)
                layer.ckpt.copy_(S0.half() if ck == "f16sr" else S0)
                del S0
            if rc != "none":
                layer.refresh_read_copy()
            nd = 8
            drafts = [W.draft_inputs_torch(sh, 0, r, T, device=dev) for r in range(nd)]
            accs = [W.accepted_torch(sh.batch, T, 1, r, device=dev) for r in range(rounds)]
            zero = torch.zeros_like(accs[0])
            o = torch.empty((sh.batch, T, sh.n_vheads, sh.dim_v), device=dev)

            def rep(i):
                layer.spec_verify(*drafts[i % nd], o)
                layer.commit(accs[i])

            def rep_v(i):
                layer.spec_verify(*drafts[i % nd], o)
                layer.commit(zero)
            for i in range(2):
                rep_v(i)
            t_rep = time_loop(rep, rounds, stream)
            t_v = time_loop(rep_v, rounds, stream)
            assert layer.read_error() == 0
            emit({"suite": "spec_copies", "ckpt": ck, "read_copy": rc, "T": T, "batch": sh.batch,
                  "heads_per_tile": sh.n_vheads // layer.tiles,
                  "us_per_round": t_rep / rounds * 1e6, "verify_only_us": t_v / rounds * 1e6,
                  "verified_tokens_per_s": sh.batch * T * rounds / t_rep})
            del layer, drafts, o
            torch.cuda.empty_cache()


def suite_copies(dev, stream, emit):
    """Decode with a low-precision read copy and/or an fp16 or fp8 checkpoint
    (long-decode shape, and the Mamba-2 serving shape)."""
    from ssm_layer_decode_amd import workloads as W
    for base, name in ((W.LONG, "long"), (W.MAMBA2, "mamba2")):
        for ck in ("f32", "f16sr", "fp8sr"):
            for rc in ("none", "bf16", "fp8", "mxfp4"):
                if ck == "f16sr" and rc == "bf16":
                    continue                               # a bf16 copy of an fp16 checkpoint saves nothing
                if ck == "fp8sr" and rc == "none":
                    continue                               # an fp8 checkpoint is read through a copy
                sh = W.with_(base, read_copy=rc, ckpt=ck)
                layers = 1 if name == "mamba2" else 4      # 4 x 256 MiB checkpoints: beyond the 256 MB cache
                r, g, us = _decode_rate(sh, 64, 16, dev, stream, layers=layers)
                emit({"suite": "read_copy", "case": name, "read_copy": rc, "ckpt": ck, "workload": describe(sh),
                      "layers_rotated": layers, "tokens_per_s": r, "GBps": g, "us_per_layer_step": us})


def prefill_flops_per_token(sh) -> float:
    """Arithmetic of prefill per token and sequence: S q and the fold (2 P N
    each per value head), the chunk's scores (2 N per earlier record of the
    window, about L/2, per key head) and the replay sum (2 P per record)."""
    half = sh.window / 2
    return (4 * sh.dim_v * sh.dim_k * sh.n_vheads + 2 * sh.dim_k * half * sh.n_kheads
            + 2 * sh.dim_v * half * sh.n_vheads)


def suite_prefill(dev, stream, emit, T=512):
    """Prefill of a T-token prompt from an empty state vs T decode steps."""
    import torch
    from ssm_layer_decode_amd import bytes_model as bm
    from ssm_layer_decode_amd import workloads as W
    from ssm_layer_decode_amd.replayssm import LayerConfig, ReplaySSM
    for name, sh in (("mamba2", W.MAMBA2), ("gdn", W.GDN), ("mamba2-f16sr", W.with_(W.MAMBA2, ckpt="f16sr")),
                     ("mamba2-fp8sr-mxfp4", W.with_(W.MAMBA2, ckpt="fp8sr", read_copy="mxfp4"))):
        a, k, v, q = W.draft_inputs_torch(W.with_(sh, max_draft=T), 0, 0, T, device=dev)
        o = torch.empty((sh.batch, T, sh.n_vheads, sh.dim_v), device=dev)
        layer = ReplaySSM(LayerConfig.of(sh), device=dev)
        layer.prefill(a, k, v, q, o)                     # warm-up
        torch.cuda.synchronize()
        reps = 3
        t_pf = min(time_loop(lambda i: (layer.reset(), layer.prefill(a, k, v, q, o)), 1, stream) for _ in range(reps))
        # decode of the same tokens, step inputs made contiguous beforehand
        steps = [(a[:, t].contiguous(), k[:, t].contiguous(), v[:, t].contiguous(), q[:, t].contiguous())
                 for t in range(T)]
        o1 = torch.empty((sh.batch, sh.n_vheads, sh.dim_v), device=dev)
        layer.reset()
        t_dec = time_loop(lambda i: layer.decode_step(*steps[i], o1), T, stream)
        del steps
        d = bm.Dims.of(sh)
        e = 2 if sh.in_dtype == "bf16" else 4
        in_bytes = (sh.n_vheads * 4 + (2 * sh.n_kheads * sh.dim_k + sh.n_vheads * sh.dim_v) * e
                    + sh.n_vheads * sh.dim_v * 4)       # alpha, k, q, v read; o written
        tot = sh.batch * (T * in_bytes + 2 * bm.state_bytes(d))
        fl = sh.batch * T * prefill_flops_per_token(sh)
        mfma = sh.window == 16 and sh.dim_v % 16 == 0 and sh.dim_k % 16 == 0
        # the reset kernel zeroes the checkpoint inside the timed call: time it alone
        t_reset = min(time_loop(lambda i: layer.reset(), 1, stream) for _ in range(reps))
        t_net = t_pf - t_reset
        emit({"suite": "prefill", "case": name, "workload": describe(sh), "T": T,
              "prefill_ms": t_net * 1e3, "prefill_tokens_per_s": sh.batch * T / t_net,
              "decode_tokens_per_s": sh.batch * T / t_dec, "speedup_vs_decode": t_dec / t_net,
              "algorithmic_GBps": tot / t_net / 1e9, "TFLOPs": fl / t_net / 1e12,
              # 16-record windows with P, N multiples of 16 run on the fp32 matrix cores
              "kernel": "rssm_prefill_mfma_kernel" if mfma else "rssm_prefill_kernel",
              "TFLOPs_peak": 157.3 if mfma else 78.6,
              "peak_of": "fp32 MFMA" if mfma else "fp32 VALU (packed ops disabled)"})
        del a, k, v, q, o, layer
        torch.cuda.empty_cache()


def run_suite(parts):
    import torch
    from ssm_layer_decode_amd import _lib
    _lib.load()
    dev = torch.device("cuda:0")
    stream = torch.cuda.current_stream()
    emit = lambda d: print(json.dumps(d), flush=True)
    if "decode" in parts:
        suite_decode(dev, stream, emit)
    if "spec" in parts:
        suite_spec(dev, stream, emit)
    if "copies" in parts:
        suite_copies(dev, stream, emit)
    if "spec_copies" in parts:
        suite_spec_copies(dev, stream, emit)
    if "verify_h7" in parts:
        suite_verify_h7(dev, stream, emit)
    if "graph" in parts:
        suite_graph(dev, stream, emit)
    if "ceiling" in parts:
        suite_ceiling(dev, stream, emit)
    if "prefill" in parts:
        suite_prefill(dev, stream, emit)


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=None, help="timed decode steps (default: the workload's)")
    ap.add_argument("--warmup", type=int, default=16)
    ap.add_argument("--workload", default="mamba2")
    ap.add_argument("--batch", type=int, default=None)
    ap.add_argument("--heads-per-tile", type=int, default=0)
    ap.add_argument("--no-cpu", action="store_true")
    ap.add_argument("--no-baselines", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=15.0)
    ap.add_argument("--copy-probe", action="store_true",
                    help="after the decode, one 2 GiB copy by the library's copy probe (the calibration "
                         "kernel of FETCH_SIZE / WRITE_SIZE counter runs)")
    ap.add_argument("--suite", default=None,
                    help="comma list of secondary measurements: decode,spec,copies,spec_copies,verify_h7,graph,prefill,ceiling "
                         "(one JSON line each)")
    args = ap.parse_args()

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py measures one GPU: the ReplaySSM layer shards by sequence and head with no "
              "exchange between GPUs, so the multi-GPU rate is N times the single-GPU rate of each "
              f"shard; run it with --gpus 1 (asked for --gpus {args.gpus}).", file=sys.stderr)
        sys.exit(2)

    if args.suite:
        run_suite(args.suite.split(","))
        return

    import torch
    from ssm_layer_decode_amd import _lib
    from ssm_layer_decode_amd import bytes_model as bm
    from ssm_layer_decode_amd import workloads as W
    from ssm_layer_decode_amd.replayssm import LayerConfig, ReplaySSM, convssm_decode_step

    _lib.load()
    if not torch.cuda.is_available():
        raise SystemExit("bench.py needs a GPU")
    dev = torch.device("cuda:0")
    stream = torch.cuda.current_stream()

    sh, default_steps = workload_shape(args.workload, args.batch)
    K = args.steps if args.steps is not None else default_steps
    Wm = args.warmup
    L = sh.window
    dims = bm.Dims.of(sh)

    # inputs for warmup + timed steps, resident in HBM before timing
    a, k, v, q = W.decode_inputs_torch_steps(sh, 0, Wm + K, device=dev)
    o = torch.empty((sh.batch, sh.n_vheads, sh.dim_v), dtype=torch.float32, device=dev)

    layer = ReplaySSM(LayerConfig.of(sh, heads_per_tile=args.heads_per_tile), device=dev)
    step = lambda i: layer.decode_step(a[i], k[i], v[i], q[i], o)
    for i in range(Wm):
        step(i)
    flushes = sum(1 for i in range(Wm, Wm + K) if (i + 1) % L == 0)
    t = time_loop(lambda i: step(Wm + i), K, stream)
    assert layer.read_error() == 0

    tokens_s = sh.batch * K / t
    ms_step = t / K * 1e3
    # algorithmic bytes of exactly the timed launches (window position of each step)
    alg_bytes = sum(bm.replay_step_bytes(dims, (i % L)) for i in range(Wm, Wm + K)) * sh.batch
    achieved = alg_bytes / t / 1e9
    sha = kernel_source_sha()

    extras = {"kernel_src_sha": sha, "flush_steps_timed": flushes,
              "bytes_per_token": bm.replay_bytes_per_token(dims),
              "state_bytes_per_token": bm.replay_state_bytes_per_token(dims),
              "tiles_per_seq": layer.tiles}
    # per-launch durations (a separate pass over the next two windows, after the
    # timed steps): each launch is labelled by the window position the layer
    # is at when it starts, read from the layer's record count
    torch.cuda.synchronize()
    h0 = int(layer.count[0, 0])
    lt = per_launch_times(lambda i: step(Wm + (i % K)), 2 * L, stream)
    nonflush, flush, per_pos = split_launch_times(lt, h0, L)
    extras["per_launch_start_position"] = h0
    if nonflush:
        extras["nonflush_launch_us"] = 1e6 * sum(nonflush) / len(nonflush)
        nf_bytes = sh.batch * sum(bm.replay_step_bytes(dims, h) for h in range(L - 1)) / (L - 1)
        extras["nonflush_GBps"] = nf_bytes / 1e9 / (extras["nonflush_launch_us"] / 1e6)
    extras["flush_launch_us"] = 1e6 * sum(flush) / len(flush)
    extras["flush_GBps"] = sh.batch * bm.replay_step_bytes(dims, L - 1) / 1e9 / (extras["flush_launch_us"] / 1e6)
    # whole-window figure from the per-position launch times, comparable with
    # a headline whose step count is not a multiple of L
    extras["window_avg_us"] = 1e6 * sum(per_pos) / L
    extras["window_avg_GBps"] = (sh.batch * bm.replay_bytes_per_token(dims) / 1e9
                                 / (extras["window_avg_us"] / 1e6))
    if not args.no_baselines:
        # The same decode with NL independent layers rotated: a step's earlier
        # records were then written NL layer-steps ago, as in a model with many
        # layers, instead of partly sitting in the 256 MB on-die cache (one
        # layer at this shape writes ~25 MB of records per step).
        NL = 4
        layers = [layer] + [ReplaySSM(LayerConfig.of(sh, heads_per_tile=args.heads_per_tile), device=dev)
                            for _ in range(NL - 1)]
        for lyr in layers[1:]:
            for i in range(Wm):
                lyr.decode_step(a[i], k[i], v[i], q[i], o)
        nc = NL * 2 * L
        cold = lambda i: layers[i % NL].decode_step(*(x[Wm + (i // NL) % K] for x in (a, k, v, q)), o)
        tcold = time_loop(cold, nc, stream)
        assert all(lyr.read_error() == 0 for lyr in layers)
        cold_bytes = sh.batch * bm.replay_bytes_per_token(dims) * nc
        extras["records_cache_cold"] = {"layers_rotated": NL, "tokens_per_s": sh.batch * nc / tcold,
                                        "ms_per_layer_step": tcold / nc * 1e3,
                                        "achieved_GBps": cold_bytes / tcold / 1e9,
                                        "frac": cold_bytes / tcold / 1e9 / HBM_PEAK_GBS}
        del layers, lyr
    del layer

    if not args.no_baselines:
        conv_fmt = "f32"
        state = torch.zeros((sh.batch, sh.n_vheads, sh.dim_v, sh.dim_k), dtype=torch.float32, device=dev)
        ccfg = LayerConfig.of(sh, heads_per_tile=args.heads_per_tile)
        cstep = lambda i: convssm_decode_step(ccfg, state, None, conv_fmt, a[i], k[i], v[i], q[i], o)
        for i in range(Wm):
            cstep(i)
        tc = time_loop(lambda i: cstep(Wm + i), K, stream)
        conv_bytes = bm.conv_bytes_per_token(dims) * sh.batch * K
        extras["conventional"] = {"tokens_per_s": sh.batch * K / tc, "ms_per_step": tc / K * 1e3,
                                  "achieved_GBps": conv_bytes / tc / 1e9,
                                  "bytes_per_token": bm.conv_bytes_per_token(dims),
                                  "state_bytes_per_token": bm.conv_state_bytes_per_token(dims)}
        extras["speedup_vs_conventional"] = tokens_s / extras["conventional"]["tokens_per_s"]
        extras["state_bytes_ratio_conv_over_replay"] = (bm.conv_state_bytes_per_token(dims) /
                                                        bm.replay_state_bytes_per_token(dims))
        del state
        torch.cuda.empty_cache()
        extras["hbm_probe"] = hbm_probes(dev, stream)

    del a, k, v, q
    torch.cuda.empty_cache()
    if args.copy_probe:
        from ssm_layer_decode_amd.probes import rssm_probe_copy
        src = torch.empty((2 << 30) // 4, dtype=torch.float32, device=dev).uniform_()
        dst = torch.empty_like(src)
        rssm_probe_copy(dst, src)
        torch.cuda.synchronize()
        del src, dst
        torch.cuda.empty_cache()

    roofline = {"bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": achieved / HBM_PEAK_GBS,
                "traffic": load_traffic(sha, args.workload, alg_bytes / K),
                "kernel": "rssm_decode_kernel", "algorithmic_bytes_per_launch": alg_bytes / K,
                "avg_launch_us": t / K * 1e6}

    cpu = None
    if not args.no_cpu:
        cpu, extras["cpu_oracle_one_core"] = cpu_baseline(sh, args.cpu_seconds, K)

    bad = over_peak(extras) + (["roofline.achieved"] if achieved > HBM_PEAK_GBS else [])
    if bad:
        print(f"bench.py: bandwidth figures above the {HBM_PEAK_GBS:.0f} GB/s peak: {bad}", file=sys.stderr)
        extras["over_peak"] = bad

    line = {
        "metric": METRIC, "value": tokens_s, "unit": "tokens/s", "n_gpus": 1, "steps": K,
        "warmup": Wm, "ms_per_step": ms_step, "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "f32", "data": "synthetic",
        "config": {"workload": f"{args.workload} layer decode, {describe(sh)}", "batch": sh.batch,
                   "heads": sh.n_vheads, "dim_v": sh.dim_v, "dim_k": sh.dim_k, "window": L,
                   "parallelism": "single GPU"},
        "roofline": roofline, "cpu_baseline": cpu, "extras": extras,
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
