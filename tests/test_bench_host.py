"""Host-side checks of bench.py's command line: more than one GPU is refused
with a message before any device is touched."""
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _bench(*args, env=None):
    return subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), *args], capture_output=True,
                          text=True, timeout=300, env=env, cwd=ROOT)


def test_more_than_one_gpu_is_refused():
    r = _bench("--gpus", "2")
    assert r.returncode == 2
    assert "one GPU" in r.stderr and "--gpus 2" in r.stderr
    assert r.stdout == ""


def test_distributed_launch_is_refused():
    env = dict(os.environ, WORLD_SIZE="4", RANK="0", LOCAL_RANK="0")
    r = _bench("--gpus", "1", env=env)
    assert r.returncode == 2
    assert "one GPU" in r.stderr


def _bench_mod():
    import importlib.util
    spec = importlib.util.spec_from_file_location("bench_mod", os.path.join(ROOT, "bench.py"))
    m = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(m)
    return m


def test_per_launch_labels_follow_the_layer_position():
    """The per-launch pass starts wherever the timed steps left the layer:
    after W warm-up and K timed steps a layer started empty sits at position
    (W + K) mod L.  Labels must follow that position, also when K is not a
    multiple of L (20 timed steps after 5 warm-up steps at L = 16)."""
    bench = _bench_mod()
    L = 16
    for Wm, K in ((5, 20), (16, 256), (3, 7), (0, 1), (15, 16), (7, 33)):
        h0 = (Wm + K) % L
        pos = bench.window_positions(h0, 2 * L, L)
        # brute force: simulate the record count through warm-up, timed and labelled steps
        h, sim = 0, []
        for i in range(Wm + K + 2 * L):
            if i >= Wm + K:
                sim.append(h)
            h = 0 if h + 1 == L else h + 1
        assert pos == sim, (Wm, K)
        # durations that reveal the label: flush steps take 2.0, others 1.0 + position / 100
        times = [2.0 if p == L - 1 else 1.0 + p / 100 for p in sim]
        nonflush, flush, per_pos = bench.split_launch_times(times, h0, L)
        assert flush == [2.0, 2.0] and len(nonflush) == 2 * (L - 1)
        assert all(x < 2.0 for x in nonflush)
        assert per_pos == [1.0 + j / 100 for j in range(L - 1)] + [2.0]


def test_window_of_one_record():
    bench = _bench_mod()
    nonflush, flush, per_pos = bench.split_launch_times([3.0, 5.0], 0, 1)
    assert nonflush == [] and flush == [3.0, 5.0] and per_pos == [4.0]


def test_bandwidth_fields_above_peak_are_flagged():
    bench = _bench_mod()
    ok = {"nonflush_GBps": 6200.0, "flush_GBps": 5700.0, "nested": {"achieved_GBps": 7999.0},
          "bytes_per_token": 1e9}
    assert bench.over_peak(ok) == []
    bad = {"flush_GBps": 13196.0, "nested": {"achieved_GBps": 8001.0, "x": 1}}
    assert bench.over_peak(bad) == ["flush_GBps", "nested.achieved_GBps"]


def test_fp8_checkpoint_workloads_and_bytes():
    """The fp8-checkpoint workloads name their copy; the byte model counts
    the checkpoint's codes and one fp32 scale per row (not the unused bytes
    of its 16-byte row trailer)."""
    from ssm_layer_decode_amd import bytes_model as bm
    from ssm_layer_decode_amd import workloads as W
    bench = _bench_mod()
    for rc in ("bf16", "fp8", "mxfp4"):
        sh, _ = bench.workload_shape(f"mamba2-fp8sr-{rc}")
        assert sh.ckpt == "fp8sr" and sh.read_copy == rc
    d = bm.Dims.of(W.with_(W.MAMBA2, ckpt="fp8sr", read_copy="mxfp4"))
    assert bm.state_bytes(d) == 128 * 64 * (128 + 4)
    assert bm.state_bytes(bm.Dims.of(W.MAMBA2)) == 128 * 64 * 128 * 4


def test_window_byte_optimum_moves_with_the_record():
    """The byte model's best window: near sqrt(2 S / record per head).  With a
    key per head (Mamba-2 serving shape) it is L = 8; with keys shared by
    groups of 16 heads the record shrinks and L = 16 is best."""
    from ssm_layer_decode_amd import bytes_model as bm
    from ssm_layer_decode_amd import workloads as W

    def best(hk):
        per = {L: bm.replay_bytes_per_token(bm.Dims.of(W.with_(W.MAMBA2, window=L, n_kheads=hk)))
               for L in (4, 8, 16, 32)}
        return min(per, key=per.get)

    assert best(128) == 8
    assert best(8) == 16
    assert best(1) == 16
