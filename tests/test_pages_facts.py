"""The byte model against the traffic facts the pages state in prose
(tests/golden/pages_facts.json, each entry cited)."""
import json
import os

import pytest

from ssm_layer_decode_amd import bytes_model as bm
from ssm_layer_decode_amd import workloads as W

FACTS = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "pages_facts.json")))


@pytest.mark.parametrize("shape", [W.MAMBA2, W.GDN, W.SPEC, W.LONG])
def test_serving_shapes_hold_four_mib_of_state(shape):
    assert bm.state_bytes(bm.Dims.of(shape)) == FACTS["state_bytes_per_sequence_per_layer"]["value"]


def test_state_equals_kv_of_8k_tokens():
    f = FACTS
    assert f["state_bytes_per_sequence_per_layer"]["value"] // f["kv_entry_bytes_per_token"]["value"] \
        == f["state_equivalent_kv_tokens"]["value"]


def test_state_traffic_per_window():
    """conv: L reads + L writes; replay: L reads + 1 write  ->  ratio 2L/(L+1),
    'roughly half'."""
    d = bm.Dims.of(W.MAMBA2)
    L = FACTS["window_records"]["value"]
    assert d.window == L
    S = bm.state_bytes(d)
    conv = (FACTS["conv_state_reads_per_window"]["value"] + FACTS["conv_state_writes_per_window"]["value"]) * S / L
    rep = (FACTS["replay_state_reads_per_window"]["value"] + FACTS["replay_state_writes_per_window"]["value"]) * S / L
    assert bm.conv_state_bytes_per_token(d) == conv
    assert bm.replay_state_bytes_per_token(d) == rep
    ratio = conv / rep
    assert ratio == pytest.approx(2 * L / (L + 1))
    assert abs(ratio - FACTS["dominant_traffic_ratio_approx"]["value"]) < 0.15


def test_total_bytes_per_token_serving_shape():
    d = bm.Dims.of(W.MAMBA2)
    # conventional: 2 x 4 MiB state + k, q (64 KiB each), v (32 KiB), alpha, o (32 KiB)
    assert bm.conv_bytes_per_token(d) == 8 * 2 ** 20 + 65536 * 2 + 32768 + 512 + 32768
    rep = bm.replay_bytes_per_token(d)
    rec = 65536 + 32768 + 512
    expect = 4 * 2 ** 20 + 4 * 2 ** 20 / 16 + 7.5 * rec + rec + rec * 15 / 16 + 65536 + 32768
    assert rep == pytest.approx(expect)
    assert 1.5 < bm.conv_bytes_per_token(d) / rep < 1.7


def test_config_constants_match_pages():
    assert W.MAMBA2.batch == FACTS["serving_batch"]["value"]
    assert W.SPEC.batch == FACTS["spec_batch"]["value"] and W.SPEC_T == FACTS["draft_length"]["value"]
    f = FACTS["tiny_workload_flushes"]
    assert (W.TINY_STEPS, W.TINY.window) == (f["steps"], f["window"])
    assert W.TINY_STEPS // W.TINY.window == f["value"]
