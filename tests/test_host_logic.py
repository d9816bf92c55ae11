"""Host-side logic pinned to what the pages fix: combination counts, the iso-parameter /
iso-FLOP algebra of fine-grained segmentation, and the bench's work counters."""
import json
import math
import os

import pytest

import bench
import synth

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def load(name):
    with open(os.path.join(GOLDEN, name)) as fh:
        return json.load(fh)


def test_combination_counts_printed_on_the_pages():
    g = load("combinatorics.json")
    for c in g["cases"]:
        assert math.comb(c["n"], c["k"]) == c["value"], c["cite"]
    for c in g["approx"]:
        assert abs(math.comb(c["n"], c["k"]) / c["value"] - 1) <= c["rel"], c["cite"]


@pytest.mark.parametrize("act_swiglu", [True, False])
def test_iso_parameter_iso_flop_counters(act_swiglu):
    """Splitting N experts of width M into mN of width M/m, top-mK: parameters and activated
    FLOPs unchanged (llm-infra-atlas 02, section 2.1)."""
    for c in load("iso_budget.json")["cases"]:
        N, K, M, H, m = c["N"], c["K"], c["M"], c["H"], c["m"]
        assert bench.ffn_params(m * N, H, M // m, act_swiglu) == bench.ffn_params(N, H, M, act_swiglu)
        assert bench.ffn_flops_per_token(m * K, H, M // m, act_swiglu) == \
            bench.ffn_flops_per_token(K, H, M, act_swiglu)
        # and the counters are linear in the expert count and width (not e.g. quadratic)
        assert bench.ffn_params(2 * N, H, M, act_swiglu) == 2 * bench.ffn_params(N, H, M, act_swiglu)
        assert bench.ffn_flops_per_token(K, H, 2 * M, act_swiglu) == 2 * bench.ffn_flops_per_token(K, H, M,
                                                                                                  act_swiglu)


def test_layer_flop_count_at_the_v3_shape():
    w = synth.WORKLOADS["c3p"]
    # router 2*T*H*N_r + gate/up/down of the 8 routed and 1 shared experts
    expect = 2 * w.T * w.H * w.N_r + 2 * w.T * 9 * 3 * w.H * w.I
    assert bench.layer_flops(w) == expect
    assert bench.routed_up_flops(w) == 2 * w.T * 8 * 2 * w.I * w.H
    # shared experts count at the same iso budget as routed ones: Ks=1 adds one expert's FLOPs
    assert bench.layer_flops(w.with_(Ks=0)) + 2 * w.T * 3 * w.H * w.I == expect


def test_decode_byte_count():
    w = synth.WORKLOADS["c3d"]
    per_expert = 3 * w.H * w.I * 2
    b = bench.decode_bytes(w, 140)
    assert b == 141 * per_expert + w.N_r * w.H * 2 + 2 * w.T * w.H * 2
    assert bench.decode_bytes(w, 141) - b == per_expert


def test_gpus_above_one_exit_with_a_message(capsys):
    import subprocess
    import sys
    r = subprocess.run([sys.executable, os.path.join(bench.ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True)
    assert r.returncode == 2 and "one GPU" in r.stderr


def test_traffic_is_reported_only_for_the_measured_source(tmp_path, monkeypatch):
    k = bench.dominant_kernel(0)
    t = {"traffic_bytes_per_launch": 123.0, "source_sha256": bench.kernel_source_hash(), "dominant_kernel": k}
    p = tmp_path / "t.json"
    p.write_text(json.dumps(t))
    monkeypatch.setattr(bench, "TRAFFIC_FILE", str(p))
    monkeypatch.setattr(bench, "ROOT", bench.ROOT)
    assert bench.measured_traffic(k) == 123.0
    # counters of the other dominant kernel (the other weight layout) are not reported
    assert bench.measured_traffic(bench.dominant_kernel(1)) is None
    t["source_sha256"] = "0" * 64
    p.write_text(json.dumps(t))
    assert bench.measured_traffic(k) is None
