"""The measurement model of bench.py (CPU only): the algorithmic bytes and
FLOP that every roofline fraction divides by, checked against figures derived
independently from the model shapes (a hand-derived decode-bytes and
prefill-FLOP table), and the gating of the measured-traffic record."""
import json
import os

import pytest

import synthetic as S

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.fixture(scope="module")
def bench():
    import importlib.util
    spec = importlib.util.spec_from_file_location("bench_under_test", os.path.join(ROOT, "bench.py"))
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    return mod


def mid_context(w):
    return w.prompt_len + (w.decode_steps - 1) / 2.0


@pytest.mark.parametrize("name,mb", [("0.5b", 990.3), ("1.5b", 3105.5), ("1.5b-prefill", 3560.6),
                                     ("1.5b-longctx", 10662.0)])
def test_decode_step_bytes(bench, name, mb):
    w = S.WORKLOADS[name]
    assert bench.decode_step_bytes(w, mid_context(w)) / 1e6 == pytest.approx(mb, rel=2e-3)


def test_decode_step_bytes_by_hand(bench):
    # 0.5B: every weight once (bf16) + K and V of 192.5 positions, written by hand
    w = S.WORKLOADS["0.5b"]
    per_layer = 896 * (896 + 2 * 128) + 896 * 896 + 3 * 896 * 4864
    weights = 2 * (24 * per_layer + 151936 * 896)
    kv = 24 * 2 * 128 * 2 * (191.5 + 1)
    assert bench.decode_step_bytes(w, 191.5) == pytest.approx(weights + kv)


@pytest.mark.parametrize("name,tflop", [("0.5b", 0.0926), ("1.5b", 1.365), ("1.5b-prefill", 45.82),
                                        ("1.5b-longctx", 871.7)])
def test_prefill_flops(bench, name, tflop):
    w = S.WORKLOADS[name]
    L = w.model.n_layers
    per_layer = sum(bench.prefill_family_flops(w, f) for f in ("gemm_qkv", "gemm_o", "gemm_gate_up", "gemm_down",
                                                                "attention"))
    total = L * per_layer + bench.prefill_family_flops(w, "lm_head")
    assert total / 1e12 == pytest.approx(tflop, rel=3e-3)


def test_mlp_family_bytes_is_three_weight_matrices(bench):
    w = S.WORKLOADS["0.5b"]
    m = w.model
    assert bench.decode_family_bytes(w, "mlp", 0.0) == 3 * m.intermediate * m.hidden * 2 + 2 * m.hidden * 8


def test_traffic_record_is_gated(bench, tmp_path):
    rec = {"family": "mlp", "workload": "0.5b", "kernel_source": "bench.py",
           "fetch_bytes_per_launch": 100, "write_bytes_per_launch": 20}
    import hashlib
    sha = hashlib.sha256(open(os.path.join(ROOT, "bench.py"), "rb").read()).hexdigest()
    f = tmp_path / "a_hbm_traffic.json"
    f.write_text(json.dumps(dict(rec, kernel_source_sha256=sha)))
    pat = str(tmp_path / "*_hbm_traffic.json")
    assert bench.measured_traffic("0.5b", "mlp", pat) == 120
    assert bench.measured_traffic("1.5b", "mlp", pat) is None          # other workload
    assert bench.measured_traffic("0.5b", "attention", pat) is None    # other kernel family
    g = tmp_path / "b_hbm_traffic.json"
    g.write_text(json.dumps(dict(rec, family="attention", fetch_bytes_per_launch=7, kernel_source_sha256=sha)))
    assert bench.measured_traffic("0.5b", "attention", pat) == 27      # a second record
    f.write_text(json.dumps(dict(rec, kernel_source_sha256="0" * 64)))
    assert bench.measured_traffic("0.5b", "mlp", pat) is None          # source changed since the counters
    assert bench.measured_traffic("0.5b", "mlp", str(tmp_path / "none_*.json")) is None


def test_default_workload_is_the_largest_single_gpu_config(bench):
    w = S.WORKLOADS[bench.DEFAULT_WORKLOAD]
    assert (w.batch, w.prompt_len, w.decode_steps) == (32, 8192, 128)
    assert w.model.hidden == 1536 and w.model.n_layers == 28


def test_cpu_info(bench):
    model, n = bench.cpu_info()
    assert isinstance(model, str) and n >= 1
