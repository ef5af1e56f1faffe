"""Host-side checks of the benchmark: the algorithmic work it divides by, the profile
lookup that guards the counter figures, and the one-GPU contract.  No GPU needed."""
import json
import os
import subprocess
import sys

import bench
import polar_inputs as pin

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_prefill_flops_are_four_d_per_causal_pair():
    # 4 d flops per computed (query, key) pair, B H T (T + 1) / 2 causal pairs
    for name, d, H, T in (("bf16_b1_h16_t65536_d64_lentemp", 64, 16, 65536),
                          ("bf16_b1_h16_t16384_d128_groups", 128, 16, 16384)):
        assert bench.prefill_flops(pin.WORKLOADS[name]) == 4 * d * H * T * (T + 1) // 2
    assert bench.prefill_flops(pin.WORKLOADS["bf16_b1_h16_t65536_d64_lentemp"]) == 8_796_227_239_936
    assert bench.prefill_flops(pin.WORKLOADS["bf16_b1_h16_t16384_d128_groups"]) == 1_099_578_736_640
    assert bench.prefill_flops(pin.WORKLOADS[bench.NEEDLE]) == 68_736_253_952


def test_backward_flops_are_ten_d_per_causal_pair():
    w = pin.WORKLOADS["bf16_bwd_b1_h16_kv4_t16384_d128"]
    assert bench.backward_flops(w) == 10 * 128 * 16 * 16384 * 16385 // 2


def test_decode_bytes_are_k_and_v_once_plus_q_and_outputs():
    w = pin.WORKLOADS["bf16_decode_b64_h8_tk65536_d128"]
    kv = 2 * 64 * 8 * 65536 * 128 * 2
    assert bench.decode_bytes(w) == kv + 64 * 8 * 128 * 2 + 64 * 8 * 131 * 4 == 17_180_268_544
    # grouped heads: the same K and V bytes serve four times the query heads
    wp = pin.WORKLOADS["bf16_paged_decode_b64_h32_kv8_tk65536_d128"]
    assert bench.decode_bytes(wp) - bench.decode_bytes(w) == 64 * 24 * (128 * 2 + 131 * 4)


def test_window_pairs_brute_force():
    for T in (1, 5, 64, 200):
        for W in (1, 3, 64, 150, 500):
            want = sum(min(i + 1, W) for i in range(T))
            assert bench.window_pairs(T, W) == want, (T, W)


def test_profile_figures_only_while_the_sources_match(tmp_path, monkeypatch):
    key = "fwd_bf16_t65536_d64"
    good = {key: {"source_digest": bench.source_digest(key), "hbm_bytes_per_launch": 123.0, "mfma_busy": 0.5}}
    path = tmp_path / "traffic.json"
    path.write_text(json.dumps(good))
    monkeypatch.setattr(bench, "TRAFFIC_FILE", str(path))
    assert bench.measured_traffic(key) == 123.0 and bench.profiled(key, "mfma_busy") == 0.5
    good[key]["source_digest"] = "0" * 16
    path.write_text(json.dumps(good))
    assert bench.measured_traffic(key) is None and bench.profiled(key, "mfma_busy") is None
    assert bench.profiled("decode_b64_h8_tk65536_d128", "hbm_bytes_per_launch") is None


def test_committed_profiles_match_the_sources():
    """Every committed counter figure belongs to the current kernel sources."""
    for key in bench.KERNEL_SOURCES:
        assert bench.measured_traffic(key) is not None, key


def test_more_than_one_gpu_is_refused():
    res = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                         text=True, timeout=60)
    assert res.returncode == 2 and "one GPU" in res.stderr
