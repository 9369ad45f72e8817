"""bench.py's host-side contract (no GPU): more than one GPU is refused with
a message and exit status 2 before anything touches a device, and the
algorithmic FLOP counts it reports follow from the model's shapes."""

import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402
from multimodal_encoder_prefill_amd import synth  # noqa: E402


def test_multi_gpu_request_is_refused():
    proc = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                          capture_output=True, text=True, timeout=120)
    assert proc.returncode == 2
    assert "one GPU" in proc.stderr
    assert proc.stdout == ""


def test_layer_flops_of_the_full_width_layer():
    fl = bench.layer_flops(synth.FULL, 4096)
    S = 4096
    # q/k/v: 5120 -> (64 + 2*8) * 128; o: 8192 -> 5120; gate/up: 5120 -> 2 * 25600; down
    assert fl["qkv"] == 2 * S * 5120 * 10240
    assert fl["o_proj"] == 2 * S * 8192 * 5120
    assert fl["gate_up"] == 2 * S * 5120 * 51200
    assert fl["down"] == 2 * S * 25600 * 5120
    assert fl["attention"] == 4 * 128 * 64 * S * (S + 1) // 2
    # 213.46 TFLOP per 50-layer encode at seq 4096
    assert abs(fl["total"] * 50 / 1e12 - 213.46) < 0.01


def test_traffic_record_is_tied_to_the_gemm_source():
    t = bench.stored_traffic(4096)
    if t is not None:   # only while the committed counters match the source
        assert t > 0 and bench.stored_traffic(4096, "fp8") > 0
    assert bench.stored_traffic(512) is None
