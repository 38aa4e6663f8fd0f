"""Host-side checks of bench.py (no GPU): the HIP event wrapper declares full
signatures (an undeclared 64-bit handle would be truncated to a C int), the
multi-GPU request is refused with a message, the byte/flop model, and that
measured traffic is reported only for the workload it was measured on."""
import subprocess
import sys

import bench
import workloads as W


def test_hip_event_functions_have_full_signatures():
    h = bench.Hip()
    for fn in ("hipEventCreate", "hipEventElapsedTime"):
        assert getattr(h.lib, fn).argtypes is not None, fn


def test_multi_gpu_request_exits_with_message():
    r = subprocess.run([sys.executable, bench.__file__, "--gpus", "2"], capture_output=True, text=True)
    assert r.returncode == 2
    assert "one GPU" in r.stderr


def test_algorithmic_work_model():
    cfg = W.CONFIGS["moe1k"]
    flop, byts = bench.layer_work(cfg, 512)
    # 6*R*I*H + 6*T*Is*H flop; weights 512 experts * 6 MiB dominate the bytes
    assert flop == 6 * 10240 * 512 * 2048 + 6 * 1024 * 512 * 2048
    assert 3.2e9 < byts < 3.5e9
    up = bench.ffn_up_bytes(cfg, 512)
    assert up > 512 * 4 * 2**20


def test_measured_traffic_is_reported_only_for_its_workload():
    # the committed counter summary covers the 1024-token up projection only
    for name in ("tiny", "moe8k", "skew16k", "bwd4k"):
        assert bench.traffic_from_profile(name) is None
    t = bench.traffic_from_profile("moe1k")
    assert t is None or 2.0e9 < t < 3.0e9
