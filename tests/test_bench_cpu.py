"""Host-side parts of bench.py that run without a GPU: the one-GPU contract,
the algorithmic byte count behind the HBM figure, and the rule that a
counter-derived traffic figure is reported only for the sources it was
measured on."""
import os
import subprocess
import sys

import pytest

import bench

REPO = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_exits_with_a_message():
    r = subprocess.run([sys.executable, os.path.join(REPO, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr and r.stdout == ""


def test_algorithmic_scan_bytes():
    # bf16 io, no h0, with h_last: x, delta, z read and y written (2 B each),
    # B and C rows (2 B per state), A and D, and the final state.
    b, L, d, n = 32, 4096, 4096, 16
    want = 4 * b * L * d * 2 + 2 * b * L * n * 2 + d * n * 4 + d * 4 + b * d * n * 4
    assert bench.algorithmic_scan_bytes(b, L, d, n, 2, False, True) == want == 4312023040
    # An initial state adds one more state read.
    assert bench.algorithmic_scan_bytes(b, L, d, n, 2, True, True) == want + b * d * n * 4


def test_traffic_follows_the_kernel_sources():
    sha = bench._kernel_source_sha("scan")
    assert len(sha) == 16 and sha != bench._kernel_source_sha("decode")
    assert bench._traffic("mamba-1.4b-layer", "0" * 16) is None
    assert bench._traffic("no-such-workload", sha) is None
    got = bench._traffic("mamba-1.4b-layer", sha)
    if got is None:
        pytest.skip("the scan kernel changed since its traffic counters were taken")
    # Measured traffic sits within a few percent of the algorithmic bytes.
    assert abs(got / 4312023040 - 1) < 0.05


def test_valu_slot_model():
    # The peak: 256 CUs x 4 SIMDs x 32 lanes x 2.4 GHz, half the 157.3 TFLOP/s
    # fp32 vector rate (an FMA is two flops).
    assert abs(bench.VALU_PEAK_TSLOTS - 157.3 / 2) < 0.1
    # General A: 8 slots per state (mul, exp = 4, mul, two FMAs) + 18 per
    # element (10 full-rate ops and the gate's exp and rcp).
    assert bench.scan_slots_per_element(16) == 8 * 16 + 18 == 146
    # Structured A: exp2 at y, 2y, 4y, 8y, 16y (4 slots each), four scalings,
    # y itself, 11 products, then 3 slots per state + 18 per element.
    assert bench.scan_slots_per_element(16, linear_a=True) == 20 + 4 + 1 + 11 + 48 + 18 == 102
    # With bf16 io: exp2 at y only, y itself and 15 products.
    assert bench.scan_slots_per_element(16, linear_a=True, io_bf16=True) == 4 + 1 + 15 + 48 + 18 == 86
    # Backward: 18 per state and step + 38 per element.
    assert bench.bwd_slots_per_element(16) == 18 * 16 + 38 == 326
