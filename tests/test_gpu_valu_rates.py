"""The VALU issue rates behind bench.py's VALU-slot roof, measured on the device.

bench.py prices the scan against 256 CUs x 4 SIMDs x 32 lanes x 2.4 GHz
(half of MI355X's published 157.3 TFLOP/s fp32 vector rate: a wave64 fp32
FMA occupies a SIMD for two cycles) with a transcendental at four slots.  This
test times register-only streams (tests/valu_rate_probe.hip) and checks the
two ratios that model rests on, which do not depend on the clock:
- one wave alone issues a VALU instruction about every four cycles, so two
  or more waves per SIMD complete FMAs about twice as fast;
- v_exp_f32 runs at about a quarter of the FMA rate.
It also times the scan's per-state mix (four full-rate operations and one
exponential): at 2.4 GHz such a state costs 16 cycles of VALU time by the
slot count, and the printed figure shows what a SIMD actually sustains.
Three further facts explain where the scan's time goes beyond the slot count:
- an FMA with a wave-uniform SGPR operand (B_t and C_t in the scan) takes
  about twice as long as one with VGPR operands when it is all a SIMD issues;
- in the structured scan's state mix (no exponential per state) the scalar
  unit's unpacking of bf16 B and C costs the waves issue slots: at two waves
  per SIMD the mix takes clearly longer than with fp32 values;
- an exponential-only wave and an FMA-only wave sharing a SIMD barely
  overlap: the exponentials hold the vector unit.
"""
import ctypes
import os
import subprocess

import pytest

torch = pytest.importorskip("torch")

HERE = os.path.dirname(os.path.abspath(__file__))
pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def probe(tmp_path_factory):
    if not torch.cuda.is_available():
        pytest.skip("needs a GPU")
    so = str(tmp_path_factory.mktemp("valu") / "libvalu_rate_probe.so")
    subprocess.run(["/opt/rocm/bin/hipcc", "--offload-arch=gfx950", "-O3", "-shared", "-fPIC", "-Xclang",
                    "-target-feature", "-Xclang", "-packed-fp32-ops", os.path.join(HERE, "valu_rate_probe.hip"),
                    "-o", so], check=True, capture_output=True)
    lib = ctypes.CDLL(so)
    lib.valu_rate_probe.argtypes = [ctypes.c_int, ctypes.c_void_p, ctypes.c_int, ctypes.c_int, ctypes.c_void_p]
    lib.valu_rate_probe.restype = ctypes.c_int
    lib.valu_split_probe.argtypes = [ctypes.c_void_p, ctypes.c_int, ctypes.c_int, ctypes.c_void_p]
    lib.valu_split_probe.restype = ctypes.c_int
    return lib


def _ns_per_instruction(lib, kind, waves_per_simd, iters=2000, per_iter=64):
    """Kernel time per wave instruction (or per unit: per_iter units per loop
    iteration) per SIMD."""
    blocks = 1024 * waves_per_simd
    out = torch.empty(blocks * 64, device="cuda")
    assert out.numel() == blocks * 64
    st = torch.cuda.current_stream().cuda_stream
    best = None
    for _ in range(4):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        assert lib.valu_rate_probe(kind, out.data_ptr(), blocks, iters, st) == 0
        e1.record()
        torch.cuda.synchronize()
        ms = e0.elapsed_time(e1)
        best = ms if best is None else min(best, ms)
    return best * 1e6 / (iters * per_iter * waves_per_simd)


def test_fma_and_exp_issue_rates(probe):
    fma1 = _ns_per_instruction(probe, 0, 1)
    fma4 = _ns_per_instruction(probe, 0, 4)
    exp8 = _ns_per_instruction(probe, 1, 8)
    fma8 = _ns_per_instruction(probe, 0, 8)
    print("ns per wave64 instruction per SIMD: fma 1 wave %.3f, 4 waves %.3f, 8 waves %.3f; exp 8 waves %.3f "
          "(x 2.4 GHz: %.2f, %.2f, %.2f, %.2f cycles)" % (fma1, fma4, fma8, exp8, fma1 * 2.4, fma4 * 2.4, fma8 * 2.4,
                                                       exp8 * 2.4))
    # Several waves per SIMD complete FMAs at least ~1.6x as fast as one wave.
    assert fma4 < 0.65 * fma1
    # At 2.4 GHz (the peak clock) a wave64 FMA from a full SIMD takes at most
    # ~3 cycles: the SIMD is 32 lanes wide for fp32 FMA, not 16.
    assert fma8 * 2.4 < 3.2
    # Transcendentals: about four FMA times each.
    assert 2.8 < exp8 / fma8 < 5.5
    # The scan's state mix, per state update (16 per loop iteration).
    st2 = _ns_per_instruction(probe, 2, 2, per_iter=16)
    st8 = _ns_per_instruction(probe, 2, 8, per_iter=16)
    print("scan state mix, ns per state per SIMD: 2 waves %.3f, 8 waves %.3f (x 2.4 GHz: %.1f, %.1f cycles; "
          "slot count 4 x fma + 1 exp)" % (st2, st8, st2 * 2.4, st8 * 2.4))
    assert 4 * fma8 + exp8 * 0.9 < st8 < 4 * (4 * fma8 + exp8)


def test_sgpr_operands_and_scalar_unpacking(probe):
    fma8 = _ns_per_instruction(probe, 0, 8)
    sgpr8 = _ns_per_instruction(probe, 3, 8)
    unpack2 = _ns_per_instruction(probe, 4, 2, per_iter=16)
    f32_2 = _ns_per_instruction(probe, 5, 2, per_iter=16)
    print("ns per wave64 FMA per SIMD at 8 waves: VGPR operands %.3f, an SGPR operand %.3f (x 2.4 GHz: %.2f, %.2f "
          "cycles)" % (fma8, sgpr8, fma8 * 2.4, sgpr8 * 2.4))
    print("structured state mix at 2 waves per SIMD, ns per state: bf16 B/C unpacked on the scalar unit %.3f, fp32 "
          "%.3f (x 2.4 GHz: %.1f, %.1f cycles)" % (unpack2, f32_2, unpack2 * 2.4, f32_2 * 2.4))
    assert sgpr8 > 1.4 * fma8
    assert unpack2 > 1.2 * f32_2


def test_exp_and_fma_waves_share_the_vector_unit(probe):
    out = torch.empty(256 * 512, device="cuda")
    st = torch.cuda.current_stream().cuda_stream

    def us(ie, if_):
        best = None
        for _ in range(4):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            assert probe.valu_split_probe(out.data_ptr(), ie, if_, st) == 0
            e1.record()
            torch.cuda.synchronize()
            ms = e0.elapsed_time(e1)
            best = ms if best is None else min(best, ms)
        return best * 1e3

    exp_only, fma_only, both = us(1000, 0), us(0, 2000), us(1000, 2000)
    print("one exp wave + one FMA wave per SIMD: exp alone %.1f us, FMA alone %.1f us, together %.1f us "
          "(sum %.1f)" % (exp_only, fma_only, both, exp_only + fma_only))
    # Perfect overlap would take the longer of the two; they nearly add up.
    assert both > 1.4 * max(exp_only, fma_only)
