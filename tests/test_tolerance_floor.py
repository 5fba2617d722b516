"""Where the fp32 gates come from.

A float32 emulation (numpy) of the kernel's operation order, with correctly
rounded exp2 / log2, is compared with the fp64 oracle under the floored
metric.  It shows that

  * the plain scan stays inside the 1e-5 fp32 parity gate (with little
    room at d_state 64: ~9e-6 on this case),
  * the softplus-step variant reaches ~1.2e-5 on some shapes even with
    correctly rounded transcendentals, so its fp32 gate must be looser:
    VARIANT_F32_GATE = 3e-5 leaves 2.5x room for the hardware's 1-ulp
    exp2 / log2 / rcp.

The emulation is test-side arithmetic only (neither the oracle nor the device
path); it restates the same fp32 steps as the kernel for one purpose: to size
the tolerance.
"""
import numpy as np
import pytest

import oracle
from conftest import floored_rel_err
from selective_state_space_84_amd import inputs

VARIANT_F32_GATE = 3e-5
PLAIN_F32_GATE = 1e-5

f = np.float32
L2E = f(1.4426950408889634)
L2E_LO = f(1.925963e-8)
LN2 = f(0.6931471805599453)


def _exp2(v):
    return np.exp2(v.astype(np.float64)).astype(np.float32)


def _softplus_f32(v):
    yh = (v * L2E).astype(np.float32)
    yl = ((v.astype(np.float64) * float(L2E) - yh).astype(np.float32) + v * L2E_LO).astype(np.float32)
    e = _exp2(yh)
    e = (e + e * (yl * LN2)).astype(np.float32)
    u = (f(1) + e).astype(np.float32)
    um1 = (u - f(1)).astype(np.float32)
    lg = np.log2(u.astype(np.float64)).astype(np.float32)
    r = np.where(um1 == 0, e, (lg * LN2) * (e * (f(1) / np.where(um1 == 0, f(1), um1))))
    return np.where(v > 20, v, r).astype(np.float32)


def _emulate(inp, softplus):
    x, dl, A, Bm, Cm, Dv, z, h0, dtb = (inp[k] for k in ("x", "delta", "A", "B", "C", "D", "z", "h0", "dt_bias"))
    Al2 = (A * L2E).astype(np.float32)
    h = h0.copy() if h0 is not None else np.zeros((x.shape[0], x.shape[2], A.shape[1]), np.float32)
    y = np.zeros_like(x)
    for t in range(x.shape[1]):
        xv = x[:, t]
        dv = _softplus_f32((dl[:, t] + dtb[None, :]).astype(np.float32)) if softplus else dl[:, t]
        acc = (Dv * xv).astype(np.float32)
        wx = (dv * xv).astype(np.float32)
        for n in range(A.shape[1]):
            ab = _exp2((dv * Al2[None, :, n]).astype(np.float32))
            h[:, :, n] = (ab * h[:, :, n] + (wx * Bm[:, t, None, n]).astype(np.float32)).astype(np.float32)
            acc = (Cm[:, t, None, n] * h[:, :, n] + acc).astype(np.float32)
        zz = z[:, t]
        y[:, t] = acc * (zz * (f(1) / (f(1) + np.exp(-zz.astype(np.float64)).astype(np.float32))))
    return y, h


def _floor(N, seed, softplus):
    inp = inputs.make_scan_inputs(2, 40, 70, N, "f32", seed, nonzero_h0=True, raw_delta=softplus)
    y, h = _emulate(inp, softplus)
    ry, rh = oracle.scan(inp["x"], inp["delta"], inp["A"], inp["B"], inp["C"], inp["D"], inp["z"], inp["h0"],
                         inp["dt_bias"] if softplus else None, delta_softplus=softplus)
    return max(floored_rel_err(y, ry), floored_rel_err(h, rh))


@pytest.mark.parametrize("N,seed", [(16, 1014), (64, 1014)])
def test_plain_scan_fp32_floor_is_inside_the_gate(N, seed):
    assert _floor(N, seed, softplus=False) < PLAIN_F32_GATE


def test_softplus_variant_fp32_floor_sets_its_gate():
    worst = max(_floor(N, 1014, softplus=True) for N in (16, 64))
    # A correctly rounded fp32 implementation already exceeds the plain gate ...
    assert worst > PLAIN_F32_GATE
    # ... and the variant gate leaves 2x room for 1-ulp hardware transcendentals.
    assert VARIANT_F32_GATE >= 2 * worst
