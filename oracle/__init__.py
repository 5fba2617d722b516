"""fp64 CPU oracle for the selective scan and the recurrent state update.

TEST INFRASTRUCTURE ONLY: the test suite, the smoke check and the benchmark's
CPU-baseline leg may import this package; the product path never does.  It
shares no code with the HIP library (no common kernels, headers, helpers or
pre/post-processing) and imports nothing from it.

The arithmetic lives in ``ssm_oracle.c`` (plain sequential fp64 loops; see its
header for the passages of the pages each step follows).  This module only
builds that file with the system C compiler, loads it with ctypes, and turns
inputs into fp64 arrays.  Inputs given as bf16 are passed as their raw 16-bit
patterns (``numpy.uint16``); they are widened here, exactly, to fp64, so the
oracle sees precisely the values the device sees.

Pins: every function here is checked against closed forms, a textbook IIR
filter, a library ZOH discretisation and brute-force unrolled sums by the
CPU tests (``tests/test_oracle_pins.py``, ``tests/test_oracle_conv_pins.py``);
the gradient ``scan_bwd`` against central finite differences of ``scan``,
Euler identities of the parts of the scan that are linear, and hand-derived
one-step derivatives (``tests/test_oracle_bwd_pins.py``); ``ssd`` against the
Mamba-1 scan with the decay broadcast over states, the section 6.1 masked
matrix, and a block (chunked) decomposition (``tests/test_oracle_ssd_pins.py``).
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from typing import Optional

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "ssm_oracle.c")
_LIB = os.path.join(_HERE, "libssm_oracle.so")

_lib = None


def build(force: bool = True) -> str:
    """Compile ssm_oracle.c into libssm_oracle.so (gcc, -O2, no fast-math)."""
    if not force and os.path.exists(_LIB) and os.path.getmtime(_LIB) >= os.path.getmtime(_SRC):
        return _LIB
    tmp = _LIB + ".tmp%d" % os.getpid()
    cmd = ["gcc", "-O2", "-fno-fast-math", "-ffp-contract=off", "-std=c99", "-shared", "-fPIC",
           "-o", tmp, _SRC, "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(tmp, _LIB)
    return _LIB


def _load():
    global _lib
    if _lib is not None:
        return _lib
    # SSM_ORACLE_LIB names a separately built copy of the oracle (the mutation
    # tests load deliberately broken copies through it); it is never rebuilt.
    path = os.environ.get("SSM_ORACLE_LIB")
    if path is None:
        path = _LIB
        if not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
            build()
    lib = ctypes.CDLL(path)
    P = ctypes.c_void_p
    I64 = ctypes.c_int64
    lib.ssm_oracle_scan_f64.argtypes = [P] * 11 + [I64] * 4 + [ctypes.c_int, ctypes.c_int]
    lib.ssm_oracle_scan_f64.restype = ctypes.c_int
    lib.ssm_oracle_update_f64.argtypes = [P] * 10 + [I64] * 3 + [ctypes.c_int, ctypes.c_int]
    lib.ssm_oracle_update_f64.restype = ctypes.c_int
    lib.ssm_oracle_conv1d_f64.argtypes = [P] * 6 + [I64] * 4 + [ctypes.c_int]
    lib.ssm_oracle_conv1d_f64.restype = ctypes.c_int
    lib.ssm_oracle_scan_bwd_f64.argtypes = [P] * 20 + [I64] * 4 + [ctypes.c_int, ctypes.c_int]
    lib.ssm_oracle_scan_bwd_f64.restype = ctypes.c_int
    lib.ssm_oracle_ssd_f64.argtypes = [P] * 11 + [I64] * 6 + [ctypes.c_int]
    lib.ssm_oracle_ssd_f64.restype = ctypes.c_int
    _lib = lib
    return lib


def to_f64(a) -> Optional[np.ndarray]:
    """Widen an input to a C-contiguous fp64 array.

    ``numpy.uint16`` arrays are bf16 bit patterns: the 16 bits are the top half
    of an IEEE binary32, so the widening is exact.
    """
    if a is None:
        return None
    a = np.asarray(a)
    if a.dtype == np.uint16:
        a = (a.astype(np.uint32) << np.uint32(16)).view(np.float32)
    return np.ascontiguousarray(a, dtype=np.float64)


def _ptr(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def scan(x, delta, A, B, C, D=None, z=None, h0=None, dt_bias=None, *, exact_zoh=False, delta_softplus=False):
    """Selective scan over the whole sequence.

    Shapes: x, delta, z: (batch, seqlen, d_inner); A: (d_inner, d_state);
    B, C: (batch, seqlen, d_state); D, dt_bias: (d_inner,); h0: (batch, d_inner, d_state).
    Returns (y, h_last) in fp64.
    """
    lib = _load()
    x, delta, A, B, C = (to_f64(v) for v in (x, delta, A, B, C))
    D, z, h0, dt_bias = (to_f64(v) for v in (D, z, h0, dt_bias))
    batch, seqlen, d_inner = x.shape
    d_state = A.shape[1]
    assert delta.shape == x.shape and A.shape == (d_inner, d_state)
    assert B.shape == (batch, seqlen, d_state) and C.shape == B.shape
    assert D is None or D.shape == (d_inner,)
    assert z is None or z.shape == x.shape
    assert h0 is None or h0.shape == (batch, d_inner, d_state)
    assert dt_bias is None or dt_bias.shape == (d_inner,)
    y = np.empty_like(x)
    h_last = np.empty((batch, d_inner, d_state), dtype=np.float64)
    rc = lib.ssm_oracle_scan_f64(_ptr(x), _ptr(delta), _ptr(A), _ptr(B), _ptr(C), _ptr(D), _ptr(z), _ptr(h0),
                                 _ptr(dt_bias), _ptr(y), _ptr(h_last), batch, seqlen, d_inner, d_state,
                                 1 if exact_zoh else 0, 1 if delta_softplus else 0)
    if rc != 0:
        raise ValueError("oracle scan rejected its arguments (%d)" % rc)
    return y, h_last


def update(h, x_t, delta_t, A, B_t, C_t, D=None, z_t=None, dt_bias=None, *, exact_zoh=False,
           delta_softplus=False):
    """One recurrent step.  h: (batch, d_inner, d_state) is NOT modified;
    returns (y_t, h_new).  x_t, delta_t, z_t: (batch, d_inner); B_t, C_t: (batch, d_state)."""
    lib = _load()
    hn = to_f64(h).copy()
    x_t, delta_t, A, B_t, C_t = (to_f64(v) for v in (x_t, delta_t, A, B_t, C_t))
    D, z_t, dt_bias = (to_f64(v) for v in (D, z_t, dt_bias))
    batch, d_inner, d_state = hn.shape
    assert x_t.shape == (batch, d_inner) and delta_t.shape == x_t.shape
    assert B_t.shape == (batch, d_state) and C_t.shape == B_t.shape
    y_t = np.empty((batch, d_inner), dtype=np.float64)
    rc = lib.ssm_oracle_update_f64(_ptr(hn), _ptr(x_t), _ptr(delta_t), _ptr(A), _ptr(B_t), _ptr(C_t), _ptr(D),
                                   _ptr(z_t), _ptr(dt_bias), _ptr(y_t), batch, d_inner, d_state,
                                   1 if exact_zoh else 0, 1 if delta_softplus else 0)
    if rc != 0:
        raise ValueError("oracle update rejected its arguments (%d)" % rc)
    return y_t, hn


def scan_bwd(x, delta, A, B, C, D=None, z=None, h0=None, dt_bias=None, *, dy, dh_last=None, exact_zoh=False,
             delta_softplus=False):
    """Gradient of L = sum(dy * y) + sum(dh_last * h_last) for the scan above.

    Returns a dict of fp64 arrays: dx, ddelta (w.r.t. the delta input as
    given, i.e. the raw value when delta_softplus), dA, dB, dC, dh0, and dD,
    dz, d_dt_bias when D, z, delta_softplus are used.
    """
    lib = _load()
    x, delta, A, B, C = (to_f64(v) for v in (x, delta, A, B, C))
    D, z, h0, dt_bias = (to_f64(v) for v in (D, z, h0, dt_bias))
    dy, dh_last = to_f64(dy), to_f64(dh_last)
    batch, seqlen, d_inner = x.shape
    d_state = A.shape[1]
    assert delta.shape == x.shape and dy.shape == x.shape and A.shape == (d_inner, d_state)
    assert B.shape == (batch, seqlen, d_state) and C.shape == B.shape
    assert dh_last is None or dh_last.shape == (batch, d_inner, d_state)
    assert h0 is None or h0.shape == (batch, d_inner, d_state)
    g = {"dx": np.empty_like(x), "ddelta": np.empty_like(x), "dA": np.empty_like(A), "dB": np.empty_like(B),
         "dC": np.empty_like(C), "dh0": np.empty((batch, d_inner, d_state))}
    if D is not None:
        g["dD"] = np.empty(d_inner)
    if z is not None:
        g["dz"] = np.empty_like(x)
    if delta_softplus:
        g["d_dt_bias"] = np.empty(d_inner)
    rc = lib.ssm_oracle_scan_bwd_f64(
        _ptr(x), _ptr(delta), _ptr(A), _ptr(B), _ptr(C), _ptr(D), _ptr(z), _ptr(h0), _ptr(dt_bias), _ptr(dy),
        _ptr(dh_last), _ptr(g["dx"]), _ptr(g["ddelta"]), _ptr(g["dA"]), _ptr(g["dB"]), _ptr(g["dC"]),
        _ptr(g.get("dD")), _ptr(g.get("dz")), _ptr(g["dh0"]), _ptr(g.get("d_dt_bias")), batch, seqlen, d_inner,
        d_state, 1 if exact_zoh else 0, 1 if delta_softplus else 0)
    if rc != 0:
        raise ValueError("oracle scan_bwd rejected its arguments (%d)" % rc)
    return g


def ssd(x, dt, A, B, C, D=None, z=None, h0=None, dt_bias=None, *, delta_softplus=False):
    """Scan with a scalar decay per head (Mamba-2 / SSD form).

    Shapes: x, z: (batch, seqlen, nheads, headdim); dt: (batch, seqlen, nheads);
    A, D, dt_bias: (nheads,); B, C: (batch, seqlen, ngroups, d_state);
    h0: (batch, nheads, headdim, d_state).  Returns (y, h_last) in fp64.
    """
    lib = _load()
    x, dt, A, B, C = (to_f64(v) for v in (x, dt, A, B, C))
    D, z, h0, dt_bias = (to_f64(v) for v in (D, z, h0, dt_bias))
    batch, seqlen, nheads, headdim = x.shape
    ngroups, d_state = B.shape[2], B.shape[3]
    assert dt.shape == (batch, seqlen, nheads) and A.shape == (nheads,)
    assert B.shape == (batch, seqlen, ngroups, d_state) and C.shape == B.shape
    assert z is None or z.shape == x.shape
    assert h0 is None or h0.shape == (batch, nheads, headdim, d_state)
    y = np.empty_like(x)
    h_last = np.empty((batch, nheads, headdim, d_state))
    rc = lib.ssm_oracle_ssd_f64(_ptr(x), _ptr(dt), _ptr(A), _ptr(B), _ptr(C), _ptr(D), _ptr(z), _ptr(h0),
                                _ptr(dt_bias), _ptr(y), _ptr(h_last), batch, seqlen, nheads, headdim, ngroups,
                                d_state, 1 if delta_softplus else 0)
    if rc != 0:
        raise ValueError("oracle ssd rejected its arguments (%d)" % rc)
    return y, h_last


def scan_channels(inputs, channels, *, exact_zoh=False, delta_softplus=False):
    """Oracle for a sample of whole channels of one scan.

    ``inputs`` maps names (x, delta, A, B, C, D, z, h0, dt_bias) to host arrays
    in the scan layout; ``channels`` is a list of (b, d).  Each channel is run
    on its own (batch 1, d_inner 1), which is exact for that channel because
    channels never interact.  Returns (y[k, t], h_last[k, n]) for the k-th channel.
    """
    x, delta, A, B, C = (inputs[k] for k in ("x", "delta", "A", "B", "C"))
    D, z, h0, dt_bias = (inputs.get(k) for k in ("D", "z", "h0", "dt_bias"))
    seqlen = x.shape[1]
    d_state = A.shape[1]
    ys = np.empty((len(channels), seqlen))
    hs = np.empty((len(channels), d_state))
    for k, (b, d) in enumerate(channels):
        y, h = scan(x[b:b + 1, :, d:d + 1], delta[b:b + 1, :, d:d + 1], A[d:d + 1], B[b:b + 1], C[b:b + 1],
                    None if D is None else D[d:d + 1], None if z is None else z[b:b + 1, :, d:d + 1],
                    None if h0 is None else h0[b:b + 1, d:d + 1], None if dt_bias is None else dt_bias[d:d + 1],
                    exact_zoh=exact_zoh, delta_softplus=delta_softplus)
        ys[k] = y[0, :, 0]
        hs[k] = h[0, 0]
    return ys, hs


def conv1d(x, w, bias=None, state_in=None, *, silu=True):
    """Causal depthwise conv over time (+ SiLU).  x: (batch, seqlen, d_inner);
    w: (d_inner, d_conv); bias: (d_inner,); state_in: (batch, d_inner, d_conv-1).
    Returns (y, state_out) in fp64."""
    lib = _load()
    x, w, bias, state_in = (to_f64(v) for v in (x, w, bias, state_in))
    batch, seqlen, d_inner = x.shape
    d_conv = w.shape[1]
    assert w.shape == (d_inner, d_conv)
    assert bias is None or bias.shape == (d_inner,)
    assert state_in is None or state_in.shape == (batch, d_inner, d_conv - 1)
    y = np.empty_like(x)
    state_out = np.empty((batch, d_inner, d_conv - 1), dtype=np.float64)
    rc = lib.ssm_oracle_conv1d_f64(_ptr(x), _ptr(w), _ptr(bias), _ptr(state_in), _ptr(y), _ptr(state_out),
                                   batch, seqlen, d_inner, d_conv, 1 if silu else 0)
    if rc != 0:
        raise ValueError("oracle conv1d rejected its arguments (%d)" % rc)
    return y, state_out


def conv1d_update(state, x_t, w, bias=None, *, silu=True):
    """One decode step of the conv: state (batch, d_inner, d_conv-1) is NOT
    modified; returns (y_t, new_state).  x_t: (batch, d_inner)."""
    y, st = conv1d(np.asarray(to_f64(x_t))[:, None, :], w, bias, state, silu=silu)
    return y[:, 0, :], st
