"""Seeded synthetic inputs for the selective scan and the decode update.

This module is shared by the device path, the tests and the benchmark; it
holds none of the scan's arithmetic.  It draws random tensors with the
distributions of a freshly initialised Mamba layer and rounds them to the
element type the library receives.

Recipe (the same for every consumer):
  * ``numpy.random.SeedSequence(seed).spawn(7)`` gives one child per tensor,
    in the order [dt_bias, x, z, delta-noise, B, C, h0].
  * dt_bias[d] ~ U[1e-3, 1e-1] (linear-uniform, one value per channel,
    fixed across batch, time and decode steps).  Step
    delta = softplus(0.5 * N(0,1) + inv_softplus(dt_bias[d])) with
    softplus(v) = log(1 + e^v), inv_softplus(u) = log(e^u - 1); the noise is
    per element.  (Selection step with a positive step size and its
    initialisation range: "Deriving and implementing Mamba from scratch"
    (dpshk.com/news/3333417) section 4.1; "SSMs for long-document QA"
    (pwwt.cn/news/5168881) section 3.3.)
  * x, z, B, C ~ N(0, 1) per element.
  * A[d, n] = -(n + 1) for every channel (S4D-real initialisation: A_log =
    log(1..N), A = -exp(A_log); "Mamba from principle to code"
    (lshu.cn/news/79586) section 6.2, derivation page section 5.1).
  * D[d] = 1 (derivation page section 5.1).
  * ``params="random"`` instead draws the per-channel parameters a trained
    layer would hold (A_log and D are learnable per channel, derivation page
    section 5.1): A[d, n] = -exp(N(0, 1)) clipped to [-20, -0.05], independent
    per (d, n), and D[d] ~ N(0, 1), from their own stream
    ``SeedSequence([seed, 0xA11]).spawn(2)`` = [A, D], so the other tensors
    are the same as with the default ``params="s4d"``.  The parity tests use
    it so that every per-channel index of A and D is checked; the layer
    configs keep the S4D-real initialisation.  ``params="linear"`` keeps the
    S4D-real structure with a per-channel scale, A[d, n] = (n + 1) A[d, 0]
    with A[d, 0] = -exp(U[-0.5, 0.5]) (rounded to fp32 before the multiple),
    and D ~ N(1, 0.5): inputs for the structured-A path.
  * h0 ~ N(0, 0.1^2) per state when a nonzero initial state is asked for.
  * Values are drawn and computed in float64, rounded to float32 (nearest
    even), and for bf16 tensors rounded again to bfloat16 (nearest even).
    bf16 tensors are returned as their raw 16-bit patterns (numpy.uint16).
  * Scan tensors are drawn per (batch row, segment of 4096 timesteps): the
    tensor's child is spawned into batch * ceil(seqlen / 4096) grandchildren
    in row-major (row, segment) order, each filling its (segment, d) block in
    C order.  Decode tensors are drawn per step: the child is spawned into
    ``steps`` grandchildren, each filling one (batch, width) slab.
"""
from __future__ import annotations

import os
from concurrent.futures import ThreadPoolExecutor
from dataclasses import dataclass
from typing import Dict, Optional

import numpy as np

SEGMENT = 4096
_ORDER = ("dt_bias", "x", "z", "delta_noise", "B", "C", "h0")


@dataclass(frozen=True)
class ScanConfig:
    name: str
    batch: int
    seqlen: int
    d_inner: int
    d_state: int
    dtype: str  # "f32" or "bf16"
    nonzero_h0: bool
    seed: int


@dataclass(frozen=True)
class DecodeConfig:
    name: str
    batch: int
    d_inner: int
    d_state: int
    dtype: str
    steps: int
    seed: int


# Layer shapes the library is measured on (seed = position in this list).
TINY = ScanConfig("tiny", 2, 64, 32, 16, "f32", False, 0)
MAMBA_130M = ScanConfig("mamba-130m-layer", 8, 2048, 1536, 16, "bf16", False, 1)
MAMBA_1P4B = ScanConfig("mamba-1.4b-layer", 32, 4096, 4096, 16, "bf16", False, 2)
MAMBA_2P8B_LONG = ScanConfig("mamba-2.8b-long-layer", 4, 32768, 5120, 16, "bf16", True, 3)
DECODE = DecodeConfig("decode-256x5120", 256, 5120, 16, "bf16", 1000, 4)

SCAN_CONFIGS = {c.name: c for c in (TINY, MAMBA_130M, MAMBA_1P4B, MAMBA_2P8B_LONG)}


@dataclass(frozen=True)
class SsdConfig:
    name: str
    batch: int
    seqlen: int
    nheads: int
    headdim: int
    ngroups: int
    d_state: int
    seed: int


# Scan with a scalar decay per head: a Mamba-2 layer of the 2.7B shape
# (d_model 2560, expand 2 -> 5120 channels = 80 heads of 64, d_state 128, one
# group of B/C).
SSD_2P7B = SsdConfig("mamba2-2.7b-layer", 8, 4096, 80, 64, 1, 128, 5)


def round_to_f32(a: np.ndarray) -> np.ndarray:
    return np.asarray(a, dtype=np.float64).astype(np.float32)


def f32_to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """Round float32 values to bfloat16 (nearest, ties to even); raw uint16 bits."""
    u = np.ascontiguousarray(a, dtype=np.float32).view(np.uint32)
    r = (u + np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))) >> np.uint32(16)
    return r.astype(np.uint16)


def bf16_bits_to_f32(bits: np.ndarray) -> np.ndarray:
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def _to_io(a64: np.ndarray, dtype: str) -> np.ndarray:
    f = round_to_f32(a64)
    return f32_to_bf16_bits(f) if dtype == "bf16" else f


def _softplus(v: np.ndarray) -> np.ndarray:
    return np.logaddexp(0.0, v)


def _inv_softplus(u: np.ndarray) -> np.ndarray:
    return np.log(np.expm1(u))


def channel_params(d_inner: int, d_state: int, seed: int, params: str = "s4d"):
    """(A, D) fp32 of make_scan_inputs(..., params=params) for these sizes and seed."""
    return _channel_params(d_inner, d_state, seed, params)


def _channel_params(d_inner: int, d_state: int, seed: int, params: str):
    """(A, D) fp32: the S4D-real initialisation, or random per-channel values."""
    if params == "s4d":
        A = np.ascontiguousarray(
            np.broadcast_to(-(np.arange(1, d_state + 1, dtype=np.float64)), (d_inner, d_state))).astype(np.float32)
        return A, np.ones(d_inner, dtype=np.float32)
    ka, kd = np.random.SeedSequence([seed, 0xA11]).spawn(2)
    if params == "random":
        scale = np.exp(np.random.default_rng(ka).uniform(-0.5, 0.5, (d_inner, d_state)))
        A = round_to_f32(-(np.arange(1, d_state + 1, dtype=np.float64))[None, :] * scale)
        D = round_to_f32(1.0 + 0.5 * np.random.default_rng(kd).standard_normal(d_inner))
        return A, D
    if params == "linear":
        a0 = np.exp(np.random.default_rng(ka).uniform(-0.5, 0.5, d_inner))
        A = round_to_f32(-(np.arange(1, d_state + 1, dtype=np.float64))[None, :] * round_to_f32(a0)[:, None])
        D = round_to_f32(1.0 + 0.5 * np.random.default_rng(kd).standard_normal(d_inner))
        return A, D
    if params == "wide":
        a = np.exp(np.random.default_rng(ka).standard_normal((d_inner, d_state)))
        A = round_to_f32(-np.clip(a, 0.05, 20.0))
        D = round_to_f32(np.random.default_rng(kd).standard_normal(d_inner))
        return A, D
    raise ValueError("params must be 's4d', 'random', 'linear' or 'wide', got %r" % (params,))


def _threads(threads: Optional[int]) -> int:
    if threads:
        return threads
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:
        n = os.cpu_count() or 1
    return max(1, min(16, n))


def make_scan_inputs(batch: int, seqlen: int, d_inner: int, d_state: int, dtype: str, seed: int,
                     nonzero_h0: bool = False, threads: Optional[int] = None,
                     raw_delta: bool = False, params: str = "s4d") -> Dict[str, np.ndarray]:
    """Host tensors for one scan call.

    Returns x, delta, z (batch, seqlen, d_inner), B, C (batch, seqlen, d_state)
    in the io type; A (d_inner, d_state), D (d_inner,), dt_bias (d_inner,) fp32;
    h0 (batch, d_inner, d_state) fp32 or None.  With ``raw_delta`` the
    returned ``delta`` is the pre-activation 0.5*noise (io type) and
    ``dt_bias`` is inv_softplus(U) (fp32), so that softplus(delta + dt_bias)
    is the step; otherwise ``delta`` is the step itself and ``dt_bias`` the
    uniform draw.
    """
    assert dtype in ("f32", "bf16")
    kids = dict(zip(_ORDER, np.random.SeedSequence(seed).spawn(len(_ORDER))))
    u = np.random.default_rng(kids["dt_bias"]).uniform(1e-3, 1e-1, size=d_inner)
    inv_sp = _inv_softplus(u)
    nseg = max(1, -(-seqlen // SEGMENT))
    io_t = np.uint16 if dtype == "bf16" else np.float32
    out = {k: np.empty((batch, seqlen, d_inner), dtype=io_t) for k in ("x", "z", "delta")}
    out["B"] = np.empty((batch, seqlen, d_state), dtype=io_t)
    out["C"] = np.empty((batch, seqlen, d_state), dtype=io_t)
    grand = {k: kids[k].spawn(batch * nseg) for k in ("x", "z", "delta_noise", "B", "C")}

    def fill(task: int):
        b, s = divmod(task, nseg)
        t0, t1 = s * SEGMENT, min(seqlen, (s + 1) * SEGMENT)
        n = t1 - t0
        if n <= 0:
            return
        for k in ("x", "z"):
            out[k][b, t0:t1] = _to_io(np.random.default_rng(grand[k][task]).standard_normal((n, d_inner)), dtype)
        noise = np.random.default_rng(grand["delta_noise"][task]).standard_normal((n, d_inner))
        if raw_delta:
            out["delta"][b, t0:t1] = _to_io(0.5 * noise, dtype)
        else:
            out["delta"][b, t0:t1] = _to_io(_softplus(0.5 * noise + inv_sp[None, :]), dtype)
        for k in ("B", "C"):
            out[k][b, t0:t1] = _to_io(np.random.default_rng(grand[k][task]).standard_normal((n, d_state)), dtype)

    tasks = batch * nseg
    if tasks > 1 and batch * seqlen * d_inner > (1 << 20):
        with ThreadPoolExecutor(_threads(threads)) as ex:
            list(ex.map(fill, range(tasks)))
    else:
        for t in range(tasks):
            fill(t)
    out["A"], out["D"] = _channel_params(d_inner, d_state, seed, params)
    out["dt_bias"] = round_to_f32(inv_sp) if raw_delta else round_to_f32(u)
    if nonzero_h0:
        out["h0"] = round_to_f32(0.1 * np.random.default_rng(kids["h0"]).standard_normal((batch, d_inner, d_state)))
    else:
        out["h0"] = None
    return out


def scan_inputs(cfg: ScanConfig, threads: Optional[int] = None) -> Dict[str, np.ndarray]:
    return make_scan_inputs(cfg.batch, cfg.seqlen, cfg.d_inner, cfg.d_state, cfg.dtype, cfg.seed, cfg.nonzero_h0,
                            threads)


def make_decode_inputs(batch: int, d_inner: int, d_state: int, dtype: str, steps: int, seed: int,
                       threads: Optional[int] = None, raw_delta: bool = False,
                       params: str = "s4d") -> Dict[str, np.ndarray]:
    """Host tensors for ``steps`` consecutive decode steps.

    x, delta, z: (steps, batch, d_inner); B, C: (steps, batch, d_state) in the
    io type; A (d_inner, d_state), D, dt_bias (d_inner,) fp32; the state
    starts at zero.
    """
    kids = dict(zip(_ORDER, np.random.SeedSequence(seed).spawn(len(_ORDER))))
    u = np.random.default_rng(kids["dt_bias"]).uniform(1e-3, 1e-1, size=d_inner)
    inv_sp = _inv_softplus(u)
    io_t = np.uint16 if dtype == "bf16" else np.float32
    out = {k: np.empty((steps, batch, d_inner), dtype=io_t) for k in ("x", "z", "delta")}
    out["B"] = np.empty((steps, batch, d_state), dtype=io_t)
    out["C"] = np.empty((steps, batch, d_state), dtype=io_t)
    grand = {k: kids[k].spawn(steps) for k in ("x", "z", "delta_noise", "B", "C")}

    def fill(s: int):
        for k in ("x", "z"):
            out[k][s] = _to_io(np.random.default_rng(grand[k][s]).standard_normal((batch, d_inner)), dtype)
        noise = np.random.default_rng(grand["delta_noise"][s]).standard_normal((batch, d_inner))
        if raw_delta:
            out["delta"][s] = _to_io(0.5 * noise, dtype)
        else:
            out["delta"][s] = _to_io(_softplus(0.5 * noise + inv_sp[None, :]), dtype)
        for k in ("B", "C"):
            out[k][s] = _to_io(np.random.default_rng(grand[k][s]).standard_normal((batch, d_state)), dtype)

    if steps > 1 and steps * batch * d_inner > (1 << 20):
        with ThreadPoolExecutor(_threads(threads)) as ex:
            list(ex.map(fill, range(steps)))
    else:
        for s in range(steps):
            fill(s)
    out["A"], out["D"] = _channel_params(d_inner, d_state, seed, params)
    out["dt_bias"] = round_to_f32(inv_sp) if raw_delta else round_to_f32(u)
    return out


def make_scan_grads(batch: int, seqlen: int, d_inner: int, d_state: int, dtype: str, seed: int,
                    threads: Optional[int] = None) -> Dict[str, np.ndarray]:
    """Upstream gradients for the scan's backward pass: dy (batch, seqlen,
    d_inner) ~ N(0, 1) in the io type and dh_last (batch, d_inner, d_state)
    ~ N(0, 1) fp32, from their own seed stream (drawn per batch row and
    4096-step segment, like the inputs)."""
    dy_kid, dh_kid = np.random.SeedSequence([seed, 0xB4C4]).spawn(2)
    nseg = max(1, -(-seqlen // SEGMENT))
    io_t = np.uint16 if dtype == "bf16" else np.float32
    dy = np.empty((batch, seqlen, d_inner), dtype=io_t)
    grand = dy_kid.spawn(batch * nseg)

    def fill(task: int):
        b, s = divmod(task, nseg)
        t0, t1 = s * SEGMENT, min(seqlen, (s + 1) * SEGMENT)
        if t1 > t0:
            dy[b, t0:t1] = _to_io(np.random.default_rng(grand[task]).standard_normal((t1 - t0, d_inner)), dtype)

    tasks = batch * nseg
    if tasks > 1 and batch * seqlen * d_inner > (1 << 20):
        with ThreadPoolExecutor(_threads(threads)) as ex:
            list(ex.map(fill, range(tasks)))
    else:
        for k in range(tasks):
            fill(k)
    dh = round_to_f32(np.random.default_rng(dh_kid).standard_normal((batch, d_inner, d_state)))
    return {"dy": dy, "dh_last": dh}


def make_ssd_inputs(batch: int, seqlen: int, nheads: int, headdim: int, ngroups: int, d_state: int, seed: int,
                    nonzero_h0: bool = False, raw_dt: bool = False,
                    threads: Optional[int] = None, params: str = "s4d") -> Dict[str, np.ndarray]:
    """Host tensors for the scan with a scalar decay per head (bf16 io).

    x, z: (batch, seqlen, nheads, headdim) ~ N(0,1); dt: (batch, seqlen,
    nheads) = softplus(0.5*N(0,1) + inv_softplus(U[1e-3, 1e-1]_h)) (with
    ``raw_dt`` the raw 0.5*N(0,1) and dt_bias = inv_softplus(U)); B, C:
    (batch, seqlen, ngroups, d_state) ~ N(0,1); A_h = -U[1, 16]; D = 1; h0 ~
    N(0, 0.1^2) if requested.  Per-row streams, like the other generators.
    ``params="random"`` draws D_h ~ N(0, 1) per head instead (its own stream,
    ``SeedSequence([seed, 0xA11, 1])``), so a head-indexing mistake in the
    skip term shows.
    """
    kids = np.random.SeedSequence([seed, 0x55D]).spawn(8)
    r = np.random.default_rng(kids[0])
    u = r.uniform(1e-3, 1e-1, size=nheads)
    inv_sp = _inv_softplus(u)
    A = -(1.0 + 15.0 * np.random.default_rng(kids[1]).uniform(size=nheads))
    out = {"x": np.empty((batch, seqlen, nheads, headdim), np.uint16),
           "z": np.empty((batch, seqlen, nheads, headdim), np.uint16),
           "dt": np.empty((batch, seqlen, nheads), np.uint16),
           "B": np.empty((batch, seqlen, ngroups, d_state), np.uint16),
           "C": np.empty((batch, seqlen, ngroups, d_state), np.uint16)}
    grand = {k: kids[2 + i].spawn(batch) for i, k in enumerate(("x", "z", "dt", "B", "C"))}

    def fill(b: int):
        for k in ("x", "z"):
            out[k][b] = _to_io(np.random.default_rng(grand[k][b]).standard_normal((seqlen, nheads, headdim)), "bf16")
        noise = 0.5 * np.random.default_rng(grand["dt"][b]).standard_normal((seqlen, nheads))
        out["dt"][b] = _to_io(noise if raw_dt else _softplus(noise + inv_sp[None, :]), "bf16")
        for k in ("B", "C"):
            out[k][b] = _to_io(np.random.default_rng(grand[k][b]).standard_normal((seqlen, ngroups, d_state)), "bf16")

    if batch > 1 and batch * seqlen * nheads * headdim > (1 << 20):
        with ThreadPoolExecutor(_threads(threads)) as ex:
            list(ex.map(fill, range(batch)))
    else:
        for b in range(batch):
            fill(b)
    out["A"] = round_to_f32(A)
    if params == "random":
        out["D"] = round_to_f32(np.random.default_rng(np.random.SeedSequence([seed, 0xA11, 1])).standard_normal(nheads))
    elif params == "s4d":
        out["D"] = np.ones(nheads, dtype=np.float32)
    else:
        raise ValueError("params must be 's4d' or 'random', got %r" % (params,))
    out["dt_bias"] = round_to_f32(inv_sp) if raw_dt else round_to_f32(u)
    out["h0"] = (round_to_f32(0.1 * np.random.default_rng(kids[7]).standard_normal((batch, nheads, headdim, d_state)))
                 if nonzero_h0 else None)
    return out


def decode_inputs(cfg: DecodeConfig, steps: Optional[int] = None, threads: Optional[int] = None):
    return make_decode_inputs(cfg.batch, cfg.d_inner, cfg.d_state, cfg.dtype, steps or cfg.steps, cfg.seed, threads)


def make_conv_inputs(batch: int, seqlen: int, d_inner: int, d_conv: int, dtype: str, seed: int,
                     with_state: bool = False, threads: Optional[int] = None) -> Dict[str, np.ndarray]:
    """Host tensors for the causal conv: x (batch, seqlen, d_inner) ~ N(0,1) in
    the io type; w (d_inner, d_conv) and bias (d_inner,) ~ U(-1/sqrt(d_conv),
    1/sqrt(d_conv)) fp32 (the default initialisation of a depthwise Conv1d,
    fan-in d_conv); state (batch, d_inner, d_conv-1) ~ N(0,1) fp32 or None.
    SeedSequence(seed).spawn(4) gives [w, bias, x, state]; x is drawn per
    (batch row, 4096-step segment) like the scan inputs."""
    kw, kb, kx, ks = np.random.SeedSequence(seed).spawn(4)
    bound = 1.0 / np.sqrt(d_conv)
    out = {"w": round_to_f32(np.random.default_rng(kw).uniform(-bound, bound, (d_inner, d_conv))),
           "bias": round_to_f32(np.random.default_rng(kb).uniform(-bound, bound, d_inner))}
    nseg = max(1, -(-seqlen // SEGMENT))
    io_t = np.uint16 if dtype == "bf16" else np.float32
    x = np.empty((batch, seqlen, d_inner), dtype=io_t)
    grand = kx.spawn(batch * nseg)

    def fill(task: int):
        b, s = divmod(task, nseg)
        t0, t1 = s * SEGMENT, min(seqlen, (s + 1) * SEGMENT)
        if t1 > t0:
            x[b, t0:t1] = _to_io(np.random.default_rng(grand[task]).standard_normal((t1 - t0, d_inner)), dtype)

    tasks = batch * nseg
    if tasks > 1 and batch * seqlen * d_inner > (1 << 20):
        with ThreadPoolExecutor(_threads(threads)) as ex:
            list(ex.map(fill, range(tasks)))
    else:
        for t in range(tasks):
            fill(t)
    out["x"] = x
    out["state"] = (round_to_f32(np.random.default_rng(ks).standard_normal((batch, d_inner, d_conv - 1)))
                    if with_state else None)
    return out


def _io_values(a: np.ndarray) -> np.ndarray:
    """float32 values of an io tensor (bf16 bit patterns or float32)."""
    return bf16_bits_to_f32(a) if a.dtype == np.uint16 else a.astype(np.float32)


def _like_io(v: np.ndarray, ref: np.ndarray) -> np.ndarray:
    v = np.ascontiguousarray(v, dtype=np.float32)
    return f32_to_bf16_bits(v) if ref.dtype == np.uint16 else v


def make_degenerate(inp: Dict[str, np.ndarray], seed: int, raw_delta: bool = False,
                    keep_linear_a: bool = False) -> Dict[str, np.ndarray]:
    """A copy of scan or decode inputs with the method's degenerate values
    planted at seeded positions (every value below is exact in bf16):

      * steps that stop time: delta = 0 on 5% of elements (with ``raw_delta``
        the raw input -100, whose softplus lies below fp32's normal range);
      * steps long enough that most decays underflow to zero: delta = 30 (raw
        40) on 3% of elements, with x = 1/32 there so that delta * x stays of
        order one;
      * x = 0 on 3% of the other elements;
      * gate inputs far into both tails: z = 60, -60 and -200 (e^200
        overflows fp32) on 3% of elements each;
      * whole rows of B, and of C, set to zero on 6% of (row, step) pairs;
      * A = 0 (no decay) on every 19th channel and, unless ``keep_linear_a``
        (inputs of the structured path, which must keep A[d, n] = (n + 1)
        A[d, 0]), on every 7th channel's third state;
      * D = 0 on every 5th channel and D negated on the channel after it.

    Works on (batch, seqlen, .) scan tensors and on (steps, batch, .) decode
    tensors alike: the positions are drawn per element of x and per row of B
    and C from ``SeedSequence([seed, 0xDE6]).spawn(4)`` = [step, x, z, rows]."""
    ks, kx, kz, kr = np.random.SeedSequence([seed, 0xDE6]).spawn(4)
    out = dict(inp)
    x, dl, z = (_io_values(inp[k]) for k in ("x", "delta", "z"))
    B, C = _io_values(inp["B"]), _io_values(inp["C"])
    u = np.random.default_rng(ks).random(x.shape)
    dl[u < 0.05] = -100.0 if raw_delta else 0.0
    big = (u >= 0.05) & (u < 0.08)
    dl[big] = 40.0 if raw_delta else 30.0
    x[big] = 1.0 / 32.0
    x[(np.random.default_rng(kx).random(x.shape) < 0.03) & ~big] = 0.0
    v = np.random.default_rng(kz).random(z.shape)
    z[v < 0.03] = 60.0
    z[(v >= 0.03) & (v < 0.06)] = -60.0
    z[(v >= 0.06) & (v < 0.09)] = -200.0
    rows = np.random.default_rng(kr).random((2,) + B.shape[:2])
    B[rows[0] < 0.06] = 0.0
    C[rows[1] < 0.06] = 0.0
    for k, val in (("x", x), ("delta", dl), ("z", z), ("B", B), ("C", C)):
        out[k] = _like_io(val, inp[k])
    A = inp["A"].copy()
    A[3::19, :] = 0.0
    if not keep_linear_a and A.shape[1] > 2:
        A[::7, 2] = 0.0
    D = inp["D"].copy()
    D[::5] = 0.0
    D[1::5] = -D[1::5]
    out["A"], out["D"] = A, D
    return out


def make_degenerate_ssd(inp: Dict[str, np.ndarray], seed: int, raw_dt: bool = False) -> Dict[str, np.ndarray]:
    """make_degenerate for the scalar-decay (SSD) inputs of make_ssd_inputs:
    per (row, step, head) 5% zero steps (raw -100 with ``raw_dt``) and 3%
    steps of 30 (raw 40) with that head's x row set to 1/32; x = 0 on 3% of
    the other elements; z = 60, -60, -200 on 3% of elements each; 6% of the
    (row, step, group) B rows and of the C rows zero; A = 0 (no decay) on the
    first head; D = 0 on every 3rd head and negated on the next.  Positions
    from ``SeedSequence([seed, 0xDE7]).spawn(4)`` = [step, x, z, rows]."""
    ks, kx, kz, kr = np.random.SeedSequence([seed, 0xDE7]).spawn(4)
    out = dict(inp)
    x, dt, z = (_io_values(inp[k]) for k in ("x", "dt", "z"))
    B, C = _io_values(inp["B"]), _io_values(inp["C"])
    u = np.random.default_rng(ks).random(dt.shape)
    dt[u < 0.05] = -100.0 if raw_dt else 0.0
    big = (u >= 0.05) & (u < 0.08)
    dt[big] = 40.0 if raw_dt else 30.0
    x[big] = 1.0 / 32.0
    x[(np.random.default_rng(kx).random(x.shape) < 0.03) & ~big[..., None]] = 0.0
    v = np.random.default_rng(kz).random(z.shape)
    z[v < 0.03] = 60.0
    z[(v >= 0.03) & (v < 0.06)] = -60.0
    z[(v >= 0.06) & (v < 0.09)] = -200.0
    rows = np.random.default_rng(kr).random((2,) + B.shape[:3])
    B[rows[0] < 0.06] = 0.0
    C[rows[1] < 0.06] = 0.0
    for k, val in (("x", x), ("dt", dt), ("z", z), ("B", B), ("C", C)):
        out[k] = _like_io(val, inp[k])
    A = inp["A"].copy()
    A[0] = 0.0
    D = inp["D"].copy()
    D[::3] = 0.0
    D[1::3] = -D[1::3]
    out["A"], out["D"] = A, D
    return out
