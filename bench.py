#!/usr/bin/env python3
"""Benchmark of the gfx950 selective-scan library on one MI355X.

One step = one ssm_scan_fwd call over a whole Mamba layer's batch (all of the
scan's steps: load and unpack, decay, input term, recurrence, readout, gate,
store, final state), with inputs already resident in HBM.  The headline
workload is the Mamba-1.4B layer shape (batch 32, L 4096, d_inner 4096,
d_state 16, bf16 io, fp32 state) on the general path (the plain entry point:
one exponential per state), measured against the HBM roofline.  The same JSON
line also carries, each as its own object:
  * structured_a: the same layer with SSM_FLAG_A_LINEAR_N (its A = -(n+1)
    has that structure);
  * scan_c4 / scan_c2: the Mamba-2.8B long-context layer (batch 4, L 32768,
    d_inner 5120, h0 != 0) and the Mamba-130M layer, general and structured,
    with whole-row parity against the oracle;
  * parity_channel_params: the 1.4B layer's inputs with random per-channel A
    and D, whole rows against the oracle;
  * the scan's backward pass, the causal conv1d, the decode update (256 x
    5120 x 16 state, 1000 in-place steps), the Mamba-2 SSD form, and the fp64
    CPU oracle on a bounded sample of the headline workload (cpu_baseline).
The oracle (test infrastructure under oracle/) is used only by the
cpu_baseline leg: its timed sample, and the whole-row comparisons of GPU
outputs with it (the parity objects above).  --no-cpu-baseline skips that
leg entirely, and then nothing under oracle/ is loaded.
Prints one JSON line.

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]
                       [--no-decode] [--no-conv] [--no-bwd] [--no-ssd] [--no-cpu-baseline]
                       [--no-extra-scans]
"""
import argparse
import hashlib
import json
import os
import sys
import time

REPO = os.path.dirname(os.path.abspath(__file__))
if REPO not in sys.path:
    sys.path.insert(0, REPO)

HBM_PEAK_GBPS = 8000.0
# VALU lane-slots on MI355X: the published 157.3 TFLOP/s fp32 vector rate
# counts an FMA as two flops, i.e. 256 CUs x 4 SIMDs x 32 lanes x 2.4 GHz =
# 78.6 T full-rate fp32 lane-ops/s; a wave64 v_fmac_f32 occupies a SIMD for
# two cycles (measured on the device: independent FMAs from two or more
# waves per SIMD ran at 2.5-2.6 cycles each, clock and loop overhead
# included; one wave alone issues one VALU instruction per ~4.7 cycles).
# Transcendentals (exp, rcp) run at a quarter of that rate (measured 8.2
# cycles per wave64 v_exp_f32 per SIMD) and count 4 slots.  Packed fp32 is
# not used.
VALU_PEAK_TSLOTS = 256 * 4 * 32 * 2.4e9 / 1e12
TRANS_SLOTS = 4


# Minimum VALU slots per scan element.  Per state: mul (delta*A), exp,
# mul (delta*x*B), FMA (state), FMA (readout) = 4 + exp.  Per element: widen
# x, delta and z, delta*x, D*x, -z*log2e, exp, +1, rcp, z*r, y*silu, narrow y
# = 10 + 2 transcendentals.
def scan_slots_per_element(d_state: int, linear_a: bool = False, io_bf16: bool = False) -> int:
    per_element = 10 + 2 * TRANS_SLOTS
    if not linear_a:
        return (4 + TRANS_SLOTS) * d_state + per_element
    # Structured A (one wave per tile), y = delta * A[d, 0] log2 e: with fp32
    # io exp2 at y, 2y, 4y, 8y, 16y with their scalings, the other decays as
    # one product each; with bf16 io exp2 at y only and every other decay as
    # one product.  Per state mul (delta*x*B), FMA (state), FMA (readout).
    n = min(d_state, 16)
    exps = 1 if io_bf16 else 1 + (n > 1) + (n > 3) + (n > 7) + (n > 15)
    return TRANS_SLOTS * exps + (exps - 1) + 1 + (n - exps) + 3 * d_state + per_element


# Minimum VALU slots per element of the scan's backward pass with the decays
# computed once: per state and step 5 + exp for the forward recomputation
# (mul, exp, mul, FMA, readout FMA, g*h row), 7 for the adjoint step (FMA,
# mul, 3 FMA, dB row mul, lam*abar) and 2 for the channel sums of dB and dC;
# per element 22 + 4 transcendentals (widening, two sigmoids, dz, dx, ddelta,
# narrowing).
def bwd_slots_per_element(d_state: int) -> int:
    return (14 + TRANS_SLOTS) * d_state + 22 + 4 * TRANS_SLOTS


# Sources each kernel family is built from; a traffic figure is reported only
# while the sources of its own kernel still match the ones it was taken on.
_KERNEL_SOURCES = {
    "scan": ("scan_sweep.h", "scan_mode0.hip", "scan_aux.hip"),
    "decode": ("update_kernel.hip",),
    "conv": ("conv_kernels.hip",),
    "bwd": ("scan_bwd.hip", "scan_sweep.h"),
    "ssd": ("ssd_kernel.hip",),
}


def _kernel_source_sha(kind: str) -> str:
    h = hashlib.sha256()
    for f in _KERNEL_SOURCES[kind] + ("ssm_device.h", "ssm_internal.h"):
        with open(os.path.join(REPO, "selective_state_space_84_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def _traffic(workload: str, source_sha: str):
    """HBM bytes per launch from the committed rocprofv3 counter summary, if
    the counters were taken on the current kernel sources; else None."""
    path = os.path.join(REPO, "profiles", "hbm_traffic.txt")
    if not os.path.exists(path):
        return None
    with open(path) as fh:
        for line in fh:
            f = line.split()
            if not f or f[0].startswith("#"):
                continue
            if f[0] == workload and f[2] == source_sha:
                return int(f[7])
    return None


def algorithmic_scan_bytes(batch, seqlen, d_inner, d_state, io_bytes, h0, h_last):
    el = batch * seqlen * d_inner
    return (4 * el * io_bytes                      # x, delta, z read; y written
            + 2 * batch * seqlen * d_state * io_bytes  # B, C
            + d_inner * d_state * 4 + d_inner * 4      # A, D
            + (batch * d_inner * d_state * 4 if h0 else 0)
            + (batch * d_inner * d_state * 4 if h_last else 0))


def to_dev(a, dev):
    import numpy as np
    import torch
    if a is None:
        return None
    if a.dtype == np.uint16:
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).to(dev).view(torch.bfloat16)
    return torch.from_numpy(np.ascontiguousarray(a)).to(dev)


# The GPU's clock ramps up over the first ~50-100 ms of a kernel's load
# (measured: the first 10 back-to-back SSD calls after 2 s idle average
# 0.53 ms, the 100th 0.43 ms; the first 20 Mamba-1.4B scans 2.06 ms, later
# ones 1.78 ms), and a different kernel's load (fp32 matrix products) does
# not bring it there.  Before each leg's warm-up steps the leg's own step
# therefore runs for SETTLE_MS, untimed, so that the timed steps measure the
# kernels at their steady clock rather than the ramp.  The timed region is
# unchanged (exactly the requested steps).
SETTLE_MS = 150.0
_settle_ms = [SETTLE_MS]  # this run's value (--settle-ms)


def settle(fn):
    """Runs fn() back to back for the settle time (untimed); returns the call count."""
    import torch
    t0 = time.time()
    n = 0
    while (time.time() - t0) * 1e3 < _settle_ms[0]:
        for _ in range(4):
            fn()
        n += 4
        torch.cuda.synchronize()
    return n


def bench_scan(cfg, steps, warmup, dev, n_split=0, chunk_len=0, flags=0, inp=None, d=None):
    """Times ssm_scan_fwd on cfg's workload (inputs generated unless given)."""
    import torch
    from selective_state_space_84_amd import binding, inputs
    t0 = time.time()
    softplus = bool(flags & binding.SSM_FLAG_DELTA_SOFTPLUS)
    if inp is None:
        inp = inputs.make_scan_inputs(cfg.batch, cfg.seqlen, cfg.d_inner, cfg.d_state, cfg.dtype, cfg.seed,
                                      cfg.nonzero_h0, raw_delta=softplus)
    gen_s = time.time() - t0
    if d is None:
        d = {k: to_dev(inp.get(k), dev) for k in ("x", "delta", "A", "B", "C", "D", "z", "h0", "dt_bias")}
    y = torch.empty_like(d["x"])
    hl = torch.empty((cfg.batch, cfg.d_inner, cfg.d_state), dtype=torch.float32, device=dev)
    g, chunk_len, n_chunks = binding.scan_plan(cfg.batch, cfg.seqlen, cfg.d_inner, cfg.d_state, n_split, chunk_len,
                                               flags)
    ws_bytes = binding.scan_workspace_size(cfg.batch, cfg.seqlen, cfg.d_inner, cfg.d_state, g, chunk_len, flags)
    ws = torch.empty(ws_bytes, dtype=torch.uint8, device=dev) if ws_bytes else None

    # A call whose inputs and outputs fit the 256 MB Infinity Cache would be
    # partly served from it when the same data is scanned back to back.  Such
    # workloads rotate three copies of their data, so every call finds its own
    # evicted by the two calls before it.
    sets = [(d, y, hl)]
    call_bytes = sum(t.numel() * t.element_size() for t in list(d.values()) + [y, hl] if t is not None)
    if call_bytes < 512 << 20:
        for _ in range(2):
            sets.append(({k: (v.clone() if v is not None else None) for k, v in d.items()}, torch.empty_like(y),
                         torch.empty_like(hl)))

    def step(i):
        di, yi, hi = sets[i % len(sets)]
        binding.ssm_scan_fwd(di["x"], di["delta"], di["A"], di["B"], di["C"], di["D"], di["z"], di["h0"], y=yi,
                             h_last=hi, workspace=ws, n_split=g, chunk_len=chunk_len, flags=flags,
                             dt_bias=di["dt_bias"] if softplus else None)

    ctr = [0]

    def settle_step():
        step(ctr[0])
        ctr[0] += 1

    settle(settle_step)
    for i in range(warmup):
        step(i)
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for i in range(steps):
        step(i)
    e1.record(stream)
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / steps
    # Spread: the same steps again, each between its own pair of events.
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(steps)]
    for i, (a, b) in enumerate(evs):
        a.record(stream)
        step(i)
        b.record(stream)
    torch.cuda.synchronize()
    per = sorted(a.elapsed_time(b) for a, b in evs)
    spread = {"median": round(per[len(per) // 2], 6), "min": round(per[0], 6), "max": round(per[-1], 6)}
    step(0)  # y, hl of the first set (every set holds the same inputs)
    torch.cuda.synchronize()
    del sets
    return inp, d, y, hl, ms, gen_s, (g, chunk_len, n_chunks), spread


def scan_record(cfg, ms, spread, plan, flags, h0, plan_is_default=True):
    """Throughput, HBM and VALU-slot figures of one timed scan leg."""
    from selective_state_space_84_amd import binding
    el = cfg.batch * cfg.seqlen * cfg.d_inner
    io_bytes = 2 if cfg.dtype == "bf16" else 4
    alg = algorithmic_scan_bytes(cfg.batch, cfg.seqlen, cfg.d_inner, cfg.d_state, io_bytes, h0, True)
    linear = bool(flags & binding.SSM_FLAG_A_LINEAR_N)
    slots = scan_slots_per_element(cfg.d_state, linear, cfg.dtype == "bf16")
    el_s = el / (ms * 1e-3)
    gbps = alg / (ms * 1e-3) / 1e9
    g, chunk_len, n_chunks = plan
    # Counter-derived HBM bytes per step (all kernels of the step), for the
    # default plan and while the kernel sources match the ones measured.
    traffic = _traffic(cfg.name + ("+linear" if linear else ""), _kernel_source_sha("scan")) if plan_is_default else None
    return {"workload": cfg.name, "batch": cfg.batch, "seqlen": cfg.seqlen, "d_inner": cfg.d_inner,
            "d_state": cfg.d_state, "io_dtype": cfg.dtype, "h0": bool(h0),
            "path": "structured A (SSM_FLAG_A_LINEAR_N)" if linear else "general A",
            "n_split": g, "chunk_len": chunk_len, "n_chunks": n_chunks,
            "ms_per_step": round(ms, 6), "step_ms": spread, "elements_per_s": round(el_s, 1),
            "algorithmic_bytes": alg, "hbm_gbps": round(gbps, 1), "hbm_frac": round(gbps / HBM_PEAK_GBPS, 4),
            "valu_slots_per_element": slots,
            "valu_frac": round(el_s * slots / 1e12 / VALU_PEAK_TSLOTS, 4),
            "traffic_bytes_per_step": traffic,
            "traffic_vs_algorithmic": round(traffic / alg, 4) if traffic else None,
            "note": "valu_frac counts the unchunked sweep's minimum slots; a chunked plan also runs a summary "
                    "sweep over all chunks but the last" if n_chunks > 1 else ""}


def _host_f64(t):
    import numpy as np
    import torch
    from selective_state_space_84_amd.inputs import bf16_bits_to_f32
    if t.dtype == torch.bfloat16:
        return bf16_bits_to_f32(t.view(torch.int16).cpu().numpy().view(np.uint16)).astype(np.float64)
    return t.cpu().numpy().astype(np.float64)


def _floored(g, r):
    import numpy as np
    floor = 0.1 * float(np.sqrt(np.mean(r * r)))
    return float(np.max(np.abs(g - r) / np.maximum(np.abs(r), floor)))


def oracle_rows(cfg, inp, rows, flags=0, width=256):
    """Oracle y[b] (L, d_inner) and h_last[b] for whole batch rows, channel slices on threads."""
    from concurrent.futures import ThreadPoolExecutor

    import numpy as np

    import oracle
    out = {}

    def run_slice(b, c0):
        c1 = min(cfg.d_inner, c0 + width)
        sl, c = slice(b, b + 1), slice(c0, c1)
        return oracle.scan(inp["x"][sl, :, c], inp["delta"][sl, :, c], inp["A"][c], inp["B"][sl], inp["C"][sl],
                           inp["D"][c], inp["z"][sl, :, c], None if inp.get("h0") is None else inp["h0"][sl, c],
                           inp["dt_bias"][c] if flags & 1 else None, exact_zoh=bool(flags & 2),
                           delta_softplus=bool(flags & 1))

    with ThreadPoolExecutor(_host_threads()) as ex:
        for b in rows:
            parts = list(ex.map(lambda c0: run_slice(b, c0), range(0, cfg.d_inner, width)))
            out[b] = (np.concatenate([p[0][0] for p in parts], axis=1),
                      np.concatenate([p[1][0] for p in parts], axis=0))
    return out


# False with --no-cpu-baseline: the oracle leg (its timing and every whole-row
# comparison with it) is skipped.
_ORACLE_LEG = True


def row_parity(cfg, inp, y, hl, rows, flags=0):
    """Floored errors of whole GPU rows against the oracle (part of the
    cpu_baseline leg)."""
    if not _ORACLE_LEG:
        return {"skipped": "--no-cpu-baseline"}
    ref = oracle_rows(cfg, inp, rows, flags)
    ey = max(_floored(_host_f64(y[b]), ref[b][0]) for b in rows)
    eh = max(_floored(_host_f64(hl[b]), ref[b][1]) for b in rows)
    return {"rows_checked": list(rows), "y_err": ey, "h_last_err": eh,
            "gate": 2e-2 if cfg.dtype == "bf16" else 1e-5,
            "metric": "max |g-r| / max(|r|, 0.1 rms(r)) vs fp64 oracle, whole rows"}


def bench_layer(cfg, steps, warmup, dev, rows, structured=True):
    """General and structured scan legs on one layer shape, with row parity."""
    import torch
    from selective_state_space_84_amd import binding
    inp, d, y, hl, ms, gen_s, plan, spread = bench_scan(cfg, steps, warmup, dev)
    rec = {"general": scan_record(cfg, ms, spread, plan, 0, inp["h0"] is not None), "input_gen_s": round(gen_s, 1)}
    rec["general"]["parity"] = row_parity(cfg, inp, y, hl, rows)
    if structured:
        lin = binding.SSM_FLAG_A_LINEAR_N
        _, _, y2, hl2, ms2, _, plan2, spread2 = bench_scan(cfg, steps, warmup, dev, flags=lin, inp=inp, d=d)
        rec["structured_a"] = scan_record(cfg, ms2, spread2, plan2, lin, inp["h0"] is not None)
        par = row_parity(cfg, inp, y2, hl2, rows)
        par["vs_general_all_rows"] = {"y_err": max(_floored(_host_f64(y2[b]), _host_f64(y[b])) for b in range(cfg.batch)),
                                      "h_last_err": _floored(_host_f64(hl2), _host_f64(hl))}
        rec["structured_a"]["parity"] = par
        del y2, hl2
    del y, hl, d
    torch.cuda.empty_cache()
    return rec


def bench_decode(steps, dev):
    import torch
    from selective_state_space_84_amd import binding, inputs
    cfg = inputs.DECODE
    t0 = time.time()
    inp = inputs.decode_inputs(cfg, steps=steps)
    gen_s = time.time() - t0
    A, D = to_dev(inp["A"], dev), to_dev(inp["D"], dev)
    X, DL, Z, Bm, Cm = (to_dev(inp[k], dev) for k in ("x", "delta", "z", "B", "C"))
    Y = torch.empty_like(X)
    h = torch.zeros((cfg.batch, cfg.d_inner, cfg.d_state), dtype=torch.float32, device=dev)

    def run():
        for s in range(steps):
            binding.ssm_state_update(h, X[s], DL[s], A, Bm[s], Cm[s], D, Z[s], y_t=Y[s])

    settle(lambda: binding.ssm_state_update(h, X[0], DL[0], A, Bm[0], Cm[0], D, Z[0], y_t=Y[0]))
    h.zero_()
    run()  # warm-up pass over the same inputs
    h.zero_()
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    run()
    e1.record(stream)
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / steps
    chans = cfg.batch * cfg.d_inner
    io = 2
    step_bytes = (2 * chans * cfg.d_state * 4 + 4 * chans * io + 2 * cfg.batch * cfg.d_state * io
                  + cfg.d_inner * cfg.d_state * 4 + cfg.d_inner * 4)
    return {
        "workload": cfg.name, "batch": cfg.batch, "d_inner": cfg.d_inner, "d_state": cfg.d_state,
        "io_dtype": cfg.dtype, "steps": steps, "ms_per_step": round(ms, 6),
        "tokens_per_s": round(cfg.batch / (ms * 1e-3), 1),
        "channel_updates_per_s": round(chans / (ms * 1e-3), 1),
        "algorithmic_bytes_per_step": step_bytes,
        "achieved_gbps": round(step_bytes / (ms * 1e-3) / 1e9, 1),
        "frac_of_8tbs": round(step_bytes / (ms * 1e-3) / 1e9 / HBM_PEAK_GBPS, 4),
        "input_gen_s": round(gen_s, 1),
        "traffic_bytes_per_step": _traffic(cfg.name, _kernel_source_sha("decode")),
        "note": "1000 back-to-back eager launches timed together; the kernel-trace mean per launch equals "
                "this per-step time (launches queue ahead, no gaps). The 84 MB state could stay resident "
                "in the 256 MB Infinity Cache between steps; the counters read 178.8 MB of HBM per step",
    }


def bench_conv(cfg, steps, dev, d_conv=4):
    """Causal depthwise conv1d + SiLU on the scan workload's (batch, seqlen,
    d_inner): the Mamba block step that produces the scan's x."""
    import torch
    from selective_state_space_84_amd import binding, inputs
    t0 = time.time()
    inp = inputs.make_conv_inputs(cfg.batch, cfg.seqlen, cfg.d_inner, d_conv, cfg.dtype, 100 + cfg.seed)
    gen_s = time.time() - t0
    x, w, b = (to_dev(inp[k], dev) for k in ("x", "w", "bias"))
    y = torch.empty_like(x)
    st = torch.empty((cfg.batch, cfg.d_inner, d_conv - 1), dtype=torch.float32, device=dev)
    settle(lambda: binding.ssm_conv1d_fwd(x, w, b, y=y, state_out=st))
    for _ in range(3):
        binding.ssm_conv1d_fwd(x, w, b, y=y, state_out=st)
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(steps):
        binding.ssm_conv1d_fwd(x, w, b, y=y, state_out=st)
    e1.record(stream)
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / steps
    el = cfg.batch * cfg.seqlen * cfg.d_inner
    io = 2 if cfg.dtype == "bf16" else 4
    alg = 2 * el * io + cfg.d_inner * (d_conv + 1) * 4 + cfg.batch * cfg.d_inner * (d_conv - 1) * 4
    return {"workload": cfg.name + " conv1d+silu (d_conv %d)" % d_conv, "steps": steps, "ms_per_step": round(ms, 6),
            "elements_per_s": round(el / (ms * 1e-3), 1), "algorithmic_bytes_per_step": alg,
            "achieved_gbps": round(alg / (ms * 1e-3) / 1e9, 1),
            "frac_of_8tbs": round(alg / (ms * 1e-3) / 1e9 / HBM_PEAK_GBPS, 4), "input_gen_s": round(gen_s, 1)}


def bench_bwd(cfg, inp, steps, dev, flags=0):
    """Gradient of the scan (ssm_scan_bwd) on the scan workload, with
    seeded upstream gradients dy (io type) and dh_last, under the same step
    options (softplus step, exact ZOH) as the forward leg."""
    import torch
    from selective_state_space_84_amd import binding, inputs
    gr = inputs.make_scan_grads(cfg.batch, cfg.seqlen, cfg.d_inner, cfg.d_state, cfg.dtype, 200 + cfg.seed)
    d = {k: to_dev(inp.get(k), dev) for k in ("x", "delta", "A", "B", "C", "D", "z", "h0", "dt_bias")}
    dtb = d["dt_bias"] if flags & binding.SSM_FLAG_DELTA_SOFTPLUS else None
    dy, dhl = to_dev(gr["dy"], dev), to_dev(gr["dh_last"], dev)
    ws = torch.empty(binding.scan_bwd_workspace_size(cfg.batch, cfg.seqlen, cfg.d_inner, cfg.d_state),
                     dtype=torch.uint8, device=dev)
    ck = torch.empty(binding.scan_ckpt_bytes(cfg.batch, cfg.seqlen, cfg.d_inner, cfg.d_state) // 4,
                     dtype=torch.float32, device=dev)
    y = torch.empty_like(d["x"])
    hl = torch.empty((cfg.batch, cfg.d_inner, cfg.d_state), dtype=torch.float32, device=dev)
    grads = binding.ssm_scan_bwd(d["x"], d["delta"], d["A"], d["B"], d["C"], d["D"], d["z"], d["h0"], dy=dy,
                                 dh_last=dhl, workspace=ws, flags=flags, dt_bias=dtb)

    def bwd(ckpt=None):
        binding.ssm_scan_bwd(d["x"], d["delta"], d["A"], d["B"], d["C"], d["D"], d["z"], d["h0"], dy=dy,
                             dh_last=dhl, workspace=ws, grads=grads, ckpt=ckpt, flags=flags, dt_bias=dtb)

    def fwd_ckpt():
        binding.ssm_scan_fwd(d["x"], d["delta"], d["A"], d["B"], d["C"], d["D"], d["z"], d["h0"], y=y, h_last=hl,
                             ckpt_out=ck, flags=flags, dt_bias=dtb)

    def timed(fn):
        settle(fn)
        for _ in range(2):
            fn()
        torch.cuda.synchronize()
        stream = torch.cuda.current_stream()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(steps):
            fn()
        e1.record(stream)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / steps

    ms = timed(bwd)
    ms_fc = timed(fwd_ckpt)
    ms_bc = timed(lambda: bwd(ck))
    el = cfg.batch * cfg.seqlen * cfg.d_inner
    # The slot count is that of the plain step; the options add work it does not count.
    alu = None
    if not flags:
        slots = bwd_slots_per_element(cfg.d_state)
        frac = el * slots / (ms_bc * 1e-3) / 1e12 / VALU_PEAK_TSLOTS
        alu = {"min_slots_per_element": slots, "frac_of_valu_peak_bwd_from_ckpt": round(frac, 4)}
    return {"workload": cfg.name + " scan backward (all gradients)", "steps": steps, "ms_per_step": round(ms, 6),
            "elements_per_s": round(el / (ms * 1e-3), 1),
            "training_path": {"fwd_with_ckpt_ms": round(ms_fc, 6), "bwd_from_ckpt_ms": round(ms_bc, 6),
                              "fwd_plus_bwd_ms": round(ms_fc + ms_bc, 6)},
            "alu": alu,
            "workspace_bytes": int(ws.numel()), "ckpt_bytes": int(ck.numel() * 4)}


def bench_ssd(steps, dev):
    """Scan with a scalar decay per head (Mamba-2 / SSD form) on the
    Mamba-2 2.7B layer shape, evaluated chunk-wise on the matrix cores."""
    import torch
    from selective_state_space_84_amd import binding, inputs
    cfg = inputs.SSD_2P7B
    t0 = time.time()
    inp = inputs.make_ssd_inputs(cfg.batch, cfg.seqlen, cfg.nheads, cfg.headdim, cfg.ngroups, cfg.d_state, cfg.seed)
    gen_s = time.time() - t0
    d = {k: to_dev(inp.get(k), dev) for k in ("x", "dt", "A", "B", "C", "D", "z")}
    y = torch.empty_like(d["x"])
    hl = torch.empty((cfg.batch, cfg.nheads, cfg.headdim, cfg.d_state), dtype=torch.float32, device=dev)

    def step():
        binding.ssm_ssd_fwd(d["x"], d["dt"], d["A"], d["B"], d["C"], d["D"], d["z"], y=y, h_last=hl)

    settle(step)
    for _ in range(3):
        step()
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(steps):
        step()
    e1.record(stream)
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / steps
    el = cfg.batch * cfg.seqlen * cfg.nheads * cfg.headdim
    alg = (3 * el * 2 + cfg.batch * cfg.seqlen * cfg.nheads * 2 + 2 * cfg.batch * cfg.seqlen * cfg.ngroups * cfg.d_state * 2
           + 2 * cfg.nheads * 4 + cfg.batch * cfg.nheads * cfg.headdim * cfg.d_state * 4)
    # Matrix-core work as issued per 32-step chunk and (row, head): three
    # causal 16x16 score tiles over N/32 slices, then per 16-channel wave the
    # two output tiles (masked scores x X with hi/lo scores, C x H with hi/lo
    # state over N/32 slices) and N/16 state tiles (hi/lo scaled input);
    # 16x16x32 products.
    nk = cfg.d_state // 32
    mfma = 3 * nk + 4 * (2 * (2 + 2 * nk) + 2 * (cfg.d_state // 16))
    flops = mfma * 16 * 16 * 32 * 2 * (-(-cfg.seqlen // 32)) * cfg.batch * cfg.nheads
    gbps = alg / (ms * 1e-3) / 1e9
    return {"workload": "%s ssd (batch %d, L %d, %d heads x %d, d_state %d, bf16 io)" % (
                cfg.name, cfg.batch, cfg.seqlen, cfg.nheads, cfg.headdim, cfg.d_state),
            "steps": steps, "ms_per_step": round(ms, 6), "elements_per_s": round(el / (ms * 1e-3), 1),
            "roofline": {"bound": "hbm", "achieved": round(gbps, 1), "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                         "frac": round(gbps / HBM_PEAK_GBPS, 4), "algorithmic_bytes_per_launch": alg,
                         "traffic": _traffic(cfg.name, _kernel_source_sha("ssd"))},
            "mfma": {"tflops_issued": round(flops / (ms * 1e-3) / 1e12, 2), "peak_bf16_tflops": 2500.0},
            "input_gen_s": round(gen_s, 1)}


def _host_threads() -> int:
    """Worker threads for the CPU baseline: the cores this process may run
    on, at most 16 (the host share of one GPU)."""
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:
        n = os.cpu_count() or 1
    return max(1, min(16, n))


def cpu_baseline(cfg, inp, y_dev, hl_dev, cpu_budget_s=24.0, flags=0):
    """fp64 oracle on whole batch rows of the same workload, each row's
    channels cut into slices run on a thread pool (channels never interact,
    and the C oracle releases the GIL), row after row until about
    cpu_budget_s seconds of CPU work are spent; also compares those rows'
    GPU outputs with the oracle."""
    from concurrent.futures import ThreadPoolExecutor

    import numpy as np
    import torch

    import oracle
    from selective_state_space_84_amd.inputs import bf16_bits_to_f32
    threads = _host_threads()
    width = 256
    rows = 0
    el = 0
    spent = 0.0
    worst_y = worst_h = 0.0

    def err(g, r):
        floor = 0.1 * float(np.sqrt(np.mean(r * r)))
        return float(np.max(np.abs(g - r) / np.maximum(np.abs(r), floor)))

    def run_slice(b, c0):
        c1 = min(cfg.d_inner, c0 + width)
        s, c = slice(b, b + 1), slice(c0, c1)
        pick = lambda k: None if inp.get(k) is None else inp[k]
        return oracle.scan(inp["x"][s, :, c], inp["delta"][s, :, c], inp["A"][c], inp["B"][s], inp["C"][s],
                           None if pick("D") is None else inp["D"][c], None if pick("z") is None else inp["z"][s, :, c],
                           None if pick("h0") is None else inp["h0"][s, c],
                           inp["dt_bias"][c] if flags & 1 else None, exact_zoh=bool(flags & 2),
                           delta_softplus=bool(flags & 1))

    with ThreadPoolExecutor(threads) as ex:
        while rows < cfg.batch and spent * threads < cpu_budget_s:
            b = rows
            t0 = time.perf_counter()
            parts = list(ex.map(lambda c0: run_slice(b, c0), range(0, cfg.d_inner, width)))
            spent += time.perf_counter() - t0
            ry = np.concatenate([p[0][0] for p in parts], axis=1)
            rh = np.concatenate([p[1][0] for p in parts], axis=0)
            rows += 1
            el += cfg.seqlen * cfg.d_inner
            yb = y_dev[b]
            if yb.dtype == torch.bfloat16:
                g = bf16_bits_to_f32(yb.view(torch.int16).cpu().numpy().view(np.uint16)).astype(np.float64)
            else:
                g = yb.cpu().numpy().astype(np.float64)
            worst_y = max(worst_y, err(g, ry))
            worst_h = max(worst_h, err(hl_dev[b].cpu().numpy().astype(np.float64), rh))
    # The same oracle on one thread: one slice of row 0.
    t0 = time.perf_counter()
    run_slice(0, 0)
    t1 = time.perf_counter() - t0
    el1 = cfg.seqlen * min(width, cfg.d_inner)
    return {
        "value": round(el / spent, 1), "unit": "elements/s", "cores": threads, "kind": "oracle",
        "sample": "batch rows 0..%d of the same workload (all %d channels x %d timesteps each, %d elements), "
                  "fp64 C loop on %d threads over %d-channel slices, %.2f s wall" % (
                      rows - 1, cfg.d_inner, cfg.seqlen, el, threads, width, spent),
        "single_thread": {"value": round(el1 / t1, 1), "unit": "elements/s", "cores": 1,
                          "sample": "channels 0..%d of row 0 (%d elements), %.3f s" % (
                              min(width, cfg.d_inner) - 1, el1, t1)},
    }, {"rows_checked": rows, "y_err": worst_y, "h_last_err": worst_h,
        "metric": "max |g-r| / max(|r|, 0.1 rms(r)) vs fp64 oracle", "gate": 2e-2 if cfg.dtype == "bf16" else 1e-5}


def log(msg):
    """Progress on stderr (stdout carries only the JSON line)."""
    print("[bench %6.1fs] %s" % (time.time() - _T0, msg), file=sys.stderr, flush=True)


_T0 = time.time()


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    from selective_state_space_84_amd.inputs import SCAN_CONFIGS
    ap.add_argument("--workload", default="mamba-1.4b-layer", choices=sorted(SCAN_CONFIGS))
    ap.add_argument("--decode-steps", type=int, default=1000)
    ap.add_argument("--no-decode", action="store_true")
    ap.add_argument("--no-conv", action="store_true")
    ap.add_argument("--no-bwd", action="store_true")
    ap.add_argument("--no-ssd", action="store_true")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--settle-ms", type=float, default=SETTLE_MS,
                    help="untimed run of each leg's own step before its warm-up (0: none; counter runs use 0 so "
                         "that their dispatch sequence does not depend on timing)")
    ap.add_argument("--no-extra-scans", action="store_true",
                    help="skip the structured-A, 2.8B-long, 130M and per-channel-parameter legs")
    ap.add_argument("--n-split", type=int, default=0, help="override the launch plan (tuning)")
    ap.add_argument("--chunk-len", type=int, default=0, help="override the launch plan (tuning)")
    ap.add_argument("--flags", default="",
                    help="comma list: softplus (fused softplus step), zoh (exact ZOH), linear (structured A)")
    args = ap.parse_args()
    global _ORACLE_LEG
    _ORACLE_LEG = not args.no_cpu_baseline
    _settle_ms[0] = max(0.0, args.settle_ms)
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py measures one GPU only: this library runs the scan on a single MI355X and has no "
              "multi-GPU path (--gpus %d requested)" % args.gpus, file=sys.stderr)
        sys.exit(2)

    import torch
    from selective_state_space_84_amd import binding, inputs
    dev = "cuda:0"
    binding.load_library()
    cfg = inputs.SCAN_CONFIGS[args.workload]
    flag_bits = {"softplus": binding.SSM_FLAG_DELTA_SOFTPLUS, "zoh": binding.SSM_FLAG_EXACT_ZOH,
                 "linear": binding.SSM_FLAG_A_LINEAR_N}
    flag_names = [f for f in args.flags.split(",") if f]
    unknown = [f for f in flag_names if f not in flag_bits]
    if unknown:
        ap.error("unknown --flags %s (known: %s)" % (",".join(unknown), ",".join(flag_bits)))
    flags = sum(flag_bits[f] for f in flag_names)
    log("headline: %s scan, flags %d" % (cfg.name, flags))
    inp, d, y, hl, ms, gen_s, plan, spread = bench_scan(cfg, args.steps, args.warmup, dev, args.n_split,
                                                        args.chunk_len, flags)
    g, chunk_len, n_chunks = plan
    rec = scan_record(cfg, ms, spread, plan, flags & binding.SSM_FLAG_A_LINEAR_N, inp["h0"] is not None,
                      plan_is_default=not (args.n_split or args.chunk_len or flags & 3))
    alg_bytes = rec["algorithmic_bytes"]
    gbps = rec["hbm_gbps"]
    slots = rec["valu_slots_per_element"]
    achieved_slots = rec["elements_per_s"] * slots / 1e12
    sha = _kernel_source_sha("scan")
    out = {
        "metric": "selective-scan elements/s (B·L·d_inner) and achieved HBM GB/s vs peak",
        "value": rec["elements_per_s"],
        "unit": "elements/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "clock_settle": {"ms": _settle_ms[0], "note": "before its warm-up steps each leg's own step runs back to back, "
                         "untimed, for this long, so that the GPU clock has left its ramp (the first ~50-100 ms of a "
                         "kernel's load run up to 25% slower); the timed steps are exactly the requested ones"},
        "ms_per_step": round(ms, 6),
        "step_ms": spread,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "io_dtype": cfg.dtype,
        "data": "synthetic (seeded; Mamba layer init distributions)",
        "config": {"workload": cfg.name + " scan", "batch": cfg.batch, "seqlen": cfg.seqlen,
                   "d_inner": cfg.d_inner, "d_state": cfg.d_state, "io_dtype": cfg.dtype, "state_dtype": "f32",
                   "h0": inp["h0"] is not None, "n_split": g, "n_chunks": n_chunks,
                   "variant": "+".join(flag_names) or "plain (general A)"},
        "hbm_gbps": gbps,
        "hbm_frac_of_peak": rec["hbm_frac"],
        "roofline": {"bound": "hbm", "achieved": gbps, "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                     "frac": rec["hbm_frac"],
                     "traffic": rec["traffic_bytes_per_step"],
                     "algorithmic_bytes_per_launch": alg_bytes,
                     "kernel": "k_scan_sweep (one launch per step)" if n_chunks == 1 else
                               "k_scan_sweep summary + k_chunk_carry + k_scan_sweep (per step)"},
        "roofline_alu": {"bound": "alu", "achieved": round(achieved_slots, 3), "peak": round(VALU_PEAK_TSLOTS, 3),
                         "unit": "Tslot/s", "frac": round(achieved_slots / VALU_PEAK_TSLOTS, 4),
                         "slots_per_element": slots,
                         "note": "VALU lane-slots of the sweep (exp and rcp 4 slots, non-packed fp32): the "
                                 "bound of the general-A scan, whose slot roof lies at ~54% of the HBM roof"},
        "kernel_source_sha": sha,
        "input_gen_s": round(gen_s, 1),
    }
    if not args.no_cpu_baseline:
        log("cpu baseline")
        cb, par = cpu_baseline(cfg, inp, y, hl, flags=flags)
        out["cpu_baseline"] = cb
        out["parity"] = par
    extra = not args.no_extra_scans and args.workload == "mamba-1.4b-layer" and not flags
    if extra:
        lin = binding.SSM_FLAG_A_LINEAR_N
        log("structured A on the headline workload")
        _, _, y2, hl2, ms2, _, plan2, spread2 = bench_scan(cfg, args.steps, args.warmup, dev, flags=lin, inp=inp, d=d)
        sa = scan_record(cfg, ms2, spread2, plan2, lin, inp["h0"] is not None)
        sa["roofline"] = {"bound": "hbm", "achieved": sa["hbm_gbps"], "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                          "frac": sa["hbm_frac"], "algorithmic_bytes_per_launch": sa["algorithmic_bytes"]}
        rows = [0, cfg.batch - 1]
        sa["parity"] = row_parity(cfg, inp, y2, hl2, rows)
        sa["parity"]["vs_general_all_rows"] = {
            "y_err": max(_floored(_host_f64(y2[b]), _host_f64(y[b])) for b in range(cfg.batch)),
            "h_last_err": _floored(_host_f64(hl2), _host_f64(hl))}
        out["structured_a"] = sa
        del y2, hl2
        log("per-channel parameters on the headline workload")
        A, Dv = inputs.channel_params(cfg.d_inner, cfg.d_state, cfg.seed, "random")
        d["A"], d["D"] = to_dev(A, dev), to_dev(Dv, dev)
        pin = dict(inp, A=A, D=Dv)
        yp, hp = binding.ssm_scan_fwd(d["x"], d["delta"], d["A"], d["B"], d["C"], d["D"], d["z"], d["h0"])
        torch.cuda.synchronize()
        out["parity_channel_params"] = dict(row_parity(cfg, pin, yp, hp, rows),
                                            params="A[d,n] = -(n+1) exp(U[-0.5,0.5]), D ~ N(1, 0.5)")
        del yp, hp
    del y, hl, d
    torch.cuda.empty_cache()
    if extra:
        log("mamba-2.8b long layer")
        out["scan_c4"] = bench_layer(inputs.MAMBA_2P8B_LONG, max(3, args.steps // 2), args.warmup, dev, rows=[1])
        log("mamba-130m layer")
        out["scan_c2"] = bench_layer(inputs.MAMBA_130M, args.steps, args.warmup, dev, rows=[0, 7])
    if not args.no_bwd and cfg.d_state <= 16:
        log("backward")
        out["scan_bwd"] = bench_bwd(cfg, inp, max(1, args.steps // 2), dev, flags & 3)
        torch.cuda.empty_cache()
    if not args.no_conv:
        log("conv1d")
        out["conv1d"] = bench_conv(cfg, args.steps, dev)
        torch.cuda.empty_cache()
    if not args.no_decode:
        log("decode")
        out["decode"] = bench_decode(args.decode_steps, dev)
        torch.cuda.empty_cache()
    if not args.no_ssd:
        log("ssd")
        out["ssd"] = bench_ssd(args.steps, dev)
    log("done")
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
