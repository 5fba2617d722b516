"""Whole batch rows of the full layer shapes against the fp64 oracle.

The sampled-channel tests pick a few dozen channels; here every channel of
the chosen rows is compared, so each 64-channel tile, each sequence chunk of
the automatic plan (its summary, carry and main sweep) and each tile edge is
covered at the size the benchmark times:

* Mamba-130M layer (8 x 2048 x 1536, 32 chunks): all 8 rows, general and
  structured A;
* Mamba-2.8B long layer (4 x 32768 x 5120, h0 != 0, 52 chunks): all 4 rows;
* decode, 256 x 5120 x 16 over 1000 steps: rows 0, 1, 128 and 255, every
  channel and every step, and their final states.

Gate: the bf16 one (2e-2, floored metric).  The oracle runs on slices of 256
channels in a thread pool (the C oracle releases the GIL)."""
import os
from concurrent.futures import ThreadPoolExecutor

import numpy as np
import pytest

import oracle
from conftest import floored_rel_err
from selective_state_space_84_amd import inputs

pytestmark = pytest.mark.gpu

WIDTH = 256


def _threads():
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:
        n = os.cpu_count() or 1
    return max(1, min(16, n))


def _oracle_rows(inp, rows):
    """y[b] (L, d_inner) and h_last[b] (d_inner, N) for whole rows."""
    d_inner = inp["x"].shape[2]
    h0 = inp.get("h0")

    def run(b, c0):
        sl, c = slice(b, b + 1), slice(c0, min(d_inner, c0 + WIDTH))
        return oracle.scan(inp["x"][sl, :, c], inp["delta"][sl, :, c], inp["A"][c], inp["B"][sl], inp["C"][sl],
                           inp["D"][c], inp["z"][sl, :, c], None if h0 is None else h0[sl, c])

    out = {}
    with ThreadPoolExecutor(_threads()) as ex:
        for b in rows:
            parts = list(ex.map(lambda c0: run(b, c0), range(0, d_inner, WIDTH)))
            out[b] = (np.concatenate([p[0][0] for p in parts], axis=1),
                      np.concatenate([p[1][0] for p in parts], axis=0))
    return out


@pytest.mark.parametrize("name,rows", [("mamba-130m-layer", list(range(8))), ("mamba-2.8b-long-layer", [0, 1, 2, 3])])
@pytest.mark.parametrize("structured", [False, True])
def test_layer_whole_rows(lib, name, rows, structured):
    import torch
    from gpu_util import dev_inputs, to_host_f64
    from selective_state_space_84_amd import binding
    cfg = inputs.SCAN_CONFIGS[name]
    print("generating", name, flush=True)
    inp = inputs.scan_inputs(cfg)
    d = dev_inputs(inp)
    flags = binding.SSM_FLAG_A_LINEAR_N if structured else 0
    print("launching", name, "flags", flags, "plan", binding.scan_plan(cfg.batch, cfg.seqlen, cfg.d_inner,
                                                                     cfg.d_state, flags=flags), flush=True)
    y, hl = binding.ssm_scan_fwd(d["x"], d["delta"], d["A"], d["B"], d["C"], d["D"], d["z"], d["h0"], flags=flags)
    torch.cuda.synchronize()
    got = {b: (to_host_f64(y[b]), to_host_f64(hl[b])) for b in rows}
    del y, hl, d
    torch.cuda.empty_cache()
    print("oracle on rows", rows, flush=True)
    ref = _oracle_rows(inp, rows)
    for b in rows:
        ey, eh = floored_rel_err(got[b][0], ref[b][0]), floored_rel_err(got[b][1], ref[b][1])
        print(name, "row", b, "y %.3g h %.3g" % (ey, eh), flush=True)
        assert ey <= 2e-2 and eh <= 2e-2, (b, ey, eh)


def test_decode_whole_rows(lib):
    import torch
    from gpu_util import to_dev, to_host_f64
    from selective_state_space_84_amd import binding
    cfg = inputs.DECODE
    print("generating decode inputs", flush=True)
    inp = inputs.decode_inputs(cfg)
    A, D = to_dev(inp["A"]), to_dev(inp["D"])
    h = torch.zeros((cfg.batch, cfg.d_inner, cfg.d_state), dtype=torch.float32, device="cuda:0")
    X, DL, Z, Bm, Cm = (to_dev(inp[k]) for k in ("x", "delta", "z", "B", "C"))
    Y = torch.empty_like(X)
    print("running %d steps" % cfg.steps, flush=True)
    for s in range(cfg.steps):
        binding.ssm_state_update(h, X[s], DL[s], A, Bm[s], Cm[s], D, Z[s], y_t=Y[s])
    torch.cuda.synchronize()
    rows = [0, 1, cfg.batch // 2, cfg.batch - 1]
    # Row b's decode sequence is a scan over the steps of (1, steps, d_inner).
    seq = {k: inp[k][:, rows].transpose(1, 0, 2) for k in ("x", "delta", "z", "B", "C")}
    seq.update(A=inp["A"], D=inp["D"])
    print("oracle on rows", rows, flush=True)
    ref = _oracle_rows(seq, range(len(rows)))
    for i, b in enumerate(rows):
        ey = floored_rel_err(to_host_f64(Y[:, b]), ref[i][0])
        eh = floored_rel_err(to_host_f64(h[b]), ref[i][1])
        print("decode row", b, "y %.3g h %.3g" % (ey, eh), flush=True)
        assert ey <= 2e-2 and eh <= 2e-2, (b, ey, eh)


def test_ssd_whole_rows(lib):
    """The Mamba-2 2.7B layer (SSD form, 8 x 4096, 80 heads x 64, d_state 128):
    every head of batch rows 0 and 7 against the oracle (one head per task;
    heads never interact)."""
    import torch
    from gpu_util import to_dev, to_host_f64
    from selective_state_space_84_amd import binding
    cfg = inputs.SSD_2P7B
    print("generating", cfg.name, flush=True)
    inp = inputs.make_ssd_inputs(cfg.batch, cfg.seqlen, cfg.nheads, cfg.headdim, cfg.ngroups, cfg.d_state, cfg.seed)
    d = {k: to_dev(inp.get(k)) for k in ("x", "dt", "A", "B", "C", "D", "z")}
    y, hl = binding.ssm_ssd_fwd(d["x"], d["dt"], d["A"], d["B"], d["C"], d["D"], d["z"])
    torch.cuda.synchronize()
    rows = [0, cfg.batch - 1]
    got = {b: (to_host_f64(y[b]), to_host_f64(hl[b])) for b in rows}
    del y, hl, d
    hpg = cfg.nheads // cfg.ngroups

    def run(b, h):
        sl = lambda k: inp[k][b:b + 1, :, h:h + 1]
        g = h // hpg
        return oracle.ssd(sl("x"), sl("dt"), inp["A"][h:h + 1], inp["B"][b:b + 1, :, g:g + 1],
                          inp["C"][b:b + 1, :, g:g + 1], inp["D"][h:h + 1], sl("z"))

    print("oracle on rows", rows, flush=True)
    with ThreadPoolExecutor(_threads()) as ex:
        for b in rows:
            parts = list(ex.map(lambda h: run(b, h), range(cfg.nheads)))
            ry = np.concatenate([p[0][0] for p in parts], axis=1)   # (L, heads, headdim)
            rh = np.concatenate([p[1][0] for p in parts], axis=0)   # (heads, headdim, N)
            ey, eh = floored_rel_err(got[b][0], ry), floored_rel_err(got[b][1], rh)
            print("ssd row", b, "y %.3g h %.3g" % (ey, eh), flush=True)
            assert ey <= 2e-2 and eh <= 2e-2, (b, ey, eh)
