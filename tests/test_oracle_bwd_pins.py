"""Pins for the oracle's scan gradient (oracle.scan_bwd), CPU only.

The gradient is checked against things that do not share its derivation:
  * central finite differences of the (separately pinned) forward oracle, for
    every element of every input, in every mode;
  * Euler identities: the loss is homogeneous of degree one in (x, h0), in
    (B, h0) apart from the skip term, and in C apart from the skip term, so
    sum(grad * input) must equal fixed parts of the loss;
  * a one-step, one-state problem differentiated by hand;
  * autograd over an fp64 torch recurrence written here from the definition;
  * the LTI closed form dh0 = dh_last * exp(A * sum(delta)) when dy = 0.
A dropped term, a wrong sign or a swapped operand in the gradient fails one
of these.
"""
import math

import numpy as np
import pytest

import oracle

MODES = [(False, False), (True, False), (False, True), (True, True)]  # (exact_zoh, delta_softplus)


def _problem(seed, batch=2, seqlen=6, d_inner=3, d_state=4, softplus=False, zero_a=False):
    r = np.random.default_rng(seed)
    p = {
        "x": r.normal(size=(batch, seqlen, d_inner)),
        "A": -r.uniform(0.3, 2.0, size=(d_inner, d_state)),
        "B": r.normal(size=(batch, seqlen, d_state)),
        "C": r.normal(size=(batch, seqlen, d_state)),
        "D": r.normal(size=d_inner),
        "z": r.normal(size=(batch, seqlen, d_inner)),
        "h0": r.normal(size=(batch, d_inner, d_state)),
    }
    if softplus:
        p["delta"] = r.normal(-1.0, 1.0, size=(batch, seqlen, d_inner))
        p["dt_bias"] = r.uniform(-2.0, 0.0, size=d_inner)
    else:
        p["delta"] = r.uniform(0.05, 0.6, size=(batch, seqlen, d_inner))
    if zero_a:
        p["A"][0, 1] = 0.0
    dy = r.normal(size=(batch, seqlen, d_inner))
    dhl = r.normal(size=(batch, d_inner, d_state))
    return p, dy, dhl


def _loss(p, dy, dhl, zoh, sp):
    y, hl = oracle.scan(p["x"], p["delta"], p["A"], p["B"], p["C"], p.get("D"), p.get("z"), p.get("h0"),
                        p.get("dt_bias"), exact_zoh=zoh, delta_softplus=sp)
    return float(np.sum(dy * y) + (0.0 if dhl is None else np.sum(dhl * hl)))


def _grads(p, dy, dhl, zoh, sp):
    return oracle.scan_bwd(p["x"], p["delta"], p["A"], p["B"], p["C"], p.get("D"), p.get("z"), p.get("h0"),
                           p.get("dt_bias"), dy=dy, dh_last=dhl, exact_zoh=zoh, delta_softplus=sp)


GRAD_OF = {"x": "dx", "delta": "ddelta", "A": "dA", "B": "dB", "C": "dC", "D": "dD", "z": "dz", "h0": "dh0",
           "dt_bias": "d_dt_bias"}


@pytest.mark.parametrize("zoh,sp", MODES)
def test_bwd_matches_central_differences(zoh, sp):
    p, dy, dhl = _problem(10 + 2 * zoh + sp, softplus=sp, zero_a=zoh)
    g = _grads(p, dy, dhl, zoh, sp)
    for name, arr in p.items():
        fd = np.empty_like(arr)
        flat = arr.reshape(-1)
        for i in range(flat.size):
            v = flat[i]
            h = 1e-6 * max(1.0, abs(v))
            flat[i] = v + h
            lp = _loss(p, dy, dhl, zoh, sp)
            flat[i] = v - h
            lm = _loss(p, dy, dhl, zoh, sp)
            flat[i] = v
            fd.reshape(-1)[i] = (lp - lm) / (2 * h)
        an = g[GRAD_OF[name]]
        scale = max(1.0, float(np.max(np.abs(an))))
        assert np.max(np.abs(fd - an)) <= 2e-7 * scale, name


def test_bwd_optional_inputs_absent():
    """D, z, h0 and dh_last absent: the gradient is that of the reduced loss."""
    p, dy, _ = _problem(30)
    for k in ("D", "z", "h0"):
        del p[k]
    g = _grads(p, dy, None, False, False)
    assert set(g) == {"dx", "ddelta", "dA", "dB", "dC", "dh0"}
    for name in ("x", "B", "A"):
        arr = p[name]
        flat = arr.reshape(-1)
        for i in range(0, flat.size, 3):
            v = flat[i]
            h = 1e-6 * max(1.0, abs(v))
            flat[i] = v + h
            lp = _loss(p, dy, None, False, False)
            flat[i] = v - h
            lm = _loss(p, dy, None, False, False)
            flat[i] = v
            assert abs((lp - lm) / (2 * h) - g[GRAD_OF[name]].reshape(-1)[i]) <= 2e-7 * max(
                1.0, float(np.max(np.abs(g[GRAD_OF[name]])))), name


@pytest.mark.parametrize("zoh,sp", MODES)
def test_bwd_euler_identities(zoh, sp):
    p, dy, dhl = _problem(40 + 2 * zoh + sp, batch=2, seqlen=9, d_inner=4, d_state=5, softplus=sp)
    y, hl = oracle.scan(p["x"], p["delta"], p["A"], p["B"], p["C"], p["D"], p["z"], p["h0"], p.get("dt_bias"),
                        exact_zoh=zoh, delta_softplus=sp)
    g = _grads(p, dy, dhl, zoh, sp)
    L = float(np.sum(dy * y) + np.sum(dhl * hl))
    silu_z = p["z"] / (1.0 + np.exp(-p["z"]))
    skip = float(np.sum(dy * silu_z * p["D"][None, None, :] * p["x"]))  # sum dy * silu(z) * D x
    tol = 1e-11 * max(1.0, abs(L))
    # Degree one in (x, h0) jointly.
    assert abs(np.sum(g["dx"] * p["x"]) + np.sum(g["dh0"] * p["h0"]) - L) <= tol
    # Degree one in (B, h0) jointly, apart from the skip term.
    assert abs(np.sum(g["dB"] * p["B"]) + np.sum(g["dh0"] * p["h0"]) - (L - skip)) <= tol
    # Degree one in C for the readout part of y; h_last does not depend on C.
    assert abs(np.sum(g["dC"] * p["C"]) - (float(np.sum(dy * y)) - skip)) <= tol
    # The skip term is linear in D.
    assert abs(np.sum(g["dD"] * p["D"]) - skip) <= tol


def test_bwd_one_step_by_hand():
    """batch = seqlen = d_inner = d_state = 1, simplified input term."""
    x, dl, A, B, C, D, z, h0 = 0.7, 0.3, -1.3, 0.4, -0.9, 0.25, 0.6, 1.1
    dy, dhl = 0.8, -0.5
    a = math.exp(dl * A)
    h = a * h0 + dl * B * x
    ypre = C * h + D * x
    s = 1.0 / (1.0 + math.exp(-z))
    lam = dy * z * s * C + dhl  # dL/dh
    want = {
        "dx": dy * z * s * D + lam * dl * B,
        "ddelta": lam * (A * a * h0 + B * x),
        "dA": lam * dl * a * h0,
        "dB": lam * dl * x,
        "dC": dy * z * s * h,
        "dD": dy * z * s * x,
        "dz": dy * ypre * (s + z * s * (1.0 - s)),
        "dh0": lam * a,
    }
    g = oracle.scan_bwd(np.full((1, 1, 1), x), np.full((1, 1, 1), dl), np.full((1, 1), A), np.full((1, 1, 1), B),
                        np.full((1, 1, 1), C), np.full(1, D), np.full((1, 1, 1), z), np.full((1, 1, 1), h0),
                        dy=np.full((1, 1, 1), dy), dh_last=np.full((1, 1, 1), dhl))
    for k, v in want.items():
        assert abs(float(g[k].reshape(-1)[0]) - v) <= 1e-14 * max(1.0, abs(v)), k


def test_bwd_one_step_by_hand_zoh_softplus():
    """One step with the exact-ZOH input term and softplus(raw + bias)."""
    x, raw, bias, A, B, C, h0 = -0.6, 0.2, -1.1, -2.2, 0.9, 0.5, -0.4
    dy, dhl = 1.3, 0.7
    v = raw + bias
    dt = math.log1p(math.exp(v))
    sg = 1.0 / (1.0 + math.exp(-v))
    a = math.exp(dt * A)
    coef = (a - 1.0) / A
    h = a * h0 + coef * B * x
    lam = dy * C + dhl
    dcoef_dA = (dt * a * A - (a - 1.0)) / (A * A)
    want = {
        "dx": lam * coef * B,
        "ddelta": lam * (A * a * h0 + a * B * x) * sg,
        "d_dt_bias": lam * (A * a * h0 + a * B * x) * sg,
        "dA": lam * (dt * a * h0 + dcoef_dA * B * x),
        "dB": lam * coef * x,
        "dC": dy * h,
        "dh0": lam * a,
    }
    g = oracle.scan_bwd(np.full((1, 1, 1), x), np.full((1, 1, 1), raw), np.full((1, 1), A), np.full((1, 1, 1), B),
                        np.full((1, 1, 1), C), None, None, np.full((1, 1, 1), h0), np.full(1, bias),
                        dy=np.full((1, 1, 1), dy), dh_last=np.full((1, 1, 1), dhl), exact_zoh=True,
                        delta_softplus=True)
    for k, v in want.items():
        assert abs(float(g[k].reshape(-1)[0]) - v) <= 1e-13 * max(1.0, abs(v)), k


def _torch_scan(x, delta, A, B, C, D, z, h0, dt_bias, zoh, sp):
    """The scan written from its definition with torch fp64 ops (one step per
    loop iteration), for autograd to differentiate."""
    import torch
    batch, seqlen, d_inner = x.shape
    dt = torch.nn.functional.softplus(delta + dt_bias) if sp else delta
    h = h0.clone()
    ys = []
    for t in range(seqlen):
        dA = dt[:, t, :, None] * A[None]  # (b, d, n)
        abar = torch.exp(dA)
        if zoh:
            bbar = torch.expm1(dA) / A[None] * B[:, t, None, :]
        else:
            bbar = dt[:, t, :, None] * B[:, t, None, :]
        h = abar * h + bbar * x[:, t, :, None]
        y = (h * C[:, t, None, :]).sum(-1) + D[None] * x[:, t]
        ys.append(y * torch.nn.functional.silu(z[:, t]))
    return torch.stack(ys, 1), h


@pytest.mark.parametrize("zoh,sp", MODES)
def test_bwd_matches_torch_autograd(zoh, sp):
    import torch
    p, dy, dhl = _problem(60 + 2 * zoh + sp, batch=3, seqlen=11, d_inner=5, d_state=6, softplus=sp)
    if not sp:
        p["dt_bias"] = np.zeros(5)
    t = {k: torch.tensor(v, dtype=torch.float64, requires_grad=True) for k, v in p.items()}
    y, hl = _torch_scan(t["x"], t["delta"], t["A"], t["B"], t["C"], t["D"], t["z"], t["h0"], t["dt_bias"], zoh, sp)
    L = (torch.tensor(dy) * y).sum() + (torch.tensor(dhl) * hl).sum()
    names = list(t)
    tg = dict(zip(names, torch.autograd.grad(L, [t[k] for k in names], allow_unused=True)))
    g = _grads(p, dy, dhl, zoh, sp)
    for k in names:
        if k == "dt_bias" and not sp:
            continue
        ref = tg[k].numpy()
        assert np.max(np.abs(g[GRAD_OF[k]] - ref)) <= 1e-11 * max(1.0, float(np.max(np.abs(ref)))), k


def test_bwd_lti_state_gradient_closed_form():
    """dy = 0: only h_last carries loss, and h_last = exp(A sum(delta)) h0 + (terms
    free of h0), so dh0 = dh_last * exp(A * sum_t delta_t)."""
    p, _, dhl = _problem(70, batch=2, seqlen=13, d_inner=3, d_state=4)
    dy = np.zeros_like(p["x"])
    g = _grads(p, dy, dhl, False, False)
    want = dhl * np.exp(p["A"][None] * p["delta"].sum(1)[:, :, None])
    assert np.max(np.abs(g["dh0"] - want)) <= 1e-14 * np.max(np.abs(want))
    assert np.all(g["dz"] == 0.0) and np.all(g["dC"] == 0.0) and np.all(g["dD"] == 0.0)


def test_bwd_empty_sequence():
    p, _, dhl = _problem(80, seqlen=0)
    dy = np.zeros((2, 0, 3))
    g = _grads(p, dy, dhl, False, False)
    assert g["dx"].shape == (2, 0, 3) and g["dB"].shape == (2, 0, 4)
    assert np.all(g["dA"] == 0.0) and np.all(g["dD"] == 0.0)
    assert np.array_equal(g["dh0"], dhl)
