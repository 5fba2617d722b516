"""Pins for the oracle's scan with a scalar decay per head (oracle.ssd), CPU only.

  * It is the Mamba-1 selective scan (pinned on its own in
    test_oracle_pins.py) with the decay broadcast over the states of a head
    and the step shared by the head's channels, for every group of heads.
  * It is y = M x with the lower-triangular masked matrix of "Deriving and
    implementing Mamba from scratch", section 6.1, built entry by entry.
  * A block decomposition written here in numpy (diagonal blocks as masked
    matrix products, chunk states carried between blocks: the block-wise form
    of "SSMs for long-document QA", section 2.3) gives the same result for
    every block length.
"""
import numpy as np
import pytest

import oracle


def _problem(seed, batch=2, L=13, nheads=4, headdim=3, ngroups=2, N=5, softplus=False, h0=True):
    r = np.random.default_rng(seed)
    p = {
        "x": r.normal(size=(batch, L, nheads, headdim)),
        "A": -r.uniform(0.5, 4.0, size=nheads),
        "B": r.normal(size=(batch, L, ngroups, N)),
        "C": r.normal(size=(batch, L, ngroups, N)),
        "D": r.normal(size=nheads),
        "z": r.normal(size=(batch, L, nheads, headdim)),
        "h0": r.normal(size=(batch, nheads, headdim, N)) if h0 else None,
    }
    if softplus:
        p["dt"] = r.normal(-1.0, 1.0, size=(batch, L, nheads))
        p["dt_bias"] = r.uniform(-2.0, 0.0, size=nheads)
    else:
        p["dt"] = r.uniform(0.01, 0.4, size=(batch, L, nheads))
        p["dt_bias"] = None
    return p


def _ssd(p, sp=False):
    return oracle.ssd(p["x"], p["dt"], p["A"], p["B"], p["C"], p["D"], p["z"], p["h0"], p["dt_bias"],
                      delta_softplus=sp)


@pytest.mark.parametrize("sp", [False, True])
@pytest.mark.parametrize("ngroups", [1, 2])
def test_ssd_is_mamba1_scan_with_broadcast_decay(sp, ngroups):
    p = _problem(1 + ngroups + 2 * sp, ngroups=ngroups, softplus=sp)
    y, hl = _ssd(p, sp)
    batch, L, H, P = p["x"].shape
    N = p["B"].shape[3]
    per = H // ngroups
    for g in range(ngroups):
        hs = list(range(g * per, (g + 1) * per))
        x1 = p["x"][:, :, hs].reshape(batch, L, per * P)
        z1 = p["z"][:, :, hs].reshape(batch, L, per * P)
        d1 = np.repeat(p["dt"][:, :, hs], P, axis=2)
        A1 = np.repeat(p["A"][hs], P)[:, None] * np.ones((1, N))
        D1 = np.repeat(p["D"][hs], P)
        h01 = p["h0"][:, hs].reshape(batch, per * P, N)
        bias1 = np.repeat(p["dt_bias"][hs], P) if sp else None
        y1, hl1 = oracle.scan(x1, d1, A1, p["B"][:, :, g], p["C"][:, :, g], D1, z1, h01, bias1, delta_softplus=sp)
        assert np.max(np.abs(y[:, :, hs].reshape(batch, L, -1) - y1)) <= 1e-13 * np.max(np.abs(y1))
        assert np.max(np.abs(hl[:, hs].reshape(batch, per * P, N) - hl1)) <= 1e-13 * np.max(np.abs(hl1))


def test_ssd_is_masked_matrix_times_input():
    """Derivation page section 6.1: y_k = sum_{i<=k} c_k (prod_{j=i+1..k} a_j) b_i x_i,
    with b_i = dt_i B_i here, plus the decayed initial state and the skip term."""
    p = _problem(7, batch=1, L=9, nheads=2, headdim=2, ngroups=1, N=3)
    y, _ = _ssd(p)
    x, dt, A, B, C, D, z, h0 = (p[k] for k in ("x", "dt", "A", "B", "C", "D", "z", "h0"))
    L = x.shape[1]
    for h in range(2):
        a = np.exp(dt[0, :, h] * A[h])
        M = np.zeros((L, L))
        for k in range(L):
            for i in range(k + 1):
                M[k, i] = (C[0, k, 0] @ B[0, i, 0]) * np.prod(a[i + 1:k + 1]) * dt[0, i, h]
        for pp in range(2):
            init = np.array([C[0, k, 0] @ (np.prod(a[:k + 1]) * h0[0, h, pp]) for k in range(L)])
            ypre = M @ x[0, :, h, pp] + init + D[h] * x[0, :, h, pp]
            want = ypre * z[0, :, h, pp] / (1 + np.exp(-z[0, :, h, pp]))
            assert np.max(np.abs(y[0, :, h, pp] - want)) <= 1e-12 * np.max(np.abs(want))


def test_ssd_rank_one_when_one_state():
    """With one state the masked matrix is rank one inside its lower triangle:
    M[k,i] = (c_k * prod_{j<=k} a_j) * (b_i / prod_{j<=i} a_j)."""
    p = _problem(8, batch=1, L=7, nheads=1, headdim=1, ngroups=1, N=1, h0=False)
    p["D"] = None
    p["z"] = None
    y, _ = _ssd(p)
    a = np.exp(p["dt"][0, :, 0] * p["A"][0])
    cum = np.cumprod(a)
    u = p["C"][0, :, 0, 0] * cum
    v = p["B"][0, :, 0, 0] * p["dt"][0, :, 0] / cum
    want = np.tril(np.outer(u, v)) @ p["x"][0, :, 0, 0]
    assert np.max(np.abs(y[0, :, 0, 0] - want)) <= 1e-12 * np.max(np.abs(want))


def _blockwise(p, Q):
    """Block decomposition: for each block of Q steps, the diagonal block is a
    masked matrix product, the off-diagonal part reads the state entering the
    block, and the block's end state is the decayed entry state plus the
    block's own contribution."""
    x, dt, A, B, C, D, z, h0 = (p[k] for k in ("x", "dt", "A", "B", "C", "D", "z", "h0"))
    batch, L, H, P = x.shape
    G, N = B.shape[2], B.shape[3]
    per = H // G
    y = np.zeros_like(x)
    hl = np.zeros((batch, H, P, N))
    for b in range(batch):
        for h in range(H):
            g = h // per
            S = h0[b, h].T.copy() if h0 is not None else np.zeros((N, P))  # [n, p]
            for c0 in range(0, L, Q):
                c1 = min(L, c0 + Q)
                l = np.cumsum(dt[b, c0:c1, h] * A[h])  # log of the decay from the block start
                Cb, Bb, Xb = C[b, c0:c1, g], B[b, c0:c1, g], x[b, c0:c1, h]
                seg = l[:, None] - l[None, :]
                mask = np.tril(np.exp(np.where(np.tril(np.ones_like(seg)) > 0, seg, -np.inf)))
                Wd = (Cb @ Bb.T) * mask * dt[b, c0:c1, h][None, :]
                Yb = Wd @ Xb + np.exp(l)[:, None] * (Cb @ S)
                if D is not None:
                    Yb = Yb + D[h] * Xb
                if z is not None:
                    zb = z[b, c0:c1, h]
                    Yb = Yb * zb / (1 + np.exp(-zb))
                y[b, c0:c1, h] = Yb
                w = np.exp(l[-1] - l) * dt[b, c0:c1, h]
                S = np.exp(l[-1]) * S + Bb.T @ (w[:, None] * Xb)
            hl[b, h] = S.T
    return y, hl


@pytest.mark.parametrize("Q", [1, 4, 5, 13, 64])
def test_ssd_block_decomposition(Q):
    p = _problem(9, batch=2, L=13, nheads=4, headdim=3, ngroups=2, N=5)
    y, hl = _ssd(p)
    yb, hb = _blockwise(p, Q)
    assert np.max(np.abs(yb - y)) <= 1e-11 * np.max(np.abs(y))
    assert np.max(np.abs(hb - hl)) <= 1e-11 * np.max(np.abs(hl))


def test_ssd_empty_sequence_hands_state_over():
    p = _problem(10, L=0)
    y, hl = _ssd(p)
    assert y.shape == (2, 0, 4, 3) and np.array_equal(hl, p["h0"])


def test_ssd_linearity_in_input_and_state():
    p = _problem(11)
    p["z"] = None
    y1, h1 = _ssd(p)
    q = dict(p)
    q["x"] = 2.0 * p["x"]
    q["h0"] = 2.0 * p["h0"]
    y2, h2 = _ssd(q)
    assert np.max(np.abs(y2 - 2 * y1)) <= 1e-12 * np.max(np.abs(y1))
    assert np.max(np.abs(h2 - 2 * h1)) <= 1e-12 * np.max(np.abs(h1))
