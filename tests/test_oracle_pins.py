"""Pins of the fp64 oracle against mathematics it does not share code with.

Each test derives the expected result independently of the oracle's loop:
closed forms, a textbook IIR filter (scipy.signal.lfilter), direct
convolution (numpy.convolve), a library ZOH discretisation
(scipy.signal.cont2discrete), brute-force unrolled sums, and invariants.
Sources for the relations used:
  * recurrent and convolutional modes, kernel K_k = C Abar^k Bbar and the
    unrolled outputs y_0, y_1, y_2: "Deriving and implementing Mamba from
    scratch" (dpshk.com/news/3333417) section 2.3; "Mamba from principle to
    code" (lshu.cn/news/79586) section 2.3;
  * diagonal update h^(i) = exp(delta a_i) h^(i) + delta b_i x: derivation page section 3.2;
  * exact ZOH Bbar = (delta A)^-1 (exp(delta A) - I) delta B: derivation page section 2.2;
  * unrolled semiseparable form y_k = c_k sum_{i<=k} (prod_{j=i+1..k} a_j) b_i x_i
    (scalar state; applied here per state n): derivation page section 6.1;
  * segment hand-over of the final state: "SSMs for long-document QA"
    (pwwt.cn/news/5168881) section 3.1;
  * output gate y * SiLU(z): derivation page section 5.2.
"""
import numpy as np
import pytest
from scipy import signal, special

import oracle

RTOL = 1e-12


def _silu(z):
    return z * special.expit(z)


def _rand_case(rng, batch=2, L=20, d=3, N=4, h0=True):
    x = rng.standard_normal((batch, L, d))
    delta = rng.uniform(0.01, 0.5, (batch, L, d))
    A = -rng.uniform(0.3, 3.0, (d, N))
    B = rng.standard_normal((batch, L, N))
    C = rng.standard_normal((batch, L, N))
    D = rng.standard_normal(d)
    z = rng.standard_normal((batch, L, d))
    h = rng.standard_normal((batch, d, N)) if h0 else None
    return x, delta, A, B, C, D, z, h


def _close(a, b, rtol=RTOL, atol=1e-13):
    np.testing.assert_allclose(a, b, rtol=rtol, atol=atol)


def test_constant_input_geometric_series():
    rng = np.random.default_rng(1)
    batch, L, d, N = 2, 60, 3, 5
    dl = rng.uniform(0.05, 0.4, d)
    xv = rng.standard_normal(d)
    zv = rng.standard_normal(d)
    Bv = rng.standard_normal((batch, N))
    Cv = rng.standard_normal((batch, N))
    A = -rng.uniform(0.2, 2.0, (d, N))
    D = rng.standard_normal(d)
    h0 = rng.standard_normal((batch, d, N))
    x = np.broadcast_to(xv, (batch, L, d)).copy()
    delta = np.broadcast_to(dl, (batch, L, d)).copy()
    z = np.broadcast_to(zv, (batch, L, d)).copy()
    B = np.broadcast_to(Bv[:, None, :], (batch, L, N)).copy()
    C = np.broadcast_to(Cv[:, None, :], (batch, L, N)).copy()
    y, hl = oracle.scan(x, delta, A, B, C, D, z, h0)
    t = np.arange(L)[:, None]
    for b in range(batch):
        for c in range(d):
            a = np.exp(dl[c] * A[c])                      # (N,)
            u = dl[c] * Bv[b] * xv[c]                      # (N,)
            p = a[None, :] ** (t + 1)                      # (L, N)
            h = p * h0[b, c] + u * (1 - p) / (1 - a)       # geometric sum
            yy = (h @ Cv[b] + D[c] * xv[c]) * _silu(zv[c])
            _close(y[b, :, c], yy)
            _close(hl[b, c], h[-1])


def test_zero_step_gives_skip_and_initial_state():
    rng = np.random.default_rng(2)
    x, delta, A, B, C, D, z, h0 = _rand_case(rng)
    delta[:] = 0.0
    y, hl = oracle.scan(x, delta, A, B, C, D, z, h0)
    ref = (np.einsum("btn,bdn->btd", C, h0) + D * x) * _silu(z)
    _close(y, ref)
    _close(hl, h0)
    y2, _ = oracle.scan(x, delta, A, B, C, D, z, None)
    _close(y2, D * x * _silu(z))


def test_small_step_matches_first_order():
    # delta -> 0: abar = 1 + delta*A + O(delta^2), so one step from zero gives
    # h = delta*B*x and y = (C.B) delta x + D x to first order.
    rng = np.random.default_rng(3)
    x, _, A, B, C, D, _, _ = _rand_case(rng, L=1, h0=False)
    eps = 1e-7
    delta = np.full(x.shape, eps)
    y, _ = oracle.scan(x, delta, A, B, C, D)
    ref = np.einsum("btn,btn->bt", C, B)[:, :, None] * eps * x + D * x
    np.testing.assert_allclose(y, ref, rtol=1e-6)


def test_zero_input_exponential_decay():
    rng = np.random.default_rng(4)
    x, delta, A, B, C, D, z, h0 = _rand_case(rng, L=40)
    x[:] = 0.0
    y, hl = oracle.scan(x, delta, A, B, C, D, z, h0)
    cum = np.cumsum(delta, axis=1)                              # (b, L, d)
    h = np.exp(cum[..., None] * A[None, None]) * h0[:, None]    # (b, L, d, N)
    ref = np.einsum("btn,btdn->btd", C, h) * _silu(z)
    _close(y, ref)
    _close(hl, h[:, -1])


@pytest.mark.parametrize("with_h0", [False, True])
def test_lti_convolution_duality(with_h0):
    # Time-invariant delta, B, C: y = K * x + D x with K_k = sum_n C_n a_n^k delta B_n,
    # plus the free response sum_n C_n a_n^(t+1) h0_n.
    rng = np.random.default_rng(5 + with_h0)
    batch, L, d, N = 2, 80, 3, 6
    dl = rng.uniform(0.02, 0.3, d)
    A = -rng.uniform(0.1, 2.0, (d, N))
    Bv = rng.standard_normal((batch, N))
    Cv = rng.standard_normal((batch, N))
    D = rng.standard_normal(d)
    x = rng.standard_normal((batch, L, d))
    h0 = rng.standard_normal((batch, d, N)) if with_h0 else None
    delta = np.broadcast_to(dl, (batch, L, d)).copy()
    B = np.broadcast_to(Bv[:, None], (batch, L, N)).copy()
    C = np.broadcast_to(Cv[:, None], (batch, L, N)).copy()
    y, _ = oracle.scan(x, delta, A, B, C, D, None, h0)
    k = np.arange(L)
    for b in range(batch):
        for c in range(d):
            a = np.exp(dl[c] * A[c])
            K = (Cv[b] * dl[c] * Bv[b])[None, :] * a[None, :] ** k[:, None]
            K = K.sum(axis=1)
            ref = np.convolve(x[b, :, c], K)[:L] + D[c] * x[b, :, c]
            # Same response through a first-order IIR filter per state.
            hs = np.stack([signal.lfilter([dl[c] * Bv[b, n]], [1.0, -a[n]], x[b, :, c]) for n in range(N)], 1)
            ref2 = hs @ Cv[b] + D[c] * x[b, :, c]
            if with_h0:
                free = (a[None, :] ** (k[:, None] + 1) * h0[b, c]) @ Cv[b]
                ref = ref + free
                ref2 = ref2 + free
            _close(y[b, :, c], ref, rtol=1e-11, atol=1e-12)
            _close(y[b, :, c], ref2, rtol=1e-11, atol=1e-12)


def test_brute_force_unrolled_sum():
    rng = np.random.default_rng(7)
    x, delta, A, B, C, D, z, h0 = _rand_case(rng, batch=2, L=24, d=3, N=4)
    y, hl = oracle.scan(x, delta, A, B, C, D, z, h0)
    batch, L, d = x.shape
    N = A.shape[1]
    ref = np.zeros_like(y)
    for b in range(batch):
        for c in range(d):
            for k in range(L):
                tot = D[c] * x[b, k, c]
                for n in range(N):
                    s = np.exp(A[c, n] * delta[b, :k + 1, c].sum()) * h0[b, c, n]
                    for i in range(k + 1):
                        decay = np.exp(A[c, n] * delta[b, i + 1:k + 1, c].sum())
                        s += decay * delta[b, i, c] * B[b, i, n] * x[b, i, c]
                    tot += C[b, k, n] * s
                ref[b, k, c] = tot * _silu(z[b, k, c])
    _close(y, ref, rtol=1e-11, atol=1e-12)


def test_split_and_resume_is_exact():
    rng = np.random.default_rng(8)
    x, delta, A, B, C, D, z, h0 = _rand_case(rng, L=37)
    y, hl = oracle.scan(x, delta, A, B, C, D, z, h0)
    for s in (1, 5, 18, 36):
        y1, h1 = oracle.scan(x[:, :s], delta[:, :s], A, B[:, :s], C[:, :s], D, z[:, :s], h0)
        y2, h2 = oracle.scan(x[:, s:], delta[:, s:], A, B[:, s:], C[:, s:], D, z[:, s:], h1)
        assert np.array_equal(np.concatenate([y1, y2], axis=1), y)
        assert np.array_equal(h2, hl)


def test_update_equals_scan_steps():
    rng = np.random.default_rng(9)
    x, delta, A, B, C, D, z, h0 = _rand_case(rng, L=12)
    y, hl = oracle.scan(x, delta, A, B, C, D, z, h0)
    h = h0.copy()
    for t in range(x.shape[1]):
        yt, h = oracle.update(h, x[:, t], delta[:, t], A, B[:, t], C[:, t], D, z[:, t])
        assert np.array_equal(yt, y[:, t])
    assert np.array_equal(h, hl)


def test_linear_in_input_and_initial_state():
    rng = np.random.default_rng(10)
    x1, delta, A, B, C, D, _, h1 = _rand_case(rng)
    x2 = rng.standard_normal(x1.shape)
    h2 = rng.standard_normal(h1.shape)
    al, be = 0.7, -1.9
    y, hl = oracle.scan(al * x1 + be * x2, delta, A, B, C, D, None, al * h1 + be * h2)
    ya, ha = oracle.scan(x1, delta, A, B, C, D, None, h1)
    yb, hb = oracle.scan(x2, delta, A, B, C, D, None, h2)
    _close(y, al * ya + be * yb, rtol=1e-11, atol=1e-12)
    _close(hl, al * ha + be * hb, rtol=1e-11, atol=1e-12)


def test_channel_permutation_and_batch_independence():
    rng = np.random.default_rng(11)
    x, delta, A, B, C, D, z, h0 = _rand_case(rng, batch=3, d=5)
    y, hl = oracle.scan(x, delta, A, B, C, D, z, h0)
    perm = rng.permutation(x.shape[2])
    yp, hp = oracle.scan(x[:, :, perm], delta[:, :, perm], A[perm], B, C, D[perm], z[:, :, perm], h0[:, perm])
    assert np.array_equal(yp, y[:, :, perm])
    assert np.array_equal(hp, hl[:, perm])
    for b in range(x.shape[0]):
        s = slice(b, b + 1)
        yb, hb = oracle.scan(x[s], delta[s], A, B[s], C[s], D, z[s], h0[s])
        assert np.array_equal(yb, y[s])
        assert np.array_equal(hb, hl[s])


def test_zero_B_or_C_leaves_skip_path():
    rng = np.random.default_rng(12)
    x, delta, A, B, C, D, z, _ = _rand_case(rng, h0=False)
    y, hl = oracle.scan(x, delta, A, np.zeros_like(B), C, D, z, None)
    _close(y, D * x * _silu(z))
    assert np.all(hl == 0)
    y, _ = oracle.scan(x, delta, A, B, np.zeros_like(C), D, z, None)
    _close(y, D * x * _silu(z))


def test_optional_arguments_default_to_zero_and_no_gate():
    rng = np.random.default_rng(13)
    x, delta, A, B, C, D, z, h0 = _rand_case(rng)
    y0, _ = oracle.scan(x, delta, A, B, C, np.zeros_like(D), np.full_like(z, 60.0), np.zeros_like(h0))
    y1, _ = oracle.scan(x, delta, A, B, C, None, None, None)
    # silu(60) = 60 * (1 - 8.8e-27): the gate-free output times 60.
    _close(y0, 60.0 * y1, rtol=1e-14, atol=0)


def test_empty_sequence_hands_state_over():
    rng = np.random.default_rng(14)
    x, delta, A, B, C, D, z, h0 = _rand_case(rng, L=0)
    y, hl = oracle.scan(x, delta, A, B, C, D, z, h0)
    assert y.shape == x.shape
    assert np.array_equal(hl, h0)


def test_exact_zoh_matches_library_discretisation():
    rng = np.random.default_rng(15)
    batch, L, d, N = 1, 50, 2, 4
    dl = rng.uniform(0.05, 0.6, d)
    A = -rng.uniform(0.2, 3.0, (d, N))
    Bv = rng.standard_normal((batch, N))
    Cv = rng.standard_normal((batch, N))
    D = rng.standard_normal(d)
    x = rng.standard_normal((batch, L, d))
    delta = np.broadcast_to(dl, (batch, L, d)).copy()
    B = np.broadcast_to(Bv[:, None], (batch, L, N)).copy()
    C = np.broadcast_to(Cv[:, None], (batch, L, N)).copy()
    y, _ = oracle.scan(x, delta, A, B, C, D, exact_zoh=True)
    for c in range(d):
        hs = []
        for n in range(N):
            Ad, Bd, _, _, _ = signal.cont2discrete((np.array([[A[c, n]]]), np.array([[Bv[0, n]]]),
                                                    np.eye(1), np.zeros((1, 1))), dl[c], method="zoh")
            hs.append(signal.lfilter([Bd[0, 0]], [1.0, -Ad[0, 0]], x[0, :, c]))
        ref = np.stack(hs, 1) @ Cv[0] + D[c] * x[0, :, c]
        _close(y[0, :, c], ref, rtol=1e-10, atol=1e-12)


def test_exact_zoh_small_decay_limit_is_first_order_term():
    rng = np.random.default_rng(16)
    x, delta, A, B, C, D, z, h0 = _rand_case(rng)
    A0 = np.zeros_like(A)
    y_exact, h_exact = oracle.scan(x, delta, A0, B, C, D, z, h0, exact_zoh=True)
    y_simple, h_simple = oracle.scan(x, delta, A0, B, C, D, z, h0)
    _close(y_exact, y_simple)
    _close(h_exact, h_simple)


def test_delta_softplus_mode_matches_library_softplus():
    rng = np.random.default_rng(17)
    x, _, A, B, C, D, z, h0 = _rand_case(rng)
    raw = rng.standard_normal(x.shape) * 2.0
    bias = rng.uniform(-7.0, -2.0, x.shape[2])
    raw[0, 0, 0] = 45.0  # large argument: softplus(v) = v to double precision
    y, hl = oracle.scan(x, raw, A, B, C, D, z, h0, bias, delta_softplus=True)
    step = np.logaddexp(0.0, raw + bias)
    y2, h2 = oracle.scan(x, step, A, B, C, D, z, h0)
    _close(y, y2, rtol=1e-13, atol=1e-14)
    _close(hl, h2, rtol=1e-13, atol=1e-14)


def test_bf16_bits_are_widened_exactly():
    bits = np.array([0x3F80, 0xBF80, 0x4049, 0x0001, 0x7F7F, 0x8000], dtype=np.uint16)
    vals = oracle.to_f64(bits)
    np.testing.assert_array_equal(vals, [1.0, -1.0, 3.140625, np.ldexp(1.0, -133), np.ldexp(255.0 / 128.0, 127), -0.0])
