"""Pins of the oracle's causal depthwise conv (+ SiLU) and its carried state.

Independent references:
  * torch.nn.functional.conv1d (CPU, float64) with padding d_conv-1,
    groups=d_inner and the output cut to the first seqlen positions, then
    SiLU -- the Mamba block of "Deriving and implementing Mamba from
    scratch" (dpshk.com/news/3333417) section 5.2, run by a library;
  * scipy.signal.lfilter as a textbook FIR filter (taps reversed), per channel;
  * the impulse response, which must replay the filter taps in time order;
  * state hand-over: a split sequence with the carried state equals one pass,
    and the decode step equals a one-step pass (the cache holds a conv state
    next to the SSM state: "SSM series #12" page, dpshk.com/news/5205047, section 1.3).
"""
import numpy as np
import pytest
import torch
from scipy import signal, special

import oracle


def _case(rng, batch=2, L=30, d=5, K=4):
    x = rng.standard_normal((batch, L, d))
    w = rng.uniform(-0.5, 0.5, (d, K))
    bias = rng.standard_normal(d)
    return x, w, bias


@pytest.mark.parametrize("K", [2, 3, 4])
@pytest.mark.parametrize("silu", [False, True])
def test_matches_torch_conv1d_block(K, silu):
    rng = np.random.default_rng(K)
    x, w, bias = _case(rng, K=K)
    y, _ = oracle.conv1d(x, w, bias, silu=silu)
    xt = torch.from_numpy(x).transpose(1, 2)                      # (b, d, L)
    ref = torch.nn.functional.conv1d(xt, torch.from_numpy(w)[:, None, :], torch.from_numpy(bias),
                                     padding=K - 1, groups=x.shape[2])[:, :, :x.shape[1]]
    if silu:
        ref = torch.nn.functional.silu(ref)
    np.testing.assert_allclose(y, ref.transpose(1, 2).numpy(), rtol=1e-13, atol=1e-14)


def test_matches_fir_filter_with_state():
    rng = np.random.default_rng(7)
    x, w, bias = _case(rng, K=4)
    st = rng.standard_normal((x.shape[0], x.shape[2], 3))
    y, _ = oracle.conv1d(x, w, bias, st, silu=True)
    for b in range(x.shape[0]):
        for d in range(x.shape[2]):
            ext = np.concatenate([st[b, d], x[b, :, d]])
            full = signal.lfilter(w[d, ::-1], [1.0], ext)[3:] + bias[d]
            np.testing.assert_allclose(y[b, :, d], full * special.expit(full), rtol=1e-13, atol=1e-14)


def test_impulse_response_replays_taps():
    K, L = 4, 12
    w = np.array([[0.1, -0.2, 0.3, 0.7]])
    x = np.zeros((1, L, 1))
    x[0, 5, 0] = 1.0
    y, _ = oracle.conv1d(x, w, None, silu=False)
    expect = np.zeros(L)
    expect[5:5 + K] = w[0, ::-1]           # input at t0 meets w[K-1] at t0, w[K-2] at t0+1, ...
    np.testing.assert_array_equal(y[0, :, 0], expect)


def test_state_out_is_last_inputs_and_split_is_exact():
    rng = np.random.default_rng(9)
    x, w, bias = _case(rng, L=23, K=4)
    st = rng.standard_normal((2, 5, 3))
    y, so = oracle.conv1d(x, w, bias, st)
    np.testing.assert_array_equal(so, x[:, -3:, :].transpose(0, 2, 1))
    for s in (1, 2, 3, 11, 22):
        y1, s1 = oracle.conv1d(x[:, :s], w, bias, st)
        y2, s2 = oracle.conv1d(x[:, s:], w, bias, s1)
        assert np.array_equal(np.concatenate([y1, y2], axis=1), y)
        assert np.array_equal(s2, so)
    # a sequence shorter than the state keeps the older state entries
    y1, s1 = oracle.conv1d(x[:, :2], w, bias, st)
    np.testing.assert_array_equal(s1[:, :, 0], st[:, :, 2])
    np.testing.assert_array_equal(s1[:, :, 1:], x[:, :2, :].transpose(0, 2, 1))


def test_decode_steps_equal_one_pass():
    rng = np.random.default_rng(10)
    x, w, bias = _case(rng, L=9, K=4)
    y, so = oracle.conv1d(x, w, bias)
    st = np.zeros((2, 5, 3))
    for t in range(x.shape[1]):
        yt, st = oracle.conv1d_update(st, x[:, t], w, bias)
        assert np.array_equal(yt, y[:, t])
    assert np.array_equal(st, so)
