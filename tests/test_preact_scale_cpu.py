"""Pins of the pre-activation rounding term the GPU chain tests add to their
error scales (gpu_harness.preact_scale, SILU1_MAX, SILU2_MAX, GAMMA_PRE).

  * SILU1_MAX and SILU2_MAX bound |silu'| and |silu''| everywhere (the
    derivatives written out from silu(v) = v sigmoid(v), checked on a fine
    grid and in the tails), and 0.5 is silu'' at 0;
  * preact_scale is kappa (|b| + sum_k |w x|) with the conv context in front
    of each sequence, written out here as a loop over taps;
  * an fp32 evaluation of the pre-activation in several summation orders
    stays within GAMMA_PRE * 2^-24 * (|b| + sum |w x|) of the exact value, on
    inputs drawn so that the sum often cancels.
"""
from __future__ import annotations

import numpy as np

import synth
from tests.gpu_harness import GAMMA_PRE, SILU1_MAX, SILU2_MAX, preact_scale


def _sig(v):
    with np.errstate(over="ignore"):
        return 1.0 / (1.0 + np.exp(-v))


def test_silu_derivative_bounds():
    v = np.concatenate([np.linspace(-60.0, 60.0, 2_400_001), [-1e3, 1e3]])
    s = _sig(v)
    d1 = s * (1.0 + v * (1.0 - s))
    d2 = s * (1.0 - s) * (2.0 + v * (1.0 - 2.0 * s))
    # the derivatives written above, against central differences of silu
    h = 1e-5
    vv = np.linspace(-8.0, 8.0, 1601)
    silu = lambda a: a * _sig(a)  # noqa: E731
    s1 = lambda a: _sig(a) * (1.0 + a * (1.0 - _sig(a)))  # noqa: E731
    sv = _sig(vv)
    assert np.allclose((silu(vv + h) - silu(vv - h)) / (2 * h), s1(vv), atol=1e-8)
    assert np.allclose((s1(vv + h) - s1(vv - h)) / (2 * h), sv * (1.0 - sv) * (2.0 + vv * (1.0 - 2.0 * sv)),
                       atol=1e-7)
    assert np.max(np.abs(d1)) <= SILU1_MAX
    assert np.max(np.abs(d2)) <= SILU2_MAX
    assert np.isclose(np.max(np.abs(d2)), SILU2_MAX, rtol=1e-12)  # tight: silu''(0) = 2 sigmoid'(0)
    # silu' crosses zero near -1.2785, where the conv backward's factor cancels
    band = (v > -2) & (v < -1)
    assert abs(v[band][np.argmin(np.abs(d1[band]))] + 1.2785) < 1e-3


def _conv_mag_loop(x, w, b, cu, xc0):
    T, D = x.shape
    W = w.shape[1]
    out = np.zeros((T, D))
    for s in range(len(cu) - 1):
        for t in range(int(cu[s]), int(cu[s + 1])):
            for d in range(D):
                acc = abs(b[d]) if b is not None else 0.0
                for k in range(W):
                    i = t - k
                    if i >= cu[s]:
                        xi = x[i, d]
                    elif xc0 is not None:
                        xi = xc0[s, i - (int(cu[s]) - (W - 1)), d]
                    else:
                        xi = 0.0
                    acc += abs(w[d, W - 1 - k] * xi)
                out[t, d] = acc
    return out


def test_preact_scale_is_the_magnitude_sum(orc):
    rng = np.random.default_rng(11)
    lengths = [3, 1, 0, 6]
    cu = synth.cu_seqlens_of(lengths)
    T, D, W = int(cu[-1]), 5, 4
    x, w, b = rng.standard_normal((T, D)), rng.standard_normal((D, W)), rng.standard_normal(D)
    xc0 = rng.standard_normal((len(lengths), W - 1, D))
    tol = 1e-4
    kappa = GAMMA_PRE * 2.0 ** -24 / tol
    for bb, cc in ((b, xc0), (None, xc0), (b, None)):
        got = preact_scale(orc, x, w, bb, cu, cc, tol)
        assert np.allclose(got, kappa * _conv_mag_loop(x, w, bb, cu, cc), rtol=1e-14, atol=0)


def test_fp32_preactivation_within_gamma(orc):
    """The bound the term rests on, for every order of a width-4 sum plus bias
    evaluated in fp32 (plain products and adds, or each product added as one
    fused step emulated in fp64 then rounded)."""
    rng = np.random.default_rng(12)
    T, D, W = 4096, 64, 4
    cu = synth.cu_seqlens_of([T])
    x = rng.standard_normal((T, D)).astype(np.float32).astype(np.float64)
    w = rng.uniform(-1, 1, (D, W)).astype(np.float32).astype(np.float64)
    b = rng.standard_normal(D).astype(np.float32).astype(np.float64)
    # make about one channel in eight cancel: the bias undoes the taps
    v_exact, _, _ = orc.conv_fwd_state(x, w, None, cu, None, silu=False, threads=4)
    cancel = rng.random(D) < 0.125
    b[cancel] = (-v_exact[T // 2, cancel]).astype(np.float32)
    v, _, _ = orc.conv_fwd_state(x, w, b, cu, None, silu=False, threads=4)
    vs = preact_scale(orc, x, w, b, cu, None, 1.0) / (GAMMA_PRE * 2.0 ** -24)
    f = np.float32
    taps = [(w[:, W - 1 - k][None, :], np.vstack([np.zeros((k, D)), x[:T - k]])) for k in range(W)]
    orders = [list(range(W)), list(reversed(range(W))), [1, 3, 0, 2]]
    worst = 0.0
    for order in orders:
        for fused in (False, True):
            for bias_first in (True, False):
                acc = np.broadcast_to(b.astype(f), (T, D)).copy() if bias_first else np.zeros((T, D), f)
                for k in order:
                    wk, xk = taps[k]
                    if fused:
                        acc = (acc.astype(np.float64) + wk * xk).astype(f)
                    else:
                        acc = (acc + (wk * xk).astype(f)).astype(f)
                if not bias_first:
                    acc = (acc + b.astype(f)).astype(f)
                err = np.abs(acc.astype(np.float64) - v)
                assert np.all(err <= GAMMA_PRE * 2.0 ** -24 * vs), (order, fused, bias_first)
                worst = max(worst, float(np.max(err / np.maximum(vs, 1e-300))))
    # not vacuous: some evaluation is off by more than 2^-24 vs
    assert worst > 2.0 ** -24
