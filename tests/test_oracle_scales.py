"""Pins of the oracle's error-scale mode (Oracle.error_scales), which the GPU
tests use to bound sums that cancel.

In that mode every backward output is the sum of the magnitudes of its
terms. Three properties fix it without trusting its own code:
  * with every term non-negative (non-negative inputs, A < 0, z >= 0, conv
    pre-activations >= 0) the scales equal the plain outputs bit for bit;
  * for signed inputs each scale bounds its output (triangle inequality),
    strictly somewhere;
  * the scales of the sums with a closed form over the inputs (dDskip and
    the conv bias gradient) equal that form written out in numpy.
"""
from __future__ import annotations

import numpy as np
import pytest

import synth


def _scan_inputs(rng, T, D, N, nonneg):
    f = (lambda a: np.abs(a)) if nonneg else (lambda a: a)
    u = f(rng.standard_normal((T, D)))
    delta = rng.uniform(0.01, 0.2, (T, D))
    A = -rng.uniform(0.5, 3.0, (D, N))
    B, C = f(rng.standard_normal((T, N))), f(rng.standard_normal((T, N)))
    Dp = f(rng.standard_normal(D))
    z = np.abs(rng.standard_normal((T, D))) if nonneg else rng.standard_normal((T, D))
    dout = f(rng.standard_normal((T, D)))
    return u, delta, A, B, C, Dp, z, dout


LENGTHS = [5, 1, 17, 9]


def _scan_both(orc, args, dout, states, rng):
    cu = synth.cu_seqlens_of(LENGTHS)
    T = int(cu[-1])
    u, delta, A, B, C, Dp, z = args
    D, N = A.shape
    if states:
        h0 = np.abs(rng.standard_normal((len(LENGTHS), D, N)))
        dhT = np.abs(rng.standard_normal((len(LENGTHS), D, N)))
        plain = orc.scan_bwd_state(u, delta, A, B, C, Dp, z, cu, dout, h0=h0, dhT=dhT, threads=2)
        with orc.error_scales():
            scale = orc.scan_bwd_state(u, delta, A, B, C, Dp, z, cu, dout, h0=h0, dhT=dhT, threads=2)
    else:
        pos, _ = orc.pack_indices(cu, T)
        plain = orc.scan_bwd(u, delta, A, B, C, Dp, z, pos, dout, threads=2)
        with orc.error_scales():
            scale = orc.scan_bwd(u, delta, A, B, C, Dp, z, pos, dout, threads=2)
    return plain, scale


@pytest.mark.parametrize("states", [False, True])
def test_scan_scales_equal_outputs_when_terms_are_nonnegative(orc, states):
    rng = np.random.default_rng(3)
    T = sum(LENGTHS)
    u, delta, A, B, C, Dp, z, dout = _scan_inputs(rng, T, 6, 4, nonneg=True)
    plain, scale = _scan_both(orc, (u, delta, A, B, C, Dp, z), dout, states, rng)
    # ddelta holds A a h terms (A < 0): not all of its terms are non-negative
    for k in ("du", "dA", "dB", "dC", "dD", "dz") + (("dh0",) if states else ()):
        assert np.array_equal(plain[k], scale[k]), k


@pytest.mark.parametrize("states", [False, True])
def test_scan_scales_bound_outputs(orc, states):
    rng = np.random.default_rng(4)
    T = sum(LENGTHS)
    u, delta, A, B, C, Dp, z, dout = _scan_inputs(rng, T, 6, 4, nonneg=False)
    plain, scale = _scan_both(orc, (u, delta, A, B, C, Dp, z), dout, states, rng)
    for k in ("du", "ddelta", "dA", "dB", "dC", "dD", "dz"):
        assert np.all(scale[k] >= np.abs(plain[k]) * (1 - 1e-12)), k
        assert np.any(scale[k] > np.abs(plain[k]) * (1 + 1e-9)), k


def test_scan_dskip_scale_closed_form(orc):
    """dDskip[d] = sum_t g u with g = dout (z sigmoid(z) + floor): its scale is
    sum_t |g u|."""
    rng = np.random.default_rng(5)
    T = sum(LENGTHS)
    u, delta, A, B, C, Dp, z, dout = _scan_inputs(rng, T, 5, 2, nonneg=False)
    cu = synth.cu_seqlens_of(LENGTHS)
    pos, _ = orc.pack_indices(cu, T)
    floor = 0.05
    with orc.error_scales():
        s = orc.scan_bwd(u, delta, A, B, C, Dp, z, pos, dout, threads=1, gate_floor=floor)
    sig = 1.0 / (1.0 + np.exp(-z))
    g = np.abs(dout) * (np.abs(z * sig) + floor)
    assert np.allclose(s["dD"], np.sum(np.abs(g * u), axis=0), rtol=1e-13, atol=0)


def test_conv_scales(orc):
    rng = np.random.default_rng(6)
    cu = synth.cu_seqlens_of(LENGTHS)
    T, D, W = int(cu[-1]), 5, 4
    pos, _ = orc.pack_indices(cu, T)
    # non-negative inputs and weights: pre-activations >= 0, SiLU' > 0
    x, w, b = np.abs(rng.standard_normal((T, D))), np.abs(rng.standard_normal((D, W))), np.abs(rng.standard_normal(D))
    du = np.abs(rng.standard_normal((T, D)))
    plain = orc.conv_bwd(x, w, b, pos, du, True, threads=2)
    with orc.error_scales():
        scale = orc.conv_bwd(x, w, b, pos, du, True, threads=2)
    for a, s in zip(plain, scale):
        assert np.array_equal(a, s)
    # signed: bounds, and the bias gradient's scale in closed form
    x, w, b = rng.standard_normal((T, D)), rng.standard_normal((D, W)), rng.standard_normal(D)
    du = rng.standard_normal((T, D))
    plain = orc.conv_bwd(x, w, b, pos, du, True, threads=2)
    with orc.error_scales():
        scale = orc.conv_bwd(x, w, b, pos, du, True, threads=2)
    for a, s in zip(plain, scale):
        assert np.all(s >= np.abs(a) * (1 - 1e-12))
    v, _ = orc.conv_fwd(x, w, b, pos, True, threads=1)
    sg = 1.0 / (1.0 + np.exp(-v))
    gv = du * sg * (1.0 + v * (1.0 - sg))
    assert np.allclose(scale[2], np.sum(np.abs(gv), axis=0), rtol=1e-13, atol=0)
    # with contexts, zero contexts give the reset-only scales
    z0 = np.zeros((len(LENGTHS), W - 1, D))
    with orc.error_scales():
        st = orc.conv_bwd_state(x, w, b, cu, du, z0, z0, True, threads=2)
    for a, s in zip(scale, st[:3]):
        assert np.allclose(a, s, rtol=1e-13, atol=1e-300)


def test_error_scales_switch_back_off(orc):
    rng = np.random.default_rng(7)
    T = sum(LENGTHS)
    u, delta, A, B, C, Dp, z, dout = _scan_inputs(rng, T, 3, 2, nonneg=False)
    cu = synth.cu_seqlens_of(LENGTHS)
    pos, _ = orc.pack_indices(cu, T)
    a = orc.scan_bwd(u, delta, A, B, C, Dp, z, pos, dout, threads=1)
    with orc.error_scales():
        orc.scan_bwd(u, delta, A, B, C, Dp, z, pos, dout, threads=1)
    b = orc.scan_bwd(u, delta, A, B, C, Dp, z, pos, dout, threads=1)
    for k in a:
        if a[k] is not None:
            assert np.array_equal(a[k], b[k]), k
