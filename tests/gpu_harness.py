"""Helpers for the GPU parity tests: run the HIP path through the C ABI and the
fp64 oracle on the same seeded inputs, and compare to the stated tolerances.

Tolerances (max |err| over a tensor, relative to max |reference| of it):
  outputs:   1e-5 for fp32 inputs, 2e-2 for bf16 inputs (fp32 state)
  gradients: 1e-4 for fp32 inputs, 2e-2 for bf16 inputs
The bf16 bound covers the rounding of every bf16 result (2^-9 relative) plus
fp32 accumulation; the oracle reads the same rounded input values.
"""
from __future__ import annotations

import numpy as np
import torch

import synth

TOL_OUT = {torch.float32: 1e-5, torch.bfloat16: 2e-2}
TOL_GRAD = {torch.float32: 1e-4, torch.bfloat16: 2e-2}


def dev():
    return torch.device("cuda:0")


def to_dev(t):
    return None if t is None else t.to(dev()).contiguous()


def npy(t):
    return None if t is None else t.detach().to("cpu").to(torch.float64).numpy()


def nan_buffer(nbytes: int) -> torch.Tensor:
    """A device byte buffer whose every fp32 word is a NaN (0xFFFFFFFF):
    workspaces start this way, so that a read of anything a kernel did not
    write shows up in the results."""
    return torch.full((max(nbytes, 1),), 255, dtype=torch.uint8, device=dev())


def scan_workspace(T: int, D: int, N: int) -> torch.Tensor:
    import selective_state_space_varlen_amd as ssp
    return nan_buffer(ssp.selective_scan_pack_workspace_bytes(T, D, N))


def poison_scan_scratch(ws: torch.Tensor, T: int, D: int, N: int) -> None:
    """NaN-fill the part of a single scan workspace after the forward's kept
    states (the backward's scratch), between forward and backward."""
    import selective_state_space_varlen_amd as ssp
    ws[ssp.selective_scan_pack_saved_bytes(T, D, N, 4):].fill_(255)


def assert_close(got, ref, tol, name):
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    assert got.shape == ref.shape, f"{name}: shape {got.shape} vs {ref.shape}"
    if ref.size == 0:
        return
    scale = float(np.max(np.abs(ref)))
    err = np.abs(got - ref)
    worst = float(np.max(err)) if np.all(np.isfinite(err)) else float("inf")
    assert worst <= tol * max(scale, 1e-30), (
        f"{name}: max|err| {worst:.3e} > {tol:g} * max|ref| {scale:.3e} "
        f"at {np.unravel_index(int(np.nanargmax(np.where(np.isfinite(err), err, np.inf))), err.shape)}")


# Rounding of the conv pre-activation v = b + sum_k w x. The library forms v
# in fp32 whatever the storage dtype, so v is off by at most about
# GAMMA_PRE * 2^-24 * vs, vs = |b| + sum_k |w x| (the forward error bound of
# a short dot product, Higham, Accuracy and Stability of Numerical
# Algorithms, section 3.1). Where v cancels (|v| << vs) that is far above the
# rounding of v's own size: u = silu(v) moves by up to max|silu'| (< 1.1)
# times it, and silu'(v) in the conv backward by up to max|silu''| (= 0.5,
# at v = 0) times it, most visibly near v = -1.2785 where silu' is zero. A
# sum over channels that holds one or a few such terms inherits that error,
# which the magnitudes of its terms do not bound.
GAMMA_PRE = 8
SILU1_MAX = 1.1
SILU2_MAX = 0.5


def preact_scale(orc, x, w, b, cu_seqlens, xc0, tol):
    """kappa * vs per token and channel, kappa = GAMMA_PRE * 2^-24 / tol: the
    pre-activation's rounding bound in units of the tolerance. A chain's
    error scales taken with |u| + SILU1_MAX * this in place of u (in the
    scan) and with SILU2_MAX * this times the scale of du added to silu'(v)
    (in the conv backward) bound, times tol, the rounding of each sum plus
    what the pre-activation's rounding adds to it. vs comes from the
    oracle's conv on the magnitudes of its inputs, without the activation."""
    def ab(a):
        return None if a is None else np.abs(a)
    vs, _, _ = orc.conv_fwd_state(ab(x), ab(w), ab(b), cu_seqlens, ab(xc0), silu=False, threads=8)
    return vs * (GAMMA_PRE * 2.0 ** -24 / tol)


def assert_sum_close(got, ref, scale, tol, name):
    """A sum that may cancel, element by element: |got - ref| <= tol * scale,
    where scale is the sum of the magnitudes of the terms of each element
    (the oracle's error_scales mode), the scale of any evaluation's rounding
    error. A bound relative to max |ref| would instead compare the rounding
    of the terms whenever the sum cancels to near zero."""
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    scale = np.asarray(scale, dtype=np.float64)
    assert got.shape == ref.shape == scale.shape, f"{name}: shapes {got.shape} {ref.shape} {scale.shape}"
    if ref.size == 0:
        return
    assert np.all(scale >= np.abs(ref) * (1 - 1e-9)), f"{name}: scale below |ref| (not an error scale)"
    err = np.abs(got - ref)
    bound = tol * scale
    ok = err <= bound
    if not np.all(ok):
        ratio = np.where(bound > 0, err / np.where(bound > 0, bound, 1.0), np.inf)
        at = np.unravel_index(int(np.nanargmax(ratio)), err.shape)
        raise AssertionError(f"{name}: |err| {err[at]:.3e} > {tol:g} * scale {scale[at]:.3e} at {at} "
                             f"(ref {ref[at]:.3e}, got {got[at]:.3e}); {int((~ok).sum())} elements out")


class Dev:
    """Device copies of an Inputs batch plus cu_seqlens and pos."""

    def __init__(self, inp: synth.Inputs):
        self.inp = inp
        import selective_state_space_varlen_amd as ssp
        self.ssp = ssp
        for k in ("x", "z", "B", "C", "delta", "A", "Dp", "w", "b", "dout", "u"):
            setattr(self, k, to_dev(getattr(inp, k)))
        self.cu = torch.from_numpy(inp.cu_seqlens).to(dev())
        self.pos, self.heads, self.err = ssp.varlen_pack_indices(self.cu, inp.T)

    def forward(self, gate=True, skip=True, bias=True):
        return self.ssp.forward(self.x, self.w, self.b if bias else None, self.delta, self.A, self.B, self.C,
                                self.Dp if skip else None, self.z if gate else None, self.cu, pos=self.pos)

    def backward(self, fwd, gate=True, skip=True, bias=True):
        return self.ssp.backward(self.x, self.w, self.b if bias else None, self.delta, self.A, self.B, self.C,
                                 self.Dp if skip else None, self.z if gate else None, fwd, self.dout)


def oracle_pipeline(orc, inp: synth.Inputs, gate=True, skip=True, bias=True, threads=8, backward=False,
                    channels=None):
    """Oracle forward (and backward) of the whole pipeline, optionally on a
    channel subset (channels never interact except through dB/dC, which a
    subset run does not give in full)."""
    sl = slice(None) if channels is None else channels
    x = synth.f64(inp.x)[:, sl]
    w = synth.f64(inp.w)[sl]
    b = synth.f64(inp.b)[sl] if bias else None
    delta = synth.f64(inp.delta)[:, sl]
    A = synth.f64(inp.A)[sl]
    Dp = synth.f64(inp.Dp)[sl] if skip else None
    z = synth.f64(inp.z)[:, sl] if gate else None
    B = synth.f64(inp.B)
    C = synth.f64(inp.C)
    F = orc.forward(x, w, b, delta, A, B, C, Dp, z, inp.cu_seqlens, threads=threads)
    if not backward:
        return F
    dout = synth.f64(inp.dout)[:, sl]
    G = orc.backward(x, w, b, delta, A, B, C, Dp, z, inp.cu_seqlens, dout, threads=threads)
    F.update(G)
    return F
