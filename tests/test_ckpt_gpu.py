"""GPU parity of the checkpoint-interval entry points (selective_scan_pack_fwd_ck
and _bwd_ck).

The interval only decides which states the forward keeps and how the backward
gets the others back (read, replayed from sparser ones, or recomputed from the
inputs). The replay repeats the forward's arithmetic operation for operation
within a forward chunk (64 tokens or more), so intervals up to 64 and the
recomputing interval 0 must give the same bits as the forward that keeps
every 4th state (which the backward reads every 8th of). Longer intervals replay across chunk boundaries, where the
forward restarted from its carry pass's state: the same states up to
rounding, so those results agree to the gradient tolerance. Intervals 0, 64
and 2048 are also checked against the fp64 oracle.
Scratch and kept-state buffers are filled with NaN before each call, so a
read of anything a pass did not write shows up in the results.
"""
from __future__ import annotations

import numpy as np
import pytest
import torch

import synth
from tests.gpu_harness import TOL_GRAD, TOL_OUT, Dev, assert_close, nan_buffer, npy, to_dev

pytestmark = pytest.mark.gpu

BITWISE = (0, 4, 8, 16, 64)
LONG = (256, 2048)


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    assert torch.cuda.is_available(), "GPU tests need an MI355X"
    import selective_state_space_varlen_amd as ssp
    ssp.load()


def ssp():
    import selective_state_space_varlen_amd as m
    return m


CASES = {
    # several forward chunks (64 tokens here) and backward chunks, heads on and
    # off chunk and interval boundaries, single-token sequences, a ragged tail
    "bf16-gate-skip": dict(wl=2, lengths=[700, 1, 400, 1203, 3, 900], D=128),
    "fp32-n8-no-gate": dict(wl=2, lengths=[257, 1, 1029, 64, 511], D=96, N=8, dtype=torch.float32, gate=False),
    "states-step-map": dict(wl=2, lengths=[1000, 5, 1500, 0, 333], D=64, states=True, opts=(True, 0.05)),
    "long-sequence-n4": dict(wl=3, lengths=[6001], D=64, N=4),
}


def _case(name):
    spec = dict(CASES[name])
    gate = spec.pop("gate", True)
    states = spec.pop("states", False)
    opts = spec.pop("opts", None)
    inp = synth.make_inputs(spec.pop("wl"), with_u=True, with_dout=True, **spec)
    rng = np.random.default_rng(23)
    kw, okw = {}, {}
    if opts is not None:
        bias = (rng.standard_normal(inp.D) * 0.5).astype(np.float32)
        raw = np.log(np.expm1(synth.f64(inp.delta))) - bias[None, :]
        inp.delta = synth.to_dtype(raw, inp.dtype)
        kw = dict(delta_bias=to_dev(torch.from_numpy(bias)), delta_softplus=True, gate_floor=opts[1])
        okw = dict(delta_bias=bias.astype(np.float64), delta_softplus=True, gate_floor=opts[1])
    st, ost = {}, None
    if states:
        h0 = rng.standard_normal((inp.nseq, inp.D, inp.N)).astype(np.float32)
        dhT = rng.standard_normal((inp.nseq, inp.D, inp.N)).astype(np.float32)
        st = dict(initial_state=to_dev(torch.from_numpy(h0)), dfinal_state=to_dev(torch.from_numpy(dhT)))
        ost = (h0, dhT)
    return inp, gate, kw, okw, st, ost


def _run(d, inp, gate, kw, st, ci):
    T, D, N = inp.T, inp.D, inp.N
    b = ssp()
    z = d.z if gate else None
    saved = nan_buffer(b.selective_scan_pack_saved_bytes(T, D, N, ci)) if ci else None
    fscr = nan_buffer(b.selective_scan_pack_fwd_scratch_bytes(T, D, N))
    fst = {}
    if st:
        fst = dict(cu_seqlens=d.cu, initial_state=st["initial_state"], final_state=True)
    out, saved, hT = b.selective_scan_pack_fwd_ck(d.u, d.delta, d.A, d.B, d.C, d.Dp, z, d.pos, ci, saved=saved,
                                                  scratch=fscr, **kw, **fst)
    bscr = nan_buffer(b.selective_scan_pack_bwd_scratch_bytes(T, D, N, ci))
    bst = {}
    if st:
        bst = dict(cu_seqlens=d.cu, initial_state=st["initial_state"], dfinal_state=st["dfinal_state"],
                   dinitial_state=True)
    g = b.selective_scan_pack_bwd_ck(d.u, d.delta, d.A, d.B, d.C, d.Dp, z, d.pos, d.dout, ci, saved, scratch=bscr,
                                     **kw, **bst)
    torch.cuda.synchronize()
    return out, hT, g


@pytest.mark.parametrize("name", list(CASES))
def test_every_interval_gives_the_same_bits(name):
    inp, gate, kw, _, st, _ = _case(name)
    d = Dev(inp)
    ref_out, ref_hT, ref_g = _run(d, inp, gate, kw, st, 4)
    # the single-workspace entry points are the interval-8 case
    lw = {}
    if st:
        lw = dict(cu_seqlens=d.cu, initial_state=st["initial_state"], final_state=True)
    z = d.z if gate else None
    res = ssp().selective_scan_pack_fwd(d.u, d.delta, d.A, d.B, d.C, d.Dp, z, d.pos, **kw, **lw)
    assert torch.equal(res[0], ref_out)
    for ci in BITWISE:
        out, hT, g = _run(d, inp, gate, kw, st, ci)
        assert torch.equal(out, ref_out), ci
        if st:
            assert torch.equal(hT, ref_hT), ci
        for k, v in ref_g.items():
            if v is not None:
                assert torch.equal(g[k], v), (ci, k)
    tg = TOL_GRAD[inp.dtype]
    for ci in LONG:
        out, hT, g = _run(d, inp, gate, kw, st, ci)
        assert torch.equal(out, ref_out), ci  # the output pass does not depend on the interval
        for k, v in ref_g.items():
            if v is not None:
                assert_close(npy(g[k]), npy(v), tg, f"{k} ci={ci}")


@pytest.mark.parametrize("name", list(CASES))
def test_sparse_and_recomputed_states_match_oracle(orc, name):
    inp, gate, kw, okw, st, ost = _case(name)
    d = Dev(inp)
    args = (synth.f64(inp.u), synth.f64(inp.delta), synth.f64(inp.A), synth.f64(inp.B), synth.f64(inp.C),
            synth.f64(inp.Dp), synth.f64(inp.z) if gate else None)
    if st:
        h0, dhT = ost
        _, rout, rhT = orc.scan_fwd_state(*args, inp.cu_seqlens, h0=h0, threads=8, **okw)
        rg = orc.scan_bwd_state(*args, inp.cu_seqlens, synth.f64(inp.dout), h0=h0, dhT=dhT, threads=8, **okw)
    else:
        pos, _ = orc.pack_indices(inp.cu_seqlens, inp.T)
        _, rout = orc.scan_fwd(*args, pos, threads=8, **okw)
        rg = orc.scan_bwd(*args, pos, synth.f64(inp.dout), threads=8, **okw)
    to, tg = TOL_OUT[inp.dtype], TOL_GRAD[inp.dtype]
    for ci in (0, 64, 2048):
        out, hT, g = _run(d, inp, gate, kw, st, ci)
        assert_close(npy(out), rout, to, f"out ci={ci}")
        for k in ("du", "ddelta", "dA", "dB", "dC", "dD"):
            assert_close(npy(g[k]), rg[k], tg, f"{k} ci={ci}")
        if gate:
            assert_close(npy(g["dz"]), rg["dz"], tg, f"dz ci={ci}")
        if kw:
            assert_close(npy(g["ddelta_bias"]), rg["ddelta_bias"], tg, f"ddelta_bias ci={ci}")
        if st:
            assert_close(npy(hT), rhT, to, f"final_state ci={ci}")
            assert_close(npy(g["dinitial_state"]), rg["dh0"], tg, f"dinitial_state ci={ci}")


def test_forward_only_keeps_nothing():
    """Interval 0: no kept-state buffer, a scratch far below the dense states,
    and the same output as a forward that keeps states."""
    inp, gate, kw, _, st, _ = _case("bf16-gate-skip")
    d = Dev(inp)
    T, D, N = inp.T, inp.D, inp.N
    b = ssp()
    assert b.selective_scan_pack_saved_bytes(T, D, N, 0) == 0
    scr = nan_buffer(b.selective_scan_pack_fwd_scratch_bytes(T, D, N))
    out0, saved, _ = b.selective_scan_pack_fwd_ck(d.u, d.delta, d.A, d.B, d.C, d.Dp, d.z, d.pos, 0, scratch=scr)
    assert saved is None
    out4, _, _ = b.selective_scan_pack_fwd_ck(d.u, d.delta, d.A, d.B, d.C, d.Dp, d.z, d.pos, 4)
    torch.cuda.synchronize()
    assert torch.equal(out0, out4)
    assert b.selective_scan_pack_fwd_scratch_bytes(T, D, N) < b.selective_scan_pack_saved_bytes(T, D, N, 4)
