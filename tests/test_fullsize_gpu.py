"""GPU parity at the full workload sizes, through the same library calls the
benchmark times (varlen_pack_indices -> conv1d_pack_fwd ->
selective_scan_pack_fwd -> selective_scan_pack_bwd -> conv1d_pack_bwd).

The oracle cannot redo the whole batch in seconds, so it checks samples it
can compute exactly:
  * every token of a spread of channels (first, last, and ones inside each
    64-channel group boundary region): channels interact only through dB and
    dC, so a channel-subset oracle run gives exact references for u, out,
    dx, du, ddelta, dz and the per-channel sums dA, dD, dconv_w, dconv_b;
  * dB and dC of sampled whole sequences, from the oracle run on those
    sequences alone with every channel (packed == each sequence alone).
Position indices are compared in full, bit for bit.
"""
from __future__ import annotations

import numpy as np
import pytest
import torch

import synth
from tests.gpu_harness import TOL_GRAD, TOL_OUT, Dev, assert_close, npy

pytestmark = pytest.mark.gpu


def sampled_channels(D):
    ch = {0, 1, 31, 32, 63, 64, D // 2 - 1, D // 2, D - 65, D - 64, D - 2, D - 1}
    rng = np.random.default_rng(D)
    ch |= set(int(v) for v in rng.integers(0, D, 8))
    return np.array(sorted(c for c in ch if 0 <= c < D))


def pick_sequences(lengths, k=2):
    """The shortest sequence and one of middling length."""
    order = np.argsort(lengths, kind="stable")
    return sorted({int(order[0]), int(order[len(order) // 2])})[:k]


def test_fullsize_every_element(orc):
    """The benchmark workload (d_inner 4096, 8 x 4096 tokens, bf16) through
    the benchmark's calls, every output and gradient compared with the
    oracle's fp64 chain element by element (the oracle on every host core).
    Per-token tensors are compared relative to their largest value; sums over
    tokens or channels (dA, dB, dC, dDskip, dconv_w, dconv_b) against the
    sum of the magnitudes of their terms (the oracle's error-scale mode)."""
    import os
    from tests.gpu_harness import assert_sum_close
    assert torch.cuda.is_available()
    threads = os.cpu_count() or 1
    print(f"[fullsize] workload 4, every element, oracle on {threads} threads", flush=True)
    inp = synth.make_inputs(4, with_dout=True)
    d = Dev(inp)
    F = d.forward()
    G = d.backward(F)
    torch.cuda.synchronize()
    to, tg = TOL_OUT[inp.dtype], TOL_GRAD[inp.dtype]
    f = synth.f64
    args = (f(inp.x), f(inp.w), f(inp.b), f(inp.delta), f(inp.A), f(inp.B), f(inp.C), f(inp.Dp), f(inp.z),
            inp.cu_seqlens)
    Rf = orc.forward(*args, threads=threads)
    assert np.array_equal(F["pos"].cpu().numpy(), Rf["pos"])
    assert_close(npy(F["u"]), Rf["u"], to, "u")
    assert_close(npy(F["out"]), Rf["out"], to, "out")
    del Rf
    dout = f(inp.dout)
    Rb = orc.backward(*args, dout, threads=threads)
    for k in ("dx", "du", "ddelta", "dz"):
        assert_close(npy(G[k]), Rb[k], tg, k)
    with orc.error_scales():
        Sb = orc.backward(*args, dout, threads=threads)
    for k in ("dA", "dB", "dC", "dD", "dw", "db"):
        assert_sum_close(npy(G[k]), Rb[k], Sb[k], tg, k)
    print(f"[fullsize] every element of {len(Rb)} outputs checked", flush=True)


@pytest.mark.parametrize("workload", [4, 1, 3])
def test_fullsize_sampled(orc, workload):
    assert torch.cuda.is_available()
    print(f"[fullsize] workload {workload} ({synth.NAMES[workload]})", flush=True)
    inp = synth.make_inputs(workload, with_dout=True)
    d = Dev(inp)
    F = d.forward()
    G = d.backward(F)
    torch.cuda.synchronize()
    dt = inp.dtype
    to, tg = TOL_OUT[dt], TOL_GRAD[dt]

    rpos, _ = orc.pack_indices(inp.cu_seqlens, inp.T)
    assert np.array_equal(F["pos"].cpu().numpy(), rpos)

    # every token of sampled channels
    ch = sampled_channels(inp.D)
    f = synth.f64
    x, w, b = f(inp.x)[:, ch], f(inp.w)[ch], f(inp.b)[ch]
    delta, A, Dp, z, dout = f(inp.delta)[:, ch], f(inp.A)[ch], f(inp.Dp)[ch], f(inp.z)[:, ch], f(inp.dout)[:, ch]
    B, C = f(inp.B), f(inp.C)
    Rf = orc.forward(x, w, b, delta, A, B, C, Dp, z, inp.cu_seqlens, threads=16)
    Rb = orc.backward(x, w, b, delta, A, B, C, Dp, z, inp.cu_seqlens, dout, threads=16)
    cht = torch.from_numpy(ch).cuda()
    assert_close(npy(F["u"][:, cht]), Rf["u"], to, "u")
    assert_close(npy(F["out"][:, cht]), Rf["out"], to, "out")
    for k in ("dx", "du", "ddelta", "dz"):
        assert_close(npy(G[k][:, cht]), Rb[k], tg, k)
    for k in ("dA", "dw"):
        assert_close(npy(G[k][cht]), Rb[k], tg, k)
    for k in ("dD", "db"):
        assert_close(npy(G[k][cht]), Rb[k], tg, k)

    # dB, dC of sampled sequences, all channels
    for s in pick_sequences(inp.lengths):
        lo, hi = int(inp.cu_seqlens[s]), int(inp.cu_seqlens[s + 1])
        one = np.array([0, hi - lo], dtype=np.int32)
        sl = slice(lo, hi)
        R = orc.backward(f(inp.x)[sl], f(inp.w), f(inp.b), f(inp.delta)[sl], f(inp.A), f(inp.B)[sl], f(inp.C)[sl],
                         f(inp.Dp), f(inp.z)[sl], one, f(inp.dout)[sl], threads=16)
        assert_close(npy(G["dB"][lo:hi]), R["dB"], tg, f"dB seq {s} (len {hi - lo})")
        assert_close(npy(G["dC"][lo:hi]), R["dC"], tg, f"dC seq {s} (len {hi - lo})")


def test_fullsize_carried_states(orc):
    """The benchmark pack (workload 4) with every sequence carrying an SSM state
    and a conv context in and out, forward and backward, through the block
    chain: every token of sampled channels against the oracle's
    state-carrying pipeline, and the states and their gradients of those
    channels for every sequence."""
    import selective_state_space_varlen_amd as ssp
    print("[fullsize] workload 4 with carried states", flush=True)
    inp = synth.make_inputs(4, with_dout=True)
    nseq, D, N, W = inp.nseq, inp.D, inp.N, inp.W
    rng = np.random.default_rng(77)
    h0 = (rng.standard_normal((nseq, D, N)) * 0.5).astype(np.float32)
    dhT = rng.standard_normal((nseq, D, N)).astype(np.float32)
    ci = synth.to_dtype(rng.standard_normal((nseq, W - 1, D)), inp.dtype)
    dcf = synth.to_dtype(rng.standard_normal((nseq, W - 1, D)), inp.dtype)
    d = Dev(inp)
    dev = lambda a: torch.from_numpy(a).cuda() if isinstance(a, np.ndarray) else a.cuda()
    F = ssp.forward(d.x, d.w, d.b, d.delta, d.A, d.B, d.C, d.Dp, d.z, d.cu, pos=d.pos,
                    initial_states={"ssm": dev(h0), "conv": dev(ci)}, final_states=True)
    G = ssp.backward(d.x, d.w, d.b, d.delta, d.A, d.B, d.C, d.Dp, d.z, F, d.dout,
                     dfinal_states={"ssm": dev(dhT), "conv": dev(dcf)})
    torch.cuda.synchronize()
    to, tg = TOL_OUT[inp.dtype], TOL_GRAD[inp.dtype]

    ch = sampled_channels(D)
    f = synth.f64
    cu = inp.cu_seqlens
    x, w, b = f(inp.x)[:, ch], f(inp.w)[ch], f(inp.b)[ch]
    delta, A, Dp, z, dout = f(inp.delta)[:, ch], f(inp.A)[ch], f(inp.Dp)[ch], f(inp.z)[:, ch], f(inp.dout)[:, ch]
    B, C = f(inp.B), f(inp.C)
    ci_s, dcf_s = f(ci)[:, :, ch], f(dcf)[:, :, ch]
    h0_s, dhT_s = h0[:, ch].astype(np.float64), dhT[:, ch].astype(np.float64)
    _, u, cf = orc.conv_fwd_state(x, w, b, cu, ci_s, threads=16)
    _, out, hT = orc.scan_fwd_state(u, delta, A, B, C, Dp, z, cu, h0=h0_s, threads=16)
    Rg = orc.scan_bwd_state(u, delta, A, B, C, Dp, z, cu, dout, h0=h0_s, dhT=dhT_s, threads=16)
    dx, dw, db, dci = orc.conv_bwd_state(x, w, b, cu, Rg["du"], ci_s, dcf_s, threads=16)
    cht = torch.from_numpy(ch).cuda()
    assert_close(npy(F["u"][:, cht]), u, to, "u")
    assert_close(npy(F["out"][:, cht]), out, to, "out")
    assert_close(npy(F["final_states"]["ssm"][:, cht]), hT, to, "final ssm state")
    assert np.array_equal(npy(F["final_states"]["conv"][:, :, cht]), cf), "final conv context"
    for k in ("du", "ddelta", "dz"):
        assert_close(npy(G[k][:, cht]), Rg[k], tg, k)
    assert_close(npy(G["dx"][:, cht]), dx, tg, "dx")
    assert_close(npy(G["dA"][cht]), Rg["dA"], tg, "dA")
    assert_close(npy(G["dD"][cht]), Rg["dD"], tg, "dD")
    assert_close(npy(G["dw"][cht]), dw, tg, "dw")
    assert_close(npy(G["db"][cht]), db, tg, "db")
    assert_close(npy(G["dinitial_states"]["ssm"][:, cht]), Rg["dh0"], tg, "dinitial ssm state")
    assert_close(npy(G["dinitial_states"]["conv"][:, :, cht]), dci, tg, "dinitial conv context")


def test_fullsize_step_map_gate_floor(orc):
    """The benchmark pack (workload 4) through the scan with the step map
    softplus(delta + bias) and the gate floor computed inside it, the form the
    benchmark's step-map layout times: every token of sampled channels, the
    per-channel sums (dA, dD, d bias) of those channels, and dB/dC of sampled
    whole sequences."""
    import selective_state_space_varlen_amd as ssp
    print("[fullsize] workload 4 with step map and gate floor", flush=True)
    inp = synth.make_inputs(4, with_dout=True, with_u=True)
    D = inp.D
    rng = np.random.default_rng(78)
    bias = (rng.standard_normal(D) * 0.1).astype(np.float32)
    floor = 0.05
    d = Dev(inp)
    bias_d = torch.from_numpy(bias).cuda()
    ext = dict(delta_bias=bias_d, delta_softplus=True, gate_floor=floor)
    ws = torch.empty(ssp.selective_scan_pack_workspace_bytes(inp.T, D, inp.N), dtype=torch.uint8, device="cuda")
    out, _ = ssp.selective_scan_pack_fwd(d.u, d.delta, d.A, d.B, d.C, d.Dp, d.z, d.pos, workspace=ws, **ext)
    G = ssp.selective_scan_pack_bwd(d.u, d.delta, d.A, d.B, d.C, d.Dp, d.z, d.pos, d.dout, ws, **ext)
    torch.cuda.synchronize()
    to, tg = TOL_OUT[inp.dtype], TOL_GRAD[inp.dtype]

    rpos, _ = orc.pack_indices(inp.cu_seqlens, inp.T)
    ch = sampled_channels(D)
    f = synth.f64
    oext = dict(delta_softplus=True, gate_floor=floor)
    sub = lambda a: f(a)[:, ch]
    _, ref = orc.scan_fwd(sub(inp.u), sub(inp.delta), f(inp.A)[ch], f(inp.B), f(inp.C), f(inp.Dp)[ch], sub(inp.z),
                          rpos, threads=16, delta_bias=bias[ch].astype(np.float64), **oext)
    R = orc.scan_bwd(sub(inp.u), sub(inp.delta), f(inp.A)[ch], f(inp.B), f(inp.C), f(inp.Dp)[ch], sub(inp.z), rpos,
                     sub(inp.dout), threads=16, delta_bias=bias[ch].astype(np.float64), **oext)
    cht = torch.from_numpy(ch).cuda()
    assert_close(npy(out[:, cht]), ref, to, "out")
    for k in ("du", "ddelta", "dz"):
        assert_close(npy(G[k][:, cht]), R[k], tg, k)
    for k in ("dA", "dD", "ddelta_bias"):
        assert_close(npy(G[k][cht]), R[k], tg, k)

    for s in pick_sequences(inp.lengths):
        lo, hi = int(inp.cu_seqlens[s]), int(inp.cu_seqlens[s + 1])
        sl = slice(lo, hi)
        pos = np.arange(hi - lo, dtype=np.int32)
        Rs = orc.scan_bwd(f(inp.u)[sl], f(inp.delta)[sl], f(inp.A), f(inp.B)[sl], f(inp.C)[sl], f(inp.Dp),
                          f(inp.z)[sl], pos, f(inp.dout)[sl], threads=16, delta_bias=bias.astype(np.float64), **oext)
        assert_close(npy(G["dB"][lo:hi]), Rs["dB"], tg, f"dB seq {s} (len {hi - lo})")
        assert_close(npy(G["dC"][lo:hi]), Rs["dC"], tg, f"dC seq {s} (len {hi - lo})")
