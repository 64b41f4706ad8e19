"""A pack past the 32-bit element range: T * D > 2^31 for every (T, D) tensor.

T = 2^20 + 123 tokens at d_inner 2048 (bf16), so any offset computed in 32
bits would wrap in the second half of each tensor. Inputs are drawn on the
device from a seeded generator (the host only ever holds samples). The oracle
checks every token of a few channels (forward, backward and the per-channel
sums) and dB/dC of the last sequence, which lies past 2^31 elements;
positions are compared in full.
"""
from __future__ import annotations

import numpy as np
import pytest
import torch

import synth
from tests.gpu_harness import TOL_GRAD, TOL_OUT, assert_close, npy

pytestmark = pytest.mark.gpu

T, D, N, W = (1 << 20) + 123, 2048, 16, 4


def lengths_for(total: int, seed: int) -> list:
    """Uniform lengths in [64, 8192] with the last cut to fill, one
    single-token sequence near the end, and a last sequence of 100 tokens
    (so that it starts past 2^31 elements at d_inner 2048)."""
    rng = np.random.default_rng(seed)
    out, left = [], total - 101
    while left > 0:
        L = int(min(rng.integers(64, 8193), left))
        out.append(L)
        left -= L
    out.insert(len(out) - 2, 1)
    return out + [100]


def test_past_32_bit_offsets(orc):
    import selective_state_space_varlen_amd as ssp
    assert T * D > 2**31
    lengths = lengths_for(T, 41)
    cu_np = synth.cu_seqlens_of(lengths)
    print(f"[large] T={T} D={D} N={N} bf16, {len(lengths)} sequences", flush=True)
    dev = torch.device("cuda:0")
    g = torch.Generator(device=dev).manual_seed(41)
    bf = torch.bfloat16
    rn = lambda *s: torch.randn(*s, generator=g, device=dev, dtype=torch.float32).to(bf)
    x, z, dout = rn(T, D), rn(T, D), rn(T, D)
    B, C = rn(T, N), rn(T, N)
    delta = (torch.rand(T, D, generator=g, device=dev) * 0.099 + 0.001).to(bf)
    A = -torch.arange(1, N + 1, dtype=torch.float32, device=dev).repeat(D, 1).contiguous()
    Dp = torch.ones(D, dtype=torch.float32, device=dev)
    w = (torch.rand(D, W, generator=g, device=dev) - 0.5).contiguous()
    b = torch.zeros(D, dtype=torch.float32, device=dev)
    cu = torch.from_numpy(cu_np).to(dev)

    F = ssp.forward(x, w, b, delta, A, B, C, Dp, z, cu)
    G = ssp.backward(x, w, b, delta, A, B, C, Dp, z, F, dout)
    torch.cuda.synchronize()

    rpos, _ = orc.pack_indices(cu_np, T)
    assert np.array_equal(npy(F["pos"]), rpos)

    ch = np.array([0, 1, 1031, D - 1])
    cht = torch.from_numpy(ch).to(dev)
    f64 = lambda t: npy(t).astype(np.float64)
    xs, zs, ds, gs = (f64(t[:, cht]) for t in (x, z, delta, dout))
    Bh, Ch = f64(B), f64(C)
    to, tg = TOL_OUT[bf], TOL_GRAD[bf]
    _, u = orc.conv_fwd(xs, f64(w[cht]), f64(b[cht]), rpos, threads=16)
    assert_close(f64(F["u"][:, cht]), u, to, "u")
    # the scan and the conv backward on the stored u and du they consumed
    us = f64(F["u"][:, cht])
    _, out = orc.scan_fwd(us, ds, f64(A[cht]), Bh, Ch, f64(Dp[cht]), zs, rpos, threads=16)
    assert_close(f64(F["out"][:, cht]), out, to, "out")
    R = orc.scan_bwd(us, ds, f64(A[cht]), Bh, Ch, f64(Dp[cht]), zs, rpos, gs, threads=16)
    for k in ("du", "ddelta", "dz"):
        assert_close(f64(G[k][:, cht]), R[k], tg, k)
    for k in ("dA", "dD"):
        assert_close(f64(G[k][cht]), R[k], tg, k)
    dx, dw, db = orc.conv_bwd(xs, f64(w[cht]), f64(b[cht]), rpos, f64(G["du"][:, cht]), threads=16)
    assert_close(f64(G["dx"][:, cht]), dx, tg, "dx")
    assert_close(f64(G["dw"][cht]), dw, tg, "dw")
    assert_close(f64(G["db"][cht]), db, tg, "db")

    # dB, dC of the last sequence (all channels), past 2^31 elements
    lo, hi = int(cu_np[-2]), int(cu_np[-1])
    assert lo * D > 2**31
    sl = slice(lo, hi)
    one = np.arange(hi - lo, dtype=np.int32)
    Rs = orc.scan_bwd(f64(F["u"][sl]), f64(delta[sl]), f64(A), f64(B[sl]), f64(C[sl]), f64(Dp), f64(z[sl]), one,
                      f64(dout[sl]), threads=16)
    assert_close(f64(G["dB"][sl]), Rs["dB"], tg, f"dB of the last sequence ({hi - lo} tokens)")
    assert_close(f64(G["dC"][sl]), Rs["dC"], tg, f"dC of the last sequence ({hi - lo} tokens)")
