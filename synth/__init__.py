"""Seeded synthetic packed variable-length inputs.

This module is shared by the tests, the benchmark and the CPU oracle's callers.
It only draws random numbers and arranges them; it holds none of the method's
arithmetic (no convolution, no scan, no gradient).

Workloads (the recipe is restated in the design notes):

  0  tiny fp32 pack of lengths [4, 2, 3, 7], d_inner 8, d_state 4, width 4
     (the packing example of the Shanghai AI Lab article on packed Mamba-1
     training, section "conv1d_pack 算子", figure (a))
  1  Mamba-130m block shape: d_inner 1536, d_state 16, bf16; 8 packs of 4096
     tokens, lengths log-normal with median 800 clipped to [16, 4096]
  2  Mamba-1.4B block shape: d_inner 4096, d_state 16, bf16; 8 packs of 4096
     tokens, lengths uniform integers in [64, 2048]
  3  long-pack stress: d_inner 4096, bf16; 2 packs of 32768 tokens, lengths
     from buckets {512, 1024, 2048, 4096, 8192}, plus one length-1 sequence
     per pack
  4  workload 2 plus an upstream gradient dout ~ N(0, 1)

Value distributions: x, z, B, C ~ N(0, 1); delta = softplus(r + log(expm1(dt)))
with r ~ N(0, 0.5) per (token, channel) and dt ~ U[1e-3, 0.1] per channel;
A[d, n] = -(n + 1); D = 1; conv weight ~ U(-0.5, 0.5); conv bias 0.
bf16 values are rounded once, round-to-nearest-even, so every consumer reads
identical bits.
"""
from __future__ import annotations

import dataclasses
import math
from typing import Optional

import numpy as np
import torch

BUCKETS = (512, 1024, 2048, 4096, 8192)


@dataclasses.dataclass(frozen=True)
class Workload:
    n_packs: int
    pack_len: int
    D: int
    N: int
    W: int
    dtype: torch.dtype
    lengths: str  # "fixed" | "lognormal" | "uniform" | "buckets"


WORKLOADS = {
    0: Workload(1, 16, 8, 4, 4, torch.float32, "fixed"),
    1: Workload(8, 4096, 1536, 16, 4, torch.bfloat16, "lognormal"),
    2: Workload(8, 4096, 4096, 16, 4, torch.bfloat16, "uniform"),
    3: Workload(2, 32768, 4096, 16, 4, torch.bfloat16, "buckets"),
    4: Workload(8, 4096, 4096, 16, 4, torch.bfloat16, "uniform"),
}

NAMES = {
    0: "tiny-fp32-pack-4-2-3-7",
    1: "mamba130m-block-d1536-n16-8x4096",
    2: "mamba1.4b-block-d4096-n16-8x4096",
    3: "long-pack-d4096-n16-2x32768",
    4: "mamba1.4b-block-d4096-n16-8x4096-bwd",
}


@dataclasses.dataclass
class Inputs:
    """One packed batch. Token-major (T, .) tensors, all on the CPU."""
    workload: int
    lengths: list
    cu_seqlens: np.ndarray  # int32 [nseq + 1]
    T: int
    D: int
    N: int
    W: int
    dtype: torch.dtype
    x: torch.Tensor       # (T, D) conv input
    z: torch.Tensor       # (T, D) gate input
    B: torch.Tensor       # (T, N)
    C: torch.Tensor       # (T, N)
    delta: torch.Tensor   # (T, D), already positive (softplus applied here)
    A: torch.Tensor       # (D, N) fp32
    Dp: torch.Tensor      # (D,) fp32 skip weight
    w: torch.Tensor       # (D, W) fp32 conv weight; w[:, W-1] multiplies the current token
    b: torch.Tensor       # (D,) fp32 conv bias
    dout: Optional[torch.Tensor] = None  # (T, D) upstream gradient of the gated output
    u: Optional[torch.Tensor] = None     # (T, D) standalone scan input (scan-only tests)

    @property
    def nseq(self) -> int:
        return len(self.lengths)


def _draw_length(rng: np.random.Generator, kind: str) -> int:
    """One document length from a workload's length distribution."""
    if kind == "lognormal":
        L = int(round(math.exp(rng.normal(math.log(800.0), 1.0))))
        return min(max(L, 16), 4096)
    if kind == "uniform":
        return int(rng.integers(64, 2048, endpoint=True))
    if kind == "buckets":
        k = int(rng.integers(0, len(BUCKETS)))
        lo = 0 if k == 0 else BUCKETS[k - 1]
        return int(rng.integers(lo + 1, BUCKETS[k], endpoint=True))
    raise ValueError(kind)


def document_lengths(workload: int, n: int, seed: int = 0) -> list:
    """A stream of `n` whole (uncut) document lengths drawn from a workload's
    length distribution, in arrival order: the input of a packer."""
    rng = np.random.default_rng(seed)
    return [_draw_length(rng, WORKLOADS[workload].lengths) for _ in range(n)]


def _pack_lengths(rng: np.random.Generator, kind: str, n_packs: int, pack_len: int) -> list:
    """Sequence lengths, pack by pack; every pack is filled exactly (the last
    sequence of a pack is cut to the remainder)."""
    if kind == "fixed":
        assert n_packs == 1 and pack_len == 16
        return [4, 2, 3, 7]
    out = []
    for _ in range(n_packs):
        left = pack_len
        pack = []
        while left > 0:
            L = min(_draw_length(rng, kind), left)
            pack.append(L)
            left -= L
        if kind == "buckets":
            # one single-token sequence per pack, at a seeded position; the
            # pack total is kept by shortening the longest sequence by one
            i = int(np.argmax(pack))
            pack[i] -= 1
            at = int(rng.integers(0, len(pack) + 1))
            pack.insert(at, 1)
            pack = [L for L in pack if L > 0]
        out.extend(pack)
    return out


def cu_seqlens_of(lengths) -> np.ndarray:
    """FlashAttention-style cumulative lengths: [0, L0, L0+L1, ...] (int32)."""
    cu = np.zeros(len(lengths) + 1, dtype=np.int64)
    cu[1:] = np.cumsum(np.asarray(lengths, dtype=np.int64))
    assert cu[-1] < 2**31
    return cu.astype(np.int32)


def to_dtype(a: np.ndarray, dtype: torch.dtype) -> torch.Tensor:
    """fp32/fp64 numpy -> torch dtype; bf16 uses torch's round-to-nearest-even."""
    t = torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32))
    return t.to(dtype) if dtype != torch.float32 else t


def make_inputs(workload: int, *, n_packs: Optional[int] = None, pack_len: Optional[int] = None,
                D: Optional[int] = None, N: Optional[int] = None, dtype: Optional[torch.dtype] = None,
                seed: Optional[int] = None, lengths: Optional[list] = None,
                with_dout: Optional[bool] = None, with_u: bool = False) -> Inputs:
    """Draw one packed batch of a workload.

    The overrides shrink a workload (fewer packs, shorter packs, fewer
    channels) while keeping its length distribution; `lengths` replaces the
    drawn lengths altogether. Draw order: lengths, x, z, B, C, r, dt, w, then
    dout; the standalone scan input u comes from a second stream.
    """
    wl = WORKLOADS[workload]
    n_packs = wl.n_packs if n_packs is None else n_packs
    pack_len = wl.pack_len if pack_len is None else pack_len
    D = wl.D if D is None else D
    N = wl.N if N is None else N
    W = wl.W
    dtype = wl.dtype if dtype is None else dtype
    if seed is None:
        seed = 2 if workload == 4 else workload
    if with_dout is None:
        with_dout = workload == 4
    rng = np.random.default_rng(seed)
    drawn = _pack_lengths(rng, wl.lengths, n_packs, pack_len)
    if lengths is None:
        lengths = drawn
    lengths = [int(L) for L in lengths]
    T = int(sum(lengths))
    cu = cu_seqlens_of(lengths)

    x = rng.standard_normal((T, D), dtype=np.float32)
    z = rng.standard_normal((T, D), dtype=np.float32)
    B = rng.standard_normal((T, N), dtype=np.float32)
    C = rng.standard_normal((T, N), dtype=np.float32)
    r = rng.standard_normal((T, D), dtype=np.float32) * np.float32(0.5)
    dt = rng.uniform(1e-3, 0.1, size=D)
    # softplus(r + log(expm1(dt))) in fp64, then stored in the workload dtype
    pre = r.astype(np.float64) + np.log(np.expm1(dt))[None, :]
    delta = np.logaddexp(0.0, pre)
    w = rng.uniform(-0.5, 0.5, size=(D, W)).astype(np.float32)
    A = -np.tile(np.arange(1, N + 1, dtype=np.float32), (D, 1))
    dout = rng.standard_normal((T, D), dtype=np.float32) if with_dout else None
    u = None
    if with_u:
        rng_u = np.random.default_rng([seed, 1])
        u = to_dtype(rng_u.standard_normal((T, D), dtype=np.float32), dtype)

    return Inputs(
        workload=workload, lengths=lengths, cu_seqlens=cu, T=T, D=D, N=N, W=W, dtype=dtype,
        x=to_dtype(x, dtype), z=to_dtype(z, dtype), B=to_dtype(B, dtype), C=to_dtype(C, dtype),
        delta=to_dtype(delta, dtype),
        A=torch.from_numpy(A), Dp=torch.ones(D, dtype=torch.float32),
        w=torch.from_numpy(w), b=torch.zeros(D, dtype=torch.float32),
        dout=None if dout is None else to_dtype(dout, dtype), u=u,
    )


def f64(t: torch.Tensor) -> np.ndarray:
    """Exact widening of a stored tensor to fp64 numpy (bf16 and fp32 both
    embed exactly in fp64)."""
    return t.detach().to("cpu").to(torch.float64).numpy()


def sub_pack(inp: Inputs, seq_ids) -> dict:
    """Token rows of the chosen sequences, in order, with their own cu_seqlens.
    Pure indexing: used to run chosen sequences alone."""
    rows = np.concatenate([np.arange(inp.cu_seqlens[s], inp.cu_seqlens[s + 1]) for s in seq_ids])
    lengths = [int(inp.cu_seqlens[s + 1] - inp.cu_seqlens[s]) for s in seq_ids]
    return {"rows": rows, "lengths": lengths, "cu_seqlens": cu_seqlens_of(lengths)}
