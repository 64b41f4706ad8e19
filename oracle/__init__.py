"""ctypes wrapper of the fp64 CPU oracle (ssm_oracle.c).

TEST INFRASTRUCTURE ONLY: imported by tests, the smoke check and the
benchmark's CPU-baseline leg, never by the product path. It shares no code
with the HIP library.

Every function takes numpy arrays (any float dtype is widened to fp64; the
stored bf16/fp32 values embed exactly) and returns fp64 numpy arrays.
`threads` splits the channel axis into contiguous blocks, one C call per block
(ctypes releases the GIL); the channel split is exact for every output except
dB/dC, whose per-block partials are summed here in block order.
"""
from __future__ import annotations

import contextlib
import ctypes
import os
import subprocess
from concurrent.futures import ThreadPoolExecutor

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "ssm_oracle.c")
_LIB = os.path.join(_HERE, "libssm_oracle.so")

_dp = ctypes.POINTER(ctypes.c_double)
_ip = ctypes.POINTER(ctypes.c_int32)
_u8p = ctypes.POINTER(ctypes.c_uint8)


def build(out: str = _LIB, extra_flags=()) -> str:
    """Compile the oracle with gcc (-O2, strict IEEE: no -ffast-math, no FMA
    contraction, so every operation rounds as written)."""
    cmd = ["gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-ffp-contract=off", "-fno-fast-math",
           *extra_flags, _SRC, "-o", out, "-lm"]
    subprocess.run(cmd, check=True)
    return out


class Oracle:
    """One loaded copy of the oracle library (tests may load variants)."""

    def __init__(self, path: str = _LIB):
        if not os.path.exists(path):
            build(path)
        self.lib = ctypes.CDLL(path)
        L = self.lib
        L.oracle_pack_indices.restype = ctypes.c_int
        L.oracle_pack_indices.argtypes = [_ip, ctypes.c_int32, ctypes.c_int64, _ip, _u8p]
        L.oracle_conv_fwd.restype = None
        L.oracle_conv_fwd.argtypes = [ctypes.c_int64, ctypes.c_int32, ctypes.c_int32, _ip,
                                      _dp, _dp, _dp, ctypes.c_int, ctypes.c_int32, ctypes.c_int32,
                                      _dp, _dp]
        L.oracle_scan_fwd_ex.restype = ctypes.c_int
        L.oracle_scan_fwd_ex.argtypes = [ctypes.c_int64, ctypes.c_int32, ctypes.c_int32, _ip,
                                         _dp, _dp, _dp, _dp, _dp, _dp, _dp,
                                         _dp, ctypes.c_int32, ctypes.c_double,
                                         ctypes.c_int32, ctypes.c_int32, _dp, _dp, _dp]
        L.oracle_scan_bwd_ex.restype = ctypes.c_int
        L.oracle_scan_bwd_ex.argtypes = [ctypes.c_int64, ctypes.c_int32, ctypes.c_int32, _ip,
                                         _dp, _dp, _dp, _dp, _dp, _dp, _dp,
                                         _dp, ctypes.c_int32, ctypes.c_double, _dp,
                                         ctypes.c_int32, ctypes.c_int32,
                                         _dp, _dp, _dp, _dp, _dp, _dp, _dp, _dp]
        L.oracle_conv_bwd.restype = ctypes.c_int
        L.oracle_conv_bwd.argtypes = [ctypes.c_int64, ctypes.c_int32, ctypes.c_int32, _ip,
                                      _dp, _dp, _dp, ctypes.c_int, _dp,
                                      ctypes.c_int32, ctypes.c_int32, _dp, _dp, _dp]
        i64, i32 = ctypes.c_int64, ctypes.c_int32
        L.oracle_conv_fwd_state.restype = ctypes.c_int
        L.oracle_conv_fwd_state.argtypes = [i64, i32, i32, _ip, i32, _dp, _dp, _dp, ctypes.c_int, _dp,
                                            i32, i32, _dp, _dp, _dp]
        L.oracle_conv_bwd_state.restype = ctypes.c_int
        L.oracle_conv_bwd_state.argtypes = [i64, i32, i32, _ip, i32, _dp, _dp, _dp, ctypes.c_int, _dp, _dp, _dp,
                                            i32, i32, _dp, _dp, _dp, _dp]
        L.oracle_scan_fwd_state.restype = ctypes.c_int
        L.oracle_scan_fwd_state.argtypes = [i64, i32, i32, _ip, i32, _dp, _dp, _dp, _dp, _dp, _dp, _dp,
                                            _dp, i32, ctypes.c_double, _dp, i32, i32, _dp, _dp, _dp]
        L.oracle_set_abs_terms.restype = None
        L.oracle_set_abs_terms.argtypes = [ctypes.c_int]
        L.oracle_scan_bwd_state.restype = ctypes.c_int
        L.oracle_scan_bwd_state.argtypes = [i64, i32, i32, _ip, i32, _dp, _dp, _dp, _dp, _dp, _dp, _dp,
                                            _dp, i32, ctypes.c_double, _dp, _dp, _dp, i32, i32,
                                            _dp, _dp, _dp, _dp, _dp, _dp, _dp, _dp, _dp]

    # ---------------------------------------------------------------- helpers
    @staticmethod
    def _d(a):
        return None if a is None else np.ascontiguousarray(a, dtype=np.float64)

    @staticmethod
    def _p(a, typ=_dp):
        return None if a is None else a.ctypes.data_as(typ)

    @staticmethod
    def _blocks(D: int, threads: int):
        threads = max(1, min(int(threads), D)) if D > 0 else 1
        edges = np.linspace(0, D, threads + 1).round().astype(int)
        return [(int(edges[i]), int(edges[i + 1])) for i in range(threads) if edges[i + 1] > edges[i]]

    @staticmethod
    def _run(blocks, fn):
        if len(blocks) <= 1:
            return [fn(*blk) for blk in blocks]
        with ThreadPoolExecutor(max_workers=len(blocks)) as ex:
            return list(ex.map(lambda blk: fn(*blk), blocks))

    # -------------------------------------------------------------- interface
    @contextlib.contextmanager
    def error_scales(self):
        """Within the block, the backward functions (scan_bwd, scan_bwd_state,
        conv_bwd, conv_bwd_state, backward) return for every output the sum
        of the magnitudes of the terms that make it up, the scale of the
        rounding error of that sum (see oracle_set_abs_terms in the C file)."""
        self.lib.oracle_set_abs_terms(1)
        try:
            yield
        finally:
            self.lib.oracle_set_abs_terms(0)

    def pack_indices(self, cu_seqlens, T: int):
        cu = np.ascontiguousarray(cu_seqlens, dtype=np.int32)
        nseq = len(cu) - 1
        pos = np.zeros(max(T, 1), dtype=np.int32)
        head = np.zeros(max(T, 1), dtype=np.uint8)
        rc = self.lib.oracle_pack_indices(self._p(cu, _ip), nseq, T, self._p(pos, _ip), self._p(head, _u8p))
        if rc != 0:
            raise ValueError(f"invalid cu_seqlens (oracle status {rc})")
        return pos[:T], head[:T]

    def conv_fwd(self, x, w, b, pos, silu: bool = True, threads: int = 1):
        x = self._d(x); w = self._d(w); b = self._d(b)
        pos = np.ascontiguousarray(pos, dtype=np.int32)
        T, D = x.shape
        W = w.shape[1]
        v = np.zeros((T, D)); u = np.zeros((T, D))
        self._run(self._blocks(D, threads), lambda d0, d1: self.lib.oracle_conv_fwd(
            T, D, W, self._p(pos, _ip), self._p(x), self._p(w), self._p(b), int(silu), d0, d1,
            self._p(v), self._p(u)))
        return v, u

    def scan_fwd(self, u, delta, A, B, C, Dp, z, pos, threads: int = 1, states: bool = False,
                 delta_bias=None, delta_softplus: bool = False, gate_floor: float = 0.0):
        """delta_bias / delta_softplus: the step is softplus(delta + bias) (or
        delta + bias); gate_floor: the gate is silu(z) + gate_floor."""
        u = self._d(u); delta = self._d(delta); A = self._d(A); B = self._d(B); C = self._d(C)
        Dp = self._d(Dp); z = self._d(z); db = self._d(delta_bias)
        pos = np.ascontiguousarray(pos, dtype=np.int32)
        T, D = u.shape
        N = A.shape[1]
        y = np.zeros((T, D)); out = np.zeros((T, D))
        hs = np.zeros((T, D, N)) if states else None
        rcs = self._run(self._blocks(D, threads), lambda d0, d1: self.lib.oracle_scan_fwd_ex(
            T, D, N, self._p(pos, _ip), self._p(u), self._p(delta), self._p(A), self._p(B), self._p(C),
            self._p(Dp), self._p(z), self._p(db), int(delta_softplus), float(gate_floor),
            d0, d1, self._p(y), self._p(out), self._p(hs)))
        if any(rcs):
            raise MemoryError("oracle_scan_fwd failed")
        return (y, out, hs) if states else (y, out)

    def scan_bwd(self, u, delta, A, B, C, Dp, z, pos, dout, threads: int = 1,
                 delta_bias=None, delta_softplus: bool = False, gate_floor: float = 0.0):
        u = self._d(u); delta = self._d(delta); A = self._d(A); B = self._d(B); C = self._d(C)
        Dp = self._d(Dp); z = self._d(z); dout = self._d(dout); db = self._d(delta_bias)
        pos = np.ascontiguousarray(pos, dtype=np.int32)
        T, D = u.shape
        N = A.shape[1]
        du = np.zeros((T, D)); ddelta = np.zeros((T, D)); dA = np.zeros((D, N))
        dDp = np.zeros(D); dz = np.zeros((T, D)); ddb = np.zeros(D)
        blocks = self._blocks(D, threads)
        parts = [(np.zeros((T, N)), np.zeros((T, N))) for _ in blocks]

        def one(i):
            d0, d1 = blocks[i]
            dB_i, dC_i = parts[i]
            return self.lib.oracle_scan_bwd_ex(
                T, D, N, self._p(pos, _ip), self._p(u), self._p(delta), self._p(A), self._p(B),
                self._p(C), self._p(Dp), self._p(z), self._p(db), int(delta_softplus), float(gate_floor),
                self._p(dout), d0, d1,
                self._p(du), self._p(ddelta), self._p(dA), self._p(dB_i), self._p(dC_i),
                self._p(dDp), self._p(dz), self._p(ddb))

        if len(blocks) <= 1:
            rcs = [one(0)] if blocks else []
        else:
            with ThreadPoolExecutor(max_workers=len(blocks)) as ex:
                rcs = list(ex.map(one, range(len(blocks))))
        if any(rcs):
            raise MemoryError("oracle_scan_bwd failed")
        dB = np.zeros((T, N)); dC = np.zeros((T, N))
        for dB_i, dC_i in parts:
            dB += dB_i
            dC += dC_i
        res = {"du": du, "ddelta": ddelta, "dA": dA, "dB": dB, "dC": dC, "dz": dz}
        res["dD"] = dDp if Dp is not None else None
        res["ddelta_bias"] = ddb if db is not None else None
        return res

    def conv_bwd(self, x, w, b, pos, du, silu: bool = True, threads: int = 1):
        x = self._d(x); w = self._d(w); b = self._d(b); du = self._d(du)
        pos = np.ascontiguousarray(pos, dtype=np.int32)
        T, D = x.shape
        W = w.shape[1]
        dx = np.zeros((T, D)); dw = np.zeros((D, W)); db = np.zeros(D)
        rcs = self._run(self._blocks(D, threads), lambda d0, d1: self.lib.oracle_conv_bwd(
            T, D, W, self._p(pos, _ip), self._p(x), self._p(w), self._p(b), int(silu), self._p(du),
            d0, d1, self._p(dx), self._p(dw), self._p(db)))
        if any(rcs):
            raise MemoryError("oracle_conv_bwd failed")
        return dx, dw, db

    # ------------------------------------- sequences that continue across packs
    # State layouts: h0/hT/dhT/dh0 (nseq, D, N); xc0/xcT/dxcT/dxc0 (nseq, W-1, D).
    def conv_fwd_state(self, x, w, b, cu_seqlens, xc0=None, silu: bool = True, threads: int = 1):
        """conv1d_pack with per-sequence conv context; returns (v, u, xcT)."""
        x = self._d(x); w = self._d(w); b = self._d(b); xc0 = self._d(xc0)
        cu = np.ascontiguousarray(cu_seqlens, dtype=np.int32)
        T, D = x.shape
        W = w.shape[1]
        nseq = len(cu) - 1
        v = np.zeros((T, D)); u = np.zeros((T, D)); xcT = np.zeros((nseq, W - 1, D))
        rcs = self._run(self._blocks(D, threads), lambda d0, d1: self.lib.oracle_conv_fwd_state(
            T, D, W, self._p(cu, _ip), nseq, self._p(x), self._p(w), self._p(b), int(silu), self._p(xc0),
            d0, d1, self._p(v), self._p(u), self._p(xcT)))
        if any(rcs):
            raise ValueError(f"oracle_conv_fwd_state failed {rcs}")
        return v, u, xcT

    def conv_bwd_state(self, x, w, b, cu_seqlens, du, xc0=None, dxcT=None, silu: bool = True, threads: int = 1):
        """Returns (dx, dw, db, dxc0)."""
        x = self._d(x); w = self._d(w); b = self._d(b); du = self._d(du)
        xc0 = self._d(xc0); dxcT = self._d(dxcT)
        cu = np.ascontiguousarray(cu_seqlens, dtype=np.int32)
        T, D = x.shape
        W = w.shape[1]
        nseq = len(cu) - 1
        dx = np.zeros((T, D)); dw = np.zeros((D, W)); db = np.zeros(D); dxc0 = np.zeros((nseq, W - 1, D))
        rcs = self._run(self._blocks(D, threads), lambda d0, d1: self.lib.oracle_conv_bwd_state(
            T, D, W, self._p(cu, _ip), nseq, self._p(x), self._p(w), self._p(b), int(silu), self._p(xc0),
            self._p(du), self._p(dxcT), d0, d1, self._p(dx), self._p(dw), self._p(db), self._p(dxc0)))
        if any(rcs):
            raise ValueError(f"oracle_conv_bwd_state failed {rcs}")
        return dx, dw, db, dxc0

    def scan_fwd_state(self, u, delta, A, B, C, Dp, z, cu_seqlens, h0=None, threads: int = 1,
                       delta_bias=None, delta_softplus: bool = False, gate_floor: float = 0.0):
        """Returns (y, out, hT)."""
        u = self._d(u); delta = self._d(delta); A = self._d(A); B = self._d(B); C = self._d(C)
        Dp = self._d(Dp); z = self._d(z); db = self._d(delta_bias); h0 = self._d(h0)
        cu = np.ascontiguousarray(cu_seqlens, dtype=np.int32)
        T, D = u.shape
        N = A.shape[1]
        nseq = len(cu) - 1
        y = np.zeros((T, D)); out = np.zeros((T, D)); hT = np.zeros((nseq, D, N))
        rcs = self._run(self._blocks(D, threads), lambda d0, d1: self.lib.oracle_scan_fwd_state(
            T, D, N, self._p(cu, _ip), nseq, self._p(u), self._p(delta), self._p(A), self._p(B), self._p(C),
            self._p(Dp), self._p(z), self._p(db), int(delta_softplus), float(gate_floor), self._p(h0),
            d0, d1, self._p(y), self._p(out), self._p(hT)))
        if any(rcs):
            raise ValueError(f"oracle_scan_fwd_state failed {rcs}")
        return y, out, hT

    def scan_bwd_state(self, u, delta, A, B, C, Dp, z, cu_seqlens, dout, h0=None, dhT=None, threads: int = 1,
                       delta_bias=None, delta_softplus: bool = False, gate_floor: float = 0.0):
        """scan_bwd's gradients plus "dh0" (nseq, D, N)."""
        u = self._d(u); delta = self._d(delta); A = self._d(A); B = self._d(B); C = self._d(C)
        Dp = self._d(Dp); z = self._d(z); dout = self._d(dout); db = self._d(delta_bias)
        h0 = self._d(h0); dhT = self._d(dhT)
        cu = np.ascontiguousarray(cu_seqlens, dtype=np.int32)
        T, D = u.shape
        N = A.shape[1]
        nseq = len(cu) - 1
        du = np.zeros((T, D)); ddelta = np.zeros((T, D)); dA = np.zeros((D, N))
        dDp = np.zeros(D); dz = np.zeros((T, D)); ddb = np.zeros(D); dh0 = np.zeros((nseq, D, N))
        blocks = self._blocks(D, threads)
        parts = [(np.zeros((T, N)), np.zeros((T, N))) for _ in blocks]

        def one(i):
            d0, d1 = blocks[i]
            dB_i, dC_i = parts[i]
            return self.lib.oracle_scan_bwd_state(
                T, D, N, self._p(cu, _ip), nseq, self._p(u), self._p(delta), self._p(A), self._p(B),
                self._p(C), self._p(Dp), self._p(z), self._p(db), int(delta_softplus), float(gate_floor),
                self._p(h0), self._p(dout), self._p(dhT), d0, d1,
                self._p(du), self._p(ddelta), self._p(dA), self._p(dB_i), self._p(dC_i),
                self._p(dDp), self._p(dz), self._p(ddb), self._p(dh0))

        rcs = self._run([(i,) for i in range(len(blocks))], one)
        if any(rcs):
            raise ValueError(f"oracle_scan_bwd_state failed {rcs}")
        dB = np.zeros((T, N)); dC = np.zeros((T, N))
        for dB_i, dC_i in parts:
            dB += dB_i
            dC += dC_i
        res = {"du": du, "ddelta": ddelta, "dA": dA, "dB": dB, "dC": dC, "dz": dz, "dh0": dh0}
        res["dD"] = dDp if Dp is not None else None
        res["ddelta_bias"] = ddb if db is not None else None
        return res

    # ------------------------------------------------------ the whole pipeline
    def forward(self, x, w, b, delta, A, B, C, Dp, z, cu_seqlens, threads: int = 1):
        """pack indices -> conv (+SiLU) -> gated selective scan."""
        T = int(np.asarray(x).shape[0])
        pos, head = self.pack_indices(cu_seqlens, T)
        v, u = self.conv_fwd(x, w, b, pos, True, threads)
        y, out = self.scan_fwd(u, delta, A, B, C, Dp, z, pos, threads)
        return {"pos": pos, "head": head, "v": v, "u": u, "y": y, "out": out}

    def backward(self, x, w, b, delta, A, B, C, Dp, z, cu_seqlens, dout, threads: int = 1):
        """Gradients of sum(dout * out) for the whole pipeline."""
        T = int(np.asarray(x).shape[0])
        pos, _ = self.pack_indices(cu_seqlens, T)
        _, u = self.conv_fwd(x, w, b, pos, True, threads)
        g = self.scan_bwd(u, delta, A, B, C, Dp, z, pos, dout, threads)
        dx, dw, db = self.conv_bwd(x, w, b, pos, g["du"], True, threads)
        g.update({"dx": dx, "dw": dw, "db": db, "u": u})
        return g


_default = None


def get() -> Oracle:
    """The oracle library built from ssm_oracle.c (built on first use)."""
    global _default
    if _default is None:
        if (not os.path.exists(_LIB)) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
            build(_LIB)
        _default = Oracle(_LIB)
    return _default
