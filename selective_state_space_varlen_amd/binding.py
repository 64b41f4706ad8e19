"""ctypes binding of libssmpack.so: argument marshalling only.

Each function here has the name of the C entry point it calls and does
nothing but check tensors, allocate outputs and workspaces with torch, and
pass raw device pointers and the current HIP stream. Every step of the
computation runs in the library's HIP kernels; there is no CPU path. If the
library is missing, every call raises.
"""
from __future__ import annotations

import ctypes
import dataclasses
import os
from typing import Optional

import numpy as np
import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libssmpack.so")

SSMP_F32, SSMP_BF16 = 0, 1
SSMP_PACK_SEQUENTIAL, SSMP_PACK_LOCAL_GREEDY = 0, 1

_c_i32, _c_i64, _c_sz, _c_vp = ctypes.c_int32, ctypes.c_int64, ctypes.c_size_t, ctypes.c_void_p

_SIGNATURES = {
    "ssmp_status_string": (ctypes.c_char_p, [ctypes.c_int]),
    "ssmp_abi_version": (ctypes.c_int, []),
    "varlen_pack_indices": (ctypes.c_int, [_c_vp, _c_i32, _c_i64, _c_vp, _c_vp, _c_vp, _c_vp]),
    "conv1d_pack_fwd": (ctypes.c_int, [_c_vp, _c_vp, _c_vp, _c_vp, _c_vp, _c_i64, _c_i32, _c_i32, _c_i32, _c_i32,
                                       _c_vp]),
    "conv1d_pack_bwd_workspace_bytes": (_c_sz, [_c_i64, _c_i32, _c_i32]),
    "conv1d_pack_bwd": (ctypes.c_int, [_c_vp, _c_vp, _c_vp, _c_vp, _c_vp, _c_vp, _c_vp, _c_vp, _c_vp, _c_sz,
                                       _c_i64, _c_i32, _c_i32, _c_i32, _c_i32, _c_vp]),
    "selective_scan_pack_workspace_bytes": (_c_sz, [_c_i64, _c_i32, _c_i32]),
    "selective_scan_pack_fwd": (ctypes.c_int, [_c_vp, _c_vp, _c_vp, _c_vp, _c_vp, _c_vp, _c_vp, _c_vp, _c_vp,
                                               _c_vp, _c_sz, _c_i64, _c_i32, _c_i32, _c_i32, _c_vp]),
    "selective_scan_pack_bwd": (ctypes.c_int, [_c_vp, _c_vp, _c_vp, _c_vp, _c_vp, _c_vp, _c_vp, _c_vp, _c_vp,
                                               _c_vp, _c_sz, _c_vp, _c_vp, _c_vp, _c_vp, _c_vp, _c_vp, _c_vp,
                                               _c_i64, _c_i32, _c_i32, _c_i32, _c_vp]),
    "selective_scan_pack_fwd_ex": (ctypes.c_int, [_c_vp, _c_vp, _c_vp, _c_vp, _c_vp, _c_vp, _c_vp, _c_vp, _c_vp,
                                                  _c_vp, _c_sz, _c_i64, _c_i32, _c_i32, _c_i32,
                                                  _c_vp, _c_i32, ctypes.c_float, _c_vp]),
    "selective_scan_pack_bwd_ex": (ctypes.c_int, [_c_vp, _c_vp, _c_vp, _c_vp, _c_vp, _c_vp, _c_vp, _c_vp, _c_vp,
                                                  _c_vp, _c_sz, _c_vp, _c_vp, _c_vp, _c_vp, _c_vp, _c_vp, _c_vp,
                                                  _c_i64, _c_i32, _c_i32, _c_i32,
                                                  _c_vp, _c_i32, ctypes.c_float, _c_vp, _c_vp]),
    "selective_scan_pack_fwd_states": (ctypes.c_int, [_c_vp, _c_vp, _c_vp, _c_vp, _c_vp, _c_vp, _c_vp, _c_vp,
                                                      _c_vp, _c_vp, _c_sz, _c_i64, _c_i32, _c_i32, _c_i32,
                                                      _c_vp, _c_i32, ctypes.c_float, _c_vp, _c_i32, _c_vp, _c_vp,
                                                      _c_vp]),
    "selective_scan_pack_bwd_states": (ctypes.c_int, [_c_vp, _c_vp, _c_vp, _c_vp, _c_vp, _c_vp, _c_vp, _c_vp,
                                                      _c_vp, _c_vp, _c_sz, _c_vp, _c_vp, _c_vp, _c_vp, _c_vp,
                                                      _c_vp, _c_vp, _c_i64, _c_i32, _c_i32, _c_i32,
                                                      _c_vp, _c_i32, ctypes.c_float, _c_vp, _c_vp, _c_i32,
                                                      _c_vp, _c_vp, _c_vp, _c_vp]),
    "selective_scan_pack_saved_bytes": (_c_sz, [_c_i64, _c_i32, _c_i32, _c_i32]),
    "selective_scan_pack_fwd_scratch_bytes": (_c_sz, [_c_i64, _c_i32, _c_i32]),
    "selective_scan_pack_bwd_scratch_bytes": (_c_sz, [_c_i64, _c_i32, _c_i32, _c_i32]),
    "selective_scan_pack_fwd_ck": (ctypes.c_int, [_c_vp, _c_vp, _c_vp, _c_vp, _c_vp, _c_vp, _c_vp, _c_vp, _c_vp,
                                                  _c_i64, _c_i32, _c_i32, _c_i32, _c_vp, _c_i32, ctypes.c_float,
                                                  _c_vp, _c_i32, _c_vp, _c_vp, _c_i32, _c_vp, _c_sz, _c_vp, _c_sz,
                                                  _c_vp]),
    "selective_scan_pack_bwd_ck": (ctypes.c_int, [_c_vp, _c_vp, _c_vp, _c_vp, _c_vp, _c_vp, _c_vp, _c_vp, _c_vp,
                                                  _c_vp, _c_vp, _c_vp, _c_vp, _c_vp, _c_vp, _c_vp,
                                                  _c_i64, _c_i32, _c_i32, _c_i32, _c_vp, _c_i32, ctypes.c_float,
                                                  _c_vp, _c_vp, _c_i32, _c_vp, _c_vp, _c_vp, _c_i32, _c_vp, _c_sz,
                                                  _c_vp, _c_sz, _c_vp]),
    "selective_scan_pack_fwd_noalloc": (ctypes.c_int, [_c_vp, _c_vp, _c_vp, _c_vp, _c_vp, _c_vp, _c_vp, _c_vp,
                                                       _c_vp, _c_i64, _c_i32, _c_i32, _c_i32, _c_vp, _c_i32,
                                                       ctypes.c_float, _c_vp, _c_i32, _c_vp, _c_vp, _c_vp]),
    "conv1d_pack_fwd_states": (ctypes.c_int, [_c_vp, _c_vp, _c_vp, _c_vp, _c_vp, _c_i64, _c_i32, _c_i32, _c_i32,
                                              _c_i32, _c_vp, _c_i32, _c_vp, _c_vp, _c_vp]),
    "conv1d_pack_bwd_states_workspace_bytes": (_c_sz, [_c_i64, _c_i32, _c_i32, _c_i32]),
    "conv1d_pack_bwd_states": (ctypes.c_int, [_c_vp, _c_vp, _c_vp, _c_vp, _c_vp, _c_vp, _c_vp, _c_vp, _c_vp, _c_sz,
                                              _c_i64, _c_i32, _c_i32, _c_i32, _c_i32, _c_vp, _c_i32, _c_vp, _c_vp,
                                              _c_vp, _c_vp]),
    "varlen_pack_plan": (ctypes.c_int, [_c_vp, _c_i32, _c_i32, _c_i32, _c_i32, _c_vp, _c_vp, _c_vp, _c_vp,
                                        _c_vp, _c_vp]),
}

EXPORTED = tuple(_SIGNATURES)

_lib = None


class SsmpError(RuntimeError):
    def __init__(self, fn: str, status: int):
        self.status = status
        msg = load().ssmp_status_string(status).decode() if status >= 0 else "?"
        super().__init__(f"{fn} failed: status {status} ({msg})")


def load(path: str = LIB_PATH) -> ctypes.CDLL:
    """Load the library (once). Raises if it has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise RuntimeError(f"libssmpack.so not found at {path}; build it with "
                           f"`python -m selective_state_space_varlen_amd.build`")
    lib = ctypes.CDLL(path)
    for name, (res, args) in _SIGNATURES.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    _lib = lib
    return lib


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(t: torch.Tensor):
    return ctypes.c_void_p(torch.cuda.current_stream(t.device).cuda_stream)


def _dtype_code(t: torch.Tensor) -> int:
    if t.dtype == torch.bfloat16:
        return SSMP_BF16
    if t.dtype == torch.float32:
        return SSMP_F32
    raise TypeError(f"unsupported dtype {t.dtype} (bfloat16 or float32)")


def _check(t: Optional[torch.Tensor], name: str, shape=None, dtype=None, device=None):
    if t is None:
        return
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")
    if dtype is not None and t.dtype != dtype:
        raise ValueError(f"{name} has dtype {t.dtype}, expected {dtype}")
    if device is not None and t.device != device:
        raise ValueError(f"{name} is on {t.device}, expected {device}")


def _call(name: str, *args):
    st = getattr(load(), name)(*args)
    if st != 0:
        raise SsmpError(name, st)


# ---------------------------------------------------------------------------
@dataclasses.dataclass
class PackPlan:
    """Result of varlen_pack_plan (host arrays). Pack p holds the sequences
    order[pack_bounds[p]:pack_bounds[p+1]]; cu_seqlens runs along `order`."""
    capacity: int
    order: np.ndarray        # int32 [nseq]
    pack_bounds: np.ndarray  # int32 [n_packs + 1]
    cu_seqlens: np.ndarray   # int32 [nseq + 1]
    max_seqlen: np.ndarray   # int32 [n_packs]
    padding: int             # n_packs * capacity - total tokens

    @property
    def n_packs(self) -> int:
        return len(self.pack_bounds) - 1

    @property
    def padding_rate(self) -> float:
        """Share of the packs' token slots left as padding."""
        slots = self.n_packs * self.capacity
        return self.padding / slots if slots else 0.0


def varlen_pack_plan(lengths, capacity: int, strategy: int = SSMP_PACK_SEQUENTIAL, window: int = 1) -> PackPlan:
    """Host call: group sequences of the given lengths (arrival order) into
    packs of `capacity` tokens. No GPU is used."""
    ln = np.ascontiguousarray(np.asarray(lengths, dtype=np.int64))
    if ln.ndim != 1 or (ln.size and (ln.min() < np.iinfo(np.int32).min or ln.max() > np.iinfo(np.int32).max)):
        raise ValueError("lengths must be a 1-D sequence of int32 values")
    ln = ln.astype(np.int32)
    n = ln.size
    order = np.empty(n, np.int32)
    bounds = np.empty(n + 1, np.int32)
    cu = np.empty(n + 1, np.int32)
    mx = np.empty(max(n, 1), np.int32)
    npk = np.zeros(1, np.int32)
    pad = np.zeros(1, np.int64)
    _call("varlen_pack_plan", ln.ctypes.data_as(_c_vp), n, capacity, strategy, window, order.ctypes.data_as(_c_vp),
          bounds.ctypes.data_as(_c_vp), cu.ctypes.data_as(_c_vp), mx.ctypes.data_as(_c_vp),
          npk.ctypes.data_as(_c_vp), pad.ctypes.data_as(_c_vp))
    k = int(npk[0])
    return PackPlan(capacity, order, bounds[:k + 1].copy(), cu, mx[:k].copy(), int(pad[0]))


def varlen_pack_indices(cu_seqlens: torch.Tensor, T: int, heads: bool = True, dev_err: bool = True,
                        out: Optional[torch.Tensor] = None):
    """cu_seqlens (int32, device) -> (pos int32 [T], heads uint8 [T] or None,
    dev_err int32 [1] or None). dev_err holds 0 or SSMP_ERR_CU_SEQLENS."""
    _check(cu_seqlens, "cu_seqlens", dtype=torch.int32)
    dev = cu_seqlens.device
    pos = torch.empty(T, dtype=torch.int32, device=dev) if out is None else out
    _check(pos, "pos", (T,), torch.int32, dev)
    hd = torch.empty(T, dtype=torch.uint8, device=dev) if heads else None
    err = torch.empty(1, dtype=torch.int32, device=dev) if dev_err else None
    _call("varlen_pack_indices", _ptr(cu_seqlens), cu_seqlens.numel() - 1, T, _ptr(pos), _ptr(hd), _ptr(err),
          _stream(cu_seqlens))
    return pos, hd, err


def _out_or_new(spec, shape, dtype, dev):
    if spec is True:
        return torch.empty(shape, dtype=dtype, device=dev)
    return spec if isinstance(spec, torch.Tensor) else None


def _nseq(cu_seqlens, dev) -> int:
    if cu_seqlens is None:
        raise ValueError("sequence states need cu_seqlens")
    _check(cu_seqlens, "cu_seqlens", dtype=torch.int32, device=dev)
    return cu_seqlens.numel() - 1


def conv1d_pack_fwd(x: torch.Tensor, w: torch.Tensor, b: Optional[torch.Tensor], pos: torch.Tensor,
                    silu: bool = True, out: Optional[torch.Tensor] = None, cu_seqlens: Optional[torch.Tensor] = None,
                    conv_initial: Optional[torch.Tensor] = None, conv_final=False):
    """Returns u. cu_seqlens (with optional conv_initial (nseq, W-1, D) and
    conv_final: True, or an output tensor) selects conv1d_pack_fwd_states;
    the return value is then (u, conv_final or None)."""
    T, D = x.shape
    W = w.shape[1]
    _check(x, "x"); _check(w, "w", (D, W), torch.float32, x.device); _check(b, "b", (D,), torch.float32, x.device)
    _check(pos, "pos", (T,), torch.int32, x.device)
    u = torch.empty_like(x) if out is None else out
    _check(u, "u", (T, D), x.dtype, x.device)
    if cu_seqlens is not None or conv_initial is not None or conv_final is not False:
        nseq = _nseq(cu_seqlens, x.device)
        cf = _out_or_new(conv_final, (nseq, W - 1, D), x.dtype, x.device)
        _check(conv_initial, "conv_initial", (nseq, W - 1, D), x.dtype, x.device)
        _check(cf, "conv_final", (nseq, W - 1, D), x.dtype, x.device)
        _call("conv1d_pack_fwd_states", _ptr(x), _ptr(w), _ptr(b), _ptr(pos), _ptr(u), T, D, W, _dtype_code(x),
              int(silu), _ptr(cu_seqlens), nseq, _ptr(conv_initial), _ptr(cf), _stream(x))
        return u, cf
    _call("conv1d_pack_fwd", _ptr(x), _ptr(w), _ptr(b), _ptr(pos), _ptr(u), T, D, W, _dtype_code(x), int(silu),
          _stream(x))
    return u


def conv1d_pack_bwd_workspace_bytes(T: int, D: int, W: int) -> int:
    return int(load().conv1d_pack_bwd_workspace_bytes(T, D, W))


def conv1d_pack_bwd_states_workspace_bytes(T: int, D: int, W: int, nseq: int) -> int:
    return int(load().conv1d_pack_bwd_states_workspace_bytes(T, D, W, nseq))


def conv1d_pack_bwd(x: torch.Tensor, w: torch.Tensor, b: Optional[torch.Tensor], pos: torch.Tensor,
                    du: torch.Tensor, silu: bool = True, workspace: Optional[torch.Tensor] = None,
                    want_db: bool = True, out: Optional[tuple] = None, cu_seqlens: Optional[torch.Tensor] = None,
                    conv_initial: Optional[torch.Tensor] = None, dconv_final: Optional[torch.Tensor] = None,
                    dconv_initial=False):
    """Returns (dx, dw, db); `out` may supply those three buffers.
    cu_seqlens (with optional conv_initial, dconv_final and dconv_initial:
    True, or an output tensor) selects conv1d_pack_bwd_states; the return
    value is then (dx, dw, db, dconv_initial or None)."""
    T, D = x.shape
    W = w.shape[1]
    _check(x, "x"); _check(w, "w", (D, W), torch.float32, x.device); _check(b, "b", (D,), torch.float32, x.device)
    _check(pos, "pos", (T,), torch.int32, x.device); _check(du, "du", (T, D), x.dtype, x.device)
    if out is not None:
        dx, dw, db = out
    else:
        dx = torch.empty_like(x)
        dw = torch.empty((D, W), dtype=torch.float32, device=x.device)
        db = torch.empty((D,), dtype=torch.float32, device=x.device) if want_db else None
    _check(dx, "dx", (T, D), x.dtype, x.device); _check(dw, "dw", (D, W), torch.float32, x.device)
    _check(db, "db", (D,), torch.float32, x.device)
    if cu_seqlens is not None or conv_initial is not None or dconv_final is not None or dconv_initial is not False:
        nseq = _nseq(cu_seqlens, x.device)
        dci = _out_or_new(dconv_initial, (nseq, W - 1, D), x.dtype, x.device)
        for name, t in (("conv_initial", conv_initial), ("dconv_final", dconv_final), ("dconv_initial", dci)):
            _check(t, name, (nseq, W - 1, D), x.dtype, x.device)
        nbytes = conv1d_pack_bwd_states_workspace_bytes(T, D, W, nseq)
        if workspace is None:
            workspace = torch.empty(max(nbytes, 1), dtype=torch.uint8, device=x.device)
        _call("conv1d_pack_bwd_states", _ptr(x), _ptr(w), _ptr(b), _ptr(pos), _ptr(du), _ptr(dx), _ptr(dw),
              _ptr(db), _ptr(workspace), workspace.numel() * workspace.element_size(), T, D, W, _dtype_code(x),
              int(silu), _ptr(cu_seqlens), nseq, _ptr(conv_initial), _ptr(dconv_final), _ptr(dci), _stream(x))
        return dx, dw, db, dci
    nbytes = conv1d_pack_bwd_workspace_bytes(T, D, W)
    if workspace is None:
        workspace = torch.empty(max(nbytes, 1), dtype=torch.uint8, device=x.device)
    _call("conv1d_pack_bwd", _ptr(x), _ptr(w), _ptr(b), _ptr(pos), _ptr(du), _ptr(dx), _ptr(dw), _ptr(db),
          _ptr(workspace), workspace.numel() * workspace.element_size(), T, D, W, _dtype_code(x), int(silu),
          _stream(x))
    return dx, dw, db


def selective_scan_pack_workspace_bytes(T: int, D: int, N: int) -> int:
    return int(load().selective_scan_pack_workspace_bytes(T, D, N))


def _extended(delta_bias, delta_softplus, gate_floor) -> bool:
    return delta_bias is not None or bool(delta_softplus) or float(gate_floor) != 0.0


def _check_states(nseq, named, D, N, dev):
    for name, t in named:
        _check(t, name, (nseq, D, N), torch.float32, dev)


def _bias_grad(delta_bias, out, D, dev):
    """The d bias output (from `out` when given there), or None without a bias."""
    if delta_bias is None:
        return None
    ddb = out.get("ddelta_bias") if out is not None else None
    if ddb is None:
        ddb = torch.empty((D,), dtype=torch.float32, device=dev)
    _check(ddb, "ddelta_bias", (D,), torch.float32, dev)
    return ddb


def selective_scan_pack_fwd(u, delta, A, B, C, Dskip, z, pos, workspace: Optional[torch.Tensor] = None,
                            out: Optional[torch.Tensor] = None, delta_bias: Optional[torch.Tensor] = None,
                            delta_softplus: bool = False, gate_floor: float = 0.0,
                            cu_seqlens: Optional[torch.Tensor] = None, initial_state: Optional[torch.Tensor] = None,
                            final_state=False):
    """Returns (out, workspace); keep the workspace for the backward.
    delta_bias / delta_softplus / gate_floor select selective_scan_pack_fwd_ex.
    cu_seqlens (with optional initial_state (nseq, D, N) fp32 and final_state:
    True, or an output tensor) selects selective_scan_pack_fwd_states; the
    return value is then (out, workspace, final_state or None)."""
    T, D = u.shape
    N = A.shape[1]
    dev = u.device
    _check(u, "u"); _check(delta, "delta", (T, D), u.dtype, dev); _check(A, "A", (D, N), torch.float32, dev)
    _check(B, "B", (T, N), u.dtype, dev); _check(C, "C", (T, N), u.dtype, dev)
    _check(Dskip, "Dskip", (D,), torch.float32, dev); _check(z, "z", (T, D), u.dtype, dev)
    _check(pos, "pos", (T,), torch.int32, dev)
    nbytes = selective_scan_pack_workspace_bytes(T, D, N)
    if workspace is None:
        workspace = torch.empty(max(nbytes, 1), dtype=torch.uint8, device=dev)
    o = torch.empty_like(u) if out is None else out
    _check(o, "out", (T, D), u.dtype, dev)
    args = (_ptr(u), _ptr(delta), _ptr(A), _ptr(B), _ptr(C), _ptr(Dskip), _ptr(z), _ptr(pos), _ptr(o),
            _ptr(workspace), workspace.numel() * workspace.element_size(), T, D, N, _dtype_code(u))
    if cu_seqlens is not None or initial_state is not None or final_state is not False:
        _check(delta_bias, "delta_bias", (D,), torch.float32, dev)
        nseq = _nseq(cu_seqlens, dev)
        fs = _out_or_new(final_state, (nseq, D, N), torch.float32, dev)
        _check_states(nseq, (("initial_state", initial_state), ("final_state", fs)), D, N, dev)
        _call("selective_scan_pack_fwd_states", *args, _ptr(delta_bias), int(bool(delta_softplus)),
              float(gate_floor), _ptr(cu_seqlens), nseq, _ptr(initial_state), _ptr(fs), _stream(u))
        return o, workspace, fs
    if _extended(delta_bias, delta_softplus, gate_floor):
        _check(delta_bias, "delta_bias", (D,), torch.float32, dev)
        _call("selective_scan_pack_fwd_ex", *args, _ptr(delta_bias), int(bool(delta_softplus)), float(gate_floor),
              _stream(u))
    else:
        _call("selective_scan_pack_fwd", *args, _stream(u))
    return o, workspace


def selective_scan_pack_bwd(u, delta, A, B, C, Dskip, z, pos, dout, workspace: torch.Tensor,
                            out: Optional[dict] = None, delta_bias: Optional[torch.Tensor] = None,
                            delta_softplus: bool = False, gate_floor: float = 0.0,
                            cu_seqlens: Optional[torch.Tensor] = None, initial_state: Optional[torch.Tensor] = None,
                            dfinal_state: Optional[torch.Tensor] = None, dinitial_state=False):
    """Gradients of sum(dout * out); the workspace must come from the forward,
    called with the same options. `out` may supply the result buffers (a dict
    shaped like the return value; "ddelta_bias" is present iff delta_bias is).
    cu_seqlens (with optional initial_state, dfinal_state, dinitial_state:
    True, or an output tensor) selects selective_scan_pack_bwd_states; the
    result then holds "dinitial_state" (None unless asked for)."""
    T, D = u.shape
    N = A.shape[1]
    dev = u.device
    _check(u, "u"); _check(delta, "delta", (T, D), u.dtype, dev); _check(A, "A", (D, N), torch.float32, dev)
    _check(B, "B", (T, N), u.dtype, dev); _check(C, "C", (T, N), u.dtype, dev)
    _check(Dskip, "Dskip", (D,), torch.float32, dev); _check(z, "z", (T, D), u.dtype, dev)
    _check(pos, "pos", (T,), torch.int32, dev); _check(dout, "dout", (T, D), u.dtype, dev)
    _check(workspace, "workspace", device=dev)
    if out is not None:
        du, ddelta, dA, dB, dC, dD, dz = (out[k] for k in ("du", "ddelta", "dA", "dB", "dC", "dD", "dz"))
    else:
        du = torch.empty_like(u)
        ddelta = torch.empty_like(u)
        dA = torch.empty((D, N), dtype=torch.float32, device=dev)
        dB = torch.empty((T, N), dtype=torch.float32, device=dev)
        dC = torch.empty((T, N), dtype=torch.float32, device=dev)
        dD = torch.empty((D,), dtype=torch.float32, device=dev) if Dskip is not None else None
        dz = torch.empty_like(u) if z is not None else None
    _check(du, "du", (T, D), u.dtype, dev); _check(ddelta, "ddelta", (T, D), u.dtype, dev)
    _check(dA, "dA", (D, N), torch.float32, dev); _check(dB, "dB", (T, N), torch.float32, dev)
    _check(dC, "dC", (T, N), torch.float32, dev); _check(dD, "dD", (D,), torch.float32, dev)
    _check(dz, "dz", (T, D), u.dtype, dev)
    args = (_ptr(u), _ptr(delta), _ptr(A), _ptr(B), _ptr(C), _ptr(Dskip), _ptr(z), _ptr(pos), _ptr(dout),
            _ptr(workspace), workspace.numel() * workspace.element_size(), _ptr(du), _ptr(ddelta), _ptr(dA),
            _ptr(dB), _ptr(dC), _ptr(dD), _ptr(dz), T, D, N, _dtype_code(u))
    res = {"du": du, "ddelta": ddelta, "dA": dA, "dB": dB, "dC": dC, "dD": dD, "dz": dz}
    if (cu_seqlens is not None or initial_state is not None or dfinal_state is not None
            or dinitial_state is not False):
        _check(delta_bias, "delta_bias", (D,), torch.float32, dev)
        ddb = _bias_grad(delta_bias, out, D, dev)
        nseq = _nseq(cu_seqlens, dev)
        di = _out_or_new(dinitial_state, (nseq, D, N), torch.float32, dev)
        _check_states(nseq, (("initial_state", initial_state), ("dfinal_state", dfinal_state),
                             ("dinitial_state", di)), D, N, dev)
        _call("selective_scan_pack_bwd_states", *args, _ptr(delta_bias), int(bool(delta_softplus)),
              float(gate_floor), _ptr(ddb), _ptr(cu_seqlens), nseq, _ptr(initial_state), _ptr(dfinal_state),
              _ptr(di), _stream(u))
        res["ddelta_bias"] = ddb
        res["dinitial_state"] = di
        return res
    if _extended(delta_bias, delta_softplus, gate_floor):
        _check(delta_bias, "delta_bias", (D,), torch.float32, dev)
        ddb = _bias_grad(delta_bias, out, D, dev)
        _call("selective_scan_pack_bwd_ex", *args, _ptr(delta_bias), int(bool(delta_softplus)), float(gate_floor),
              _ptr(ddb), _stream(u))
        res["ddelta_bias"] = ddb
    else:
        _call("selective_scan_pack_bwd", *args, _stream(u))
    return res


def selective_scan_pack_saved_bytes(T: int, D: int, N: int, ckpt_interval: int) -> int:
    return int(load().selective_scan_pack_saved_bytes(T, D, N, ckpt_interval))


def selective_scan_pack_fwd_scratch_bytes(T: int, D: int, N: int) -> int:
    return int(load().selective_scan_pack_fwd_scratch_bytes(T, D, N))


def selective_scan_pack_bwd_scratch_bytes(T: int, D: int, N: int, ckpt_interval: int) -> int:
    return int(load().selective_scan_pack_bwd_scratch_bytes(T, D, N, ckpt_interval))


def _nbytes(t: Optional[torch.Tensor]) -> int:
    return 0 if t is None else t.numel() * t.element_size()


def _scratch(scratch, nbytes, dev):
    if scratch is None:
        scratch = torch.empty(max(nbytes, 1), dtype=torch.uint8, device=dev)
    _check(scratch, "scratch", device=dev)
    return scratch


def selective_scan_pack_fwd_ck(u, delta, A, B, C, Dskip, z, pos, ckpt_interval: int,
                               saved: Optional[torch.Tensor] = None, scratch: Optional[torch.Tensor] = None,
                               out: Optional[torch.Tensor] = None, delta_bias: Optional[torch.Tensor] = None,
                               delta_softplus: bool = False, gate_floor: float = 0.0,
                               cu_seqlens: Optional[torch.Tensor] = None,
                               initial_state: Optional[torch.Tensor] = None, final_state=False):
    """The forward keeping the states of every ckpt_interval-th token (0:
    none) in `saved` for the backward. Returns (out, saved or None,
    final_state or None); the scratch is free again once the call's work on
    the current stream is done."""
    T, D = u.shape
    N = A.shape[1]
    dev = u.device
    _check(u, "u"); _check(delta, "delta", (T, D), u.dtype, dev); _check(A, "A", (D, N), torch.float32, dev)
    _check(B, "B", (T, N), u.dtype, dev); _check(C, "C", (T, N), u.dtype, dev)
    _check(Dskip, "Dskip", (D,), torch.float32, dev); _check(z, "z", (T, D), u.dtype, dev)
    _check(pos, "pos", (T,), torch.int32, dev); _check(delta_bias, "delta_bias", (D,), torch.float32, dev)
    if saved is None and ckpt_interval:
        saved = torch.empty(max(selective_scan_pack_saved_bytes(T, D, N, ckpt_interval), 1), dtype=torch.uint8,
                            device=dev)
    _check(saved, "saved", device=dev)
    scratch = _scratch(scratch, selective_scan_pack_fwd_scratch_bytes(T, D, N), dev)
    o = torch.empty_like(u) if out is None else out
    _check(o, "out", (T, D), u.dtype, dev)
    nseq, fs = 0, None
    if cu_seqlens is not None or initial_state is not None or final_state is not False:
        nseq = _nseq(cu_seqlens, dev)
        fs = _out_or_new(final_state, (nseq, D, N), torch.float32, dev)
        _check_states(nseq, (("initial_state", initial_state), ("final_state", fs)), D, N, dev)
    _call("selective_scan_pack_fwd_ck", _ptr(u), _ptr(delta), _ptr(A), _ptr(B), _ptr(C), _ptr(Dskip), _ptr(z),
          _ptr(pos), _ptr(o), T, D, N, _dtype_code(u), _ptr(delta_bias), int(bool(delta_softplus)),
          float(gate_floor), _ptr(cu_seqlens), nseq, _ptr(initial_state), _ptr(fs), int(ckpt_interval),
          _ptr(saved), _nbytes(saved), _ptr(scratch), _nbytes(scratch), _stream(u))
    return o, saved, fs


def selective_scan_pack_bwd_ck(u, delta, A, B, C, Dskip, z, pos, dout, ckpt_interval: int,
                               saved: Optional[torch.Tensor], scratch: Optional[torch.Tensor] = None,
                               out: Optional[dict] = None, delta_bias: Optional[torch.Tensor] = None,
                               delta_softplus: bool = False, gate_floor: float = 0.0,
                               cu_seqlens: Optional[torch.Tensor] = None,
                               initial_state: Optional[torch.Tensor] = None,
                               dfinal_state: Optional[torch.Tensor] = None, dinitial_state=False):
    """Gradients of sum(dout * out) from the states the forward kept at the
    same ckpt_interval (saved; None for 0). Result dict as
    selective_scan_pack_bwd's, with "ddelta_bias" and "dinitial_state"."""
    T, D = u.shape
    N = A.shape[1]
    dev = u.device
    _check(u, "u"); _check(delta, "delta", (T, D), u.dtype, dev); _check(A, "A", (D, N), torch.float32, dev)
    _check(B, "B", (T, N), u.dtype, dev); _check(C, "C", (T, N), u.dtype, dev)
    _check(Dskip, "Dskip", (D,), torch.float32, dev); _check(z, "z", (T, D), u.dtype, dev)
    _check(pos, "pos", (T,), torch.int32, dev); _check(dout, "dout", (T, D), u.dtype, dev)
    _check(delta_bias, "delta_bias", (D,), torch.float32, dev); _check(saved, "saved", device=dev)
    scratch = _scratch(scratch, selective_scan_pack_bwd_scratch_bytes(T, D, N, ckpt_interval), dev)
    if out is not None:
        du, ddelta, dA, dB, dC, dD, dz = (out[k] for k in ("du", "ddelta", "dA", "dB", "dC", "dD", "dz"))
    else:
        du = torch.empty_like(u)
        ddelta = torch.empty_like(u)
        dA = torch.empty((D, N), dtype=torch.float32, device=dev)
        dB = torch.empty((T, N), dtype=torch.float32, device=dev)
        dC = torch.empty((T, N), dtype=torch.float32, device=dev)
        dD = torch.empty((D,), dtype=torch.float32, device=dev) if Dskip is not None else None
        dz = torch.empty_like(u) if z is not None else None
    _check(du, "du", (T, D), u.dtype, dev); _check(ddelta, "ddelta", (T, D), u.dtype, dev)
    _check(dA, "dA", (D, N), torch.float32, dev); _check(dB, "dB", (T, N), torch.float32, dev)
    _check(dC, "dC", (T, N), torch.float32, dev); _check(dD, "dD", (D,), torch.float32, dev)
    _check(dz, "dz", (T, D), u.dtype, dev)
    ddb = _bias_grad(delta_bias, out, D, dev)
    nseq, di = 0, None
    if (cu_seqlens is not None or initial_state is not None or dfinal_state is not None
            or dinitial_state is not False):
        nseq = _nseq(cu_seqlens, dev)
        di = _out_or_new(dinitial_state, (nseq, D, N), torch.float32, dev)
        _check_states(nseq, (("initial_state", initial_state), ("dfinal_state", dfinal_state),
                             ("dinitial_state", di)), D, N, dev)
    _call("selective_scan_pack_bwd_ck", _ptr(u), _ptr(delta), _ptr(A), _ptr(B), _ptr(C), _ptr(Dskip), _ptr(z),
          _ptr(pos), _ptr(dout), _ptr(du), _ptr(ddelta), _ptr(dA), _ptr(dB), _ptr(dC), _ptr(dD), _ptr(dz), T, D, N,
          _dtype_code(u), _ptr(delta_bias), int(bool(delta_softplus)), float(gate_floor), _ptr(ddb),
          _ptr(cu_seqlens), nseq, _ptr(initial_state), _ptr(dfinal_state), _ptr(di), int(ckpt_interval),
          _ptr(saved), _nbytes(saved), _ptr(scratch), _nbytes(scratch), _stream(u))
    return {"du": du, "ddelta": ddelta, "dA": dA, "dB": dB, "dC": dC, "dD": dD, "dz": dz, "ddelta_bias": ddb,
            "dinitial_state": di}


NOALLOC_SCRATCH_BYTES = 128 << 20  # SSMP_NOALLOC_SCRATCH_BYTES


def selective_scan_pack_fwd_noalloc(u, delta, A, B, C, Dskip, z, pos, out: Optional[torch.Tensor] = None,
                                    delta_bias: Optional[torch.Tensor] = None, delta_softplus: bool = False,
                                    gate_floor: float = 0.0, cu_seqlens: Optional[torch.Tensor] = None,
                                    initial_state: Optional[torch.Tensor] = None, final_state=False):
    """The forward-only scan on the library's own scratch (the C entry point
    allocates nothing; pass `out` and a final_state tensor to allocate
    nothing here either). Returns (out, final_state or None). Calls that
    may overlap on one device race."""
    T, D = u.shape
    N = A.shape[1]
    dev = u.device
    _check(u, "u"); _check(delta, "delta", (T, D), u.dtype, dev); _check(A, "A", (D, N), torch.float32, dev)
    _check(B, "B", (T, N), u.dtype, dev); _check(C, "C", (T, N), u.dtype, dev)
    _check(Dskip, "Dskip", (D,), torch.float32, dev); _check(z, "z", (T, D), u.dtype, dev)
    _check(pos, "pos", (T,), torch.int32, dev); _check(delta_bias, "delta_bias", (D,), torch.float32, dev)
    o = torch.empty_like(u) if out is None else out
    _check(o, "out", (T, D), u.dtype, dev)
    nseq, fs = 0, None
    if cu_seqlens is not None or initial_state is not None or final_state is not False:
        nseq = _nseq(cu_seqlens, dev)
        fs = _out_or_new(final_state, (nseq, D, N), torch.float32, dev)
        _check_states(nseq, (("initial_state", initial_state), ("final_state", fs)), D, N, dev)
    _call("selective_scan_pack_fwd_noalloc", _ptr(u), _ptr(delta), _ptr(A), _ptr(B), _ptr(C), _ptr(Dskip),
          _ptr(z), _ptr(pos), _ptr(o), T, D, N, _dtype_code(u), _ptr(delta_bias), int(bool(delta_softplus)),
          float(gate_floor), _ptr(cu_seqlens), nseq, _ptr(initial_state), _ptr(fs), _stream(u))
    return o, fs
