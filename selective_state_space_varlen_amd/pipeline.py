"""The sequence-wise part of one Mamba-1 block on a packed batch, as a chain
of library calls (no arithmetic here):

  forward:  varlen_pack_indices -> conv1d_pack_fwd (SiLU) -> selective_scan_pack_fwd
  backward: selective_scan_pack_bwd -> conv1d_pack_bwd

Shanghai AI Lab article on packed variable-length Mamba-1 training
(gitcode.csdn.net/69d8cc1b54b52172bc6872cb.html), section "Mamba block中的步骤":
conv1d and the SSM are the block's two sequence-wise steps; the conv feeds
the scan through SiLU (Mamba-1's block order).
"""
from __future__ import annotations

from typing import Optional

import torch

from . import binding as _b


def forward(x: torch.Tensor, w: torch.Tensor, b: Optional[torch.Tensor], delta: torch.Tensor, A: torch.Tensor,
            B: torch.Tensor, C: torch.Tensor, Dskip: Optional[torch.Tensor], z: Optional[torch.Tensor],
            cu_seqlens: torch.Tensor, pos: Optional[torch.Tensor] = None, ws: Optional[dict] = None,
            initial_states: Optional[dict] = None, final_states: bool = False,
            delta_bias: Optional[torch.Tensor] = None, delta_softplus: bool = False,
            gate_floor: float = 0.0) -> dict:
    """Returns {'pos', 'u', 'out', 'scan_ws', 'step_map'}; keep it for backward.

    delta_bias / delta_softplus / gate_floor: the scan's step is
    softplus(delta + bias) (or delta + bias) and its gate SiLU(z) + gate_floor;
    the backward takes them from the returned dict and adds 'ddelta_bias'.

    Sequences continued from an earlier pack (the article's section
    "结论与讨论": a sequence cut at a pack end keeps passing state) take
    initial_states = {'ssm': (nseq, D, N) fp32, 'conv': (nseq, W-1, D)} (either
    may be None: zeros); with final_states=True, or with initial states, the
    result also holds 'final_states' in the same form."""
    T = x.shape[0]
    if pos is None:
        pos, _, _ = _b.varlen_pack_indices(cu_seqlens, T, heads=False, dev_err=False)
    carry = initial_states is not None or final_states
    sm = {"delta_bias": delta_bias, "delta_softplus": delta_softplus, "gate_floor": gate_floor}
    res = {"pos": pos, "step_map": sm}
    if carry:
        st = initial_states or {}
        u, cf = _b.conv1d_pack_fwd(x, w, b, pos, silu=True, out=None if ws is None else ws.get("u"),
                                   cu_seqlens=cu_seqlens, conv_initial=st.get("conv"), conv_final=True)
        out, scan_ws, hT = _b.selective_scan_pack_fwd(u, delta, A, B, C, Dskip, z, pos,
                                                      workspace=None if ws is None else ws.get("scan"),
                                                      out=None if ws is None else ws.get("out"),
                                                      cu_seqlens=cu_seqlens, initial_state=st.get("ssm"),
                                                      final_state=True, **sm)
        res.update({"final_states": {"ssm": hT, "conv": cf}, "cu_seqlens": cu_seqlens, "initial_states": st})
    else:
        u = _b.conv1d_pack_fwd(x, w, b, pos, silu=True, out=None if ws is None else ws.get("u"))
        out, scan_ws = _b.selective_scan_pack_fwd(u, delta, A, B, C, Dskip, z, pos,
                                                  workspace=None if ws is None else ws.get("scan"),
                                                  out=None if ws is None else ws.get("out"), **sm)
    res.update({"u": u, "out": out, "scan_ws": scan_ws})
    return res


def backward(x: torch.Tensor, w: torch.Tensor, b: Optional[torch.Tensor], delta: torch.Tensor, A: torch.Tensor,
             B: torch.Tensor, C: torch.Tensor, Dskip: Optional[torch.Tensor], z: Optional[torch.Tensor],
             fwd: dict, dout: torch.Tensor, conv_ws: Optional[torch.Tensor] = None,
             dfinal_states: Optional[dict] = None) -> dict:
    """Gradients of sum(dout * out) (+ sum(dfinal * final) for carried states)
    for x, w, b, delta, A, B, C, Dskip, z. When the forward carried states, the
    result also holds 'dinitial_states' {'ssm', 'conv'}, the gradients to hand
    to the earlier pack's backward as its dfinal_states. With a step bias in
    the forward, the result also holds 'ddelta_bias'."""
    sm = fwd.get("step_map", {})
    if "cu_seqlens" not in fwd:
        g = _b.selective_scan_pack_bwd(fwd["u"], delta, A, B, C, Dskip, z, fwd["pos"], dout, fwd["scan_ws"], **sm)
        dx, dw, db = _b.conv1d_pack_bwd(x, w, b, fwd["pos"], g["du"], silu=True, workspace=conv_ws,
                                        want_db=b is not None)
        g.update({"dx": dx, "dw": dw, "db": db})
        return g
    cu, st, dfs = fwd["cu_seqlens"], fwd["initial_states"], dfinal_states or {}
    g = _b.selective_scan_pack_bwd(fwd["u"], delta, A, B, C, Dskip, z, fwd["pos"], dout, fwd["scan_ws"],
                                   cu_seqlens=cu, initial_state=st.get("ssm"), dfinal_state=dfs.get("ssm"),
                                   dinitial_state=True, **sm)
    dx, dw, db, dci = _b.conv1d_pack_bwd(x, w, b, fwd["pos"], g["du"], silu=True, workspace=conv_ws,
                                         want_db=b is not None, cu_seqlens=cu, conv_initial=st.get("conv"),
                                         dconv_final=dfs.get("conv"), dconv_initial=True)
    g.update({"dx": dx, "dw": dw, "db": db, "dinitial_states": {"ssm": g.pop("dinitial_state"), "conv": dci}})
    return g
