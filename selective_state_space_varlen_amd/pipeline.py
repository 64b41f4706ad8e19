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
            cu_seqlens: torch.Tensor, pos: Optional[torch.Tensor] = None, ws: Optional[dict] = None) -> dict:
    """Returns {'pos', 'u', 'out', 'scan_ws'}; keep it for backward."""
    T = x.shape[0]
    if pos is None:
        pos, _, _ = _b.varlen_pack_indices(cu_seqlens, T, heads=False, dev_err=False)
    u = _b.conv1d_pack_fwd(x, w, b, pos, silu=True, out=None if ws is None else ws.get("u"))
    out, scan_ws = _b.selective_scan_pack_fwd(u, delta, A, B, C, Dskip, z, pos,
                                              workspace=None if ws is None else ws.get("scan"),
                                              out=None if ws is None else ws.get("out"))
    return {"pos": pos, "u": u, "out": out, "scan_ws": scan_ws}


def backward(x: torch.Tensor, w: torch.Tensor, b: Optional[torch.Tensor], delta: torch.Tensor, A: torch.Tensor,
             B: torch.Tensor, C: torch.Tensor, Dskip: Optional[torch.Tensor], z: Optional[torch.Tensor],
             fwd: dict, dout: torch.Tensor, conv_ws: Optional[torch.Tensor] = None) -> dict:
    """Gradients of sum(dout * out) for x, w, b, delta, A, B, C, Dskip, z."""
    g = _b.selective_scan_pack_bwd(fwd["u"], delta, A, B, C, Dskip, z, fwd["pos"], dout, fwd["scan_ws"])
    dx, dw, db = _b.conv1d_pack_bwd(x, w, b, fwd["pos"], g["du"], silu=True, workspace=conv_ws,
                                    want_db=b is not None)
    g.update({"dx": dx, "dw": dw, "db": db})
    return g
