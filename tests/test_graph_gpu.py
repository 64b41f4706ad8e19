"""GPU: the library's calls inside a captured HIP graph.

Every kernel launch goes to the caller's stream and no call uses a memset,
so a block's forward and backward can be captured once and replayed. The
graph is replayed several times, with eager work and synchronisations in
between and fresh inputs copied into its static buffers, and every replay
must equal the eager run bit for bit (the kernels are deterministic).
"""
from __future__ import annotations

import numpy as np
import pytest
import torch

import synth
from tests.gpu_harness import Dev

pytestmark = pytest.mark.gpu


def _run(ssp, d, x, delta, dout, states=None, ext=None):
    F = ssp.forward(x, d.w, d.b, delta, d.A, d.B, d.C, d.Dp, d.z, d.cu, pos=d.pos,
                    initial_states=states, final_states=states is not None, **(ext or {}))
    G = ssp.backward(x, d.w, d.b, delta, d.A, d.B, d.C, d.Dp, d.z, F, dout,
                     dfinal_states=None if states is None else {"ssm": states["ssm"], "conv": None})
    out = {"out": F["out"], **{k: G[k] for k in ("dx", "dw", "db", "ddelta", "dA", "dB", "dC", "dD", "dz")}}
    if ext:
        out["ddelta_bias"] = G["ddelta_bias"]
    if states is not None:
        out["hT"] = F["final_states"]["ssm"]
        out["dh0"] = G["dinitial_states"]["ssm"]
    return out


@pytest.mark.parametrize("with_states,step_map", [(False, False), (True, False), (False, True), (True, True)])
def test_graph_replay_matches_eager(with_states, step_map):
    import selective_state_space_varlen_amd as ssp
    inp = synth.make_inputs(2, n_packs=2, D=256, with_dout=True)
    d = Dev(inp)
    ext = None
    if step_map:
        gb = torch.Generator().manual_seed(4)
        ext = dict(delta_bias=(torch.randn(inp.D, generator=gb) * 0.1).cuda(), delta_softplus=True, gate_floor=0.05)
    states = None
    if with_states:
        g = torch.Generator().manual_seed(3)
        states = {"ssm": torch.randn(inp.nseq, inp.D, inp.N, generator=g).cuda(),
                  "conv": torch.randn(inp.nseq, inp.W - 1, inp.D, generator=g).to(inp.dtype).cuda()}
    rng = np.random.default_rng(5)
    batches = []
    for _ in range(3):
        batches.append(tuple(synth.to_dtype(rng.standard_normal((inp.T, inp.D)) * s, inp.dtype).cuda()
                             for s in (1.0, 0.02, 1.0)))
    # static input buffers of the graph
    sx, sdelta, sdout = (torch.empty_like(t) for t in batches[0])
    sdelta.copy_(d.delta)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):  # warm up outside the graph
        sx.copy_(batches[0][0]); sdout.copy_(batches[0][2])
        _run(ssp, d, sx, sdelta, sdout, states, ext)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        res = _run(ssp, d, sx, sdelta, sdout, states, ext)
    torch.cuda.synchronize()
    for i, (bx, bd, bo) in enumerate(batches):
        # eager reference on the same inputs, then the replay
        delta = (d.delta.float() + bd.float().abs()).to(inp.dtype)
        ref = _run(ssp, d, bx, delta, bo, states, ext)
        torch.cuda.synchronize()
        ref = {k: v.clone() for k, v in ref.items()}
        sx.copy_(bx); sdelta.copy_(delta); sdout.copy_(bo)
        graph.replay()
        torch.cuda.synchronize()
        for k, v in ref.items():
            assert torch.equal(res[k], v), f"replay {i}: {k} differs from the eager run"


def test_concurrent_streams_match_sequential():
    """The library keeps no state between calls: two batches' forward and
    backward issued at the same time on two streams (each with its own
    workspaces) give bit for bit what each gives alone."""
    import selective_state_space_varlen_amd as ssp
    ins = [synth.make_inputs(2, n_packs=2, D=192, seed=s, with_dout=True) for s in (11, 12)]
    devs = [Dev(i) for i in ins]
    ref = []
    for d in devs:
        r = _run(ssp, d, d.x, d.delta, d.dout)
        torch.cuda.synchronize()
        ref.append({k: v.clone() for k, v in r.items()})
    streams = [torch.cuda.Stream(), torch.cuda.Stream()]
    for rep in range(3):
        cur = torch.cuda.current_stream()
        outs = [None, None]
        for j, (d, s) in enumerate(zip(devs, streams)):
            s.wait_stream(cur)
            with torch.cuda.stream(s):
                outs[j] = _run(ssp, d, d.x, d.delta, d.dout)
        for s in streams:
            cur.wait_stream(s)
        torch.cuda.synchronize()
        for j in range(2):
            for k, v in ref[j].items():
                assert torch.equal(outs[j][k], v), f"repeat {rep}, batch {j}: {k} differs from its sequential run"
