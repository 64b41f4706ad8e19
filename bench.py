"""Benchmark: packed conv1d_pack + selective_scan_pack, forward and backward,
at the Mamba-1.4B block shape (d_inner 4096, d_state 16, conv width 4, bf16
inputs with fp32 state; 8 packs of 4096 tokens, lengths uniform in
[64, 2048]; upstream gradient N(0, 1)).

One step = the whole hot path over one batch already resident in HBM:
varlen_pack_indices -> conv1d_pack_fwd -> selective_scan_pack_fwd ->
selective_scan_pack_bwd -> conv1d_pack_bwd. Prints one JSON line.

  python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-layouts] [--no-cpu]
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np
import torch

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

import synth  # noqa: E402

COPY_CALIB_BYTES = 1 << 30
PEAK_HBM_GBS = 8000.0    # MI355X HBM3E, vendor figure
# MI355X fp32 vector peak without packed-FP32 instructions (256 CUs x 4 SIMD16
# x 2 FLOP per FMA x 2.4 GHz); the vendor's 157.3 TFLOP/s counts packed FP32,
# which the library's kernels are compiled without
PEAK_FP32_TFLOPS = 78.6

# Floating-point operations of the scan backward's own arithmetic per (token,
# channel, state), FMA = 2, without the forward recompute the implementation
# adds: dh 2, the dB and dC products and their sums over channels 4, sum dh*B 2,
# r = dh*a*h_prev 2, sum A*r 2, dA 2, carry a*dh 1.
SCAN_BWD_FLOPS_PER_TDN = 15

# Algorithmic bytes (each operator reads its inputs once and writes its
# outputs once; bf16 (T, D) tensors, bf16 B/C rows, fp32 dB/dC rows, int32
# positions; per-launch parameter traffic is O(D N) and left out).
# HBM bytes per call of each library entry point at the d_inner 4096,
# 8 x 4096-token workload, from two rocprofv3 --pmc passes (FETCH_SIZE,
# WRITE_SIZE) summed over the call's kernels. The counters were calibrated
# with a plain 1 GiB device copy whose source had been evicted: FETCH_SIZE
# read half the bytes moved (factor 2), WRITE_SIZE all of them (factor 1).
# Valid only for the kernel sources they were taken on (sha256 below); any
# change to those sources reports null until the counters are taken again.
MEASURED_TRAFFIC = {
    "scan_bwd": {"bytes": 4044174784, "sources": ["scan_bwd.hip", "scan_common.h", "common.h"],
                 "sha256": "2f8ab9862d9d9441c642e95f67c5eec573b7e4647d64386fa7c592371ed7725f"},
}


def source_digest(files) -> str:
    import hashlib
    h = hashlib.sha256()
    for f in files:
        with open(os.path.join(ROOT, "selective_state_space_varlen_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()


def measured_traffic(op: str):
    m = MEASURED_TRAFFIC.get(op)
    if not m or m["bytes"] is None or m["sha256"] != source_digest(m["sources"]):
        return None
    return m["bytes"]


def algo_bytes(T: int, D: int, N: int, elt: int = 2) -> dict:
    return {
        "pack_indices": T * 4 + T * 1,                              # write pos + heads
        "conv_fwd": T * (D * 2 * elt + 4),                           # x in, u out, pos
        "scan_fwd": T * (D * 4 * elt + 2 * N * elt + 4),             # u, delta, z in; out; B, C; pos
        "scan_bwd": T * (D * 7 * elt + 2 * N * elt + 2 * N * 4 + 4),  # u,delta,z,dout in; du,ddelta,dz out; B,C; dB,dC; pos
        "conv_bwd": T * (D * 3 * elt + 4),                           # x, du in; dx out; pos
    }


def log(msg: str) -> None:
    print(msg, file=sys.stderr, flush=True)


class Workload:
    """Device-resident inputs, outputs and workspaces of one packed batch."""

    def __init__(self, inp: synth.Inputs, cu=None, dev="cuda:0", states: bool = False, ext: bool = False):
        import selective_state_space_varlen_amd as ssp
        self.ssp = ssp
        self.inp = inp
        self.T, self.D, self.N, self.W = inp.T, inp.D, inp.N, inp.W
        d = torch.device(dev)
        for k in ("x", "z", "B", "C", "delta", "A", "Dp", "w", "b", "dout"):
            setattr(self, k, getattr(inp, k).to(d).contiguous())
        cu_np = inp.cu_seqlens if cu is None else cu
        self.cu = torch.from_numpy(np.ascontiguousarray(cu_np, dtype=np.int32)).to(d)
        T, D, N, W = self.T, self.D, self.N, self.W
        e = lambda *s, dt=self.x.dtype: torch.empty(*s, dtype=dt, device=d)
        self.pos = e(T, dt=torch.int32)
        self.u = e(T, D)
        self.out = e(T, D)
        self.scan_ws = e(max(ssp.selective_scan_pack_workspace_bytes(T, D, N), 1), dt=torch.uint8)
        self.conv_ws = e(max(ssp.conv1d_pack_bwd_workspace_bytes(T, D, W), 1), dt=torch.uint8)
        self.g = {"du": e(T, D), "ddelta": e(T, D), "dz": e(T, D), "dA": e(D, N, dt=torch.float32),
                  "dB": e(T, N, dt=torch.float32), "dC": e(T, N, dt=torch.float32), "dD": e(D, dt=torch.float32)}
        self.dx = e(T, D)
        self.dw = e(D, W, dt=torch.float32)
        self.db = e(D, dt=torch.float32)
        # the step map softplus(delta + bias) and the gate floor, fused into
        # the scan (delta then holds the step before the map)
        self.ext = {}
        if ext:
            g = torch.Generator(device="cpu").manual_seed(6)
            self.ext = dict(delta_bias=(torch.randn(D, generator=g) * 0.1).to(d), delta_softplus=True,
                            gate_floor=0.05)
            self.g["ddelta_bias"] = e(D, dt=torch.float32)
        # every sequence starts from a given conv context and SSM state and
        # hands on its own (the layout of sequences cut across packs)
        self.states = states
        if states:
            nseq = len(cu_np) - 1
            g = torch.Generator(device="cpu").manual_seed(5)
            rnd = lambda *sh, dt=torch.float32: (torch.randn(*sh, generator=g) * 0.1).to(dt).to(d)
            self.st = {"h0": rnd(nseq, D, N), "hT": e(nseq, D, N, dt=torch.float32), "dhT": rnd(nseq, D, N),
                       "dh0": e(nseq, D, N, dt=torch.float32), "ci": rnd(nseq, W - 1, D, dt=self.x.dtype),
                       "cf": e(nseq, W - 1, D), "dcf": rnd(nseq, W - 1, D, dt=self.x.dtype),
                       "dci": e(nseq, W - 1, D)}
            self.conv_ws = e(max(ssp.conv1d_pack_bwd_states_workspace_bytes(T, D, W, nseq), 1), dt=torch.uint8)

    def step(self, ev=None):
        if self.states:
            return self.step_states()
        s = self.ssp
        rec = (lambda i: ev[i].record()) if ev is not None else (lambda i: None)
        rec(0)
        s.varlen_pack_indices(self.cu, self.T, heads=False, dev_err=False, out=self.pos)
        rec(1)
        s.conv1d_pack_fwd(self.x, self.w, self.b, self.pos, silu=True, out=self.u)
        rec(2)
        s.selective_scan_pack_fwd(self.u, self.delta, self.A, self.B, self.C, self.Dp, self.z, self.pos,
                                  workspace=self.scan_ws, out=self.out, **self.ext)
        rec(3)
        s.selective_scan_pack_bwd(self.u, self.delta, self.A, self.B, self.C, self.Dp, self.z, self.pos, self.dout,
                                  self.scan_ws, out=self.g, **self.ext)
        rec(4)
        s.conv1d_pack_bwd(self.x, self.w, self.b, self.pos, self.g["du"], silu=True, workspace=self.conv_ws,
                          out=(self.dx, self.dw, self.db))
        rec(5)


    def step_states(self):
        s, st, cu = self.ssp, self.st, self.cu
        s.varlen_pack_indices(cu, self.T, heads=False, dev_err=False, out=self.pos)
        s.conv1d_pack_fwd(self.x, self.w, self.b, self.pos, silu=True, out=self.u, cu_seqlens=cu,
                          conv_initial=st["ci"], conv_final=st["cf"])
        s.selective_scan_pack_fwd(self.u, self.delta, self.A, self.B, self.C, self.Dp, self.z, self.pos,
                                  workspace=self.scan_ws, out=self.out, cu_seqlens=cu, initial_state=st["h0"],
                                  final_state=st["hT"], **self.ext)
        s.selective_scan_pack_bwd(self.u, self.delta, self.A, self.B, self.C, self.Dp, self.z, self.pos, self.dout,
                                  self.scan_ws, out=self.g, cu_seqlens=cu, initial_state=st["h0"],
                                  dfinal_state=st["dhT"], dinitial_state=st["dh0"], **self.ext)
        s.conv1d_pack_bwd(self.x, self.w, self.b, self.pos, self.g["du"], silu=True, workspace=self.conv_ws,
                          out=(self.dx, self.dw, self.db), cu_seqlens=cu, conv_initial=st["ci"],
                          dconv_final=st["dcf"], dconv_initial=st["dci"])


OPS = ["pack_indices", "conv_fwd", "scan_fwd", "scan_bwd", "conv_bwd"]


def time_steps(wl: Workload, steps: int, warmup: int, per_op: bool = True):
    for _ in range(warmup):
        wl.step()
    torch.cuda.synchronize()
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(6)] for _ in range(steps)] if per_op else None
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    start.record()
    for i in range(steps):
        wl.step(evs[i] if per_op else None)
    end.record()
    torch.cuda.synchronize()
    total_ms = start.elapsed_time(end)
    ops = None
    if per_op:
        ops = {}
        for j, name in enumerate(OPS):
            ops[name] = float(np.mean([evs[i][j].elapsed_time(evs[i][j + 1]) for i in range(steps)]))
        # per-step times of the two passes (forward: indices, conv, scan; backward: scan, conv)
        wl.pass_ms = {"fwd": [evs[i][0].elapsed_time(evs[i][3]) for i in range(steps)],
                      "bwd": [evs[i][3].elapsed_time(evs[i][5]) for i in range(steps)]}
    return total_ms, ops


def padded_layout(inp: synth.Inputs, pack_len: int):
    """Each pack's sequences right-padded to that pack's longest one (zeros,
    not counted as tokens)."""
    cu = inp.cu_seqlens
    rows, lengths = [], []
    start = 0
    seqs = list(range(len(inp.lengths)))
    while start < len(seqs):
        # sequences of one pack
        p0 = cu[seqs[start]]
        end = start
        while end < len(seqs) and cu[seqs[end] + 1] <= p0 + pack_len:
            end += 1
        Lmax = max(inp.lengths[s] for s in seqs[start:end])
        for s in seqs[start:end]:
            r = np.arange(cu[s], cu[s + 1])
            rows.append(np.concatenate([r, -np.ones(Lmax - len(r), dtype=np.int64)]))
            lengths.append(Lmax)
        start = end
    rows = np.concatenate(rows)
    real = rows >= 0
    import copy
    p = copy.copy(inp)
    for k in ("x", "z", "B", "C", "delta", "dout"):
        t = getattr(inp, k)
        o = torch.zeros((len(rows),) + tuple(t.shape[1:]), dtype=t.dtype)
        o[torch.from_numpy(real)] = t[torch.from_numpy(rows[real])]
        setattr(p, k, o)
    p.lengths = lengths
    p.cu_seqlens = synth.cu_seqlens_of(lengths)
    p.T = len(rows)
    return p


# (name, strategy, window); window 0 means one window over the whole stream
PACK_STRATEGIES = (("sequential", 0, 1), ("greedy_w16", 1, 16), ("greedy_w128", 1, 128),
                   ("greedy_w1024", 1, 1024), ("greedy_all", 1, 0))


def packing_report(n_docs: int = 20000) -> dict:
    """Padding rate of the host packer (varlen_pack_plan) on streams of whole
    documents drawn from each workload's length mix, packs of the workload's
    pack length, and the packer's own host time."""
    import selective_state_space_varlen_amd as ssp
    out = {}
    for w in (1, 2, 3):
        cap = synth.WORKLOADS[w].pack_len
        docs = synth.document_lengths(w, n_docs, seed=100 + w)
        row = {"capacity": cap, "documents": n_docs, "tokens": int(sum(docs))}
        for name, strategy, window in PACK_STRATEGIES:
            t0 = time.perf_counter()
            plan = ssp.varlen_pack_plan(docs, cap, strategy, window or n_docs)
            ms = (time.perf_counter() - t0) * 1e3
            row[name] = {"padding_rate": round(plan.padding_rate, 5), "packs": plan.n_packs, "host_ms": round(ms, 3)}
        out[synth.NAMES[w]] = row
    return out


def planned_batch(wl_id: int, strategy: int):
    """Whole documents of a workload's length mix, as many as arrival-order
    packing puts into the workload's pack count, packed by `strategy` (one
    window over the batch) into packs of the pack length; each pack's unused
    tail becomes one extra segment, so the kernels run every padding slot.
    Returns (inputs, useful tokens, padding rate)."""
    import selective_state_space_varlen_amd as ssp
    spec = synth.WORKLOADS[wl_id]
    stream = synth.document_lengths(wl_id, 64 * spec.n_packs, seed=200 + wl_id)
    first = ssp.varlen_pack_plan(stream, spec.pack_len, 0)
    assert first.n_packs > spec.n_packs
    docs = stream[:int(first.pack_bounds[spec.n_packs])]
    plan = ssp.varlen_pack_plan(docs, spec.pack_len, strategy, len(docs))
    segs = []
    for p in range(plan.n_packs):
        ids = plan.order[plan.pack_bounds[p]:plan.pack_bounds[p + 1]]
        segs += [docs[i] for i in ids]
        load = sum(docs[i] for i in ids)
        if load < spec.pack_len:
            segs.append(spec.pack_len - load)
    inp = synth.make_inputs(wl_id, lengths=segs, with_dout=True)
    return inp, int(sum(docs)), plan.padding_rate


def per_sequence_loop(wl: Workload, steps: int, warmup: int) -> float:
    """The gradient-accumulation layout: one launch chain per sequence, then
    parameter gradients summed over sequences."""
    ssp = wl.ssp
    cu = wl.inp.cu_seqlens
    segs = [(int(cu[i]), int(cu[i + 1])) for i in range(len(cu) - 1) if cu[i + 1] > cu[i]]
    cus = [torch.tensor([0, b - a], dtype=torch.int32, device=wl.x.device) for a, b in segs]
    acc = {k: torch.zeros_like(wl.g[k]) for k in ("dA", "dD")}
    acc["dw"], acc["db"] = torch.zeros_like(wl.dw), torch.zeros_like(wl.db)

    def one_step():
        for k in acc:
            acc[k].zero_()
        for (a, b), c in zip(segs, cus):
            L = b - a
            pos = wl.pos[a:b]
            ssp.varlen_pack_indices(c, L, heads=False, dev_err=False, out=pos)
            x = wl.x[a:b]
            u = ssp.conv1d_pack_fwd(x, wl.w, wl.b, pos, silu=True, out=wl.u[a:b])
            args = (u, wl.delta[a:b], wl.A, wl.B[a:b], wl.C[a:b], wl.Dp, wl.z[a:b], pos)
            ssp.selective_scan_pack_fwd(*args, workspace=wl.scan_ws, out=wl.out[a:b])
            g = {k: wl.g[k][a:b] for k in ("du", "ddelta", "dz", "dB", "dC")}
            g["dA"], g["dD"] = wl.g["dA"], wl.g["dD"]
            ssp.selective_scan_pack_bwd(*args, wl.dout[a:b], wl.scan_ws, out=g)
            ssp.conv1d_pack_bwd(x, wl.w, wl.b, pos, g["du"], silu=True, workspace=wl.conv_ws,
                                out=(wl.dx[a:b], wl.dw, wl.db))
            acc["dA"].add_(wl.g["dA"]); acc["dD"].add_(wl.g["dD"])
            acc["dw"].add_(wl.dw); acc["db"].add_(wl.db)

    for _ in range(warmup):
        one_step()
    torch.cuda.synchronize()
    t0 = torch.cuda.Event(enable_timing=True); t1 = torch.cuda.Event(enable_timing=True)
    t0.record()
    for _ in range(steps):
        one_step()
    t1.record()
    torch.cuda.synchronize()
    return t0.elapsed_time(t1) / steps


def cpu_baseline(inp: synth.Inputs, channels: int, threads: int) -> dict:
    """The fp64 oracle (as it stands) on a bounded sample: every token of the
    workload, a subset of its channels; tokens/s scaled to all channels. A
    one-core figure on a sixteenth of those channels goes beside it."""
    import oracle
    orc = oracle.get()
    f = synth.f64

    def run(nch, nthreads):
        sl = slice(0, nch)
        x, w, b = f(inp.x)[:, sl], f(inp.w)[sl], f(inp.b)[sl]
        delta, A, Dp = f(inp.delta)[:, sl], f(inp.A)[sl], f(inp.Dp)[sl]
        z, dout = f(inp.z)[:, sl], f(inp.dout)[:, sl]
        B, C = f(inp.B), f(inp.C)
        t = time.perf_counter()
        orc.forward(x, w, b, delta, A, B, C, Dp, z, inp.cu_seqlens, threads=nthreads)
        orc.backward(x, w, b, delta, A, B, C, Dp, z, inp.cu_seqlens, dout, threads=nthreads)
        return time.perf_counter() - t

    sec = run(channels, threads)
    ch1 = max(1, channels // 16)
    sec1 = run(ch1, 1)
    return {"value": inp.T * (channels / inp.D) / sec, "unit": "tokens/s", "cores": threads, "kind": "oracle",
            "sample": f"fwd+bwd of all {inp.T} tokens of the workload on {channels} of {inp.D} channels "
                      f"({sec:.1f} s wall on {threads} threads), scaled by {inp.D}/{channels}",
            "one_core": {"value": inp.T * (ch1 / inp.D) / sec1, "unit": "tokens/s", "cores": 1,
                         "sample": f"all {inp.T} tokens on {ch1} channels ({sec1:.1f} s), scaled by "
                                   f"{inp.D}/{ch1}"}}


def workload_figures(wl_id: int, steps: int, warmup: int) -> dict:
    """Per-pass times, tokens/s and algorithmic HBM rates of another workload
    on the same calls (forward: indices, conv, scan; backward: scan, conv)."""
    inp = synth.make_inputs(wl_id, with_dout=True)
    T, D, N = inp.T, inp.D, inp.N
    wl = Workload(inp)
    total_ms, ops = time_steps(wl, steps, warmup, per_op=True)
    ab = algo_bytes(T, D, N)
    fwd_b = ab["pack_indices"] + ab["conv_fwd"] + ab["scan_fwd"]
    bwd_b = ab["scan_bwd"] + ab["conv_bwd"]
    fwd_ms = float(np.median(wl.pass_ms["fwd"]))
    bwd_ms = float(np.median(wl.pass_ms["bwd"]))
    step_ms = total_ms / steps
    out = {"workload": synth.NAMES[wl_id], "tokens": T, "d_inner": D, "sequences": inp.nseq, "steps": steps,
           "step_ms": round(step_ms, 4), "tokens_per_s": round(T / (step_ms * 1e-3), 1),
           "fwd_ms": round(fwd_ms, 4), "bwd_ms": round(bwd_ms, 4),
           "fwd_tokens_per_s": round(T / (fwd_ms * 1e-3), 1), "bwd_tokens_per_s": round(T / (bwd_ms * 1e-3), 1),
           "fwd_algo_gbs": round(fwd_b / (fwd_ms * 1e-3) / 1e9, 1), "bwd_algo_gbs": round(bwd_b / (bwd_ms * 1e-3) / 1e9, 1),
           "step_algo_gbs": round(sum(ab.values()) / (step_ms * 1e-3) / 1e9, 1),
           "ops_ms": {k: round(v, 4) for k, v in ops.items()}}
    out["fwd_hbm_frac"] = round(out["fwd_algo_gbs"] / PEAK_HBM_GBS, 4)
    out["bwd_hbm_frac"] = round(out["bwd_algo_gbs"] / PEAK_HBM_GBS, 4)
    out["hbm_frac"] = round(out["step_algo_gbs"] / PEAK_HBM_GBS, 4)
    del wl
    torch.cuda.empty_cache()
    return out


# checkpoint intervals of the scan (0: the forward keeps nothing)
CK_INTERVALS = (4, 8, 16, 64, 256, 2048, 0)


def _timed(fn, steps: int, warmup: int) -> float:
    """Median ms of fn() over `steps` calls, each bracketed by events on the
    current stream (where the library launches)."""
    for _ in range(warmup):
        fn()
    torch.cuda.synchronize()
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(steps)]
    for a, b in evs:
        a.record()
        fn()
        b.record()
    torch.cuda.synchronize()
    return float(np.median([a.elapsed_time(b) for a, b in evs]))


def checkpoint_modes(wl: "Workload", steps: int, warmup: int = 2) -> dict:
    """Per checkpoint interval: the bytes one layer keeps from its scan
    forward to its backward, the backward's scratch, and the scan forward
    and backward times (selective_scan_pack_fwd_ck / _bwd_ck)."""
    ssp = wl.ssp
    T, D, N = wl.T, wl.D, wl.N
    args = (wl.u, wl.delta, wl.A, wl.B, wl.C, wl.Dp, wl.z, wl.pos)
    fscr = torch.empty(max(ssp.selective_scan_pack_fwd_scratch_bytes(T, D, N), 1), dtype=torch.uint8,
                       device=wl.x.device)
    out = {}
    for ci in CK_INTERVALS:
        sb = ssp.selective_scan_pack_saved_bytes(T, D, N, ci)
        bb = ssp.selective_scan_pack_bwd_scratch_bytes(T, D, N, ci)
        saved = torch.empty(max(sb, 1), dtype=torch.uint8, device=wl.x.device) if ci else None
        bscr = torch.empty(max(bb, 1), dtype=torch.uint8, device=wl.x.device)
        fwd = lambda: ssp.selective_scan_pack_fwd_ck(*args, ci, saved=saved, scratch=fscr, out=wl.out)
        bwd = lambda: ssp.selective_scan_pack_bwd_ck(*args, wl.dout, ci, saved, scratch=bscr, out=wl.g)
        fwd()
        fms = _timed(fwd, steps, warmup)
        bms = _timed(bwd, steps, warmup)
        out[str(ci)] = {"saved_bytes_per_layer": sb, "fwd_scratch_bytes": fscr.numel(), "bwd_scratch_bytes": bb,
                        "scan_fwd_ms": round(fms, 4), "scan_bwd_ms": round(bms, 4)}
        del saved, bscr
        torch.cuda.empty_cache()
    return out


def forward_only(wl: "Workload", steps: int, warmup: int = 2) -> dict:
    """The inference forward: indices, conv, and the scan keeping no states."""
    ssp = wl.ssp
    T, D, N = wl.T, wl.D, wl.N
    fscr = torch.empty(max(ssp.selective_scan_pack_fwd_scratch_bytes(T, D, N), 1), dtype=torch.uint8,
                       device=wl.x.device)

    def fwd():
        ssp.varlen_pack_indices(wl.cu, T, heads=False, dev_err=False, out=wl.pos)
        ssp.conv1d_pack_fwd(wl.x, wl.w, wl.b, wl.pos, silu=True, out=wl.u)
        ssp.selective_scan_pack_fwd_ck(wl.u, wl.delta, wl.A, wl.B, wl.C, wl.Dp, wl.z, wl.pos, 0, scratch=fscr,
                                       out=wl.out)

    ms = _timed(fwd, steps, warmup)
    ab = algo_bytes(T, D, N)
    b = ab["pack_indices"] + ab["conv_fwd"] + ab["scan_fwd"]
    return {"ms": round(ms, 4), "tokens_per_s": round(T / (ms * 1e-3), 1),
            "algo_gbs": round(b / (ms * 1e-3) / 1e9, 1), "hbm_frac": round(b / (ms * 1e-3) / 1e9 / PEAK_HBM_GBS, 4),
            "scratch_bytes": fscr.numel(), "kept_bytes": 0}


def copy_ceiling(nbytes: int = 1 << 30, reps: int = 10) -> float:
    """GB/s (read + write) of a plain device-to-device copy of nbytes, the
    practical HBM ceiling beside the 8 TB/s vendor peak."""
    src = torch.empty(nbytes // 4, dtype=torch.float32, device="cuda:0").fill_(1.0)
    dst = torch.empty_like(src)
    dst.copy_(src)
    torch.cuda.synchronize()
    s, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    s.record()
    for _ in range(reps):
        dst.copy_(src)
    e.record()
    torch.cuda.synchronize()
    ms = s.elapsed_time(e) / reps
    del src, dst
    return 2 * nbytes / (ms * 1e-3) / 1e9


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", type=int, default=4, choices=[1, 2, 3, 4])
    ap.add_argument("--no-layouts", action="store_true")
    ap.add_argument("--no-cpu", action="store_true")
    ap.add_argument("--no-workloads", action="store_true",
                    help="skip the figures of the d_inner 1536 and long-pack workloads")
    ap.add_argument("--no-modes", action="store_true",
                    help="skip the forward-only pass and the scan's checkpoint-interval modes")
    ap.add_argument("--cpu-channels", type=int, default=4096,
                    help="channels of the workload the oracle baseline runs (all of them by default)")
    ap.add_argument("--copy-calib", action="store_true",
                    help="after timing, run one plain 1 GiB device copy (a known byte count for "
                         "calibrating hardware byte counters)")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print(json.dumps({"error": "this benchmark runs on exactly one GPU; the path has no collectives "
                                   "(packs are independent, so data parallelism needs no exchange on the path)"}))
        sys.exit(2)
    assert torch.cuda.is_available(), "needs a GPU"

    wl_id = args.workload
    spec = synth.WORKLOADS[wl_id]
    log(f"[bench] generating workload {wl_id} ({synth.NAMES[wl_id]})")
    inp = synth.make_inputs(wl_id, with_dout=True)
    T, D, N = inp.T, inp.D, inp.N
    wl = Workload(inp)
    log(f"[bench] T={T} D={D} N={N} nseq={inp.nseq}; warmup {args.warmup}, timing {args.steps} steps")
    total_ms, ops = time_steps(wl, args.steps, args.warmup, per_op=True)
    pct = lambda v: {"median": round(float(np.median(v)), 4), "p10": round(float(np.percentile(v, 10)), 4),
                     "p90": round(float(np.percentile(v, 90)), 4)}
    passes = {k: pct(v) for k, v in wl.pass_ms.items()}
    # a second timed pass without per-op events (the headline number)
    total_ms, _ = time_steps(wl, args.steps, 1, per_op=False)
    ms_step = total_ms / args.steps
    tok_s = T / (ms_step * 1e-3)
    ab = algo_bytes(T, D, N)
    step_bytes = sum(ab.values())
    hbm_gbs = step_bytes / (ms_step * 1e-3) / 1e9
    ops_gbs = {k: ab[k] / (ops[k] * 1e-3) / 1e9 for k in OPS}
    dominant = max(OPS, key=lambda k: ops[k])
    # HBM roofline of the dominant library call (all its launches), the
    # headline; its arithmetic view beside it
    roofline = {"kernel": f"{dominant} (the library call, all its launches)", "bound": "hbm",
                "achieved": round(ops_gbs[dominant], 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
                "frac": round(ops_gbs[dominant] / PEAK_HBM_GBS, 4),
                "traffic": measured_traffic(dominant) if (T, D, N) == (32768, 4096, 16) else None,
                "avg_ms": round(ops[dominant], 4), "algo_bytes_per_launch": ab[dominant]}
    if dominant == "scan_bwd":
        flops = SCAN_BWD_FLOPS_PER_TDN * T * D * N
        ach = flops / (ops[dominant] * 1e-3) / 1e12
        roofline["alu_view"] = {"achieved": round(ach, 2), "peak": PEAK_FP32_TFLOPS, "unit": "TFLOP/s",
                                "frac": round(ach / PEAK_FP32_TFLOPS, 4), "flops_per_launch": flops,
                                "flop_count": "the backward's own arithmetic, 15 FLOP per (t, d, n), FMA = 2, "
                                              "no forward recompute; peak without packed FP32"}
    log("[bench] per-op ms: " + ", ".join(f"{k} {ops[k]:.3f}" for k in OPS))
    log("[bench] per-op algorithmic GB/s: " + ", ".join(f"{k} {ops_gbs[k]:.0f}" for k in OPS))

    fo = cm = None
    if not args.no_modes:
        fo = forward_only(wl, args.steps)
        log(f"[bench] forward only (scan keeps no states): {fo}")
        cm = checkpoint_modes(wl, max(3, args.steps // 2))
        log(f"[bench] scan checkpoint modes: {cm}")

    # (counter runs take the copy calibration below instead: it must be the
    # run's only device copy)
    copy_gbs = None if args.copy_calib else copy_ceiling()
    if copy_gbs:
        log(f"[bench] device copy ceiling {copy_gbs:.0f} GB/s (read + write)")

    if args.copy_calib:
        # src is written, then a second buffer of the same size pushes it out of
        # the caches, so the copy (one hipMemcpy device-to-device dispatch)
        # reads all of src from HBM
        src = torch.empty(COPY_CALIB_BYTES // 4, dtype=torch.float32, device="cuda:0").fill_(1.0)
        evict = torch.empty_like(src).fill_(2.0)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        log(f"[bench] copy calibration: {COPY_CALIB_BYTES} bytes read, {COPY_CALIB_BYTES} bytes written")
        del src, evict, dst

    workloads = None
    if not args.no_workloads:
        workloads = {}
        for w in (1, 3):
            if w == wl_id:
                continue
            log(f"[bench] workload {w} ({synth.NAMES[w]})")
            workloads[synth.NAMES[w]] = workload_figures(w, max(3, args.steps // 2), 2)
            log(f"[bench]   {workloads[synth.NAMES[w]]}")

    layouts = None
    if not args.no_layouts:
        layouts = {"packed": round(tok_s, 1)}
        # the same pack with every sequence carrying conv and SSM states in
        # and out (forward and backward), as when sequences are cut at pack ends
        wsx = Workload(inp, states=True)
        nq = max(3, args.steps // 2)
        ms_x, _ = time_steps(wsx, nq, 2, per_op=False)
        layouts["packed_carry_states"] = round(T / (ms_x / nq * 1e-3), 1)
        del wsx
        # the same pack with the step map softplus(delta + bias) and the gate
        # floor computed inside the scan (the _ex entry points)
        wex = Workload(inp, ext=True)
        ms_e, _ = time_steps(wex, nq, 2, per_op=False)
        layouts["packed_step_map_gate_floor"] = round(T / (ms_e / nq * 1e-3), 1)
        del wex
        # both at once: carried states with the step map and gate floor
        wxe = Workload(inp, states=True, ext=True)
        ms_xe, _ = time_steps(wxe, nq, 2, per_op=False)
        layouts["packed_carry_states_step_map"] = round(T / (ms_xe / nq * 1e-3), 1)
        del wxe
        cu_concat = np.arange(0, T + 1, spec.pack_len, dtype=np.int32)
        wc = Workload(inp, cu=cu_concat)
        ms_c, _ = time_steps(wc, max(3, args.steps // 2), 2, per_op=False)
        layouts["concat_no_reset"] = round(T / (ms_c / max(3, args.steps // 2) * 1e-3), 1)
        del wc
        pinp = padded_layout(inp, spec.pack_len)
        wp = Workload(pinp)
        ms_p, _ = time_steps(wp, max(3, args.steps // 2), 2, per_op=False)
        layouts["padded"] = round(T / (ms_p / max(3, args.steps // 2) * 1e-3), 1)
        layouts["padded_rows"] = pinp.T
        del wp, pinp
        ms_s = per_sequence_loop(wl, max(2, args.steps // 5), 1)
        layouts["per_sequence_loop"] = round(T / (ms_s * 1e-3), 1)
        layouts["packed_over_per_sequence"] = round(tok_s * ms_s * 1e-3 / T, 3)
        layouts["packed_over_concat"] = round(tok_s / layouts["concat_no_reset"], 3)
        # whole documents packed by the host packer, padding run as tokens;
        # the rate counts document tokens only
        for name, strategy in (("planned_sequential", 0), ("planned_greedy", 1)):
            qinp, useful, rate = planned_batch(wl_id, strategy)
            wq = Workload(qinp)
            nq = max(3, args.steps // 2)
            ms_q, _ = time_steps(wq, nq, 2, per_op=False)
            layouts[name] = round(useful / (ms_q / nq * 1e-3), 1)
            layouts[name + "_padding_rate"] = round(rate, 5)
            del wq, qinp
        log(f"[bench] layouts tokens/s: {layouts}")
        torch.cuda.empty_cache()

    cpu = None
    if not args.no_cpu:
        # every host core the machine reports (os.cpu_count()); the cores this
        # process may run on are reported beside it
        threads = os.cpu_count() or 1
        ch = min(args.cpu_channels, D)
        log(f"[bench] oracle baseline on {ch} channels, {threads} threads")
        cpu = cpu_baseline(inp, ch, threads)
        cpu["host_cpu_count"] = os.cpu_count()
        cpu["affinity_cpus"] = len(os.sched_getaffinity(0))

    line = {
        "metric": "packed tokens/s + HBM GB/s (% peak), conv1d_pack+scan fwd/bwd, 1.4B shape",
        "value": round(tok_s, 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": synth.NAMES[wl_id], "d_inner": D, "d_state": N, "conv_width": inp.W,
                   "packs": spec.n_packs, "pack_len": spec.pack_len, "tokens": T, "sequences": inp.nseq,
                   "state_dtype": "fp32"},
        "passes_ms": passes,
        "fwd_tokens_per_s": round(T / (passes["fwd"]["median"] * 1e-3), 1),
        "fwd_hbm_frac": round((ab["pack_indices"] + ab["conv_fwd"] + ab["scan_fwd"]) / (passes["fwd"]["median"] * 1e-3)
                              / 1e9 / PEAK_HBM_GBS, 4),
        "bwd_hbm_frac": round((ab["scan_bwd"] + ab["conv_bwd"]) / (passes["bwd"]["median"] * 1e-3) / 1e9
                              / PEAK_HBM_GBS, 4),
        "forward_only": fo,
        "scan_checkpoint_modes": cm,
        "other_workloads": workloads,
        "hbm_gbs": round(hbm_gbs, 1),
        "hbm_copy_ceiling_gbs": None if copy_gbs is None else round(copy_gbs, 1),
        "hbm_frac": round(hbm_gbs / PEAK_HBM_GBS, 4),
        "ops_ms": {k: round(v, 4) for k, v in ops.items()},
        "ops_algo_gbs": {k: round(v, 1) for k, v in ops_gbs.items()},
        "roofline": roofline,
        "layouts_tokens_per_s": layouts,
        "packing": packing_report(),
        "cpu_baseline": cpu,
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
