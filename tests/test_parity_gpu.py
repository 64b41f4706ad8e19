"""GPU parity: the HIP path (through the C ABI) against the fp64 oracle,
element by element, on seeded inputs that span several tiles and a ragged
tail, plus the edge cases of the method (single-token and zero-length
sequences, heads on chunk boundaries, one sequence across many chunks,
ragged channel groups, every supported d_state and conv width)."""
from __future__ import annotations

import numpy as np
import pytest
import torch

import synth
from tests.gpu_harness import (TOL_GRAD, TOL_OUT, Dev, assert_close, nan_buffer, npy, oracle_pipeline,
                               poison_scan_scratch, scan_workspace, to_dev)
from tests.oracle_checks import read_golden

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    assert torch.cuda.is_available(), "GPU tests need an MI355X"
    import selective_state_space_varlen_amd as ssp
    ssp.load()


def ssp():
    import selective_state_space_varlen_amd as m
    return m


# ---------------------------------------------------------------------------
# varlen_pack_indices: bit-exact
# ---------------------------------------------------------------------------

def test_pack_indices_golden():
    g = read_golden("pack_4_2_3_7.txt")
    cu = torch.tensor(g["cu_seqlens"], dtype=torch.int32, device="cuda")
    pos, heads, err = ssp().varlen_pack_indices(cu, 16)
    torch.cuda.synchronize()
    assert pos.cpu().tolist() == g["position_indices"].tolist()
    assert heads.cpu().tolist() == g["heads"].tolist()
    assert int(err.item()) == 0


@pytest.mark.parametrize("seed", [0, 1, 2])
def test_pack_indices_random(orc, seed):
    rng = np.random.default_rng(seed)
    lengths = [int(v) for v in rng.integers(0, 3000, 200)]
    lengths[3] = 0
    lengths[-1] = 1
    cu = synth.cu_seqlens_of(lengths)
    T = int(cu[-1])
    pos, heads, err = ssp().varlen_pack_indices(torch.from_numpy(cu).cuda(), T)
    rpos, rhead = orc.pack_indices(cu, T)
    assert np.array_equal(pos.cpu().numpy(), rpos)
    assert np.array_equal(heads.cpu().numpy(), rhead)
    assert int(err.item()) == 0


@pytest.mark.parametrize("cu", [[1, 4, 6], [0, 4, 3, 6], [0, 4, 7]])
def test_pack_indices_rejects_bad_cu(cu):
    T = 6
    pos, _, err = ssp().varlen_pack_indices(torch.tensor(cu, dtype=torch.int32, device="cuda"), T)
    p = pos.cpu().numpy()
    assert int(err.item()) == 3
    assert np.all(p >= 0) and np.all(p <= np.arange(T))


# ---------------------------------------------------------------------------
# conv1d_pack
# ---------------------------------------------------------------------------

CONV_CASES = [
    # (dtype, D, W, silu, lengths)
    (torch.float32, 8, 4, True, [4, 2, 3, 7]),
    (torch.float32, 100, 3, True, [1, 5, 130, 2, 70, 1]),
    (torch.float32, 64, 1, False, [33, 1, 1, 200]),
    (torch.bfloat16, 512, 4, True, [700, 1, 3, 322, 129]),
    (torch.bfloat16, 100, 4, True, [1, 5, 130, 2, 70, 1]),   # D % 8 != 0: per-element path
    (torch.bfloat16, 256, 2, False, [256, 128, 3, 1]),
    (torch.bfloat16, 102, 4, True, [3, 260, 1, 40]),         # D % 4 != 0: per-element backward too
    (torch.float32, 33, 2, True, [9, 1, 300, 2]),            # odd D
    (torch.bfloat16, 520, 4, True, [300, 1, 2, 600, 17]),    # a partial 64-vector group
    (torch.bfloat16, 8192, 4, True, [700, 1, 800]),          # twice the benchmark's d_inner
]


@pytest.mark.parametrize("case", range(len(CONV_CASES)))
def test_conv_parity(orc, case):
    dtype, D, W, silu, lengths = CONV_CASES[case]
    inp = synth.make_inputs(2, D=D, dtype=dtype, lengths=lengths, seed=40 + case, with_dout=True)
    w = torch.rand((D, W), generator=torch.Generator().manual_seed(case)) - 0.5
    b = torch.randn(D, generator=torch.Generator().manual_seed(100 + case)) * 0.2
    d = Dev(inp)
    wd, bd = to_dev(w), to_dev(b)
    u = ssp().conv1d_pack_fwd(d.x, wd, bd, d.pos, silu=silu)
    cws = nan_buffer(ssp().conv1d_pack_bwd_workspace_bytes(inp.T, D, W))
    dx, dw, db = ssp().conv1d_pack_bwd(d.x, wd, bd, d.pos, d.dout, silu=silu, workspace=cws)
    pos, _ = orc.pack_indices(inp.cu_seqlens, inp.T)
    _, ru = orc.conv_fwd(synth.f64(inp.x), w.double().numpy(), b.double().numpy(), pos, silu=silu, threads=4)
    rdx, rdw, rdb = orc.conv_bwd(synth.f64(inp.x), w.double().numpy(), b.double().numpy(), pos,
                                 synth.f64(inp.dout), silu=silu, threads=4)
    assert_close(npy(u), ru, TOL_OUT[dtype], "u")
    assert_close(npy(dx), rdx, TOL_GRAD[dtype], "dx")
    assert_close(npy(dw), rdw, TOL_GRAD[dtype], "dw")
    assert_close(npy(db), rdb, TOL_GRAD[dtype], "db")


# ---------------------------------------------------------------------------
# selective_scan_pack, forward and backward
# ---------------------------------------------------------------------------

SCAN_CASES = {
    "workload0": dict(wl=0),
    "workload1-small": dict(wl=1, n_packs=1, D=96),
    "workload2-small": dict(wl=2, n_packs=2, D=128),
    "workload3-small": dict(wl=3, n_packs=1, pack_len=8192, D=64),
    "one-sequence-12-chunks": dict(wl=2, lengths=[3000], D=64),
    "all-single-tokens": dict(wl=2, lengths=[1] * 600, D=64),
    "ragged-tail-fp32": dict(wl=2, lengths=[255, 1, 256, 257, 3, 100], D=65, dtype=torch.float32),
    "heads-on-chunk-starts": dict(wl=2, lengths=[256, 256, 512, 17], D=64),
    "zero-length-sequences": dict(wl=2, lengths=[5, 0, 300, 0, 0, 40, 1000], D=70),
    "d_state-1-fp32": dict(wl=2, lengths=[300, 2, 500], D=33, N=1, dtype=torch.float32),
    # d_state 1 with an odd token count in the last 16-token block: that
    # block's B/C rows end halfway through a 16-byte piece
    "d_state-1-odd-tail-fp32": dict(wl=2, lengths=[109, 10, 1, 206, 11, 6, 6], D=130, N=1, dtype=torch.float32),
    "d_state-1-odd-tail": dict(wl=2, lengths=[109, 10, 1, 206, 11, 6, 6], D=130, N=1),
    "d_state-2": dict(wl=2, lengths=[300, 2, 500], D=64, N=2),
    "d_state-8-fp32": dict(wl=2, lengths=[700, 90], D=130, N=8, dtype=torch.float32),
    "no-gate-no-skip": dict(wl=2, lengths=[400, 1, 299], D=64, gate=False, skip=False),
    "single-token-pack": dict(wl=2, lengths=[1], D=64),
    "wide-d_inner-8192": dict(wl=2, lengths=[700, 1, 800], D=8192),
}


def _scan_case(name):
    spec = dict(SCAN_CASES[name])
    gate = spec.pop("gate", True)
    skip = spec.pop("skip", True)
    wl = spec.pop("wl")
    inp = synth.make_inputs(wl, with_u=True, with_dout=True, **spec)
    return inp, gate, skip


def run_scan_gpu(inp, gate, skip):
    d = Dev(inp)
    z = d.z if gate else None
    Dp = d.Dp if skip else None
    ws = scan_workspace(inp.T, inp.D, inp.N)
    out, ws = ssp().selective_scan_pack_fwd(d.u, d.delta, d.A, d.B, d.C, Dp, z, d.pos, workspace=ws)
    poison_scan_scratch(ws, inp.T, inp.D, inp.N)
    g = ssp().selective_scan_pack_bwd(d.u, d.delta, d.A, d.B, d.C, Dp, z, d.pos, d.dout, ws)
    torch.cuda.synchronize()
    return out, g


def run_scan_oracle(orc, inp, gate, skip, threads=8):
    pos, _ = orc.pack_indices(inp.cu_seqlens, inp.T)
    args = (synth.f64(inp.u), synth.f64(inp.delta), synth.f64(inp.A), synth.f64(inp.B), synth.f64(inp.C),
            synth.f64(inp.Dp) if skip else None, synth.f64(inp.z) if gate else None, pos)
    _, rout = orc.scan_fwd(*args, threads=threads)
    rg = orc.scan_bwd(*args, synth.f64(inp.dout), threads=threads)
    return rout, rg


@pytest.mark.parametrize("name", list(SCAN_CASES))
def test_scan_parity(orc, name):
    inp, gate, skip = _scan_case(name)
    out, g = run_scan_gpu(inp, gate, skip)
    rout, rg = run_scan_oracle(orc, inp, gate, skip)
    to, tg = TOL_OUT[inp.dtype], TOL_GRAD[inp.dtype]
    assert_close(npy(out), rout, to, "out")
    for k in ("du", "ddelta", "dA", "dB", "dC"):
        assert_close(npy(g[k]), rg[k], tg, k)
    if skip:
        assert_close(npy(g["dD"]), rg["dD"], tg, "dD")
    if gate:
        assert_close(npy(g["dz"]), rg["dz"], tg, "dz")


# the step map (delta_bias, softplus) and the gate floor (selective_scan_pack_*_ex)
EXT_CASES = {
    "softplus-bias-floor": dict(wl=2, lengths=[700, 1, 400, 1200], D=128, opts=(True, True, 0.05)),
    "bias-only": dict(wl=2, lengths=[300, 2, 500], D=64, opts=(True, False, 0.0)),
    "softplus-no-bias-no-gate": dict(wl=2, lengths=[400, 1, 299], D=64, gate=False, opts=(False, True, 0.0)),
    "floor-only-fp32-n4": dict(wl=2, lengths=[255, 1, 256, 257], D=65, N=4, dtype=torch.float32,
                               opts=(False, False, 0.1)),
    "softplus-bias-fp32-n8": dict(wl=2, lengths=[600, 90], D=130, N=8, dtype=torch.float32,
                                  opts=(True, True, 0.02)),
}


@pytest.mark.parametrize("name", list(EXT_CASES))
def test_scan_ext_parity(orc, name):
    spec = dict(EXT_CASES[name])
    has_bias, sp, floor = spec.pop("opts")
    gate = spec.pop("gate", True)
    inp = synth.make_inputs(spec.pop("wl"), with_u=True, with_dout=True, **spec)
    rng = np.random.default_rng(7)
    bias = (rng.standard_normal(inp.D) * 0.5).astype(np.float32) if has_bias else None
    # stored steps chosen so that the mapped step keeps the workload's values
    d64 = synth.f64(inp.delta)
    raw = (np.log(np.expm1(d64)) if sp else d64) - (bias[None, :] if has_bias else 0.0)
    inp.delta = synth.to_dtype(raw, inp.dtype)
    d = Dev(inp)
    z = d.z if gate else None
    bt = to_dev(torch.from_numpy(bias)) if has_bias else None
    kw = dict(delta_bias=bt, delta_softplus=sp, gate_floor=floor)
    ws = scan_workspace(inp.T, inp.D, inp.N)
    out, ws = ssp().selective_scan_pack_fwd(d.u, d.delta, d.A, d.B, d.C, d.Dp, z, d.pos, workspace=ws, **kw)
    poison_scan_scratch(ws, inp.T, inp.D, inp.N)
    g = ssp().selective_scan_pack_bwd(d.u, d.delta, d.A, d.B, d.C, d.Dp, z, d.pos, d.dout, ws, **kw)
    torch.cuda.synchronize()
    pos, _ = orc.pack_indices(inp.cu_seqlens, inp.T)
    args = (synth.f64(inp.u), synth.f64(inp.delta), synth.f64(inp.A), synth.f64(inp.B), synth.f64(inp.C),
            synth.f64(inp.Dp), synth.f64(inp.z) if gate else None, pos)
    okw = dict(delta_bias=None if bias is None else bias.astype(np.float64), delta_softplus=sp, gate_floor=floor)
    _, rout = orc.scan_fwd(*args, threads=8, **okw)
    rg = orc.scan_bwd(*args, synth.f64(inp.dout), threads=8, **okw)
    to, tg = TOL_OUT[inp.dtype], TOL_GRAD[inp.dtype]
    assert_close(npy(out), rout, to, "out")
    for k in ("du", "ddelta", "dA", "dB", "dC", "dD"):
        assert_close(npy(g[k]), rg[k], tg, k)
    if gate:
        assert_close(npy(g["dz"]), rg["dz"], tg, "dz")
    if has_bias:
        assert_close(npy(g["ddelta_bias"]), rg["ddelta_bias"], tg, "ddelta_bias")


def test_scan_deterministic():
    inp, gate, skip = _scan_case("workload2-small")
    o1, g1 = run_scan_gpu(inp, gate, skip)
    o2, g2 = run_scan_gpu(inp, gate, skip)
    assert torch.equal(o1, o2)
    for k in g1:
        if g1[k] is not None:
            assert torch.equal(g1[k], g2[k]), k


def test_scan_nonfinite_isolated():
    """Inf in one sequence's input changes no other sequence's results."""
    inp, gate, skip = _scan_case("workload2-small")
    o0, g0 = run_scan_gpu(inp, gate, skip)
    cu = inp.cu_seqlens
    victim = 1
    bad = inp.u.clone()
    bad[int(cu[victim]) + 3, 5] = float("inf")
    inp.u = bad
    o1, g1 = run_scan_gpu(inp, gate, skip)
    keep = np.ones(inp.T, dtype=bool)
    keep[cu[victim]:cu[victim + 1]] = False
    keep_t = torch.from_numpy(keep).cuda()
    assert torch.equal(o0[keep_t], o1[keep_t])
    for k in ("du", "ddelta", "dz", "dB", "dC"):
        assert torch.equal(g0[k][keep_t], g1[k][keep_t]), k


# ---------------------------------------------------------------------------
# the whole pipeline (pack indices -> conv + SiLU -> gated scan, and back)
# ---------------------------------------------------------------------------

PIPE_CASES = {
    "workload0": dict(wl=0),
    "workload2-small": dict(wl=2, n_packs=2, D=256),
    "workload1-small": dict(wl=1, n_packs=1, D=192),
}


@pytest.mark.parametrize("name", list(PIPE_CASES))
def test_pipeline_parity(orc, name):
    spec = dict(PIPE_CASES[name])
    wl = spec.pop("wl")
    inp = synth.make_inputs(wl, with_dout=True, **spec)
    d = Dev(inp)
    F = d.forward()
    G = d.backward(F)
    torch.cuda.synchronize()
    R = oracle_pipeline(orc, inp, backward=True)
    to, tg = TOL_OUT[inp.dtype], TOL_GRAD[inp.dtype]
    assert np.array_equal(F["pos"].cpu().numpy(), R["pos"])
    assert_close(npy(F["u"]), R["u"], to, "u")
    assert_close(npy(F["out"]), R["out"], to, "out")
    for k in ("dx", "dw", "db", "ddelta", "dA", "dB", "dC", "dD", "dz"):
        assert_close(npy(G[k]), R[k], tg, k)


def test_padded_layout_matches_packed():
    """Right-padded layout (pads at each sequence's end, not counted) gives
    the packed results on real tokens, on the same GPU kernels."""
    inp = synth.make_inputs(2, n_packs=1, D=128, with_u=True, with_dout=True)
    out, g = run_scan_gpu(inp, True, True)
    Lmax = max(inp.lengths)
    rows = np.concatenate([np.concatenate([np.arange(inp.cu_seqlens[s], inp.cu_seqlens[s + 1]),
                                           -np.ones(Lmax - L, dtype=np.int64)])
                           for s, L in enumerate(inp.lengths)])
    real = rows >= 0

    def pad(t):
        o = torch.zeros((len(rows),) + tuple(t.shape[1:]), dtype=t.dtype)
        o[torch.from_numpy(real)] = t[torch.from_numpy(rows[real])]
        return o

    import copy
    p = copy.copy(inp)
    for k in ("u", "delta", "z", "B", "C", "dout"):
        setattr(p, k, pad(getattr(inp, k)))
    p.lengths = [Lmax] * len(inp.lengths)
    p.cu_seqlens = synth.cu_seqlens_of(p.lengths)
    p.T = len(rows)
    pout, pg = run_scan_gpu(p, True, True)
    r = torch.from_numpy(real).cuda()
    idx = torch.from_numpy(rows[real]).cuda()
    assert_close(npy(pout[r]), npy(out[idx]), 2e-2, "out")
    for k in ("du", "ddelta", "dz"):
        assert_close(npy(pg[k][r]), npy(g[k][idx]), 2e-2, k)
    for k in ("dA", "dD"):
        assert_close(npy(pg[k]), npy(g[k]), 1e-3, k)


def test_per_sequence_loop_matches_packed():
    """The gradient-accumulation layout (each sequence alone through the
    block chain, parameter gradients summed over sequences), which the
    benchmark times against the packed one, gives the packed results."""
    import selective_state_space_varlen_amd as ss
    inp = synth.make_inputs(2, n_packs=1, D=256, with_dout=True)
    d = Dev(inp)
    F = d.forward()
    G = d.backward(F)
    per_tok = {k: torch.empty_like(F[k]) for k in ("u", "out")}
    per_tok.update({k: torch.empty_like(G[k]) for k in ("dx", "du", "ddelta", "dz", "dB", "dC")})
    acc = {k: torch.zeros_like(G[k]) for k in ("dA", "dD", "dw", "db")}
    for s in range(inp.nseq):
        a, b = int(inp.cu_seqlens[s]), int(inp.cu_seqlens[s + 1])
        if b == a:
            continue
        cu = torch.tensor([0, b - a], dtype=torch.int32, device="cuda")
        sl = slice(a, b)
        Fs = ss.forward(d.x[sl], d.w, d.b, d.delta[sl], d.A, d.B[sl], d.C[sl], d.Dp, d.z[sl], cu)
        Gs = ss.backward(d.x[sl], d.w, d.b, d.delta[sl], d.A, d.B[sl], d.C[sl], d.Dp, d.z[sl], Fs, d.dout[sl])
        for k in ("u", "out"):
            per_tok[k][sl] = Fs[k]
        for k in ("dx", "du", "ddelta", "dz", "dB", "dC"):
            per_tok[k][sl] = Gs[k]
        for k in acc:
            acc[k] += Gs[k]
    torch.cuda.synchronize()
    for k in ("u", "out"):
        assert_close(npy(per_tok[k]), npy(F[k]), TOL_OUT[inp.dtype], k)
    for k in ("dx", "du", "ddelta", "dz", "dB", "dC"):
        assert_close(npy(per_tok[k]), npy(G[k]), TOL_GRAD[inp.dtype], k)
    for k in acc:
        assert_close(npy(acc[k]), npy(G[k]), 1e-3, k)


def test_planned_layout_parity(orc):
    """Whole documents grouped by the host packer (first-fit decreasing) into
    packs of 1024 tokens, each pack's unused tail run as one extra segment:
    the pipeline matches the oracle on that layout, and every document's rows
    match the same document run in arrival order."""
    docs = synth.document_lengths(1, 400, seed=9)
    docs = [max(1, L // 4) for L in docs][:40]
    cap = 1024
    plan = ssp().varlen_pack_plan(docs, cap, 1, len(docs))
    arrival = synth.make_inputs(1, D=64, lengths=docs, with_dout=True)
    rows, segs = [], []
    for p in range(plan.n_packs):
        ids = plan.order[plan.pack_bounds[p]:plan.pack_bounds[p + 1]]
        for i in ids:
            rows.append(np.arange(arrival.cu_seqlens[i], arrival.cu_seqlens[i + 1]))
            segs.append(docs[i])
        tail = cap - sum(docs[i] for i in ids)
        if tail:
            rows.append(-np.ones(tail, dtype=np.int64))
            segs.append(tail)
    rows = np.concatenate(rows)
    real = rows >= 0
    assert plan.cu_seqlens[-1] == real.sum() == sum(docs)
    import copy
    planned = copy.copy(arrival)
    for k in ("x", "z", "B", "C", "delta", "dout"):
        t = getattr(arrival, k)
        o = torch.ones((len(rows),) + tuple(t.shape[1:]), dtype=t.dtype)  # padding slots hold ones
        o[torch.from_numpy(real)] = t[torch.from_numpy(rows[real])]
        setattr(planned, k, o)
    planned.lengths, planned.cu_seqlens, planned.T = segs, synth.cu_seqlens_of(segs), len(rows)
    assert planned.T == plan.n_packs * cap

    dp, da = Dev(planned), Dev(arrival)
    Fp, Fa = dp.forward(), da.forward()
    Gp, Ga = dp.backward(Fp), da.backward(Fa)
    torch.cuda.synchronize()
    R = oracle_pipeline(orc, planned, backward=True)
    to, tg = TOL_OUT[planned.dtype], TOL_GRAD[planned.dtype]
    assert_close(npy(Fp["out"]), R["out"], to, "out")
    for k in ("dx", "dw", "db", "ddelta", "dA", "dB", "dC", "dD", "dz"):
        assert_close(npy(Gp[k]), R[k], tg, k)
    r = torch.from_numpy(real).cuda()
    idx = torch.from_numpy(rows[real]).cuda()
    assert_close(npy(Fp["out"][r]), npy(Fa["out"][idx]), to, "out vs arrival order")
    for k in ("dx", "ddelta", "dz"):
        assert_close(npy(Gp[k][r]), npy(Ga[k][idx]), tg, k + " vs arrival order")


# ---------------------------------------------------------------------------
# sequence states (selective_scan_pack_*_states): initial and final SSM states
# ---------------------------------------------------------------------------

STATE_CASES = {
    "bf16-mixed": dict(wl=2, lengths=[700, 0, 1, 400, 1200, 0], D=128),
    "edges-on-chunk-bounds-fp32": dict(wl=2, lengths=[256, 256, 512, 17, 64, 64], D=65, dtype=torch.float32),
    "one-sequence-many-chunks": dict(wl=2, lengths=[3000], D=64),
    "single-tokens": dict(wl=2, lengths=[1] * 300, D=64),
    "only-initial": dict(wl=2, lengths=[300, 2, 500, 129], D=64, parts=("h0",)),
    "only-final": dict(wl=2, lengths=[300, 2, 500, 129], D=64, parts=("hT",)),
    "only-gradient-path": dict(wl=2, lengths=[300, 2, 500, 129], D=64, parts=("dhT", "dh0")),
    "d_state-1-fp32": dict(wl=2, lengths=[300, 2, 500], D=33, N=1, dtype=torch.float32),
    "d_state-4-fp32": dict(wl=2, lengths=[255, 1, 256, 257], D=65, N=4, dtype=torch.float32),
    "d_state-8": dict(wl=2, lengths=[700, 90, 0], D=130, N=8),
    "no-gate-no-skip": dict(wl=2, lengths=[400, 1, 299], D=64, gate=False, skip=False),
    "step-map-and-floor": dict(wl=2, lengths=[700, 1, 400, 1200], D=128, opts=(True, 0.05)),
    "workload3-small": dict(wl=3, n_packs=1, pack_len=8192, D=64),
}


@pytest.mark.parametrize("name", list(STATE_CASES))
def test_scan_states_parity(orc, name):
    spec = dict(STATE_CASES[name])
    parts = spec.pop("parts", ("h0", "hT", "dhT", "dh0"))
    gate = spec.pop("gate", True)
    skip = spec.pop("skip", True)
    opts = spec.pop("opts", None)
    inp = synth.make_inputs(spec.pop("wl"), with_u=True, with_dout=True, **spec)
    nseq, D, N = inp.nseq, inp.D, inp.N
    rng = np.random.default_rng(17)
    h0 = rng.standard_normal((nseq, D, N)).astype(np.float32) if "h0" in parts else None
    dhT = rng.standard_normal((nseq, D, N)).astype(np.float32) if "dhT" in parts else None
    kw, okw = {}, {}
    if opts is not None:
        # softplus of (stored + bias) with the stored steps chosen to keep the workload's values
        bias = (rng.standard_normal(D) * 0.5).astype(np.float32)
        raw = np.log(np.expm1(synth.f64(inp.delta))) - bias[None, :]
        inp.delta = synth.to_dtype(raw, inp.dtype)
        kw = dict(delta_bias=to_dev(torch.from_numpy(bias)), delta_softplus=True, gate_floor=opts[1])
        okw = dict(delta_bias=bias.astype(np.float64), delta_softplus=True, gate_floor=opts[1])
    d = Dev(inp)
    z = d.z if gate else None
    Dp = d.Dp if skip else None
    h0_d = to_dev(torch.from_numpy(h0)) if h0 is not None else None
    dhT_d = to_dev(torch.from_numpy(dhT)) if dhT is not None else None
    ws = scan_workspace(inp.T, inp.D, inp.N)
    out, ws, hT = ssp().selective_scan_pack_fwd(d.u, d.delta, d.A, d.B, d.C, Dp, z, d.pos, workspace=ws,
                                                cu_seqlens=d.cu, initial_state=h0_d, final_state="hT" in parts, **kw)
    poison_scan_scratch(ws, inp.T, inp.D, inp.N)
    g = ssp().selective_scan_pack_bwd(d.u, d.delta, d.A, d.B, d.C, Dp, z, d.pos, d.dout, ws, cu_seqlens=d.cu,
                                      initial_state=h0_d, dfinal_state=dhT_d, dinitial_state="dh0" in parts, **kw)
    torch.cuda.synchronize()
    args = (synth.f64(inp.u), synth.f64(inp.delta), synth.f64(inp.A), synth.f64(inp.B), synth.f64(inp.C),
            synth.f64(inp.Dp) if skip else None, synth.f64(inp.z) if gate else None, inp.cu_seqlens)
    _, rout, rhT = orc.scan_fwd_state(*args, h0=h0, threads=8, **okw)
    rg = orc.scan_bwd_state(*args, synth.f64(inp.dout), h0=h0, dhT=dhT, threads=8, **okw)
    to, tg = TOL_OUT[inp.dtype], TOL_GRAD[inp.dtype]
    assert_close(npy(out), rout, to, "out")
    for k in ("du", "ddelta", "dA", "dB", "dC"):
        assert_close(npy(g[k]), rg[k], tg, k)
    if skip:
        assert_close(npy(g["dD"]), rg["dD"], tg, "dD")
    if gate:
        assert_close(npy(g["dz"]), rg["dz"], tg, "dz")
    if opts is not None:
        assert_close(npy(g["ddelta_bias"]), rg["ddelta_bias"], tg, "ddelta_bias")
    if "hT" in parts:
        assert_close(npy(hT), rhT, to, "final_state")
    else:
        assert hT is None
    if "dh0" in parts:
        assert_close(npy(g["dinitial_state"]), rg["dh0"], tg, "dinitial_state")


def test_scan_states_zero_match_reset_only():
    """Zero initial states and zero final-state gradients give the reset-only
    entry points' results bit for bit (the same arithmetic on the same data)."""
    inp, gate, skip = _scan_case("zero-length-sequences")
    out0, g0 = run_scan_gpu(inp, gate, skip)
    d = Dev(inp)
    zeros = torch.zeros((inp.nseq, inp.D, inp.N), dtype=torch.float32, device="cuda")
    out1, ws, hT = ssp().selective_scan_pack_fwd(d.u, d.delta, d.A, d.B, d.C, d.Dp, d.z, d.pos, cu_seqlens=d.cu,
                                                 initial_state=zeros, final_state=True)
    g1 = ssp().selective_scan_pack_bwd(d.u, d.delta, d.A, d.B, d.C, d.Dp, d.z, d.pos, d.dout, ws, cu_seqlens=d.cu,
                                       initial_state=zeros, dfinal_state=zeros, dinitial_state=True)
    torch.cuda.synchronize()
    assert torch.equal(out0, out1)
    for k in ("du", "ddelta", "dz", "dA", "dB", "dC", "dD"):
        assert torch.equal(g0[k], g1[k]), k
    for s in range(inp.nseq):  # empty sequences hand on the zero state
        if inp.lengths[s] == 0:
            assert not hT[s].any() and not g1["dinitial_state"][s].any()


def test_scan_cut_across_packs():
    """One sequence cut at a pack end continues in the next pack: the second
    pack starts from the first pack's final state, and the first pack's
    backward takes the second's initial-state gradient. Per-token results
    match the uncut sequence run in one pack; parameter gradients match the
    sum over the two packs."""
    inp = synth.make_inputs(2, lengths=[900, 1500, 700], D=128, with_u=True, with_dout=True)
    cut = 900 + 611  # inside the second sequence, not on a chunk edge
    whole = Dev(inp)
    out_w, ws = ssp().selective_scan_pack_fwd(whole.u, whole.delta, whole.A, whole.B, whole.C, whole.Dp, whole.z,
                                              whole.pos)
    g_w = ssp().selective_scan_pack_bwd(whole.u, whole.delta, whole.A, whole.B, whole.C, whole.Dp, whole.z,
                                        whole.pos, whole.dout, ws)
    packs = []
    for rows, lengths in ((slice(0, cut), [900, 611]), (slice(cut, inp.T), [1500 - 611, 700])):
        import copy
        p = copy.copy(inp)
        for k in ("u", "delta", "z", "B", "C", "dout", "x"):
            setattr(p, k, getattr(inp, k)[rows].contiguous())
        p.lengths, p.cu_seqlens, p.T = lengths, synth.cu_seqlens_of(lengths), sum(lengths)
        packs.append(Dev(p))
    a, b = packs
    D, N = inp.D, inp.N
    out_a, ws_a, hT_a = ssp().selective_scan_pack_fwd(a.u, a.delta, a.A, a.B, a.C, a.Dp, a.z, a.pos,
                                                      cu_seqlens=a.cu, final_state=True)
    h0_b = torch.zeros((2, D, N), dtype=torch.float32, device="cuda")
    h0_b[0] = hT_a[1]
    out_b, ws_b, _ = ssp().selective_scan_pack_fwd(b.u, b.delta, b.A, b.B, b.C, b.Dp, b.z, b.pos, cu_seqlens=b.cu,
                                                   initial_state=h0_b)
    g_b = ssp().selective_scan_pack_bwd(b.u, b.delta, b.A, b.B, b.C, b.Dp, b.z, b.pos, b.dout, ws_b,
                                        cu_seqlens=b.cu, initial_state=h0_b, dinitial_state=True)
    dhT_a = torch.zeros((2, D, N), dtype=torch.float32, device="cuda")
    dhT_a[1] = g_b["dinitial_state"][0]
    g_a = ssp().selective_scan_pack_bwd(a.u, a.delta, a.A, a.B, a.C, a.Dp, a.z, a.pos, a.dout, ws_a,
                                        cu_seqlens=a.cu, dfinal_state=dhT_a)
    torch.cuda.synchronize()
    tol = TOL_OUT[inp.dtype]
    assert_close(npy(torch.cat([out_a, out_b])), npy(out_w), tol, "out")
    for k in ("du", "ddelta", "dz", "dB", "dC"):
        assert_close(npy(torch.cat([g_a[k], g_b[k]])), npy(g_w[k]), TOL_GRAD[inp.dtype], k)
    for k in ("dA", "dD"):
        assert_close(npy(g_a[k] + g_b[k]), npy(g_w[k]), 1e-3, k)


# ---------------------------------------------------------------------------
# conv context per sequence (conv1d_pack_*_states)
# ---------------------------------------------------------------------------

CONV_STATE_CASES = [
    # (dtype, D, W, silu, lengths, parts)
    (torch.float32, 8, 4, True, [4, 2, 3, 7], "all"),
    (torch.float32, 100, 3, True, [1, 5, 0, 130, 2, 70, 1], "all"),
    (torch.bfloat16, 512, 4, True, [700, 1, 3, 0, 322, 129, 2], "all"),
    (torch.bfloat16, 100, 4, True, [1, 5, 130, 2, 70, 1], "all"),       # per-element path
    (torch.bfloat16, 256, 2, False, [256, 128, 3, 1], "all"),
    (torch.bfloat16, 512, 4, True, [700, 1, 3, 322, 129], "initial"),
    (torch.bfloat16, 512, 4, True, [700, 1, 3, 322, 129], "gradient"),
    (torch.float32, 64, 1, True, [33, 1, 200], "all"),                 # width 1: no context at all
]


@pytest.mark.parametrize("case", range(len(CONV_STATE_CASES)))
def test_conv_states_parity(orc, case):
    dtype, D, W, silu, lengths, parts = CONV_STATE_CASES[case]
    inp = synth.make_inputs(2, lengths=lengths, D=D, dtype=dtype, with_dout=True)
    nseq = len(lengths)
    rng = np.random.default_rng(case + 50)
    w = torch.from_numpy(rng.uniform(-0.5, 0.5, (D, W)).astype(np.float32))
    b = torch.from_numpy(rng.standard_normal(D).astype(np.float32))
    ci = synth.to_dtype(rng.standard_normal((nseq, W - 1, D)), dtype) if parts in ("all", "initial") else None
    dcf = synth.to_dtype(rng.standard_normal((nseq, W - 1, D)), dtype) if parts in ("all", "gradient") else None
    d = Dev(inp)
    wd, bd = to_dev(w), to_dev(b)
    ci_d = to_dev(ci) if ci is not None else None
    dcf_d = to_dev(dcf) if dcf is not None else None
    u, cf = ssp().conv1d_pack_fwd(d.x, wd, bd, d.pos, silu=silu, cu_seqlens=d.cu, conv_initial=ci_d,
                                  conv_final=True)
    cws = nan_buffer(ssp().conv1d_pack_bwd_states_workspace_bytes(inp.T, inp.D, W, inp.nseq))
    dx, dw, db, dci = ssp().conv1d_pack_bwd(d.x, wd, bd, d.pos, d.dout, silu=silu, workspace=cws, cu_seqlens=d.cu,
                                            conv_initial=ci_d, dconv_final=dcf_d, dconv_initial=True)
    torch.cuda.synchronize()
    f = lambda t: None if t is None else synth.f64(t)
    _, ru, rcf = orc.conv_fwd_state(synth.f64(inp.x), w.double().numpy(), b.double().numpy(), inp.cu_seqlens,
                                    f(ci), silu=silu, threads=4)
    rdx, rdw, rdb, rdci = orc.conv_bwd_state(synth.f64(inp.x), w.double().numpy(), b.double().numpy(),
                                             inp.cu_seqlens, synth.f64(inp.dout), f(ci), f(dcf), silu=silu,
                                             threads=4)
    assert_close(npy(u), ru, TOL_OUT[dtype], "u")
    assert np.array_equal(npy(cf), rcf), "conv_final is a copy of inputs"
    assert_close(npy(dx), rdx, TOL_GRAD[dtype], "dx")
    assert_close(npy(dw), rdw, TOL_GRAD[dtype], "dw")
    assert_close(npy(db), rdb, TOL_GRAD[dtype], "db")
    if W > 1:
        assert_close(npy(dci), rdci, TOL_GRAD[dtype], "dconv_initial")


def test_pipeline_cut_across_packs(orc):
    """A sequence cut at a pack end continues in the next pack through both
    states: the conv context (the last W-1 inputs) and the SSM state, and
    back through their gradients. Per-token results of the two packs match
    the uncut pack; parameter gradients match the sum over the two packs; the
    cut run also matches the oracle's state-carrying pipeline."""
    lengths, cut_in = [900, 1500, 700], 611
    inp = synth.make_inputs(2, lengths=lengths, D=128, with_dout=True)
    cut = lengths[0] + cut_in
    ss = ssp()

    def run_pack(p, h0=None, ci=None, dhT=None, dcf=None):
        # through the block-level chain (pipeline.forward / backward)
        d = Dev(p)
        F = ss.forward(d.x, d.w, d.b, d.delta, d.A, d.B, d.C, d.Dp, d.z, d.cu, pos=d.pos,
                       initial_states={"ssm": h0, "conv": ci}, final_states=True)
        g = ss.backward(d.x, d.w, d.b, d.delta, d.A, d.B, d.C, d.Dp, d.z, F, d.dout,
                        dfinal_states={"ssm": dhT, "conv": dcf})
        g.update({"dinitial_state": g["dinitial_states"]["ssm"], "dci": g["dinitial_states"]["conv"],
                  "out": F["out"], "hT": F["final_states"]["ssm"], "cf": F["final_states"]["conv"]})
        return g

    import copy

    def piece(rows, lens):
        p = copy.copy(inp)
        for k in ("x", "delta", "z", "B", "C", "dout"):
            setattr(p, k, getattr(inp, k)[rows].contiguous())
        p.lengths, p.cu_seqlens, p.T = lens, synth.cu_seqlens_of(lens), sum(lens)
        return p

    pa = piece(slice(0, cut), [lengths[0], cut_in])
    pb = piece(slice(cut, inp.T), [lengths[1] - cut_in, lengths[2]])
    whole = run_pack(inp)
    D, N, W = inp.D, inp.N, inp.W
    # forward: pack a, then pack b from a's last sequence's states
    ga_fwd = run_pack(pa)
    h0_b = torch.zeros((2, D, N), dtype=torch.float32, device="cuda"); h0_b[0] = ga_fwd["hT"][1]
    ci_b = torch.zeros((2, W - 1, D), dtype=inp.x.dtype, device="cuda"); ci_b[0] = ga_fwd["cf"][1]
    gb = run_pack(pb, h0=h0_b, ci=ci_b)
    # backward: pack b first, then pack a with b's initial-state gradients
    dhT_a = torch.zeros((2, D, N), dtype=torch.float32, device="cuda"); dhT_a[1] = gb["dinitial_state"][0]
    dcf_a = torch.zeros((2, W - 1, D), dtype=inp.x.dtype, device="cuda"); dcf_a[1] = gb["dci"][0]
    ga = run_pack(pa, dhT=dhT_a, dcf=dcf_a)
    torch.cuda.synchronize()
    to, tg = TOL_OUT[inp.dtype], TOL_GRAD[inp.dtype]
    assert_close(npy(torch.cat([ga["out"], gb["out"]])), npy(whole["out"]), to, "out")
    for k in ("dx", "du", "ddelta", "dz", "dB", "dC"):
        assert_close(npy(torch.cat([ga[k], gb[k]])), npy(whole[k]), tg, k)
    for k in ("dA", "dD", "dw", "db"):
        assert_close(npy(ga[k] + gb[k]), npy(whole[k]), 1e-3, k)
    # the second pack against the oracle's state-carrying pipeline
    f64 = synth.f64
    _, u_o, _ = orc.conv_fwd_state(f64(pb.x), f64(pb.w), f64(pb.b), pb.cu_seqlens, f64(ci_b), threads=8)
    _, out_o, _ = orc.scan_fwd_state(u_o, f64(pb.delta), f64(pb.A), f64(pb.B), f64(pb.C), f64(pb.Dp), f64(pb.z),
                                     pb.cu_seqlens, h0=npy(h0_b), threads=8)
    assert_close(npy(gb["out"]), out_o, to, "out (oracle)")


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
def test_pipeline_step_map_with_states(orc, dtype):
    """The block chain with the step map softplus(delta + bias), the gate floor
    and both carried states at once, forward and backward, against the
    oracle's state-carrying functions run in the same order."""
    lengths = [300, 1, 200, 513]
    inp = synth.make_inputs(2, lengths=lengths, D=96, dtype=dtype, with_dout=True)
    nseq, D, N, W = inp.nseq, inp.D, inp.N, inp.W
    rng = np.random.default_rng(31)
    bias = (rng.standard_normal(D) * 0.2).astype(np.float32)
    h0 = (rng.standard_normal((nseq, D, N)) * 0.5).astype(np.float32)
    dhT = rng.standard_normal((nseq, D, N)).astype(np.float32)
    ci = synth.to_dtype(rng.standard_normal((nseq, W - 1, D)), dtype)
    dcf = synth.to_dtype(rng.standard_normal((nseq, W - 1, D)), dtype)
    floor = 0.05
    d = Dev(inp)
    F = ssp().forward(d.x, d.w, d.b, d.delta, d.A, d.B, d.C, d.Dp, d.z, d.cu, pos=d.pos,
                      initial_states={"ssm": to_dev(torch.from_numpy(h0)), "conv": to_dev(ci)}, final_states=True,
                      delta_bias=to_dev(torch.from_numpy(bias)), delta_softplus=True, gate_floor=floor)
    G = ssp().backward(d.x, d.w, d.b, d.delta, d.A, d.B, d.C, d.Dp, d.z, F, d.dout,
                       dfinal_states={"ssm": to_dev(torch.from_numpy(dhT)), "conv": to_dev(dcf)})
    torch.cuda.synchronize()
    f64, cu = synth.f64, inp.cu_seqlens
    ext = dict(delta_bias=bias.astype(np.float64), delta_softplus=True, gate_floor=floor)
    x, w, b, z, dout = f64(inp.x), f64(inp.w), f64(inp.b), f64(inp.z), f64(inp.dout)
    delta, A, B, C, Dp = f64(inp.delta), f64(inp.A), f64(inp.B), f64(inp.C), f64(inp.Dp)
    _, u, cf = orc.conv_fwd_state(x, w, b, cu, f64(ci), threads=8)
    _, out, hT = orc.scan_fwd_state(u, delta, A, B, C, Dp, z, cu, h0=h0.astype(np.float64), threads=8, **ext)
    R = orc.scan_bwd_state(u, delta, A, B, C, Dp, z, cu, dout, h0=h0.astype(np.float64),
                           dhT=dhT.astype(np.float64), threads=8, **ext)
    dx, dw, db, dci = orc.conv_bwd_state(x, w, b, cu, R["du"], f64(ci), f64(dcf), threads=8)
    to, tg = TOL_OUT[dtype], TOL_GRAD[dtype]
    assert_close(npy(F["u"]), u, to, "u")
    assert_close(npy(F["out"]), out, to, "out")
    assert_close(npy(F["final_states"]["ssm"]), hT, to, "final ssm state")
    assert np.array_equal(npy(F["final_states"]["conv"]), cf), "final conv context"
    for k in ("du", "ddelta", "dz", "dA", "dB", "dC", "dD", "ddelta_bias"):
        assert_close(npy(G[k]), R[k], tg, k)
    assert_close(npy(G["dx"]), dx, tg, "dx")
    assert_close(npy(G["dw"]), dw, tg, "dw")
    assert_close(npy(G["db"]), db, tg, "db")
    assert_close(npy(G["dinitial_states"]["ssm"]), R["dh0"], tg, "dinitial ssm state")
    assert_close(npy(G["dinitial_states"]["conv"]), dci, tg, "dinitial conv context")


def test_states_empty_pack():
    """No tokens at all (every sequence empty): final states are the initial
    ones and the initial-state gradients are the final-state ones, for the
    SSM state and the conv context; the parameter sums are zero."""
    ss = ssp()
    nseq, D, N, W = 3, 64, 16, 4
    cu = torch.zeros(nseq + 1, dtype=torch.int32, device="cuda")
    g = torch.Generator().manual_seed(9)
    h0 = torch.randn(nseq, D, N, generator=g).cuda()
    dhT = torch.randn(nseq, D, N, generator=g).cuda()
    ci = torch.randn(nseq, W - 1, D, generator=g).to(torch.bfloat16).cuda()
    dcf = torch.randn(nseq, W - 1, D, generator=g).to(torch.bfloat16).cuda()
    e2 = lambda *s: torch.empty(*s, dtype=torch.bfloat16, device="cuda")
    x, z, delta = e2(0, D), e2(0, D), e2(0, D)
    B, C = e2(0, N), e2(0, N)
    A = -torch.ones(D, N, device="cuda")
    Dp = torch.ones(D, device="cuda")
    w = torch.ones(D, W, device="cuda")
    b = torch.zeros(D, device="cuda")
    pos = torch.empty(0, dtype=torch.int32, device="cuda")
    u, cf = ss.conv1d_pack_fwd(x, w, b, pos, cu_seqlens=cu, conv_initial=ci, conv_final=True)
    out, ws, hT = ss.selective_scan_pack_fwd(u, delta, A, B, C, Dp, z, pos, cu_seqlens=cu, initial_state=h0,
                                             final_state=True)
    gr = ss.selective_scan_pack_bwd(u, delta, A, B, C, Dp, z, pos, e2(0, D), ws, cu_seqlens=cu, initial_state=h0,
                                    dfinal_state=dhT, dinitial_state=True)
    dx, dw, db, dci = ss.conv1d_pack_bwd(x, w, b, pos, gr["du"], cu_seqlens=cu, conv_initial=ci, dconv_final=dcf,
                                         dconv_initial=True)
    torch.cuda.synchronize()
    assert torch.equal(hT, h0) and torch.equal(cf, ci)
    assert torch.equal(gr["dinitial_state"], dhT) and torch.equal(dci, dcf)
    assert not gr["dA"].any() and not gr["dD"].any() and not dw.any() and not db.any()


def test_state_outputs_need_cu_seqlens():
    """Asking the binding for a state output without cu_seqlens is a clear
    ValueError raised before any launch."""
    import selective_state_space_varlen_amd as ssp
    inp = synth.make_inputs(2, lengths=[5, 7], D=8, N=4, with_dout=True, with_u=True)
    d = Dev(inp)
    with pytest.raises(ValueError, match="need cu_seqlens"):
        ssp.selective_scan_pack_fwd(d.u, d.delta, d.A, d.B, d.C, d.Dp, d.z, d.pos, final_state=True)
    _, ws = ssp.selective_scan_pack_fwd(d.u, d.delta, d.A, d.B, d.C, d.Dp, d.z, d.pos)
    with pytest.raises(ValueError, match="need cu_seqlens"):
        ssp.selective_scan_pack_bwd(d.u, d.delta, d.A, d.B, d.C, d.Dp, d.z, d.pos, d.dout, ws, dinitial_state=True)
    with pytest.raises(ValueError, match="need cu_seqlens"):
        ssp.conv1d_pack_fwd(d.x, d.w, d.b, d.pos, conv_final=True)
    torch.cuda.synchronize()


def test_empty_input_plain_entry_points():
    """T = 0 through the reset-only entry points: nothing to launch for the
    per-token outputs, and the parameter sums (dw, db, dA, dD) are written as
    zeros (their buffers start as NaN)."""
    ss = ssp()
    D, N, W = 96, 16, 4
    e2 = lambda *s: torch.empty(*s, dtype=torch.bfloat16, device="cuda")
    nan = lambda *s: torch.full(s, float("nan"), dtype=torch.float32, device="cuda")
    x, z, delta, dout = e2(0, D), e2(0, D), e2(0, D), e2(0, D)
    B, C = e2(0, N), e2(0, N)
    A = -torch.ones(D, N, device="cuda")
    Dp = torch.ones(D, device="cuda")
    w = torch.ones(D, W, device="cuda")
    b = torch.zeros(D, device="cuda")
    cu = torch.zeros(2, dtype=torch.int32, device="cuda")
    pos, _, err = ss.varlen_pack_indices(cu, 0)
    u = ss.conv1d_pack_fwd(x, w, b, pos)
    out, ws = ss.selective_scan_pack_fwd(u, delta, A, B, C, Dp, z, pos)
    g = {"du": e2(0, D), "ddelta": e2(0, D), "dz": e2(0, D), "dA": nan(D, N), "dB": nan(0, N), "dC": nan(0, N),
         "dD": nan(D)}
    ss.selective_scan_pack_bwd(u, delta, A, B, C, Dp, z, pos, dout, ws, out=g)
    dw, db = nan(D, W), nan(D)
    ss.conv1d_pack_bwd(x, w, b, pos, g["du"], out=(e2(0, D), dw, db))
    torch.cuda.synchronize()
    assert int(err.item()) == 0 and out.shape == (0, D)
    for name, t in (("dA", g["dA"]), ("dD", g["dD"]), ("dw", dw), ("db", db)):
        assert torch.equal(t, torch.zeros_like(t)), name


# numerical regimes at the edges of the recurrence: no decay (A = 0, the
# state is a running sum), decays that underflow to zero, steps so small the
# state keeps thousands of tokens of memory, and softplus far into its tails
REGIMES = {
    "no-decay-fp32": dict(dtype=torch.float32, A=0.0, delta=(0.01, 0.1)),
    "underflowing-decay-fp32": dict(dtype=torch.float32, A=-16.0, delta=(8.0, 12.0)),
    "long-memory-bf16": dict(dtype=torch.bfloat16, A=-1.0, delta=(1e-4, 5e-4)),
    "softplus-tails-bf16": dict(dtype=torch.bfloat16, A=-1.0, raw=(-40.0, 40.0)),
    "mixed-sign-A-fp32": dict(dtype=torch.float32, A="mixed", delta=(0.001, 0.01)),
}


@pytest.mark.parametrize("name", list(REGIMES))
def test_scan_numerical_regimes(orc, name):
    spec = REGIMES[name]
    inp = synth.make_inputs(2, lengths=[3000, 17, 1, 500], D=64, dtype=spec["dtype"], with_u=True,
                            with_dout=True)
    rng = np.random.default_rng(11)
    T, D, N = inp.T, inp.D, inp.N
    if spec["A"] == "mixed":
        # small positive A too: a growing state over a short memory
        A = rng.uniform(-2.0, 0.5, (D, N)).astype(np.float32)
    else:
        A = np.full((D, N), spec["A"], dtype=np.float32)
    inp.A = torch.from_numpy(A)
    kw, okw = {}, {}
    if "raw" in spec:
        lo, hi = spec["raw"]
        raw = rng.uniform(lo, hi, (T, D))
        inp.delta = synth.to_dtype(raw, inp.dtype)
        kw = dict(delta_softplus=True)
        okw = dict(delta_softplus=True)
    else:
        lo, hi = spec["delta"]
        inp.delta = synth.to_dtype(rng.uniform(lo, hi, (T, D)), inp.dtype)
    d = Dev(inp)
    out, ws = ssp().selective_scan_pack_fwd(d.u, d.delta, d.A, d.B, d.C, d.Dp, d.z, d.pos, **kw)
    g = ssp().selective_scan_pack_bwd(d.u, d.delta, d.A, d.B, d.C, d.Dp, d.z, d.pos, d.dout, ws, **kw)
    torch.cuda.synchronize()
    pos, _ = orc.pack_indices(inp.cu_seqlens, inp.T)
    args = (synth.f64(inp.u), synth.f64(inp.delta), synth.f64(inp.A), synth.f64(inp.B), synth.f64(inp.C),
            synth.f64(inp.Dp), synth.f64(inp.z), pos)
    _, rout = orc.scan_fwd(*args, threads=8, **okw)
    rg = orc.scan_bwd(*args, synth.f64(inp.dout), threads=8, **okw)
    to, tg = TOL_OUT[inp.dtype], TOL_GRAD[inp.dtype]
    assert np.all(np.isfinite(npy(out)))
    assert_close(npy(out), rout, to, "out")
    for k in ("du", "ddelta", "dA", "dB", "dC", "dD", "dz"):
        assert_close(npy(g[k]), rg[k], tg, k)


def test_many_sequences_with_states(orc):
    """40 000 sequences (empty, single-token and short ones mixed) with both
    carried states and the step map, through the block chain: the head's
    sequence lookup, the empty-sequence pass-through and the per-sequence
    conv contexts at scale, against the oracle (each operator on the stored
    inputs it consumed)."""
    rng = np.random.default_rng(91)
    lengths = [int(v) for v in rng.choice([0, 1, 2, 3, 5, 9], size=40000, p=[0.2, 0.3, 0.2, 0.1, 0.1, 0.1])]
    inp = synth.make_inputs(2, lengths=lengths, D=64, N=16, dtype=torch.float32, with_dout=True)
    nseq, D, N, W = inp.nseq, inp.D, inp.N, inp.W
    print(f"[many] {nseq} sequences, T={inp.T}", flush=True)
    bias = (rng.standard_normal(D) * 0.2).astype(np.float32)
    h0 = (rng.standard_normal((nseq, D, N)) * 0.5).astype(np.float32)
    dhT = rng.standard_normal((nseq, D, N)).astype(np.float32)
    ci = synth.to_dtype(rng.standard_normal((nseq, W - 1, D)), inp.dtype)
    dcf = synth.to_dtype(rng.standard_normal((nseq, W - 1, D)), inp.dtype)
    d = Dev(inp)
    s = ssp()
    F = s.forward(d.x, d.w, d.b, d.delta, d.A, d.B, d.C, d.Dp, d.z, d.cu, pos=d.pos,
                  initial_states={"ssm": to_dev(torch.from_numpy(h0)), "conv": to_dev(ci)}, final_states=True,
                  delta_bias=to_dev(torch.from_numpy(bias)), delta_softplus=True, gate_floor=0.05)
    G = s.backward(d.x, d.w, d.b, d.delta, d.A, d.B, d.C, d.Dp, d.z, F, d.dout,
                   dfinal_states={"ssm": to_dev(torch.from_numpy(dhT)), "conv": to_dev(dcf)})
    torch.cuda.synchronize()
    f64, cu = synth.f64, inp.cu_seqlens
    ext = dict(delta_bias=bias.astype(np.float64), delta_softplus=True, gate_floor=0.05)
    x, w, b, z, dout = f64(inp.x), f64(inp.w), f64(inp.b), f64(inp.z), f64(inp.dout)
    delta, A, B, C, Dp = f64(inp.delta), f64(inp.A), f64(inp.B), f64(inp.C), f64(inp.Dp)
    to, tg = TOL_OUT[inp.dtype], TOL_GRAD[inp.dtype]
    _, u, cf = orc.conv_fwd_state(x, w, b, cu, f64(ci), threads=8)
    assert_close(npy(F["u"]), u, to, "u")
    assert np.array_equal(npy(F["final_states"]["conv"]), cf), "final conv context"
    u = npy(F["u"]).astype(np.float64)
    _, out, hT = orc.scan_fwd_state(u, delta, A, B, C, Dp, z, cu, h0=h0.astype(np.float64), threads=8, **ext)
    R = orc.scan_bwd_state(u, delta, A, B, C, Dp, z, cu, dout, h0=h0.astype(np.float64),
                           dhT=dhT.astype(np.float64), threads=8, **ext)
    assert_close(npy(F["out"]), out, to, "out")
    assert_close(npy(F["final_states"]["ssm"]), hT, to, "final ssm state")
    for k in ("du", "ddelta", "dz", "dA", "dB", "dC", "dD", "ddelta_bias"):
        assert_close(npy(G[k]), R[k], tg, k)
    assert_close(npy(G["dinitial_states"]["ssm"]), R["dh0"], tg, "dinitial ssm state")
    dx, dw, db, dci = orc.conv_bwd_state(x, w, b, cu, npy(G["du"]).astype(np.float64), f64(ci), f64(dcf), threads=8)
    assert_close(npy(G["dx"]), dx, tg, "dx")
    assert_close(npy(G["dw"]), dw, tg, "dw")
    assert_close(npy(G["db"]), db, tg, "db")
    assert_close(npy(G["dinitial_states"]["conv"]), dci, tg, "dinitial conv context")
