"""CPU tests of the seeded input generator (shapes, length mixes, determinism)."""
import numpy as np
import torch

import synth


def test_workload0_is_the_pages_example():
    inp = synth.make_inputs(0)
    assert inp.lengths == [4, 2, 3, 7] and inp.T == 16 and inp.D == 8 and inp.N == 4
    assert inp.cu_seqlens.tolist() == [0, 4, 6, 9, 16]
    assert inp.x.dtype == torch.float32
    assert torch.equal(inp.A[3], -torch.arange(1, 5, dtype=torch.float32))
    assert bool((inp.delta > 0).all())


def test_length_mixes():
    for wl in (1, 2, 3):
        spec = synth.WORKLOADS[wl]
        inp = synth.make_inputs(wl, D=8)
        assert inp.T == spec.n_packs * spec.pack_len
        cu = inp.cu_seqlens
        # every pack boundary is a sequence boundary
        for p in range(spec.n_packs + 1):
            assert p * spec.pack_len in set(cu.tolist())
        L = np.diff(cu)
        assert L.min() >= 1
        if wl == 2:
            inner = [l for i, l in enumerate(L)]
            assert max(inner) <= 2048
        if wl == 3:
            assert int((L == 1).sum()) >= spec.n_packs


def test_deterministic_and_bf16():
    a = synth.make_inputs(1, n_packs=1, D=16)
    b = synth.make_inputs(1, n_packs=1, D=16)
    assert a.lengths == b.lengths and torch.equal(a.x, b.x) and torch.equal(a.delta, b.delta)
    assert a.x.dtype == torch.bfloat16
    # bf16 values widen exactly to fp64
    assert np.array_equal(synth.f64(a.x), a.x.float().double().numpy())
