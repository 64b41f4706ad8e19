"""CPU tests of the sequence packer.

The reference packer (oracle/pack_plan.py) is pinned by tests/pack_plan_checks.py;
a planted-mistake test requires each plausible slip in it to fail a pin.
"""
from __future__ import annotations

import types

import pytest

from oracle import pack_plan as ref
from tests import pack_plan_checks as pc


@pytest.mark.parametrize("check", pc.ALL_CHECKS, ids=lambda f: f.__name__)
def test_pin(check):
    check(ref.plan)


# (name, text as written, planted mistake)
MUTATIONS = [
    ("sequential: seals on an exact fit", "if not packs or load + v > capacity:", "if not packs or load + v >= capacity:"),
    ("sequential: load not reset on a new pack", "packs.append([])\n                load = 0\n", "packs.append([])\n"),
    ("greedy: sorts ascending", "idx.sort(key=lambda i: -lengths[i])", "idx.sort(key=lambda i: lengths[i])"),
    ("greedy: ties in reverse arrival order", "idx.sort(key=lambda i: -lengths[i])",
     "idx.sort(key=lambda i: (-lengths[i], -i))"),
    ("greedy: exact fit rejected", "if loads[p] + lengths[i] <= capacity:", "if loads[p] + lengths[i] < capacity:"),
    ("greedy: best fit instead of first fit", "for p in range(len(mine)):", "for p in sorted(range(len(mine)), key=lambda q: -loads[q]):"),
    ("greedy: windows overlap", "idx = list(range(w0, min(w0 + window, len(lengths))))",
     "idx = list(range(w0, min(w0 + window + 1, len(lengths))))"),
    ("layout: cu_seqlens in arrival order", "for i in order:\n        cu.append", "for i in range(len(lengths)):\n        cu.append"),
    ("layout: padding counts one pack too few", "padding = len(packs) * capacity - sum(lengths)",
     "padding = (len(packs) - 1) * capacity - sum(lengths)"),
    ("check: long sequence accepted", "if v < 0 or v > capacity:", "if v < 0 or v > 2 * capacity:"),
]


@pytest.mark.parametrize("name,orig,planted", MUTATIONS, ids=[m[0] for m in MUTATIONS])
def test_planted_mistake_is_caught(name, orig, planted):
    src = open(ref.__file__).read()
    assert src.count(orig) == 1, f"mutation anchor not unique/found: {name}"
    mod = types.ModuleType("pack_plan_mutant")
    exec(compile(src.replace(orig, planted), "pack_plan_mutant", "exec"), mod.__dict__)
    failed = []
    for check in pc.ALL_CHECKS:
        try:
            check(mod.plan)
        except (AssertionError, ValueError, IndexError, TypeError):
            failed.append(check.__name__)
    assert failed, f"no pin caught: {name}"


# --- the library's packer (host code in libssmpack.so) against the reference ---

def _lib_plan(lengths, capacity, strategy, window=1):
    """varlen_pack_plan with the reference's signature and return shape."""
    import selective_state_space_varlen_amd as S
    try:
        p = S.varlen_pack_plan(lengths, capacity, strategy, window)
    except S.SsmpError as e:
        raise ValueError(str(e)) from e
    return (p.order.tolist(), p.cu_seqlens.tolist(), p.pack_bounds.tolist(), p.max_seqlen.tolist(), p.padding)


@pytest.mark.parametrize("check", pc.ALL_CHECKS, ids=lambda f: f.__name__)
def test_library_meets_pins(check):
    check(_lib_plan)


def test_library_matches_reference_exactly():
    import numpy as np
    rng = np.random.default_rng(3)
    for trial in range(300):
        cap = int(rng.integers(1, 64))
        n = int(rng.integers(0, 200))
        L = [int(v) for v in rng.integers(0, cap + 1, n)]
        for strategy, window in ((0, 1), (1, 1), (1, int(rng.integers(1, 40))), (1, max(n, 1)), (1, 10**6)):
            assert _lib_plan(L, cap, strategy, window) == ref.plan(L, cap, strategy, window), (trial, strategy, window)


@pytest.mark.parametrize("workload,capacity", [(1, 4096), (2, 4096), (3, 32768)])
def test_library_matches_reference_on_length_mixes(workload, capacity):
    import synth
    L = synth.document_lengths(workload, 3000, seed=workload)
    for strategy, window in ((0, 1), (1, 64), (1, 1024), (1, 3000)):
        assert _lib_plan(L, capacity, strategy, window) == ref.plan(L, capacity, strategy, window)


def test_library_errors():
    import numpy as np
    import selective_state_space_varlen_amd as S
    from selective_state_space_varlen_amd import binding as bnd
    cases = [(([9], 8, 0, 1), 2), (([-1], 8, 1, 2), 2), (([1], 0, 0, 1), 2), (([1], 8, 1, 0), 2),
             (([1], 8, 7, 1), 4)]
    for args, status in cases:
        with pytest.raises(S.SsmpError) as e:
            S.varlen_pack_plan(*args)
        assert e.value.status == status
    # the int32 token total of cu_seqlens must not overflow
    with pytest.raises(S.SsmpError) as e:
        S.varlen_pack_plan(np.full(3, 2**30, np.int64), 2**30, 0)
    assert e.value.status == 2
    # NULL outputs are refused before anything is touched
    lib = bnd.load()
    ln = np.array([1, 2], np.int32)
    assert lib.varlen_pack_plan(ln.ctypes.data_as(bnd._c_vp), 2, 8, 0, 1, None, None, None, None, None, None) == 1
