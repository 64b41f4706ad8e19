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
