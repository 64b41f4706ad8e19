"""Pins of the reference packer (oracle/pack_plan.py), each a function of a
`plan` callable with the oracle's signature, so the planted-mistake test can
run all of them on a mutated copy.

What fixes the answers (Shanghai AI Lab article on packed Mamba-1 training,
section "结论与讨论", describes the two strategies; the rest is bin-packing
mathematics):
  * hand-worked small cases;
  * structure: every sequence placed once, no pack over capacity, sequential
    packs are contiguous runs sealed only when the next sequence does not fit,
    first-fit decreasing places each sequence after every earlier pack of its
    window had run out of room for it;
  * closed forms for equal lengths;
  * brute force on tiny inputs: the optimum pack count OPT from all set
    partitions, with next-fit <= 2 OPT - 1 and first-fit decreasing
    <= 11/9 OPT + 6/9 (Dosa, 2007), both >= OPT.
"""
from __future__ import annotations

import math

import numpy as np

SEQ, GREEDY = 0, 1


def _packs(res):
    order, cu, bounds, maxlen, pad = res
    return [order[bounds[p]:bounds[p + 1]] for p in range(len(bounds) - 1)]


def _check_layout(res, lengths, cap):
    order, cu, bounds, maxlen, pad = res
    assert sorted(order) == list(range(len(lengths)))
    assert bounds[0] == 0 and bounds[-1] == len(lengths)
    assert all(bounds[p] < bounds[p + 1] for p in range(len(bounds) - 1)), "empty pack"
    assert cu[0] == 0 and len(cu) == len(lengths) + 1
    assert all(cu[k + 1] - cu[k] == lengths[order[k]] for k in range(len(order)))
    packs = _packs(res)
    for p, ids in enumerate(packs):
        assert sum(lengths[i] for i in ids) <= cap
        assert maxlen[p] == max(lengths[i] for i in ids)
    assert pad == len(packs) * cap - sum(lengths)
    assert len(packs) >= math.ceil(sum(lengths) / cap)


def check_hand_worked(plan):
    L = [5, 4, 3, 2, 6]
    # arrival order into 8: [5] (4 does not fit), [4, 3] (2 does not fit), [2, 6]
    r = plan(L, 8, SEQ)
    assert _packs(r) == [[0], [1, 2], [3, 4]]
    assert r[1] == [0, 5, 9, 12, 14, 20] and r[3] == [5, 4, 6] and r[4] == 4
    # one window of 5, longest first: 6 -> new, 5 -> new, 4 -> new, 3 -> pack of 5,
    # 2 -> pack of 6
    r = plan(L, 8, GREEDY, 5)
    assert _packs(r) == [[4, 3], [0, 2], [1]]
    assert r[1] == [0, 6, 8, 13, 16, 20] and r[3] == [6, 5, 4] and r[4] == 4
    # windows of 2: {5, 4} -> [5], [4]; {3, 2} -> [3, 2]; {6} -> [6]
    r = plan(L, 8, GREEDY, 2)
    assert _packs(r) == [[0], [1], [2, 3], [4]] and r[4] == 12
    # ties keep arrival order; an exact fit is a fit
    r = plan([3, 5, 3, 5], 8, GREEDY, 4)
    assert _packs(r) == [[1, 0], [3, 2]] and r[4] == 0
    r = plan([4, 4, 8, 1], 8, SEQ)
    assert _packs(r) == [[0, 1], [2], [3]] and r[4] == 7


def check_edges(plan):
    assert plan([], 8, SEQ) == ([], [0], [0], [], 0)
    assert plan([], 8, GREEDY, 3) == ([], [0], [0], [], 0)
    for s, w in ((SEQ, 1), (GREEDY, 1), (GREEDY, 7)):
        r = plan([8], 8, s, w)
        assert _packs(r) == [[0]] and r[4] == 0
    # a window of one seals every sequence into its own pack
    r = plan([1, 1, 1], 8, GREEDY, 1)
    assert _packs(r) == [[0], [1], [2]] and r[4] == 21
    for bad in (([9], 8), ([-1], 8), ([1], 0)):
        for s in (SEQ, GREEDY):
            try:
                plan(bad[0], bad[1], s, 2)
            except ValueError:
                pass
            else:
                raise AssertionError(f"accepted {bad}")


def check_equal_lengths_closed_form(plan):
    for n, L, cap in ((17, 3, 10), (40, 7, 64), (9, 5, 5), (12, 1, 4)):
        per = cap // L
        r = plan([L] * n, cap, SEQ)
        assert len(r[2]) - 1 == math.ceil(n / per)
        for w in (1, 4, 5, n):
            r = plan([L] * n, cap, GREEDY, w)
            want = sum(math.ceil(min(w, n - w0) / per) for w0 in range(0, n, w))
            assert len(r[2]) - 1 == want


def check_structure_random(plan):
    rng = np.random.default_rng(7)
    for trial in range(60):
        cap = int(rng.integers(4, 40))
        n = int(rng.integers(0, 30))
        L = [int(v) for v in rng.integers(0, cap + 1, n)]
        r = plan(L, cap, SEQ)
        _check_layout(r, L, cap)
        packs = _packs(r)
        assert [i for p in packs for i in p] == list(range(n))  # arrival order kept
        for p in range(len(packs) - 1):
            load = sum(L[i] for i in packs[p])
            assert load + L[packs[p + 1][0]] > cap  # sealed only when the next does not fit
        w = int(rng.integers(1, 12))
        r = plan(L, cap, GREEDY, w)
        _check_layout(r, L, cap)
        packs = _packs(r)
        owner = {i: p for p, ids in enumerate(packs) for i in ids}
        for p, ids in enumerate(packs):
            win = ids[0] // w
            assert all(i // w == win for i in ids), "pack spans windows"
            lens = [L[i] for i in ids]
            assert lens == sorted(lens, reverse=True)
            for i in ids:
                for q in range(p):
                    if packs[q][0] // w == win:
                        assert sum(L[j] for j in packs[q]) + L[i] > cap, "first fit skipped a pack with room"
        assert sorted(owner) == list(range(n))
        # packs of one window come out in window order
        firsts = [ids[0] // w for ids in packs]
        assert firsts == sorted(firsts)


def _opt(lengths, cap):
    """Fewest packs over all set partitions (brute force, tiny inputs)."""
    best = [len(lengths)]

    def rec(k, loads):
        if len(loads) >= best[0]:
            return
        if k == len(lengths):
            best[0] = len(loads)
            return
        for p in range(len(loads)):
            if loads[p] + lengths[k] <= cap:
                loads[p] += lengths[k]
                rec(k + 1, loads)
                loads[p] -= lengths[k]
        loads.append(lengths[k])
        rec(k + 1, loads)
        loads.pop()

    rec(0, [])
    return best[0]


def check_brute_force_bounds(plan):
    rng = np.random.default_rng(11)
    hits_ffd_opt = 0
    for trial in range(150):
        cap = int(rng.integers(5, 20))
        n = int(rng.integers(1, 9))
        L = [int(v) for v in rng.integers(1, cap + 1, n)]
        opt = _opt(L, cap)
        nf = len(plan(L, cap, SEQ)[2]) - 1
        ffd = len(plan(L, cap, GREEDY, n)[2]) - 1
        assert opt <= nf <= 2 * opt - 1
        assert opt <= ffd and 9 * ffd <= 11 * opt + 6
        hits_ffd_opt += ffd == opt
    assert hits_ffd_opt > 100  # first-fit decreasing is optimal on most tiny inputs
    # a case where arrival order costs a pack that sorting saves
    L, cap = [2, 5, 3, 6], 8
    assert _opt(L, cap) == 2 and len(plan(L, cap, SEQ)[2]) - 1 == 3
    assert len(plan(L, cap, GREEDY, 4)[2]) - 1 == 2


ALL_CHECKS = [check_hand_worked, check_edges, check_equal_lengths_closed_form,
              check_structure_random, check_brute_force_bounds]
