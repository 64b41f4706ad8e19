"""Reference packer: which sequences share a pack of `capacity` tokens.

TEST INFRASTRUCTURE ONLY (tests, the smoke check and the benchmark's CPU
baseline may use it; the product path never does). Plain Python loops,
written from Shanghai AI Lab's article on packed variable-length Mamba-1
training (gitcode.csdn.net/69d8cc1b54b52172bc6872cb.html), section "结论与讨论":

  * sequential: take sequences in arrival order and seal the pack when the
    next one does not fit;
  * local greedy: sort a window of pending sequences, then pack them
    greedily. The article does not spell out the greedy rule; this takes the
    plainest one, first-fit decreasing inside each window of `window`
    sequences (longest first, ties in arrival order; each goes into the first
    of the window's packs with room, else a new pack), and seals the window's
    packs when the window ends.

A sequence longer than the capacity cannot be packed (ValueError).
Returns (order, cu_seqlens, pack_bounds, max_seqlen, padding_tokens):
order lists sequence indices pack by pack; pack p holds
order[pack_bounds[p]:pack_bounds[p+1]]; cu_seqlens are the cumulative
lengths along `order` (the packed token layout without padding);
padding_tokens = n_packs * capacity - sum(lengths).
"""
from __future__ import annotations

SEQUENTIAL, LOCAL_GREEDY = 0, 1


def plan(lengths, capacity: int, strategy: int, window: int = 1):
    lengths = [int(v) for v in lengths]
    if capacity < 1:
        raise ValueError("capacity must be positive")
    for v in lengths:
        if v < 0 or v > capacity:
            raise ValueError(f"length {v} does not fit a pack of {capacity}")
    packs = []  # lists of sequence indices
    if strategy == SEQUENTIAL:
        load = 0
        for i, v in enumerate(lengths):
            if not packs or load + v > capacity:
                packs.append([])
                load = 0
            packs[-1].append(i)
            load += v
    elif strategy == LOCAL_GREEDY:
        if window < 1:
            raise ValueError("window must be positive")
        for w0 in range(0, len(lengths), window):
            idx = list(range(w0, min(w0 + window, len(lengths))))
            idx.sort(key=lambda i: -lengths[i])  # stable: ties keep arrival order
            mine, loads = [], []
            for i in idx:
                for p in range(len(mine)):
                    if loads[p] + lengths[i] <= capacity:
                        mine[p].append(i)
                        loads[p] += lengths[i]
                        break
                else:
                    mine.append([i])
                    loads.append(lengths[i])
            packs.extend(mine)
    else:
        raise ValueError(f"unknown strategy {strategy}")
    order = [i for p in packs for i in p]
    cu = [0]
    for i in order:
        cu.append(cu[-1] + lengths[i])
    bounds = [0]
    for p in packs:
        bounds.append(bounds[-1] + len(p))
    max_seqlen = [max([lengths[i] for i in p], default=0) for p in packs]
    padding = len(packs) * capacity - sum(lengths)
    return order, cu, bounds, max_seqlen, padding
