"""Small random networks and random trees for property tests.

Extents are drawn from a small set that includes 1 and non-powers of two so
that index mistakes (a swapped stride, a transposed operand) change values.
"""

from __future__ import annotations

from typing import Optional, Sequence

import numpy as np

from .network import Network, Tree
from .sweep import complex_gaussian


def random_network(rng: np.random.Generator, n_leaves: int, n_closed: int, n_open: int,
                   extent_choices: Sequence[int] = (1, 2, 3, 4, 5), max_leaf_elems: int = 4096,
                   with_data: bool = True) -> Network:
    """Closed modes join two distinct random leaves; open modes hang on one
    leaf each.  Leaf mode orders and the output order are random."""
    leaves = [[] for _ in range(n_leaves)]
    extents = []
    for _ in range(n_closed):
        if n_leaves < 2:
            break
        a, b = rng.choice(n_leaves, size=2, replace=False)
        x = len(extents)
        extents.append(int(rng.choice(extent_choices)))
        leaves[a].append(x)
        leaves[b].append(x)
    open_modes = []
    for _ in range(n_open):
        a = int(rng.integers(n_leaves))
        x = len(extents)
        extents.append(int(rng.choice(extent_choices)))
        leaves[a].append(x)
        open_modes.append(x)
    ext = np.array(extents, dtype=np.int64)
    # keep leaves small: shrink extents of modes on oversized leaves to 1
    for l in leaves:
        while int(np.prod([ext[x] for x in l], dtype=np.int64)) > max_leaf_elems:
            big = max(l, key=lambda x: ext[x])
            ext[big] = 1
    leaves = [list(np.array(l)[rng.permutation(len(l))]) if l else [] for l in leaves]
    leaves = [[int(x) for x in l] for l in leaves]
    out = [int(x) for x in np.array(open_modes, dtype=np.int64)[rng.permutation(len(open_modes))]]
    data = None
    if with_data:
        data = [complex_gaussian(rng, tuple(int(ext[x]) for x in l)) for l in leaves]
    return Network(ext, leaves, out, data, name="random")


def random_tree(rng: np.random.Generator, n_leaves: int) -> Tree:
    """Merge two uniformly random live tensors until one is left."""
    live = list(range(n_leaves))
    lhs, rhs = [], []
    nxt = n_leaves
    while len(live) > 1:
        i, j = rng.choice(len(live), size=2, replace=False)
        a, b = live[i], live[j]
        for idx in sorted((i, j), reverse=True):
            live.pop(idx)
        lhs.append(int(a))
        rhs.append(int(b))
        live.append(nxt)
        nxt += 1
    return Tree(lhs, rhs)
