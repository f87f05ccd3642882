"""Square-lattice (PEPS-style) partition-function networks.

Sites (i, j) of an L x L lattice carry one tensor each; every nearest-
neighbour bond has extent D.  Site modes are declared in the order
[up, left, right, down], skipping those on the lattice edge.  Bond labels:
horizontal bond h(i, j) joins (i, j)-(i, j+1), vertical bond v(i, j) joins
(i, j)-(i+1, j).  Entries are U[0, 1) float32, scaled by 1 / (0.5 * D^(deg/2))
so that E[Z] = 1, promoted to complex64 with zero imaginary part.  There are
no open modes; the contraction yields the scalar Z.

The page ("Parallelizing Large-Scale Tensor Network Contraction on Multiple
GPUs", section 5.1) names exact 2-D PEPS contraction as a target workload but
gives no instance; this is the synthetic stand-in.
"""

from __future__ import annotations

from typing import Callable, Optional

import numpy as np

from .network import Network, Tree, caterpillar


def site_modes(L: int, i: int, j: int):
    """Bond labels of site (i, j) in [up, left, right, down] order."""
    nh = L * (L - 1)
    h = lambda a, b: a * (L - 1) + b           # 0 .. nh-1
    v = lambda a, b: nh + a * L + b            # nh .. 2*nh-1
    modes = []
    if i > 0:
        modes.append(v(i - 1, j))
    if j > 0:
        modes.append(h(i, j - 1))
    if j < L - 1:
        modes.append(h(i, j))
    if i < L - 1:
        modes.append(v(i, j))
    return modes


def peps(L: int, D: int, seed: int, fill: Optional[Callable] = None) -> Network:
    """L x L lattice with bond dimension D; sites drawn in row-major order.

    ``fill(i, j, shape, rng)`` may replace the random U[0,1) entries (used by
    closed-form tests, e.g. all-ones or rank-one sites); the 1/(0.5 D^(deg/2))
    scale is applied after it."""
    rng = np.random.default_rng(seed)
    nbonds = 2 * L * (L - 1)
    extents = np.full(nbonds, D, dtype=np.int64)
    leaves, data = [], []
    for i in range(L):
        for j in range(L):
            m = site_modes(L, i, j)
            shape = (D,) * len(m)
            if fill is None:
                t = rng.random(shape, dtype=np.float32)
            else:
                t = np.asarray(fill(i, j, shape, rng))
            scale = 1.0 / (0.5 * float(D) ** (len(m) / 2.0))
            leaves.append(m)
            data.append((t * scale).astype(np.complex64))
    return Network(extents, leaves, [], data, name=f"peps{L}x{L}_D{D}",
                   meta={"L": L, "D": D, "seed": seed})


def row_major_tree(L: int) -> Tree:
    """Boundary absorbs sites (0,0), (0,1), ..., (L-1, L-1) one at a time."""
    return caterpillar(L * L)


def column_major_tree(L: int) -> Tree:
    """Same caterpillar, absorbing the lattice column by column."""
    order = [i * L + j for j in range(L) for i in range(L)]
    return caterpillar(L * L, order)
