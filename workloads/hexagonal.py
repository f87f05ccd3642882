"""Honeycomb-lattice partition-function networks and Ising networks on
graphs: the second workload family.

The page ("Parallelizing Large-Scale Tensor Network Contraction on Multiple
GPUs", section 2.1) measures a "Hexagonal" workload and names error-
correction decoding and combinatorial optimisation among the targets
(section 0), without defining any instance.  These generators are this
project's synthetic stand-ins.

Honeycomb (``honeycomb``): the brick-wall form of the hexagonal lattice.
Sites (i, j), i < rows, j < cols, each join their left and right row
neighbours (horizontal bond h(i, j) between (i, j) and (i, j + 1)); site
(i, j) with i + j even also joins (i + 1, j) below (vertical bond v(i, j)).
Every interior site has three bonds.  Site modes are declared [up, left,
right, down] (absent ones skipped).  Entries are U[0, 1) float32 scaled by
1 / (0.5 D^(deg / 2)), complex64 with zero imaginary part, drawn in row-major
site order; no open modes.

Ising (``ising``): Z = sum over spins s in {+1, -1}^N of
prod over edges exp(beta J_e s_a s_b).  Each spin is a COPY (delta) leaf
over the edges it touches, each edge a 2 x 2 leaf
W[a, b] = exp(beta J_e (1 - 2a)(1 - 2b)) with index 0 for spin +1;
couplings J_e ~ U[-1, 1) from the seed (or all 1).  Leaves: spins first in
vertex order (modes in the order of the vertex's edges), then edges.
"""

from __future__ import annotations

from typing import Callable, List, Optional, Sequence, Tuple

import numpy as np

from .network import Network, Tree, caterpillar


def honeycomb_bonds(rows: int, cols: int):
    """(horizontal label of (i, j)-(i, j+1), vertical label of (i, j)-(i+1, j)
    or None) as two functions, and the number of bonds."""
    hid, vid = {}, {}
    n = 0
    for i in range(rows):
        for j in range(cols - 1):
            hid[i, j] = n
            n += 1
    for i in range(rows - 1):
        for j in range(cols):
            if (i + j) % 2 == 0:
                vid[i, j] = n
                n += 1
    return hid, vid, n


def honeycomb_site_modes(rows: int, cols: int, i: int, j: int, hid=None, vid=None) -> List[int]:
    if hid is None:
        hid, vid, _ = honeycomb_bonds(rows, cols)
    modes = []
    if (i - 1, j) in vid:
        modes.append(vid[i - 1, j])
    if (i, j - 1) in hid:
        modes.append(hid[i, j - 1])
    if (i, j) in hid:
        modes.append(hid[i, j])
    if (i, j) in vid:
        modes.append(vid[i, j])
    return modes


def honeycomb(rows: int, cols: int, D: int, seed: int, fill: Optional[Callable] = None) -> Network:
    """rows x cols brick-wall honeycomb with bond dimension D.  ``fill(i, j,
    shape, rng)`` may replace the random entries (closed-form tests); the
    scale is applied after it."""
    rng = np.random.default_rng(seed)
    hid, vid, nb = honeycomb_bonds(rows, cols)
    extents = np.full(nb, D, dtype=np.int64)
    leaves, data = [], []
    for i in range(rows):
        for j in range(cols):
            m = honeycomb_site_modes(rows, cols, i, j, hid, vid)
            shape = (D,) * len(m)
            t = rng.random(shape, dtype=np.float32) if fill is None else np.asarray(fill(i, j, shape, rng))
            scale = 1.0 / (0.5 * float(D) ** (len(m) / 2.0))
            leaves.append(m)
            data.append((t * scale).astype(np.complex64))
    return Network(extents, leaves, [], data, name=f"honeycomb{rows}x{cols}_D{D}",
                   meta={"rows": rows, "cols": cols, "D": D, "seed": seed, "bonds": nb})


def honeycomb_tree(rows: int, cols: int) -> Tree:
    """Boundary absorbs the sites in row-major order."""
    return caterpillar(rows * cols)


# ---------------------------------------------------------------------------
# Ising networks


def random_regular_graph(n: int, degree: int, seed: int) -> List[Tuple[int, int]]:
    """A simple degree-regular graph on n vertices by the pairing model:
    random perfect matchings of the vertex stubs, retried until no loop or
    double edge appears."""
    if (n * degree) % 2:
        raise ValueError("n * degree must be even")
    rng = np.random.default_rng(seed)
    for _ in range(1000):
        stubs = np.repeat(np.arange(n), degree)
        rng.shuffle(stubs)
        pairs = stubs.reshape(-1, 2)
        if np.any(pairs[:, 0] == pairs[:, 1]):
            continue
        edges = sorted({(int(min(a, b)), int(max(a, b))) for a, b in pairs})
        if len(edges) == len(pairs):
            return edges
    raise RuntimeError("no simple regular graph found")


def copy_tensor(rank: int) -> np.ndarray:
    """delta_{i1 ... ir} over extent 2."""
    t = np.zeros((2,) * rank, dtype=np.complex64)
    t[(0,) * rank] = 1
    t[(1,) * rank] = 1
    return t


def ising(n: int, edges: Sequence[Tuple[int, int]], beta: float, seed: Optional[int] = None,
          couplings: Optional[Sequence[float]] = None) -> Network:
    """Partition-function network of the Ising model on (n, edges).  Edge e
    carries two modes: 2e at its lower vertex, 2e + 1 at its upper one.
    Couplings: given, else U[-1, 1) from ``seed``, else all 1."""
    E = len(edges)
    if couplings is None:
        couplings = np.random.default_rng(seed).uniform(-1.0, 1.0, size=E) if seed is not None else np.ones(E)
    vmodes: List[List[int]] = [[] for _ in range(n)]
    for e, (a, b) in enumerate(edges):
        vmodes[a].append(2 * e)
        vmodes[b].append(2 * e + 1)
    leaves, data = [], []
    for v in range(n):
        if not vmodes[v]:
            raise ValueError(f"vertex {v} has no edge")
        leaves.append(vmodes[v])
        data.append(copy_tensor(len(vmodes[v])))
    sgn = np.array([1.0, -1.0])
    for e, (a, b) in enumerate(edges):
        leaves.append([2 * e, 2 * e + 1])
        w = np.exp(beta * float(couplings[e]) * np.outer(sgn, sgn))
        data.append(w.astype(np.complex64))
    return Network(np.full(2 * E, 2, dtype=np.int64), leaves, [], data, name=f"ising{n}",
                   meta={"n": n, "edges": list(edges), "beta": beta, "couplings": list(map(float, couplings))})
