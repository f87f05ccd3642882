"""Plain containers for a tensor network and a contraction tree.

A network is a list of leaf tensors, each carrying a list of integer mode
labels in the row-major order of its buffer (first mode = slowest axis), a
table of extents (one per mode label), and the ordered list of open modes
that the result must be laid out in.  Every closed mode appears in exactly
two leaves; every open mode appears in exactly one leaf and in ``out_modes``.

A tree is a list of pairwise steps in execution order.  Operands are SSA
ids: leaves are ``0 .. L-1`` and step ``s`` creates tensor ``L + s``; the
last step creates the root.
"""

from __future__ import annotations

import hashlib
from dataclasses import dataclass, field
from typing import List, Optional

import numpy as np


@dataclass
class Network:
    extents: np.ndarray                   # int64, one per mode label
    leaves: List[List[int]]               # declared mode order of each leaf
    out_modes: List[int]                  # open modes, in the result's order
    data: Optional[List[np.ndarray]] = None   # complex64 arrays, shape = extents of the leaf's modes
    name: str = ""
    meta: dict = field(default_factory=dict)

    @property
    def num_modes(self) -> int:
        return int(len(self.extents))

    @property
    def num_leaves(self) -> int:
        return len(self.leaves)

    def leaf_shape(self, i: int):
        return tuple(int(self.extents[x]) for x in self.leaves[i])

    def flat_modes(self):
        """(leaf_rank int32[L], leaf_modes int32[sum rank]) as the C-ABI wants them."""
        rank = np.array([len(l) for l in self.leaves], dtype=np.int32)
        modes = np.array([x for l in self.leaves for x in l], dtype=np.int32)
        return rank, modes

    def digest(self) -> str:
        """SHA-256 over structure and data, to record exactly which input was used."""
        h = hashlib.sha256()
        h.update(np.asarray(self.extents, dtype=np.int64).tobytes())
        for l in self.leaves:
            h.update(np.asarray(l, dtype=np.int32).tobytes())
            h.update(b"|")
        h.update(np.asarray(self.out_modes, dtype=np.int32).tobytes())
        if self.data is not None:
            for d in self.data:
                h.update(np.ascontiguousarray(d).tobytes())
        return h.hexdigest()


@dataclass
class Tree:
    lhs: List[int]
    rhs: List[int]

    @property
    def num_steps(self) -> int:
        return len(self.lhs)

    def arrays(self):
        return (np.asarray(self.lhs, dtype=np.int32), np.asarray(self.rhs, dtype=np.int32))


def caterpillar(num_leaves: int, order=None) -> Tree:
    """Tree that absorbs leaves one by one into a growing boundary tensor."""
    order = list(range(num_leaves)) if order is None else list(order)
    assert len(order) == num_leaves
    if num_leaves == 1:
        return Tree([], [])
    lhs, rhs = [order[0]], [order[1]]
    for s, leaf in enumerate(order[2:], start=1):
        lhs.append(num_leaves + s - 1)
        rhs.append(leaf)
    return Tree(lhs, rhs)


def close_open_wires(net: Network, tree: Tree, bits=None):
    """Close every open mode of ``net`` with a basis-vector leaf ([1, 0, ...]
    for bit 0) and extend ``tree`` by one step per closed mode, absorbing them
    into the old root in output order.  Returns (network, tree) with the
    new leaves placed after the old ones (SSA ids of intermediates shift)."""
    import numpy as _np
    L, S = net.num_leaves, tree.num_steps
    nopen = len(net.out_modes)
    bits = [0] * nopen if bits is None else list(bits)
    leaves = [list(l) for l in net.leaves]
    data = list(net.data) if net.data is not None else None
    for x, b in zip(net.out_modes, bits):
        leaves.append([x])
        if data is not None:
            v = _np.zeros(int(net.extents[x]), dtype=_np.complex64)
            v[b] = 1
            data.append(v)

    def remap(t):
        return t if t < L else t + nopen

    lhs = [remap(a) for a in tree.lhs]
    rhs = [remap(b) for b in tree.rhs]
    root = remap(L + S - 1) if S > 0 else 0
    for j in range(nopen):
        lhs.append(root)
        rhs.append(L + j)
        root = (L + nopen) + S + j
    out = Network(net.extents.copy(), leaves, [], data, name=net.name + "_closed", meta=dict(net.meta))
    return out, Tree(lhs, rhs)
