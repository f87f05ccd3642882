"""Brute-force references used to pin the oracle (independent of it).

* ``statevector`` simulates a circuit gate by gate on the full 2^n state;
* ``einsum_full`` evaluates a small network in one numpy.einsum call.
"""

from __future__ import annotations

import numpy as np


def statevector(n: int, gates, dtype=np.complex128) -> np.ndarray:
    """Apply two-qubit gates (a, b, U), a < b, to |0...0>; qubit 0 is the
    most significant bit.  Returns the 2^n amplitudes."""
    psi = np.zeros((2,) * n, dtype=dtype)
    psi[(0,) * n] = 1
    for a, b, u in gates:
        g = np.asarray(u, dtype=dtype).reshape(2, 2, 2, 2)
        # contract g[oa, ob, ia, ib] with psi[..., ia (axis a), ..., ib (axis b), ...]
        psi = np.tensordot(g, psi, axes=([2, 3], [a, b]))
        # result axes: oa, ob, then the remaining psi axes in order; move back
        psi = np.moveaxis(psi, [0, 1], [a, b])
    return psi.reshape(-1)


def einsum_full(extents, leaves, out_modes, data) -> np.ndarray:
    """Whole-network sum in one einsum (numpy picks its own order)."""
    letters = {}
    for l in leaves:
        for x in l:
            letters.setdefault(x, len(letters))
    for x in out_modes:
        letters.setdefault(x, len(letters))
    ops = []
    for l, d in zip(leaves, data):
        ops.append(np.asarray(d, dtype=np.complex128))
        ops.append([letters[x] for x in l])
    ops.append([letters[x] for x in out_modes])
    return np.einsum(*ops, optimize="greedy")
