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


def track_basis_state(n: int, gates, bits0=None):
    """For a circuit of monomial gates (one non-zero per column), follow the
    basis state |bits0> through every gate.  Returns (bits, amplitude) with
    U|bits0> = amplitude |bits>.  Gate matrices are taken as given (pass the
    complex64-rounded ones to match the network leaves)."""
    bits = [0] * n if bits0 is None else list(bits0)
    amp = complex(1.0)
    for a, b, u in gates:
        u = np.asarray(u)
        i = 2 * bits[a] + bits[b]
        col = u[:, i]
        nz = np.flatnonzero(np.abs(col) > 0)
        assert len(nz) == 1, "gate is not monomial"
        o = int(nz[0])
        amp *= complex(col[o])
        bits[a], bits[b] = o >> 1, o & 1
    return bits, amp


def monomial_mode_values(net, gates, n: int):
    """For the network of a circuit of monomial gates built by
    ``Circuit.to_network`` (n ket leaves, then one leaf [out_a, out_b, in_a,
    in_b] per gate in time order): the value every wire mode takes on the one
    basis-state path that starts at |0...0>, and the path's amplitude (the
    product of the gates' non-zero entries along it).  With the bra set to
    the path's final bits, every mode assignment that leaves this path
    contributes exactly zero."""
    vals = {}
    for q in range(n):
        vals[net.leaves[q][0]] = 0
    amp = complex(1.0)
    for g, (a, b, u) in enumerate(gates):
        oa, ob, ia, ib = net.leaves[n + g]
        i = 2 * vals[ia] + vals[ib]
        col = np.asarray(u)[:, i]
        nz = np.flatnonzero(np.abs(col) > 0)
        assert len(nz) == 1, "gate is not monomial"
        o = int(nz[0])
        amp *= complex(col[o])
        vals[oa], vals[ob] = o >> 1, o & 1
    return vals, amp
