"""Random quantum circuits written as tensor networks.

Conventions (fixed here because the source page only names its circuit
workloads, "Parallelizing Large-Scale Tensor Network Contraction on Multiple
GPUs", section 2.1):

* qubit 0 is the most significant bit of a basis-state index;
* a two-qubit gate on qubits (a, b) with a < b is a 4x4 unitary ``U`` acting
  on the pair index ``2*bit_a + bit_b``; its leaf tensor has modes
  ``[out_a, out_b, in_a, in_b]`` with ``G[oa, ob, ia, ib] = U[2oa+ob, 2ia+ib]``;
* the initial state is ``|0...0>`` (a ket leaf ``[1, 0]`` per qubit);
* closed qubits end in a bra leaf for the requested bit; open qubits leave
  their final wire in ``out_modes`` (in ascending qubit order unless given).

Random draws are made in a fixed order (layer-major, gates by ascending first
qubit) from ``numpy.random.default_rng(seed)``.
"""

from __future__ import annotations

from typing import Iterable, List, Optional, Sequence, Tuple

import numpy as np

from .network import Network

# --------------------------------------------------------------------------
# Random unitaries


def haar_unitary(rng: np.random.Generator, d: int) -> np.ndarray:
    """Haar-random d x d unitary: QR of a complex Gaussian matrix with the
    phases of R's diagonal moved into Q (Mezzadri's construction)."""
    z = (rng.standard_normal((d, d)) + 1j * rng.standard_normal((d, d))) / np.sqrt(2.0)
    q, r = np.linalg.qr(z)
    ph = np.diag(r) / np.abs(np.diag(r))
    return q * ph[None, :]


def haar_su2(rng: np.random.Generator) -> np.ndarray:
    """Haar-random SU(2) element [[a, -conj(b)], [b, conj(a)]] with (a, b) a
    normalised complex Gaussian 2-vector."""
    v = rng.standard_normal(4)
    v = v / np.linalg.norm(v)
    a = v[0] + 1j * v[1]
    b = v[2] + 1j * v[3]
    return np.array([[a, -np.conj(b)], [b, np.conj(a)]], dtype=np.complex128)


def fsim(theta: float, phi: float) -> np.ndarray:
    """fSim(theta, phi): iSWAP-like rotation in the {01, 10} block and a
    conditional phase on |11>."""
    c, s = np.cos(theta), np.sin(theta)
    return np.array(
        [[1, 0, 0, 0],
         [0, c, -1j * s, 0],
         [0, -1j * s, c, 0],
         [0, 0, 0, np.exp(-1j * phi)]],
        dtype=np.complex128,
    )


# --------------------------------------------------------------------------
# Circuit description → network


class Circuit:
    """A list of two-qubit gates (a, b, U) with a < b, in time order."""

    def __init__(self, n_qubits: int):
        self.n = n_qubits
        self.gates: List[Tuple[int, int, np.ndarray]] = []

    def add(self, a: int, b: int, u: np.ndarray):
        if a == b:
            raise ValueError("two-qubit gate on one qubit")
        if a > b:  # reorder the pair index so that the lower qubit is first
            perm = np.array([0, 2, 1, 3])
            u = u[np.ix_(perm, perm)]
            a, b = b, a
        self.gates.append((a, b, np.asarray(u, dtype=np.complex128)))

    def to_network(self, open_qubits: Sequence[int] = (), bits: Optional[Sequence[int]] = None,
                   out_order: Optional[Sequence[int]] = None, name: str = "") -> Network:
        """Network for <bits| U |0...0> with the wires of ``open_qubits`` left open.

        ``bits[q]`` is the bra bit of a closed qubit q (default 0).  The open
        wires appear in ``out_modes`` in ``out_order`` (default ascending)."""
        n = self.n
        open_set = set(int(q) for q in open_qubits)
        bits = [0] * n if bits is None else [int(b) for b in bits]
        extents: List[int] = []
        leaves: List[List[int]] = []
        data: List[np.ndarray] = []

        def new_mode() -> int:
            extents.append(2)
            return len(extents) - 1

        wire = []
        for q in range(n):
            w = new_mode()
            wire.append(w)
            leaves.append([w])
            data.append(np.array([1, 0], dtype=np.complex64))
        for a, b, u in self.gates:
            na, nb = new_mode(), new_mode()
            leaves.append([na, nb, wire[a], wire[b]])
            data.append(u.reshape(2, 2, 2, 2).astype(np.complex64))
            wire[a], wire[b] = na, nb
        for q in range(n):
            if q in open_set:
                continue
            leaves.append([wire[q]])
            v = np.zeros(2, dtype=np.complex64)
            v[bits[q]] = 1
            data.append(v)
        order = sorted(open_set) if out_order is None else [int(q) for q in out_order]
        assert sorted(order) == sorted(open_set)
        out_modes = [wire[q] for q in order]
        return Network(np.array(extents, dtype=np.int64), leaves, out_modes, data, name=name,
                       meta={"n_qubits": n, "n_gates": len(self.gates), "open_qubits": order})


# --------------------------------------------------------------------------
# Workload families


def brickwork(n_qubits: int, depth: int, seed: int) -> Circuit:
    """Layer t couples (q, q+1) for q = t mod 2, t mod 2 + 2, ... with
    Haar-random U(4) gates drawn layer by layer, ascending qubit."""
    rng = np.random.default_rng(seed)
    c = Circuit(n_qubits)
    for t in range(depth):
        for q in range(t % 2, n_qubits - 1, 2):
            c.add(q, q + 1, haar_unitary(rng, 4))
    return c


def grid_patterns(rows: int, cols: int):
    """The four nearest-neighbour coupler patterns A, B, C, D on a grid
    (qubit index r*cols + c): horizontal pairs with even / odd left column,
    then vertical pairs with even / odd upper row."""
    q = lambda r, c: r * cols + c
    A = [(q(r, c), q(r, c + 1)) for r in range(rows) for c in range(0, cols - 1, 2)]
    B = [(q(r, c), q(r, c + 1)) for r in range(rows) for c in range(1, cols - 1, 2)]
    C = [(q(r, c), q(r + 1, c)) for r in range(0, rows - 1, 2) for c in range(cols)]
    D = [(q(r, c), q(r + 1, c)) for r in range(1, rows - 1, 2) for c in range(cols)]
    return [sorted(A), sorted(B), sorted(C), sorted(D)]


def grid_fsim(rows: int, cols: int, depth: int, seed: int) -> Circuit:
    """Layers cycle through patterns A, B, C, D.  Each coupler is
    fSim(theta, phi) . (u_a (x) u_b) with theta, phi ~ U[0, 2pi) and u Haar
    SU(2); per gate the draws are theta, phi, u_a, u_b."""
    rng = np.random.default_rng(seed)
    pats = grid_patterns(rows, cols)
    c = Circuit(rows * cols)
    for t in range(depth):
        for a, b in pats[t % 4]:
            theta = rng.uniform(0.0, 2 * np.pi)
            phi = rng.uniform(0.0, 2 * np.pi)
            ua = haar_su2(rng)
            ub = haar_su2(rng)
            c.add(a, b, fsim(theta, phi) @ np.kron(ua, ub))
    return c


def from_gates(n_qubits: int, gates: Iterable[Tuple[int, int, np.ndarray]]) -> Circuit:
    c = Circuit(n_qubits)
    for a, b, u in gates:
        c.add(a, b, u)
    return c


HADAMARD = np.array([[1, 1], [1, -1]], dtype=np.complex128) / np.sqrt(2.0)


def grid_monomial(rows: int, cols: int, depth: int, seed: int) -> Circuit:
    """Same couplers as ``grid_fsim`` but every gate is a permutation times
    phases: fSim(pi/2, phi) (an iSWAP-like monomial) times single-qubit
    factors that are diagonal or anti-diagonal with random phases.  The
    circuit maps each basis state to one basis state with a phase, so a single
    amplitude is known exactly by tracking one basis state."""
    rng = np.random.default_rng(seed)
    pats = grid_patterns(rows, cols)

    def one_qubit():
        a, b = np.exp(1j * rng.uniform(0, 2 * np.pi, size=2))
        if rng.random() < 0.5:
            return np.array([[a, 0], [0, b]], dtype=np.complex128)
        return np.array([[0, a], [b, 0]], dtype=np.complex128)

    c = Circuit(rows * cols)
    for t in range(depth):
        for a, b in pats[t % 4]:
            phi = rng.uniform(0.0, 2 * np.pi)
            # fSim(pi/2, phi) written out exactly (cos(pi/2) is not 0 in floating point)
            g = np.array([[1, 0, 0, 0], [0, 0, -1j, 0], [0, -1j, 0, 0], [0, 0, 0, np.exp(-1j * phi)]],
                         dtype=np.complex128)
            c.add(a, b, g @ np.kron(one_qubit(), one_qubit()))
    return c
