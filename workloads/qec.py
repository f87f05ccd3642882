"""Error-correction decoding networks: the coset weight of a bit-flip error
on the planar surface code.

The page ("Parallelizing Large-Scale Tensor Network Contraction on Multiple
GPUs", section 0) names error-correction decoding among the applications of
exact contraction and defines no instance; this generator is this
project's synthetic stand-in, with the standard unrotated planar code.

Layout for distance d: sites (x, y) with 0 <= x, y <= 2d - 2.  Data qubits
sit where x + y is even (d^2 + (d - 1)^2 of them), X-type stabilizers where
x is odd and y even (d (d - 1) of them), Z-type stabilizers where x is even
and y odd; a stabilizer acts on its in-range neighbours (x +- 1, y),
(x, y +- 1).  Every data qubit belongs to one or two X stabilizers.  The
qubits (0, y), y even, form a logical X (weight d): they commute with
every Z stabilizer and are no product of X stabilizers.

Under independent bit flips with probability p, an X error E (a 0/1 vector
over the qubits) has the coset weight

    Z(E) = sum over s in {0,1}^{X stabilizers} of
           prod over qubits q of w(E_q xor (xor of s_k over the X stabilizers k that contain q)),

with w(0) = 1 - p and w(1) = p: the probability of the error class of E
(maximum-likelihood decoding compares Z(E) with Z(E xor logical)).  As a
network: every X stabilizer is a COPY (delta) leaf with one mode per qubit
it contains, every qubit a leaf over its one or two incidence modes,
W[a] = w(E_q xor a) or W[a, b] = w(E_q xor a xor b); every mode has extent 2
and the result is a scalar.  Leaves: stabilizers first in (y, x) order,
then qubits in (y, x) order; complex64 with zero imaginary part.
"""

from __future__ import annotations

from typing import Dict, List, Optional, Sequence, Tuple

import numpy as np

from .hexagonal import copy_tensor
from .network import Network


def planar_code(d: int):
    """(qubits, stabilizers, logical): qubit and X-stabilizer coordinates
    in (y, x) order, each stabilizer's qubit indices (ascending), and the
    qubit indices of the logical X."""
    if d < 2:
        raise ValueError("distance must be at least 2")
    n = 2 * d - 1
    qubits = [(x, y) for y in range(n) for x in range(n) if (x + y) % 2 == 0]
    qindex = {q: i for i, q in enumerate(qubits)}
    stabs = [(x, y) for y in range(0, n, 2) for x in range(1, n, 2)]
    support: List[List[int]] = []
    for (x, y) in stabs:
        nb = [(x - 1, y), (x + 1, y), (x, y - 1), (x, y + 1)]
        support.append(sorted(qindex[q] for q in nb if q in qindex))
    logical = [qindex[(0, y)] for y in range(0, n, 2)]
    return qubits, support, logical


def random_error(d: int, p: float, seed: int) -> np.ndarray:
    """An i.i.d. bit-flip pattern (0/1 per qubit, in (y, x) order)."""
    nq = d * d + (d - 1) * (d - 1)
    return (np.random.default_rng(seed).random(nq) < p).astype(np.int64)


def coset_network(d: int, p: float, error: Optional[Sequence[int]] = None, relative: bool = False) -> Network:
    """The coset-weight network Z(E) of the module docstring (E = 0 when
    ``error`` is None).  relative: every qubit leaf divided by w(E_q), so
    that the network gives Z(E) / P(E) with P(E) = prod_q w(E_q), the
    probability of E itself (the s = 0 term becomes 1 and no term under- or
    overflows single precision at large d; needs 0 < p < 1)."""
    if relative and not 0.0 < p < 1.0:
        raise ValueError("relative weights need 0 < p < 1")
    qubits, support, logical = planar_code(d)
    nq = len(qubits)
    E = np.zeros(nq, dtype=np.int64) if error is None else np.asarray(error, dtype=np.int64).reshape(-1)
    if E.shape != (nq,) or np.any((E != 0) & (E != 1)):
        raise ValueError(f"error must be a 0/1 vector of {nq} entries")
    # one mode per (stabilizer, qubit) incidence
    inc: Dict[Tuple[int, int], int] = {}
    for k, sup in enumerate(support):
        for q in sup:
            inc[(k, q)] = len(inc)
    qmodes: List[List[int]] = [[] for _ in range(nq)]
    for (k, q), m in sorted(inc.items()):
        qmodes[q].append(m)
    leaves, data = [], []
    for k, sup in enumerate(support):
        leaves.append([inc[(k, q)] for q in sup])
        data.append(copy_tensor(len(sup)))
    w = np.array([1.0 - p, p])
    for q in range(nq):
        r = len(qmodes[q])
        if r == 1:
            t = w[E[q] ^ np.arange(2)]
        elif r == 2:
            a = np.arange(2)
            t = w[E[q] ^ a[:, None] ^ a[None, :]]
        else:
            raise AssertionError("every qubit belongs to one or two X stabilizers")
        if relative:
            t = t / w[E[q]]
        leaves.append(qmodes[q])
        data.append(t.astype(np.complex64))
    return Network(np.full(len(inc), 2, dtype=np.int64), leaves, [], data,
                   name=f"surface_d{d}" + ("_rel" if relative else ""),
                   meta={"d": d, "p": p, "error": E.tolist(), "support": support, "logical": logical,
                         "relative": relative})


def sweep_tree(d: int, reverse: bool = False):
    """A caterpillar over the leaves in column-major site order (x, then y;
    at one site the stabilizer before the qubit; from the last column when
    ``reverse``): the running tensor's open modes are the bonds across the
    current column, about 2d of them."""
    from .network import Tree
    qubits, support, _ = planar_code(d)
    n = 2 * d - 1
    stabs = [(x, y) for y in range(0, n, 2) for x in range(1, n, 2)]
    site = [(x, y) for (x, y) in stabs] + [(x, y) for (x, y) in qubits]
    sgn = -1 if reverse else 1
    order = sorted(range(len(site)), key=lambda i: (sgn * site[i][0], site[i][1], i >= len(stabs)))
    L = len(site)
    lhs, rhs = [], []
    cur = order[0]
    for s, leaf in enumerate(order[1:]):
        lhs.append(cur)
        rhs.append(leaf)
        cur = L + s
    return Tree(lhs, rhs)
