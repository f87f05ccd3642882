"""Oracle pins for the error-correction decoding networks (the coset weight
of a bit-flip error on the planar surface code), each against something the
oracle does not compute itself: the definition summed over every stabilizer
combination, the code's structure, closed forms at p = 0 and p = 1/2, and
the invariance of the coset weight under stabilizers."""

import itertools

import numpy as np
import pytest

import oracle
from workloads import qec, trees


def _brute(d, p, E):
    """Z(E) by its definition: the sum over all 2^(d (d - 1)) stabilizer
    combinations s of prod_q w(E_q xor (H^T s)_q), in float64, with w(1) = p
    and w(0) = 1 - p rounded to float32 as the complex64 leaves hold them."""
    qubits, support, _ = qec.planar_code(d)
    H = np.zeros((len(support), len(qubits)), dtype=np.int64)
    for k, sup in enumerate(support):
        H[k, sup] = 1
    S = np.array(list(itertools.product((0, 1), repeat=len(support))), dtype=np.int64)
    flips = (S @ H + np.asarray(E)[None, :]) % 2
    w1, w0 = float(np.float32(p)), float(np.float32(1.0 - p))
    return float(np.prod(np.where(flips == 1, w1, w0), axis=1).sum())


def _z(net):
    return oracle.contract_network(net, trees.greedy_tree(net))


def test_planar_code_structure():
    for d in (2, 3, 4, 5):
        qubits, support, logical = qec.planar_code(d)
        assert len(qubits) == d * d + (d - 1) ** 2 and len(support) == d * (d - 1)
        deg = np.zeros(len(qubits), dtype=np.int64)
        for sup in support:
            assert len(sup) in (3, 4)
            deg[sup] += 1
        assert set(deg.tolist()) <= {1, 2}
        # the logical commutes with every Z stabilizer (even overlap)
        n = 2 * d - 1
        qi = {q: i for i, q in enumerate(qubits)}
        for (x, y) in [(x, y) for y in range(1, n, 2) for x in range(0, n, 2)]:
            zs = {qi[q] for q in [(x - 1, y), (x + 1, y), (x, y - 1), (x, y + 1)] if q in qi}
            assert len(zs & set(logical)) % 2 == 0
        # ... and is no product of X stabilizers (not in their row space over GF(2))
        H = np.zeros((len(support), len(qubits)), dtype=np.uint8)
        for k, sup in enumerate(support):
            H[k, sup] = 1
        L = np.zeros(len(qubits), dtype=np.uint8)
        L[logical] = 1
        assert _gf2_rank(np.vstack([H, L])) == _gf2_rank(H) + 1 == len(support) + 1


def _gf2_rank(M):
    M = M.copy() % 2
    r = 0
    for c in range(M.shape[1]):
        piv = [i for i in range(r, M.shape[0]) if M[i, c]]
        if not piv:
            continue
        M[[r, piv[0]]] = M[[piv[0], r]]
        for i in range(M.shape[0]):
            if i != r and M[i, c]:
                M[i] ^= M[r]
        r += 1
    return r


@pytest.mark.parametrize("d,p,seed", [(2, 0.1, 1), (3, 0.1, 2), (3, 0.3, 3), (4, 0.07, 4)])
def test_coset_weight_matches_the_sum_over_stabilizers(d, p, seed):
    E = qec.random_error(d, max(p, 0.2), seed)
    z = _z(qec.coset_network(d, p, E))
    ref = _brute(d, p, E)
    assert abs(z - ref) <= 1e-12 * ref


def test_closed_forms():
    for d in (3, 4, 5):
        nq, ns = d * d + (d - 1) ** 2, d * (d - 1)
        # p = 1/2: every term is 2^-nq, and there are 2^ns of them
        z = _z(qec.coset_network(d, 0.5, qec.random_error(d, 0.5, d)))
        assert abs(z - 2.0 ** (ns - nq)) <= 1e-12 * 2.0 ** (ns - nq)
        # p = 0: only the stabilizer combination that cancels E contributes,
        # so Z(0) = 1 and Z(logical) = 0 (the logical is no stabilizer)
        assert abs(_z(qec.coset_network(d, 0.0)) - 1.0) <= 1e-15
        E = np.zeros(nq, dtype=np.int64)
        E[qec.planar_code(d)[2]] = 1
        assert abs(_z(qec.coset_network(d, 0.0, E))) <= 1e-15


@pytest.mark.parametrize("d", [3, 5])
def test_coset_weight_is_invariant_under_stabilizers(d):
    _, support, logical = qec.planar_code(d)
    E = qec.random_error(d, 0.15, 7 + d)
    z = _z(qec.coset_network(d, 0.08, E))
    for k in (0, len(support) // 2, len(support) - 1):
        F = E.copy()
        F[support[k]] ^= 1
        assert abs(_z(qec.coset_network(d, 0.08, F)) - z) <= 1e-12 * z
    # the other coset (E times the logical) has another weight
    G = E.copy()
    G[logical] ^= 1
    assert abs(_z(qec.coset_network(d, 0.08, G)) - z) > 1e-6 * z


@pytest.mark.parametrize("d,p,seed", [(3, 0.1, 5), (4, 0.2, 6)])
def test_relative_weights_and_sweep_trees(d, p, seed):
    """Z(E) / P(E) from the relative network, times P(E) in float64, is
    the definition's sum; the column sweeps in both directions give the
    same value as the greedy tree."""
    E = qec.random_error(d, 0.2, seed)
    net = qec.coset_network(d, p, E, relative=True)
    zr = oracle.contract_network(net, trees.greedy_tree(net))
    w1, w0 = float(np.float32(p)), float(np.float32(1.0 - p))
    pe = float(np.prod(np.where(E == 1, w1, w0)))
    ref = _brute(d, p, E)
    assert abs(zr * pe - ref) <= 1e-6 * ref   # the leaves hold w(a) / w(E_q) rounded to float32
    for rev in (False, True):
        zs = oracle.contract_network(net, qec.sweep_tree(d, reverse=rev))
        assert abs(zs - zr) <= 1e-12 * abs(zr)
