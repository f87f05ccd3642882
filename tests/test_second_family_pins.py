"""Oracle pins for the second workload family (honeycomb lattice and Ising
partition functions), each against something the oracle does not compute
itself: closed forms, a textbook transfer-matrix result, a spin-by-spin
brute-force sum and whole-network numpy.einsum."""

import math

import numpy as np
import pytest

import oracle
from tests import brute
from workloads import hexagonal as H
from workloads import trees
from workloads.network import Tree


def _leaf_scales(net):
    # every entry of an all-ones site leaf equals its (complex64-rounded) scale
    return [float(np.asarray(d).reshape(-1)[0].real) for d in net.data]


@pytest.mark.parametrize("rows,cols,D", [(3, 4, 2), (4, 4, 3), (3, 6, 2)])
def test_honeycomb_all_ones_is_D_to_the_bonds(rows, cols, D):
    net = H.honeycomb(rows, cols, D, 0, fill=lambda i, j, shape, rng: np.ones(shape, np.float32))
    z = oracle.contract_network(net, H.honeycomb_tree(rows, cols))
    expect = math.prod(_leaf_scales(net)) * float(D) ** net.meta["bonds"]
    assert abs(z - expect) <= 1e-12 * abs(expect)


def test_honeycomb_rank_one_sites_factor_over_bonds():
    """Sites that are outer products of one vector per bond: Z is the
    product over bonds of the two vectors' inner product."""
    rows, cols, D = 4, 5, 3
    rng = np.random.default_rng(12)
    hid, vid, nb = H.honeycomb_bonds(rows, cols)
    vec = {}
    def fill(i, j, shape, r):
        vs = []
        for x in H.honeycomb_site_modes(rows, cols, i, j, hid, vid):
            v = rng.random(D).astype(np.float32)
            vec.setdefault(x, []).append(v)
            vs.append(v)
        t = vs[0]
        for v in vs[1:]:
            t = np.multiply.outer(t, v)
        return t
    net = H.honeycomb(rows, cols, D, 0, fill=fill)
    z = oracle.contract_network(net, H.honeycomb_tree(rows, cols))
    # rebuild with the stored (scaled, rounded) leaves: the factorisation uses
    # each site's scale once
    expect = math.prod(1.0 / (0.5 * D ** (len(l) / 2.0)) for l in net.leaves)
    for x in range(nb):
        a, b = vec[x]
        expect *= float(np.dot(a.astype(np.float64), b.astype(np.float64)))
    assert abs(z - expect) <= 2e-6 * abs(expect)


@pytest.mark.parametrize("seed", range(3))
def test_honeycomb_random_matches_einsum_and_any_tree(seed):
    net = H.honeycomb(4, 4, 3, seed)
    z = oracle.contract_network(net, H.honeycomb_tree(4, 4))
    zb = brute.einsum_full(net.extents, net.leaves, net.out_modes, net.data)
    zg = oracle.contract_network(net, trees.greedy_tree(net))
    assert abs(z - zb) <= 1e-12 * abs(zb)
    assert abs(zg - zb) <= 1e-12 * abs(zb)


def test_honeycomb_structure():
    """Interior sites have exactly three bonds; every bond joins two sites."""
    rows, cols = 6, 8
    net = H.honeycomb(rows, cols, 2, 0)
    deg = [len(l) for l in net.leaves]
    for i in range(1, rows - 1):
        for j in range(1, cols - 1):
            assert deg[i * cols + j] == 3
    cnt = np.bincount([x for l in net.leaves for x in l], minlength=len(net.extents))
    assert np.all(cnt == 2)


def _ising_brute(n, edges, couplings, beta, data_rounded=True):
    """Spin-by-spin sum of prod_e W_e[s_a, s_b] with the complex64-rounded
    edge weights the network holds."""
    sgn = np.array([1.0, -1.0])
    W = [np.exp(beta * float(J) * np.outer(sgn, sgn)).astype(np.complex64).astype(np.complex128) for J in couplings]
    total = 0.0
    for x in range(1 << n):
        bits = [(x >> (n - 1 - v)) & 1 for v in range(n)]
        p = 1.0 + 0j
        for e, (a, b) in enumerate(edges):
            p *= W[e][bits[a], bits[b]]
        total += p
    return total


@pytest.mark.parametrize("seed", range(3))
def test_ising_random_regular_matches_spin_sum(seed):
    n = 12
    edges = H.random_regular_graph(n, 3, seed)
    net = H.ising(n, edges, 0.35, seed=seed)
    z = oracle.contract_network(net, trees.greedy_tree(net))
    expect = _ising_brute(n, edges, net.meta["couplings"], 0.35)
    assert abs(z - expect) <= 1e-12 * abs(expect)


@pytest.mark.parametrize("n", [5, 9, 16])
def test_ising_ring_transfer_matrix(n):
    """Ring of n spins, J = 1: Z = (2 cosh b)^n + (2 sinh b)^n."""
    beta = 0.3
    edges = [(i, i + 1) for i in range(n - 1)] + [(0, n - 1)]
    net = H.ising(n, edges, beta)
    z = oracle.contract_network(net, trees.greedy_tree(net))
    expect = (2 * math.cosh(beta)) ** n + (2 * math.sinh(beta)) ** n
    assert abs(z - expect) <= 1e-6 * expect


def test_ising_tree_and_zero_temperature_limits():
    """A tree graph: Z = 2 (2 cosh b)^(n - 1).  beta = 0: Z = 2^n."""
    beta, n = 0.7, 11
    edges = [(v // 2, v) for v in range(1, n)]          # a binary tree
    z = oracle.contract_network(H.ising(n, edges, beta), trees.greedy_tree(H.ising(n, edges, beta)))
    assert abs(z - 2 * (2 * math.cosh(beta)) ** (n - 1)) <= 1e-6 * abs(z)
    edges = H.random_regular_graph(20, 3, 4)
    net = H.ising(20, edges, 0.0, seed=4)
    assert oracle.contract_network(net, trees.greedy_tree(net)) == 2.0 ** 20
