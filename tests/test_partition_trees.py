"""Recursive-bisection contraction trees (workloads.trees.partition_tree /
partition_search): every tree is a valid SSA tree over all leaves, the
contracted value does not depend on the tree (oracle, complex128, against
the greedy tree), and on the 7x8 depth-11 grid network the search reaches a
narrower tree than the randomized greedy search."""

import math

import numpy as np
import pytest

import oracle
from tests.conftest import rel_err_ok
from workloads import circuits, randnet, trees

TOL128 = 1e-10


def _valid(net, tree):
    L = net.num_leaves
    seen = set()
    for s, (a, b) in enumerate(zip(tree.lhs, tree.rhs)):
        for x in (a, b):
            assert 0 <= x < L + s, (s, x)
            assert x not in seen, f"operand {x} used twice"
            seen.add(x)
    assert len(tree.lhs) == L - 1
    assert seen == set(range(L + len(tree.lhs) - 1))


@pytest.mark.parametrize("seed", range(6))
def test_partition_tree_valid_and_tree_independent(seed):
    c = circuits.grid_fsim(3, 4, 6 + seed % 3, 40 + seed)
    net = c.to_network(open_qubits=[seed % 12])
    tr = trees.partition_tree(net, seed=seed, imbalance=0.1 + 0.1 * (seed % 3), cutoff=4 + seed)
    _valid(net, tr)
    ref = oracle.contract_network(net, trees.greedy_tree(net))
    got = oracle.contract_network(net, tr)
    ok, err = rel_err_ok(got, ref, TOL128)
    assert ok, err


@pytest.mark.parametrize("seed", range(4))
def test_partition_tree_on_random_networks(seed):
    rng = np.random.default_rng(900 + seed)
    net = randnet.random_network(rng, n_leaves=int(rng.integers(12, 24)), n_closed=int(rng.integers(14, 30)),
                                 n_open=int(rng.integers(0, 3)), extent_choices=(1, 2, 3))
    tr = trees.partition_tree(net, seed=seed, cutoff=3)
    _valid(net, tr)
    if trees.tree_cost(net, tr)["max_elems"] > 1 << 22:
        pytest.skip("too wide for the oracle")
    ref = oracle.contract_network(net, randnet.random_tree(np.random.default_rng(seed), net.num_leaves))
    got = oracle.contract_network(net, tr)
    ok, err = rel_err_ok(got, ref, TOL128)
    assert ok, err


def test_partition_search_narrower_on_7x8_grid():
    net = circuits.grid_fsim(7, 8, 11, 505).to_network()
    part = trees.tree_cost(net, trees.partition_search(net, trials=40, seed=1))
    greedy = trees.tree_cost(net, trees.search_tree(net, trials=40, seed=1))
    assert (part["max_elems"], part["flops"]) < (greedy["max_elems"], greedy["flops"]), \
        (math.log2(part["max_elems"]), math.log2(greedy["max_elems"]))
