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


@pytest.mark.parametrize("name", ["grid_7x8_d16"])
def test_stored_tree_is_valid_and_fits(name):
    """A stored tree belongs to its network, is a valid SSA tree, its
    recorded costs are the tree's own, and one slice plans within the HBM of
    one GPU (host planning only)."""
    import math
    import quantum_circuit_simulation_amd as qa
    from workloads import circuits, make_trees
    rows, cols, depth, seed, _ = make_trees.SPECS[name]
    net = circuits.grid_fsim(rows, cols, depth, seed).to_network()
    tree, sliced, rec = trees.stored_tree(name, net)
    c = trees.tree_cost(net, tree, sliced)
    assert c["flops"] == rec["flop_per_slice"]
    assert math.log2(c["max_elems"]) == rec["log2_width"] <= 34
    assert trees.tree_cost(net, tree)["flops"] == rec["flop_unsliced"]
    plan = qa.Plan.from_network(net, tree, sliced=sliced, slice_range=(0, 1))
    st = plan.stats()
    assert st["num_slices"] == 2 ** len(sliced)
    assert st["workspace_bytes"] < 250e9


@pytest.mark.parametrize("seed", range(4))
def test_optimized_tree_valid_deterministic_and_value_preserving(seed):
    """The native search returns a valid SSA tree, the same one for the same
    seed whatever the thread count, its reported cost is the tree's own
    (log2 of the sum of m n k), and the oracle gives the same value along it
    as along the greedy tree."""
    c = circuits.grid_fsim(3, 4, 6 + seed, 60 + seed)
    net = c.to_network(open_qubits=[seed])
    t1, s1, st1 = trees.optimize_tree(net, trials=12, seed=seed, threads=1)
    t2, s2, st2 = trees.optimize_tree(net, trials=12, seed=seed, threads=4)
    assert (t1.lhs, t1.rhs, s1) == (t2.lhs, t2.rhs, s2) and s1 == []
    _valid(net, t1)
    cost = trees.tree_cost(net, t1)
    assert abs(st1["log2_cost"] - math.log2(cost["flops"] / 8)) < 1e-9
    assert st1["width"] == math.log2(cost["max_elems"])
    ref = oracle.contract_network(net, trees.greedy_tree(net))
    ok, err = rel_err_ok(oracle.contract_network(net, t1), ref, TOL128)
    assert ok, err


def test_optimized_tree_beats_partition_search_on_7x8_grid():
    net = circuits.grid_fsim(7, 8, 11, 505).to_network()
    opt, _, _ = trees.optimize_tree(net, trials=16, seed=1)
    part = trees.partition_search(net, trials=16, seed=1)
    assert trees.tree_cost(net, opt)["flops"] < trees.tree_cost(net, part)["flops"] / 10


@pytest.mark.parametrize("seed", range(3))
def test_width_bound_slices_and_slices_sum_to_the_value(seed):
    """With a width bound below the tree's width the search slices modes
    until every sliced intermediate fits; the slices' oracle values add up
    to the unsliced value, and the live-entry bound holds too."""
    c = circuits.grid_fsim(3, 4, 8, 70 + seed)
    net = c.to_network()
    tree, sl, st = trees.optimize_tree(net, trials=8, seed=seed, max_log_width=7, max_log_peak=8.5)
    assert sl and st["width"] <= 7 and st["peak_log2"] <= 8.5
    assert math.log2(trees.tree_cost(net, tree, sl)["max_elems"]) <= 7
    ref = oracle.contract_network(net, trees.greedy_tree(net))
    total = 0j
    for sigma in range(1 << len(sl)):
        fixed = {x: (sigma >> (len(sl) - 1 - i)) & 1 for i, x in enumerate(sl)}
        total += complex(oracle.contract_network(net, tree, fixed=fixed))
    ok, err = rel_err_ok(total, ref, TOL128)
    assert ok, err


def test_refine_never_raises_the_cost():
    net = circuits.grid_fsim(4, 4, 10, 5).to_network()
    tree, sl, st = trees.optimize_tree(net, trials=4, seed=2, reconf_k=6)
    t2, sl2, st2 = trees.refine_tree(net, tree, sl, reconf_k=10)
    _valid(net, t2)
    assert sl2 == sl and st2["log2_cost"] <= st["log2_cost"] + 1e-12
