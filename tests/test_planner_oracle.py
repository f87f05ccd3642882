"""Pins of the plan oracle (mode orders, groups, arena) against things other
than itself: the death-sort formulation, the structural invariants of
lifetime ordering, the page's worked einsum, and arena liveness."""

import json
import os

import numpy as np
import pytest

from oracle import planner as P
from workloads import circuits, lattice, randnet, sweep, trees

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _random_case(seed):
    rng = np.random.default_rng(seed)
    net = randnet.random_network(rng, n_leaves=int(rng.integers(1, 12)), n_closed=int(rng.integers(0, 20)),
                                 n_open=int(rng.integers(0, 5)), extent_choices=(1, 2, 3, 4, 8),
                                 with_data=False)
    tree = randnet.random_tree(rng, net.num_leaves)
    return net, tree


def test_page_einsum_example():
    g = json.load(open(os.path.join(GOLDEN, "page_einsum_example.json")))
    lab = g["labels"]
    A = [lab[c] for c in g["A"]]
    B = [lab[c] for c in g["B"]]
    out = [lab[c] for c in g["out"]]
    order = P.lifetime_orders([A, B], out, [0], [1])
    assert order[0] == [lab[c] for c in g["expect"]["order_A"]]
    assert order[1] == [lab[c] for c in g["expect"]["order_B"]]
    plan = P.make_plan(g["extents"], [A, B], out, [0], [1])
    nd = plan.nodes[0]
    assert (nd.m, nd.n, nd.k) == (g["expect"]["m"], g["expect"]["n"], g["expect"]["k"])
    assert nd.interleaved == 0 and nd.swap == 0
    assert plan.staged_leaf == [1, 1]


@pytest.mark.parametrize("seed", range(60))
def test_reverse_pass_equals_death_sort(seed):
    net, tree = _random_case(seed)
    a = P.lifetime_orders(net.leaves, net.out_modes, tree.lhs, tree.rhs)
    b = P.death_sort_orders(net.leaves, net.out_modes, tree.lhs, tree.rhs)
    assert a == b


@pytest.mark.parametrize("seed", range(30))
def test_lifetime_invariants(seed):
    net, tree = _random_case(seed)
    L = net.num_leaves
    order = P.lifetime_orders(net.leaves, net.out_modes, tree.lhs, tree.rhs)
    death = P.death_steps(net.leaves, tree.lhs, tree.rhs, ())
    sets, steps = P.ssa_modes(net.leaves, tree.lhs, tree.rhs, ())
    for t, o in enumerate(order):
        assert sorted(o) == sorted(sets[t])
        d = [death[x] for x in o]
        assert all(d[i] >= d[i + 1] for i in range(len(d) - 1)), (t, o, d)
    for s, (a, b) in enumerate(zip(tree.lhs, tree.rhs)):
        K, M, N = steps[s]
        c = order[L + s]
        for op, kept in ((a, M), (b, N)):
            assert order[op][:len(kept)] == [x for x in c if x in kept]
            assert order[op][len(kept):] == sorted(K)


@pytest.mark.parametrize("policy", [P.LIFETIME, P.NAIVE])
@pytest.mark.parametrize("seed", range(25))
def test_arena_buffers_live_together_do_not_overlap(seed, policy):
    net, tree = _random_case(seed)
    plan = P.make_plan(net.extents, net.leaves, net.out_modes, tree.lhs, tree.rhs, policy=policy,
                       tiny_mnk=64, max_group=4)
    L = net.num_leaves
    ext = net.extents

    def rb(elems):
        return -(-elems * 8 // 256) * 256

    sets, _ = P.ssa_modes(net.leaves, tree.lhs, tree.rhs, ())
    elems = [int(np.prod([ext[x] for x in st], dtype=np.int64)) for st in sets]
    # intermediate t lives from its producer's group to its consumer's group
    prod_group = {nd.out: nd.group for nd in plan.nodes}
    cons = {}
    for nd in plan.nodes:
        cons[nd.lhs] = nd.group
        cons[nd.rhs] = nd.group
    for g, members in enumerate(plan.groups):
        bufs = []
        for t in range(L, L + len(tree.lhs)):
            off = plan.tensor_off[t]
            if off == P.NONE:
                continue
            if prod_group[t] <= g <= cons.get(t, len(plan.groups)):
                bufs.append((off, rb(elems[t]), ("T", t)))
        for s in members:
            nd = plan.nodes[s]
            for w, t in (("a", nd.lhs), ("b", nd.rhs)):
                if getattr(nd, "copy_" + w):
                    bufs.append((getattr(nd, w + "_off"), rb(elems[t]), ("copy", s, w)))
            if nd.splits > 1:
                bufs.append((nd.scratch_off, -(-nd.scratch_bytes // 256) * 256, ("scratch", s)))
        bufs.sort()
        for (o1, s1, n1), (o2, s2, n2) in zip(bufs, bufs[1:]):
            assert o1 + s1 <= o2, (g, n1, n2)
        for o, s_, _ in bufs:
            assert o % 256 == 0 and o + s_ <= plan.arena_bytes


@pytest.mark.parametrize("seed", range(20))
def test_groups_are_a_valid_schedule(seed):
    """Every step runs exactly once, after the steps producing its operands
    (in an earlier group), never beside them; non-tiny steps run alone and
    keep their list order relative to each other."""
    net, tree = _random_case(seed)
    plan = P.make_plan(net.extents, net.leaves, net.out_modes, tree.lhs, tree.rhs, tiny_mnk=1 << 10,
                       max_group=3)
    L = net.num_leaves
    done_group = {t: -1 for t in range(L)}
    seen = []
    for g, members in enumerate(plan.groups):
        assert 1 <= len(members) <= 3
        for s in members:
            nd = plan.nodes[s]
            assert done_group[nd.lhs] < g and done_group[nd.rhs] < g
            if len(members) > 1:
                assert nd.cls == P.CLASS_TINY
        for s in members:
            done_group[plan.nodes[s].out] = g
            seen.append(s)
    assert sorted(seen) == list(range(len(tree.lhs)))
    big = [s for s in seen if plan.nodes[s].cls != P.CLASS_TINY]
    assert big == sorted(big)


def test_aligned_sweep_case_needs_no_copies():
    net, tree = sweep.network(10, 6, 6)
    plan = P.make_plan(net.extents, net.leaves, net.out_modes, tree.lhs, tree.rhs)
    nd = plan.nodes[0]
    assert plan.staged_leaf == [0, 0]
    assert (nd.m, nd.n, nd.k, nd.swap, nd.interleaved) == (1 << 10, 1 << 6, 1 << 6, 0, 0)
    assert nd.row_runs == [(1 << 10, 1 << 6)] and nd.col_runs == [(1 << 6, 1)]
    assert plan.arena_bytes == 0


def test_peps_bulk_nodes():
    net = lattice.peps(8, 8, 404)
    tree = lattice.row_major_tree(8)
    plan = P.make_plan(net.extents, net.leaves, net.out_modes, tree.lhs, tree.rhs)
    bulk = [nd for nd in plan.nodes if (nd.m, nd.n, nd.k) == (1 << 21, 64, 64)]
    assert len(bulk) == 36
    assert plan.max_elems == 1 << 27
    assert abs(plan.flops - 2.58e12) < 0.01e12
    # intermediates never need a runtime re-layout under lifetime ordering
    for nd in plan.nodes:
        if nd.lhs >= net.num_leaves:
            assert nd.copy_a == 0
        if nd.rhs >= net.num_leaves:
            assert nd.copy_b == 0


def test_naive_policy_relayouts_intermediates():
    net = lattice.peps(4, 2, 1)
    tree = lattice.row_major_tree(4)
    plan = P.make_plan(net.extents, net.leaves, net.out_modes, tree.lhs, tree.rhs, policy=P.NAIVE)
    assert sum(nd.copy_a + nd.copy_b for nd in plan.nodes) > 0
    for nd in plan.nodes:
        assert nd.interleaved == 0


def test_validation_errors():
    with pytest.raises(P.PlanError) as e:   # hyperedge
        P.make_plan([2], [[0], [0], [0]], [], [0, 3], [1, 2])
    assert e.value.code == "UNSUPPORTED"
    with pytest.raises(P.PlanError) as e:   # dangling
        P.make_plan([2, 2], [[0, 1], [0]], [], [0], [1])
    assert e.value.code == "INVALID_NETWORK"
    with pytest.raises(P.PlanError) as e:   # reused operand
        P.make_plan([2], [[0], [0], []], [], [0, 0], [1, 2])
    assert e.value.code == "INVALID_TREE"
    with pytest.raises(P.PlanError) as e:   # open mode sliced
        P.make_plan([2], [[0]], [0], [], [], sliced=[0])
    assert e.value.code == "INVALID_ARG"
