"""Distribution schedule over P GPUs (tnc_plan_distribute) against the
exhaustive-search oracle, and pins of the oracle itself (closed forms,
special cases and the page's qualitative claims).  Host only.

Source: "Parallelizing Large-Scale Tensor Network Contraction on Multiple
GPUs", sections 1.5 (prefix split, step tags) and 1.6 (keep-or-redistribute
program, cost model)."""

import math

import numpy as np
import pytest

import oracle.distribute as OD
from oracle import planner
import quantum_circuit_simulation_amd as qa
from workloads import circuits, lattice, randnet, trees
from workloads.network import Network, Tree

REL = 1e-9


def _both(net, tree, **kw):
    P = kw.get("num_gpus", 8)
    thr = kw.get("threshold_bytes", 8 << 30)
    md = OD.model(net.extents, net.leaves, net.out_modes, tree.lhs, tree.rhs, P=P, threshold=thr,
                  B_net=kw.get("net_bytes_per_s", 7 * 76.8e9), lam=kw.get("latency_s", 5e-6))
    plan = qa.Plan.from_network(net, tree)
    steps, total = plan.distribute(**kw)
    return md, plan, steps, total


def _check_optimal(net, tree, **kw):
    md, plan, steps, total = _both(net, tree, **kw)
    best, recs, _, _ = md.best()
    assert math.isclose(total, best, rel_tol=REL, abs_tol=1e-15), (total, best)
    tags = [s["tag"] for s in steps]
    mine = md.cost_of(tags)
    assert mine is not None, "library schedule is not a valid schedule"
    assert math.isclose(mine[0], best, rel_tol=REL, abs_tol=1e-15)
    # the library's records equal the oracle's for the library's own choice
    for s, st in enumerate(steps):
        r = mine[1][s]
        assert r["tag"] == st["tag"], s
        assert r["shape"] == (st["local_m"], st["local_n"], st["local_k"], st["local_count"]), s
        assert sorted(r["dist"]) == sorted(st["dist_modes"]), s
        assert sorted(r["local"]) == sorted(st["local_modes"]), s
        assert math.isclose(r["t_gemm"], st["t_gemm"], rel_tol=REL, abs_tol=1e-18), s
        assert math.isclose(r["t_comm"], st["t_comm"], rel_tol=REL, abs_tol=1e-18), s
    return md, steps, total, best


def _size_quantile_threshold(net, tree, q, eb=8):
    order = planner.lifetime_orders(net.leaves, net.out_modes, tree.lhs, tree.rhs)
    L = net.num_leaves
    sizes = sorted(eb * math.prod(int(net.extents[x]) for x in o) for o in order[L:])
    return int(sizes[min(len(sizes) - 1, int(q * len(sizes)))])


def _max_chain(md):
    split, carry, _ = md.structure()
    return max([len(c) for c, _ in md.chains(split, carry)] + [0])


@pytest.mark.parametrize("seed", range(40))
def test_random_networks_schedule_is_optimal(seed):
    rng = np.random.default_rng(5000 + seed)
    net = randnet.random_network(rng, n_leaves=int(rng.integers(3, 12)), n_closed=int(rng.integers(4, 22)),
                                 n_open=int(rng.integers(0, 4)), extent_choices=(2, 2, 3, 4), with_data=False)
    tree = randnet.random_tree(rng, net.num_leaves) if seed % 2 else trees.greedy_tree(net)
    P = int(rng.choice([2, 3, 4, 8]))
    thr = _size_quantile_threshold(net, tree, float(rng.uniform(0.2, 0.8)))
    md = OD.model(net.extents, net.leaves, net.out_modes, tree.lhs, tree.rhs, P=P, threshold=thr)
    if _max_chain(md) > 14:
        pytest.skip("chain too long for the exhaustive oracle")
    try:
        md.best()
    except ValueError:
        with pytest.raises(qa.TncError):
            qa.Plan.from_network(net, tree).distribute(num_gpus=P, threshold_bytes=thr)
        return
    _check_optimal(net, tree, num_gpus=P, threshold_bytes=thr,
                   latency_s=float(rng.choice([0.0, 5e-6, 1e-3])), net_bytes_per_s=float(rng.choice([1e6, 5e11])))


@pytest.mark.parametrize("seed", range(30))
def test_random_caterpillar_chains_schedule_is_optimal(seed):
    """Caterpillar trees give long chains with forced and elective
    re-splits (extents 2, 3, 4 and P = 3 give uneven splits too)."""
    from workloads.network import caterpillar
    rng = np.random.default_rng(7000 + seed)
    nl = int(rng.integers(8, 15))
    net = randnet.random_network(rng, n_leaves=nl, n_closed=int(rng.integers(nl, 2 * nl + 6)),
                                 n_open=int(rng.integers(0, 4)), extent_choices=(2, 2, 3, 4), with_data=False)
    tree = caterpillar(nl, [int(x) for x in rng.permutation(nl)])
    P = int(rng.choice([2, 3, 4, 8]))
    thr = _size_quantile_threshold(net, tree, float(rng.uniform(0.05, 0.4)))
    md = OD.model(net.extents, net.leaves, net.out_modes, tree.lhs, tree.rhs, P=P, threshold=thr)
    if _max_chain(md) > 14:
        pytest.skip("chain too long for the exhaustive oracle")
    _check_optimal(net, tree, num_gpus=P, threshold_bytes=thr, latency_s=float(rng.choice([0.0, 5e-6, 1e-4])),
                   net_bytes_per_s=float(rng.choice([1e5, 1e8, 5e11])))


@pytest.mark.parametrize("P,q", [(2, 0.5), (4, 0.6), (8, 0.7)])
def test_circuit_and_peps_schedules_are_optimal(P, q):
    for net, tree in [(circuits.brickwork(12, 10, 3).to_network(open_qubits=[0, 5]), None),
                      (lattice.peps(4, 4, 1), lattice.row_major_tree(4)),
                      (lattice.peps(4, 4, 1), lattice.column_major_tree(4))]:
        net.data = None
        tree = tree or trees.greedy_tree(net)
        thr = _size_quantile_threshold(net, tree, q)
        md = OD.model(net.extents, net.leaves, net.out_modes, tree.lhs, tree.rhs, P=P, threshold=thr)
        if _max_chain(md) > 14:
            continue
        _check_optimal(net, tree, num_gpus=P, threshold_bytes=thr)


# ---------------------------------------------------------------------------
# pins of the oracle


def test_one_gpu_or_huge_threshold_is_the_replicated_roofline_sum():
    net = lattice.peps(4, 4, 1)
    tree = lattice.row_major_tree(4)
    order = planner.lifetime_orders(net.leaves, net.out_modes, tree.lhs, tree.rhs)
    expect = 0.0
    for a, b in zip(tree.lhs, tree.rhs):
        K = set(order[a]) & set(order[b])
        m = math.prod(int(net.extents[x]) for x in order[a] if x not in K)
        n = math.prod(int(net.extents[x]) for x in order[b] if x not in K)
        k = math.prod(int(net.extents[x]) for x in K)
        expect += max(8 * (m * k + n * k + m * n) / 8.0e12, 8 * m * n * k / 157.3e12)
    for P, thr in [(1, 0), (8, 1 << 60)]:
        md = OD.model(net.extents, net.leaves, net.out_modes, tree.lhs, tree.rhs, P=P, threshold=thr)
        best, recs, _, _ = md.best()
        assert all(r["tag"] == OD.REPLICATED for r in recs.values())
        assert math.isclose(best, expect, rel_tol=1e-12)


def test_split_work_is_conserved_and_prefix_is_shortest():
    """With extent-2 modes and P a power of two every split has exactly P
    slices: the GPUs' sub-GEMMs add up to the step.  Every activation splits
    on the shortest prefix of the product's order (taken here from the
    independent death-sort formulation of the orders) covering P."""
    net = circuits.brickwork(14, 12, 7).to_network(open_qubits=[0, 3, 9])
    tree = trees.greedy_tree(net)
    ds = planner.death_sort_orders(net.leaves, net.out_modes, tree.lhs, tree.rhs)
    L = net.num_leaves
    for P in (2, 4, 8):
        thr = _size_quantile_threshold(net, tree, 0.6)
        md = OD.model(net.extents, net.leaves, net.out_modes, tree.lhs, tree.rhs, P=P, threshold=thr)
        best, recs, carry, _ = md.best()
        for s, r in recs.items():
            if r["tag"] == OD.REPLICATED:
                continue
            m, n, k = md.sides(s)
            lm, ln, lk, cnt = r["shape"]
            assert cnt * lm * ln * lk * P == m * n * k, s
            if r["tag"] == OD.ACTIVATE:
                pre, q = [], 1
                for x in ds[L + s]:
                    pre.append(x)
                    q *= int(net.extents[x])
                    if q >= P:
                        break
                assert r["dist"] == pre


def _forced_only_tags(md):
    """Keep until a split mode is about to be reduced, then re-split on the
    fresh prefix: the schedule with the fewest re-splits."""
    split, carry, _ = md.structure()
    tags = {}
    for steps, merge in md.chains(split, carry):
        D = md.prefix(md.out(steps[0]))
        for i in range(1, len(steps)):
            s = steps[i]
            whole = not split[md.out(s)]
            if not whole and any(x in md.K[s] for x in D):
                D = md.prefix(md.out(steps[i - 1]), exclude=md.K[s])
                tags[s] = OD.REDISTRIBUTE
    return [tags.get(s, 0) for s in range(md.S)]


def _imbalance_network():
    """P = 3: the first split [a, c] has Q = 4 slices (two per GPU, so one
    GPU does half the work); from step 1 on, the product also carries an
    extent-3 open mode e that lives longest, so a re-split onto [e] gives
    one slice per GPU.  Modes: a 0, c 1, q 2, v 3, e 4, w 5, x 6."""
    ext = np.array([2, 2, 2, 512, 3, 512, 512], dtype=np.int64)
    leaves = [[0, 1, 2], [2, 3], [3, 4, 5], [5, 6], [0, 1, 6]]
    return Network(ext, leaves, [4], None, name="imbalance"), Tree([0, 5, 6, 7], [1, 2, 3, 4])


def test_elective_resplit_follows_the_price_of_communication():
    """Section 1.5: a re-split may be chosen to make later GEMMs denser.
    With free communication the optimum re-splits onto the balanced prefix;
    with prohibitive communication it keeps the first split."""
    net, tree = _imbalance_network()
    free = OD.model(net.extents, net.leaves, net.out_modes, tree.lhs, tree.rhs, P=3, threshold=1024,
                    B_net=1e300, lam=0.0)
    best, recs, _, _ = free.best()
    assert [recs[s]["tag"] for s in range(4)] == [OD.ACTIVATE, OD.KEEP, OD.REDISTRIBUTE, OD.GATHER]
    assert recs[0]["dist"] == [0, 1] and recs[0]["shape"][3] == 2 and recs[2]["dist"] == [4]
    assert recs[2]["shape"][3] == 1
    assert math.isclose(best, sum(r["t_gemm"] for r in recs.values()), rel_tol=1e-12)
    dear = OD.model(net.extents, net.leaves, net.out_modes, tree.lhs, tree.rhs, P=3, threshold=1024,
                    B_net=1.0, lam=1.0)
    best, recs, _, _ = dear.best()
    assert [recs[s]["tag"] for s in range(4)] == [OD.ACTIVATE, OD.KEEP, OD.KEEP, OD.GATHER]
    for kw in (dict(net_bytes_per_s=1e300, latency_s=0.0), dict(net_bytes_per_s=1.0, latency_s=1.0)):
        _check_optimal(net, tree, num_gpus=3, threshold_bytes=1024, **kw)


def _valley_network():
    """A chain whose first split mode a dies at step 3 while the tensor is
    large; the tensor passes a small "valley" (step 1's output) carrying a
    longer-lived mode b.  Modes: q 0, a 1, v 2, b 3, g 4, z 5, y 6."""
    ext = np.array([2, 2, 1024, 2, 64, 4096, 64], dtype=np.int64)
    leaves = [[1, 0], [0, 2], [2, 3, 4], [5], [1, 5, 6], [4, 6]]
    # step 0: L0 L1 -> [a v]; 1: (+L2) -> [b g a]; 2: (+L3) -> [b g a z];
    # 3: (+L4) -> [b g y]; 4: (+L5) -> [b] (root)
    return Network(ext, leaves, [3], None, name="valley"), Tree([0, 6, 7, 8, 9], [1, 2, 3, 4, 5])


def test_redistribution_goes_to_the_size_valley():
    net, tree = _valley_network()
    md = OD.model(net.extents, net.leaves, net.out_modes, tree.lhs, tree.rhs, P=2, threshold=1024)
    best, recs, _, _ = md.best()
    tags = [recs[s]["tag"] for s in range(md.S)]
    assert tags == [OD.ACTIVATE, OD.KEEP, OD.REDISTRIBUTE, OD.KEEP, OD.GATHER]
    assert recs[2]["dist"] == [3]
    # the forced-only schedule re-splits the large tensor instead, and costs more
    forced = md.cost_of(_forced_only_tags(md))
    assert _forced_only_tags(md)[3] == OD.REDISTRIBUTE and forced[0] > best
    md2, plan, steps, total = _both(net, tree, num_gpus=2, threshold_bytes=1024)
    assert [s["tag"] for s in steps] == tags
    assert math.isclose(total, best, rel_tol=REL)


def test_options_and_errors():
    net, tree = _valley_network()
    plan = qa.Plan.from_network(net, tree)
    for bad in [dict(num_gpus=0), dict(num_gpus=1 << 20), dict(hbm_bytes_per_s=0.0), dict(flops_per_s=-1.0),
                dict(net_bytes_per_s=0.0), dict(latency_s=-1.0)]:
        with pytest.raises(qa.TncError):
            plan.distribute(**bad)
    steps, total = plan.distribute(num_gpus=1)
    assert all(s["tag_name"] == "replicated" for s in steps)


def _comm_model(P):
    """One tensor T laid out [a(4), b(4), c(8), d(2)] (complex64, 2048 bytes):
    the root of a two-leaf network whose output order is that layout (a
    closed extent-1 mode joins the leaves).  B_net = 1e9 B/s, lambda = 1 us."""
    ext = [4, 4, 8, 2, 1]
    net_leaves = [[0, 1, 2, 3, 4], [4]]
    return OD.model(ext, net_leaves, [0, 1, 2, 3], [0], [1], eb=8, P=P, threshold=1, B_net=1e9, lam=1e-6)


def test_comm_time_hand_worked_cases():
    """t_comm = V / B_net + lambda * n_blk (section 1.6, in words), worked out
    by hand for one tensor; T is id 2 in the model.

    P = 4, re-split from [a] onto [c]: each GPU holds 2048 / 4 = 512 bytes
    laid out [b, c, d]; it keeps one of P pieces of 2048 / 16 = 128 bytes and
    sends the other three: V = 384.  Contiguous runs end where the new cut
    (c) falls: the bytes right of c are d's 2 entries = 16 bytes, so
    n_blk = 384 / 16 = 24.
    P = 4, all-gather of T split on [a]: V = 3 * 512 = 1536 in blocks of
    the 512 bytes right of a (b c d = 64 entries): n_blk = 3.  Split on [c]:
    blocks of 16 bytes (d), n_blk = 96.
    P = 4, all-reduce: V = 2 (P - 1) |T| / P = 3072 bytes in 2 (P - 1) = 6
    messages.
    P = 2, re-split [a] -> [d]: pieces of 2048 / 4 = 512 bytes, V = 512 in
    blocks of 8 bytes (nothing right of d): n_blk = 64; [a] -> [b]: blocks
    of 128 bytes (c d = 16 entries): n_blk = 4.  All-gather on [a]: V = 1024
    in blocks of 512: n_blk = 2.  All-reduce: V = 2048 in 2 messages."""
    a, b, c, d = 0, 1, 2, 3
    m4 = _comm_model(4)
    assert m4.size[2] == 2048 and m4.order[2] == [a, b, c, d]
    cases = [
        (m4.resplit_time(2, [a], [c]), 384e-9 + 24e-6),
        (m4.allgather_time(2, [a]), 1536e-9 + 3e-6),
        (m4.allgather_time(2, [c]), 1536e-9 + 96e-6),
        (m4.allreduce_time(2), 3072e-9 + 6e-6),
    ]
    m2 = _comm_model(2)
    cases += [
        (m2.resplit_time(2, [a], [d]), 512e-9 + 64e-6),
        (m2.resplit_time(2, [a], [b]), 512e-9 + 4e-6),
        (m2.allgather_time(2, [a]), 1024e-9 + 2e-6),
        (m2.allreduce_time(2), 2048e-9 + 2e-6),
    ]
    for i, (got, want) in enumerate(cases):
        assert math.isclose(got, want, rel_tol=1e-12), (i, got, want)
