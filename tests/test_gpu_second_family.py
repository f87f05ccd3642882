"""GPU parity on the second workload family: honeycomb-lattice networks
(random sites against the oracle; all-ones sites at the full 16 x 16, D = 8
bench size against their closed form), Ising partition functions on
random 3-regular graphs and rings, and the coset weights of surface-code
decoding.  Tolerance as for every complex64 path: |g - r| <= 1e-4 * |r|
(scalars)."""

import math

import numpy as np
import pytest

import oracle
from tests.conftest import rel_err_ok
from workloads import hexagonal as H
from workloads import trees

pytestmark = pytest.mark.gpu
TOL = 1e-4


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    yield


def _run(net, tree, **kw):
    from tests.gpu_util import run
    print(f"[gpu] {net.name} kw={kw}", flush=True)
    return run(net, tree, **kw)


@pytest.mark.parametrize("rows,cols,D,seed", [(8, 8, 8, 1), (12, 12, 8, 2), (10, 14, 4, 3)])
def test_honeycomb_random_matches_oracle(rows, cols, D, seed):
    net = H.honeycomb(rows, cols, D, seed)
    tree = H.honeycomb_tree(rows, cols)
    ref = oracle.contract_network(net, tree)
    got, _ = _run(net, tree)
    ok, err = rel_err_ok(got, ref, TOL)
    assert ok, err


def test_honeycomb_full_size_all_ones_closed_form():
    """16 x 16, D = 8 (width 2^30): all-ones sites halved, so Z is the
    product of the stored site scales times 8^bonds (close to 1)."""
    net = H.honeycomb(16, 16, 8, 0, fill=lambda i, j, shape, rng: np.full(shape, 0.5, np.float32))
    log2z = sum(math.log2(float(np.asarray(d).reshape(-1)[0].real)) for d in net.data) + 3.0 * net.meta["bonds"]
    expect = 2.0 ** log2z
    got, plan = _run(net, H.honeycomb_tree(16, 16))
    assert plan.stats()["max_intermediate"] == 1 << 30
    assert abs(got.reshape(-1)[0] - expect) <= TOL * abs(expect)


@pytest.mark.parametrize("n,seed", [(80, 11), (120, 12)])
def test_ising_random_regular_matches_oracle(n, seed):
    edges = H.random_regular_graph(n, 3, seed)
    net = H.ising(n, edges, 0.4, seed=seed)
    tree = trees.search_tree(net, trials=50, seed=1)
    ref = oracle.contract_network(net, tree)
    got, _ = _run(net, tree)
    ok, err = rel_err_ok(got, ref, TOL)
    assert ok, err
    sl = trees.choose_slices(net, tree, 3)
    got, _ = _run(net, tree, sliced=sl)
    ok, err = rel_err_ok(got, ref, TOL)
    assert ok, err


def test_ising_ring_closed_form():
    n, beta = 100, 0.2
    edges = [(i, i + 1) for i in range(n - 1)] + [(0, n - 1)]
    net = H.ising(n, edges, beta)
    got, _ = _run(net, trees.greedy_tree(net))
    expect = (2 * math.cosh(beta)) ** n + (2 * math.sinh(beta)) ** n
    assert abs(got.reshape(-1)[0] - expect) <= TOL * expect


@pytest.mark.parametrize("d,p,seed", [(5, 0.08, 21), (7, 0.05, 22), (9, 0.05, 23), (11, 0.04, 24)])
def test_surface_code_coset_weights_match_oracle(d, p, seed):
    """Maximum-likelihood decoding of a random bit-flip error on the planar
    surface code: both coset weights, Z(E) and Z(E xor logical), on the GPU
    against the oracle, and the same decision wherever the two weights are
    more than 0.1% apart."""
    from workloads import qec
    E = qec.random_error(d, p, seed)
    G = E.copy()
    G[qec.planar_code(d)[2]] ^= 1
    got, ref = [], []
    for err in (E, G):
        net = qec.coset_network(d, p, err)
        tree = trees.greedy_tree(net)
        r = oracle.contract_network(net, tree)
        g, _ = _run(net, tree)
        ok, e = rel_err_ok(g, r, TOL)
        assert ok, e
        got.append(float(np.asarray(g).reshape(-1)[0].real))
        ref.append(float(np.asarray(r).reshape(-1)[0].real))
    if abs(math.log(ref[0] / ref[1])) > 1e-3:
        assert (got[0] > got[1]) == (ref[0] > ref[1])


def test_surface_code_full_size_exact_values():
    """d = 23 (the bench distance) along the column sweep at p = 0, where
    the coset weight is exactly 1 for the identity's class and 0 for the
    logical's: Z(0) = 1, Z(stabilizer) = 1, Z(logical) = 0."""
    from workloads import qec
    d = 23
    _, support, logical = qec.planar_code(d)
    nq = d * d + (d - 1) ** 2
    tree = qec.sweep_tree(d)
    for err, expect in ((None, 1.0), (support[len(support) // 2], 1.0), (logical, 0.0)):
        E = np.zeros(nq, dtype=np.int64)
        if err is not None:
            E[err] = 1
        got, plan = _run(qec.coset_network(d, 0.0, E), tree)
        assert plan.stats()["max_intermediate"] == 1 << 24
        assert abs(complex(np.asarray(got).reshape(-1)[0]) - expect) <= TOL


def test_surface_code_full_size_relative_weights():
    """The bench instance (d = 23, p = 0.05, seed 707, relative weights):
    both column sweeps agree, and multiplying E by a stabilizer changes the
    relative weight by exactly ((1 - p) / p)^(w(F) - w(E)) (the coset's
    weight is unchanged, the representative's probability is not)."""
    from workloads import qec
    d, p = 23, 0.05
    _, support, _ = qec.planar_code(d)
    E = qec.random_error(d, p, 707)
    z = []
    for rev in (False, True):
        got, _ = _run(qec.coset_network(d, p, E, relative=True), qec.sweep_tree(d, reverse=rev))
        z.append(complex(np.asarray(got).reshape(-1)[0]))
    assert abs(z[0] - z[1]) <= TOL * abs(z[1])
    F = E.copy()
    F[support[100]] ^= 1
    got, _ = _run(qec.coset_network(d, p, F, relative=True), qec.sweep_tree(d))
    r = float(np.float32(1 - p)) / float(np.float32(p))
    expect = z[0] * r ** (int(F.sum()) - int(E.sum()))
    assert abs(complex(np.asarray(got).reshape(-1)[0]) - expect) <= 2 * TOL * abs(expect)
