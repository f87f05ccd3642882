"""complex128 path (FP64 MFMA GEMM, FP64 skinny/tiny/copy kernels) against
the oracle on complex128 inputs: |g - r| <= 1e-10 * max(|r|, rms(r))."""

import numpy as np
import pytest

import oracle
import quantum_circuit_simulation_amd as qa
from tests.conftest import rel_err_ok
from tests.test_gpu_parity import PAIR_CASES, SKINNY_CASES, _pair
from workloads import circuits, lattice, randnet, trees

pytestmark = pytest.mark.gpu
TOL = 1e-10


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    yield


def _c128(net, seed):
    """The network's leaves redrawn as full-precision complex128 values."""
    rng = np.random.default_rng(seed)
    net.data = [(rng.standard_normal(d.shape) + 1j * rng.standard_normal(d.shape)) / np.sqrt(2.0) for d in net.data]
    return net


def _run(net, tree, **kw):
    from tests.gpu_util import run
    print(f"[gpu] complex128 {net.name} kw={kw}", flush=True)
    return run(net, tree, dtype=qa.TNC_C128, **kw)


@pytest.mark.parametrize("case", PAIR_CASES + SKINNY_CASES)
@pytest.mark.parametrize("permuted", [False, True])
def test_pairwise_shapes_c128(case, permuted):
    R, S, K, ext = case
    net, tree = _pair(R, S, K, seed=sum(case) + permuted, ext=ext, permuted=permuted)
    net = _c128(net, 11 + sum(case))
    ref = oracle.contract_network(net, tree)
    got, _ = _run(net, tree)
    ok, err = rel_err_ok(got, ref, TOL)
    assert ok, err


@pytest.mark.parametrize("seed", range(8))
def test_random_networks_c128(seed):
    rng = np.random.default_rng(4000 + seed)
    net = randnet.random_network(rng, n_leaves=int(rng.integers(2, 10)), n_closed=int(rng.integers(1, 16)),
                                 n_open=int(rng.integers(0, 4)), extent_choices=(1, 2, 3, 4, 5))
    tree = randnet.random_tree(rng, net.num_leaves)
    if trees.tree_cost(net, tree)["max_elems"] > 1 << 20:
        pytest.skip("too wide")
    net = _c128(net, seed)
    ref = oracle.contract_network(net, tree)
    for order in (0, 1):
        got, _ = _run(net, tree, order=order)
        ok, err = rel_err_ok(got, ref, TOL)
        assert ok, err


def test_brickwork_and_slicing_c128():
    c = circuits.brickwork(16, 10, 3)
    net = c.to_network(open_qubits=[0, 1], name="brickwork16x10")
    net.data = [np.asarray(d, dtype=np.complex128) for d in net.data]
    for i, (a, b, u) in enumerate(c.gates):
        net.data[16 + i] = u.reshape(2, 2, 2, 2)          # gates at full precision
    tree = trees.greedy_tree(net)
    ref = oracle.contract_network(net, tree)
    got, _ = _run(net, tree)
    ok, err = rel_err_ok(got, ref, TOL)
    assert ok, err
    sl = trees.choose_slices(net, tree, 3)
    got, plan = _run(net, tree, sliced=sl)
    ok, err = rel_err_ok(got, ref, TOL)
    assert ok, err


def test_peps_c128():
    net = lattice.peps(5, 4, 7)
    net.data = [np.asarray(d, dtype=np.complex128) for d in net.data]
    tree = lattice.row_major_tree(5)
    ref = oracle.contract_network(net, tree)
    got, _ = _run(net, tree)
    ok, err = rel_err_ok(got, ref, TOL)
    assert ok, err
