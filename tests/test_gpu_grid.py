"""GPU parity for the grid-circuit family (2-D couplers A, B, C, D with
fSim-form gates), including the slice driver at full size.

* random gates, reduced 4x5 depth 16: against the oracle, unsliced and sliced;
* monomial gates (permutation x phase) on the 6x6 depth-14 network, the full
  size the bench runs (largest intermediate 2^33 entries): the exact
  amplitude is known by tracking one basis state, and the tree, modes and
  sizes are identical to the random-gate instance.
"""

import numpy as np
import pytest

import oracle
from tests.brute import track_basis_state
from tests.conftest import rel_err_ok
from workloads import circuits, trees

pytestmark = pytest.mark.gpu
TOL = 1e-4


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    yield
    torch.cuda.empty_cache()


def _gates64(c):
    return [(a, b, u.astype(np.complex64).astype(np.complex128)) for a, b, u in c.gates]


def test_reduced_grid_random_gates_sliced_and_unsliced():
    from tests.gpu_util import run
    net = circuits.grid_fsim(4, 5, 16, 505).to_network(open_qubits=[0, 7])
    tree = trees.search_tree(net, trials=40, seed=1)
    ref = oracle.contract_network(net, tree)
    print("[gpu] grid 4x5 d16 random", flush=True)
    got, plan = run(net, tree)
    ok, err = rel_err_ok(got, ref, TOL)
    assert ok, err
    for s in (2, 4):
        sl = trees.choose_slices(net, tree, s)
        got, plan = run(net, tree, sliced=sl)
        assert plan.stats()["num_slices"] == 1 << s
        ok, err = rel_err_ok(got, ref, TOL)
        assert ok, (s, err)


@pytest.mark.parametrize("s", [0, 3])
def test_grid_6x6_d14_monomial_full_size(s):
    from tests.gpu_util import run
    c = circuits.grid_monomial(6, 6, 14, 505)
    bits, amp = track_basis_state(36, _gates64(c))
    net = c.to_network(bits=bits)
    rand = circuits.grid_fsim(6, 6, 14, 505).to_network()
    tree = trees.search_tree(rand, trials=200, seed=1)   # the bench's tree
    sl = trees.choose_slices(net, tree, s) if s else []
    print(f"[gpu] grid 6x6 d14 monomial, sliced on {s} modes", flush=True)
    got, plan = run(net, tree, sliced=sl)
    if s == 0:
        assert plan.stats()["max_intermediate"] == 1 << 33
    ok, err = rel_err_ok(got, amp, TOL)
    assert ok, err
