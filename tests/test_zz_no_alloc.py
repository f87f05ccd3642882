"""tnc_execute_noalloc (the library's static per-GPU workspace) against
tnc_execute (a caller-allocated workspace) on the same plans and inputs, two
calls in a row with the second smaller than the first, then a sliced plan.
Per output entry: |g - r| <= 1e-4 * max(|r|, rms(r))."""

import numpy as np
import pytest

import quantum_circuit_simulation_amd as qa
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


def _both(net, tree, **kw):
    import torch
    plan = qa.Plan.from_network(net, tree, **kw)
    assert plan.workspace_bytes <= qa.tnc.NOALLOC_MAX_WORKSPACE_BYTES
    leaves = [torch.from_numpy(np.ascontiguousarray(d, dtype=np.complex64)).to("cuda") for d in net.data]
    size = int(np.prod(plan.out_shape, dtype=np.int64)) if plan.out_shape else 1
    ref = torch.empty(size, dtype=torch.complex64, device="cuda")
    plan.execute(leaves, ref, qa.alloc_workspace(plan))
    # the static workspace keeps the previous call's bytes: poison `out`
    got = torch.full((size,), complex(float("nan"), float("nan")), dtype=torch.complex64, device="cuda")
    plan.execute_noalloc(leaves, got)
    torch.cuda.synchronize()
    r = ref.cpu().numpy().astype(np.complex128)
    g = got.cpu().numpy().astype(np.complex128)
    assert np.all(np.isfinite(g))
    ok, err = rel_err_ok(g, r, TOL)
    print(f"[noalloc] {net.name} ws={plan.workspace_bytes} entries={size} max scaled diff {err:.2e} "
          f"identical={np.array_equal(g, r)}", flush=True)
    assert ok, err


def test_noalloc_matches_execute_twice_with_smaller_second_call_then_sliced():
    big = circuits.brickwork(30, 14, 303).to_network(open_qubits=range(6), name="brickwork30x14")
    _both(big, trees.greedy_tree(big))
    small = circuits.brickwork(12, 8, 101).to_network(open_qubits=[0, 1], name="brickwork12x8")
    tree = trees.greedy_tree(small)
    _both(small, tree)
    sl = [m for m in range(small.num_modes) if m not in small.out_modes][10:12]
    _both(small, tree, sliced=sl)



def test_noalloc_runs_fused_chains():
    """Plans whose steps run as fused chains (a pair with matrix-core phases
    and a chain of four on the vector ALU) through the static workspace."""
    from tests.test_gpu_fused import chain_n_network, chain_network
    net, tree = chain_network(4, 5, 2, 16, "s", seed=11)
    assert qa.Plan.from_network(net, tree).stats()["fused_pairs"] == 1
    _both(net, tree)
    net, tree = chain_n_network((2, 2, 2, 2), (0, 1, 1, 0), 16, "o", seed=12)
    assert qa.Plan.from_network(net, tree).fused(0)["nsteps"] == 4
    _both(net, tree)
