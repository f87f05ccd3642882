"""One plan executed concurrently on two streams with distinct workspaces and
distinct inputs (the contract of tnc_execute in the C header): interleaved
launches on two default-priority streams must each reproduce the oracle for
their own inputs.  The two networks share their structure (same circuit
layout, different seeded gates), so one plan serves both."""

import numpy as np
import pytest

import oracle
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


@pytest.mark.parametrize("sliced", [0, 2])
def test_one_plan_two_streams(sliced):
    import torch
    import quantum_circuit_simulation_amd as qa
    na = circuits.grid_fsim(4, 4, 10, 71).to_network(open_qubits=[0, 5, 10])
    nb = circuits.grid_fsim(4, 4, 10, 72).to_network(open_qubits=[0, 5, 10])
    assert [list(l) for l in na.leaves] == [list(l) for l in nb.leaves]
    tree = trees.greedy_tree(na)
    sl = trees.choose_slices(na, tree, sliced) if sliced else []
    plan = qa.Plan.from_network(na, tree, sliced=sl)
    ref_a = oracle.contract_network(na, tree)
    ref_b = oracle.contract_network(nb, tree)
    print(f"[gpu] two streams, {len(tree.lhs)} steps, "
          f"sliced={len(sl)}", flush=True)
    la = [torch.from_numpy(d).cuda() for d in na.data]
    lb = [torch.from_numpy(d).cuda() for d in nb.data]
    size = int(np.prod(plan.out_shape))
    outs = [torch.full((size,), float("nan"), dtype=torch.complex64, device="cuda") for _ in range(2)]
    wss = [qa.alloc_workspace(plan) for _ in range(2)]
    streams = [torch.cuda.Stream(), torch.cuda.Stream()]
    torch.cuda.synchronize()
    for _ in range(6):
        for i, leaves in enumerate((la, lb)):
            with torch.cuda.stream(streams[i]):
                plan.execute(leaves, outs[i], wss[i])
    torch.cuda.synchronize()
    for out, ref in zip(outs, (ref_a, ref_b)):
        got = out.cpu().numpy().astype(np.complex128).reshape(plan.out_shape)
        ok, err = rel_err_ok(got, ref, TOL)
        assert ok, err
    # the two inputs really differ
    assert not np.allclose(ref_a, ref_b)


def test_first_calls_from_two_host_threads():
    """A fresh plan's first tnc_execute calls made at the same time from two
    host threads (each on its own stream, workspace and inputs): the pinned
    descriptor copy is made once, under the plan's lock, and both results
    match the oracle; later calls from both threads reuse it."""
    import threading
    import torch
    import quantum_circuit_simulation_amd as qa
    na = circuits.grid_fsim(4, 4, 10, 73).to_network(open_qubits=[1, 6])
    nb = circuits.grid_fsim(4, 4, 10, 74).to_network(open_qubits=[1, 6])
    tree = trees.greedy_tree(na)
    plan = qa.Plan.from_network(na, tree)
    refs = [oracle.contract_network(n, tree) for n in (na, nb)]
    print("[gpu] first calls from two host threads", flush=True)
    leaves = [[torch.from_numpy(d).cuda() for d in n.data] for n in (na, nb)]
    size = int(np.prod(plan.out_shape))
    outs = [torch.full((size,), float("nan"), dtype=torch.complex64, device="cuda") for _ in range(2)]
    wss = [qa.alloc_workspace(plan) for _ in range(2)]
    streams = [torch.cuda.Stream(), torch.cuda.Stream()]
    torch.cuda.synchronize()
    start = threading.Barrier(2)
    errors = []

    def worker(i):
        try:
            start.wait()
            for _ in range(4):
                plan.execute(leaves[i], outs[i], wss[i], stream=streams[i])
            streams[i].synchronize()
        except Exception as e:  # reported below, on the main thread
            errors.append(e)

    threads = [threading.Thread(target=worker, args=(i,)) for i in range(2)]
    for t in threads:
        t.start()
    for t in threads:
        t.join(timeout=60)
    assert not any(t.is_alive() for t in threads)
    assert not errors, errors
    torch.cuda.synchronize()
    for out, ref in zip(outs, refs):
        got = out.cpu().numpy().astype(np.complex128).reshape(plan.out_shape)
        ok, err = rel_err_ok(got, ref, TOL)
        assert ok, err
