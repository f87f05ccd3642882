"""tnc_execute enqueues only kernel launches (the descriptors come from a
pinned host copy read by a kernel, or, when the first call on a plan is
captured, from one host-to-device copy), so a caller may capture it in a HIP
graph: every replay (with unrelated eager work and synchronisations in
between) must give the eager result bit for bit."""

import numpy as np
import pytest

from workloads import circuits, lattice, trees

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    yield


@pytest.mark.parametrize("which", ["brickwork12", "peps4x4_sliced"])
def test_graph_replays_match_eager(which):
    import torch
    import quantum_circuit_simulation_amd as qa
    if which == "brickwork12":
        net = circuits.brickwork(12, 8, 101).to_network(open_qubits=[0, 1])
        tree, sliced = trees.greedy_tree(net), []
    else:
        net = lattice.peps(4, 4, 7)
        tree = lattice.row_major_tree(4)
        sliced = trees.choose_slices(net, tree, 1)
    print(f"[gpu] graph capture {which}", flush=True)
    plan = qa.Plan.from_network(net, tree, sliced=sliced)
    leaves = [torch.from_numpy(d).cuda() for d in net.data]
    size = int(np.prod(plan.out_shape)) if plan.out_shape else 1
    out = torch.empty(size, dtype=torch.complex64, device="cuda")
    ws = qa.alloc_workspace(plan)
    plan.execute(leaves, out, ws)
    torch.cuda.synchronize()
    eager = out.clone()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        plan.execute(leaves, out, ws)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        plan.execute(leaves, out, ws)
    for rep in range(5):
        out.fill_(float("nan"))
        torch.randn(1 << 20, device="cuda").sum()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, eager), f"replay {rep} differs from the eager result"


def test_graph_captured_before_first_eager_call():
    """A plan whose first call is captured records the descriptor copy in the
    graph; its replays and its later eager calls match a second plan's eager
    result bit for bit."""
    import torch
    import quantum_circuit_simulation_amd as qa
    net = circuits.brickwork(12, 8, 103).to_network(open_qubits=[0, 1, 2])
    tree = trees.greedy_tree(net)
    print("[gpu] graph capture before the first eager call", flush=True)
    captured, reference = qa.Plan.from_network(net, tree), qa.Plan.from_network(net, tree)
    leaves = [torch.from_numpy(d).cuda() for d in net.data]
    size = int(np.prod(captured.out_shape))
    out = torch.empty(size, dtype=torch.complex64, device="cuda")
    ref = torch.empty_like(out)
    ws, ws_ref = qa.alloc_workspace(captured), qa.alloc_workspace(reference)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        captured.execute(leaves, out, ws)
    reference.execute(leaves, ref, ws_ref)
    torch.cuda.synchronize()
    for rep in range(3):
        out.fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, ref), f"replay {rep} differs from the eager result"
    out.fill_(float("nan"))
    captured.execute(leaves, out, ws)
    torch.cuda.synchronize()
    assert torch.equal(out, ref)
    g.replay()
    torch.cuda.synchronize()
    assert torch.equal(out, ref)
