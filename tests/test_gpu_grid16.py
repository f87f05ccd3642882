"""The 56-qubit 7x8 grid at depth 16 on its stored tree and slicing, at full
size (one slice has intermediates of up to 2^33 entries and a workspace of
144 GiB).  Pinned by the monomial circuit of the same shape: one
basis-state path carries the whole amplitude e^(i alpha), so the slice whose
digits are that path's values of the sliced modes returns e^(i alpha) (to
the complex64 tolerance) and every other slice returns exactly zero."""

import numpy as np
import pytest

import quantum_circuit_simulation_amd as qa
from tests.brute import monomial_mode_values, track_basis_state
from workloads import circuits, trees

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    yield


def test_grid_7x8_depth16_monomial_slices():
    import torch
    c = circuits.grid_monomial(7, 8, 16, 505)
    gates = [(a, b, u.astype(np.complex64).astype(np.complex128)) for a, b, u in c.gates]
    bits, amp = track_basis_state(56, gates)
    net = c.to_network(bits=bits)
    vals, _ = monomial_mode_values(net, gates, 56)
    tree, sliced, rec = trees.stored_tree("grid_7x8_d16")
    s = len(sliced)
    star = sum(vals[x] << (s - 1 - i) for i, x in enumerate(sliced))
    leaves = [torch.from_numpy(d).to("cuda") for d in net.data]
    out = torch.empty(1, dtype=torch.complex64, device="cuda")
    ws = None
    for sigma, want in ((star, amp), (star ^ 1, 0j), (star ^ (1 << (s - 1)), 0j)):
        print(f"[gpu] grid 7x8 d16 monomial, slice {sigma} of {1 << s}", flush=True)
        plan = qa.Plan.from_network(net, tree, sliced=sliced, slice_range=(sigma, sigma + 1))
        if ws is None:
            ws = qa.alloc_workspace(plan)
        plan.execute(leaves, out, ws)
        torch.cuda.synchronize()
        got = complex(out.cpu().numpy()[0])
        if want == 0:
            assert got == 0, (sigma, got)
        else:
            assert abs(got - want) <= 1e-4 * abs(want), (sigma, got, want)
