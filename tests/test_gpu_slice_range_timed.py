"""Slice ranges (partial sums over a contiguous range of slices) and the
timed executor, through the C ABI on the GPU.  Per output entry:
|g - r| <= 1e-4 * max(|r|, rms(r))."""

import numpy as np
import pytest

import oracle
import quantum_circuit_simulation_amd as qa
from tests.conftest import rel_err_ok
from workloads import circuits, sweep, trees

pytestmark = pytest.mark.gpu

TOL = 1e-4


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    yield


def _run(net, tree, **kw):
    import torch
    plan = qa.Plan.from_network(net, tree, **kw)
    leaves = [torch.from_numpy(np.ascontiguousarray(d)).to("cuda") for d in net.data]
    size = int(np.prod(plan.out_shape, dtype=np.int64)) if plan.out_shape else 1
    out = torch.empty(size, dtype=torch.complex64, device="cuda")
    ws = qa.alloc_workspace(plan)
    plan.execute(leaves, out, ws)
    torch.cuda.synchronize()
    return out.cpu().numpy().astype(np.complex128).reshape(plan.out_shape), plan, leaves, out, ws


def test_slice_ranges_add_up_to_the_whole_sum():
    net = circuits.brickwork(12, 8, 101).to_network(open_qubits=[0, 1], name="brickwork12x8")
    tree = trees.greedy_tree(net)
    sl = trees.choose_slices(net, tree, 3)
    ref = oracle.contract_network(net, tree)
    whole, plan, *_ = _run(net, tree, sliced=sl)
    assert plan.stats()["num_slices"] == 8
    parts = [_run(net, tree, sliced=sl, slice_range=r)[0] for r in ((0, 3), (3, 4), (4, 8))]
    for got in (whole, parts[0] + parts[1] + parts[2]):
        ok, err = rel_err_ok(got, ref, TOL)
        assert ok, err
    # one slice alone equals the oracle with the sliced modes fixed to its digits
    # (first sliced mode most significant)
    sigma = 5
    digits = {x: (sigma >> (len(sl) - 1 - i)) & 1 for i, x in enumerate(sl)}
    one = _run(net, tree, sliced=sl, slice_range=(sigma, sigma + 1))[0]
    ok, err = rel_err_ok(one, oracle.contract_network(net, tree, fixed=digits), TOL)
    assert ok, err


def test_timed_execute_matches_execute_and_names_every_launch():
    import torch
    net, tree = sweep.network(11, 11, 7, seed=7, with_data=True)
    got, plan, leaves, out, ws = _run(net, tree)
    ops = plan.execute_timed(leaves, out, ws)
    torch.cuda.synchronize()
    again = out.cpu().numpy().astype(np.complex128).reshape(plan.out_shape)
    assert np.array_equal(again, got)
    assert ops[0]["kind"] == "header" and ops[0]["launches"] == 1
    gemm = [o for o in ops if o["kind"] == "gemm"]
    assert len(gemm) == 1 and gemm[0]["step"] == 0 and gemm[0]["ms"] > 0
    assert gemm[0]["kernel"] == "k_cgemm_tile<128,128>", gemm[0]
    # a sliced tree: every launch ran once per slice and names its kernel
    net = circuits.brickwork(12, 8, 101).to_network(open_qubits=[0, 1], name="brickwork12x8")
    tree = trees.greedy_tree(net)
    sl = trees.choose_slices(net, tree, 2)
    ref, plan, leaves, out, ws = _run(net, tree, sliced=sl)
    ops = plan.execute_timed(leaves, out, ws)
    torch.cuda.synchronize()
    assert np.array_equal(out.cpu().numpy().astype(np.complex128).reshape(plan.out_shape), ref)
    assert ops[0]["launches"] == 1
    for o in ops[1:]:
        assert o["launches"] == 4 and o["kernel"].startswith("k_"), o


def test_peak_probes_are_near_the_published_peaks():
    """tnc_probe_peaks: the no-memory FP32 MFMA loop must sustain most of
    the published 157.3 TFLOP/s, and the copy a sizeable share of 8 TB/s
    (both well below any impossible value)."""
    import torch
    buf = torch.empty(1 << 30, dtype=torch.uint8, device="cuda")
    f, c = qa.tnc.probe_peaks(buf)
    print(f"[gpu] peaks: {f:.1f} TFLOP/s, {c:.0f} GB/s", flush=True)
    assert 100.0 < f < 170.0, f
    assert 2000.0 < c < 8500.0, c
    with pytest.raises(qa.tnc.TncError):
        qa.tnc.probe_peaks(buf[: 1 << 20])
