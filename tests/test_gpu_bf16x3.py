"""The split-bf16 precision mode (TNC_PREC_BF16X3: GEMM-class complex64
steps as hi*hi + hi*lo + lo*hi on the bf16 matrix cores) against the oracle
at the same bar as the exact path: |g - r| <= 1e-4 * max(|r|, rms(r)).
GEMM shapes with ragged tiles, split K and permuted layouts; random
networks; the PEPS 8x8 golden value; full-size sweep cases on sampled
entries."""

import json
import os

import numpy as np
import pytest

import oracle
import quantum_circuit_simulation_amd as qa
from tests.conftest import rel_err_ok
from tests.test_gpu_parity import PAIR_CASES, _pair
from workloads import lattice, randnet, sweep, trees

pytestmark = pytest.mark.gpu
TOL = 1e-4
GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    yield


def _run(net, tree, **kw):
    from tests.gpu_util import run
    print(f"[gpu] bf16x3 {net.name} kw={kw}", flush=True)
    return run(net, tree, precision=qa.PREC_BF16X3, **kw)


GEMM_CASES = [c for c in PAIR_CASES if min(c[3] ** c[0], c[3] ** c[1]) > 16 and c[3] ** (c[0] + c[1] + c[2]) > 1 << 17]


@pytest.mark.parametrize("case", GEMM_CASES)
@pytest.mark.parametrize("permuted", [False, True])
def test_gemm_shapes_bf16x3(case, permuted):
    R, S, K, ext = case
    net, tree = _pair(R, S, K, seed=sum(case) + 3 * permuted, ext=ext, permuted=permuted)
    ref = oracle.contract_network(net, tree)
    got, plan = _run(net, tree)
    assert plan.node(0)["kernel_class"] == qa.CLASS_GEMM
    ok, err = rel_err_ok(got, ref, TOL)
    assert ok, err
    if permuted:
        got, _ = _run(net, tree, order=qa.ORDER_NAIVE)
        ok, err = rel_err_ok(got, ref, TOL)
        assert ok, err


@pytest.mark.parametrize("seed", range(8))
def test_random_networks_bf16x3(seed):
    rng = np.random.default_rng(7100 + seed)
    net = randnet.random_network(rng, n_leaves=int(rng.integers(2, 9)), n_closed=int(rng.integers(4, 16)),
                                 n_open=int(rng.integers(0, 4)), extent_choices=(2, 3, 4, 5))
    tree = randnet.random_tree(rng, net.num_leaves)
    if trees.tree_cost(net, tree)["max_elems"] > 1 << 22:
        pytest.skip("too wide")
    ref = oracle.contract_network(net, tree)
    got, _ = _run(net, tree, tiny_mnk=0)
    ok, err = rel_err_ok(got, ref, TOL)
    assert ok, err


def test_peps_8x8_bf16x3_matches_golden():
    g = json.load(open(os.path.join(GOLDEN, "oracle_values.json")))["peps8x8_D8_seed404"]
    net = lattice.peps(8, 8, 404)
    got, _ = _run(net, lattice.row_major_tree(8))
    ref = complex(g["re"], g["im"])
    assert abs(got.reshape(-1)[0] - ref) <= TOL * abs(ref)


@pytest.mark.parametrize("idx", [32, 35, 44, 20])
def test_sweep_full_size_bf16x3(idx):
    import torch
    from bench import fill_gaussian
    c = sweep.cases()[idx]
    m, n, k = 1 << c["logm"], 1 << c["logn"], 1 << c["logk"]
    A = torch.empty(m * k, dtype=torch.complex64, device="cuda")
    B = torch.empty(n * k, dtype=torch.complex64, device="cuda")
    C = torch.full((m * n,), float("nan"), dtype=torch.complex64, device="cuda")
    fill_gaussian(A, 200)
    fill_gaussian(B, 201)
    net, tree = sweep.network(c["logm"], c["logn"], c["logk"])
    plan = qa.Plan.from_network(net, tree, precision=qa.PREC_BF16X3)
    ws = qa.alloc_workspace(plan)
    print(f"[gpu] bf16x3 sweep m=2^{c['logm']} n=2^{c['logn']} k=2^{c['logk']}", flush=True)
    plan.execute([A, B], C, ws)
    torch.cuda.synchronize()
    assert bool(torch.isfinite(torch.view_as_real(C)).all())
    rng = np.random.default_rng(idx)
    rows = np.sort(rng.choice(m, size=min(m, 48), replace=False))
    cols = np.sort(rng.choice(n, size=min(n, 48), replace=False))
    ri, ci = torch.from_numpy(rows).cuda(), torch.from_numpy(cols).cuda()
    a = A.view(m, k).index_select(0, ri).cpu().numpy()
    b = B.view(n, k).index_select(0, ci).cpu().numpy()
    ref = oracle.pair_block(a, b)
    got = C.view(m, n).index_select(0, ri).index_select(1, ci).cpu().numpy()
    ok, err = rel_err_ok(got, ref, TOL)
    del A, B, C, ws
    torch.cuda.empty_cache()
    assert ok, err
