"""Skinny steps on the matrix-core kernel with address-ordered stores
(k_skinny_mfma): every output entry against the oracle, for S = 1 ... 16
outputs per row with K = 2 ... 64, GEMM-class steps with a short side of 32
(K = 2 ... 8; the long side on either operand, so that the kernel also runs
with operands and runs exchanged), random interleavings of the output modes
(so the stores walk runs of every length), a sliced run (beta accumulation)
and shapes that must fall back to the other kernels.
|g - r| <= 1e-4 * max(|r|, rms(r))."""

import numpy as np
import pytest

import oracle
import quantum_circuit_simulation_amd as qa
from tests.conftest import rel_err_ok
from workloads import sweep
from workloads.network import Network, Tree

pytestmark = pytest.mark.gpu

TOL = 1e-4


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    yield


def _check(net, tree, expect_kernel=None, kind="skinny", **kw):
    import torch
    plan = qa.Plan.from_network(net, tree, **kw)
    leaves = [torch.from_numpy(np.ascontiguousarray(d)).cuda() for d in net.data]
    size = int(np.prod(plan.out_shape, dtype=np.int64)) if plan.out_shape else 1
    out = torch.empty(size, dtype=torch.complex64, device="cuda")
    ws = qa.alloc_workspace(plan)
    ops = plan.execute_timed(leaves, out, ws)
    torch.cuda.synchronize()
    got = out.cpu().numpy().astype(np.complex128).reshape(plan.out_shape)
    ref = oracle.contract_network(net, tree)
    ok, err = rel_err_ok(got, ref, TOL)
    kernels = [o["kernel"] for o in ops if o["kind"] == kind]
    print(f"[gpu] {net.name} kw={kw} kernels={kernels} err {err:.2e}", flush=True)
    assert ok, err
    if expect_kernel is not None:
        assert kernels and all(k.startswith(expect_kernel) for k in kernels), kernels
    return kernels


CASES = [(14, 0, 1), (12, 4, 4), (13, 3, 3), (14, 4, 2), (12, 2, 5), (15, 1, 4), (16, 4, 1), (13, 0, 5),
         (13, 3, 2), (14, 2, 3), (17, 4, 4), (14, 1, 1), (13, 4, 6), (12, 2, 6), (14, 0, 6)]
# GEMM-class steps (short side 32, K <= 8): log2 of (long side, K); up to
# 2^14 rows the small-GEMM kernel takes them
GEMM_CASES = [(15, 1), (16, 2), (15, 3), (17, 2), (18, 1), (17, 3)]


@pytest.mark.parametrize("i", range(len(CASES)))
@pytest.mark.parametrize("side", [0, 1])
def test_skinny_mfma_interleaved_outputs(i, side):
    logr, logs, logk = CASES[i]
    lm, ln = (logr, logs) if side == 0 else (logs, logr)
    net, tree = sweep.network(lm, ln, logk, permuted=True, seed=40 + 7 * i + side, with_data=True)
    _check(net, tree, expect_kernel="k_skinny_mfma")


@pytest.mark.parametrize("i", range(len(GEMM_CASES)))
@pytest.mark.parametrize("side", [0, 1])
def test_short_side_32_gemm_steps(i, side):
    logr, logk = GEMM_CASES[i]
    lm, ln = (logr, 5) if side == 0 else (5, logr)
    net, tree = sweep.network(lm, ln, logk, permuted=True, seed=90 + 5 * i + side, with_data=True)
    _check(net, tree, expect_kernel="k_skinny_mfma", kind="gemm")


def test_skinny_mfma_aligned_and_sliced():
    net, tree = sweep.network(14, 4, 4, seed=5, with_data=True)
    _check(net, tree, expect_kernel="k_skinny_mfma")
    # slicing a reduced mode: the root step accumulates the two slices
    _check(net, tree, expect_kernel="k_skinny_mfma", sliced=[20])


def _with_extent3():
    rng = np.random.default_rng(3)
    # rows: 2^12 * 3 (one extent-3 mode), S = 8, K = 8: runs are not all powers of two
    ext = [2] * 12 + [3] + [2] * 3 + [2] * 3
    M, N, K = list(range(13)), list(range(13, 16)), list(range(16, 19))
    A = (rng.standard_normal([ext[x] for x in M + K]) + 1j * rng.standard_normal([ext[x] for x in M + K]))
    B = (rng.standard_normal([ext[x] for x in N + K]) + 1j * rng.standard_normal([ext[x] for x in N + K]))
    out = [0, 13, 1, 2, 14, 3, 4, 5, 6, 7, 8, 15, 9, 10, 11, 12]
    return Network(np.array(ext, dtype=np.int64), [M + K, N + K], out,
                   [A.astype(np.complex64), B.astype(np.complex64)], name="extent3"), Tree([0], [1])


def test_fallbacks_keep_the_other_skinny_kernels():
    net, tree = _with_extent3()
    ks = _check(net, tree)
    assert ks and not ks[0].startswith("k_skinny_mfma"), ks
    net, tree = sweep.network(13, 3, 7, permuted=True, seed=9, with_data=True)   # K = 128
    ks = _check(net, tree)
    assert ks and not ks[0].startswith("k_skinny_mfma"), ks
    # short side 32 with K = 128, and short side 64 with K = 8: the tiled GEMM kernels
    for lm, ln, lk in [(15, 5, 7), (6, 15, 3)]:
        net, tree = sweep.network(lm, ln, lk, permuted=True, seed=lm + ln + lk, with_data=True)
        ks = _check(net, tree, kind="gemm")
        assert ks and ks[0].startswith("k_cgemm"), ks
