"""GPU parity for small GEMM-class steps (R S <= 2^19, K <= 512), which run
one workgroup per 32 x 32 block of C with K split over its four waves and
the partial blocks summed in LDS.  Cases: the R S bound itself (512 x 1024),
ragged blocks (extent-3 and extent-5 modes), K odd (single-entry loads), K
that leaves some waves without a stage (K = 20, 12), K at its bound (512,
128 entries per wave), outputs with and without paired 16-byte stores, a
re-laid operand, a sliced shared mode (slices added into the output), and
K just above the bound (the tiled kernel), and skinny-class steps with
fewer than 4096 rows, which take the same kernel.  Every output entry is compared
with the oracle on the same seeded inputs
(|g - r| <= 1e-4 max(|r|, rms(r)))."""

import numpy as np
import pytest

import oracle
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


def _pair(m_ext, n_ext, k_ext, seed, interleave=False, lhs_perm=False, sliced_ext=0):
    rng = np.random.default_rng(seed)
    nm, nn, nk = len(m_ext), len(n_ext), len(k_ext)
    M = list(range(nm))
    N = list(range(nm, nm + nn))
    K = list(range(nm + nn, nm + nn + nk))
    ext = list(m_ext) + list(n_ext) + list(k_ext)
    if sliced_ext:
        K = K + [len(ext)]
        ext.append(sliced_ext)
    extents = np.array(ext, dtype=np.int64)
    out = M + N
    if interleave:
        out = []
        for i in range(max(nm, nn)):
            out += ([M[i]] if i < nm else []) + ([N[i]] if i < nn else [])
    A, B = M + K, N + K
    if lhs_perm:
        A = [A[i] for i in rng.permutation(len(A))]
    data = [sweep.complex_gaussian(rng, tuple(int(extents[x]) for x in A)),
            sweep.complex_gaussian(rng, tuple(int(extents[x]) for x in B))]
    name = f"small m={int(np.prod(m_ext))} n={int(np.prod(n_ext))} k={int(np.prod(k_ext))}"
    return Network(extents, [A, B], out, data, name=name), Tree([0], [1])


def _check(net, tree, sliced=(), small=True):
    from tests.gpu_util import run
    print(f"[gpu] {net.name} sliced={list(sliced)}", flush=True)
    got, plan = run(net, tree, tiny_mnk=0, sliced=list(sliced))
    nd = plan.node(0)
    assert nd["kernel_class"] == 2
    R, S = (nd["n"], nd["m"]) if nd["swap"] else (nd["m"], nd["n"])
    assert (R * S <= 1 << 19 and nd["k"] <= 512) == small, (R, S, nd["k"])
    ref = oracle.contract_network(net, tree)
    ok, err = rel_err_ok(got, ref, TOL)
    assert ok, f"max scaled error {err:.3e}"


CASES = [
    # (M extents, N extents, K extents, interleave, re-laid lhs)
    ([2] * 9, [2] * 10, [2] * 4, False, False),          # 512 x 1024 x 16: the R S bound
    ([2] * 7, [2] * 8, [2] * 6, True, False),            # 128 x 256 x 64, interleaved output
    ([3] * 4, [5, 5, 2, 2], [2, 2, 2, 2, 2, 2], False, False),  # 81 x 100 x 64: ragged blocks
    ([2] * 6, [2] * 6, [3, 3, 3], False, False),         # 64 x 64 x 27: K odd
    ([2] * 5, [3, 3, 3], [5, 2, 2], True, False),        # 32 x 27 x 20: waves 2-3 without a stage
    ([2] * 5, [2] * 5, [3, 2, 2], False, True),          # 32 x 32 x 12, re-laid lhs
    ([2] * 5, [2] * 6, [2] * 9, False, False),           # 32 x 64 x 512: K at its bound
    ([2] * 4 + [3], [2] * 6, [2] * 8, True, False),      # 48 x 64 x 256
    ([2] * 6, [2] * 7, [], False, False),                # 64 x 128 x 1: outer product
    ([3] * 4, [2] * 5 + [3], [3], True, False),          # 81 x 96 x 3, interleaved, K odd
]


@pytest.mark.parametrize("case", CASES, ids=lambda c: f"R{int(np.prod(c[0]))}S{int(np.prod(c[1]))}K{int(np.prod(c[2]))}")
def test_small_gemm(case):
    m, n, k, inter, perm = case
    net, tree = _pair(m, n, k, seed=9100 + int(np.prod(k)), interleave=inter, lhs_perm=perm)
    _check(net, tree)


def test_small_gemm_sliced_accumulates():
    """A shared mode of extent 3 sliced off a 128 x 256 x 64 step: each
    slice's step adds into the output."""
    net, tree = _pair([2] * 7, [2] * 8, [2] * 6, seed=9200, sliced_ext=3)
    _check(net, tree, sliced=[net.num_modes - 1])


def test_small_shape_above_k_bound_uses_tiled_kernel():
    """32 x 64 x 1024: K above the bound, split K on the tiled kernel."""
    net, tree = _pair([2] * 5, [2] * 6, [2] * 10, seed=9300)
    _check(net, tree, small=False)


SKINNY_CASES = [
    # (M extents, N extents, K extents, interleave): skinny class (S <= 16), R < 4096
    ([2] * 9, [2] * 4, [2] * 6, False),     # 512 x 16 x 64
    ([3] * 5, [5], [2, 2, 2, 5], True),     # 243 x 5 x 40, ragged
    ([2] * 10, [2], [3, 3, 3], False),      # 1024 x 2 x 27: K odd
    ([2, 2, 2, 5, 5, 5], [], [3, 2, 2], False),  # 1000 x 1 x 12: matrix-vector
]


@pytest.mark.parametrize("case", SKINNY_CASES, ids=lambda c: f"R{int(np.prod(c[0]))}S{int(np.prod(c[1]))}K{int(np.prod(c[2]))}")
def test_small_skinny_steps(case):
    """Skinny-class steps with fewer than 4096 rows and K <= 512 also run in
    the small-GEMM kernel."""
    from tests.gpu_util import run
    m, n, k, inter = case
    net, tree = _pair(m, n, k, seed=9400 + int(np.prod(k)), interleave=inter)
    print(f"[gpu] {net.name} skinny", flush=True)
    got, plan = run(net, tree, tiny_mnk=0)
    nd = plan.node(0)
    assert nd["kernel_class"] == 1 and nd["splits"] == 1
    ref = oracle.contract_network(net, tree)
    ok, err = rel_err_ok(got, ref, TOL)
    assert ok, f"max scaled error {err:.3e}"
