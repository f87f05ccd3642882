"""GPU parity for GEMM-class steps with few rows, a short K and many columns
(after orientation: 16 < R <= 64, K from 8 to 128, S >= 2^16, one K split:
the PEPS and honeycomb bulk shapes, run by the persistent GEMM kernel with
64 x 256 or 32 x 256 tiles).  Every output entry is compared with the oracle
on the same seeded inputs (|g - r| <= 1e-4 max(|r|, rms(r))).

Cases: both row-tile heights (R <= 32 and R <= 64), K = 8 (one K stage), 20,
24 and 40 (odd stage counts, K not a power of two), 64 and 128, ragged R and S (extent-3 modes: S not a multiple of the tile width),
outputs that allow paired 16-byte stores and ones that do not (odd innermost
extent), staged (re-laid) leaves, and a sliced shared mode, whose slices are
added into the output."""

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


def _pair(m_ext, n_ext, k_ext, seed, out_order=None, lhs_order=None, sliced_ext=0):
    """Pairwise network: lhs over [M | K], rhs over [N | K] (mode extents as
    given), output [M | N] unless ``out_order`` (a permutation of M + N
    positions) is given; ``lhs_order`` permutes the lhs declaration (staged
    leaf).  ``sliced_ext`` > 0 adds one more shared mode of that extent, to be
    sliced."""
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
    A, B = M + K, N + K
    if lhs_order is not None:
        A = [A[i] for i in lhs_order]
    out = M + N
    if out_order is not None:
        out = [out[i] for i in out_order]
    data = [sweep.complex_gaussian(rng, tuple(int(extents[x]) for x in A)),
            sweep.complex_gaussian(rng, tuple(int(extents[x]) for x in B))]
    name = f"xres m={int(np.prod(m_ext))} n={int(np.prod(n_ext))} k={int(np.prod(k_ext))}"
    return Network(extents, [A, B], out, data, name=name), Tree([0], [1])


def _oriented(plan):
    nd = plan.node(0)
    R = nd["n"] if nd["swap"] else nd["m"]
    S = nd["m"] if nd["swap"] else nd["n"]
    return nd, R, S


def _check(net, tree, sliced=()):
    from tests.gpu_util import run
    print(f"[gpu] {net.name} sliced={list(sliced)}", flush=True)
    got, plan = run(net, tree, sliced=list(sliced))
    nd, R, S = _oriented(plan)
    k = nd["k"]
    # a few-rows, short-K, many-columns GEMM step
    assert nd["kernel_class"] == 2 and nd["splits"] == 1
    assert 16 < R <= 64 and S >= 1 << 16 and k % 4 == 0 and 8 <= k <= 128, (R, S, k)
    ref = oracle.contract_network(net, tree)
    ok, err = rel_err_ok(got, ref, TOL)
    assert ok, f"max scaled error {err:.3e}"


CASES = [
    # (M extents, N extents, K extents): M is the short side
    ([2] * 6, [2] * 16, [2] * 6),        # R = 64, K = 64 (the PEPS bulk shape, smaller)
    ([2] * 5, [2] * 16, [2] * 3),        # R = 32, K = 8: one K stage per tile
    ([2] * 6, [2] * 16, [2] * 7),        # R = 64, K = 128
    ([3] * 3, [3] * 11, [2] * 4),        # R = 27, S = 3^11 (last tile partial), K = 16
    ([2, 3, 7], [2] * 15 + [3], [2] * 5),  # R = 42, S = 3 * 2^15, K = 32
    ([2] * 6, [2] * 16, [2, 2, 2, 3]),   # R = 64, K = 24: three K stages per block
    ([3, 2, 2, 2, 2], [2] * 14 + [5], [2, 2, 2, 5]),  # R = 48, S = 5 * 2^14, K = 40
    ([2] * 5, [2] * 16, [2, 2, 5]),      # R = 32, K = 20: the last K stage partly empty
]


@pytest.mark.parametrize("case", CASES, ids=lambda c: f"R{int(np.prod(c[0]))}S{int(np.prod(c[1]))}K{int(np.prod(c[2]))}")
def test_few_rows_short_k_blocked_output(case):
    net, tree = _pair(*case, seed=7000 + int(np.prod(case[2])))
    _check(net, tree)


def test_few_rows_short_k_interleaved_and_staged():
    """Output [M_hi | N_hi | M_lo | N_lo] with an extent-2 innermost mode on
    the column side (paired stores), and a re-laid lhs declaration."""
    m_ext, n_ext, k_ext = [2] * 6, [2] * 16, [2] * 6
    nm, nn = 6, 16
    order = list(range(3)) + list(range(nm, nm + 13)) + list(range(3, nm)) + list(range(nm + 13, nm + nn))
    rng = np.random.default_rng(5)
    lhs = list(rng.permutation(nm + 6))
    net, tree = _pair(m_ext, n_ext, k_ext, seed=7101, out_order=order, lhs_order=lhs)
    _check(net, tree)


def test_few_rows_short_k_odd_innermost_extent():
    """Innermost output mode of extent 3 on the column side: entry-by-entry
    stores instead of paired ones."""
    m_ext, n_ext, k_ext = [2] * 4 + [3], [2] * 15 + [3], [2] * 4
    nm, nn = 5, 16
    # [N_hi | M | N_last]: N's last mode (extent 3) is a run of its own, innermost
    order = list(range(nm, nm + nn - 1)) + list(range(nm)) + [nm + nn - 1]
    net, tree = _pair(m_ext, n_ext, k_ext, seed=7102, out_order=order)
    _check(net, tree)


def test_few_rows_short_k_sliced_shared_mode_accumulates():
    """A shared mode of extent 2 is sliced: each slice's step (K = 64) is
    added into the output."""
    net, tree = _pair([2] * 6, [2] * 16, [2] * 6, seed=7103, sliced_ext=2)
    sliced = [net.num_modes - 1]
    from tests.gpu_util import run
    print(f"[gpu] {net.name} sliced", flush=True)
    got, plan = run(net, tree, sliced=sliced)
    assert plan.stats()["num_slices"] == 2
    nd, R, S = _oriented(plan)
    assert nd["kernel_class"] == 2 and R == 64 and S == 1 << 16
    ref = oracle.contract_network(net, tree)
    ok, err = rel_err_ok(got, ref, TOL)
    assert ok, f"max scaled error {err:.3e}"
