"""Thin GEMM-class steps on the streaming matrix-core kernel (k_thin_mfma):
a short side of 32, 64 or 128 against a long side of 2^14 rows or more,
K = 16, 32 (and 64 for a short side of 32 or 64), the long side on either operand, random
interleavings of the output modes, a sliced run (beta accumulation), and
shapes that must stay on the tiled GEMM kernels (a run of C that is not a
power of two, too long a K, too wide a short side).  Every output entry against
the oracle, |g - r| <= 1e-4 * max(|r|, rms(r))."""

import numpy as np
import pytest

from tests.test_gpu_skinny_mfma import _check
from workloads import sweep
from workloads.network import Network, Tree

pytestmark = pytest.mark.gpu

# log2 of (long side, short side, K)
CASES = [(14, 6, 4), (15, 6, 5), (14, 6, 6), (16, 6, 6), (14, 7, 4), (15, 7, 5), (17, 6, 4), (15, 5, 4), (16, 5, 5),
         (15, 5, 6)]


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    yield


@pytest.mark.parametrize("i", range(len(CASES)))
@pytest.mark.parametrize("side", [0, 1])
@pytest.mark.parametrize("permuted", [False, True], ids=["aligned", "permuted"])
def test_thin_steps(i, side, permuted):
    logl, logs, logk = CASES[i]
    lm, ln = (logl, logs) if side == 0 else (logs, logl)
    net, tree = sweep.network(lm, ln, logk, permuted=permuted, seed=300 + 7 * i + side, with_data=True)
    _check(net, tree, expect_kernel="k_thin_mfma", kind="gemm")


def test_thin_sliced_accumulates():
    net, tree = sweep.network(6, 14, 5, permuted=True, seed=17, with_data=True)
    # slicing a reduced mode: the step accumulates the two slices into the output
    _check(net, tree, expect_kernel="k_thin_mfma", kind="gemm", sliced=[20])


def test_thin_shape_with_extent3_mode_falls_back():
    # 3 * 2^13 long-side rows, a short side of 64, K = 32: one run of C is not a
    # power of two, so the step stays on the tiled GEMM kernel
    rng = np.random.default_rng(21)
    ext = [3] + [2] * 13 + [2] * 6 + [2] * 5
    M, N, K = list(range(14)), list(range(14, 20)), list(range(20, 25))
    A = rng.standard_normal([ext[x] for x in M + K]) + 1j * rng.standard_normal([ext[x] for x in M + K])
    B = rng.standard_normal([ext[x] for x in N + K]) + 1j * rng.standard_normal([ext[x] for x in N + K])
    out = [14, 0, 15, 1, 2, 16, 3, 4, 5, 17, 6, 7, 8, 18, 9, 10, 11, 19, 12, 13]
    net = Network(np.array(ext, dtype=np.int64), [M + K, N + K], out,
                  [A.astype(np.complex64), B.astype(np.complex64)], name="thin_extent3")
    ks = _check(net, Tree([0], [1]), kind="gemm")
    assert ks and ks[0].startswith("k_cgemm"), ks


def test_thin_fallbacks():
    # short side 128 with K = 64, K = 128, and a short side of 256: the tiled GEMM kernels
    for lm, ln, lk in [(7, 14, 6), (6, 15, 7), (15, 8, 4)]:
        net, tree = sweep.network(lm, ln, lk, permuted=True, seed=lm + ln + lk, with_data=True)
        ks = _check(net, tree, kind="gemm")
        assert ks and ks[0].startswith("k_cgemm"), ks
