"""Thin GEMM-class steps on the streaming matrix-core kernel (k_thin_mfma):
a short side of 32, 64 or 128 against a long side of 2^14 rows or more,
K = 16, 32 (and 64 for a short side of 32 or 64), the long side on either operand, random
interleavings of the output modes, a sliced run (beta accumulation), and
shapes that must stay on the tiled GEMM kernels.  Every output entry against
the oracle, |g - r| <= 1e-4 * max(|r|, rms(r))."""

import pytest

from tests.test_gpu_skinny_mfma import _check
from workloads import sweep

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


def test_thin_fallbacks():
    # short side 128 with K = 64, K = 128, and a short side of 256: the tiled GEMM kernels
    for lm, ln, lk in [(7, 14, 6), (6, 15, 7), (15, 8, 4)]:
        net, tree = sweep.network(lm, ln, lk, permuted=True, seed=lm + ln + lk, with_data=True)
        ks = _check(net, tree, kind="gemm")
        assert ks and ks[0].startswith("k_cgemm"), ks
