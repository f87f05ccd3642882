"""K-reduction steps (k_kred_valu, k_kred_mfma): both output sides at most 32
and a long K that the plan splits into chunks, as in the closing steps of
amplitude trees.  Every output entry against the oracle for the vector-ALU
form (R S <= 16, the longer side on the rows: 4 x 4, 8 x 2, 16 x 1, from
either operand side) and the matrix-core form (8 x 8, 32 x 8, 16 x 32,
32 x 32), aligned and permuted output orders
(the split-K reduction writes C through its runs), a sliced run (beta
accumulation), and a step whose K chunks are not whole multiples of 32
entries, which must stay on the other kernels.
|g - r| <= 1e-4 * max(|r|, rms(r))."""

import numpy as np
import pytest

from tests.test_gpu_skinny_mfma import _check
from workloads import sweep
from workloads.network import Network, Tree

pytestmark = pytest.mark.gpu

# log2 of (m, n, k); skinny-class steps put the longer side on the rows
VALU = [(2, 2, 20), (1, 3, 19), (3, 1, 19), (0, 4, 19), (4, 0, 19)]
MFMA = [(3, 3, 19), (5, 3, 18), (4, 5, 18), (5, 5, 18)]


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    yield


def _kind(lm, ln):
    return "gemm" if min(lm, ln) > 4 else "skinny"


@pytest.mark.parametrize("case", VALU + MFMA, ids=lambda c: f"m{c[0]}n{c[1]}k{c[2]}")
@pytest.mark.parametrize("permuted", [False, True], ids=["aligned", "permuted"])
def test_kred_steps(case, permuted):
    lm, ln, lk = case
    net, tree = sweep.network(lm, ln, lk, permuted=permuted, seed=500 + lm + 3 * ln + lk, with_data=True)
    expect = "k_kred_valu" if (1 << (lm + ln)) <= 16 and min(lm, ln) <= 4 else "k_kred_mfma"
    ks = _check(net, tree, expect_kernel=expect, kind=_kind(lm, ln))
    assert all(k.endswith("+k_split_reduce") for k in ks), ks


def test_kred_sliced_accumulates():
    net, tree = sweep.network(5, 5, 18, permuted=True, seed=7, with_data=True)
    # slicing one reduced mode: the step accumulates the two slices into the output
    _check(net, tree, expect_kernel="k_kred_mfma", kind="gemm", sliced=[12])
    net, tree = sweep.network(2, 2, 20, permuted=True, seed=8, with_data=True)
    _check(net, tree, expect_kernel="k_kred_valu", kind="skinny", sliced=[6])


def test_ragged_chunks_stay_on_the_other_kernels():
    # K = 3^9 * 2^4: the plan's 256 chunks are not whole multiples of 32 entries
    rng = np.random.default_rng(11)
    ext = [2, 2, 2, 2] + [3] * 9 + [2] * 4
    M, N, K = [0, 1], [2, 3], list(range(4, 17))
    A = rng.standard_normal([ext[x] for x in M + K]) + 1j * rng.standard_normal([ext[x] for x in M + K])
    B = rng.standard_normal([ext[x] for x in N + K]) + 1j * rng.standard_normal([ext[x] for x in N + K])
    net = Network(np.array(ext, dtype=np.int64), [M + K, N + K], [2, 0, 3, 1],
                  [A.astype(np.complex64), B.astype(np.complex64)], name="ragged_k")
    ks = _check(net, Tree([0], [1]))
    assert ks and not ks[0].startswith("k_kred"), ks
