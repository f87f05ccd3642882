"""Special cases of one pairwise step whose result is exact in any
floating-point summation order, so the GPU output must equal the expected
value bit for bit (the ingestion and lifetime-ordering sections of the
lifetime-ordering write-up fix the step; the special cases are the plain
algebra of C = A.B^T):

* B = delta (an identity over K, paired mode by mode with new open modes N'):
  C is A with K renamed to N', re-laid in the output order.  Every product
  is x*1 or x*0 and every sum adds zeros, so each entry is exact; this pins
  the addressing of A, of the output runs and of split-K partial sums.
* all-ones A and B: every entry of C is k exactly (integers below 2^24),
  which pins that every output entry is written once and sums all of K.

The expected values are the definitions themselves (a transpose of A, the
constant k), not outputs of this library."""

import numpy as np
import pytest

from workloads import sweep
from workloads.network import Network, Tree

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    yield


def _delta_network(R, Kc, ext, seed, permuted, delta_lhs, row_inner=0):
    """Data leaf over [M | K] (R and Kc modes of extent ext), delta leaf over
    [N' | K] with N'_i paired to K_i; output [M | N'].  With ``permuted`` the
    declared orders of both leaves and of the output are seeded shuffles;
    ``row_inner`` > 0 instead lays the output out as [M_hi | N' | M_lo] with
    the last ``row_inner`` modes of M innermost (an interleaved order whose
    innermost run belongs to the data leaf).
    Returns (network, tree, expected output ndarray)."""
    rng = np.random.default_rng(seed)
    M = list(range(R))
    K = list(range(R, R + Kc))
    Np = list(range(R + Kc, R + 2 * Kc))
    A, B, out = M + K, Np + K, M + Np
    if permuted:
        A = [A[i] for i in rng.permutation(len(A))]
        B = [B[i] for i in rng.permutation(len(B))]
        out = [out[i] for i in rng.permutation(len(out))]
    elif row_inner:
        out = M[:R - row_inner] + Np + M[R - row_inner:]
    extents = np.full(R + 2 * Kc, ext, dtype=np.int64)
    a = sweep.complex_gaussian(rng, tuple([ext] * len(A)))
    k = ext ** Kc
    eye = np.eye(k, dtype=np.complex64).reshape([ext] * (2 * Kc))     # axes [N' | K]
    b = np.ascontiguousarray(eye.transpose([(Np + K).index(x) for x in B]))
    # expected: A's axes relabelled K -> N', then laid out in ``out`` order
    relabel = {K[i]: Np[i] for i in range(Kc)}
    a_modes = [relabel.get(x, x) for x in A]
    expected = np.ascontiguousarray(a.transpose([a_modes.index(x) for x in out]))
    leaves = [B, A] if delta_lhs else [A, B]
    data = [b, a] if delta_lhs else [a, b]
    net = Network(extents, leaves, out, data, name=f"delta R={R} Kc={Kc} ext={ext}")
    return net, Tree([0], [1]), expected


# (R, Kc, ext): tiny, skinny (flat and row kernels), persistent GEMM,
# one-tile GEMM (K chunk above 64), split K, ragged extent-3 tiles
DELTA_CASES = [
    (2, 2, 2), (16, 2, 2), (14, 4, 2), (9, 3, 3), (12, 8, 2), (12, 10, 2),
    (8, 11, 2), (7, 5, 3), (8, 6, 3),
]


@pytest.mark.parametrize("delta_lhs", [False, True], ids=["delta_rhs", "delta_lhs"])
@pytest.mark.parametrize("permuted", [False, True], ids=["aligned", "permuted"])
@pytest.mark.parametrize("case", DELTA_CASES, ids=lambda c: f"R{c[0]}K{c[1]}x{c[2]}")
def test_delta_relayout_is_exact(case, permuted, delta_lhs):
    from tests.gpu_util import run
    R, Kc, ext = case
    net, tree, expected = _delta_network(R, Kc, ext, seed=1000 + 10 * R + Kc, permuted=permuted,
                                         delta_lhs=delta_lhs)
    print(f"[gpu] {net.name} permuted={permuted} delta_lhs={delta_lhs}", flush=True)
    got, plan = run(net, tree)
    node = plan.node(0)
    assert got.shape == expected.shape
    bad = np.flatnonzero(got.ravel() != expected.ravel().astype(np.complex128))
    assert bad.size == 0, (f"{bad.size} entries differ (class {node['kernel_class']}, splits {node['splits']}); "
                           f"first at {bad[0]}: {got.ravel()[bad[0]]} vs {expected.ravel()[bad[0]]}")


# (R, Kc, ext, row_inner): interleaved outputs [M_hi | N' | M_lo] whose
# innermost run (extent 2, 8 or 3) belongs to the data leaf, which the
# planner therefore places on the column side (paired stores for even
# extents, single stores for odd); persistent and one-tile GEMM, split K
# (17, 6, ...) and (17, 5, ...): 2^17 columns, 64 / 32 rows, K = 64 / 32
ROW_INNER_CASES = [(12, 8, 2, 1), (12, 8, 2, 3), (12, 10, 2, 3), (8, 11, 2, 1), (8, 6, 3, 1), (14, 6, 2, 3),
                   (17, 6, 2, 3), (17, 5, 2, 1)]


@pytest.mark.parametrize("delta_lhs", [False, True], ids=["delta_rhs", "delta_lhs"])
@pytest.mark.parametrize("case", ROW_INNER_CASES, ids=lambda c: f"R{c[0]}K{c[1]}x{c[2]}in{c[3]}")
def test_delta_interleaved_output_is_exact(case, delta_lhs):
    from tests.gpu_util import run
    R, Kc, ext, inner = case
    net, tree, expected = _delta_network(R, Kc, ext, seed=4000 + R + Kc, permuted=False, delta_lhs=delta_lhs,
                                         row_inner=inner)
    print(f"[gpu] {net.name} row_inner={inner} delta_lhs={delta_lhs}", flush=True)
    got, plan = run(net, tree)
    node = plan.node(0)
    assert node["interleaved"] == 1
    # the data leaf's modes (holding the innermost run) are the columns
    assert node["swap"] == (0 if delta_lhs else 1)
    assert np.array_equal(got, expected.astype(np.complex128))


@pytest.mark.parametrize("case", [(12, 8, 2), (8, 11, 2), (7, 5, 3)], ids=lambda c: f"R{c[0]}K{c[1]}x{c[2]}")
def test_delta_relayout_naive_order_is_exact(case):
    import quantum_circuit_simulation_amd as qa
    from tests.gpu_util import run
    R, Kc, ext = case
    net, tree, expected = _delta_network(R, Kc, ext, seed=2000 + R, permuted=True, delta_lhs=False)
    print(f"[gpu] {net.name} naive", flush=True)
    got, _ = run(net, tree, order=qa.ORDER_NAIVE)
    assert np.array_equal(got, expected.astype(np.complex128))


@pytest.mark.parametrize("case", [(10, 4, 2), (8, 9, 2), (6, 4, 3)], ids=lambda c: f"R{c[0]}K{c[1]}x{c[2]}")
def test_delta_relayout_complex128_is_exact(case):
    import quantum_circuit_simulation_amd as qa
    from tests.gpu_util import run
    R, Kc, ext = case
    net, tree, expected = _delta_network(R, Kc, ext, seed=3000 + R, permuted=True, delta_lhs=False)
    print(f"[gpu] {net.name} complex128", flush=True)
    got, _ = run(net, tree, dtype=qa.TNC_C128)
    assert np.array_equal(got, expected.astype(np.complex128))


# (log2 m, log2 n, log2 k, precision): GEMM (persistent, one-tile,
# split-K, few rows with short K), skinny; the split-bf16 mode represents 1
# exactly (lo part 0)
ONES_CASES = [
    (12, 12, 12, 0), (12, 12, 8, 0), (9, 9, 14, 0), (20, 2, 6, 0), (2, 20, 6, 0), (16, 4, 4, 0),
    (12, 12, 12, 1), (9, 9, 14, 1),
    (6, 17, 3, 0), (5, 17, 7, 0),            # few rows, short K, many columns
]


@pytest.mark.parametrize("case", ONES_CASES, ids=lambda c: f"m{c[0]}n{c[1]}k{c[2]}p{c[3]}")
def test_all_ones_gives_k_everywhere(case):
    import torch
    import quantum_circuit_simulation_amd as qa
    lm, ln, lk, prec = case
    R, S, Kc = lm, ln, lk
    M = list(range(R))
    N = list(range(R, R + S))
    K = list(range(R + S, R + S + Kc))
    net = Network(np.full(R + S + Kc, 2, dtype=np.int64), [M + K, N + K], M + N, None,
                  name=f"ones m=2^{lm} n=2^{ln} k=2^{lk}")
    print(f"[gpu] {net.name} precision={prec}", flush=True)
    plan = qa.Plan.from_network(net, Tree([0], [1]), precision=prec)
    A = torch.ones(1 << (lm + lk), dtype=torch.complex64, device="cuda")
    B = torch.ones(1 << (ln + lk), dtype=torch.complex64, device="cuda")
    C = torch.full((1 << (lm + ln),), float("nan"), dtype=torch.complex64, device="cuda")
    ws = qa.alloc_workspace(plan)
    plan.execute([A, B], C, ws)
    torch.cuda.synchronize()
    want = torch.tensor(float(1 << lk) + 0j, dtype=torch.complex64, device="cuda")
    wrong = int((C != want).sum().item())
    assert wrong == 0, f"{wrong} of {C.numel()} entries differ from k = {1 << lk}"
