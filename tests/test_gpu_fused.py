"""Fused chains of steps (k_fused2): a long tensor T absorbs a small W1 (2,
4, 8, 16 or 32 entries of K, as many outputs) and the product is reduced at
once against another small W2 (and, all K <= 8, up to four more), in one
pass over T.  Every output entry of the whole contraction against the
oracle, for (K1, K2) in {4, 8, 16, 32}^2 (the vector-ALU and matrix-core
phases and their mixes), pairs with K = 2, and chains of three to six
steps (K = 2, 4 and 8 mixed), with each later
step reducing 0 .. all of the modes the earlier steps brought in, random
declared orders and output orders (so the chain's product lands in many
layouts), the innermost output mode local to a pass (16-byte pair stores)
or not (single stores), sliced runs, and the same plans with fusion off.
|g - r| <= 1e-4 * max(|r|, rms(r))."""

import numpy as np
import pytest

from tests.test_gpu_skinny_mfma import _check
from workloads.network import Network, Tree

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    yield


def _cn(rng, shape):
    return ((rng.standard_normal(shape) + 1j * rng.standard_normal(shape)) / np.sqrt(2)).astype(np.complex64)


def chain_network(k1, k2, v, log_rows, last, seed, permuted=True, with_data=True):
    """T (outer modes O, A, K1) absorbs W1 (K1 -> S1, 2^k1 x 2^k1), the
    product is reduced against W2 over K2 = v modes of S1 plus the k2 - v
    modes A of T (K2 -> S2), and a last step contracts one mode of the pair's
    product with a vector V (an outer mode for last = "o", a mode of S2 for
    last = "s"), so that the pair's product is not the root.  All extents 2;
    T has 2^log_rows rows of K1 entries."""
    rng = np.random.default_rng(seed)
    n_outer = log_rows - (k2 - v)
    assert n_outer >= 2
    labels = iter(range(1000))
    O = [next(labels) for _ in range(n_outer)]
    K1 = [next(labels) for _ in range(k1)]
    S1 = [next(labels) for _ in range(k1)]
    A = [next(labels) for _ in range(k2 - v)]
    S2 = [next(labels) for _ in range(k2)]
    K2 = S1[:v] + A
    vmode = O[0] if last == "o" else S2[0]
    t_modes, w1_modes, w2_modes = O + A + K1, S1 + K1, S2 + K2
    out = [x for x in O + S1[v:] + S2 if x != vmode]
    if permuted:
        t_modes, w1_modes, w2_modes, out = (list(rng.permutation(m)) for m in (t_modes, w1_modes, w2_modes, out))
    n = next(labels)
    ext = np.full(n, 2, dtype=np.int64)
    leaves = [t_modes, w1_modes, w2_modes, [vmode]]
    data = [_cn(rng, [2] * len(l)) for l in leaves] if with_data else None
    net = Network(ext, [list(map(int, l)) for l in leaves], [int(x) for x in out], data,
                  name=f"chain_k{k1}_{k2}_v{v}_r{log_rows}_{last}")
    return net, Tree([0, 4, 5], [1, 2, 3])


def chain3_network(k1, k2, k3, v2, v3a, v3b, log_rows, last, seed, permuted=True, with_data=True):
    """Three chained absorbs: T (outer modes O, A2, A3, K1) takes W1 (K1 ->
    S1), then W2 over K2 = v2 modes of S1 + the k2 - v2 modes A2 of T (K2 ->
    S2), then W3 over K3 = v3a modes of S2 + v3b further modes of S1 + the
    rest A3 from T (K3 -> S3); a last step contracts one mode of the third
    product with a vector (an outer mode for last = "o", a mode of S3 for
    "s").  All extents 2; T has 2^log_rows rows of K1 entries."""
    rng = np.random.default_rng(seed)
    na2, na3 = k2 - v2, k3 - v3a - v3b
    assert na2 >= 0 and na3 >= 0 and v2 + v3b <= k1 and v3a <= k2
    n_outer = log_rows - na2 - na3
    assert n_outer >= 2
    labels = iter(range(1000))
    take = lambda n: [next(labels) for _ in range(n)]
    O, K1, S1, A2, S2, A3, S3 = take(n_outer), take(k1), take(k1), take(na2), take(k2), take(na3), take(k3)
    K2 = S1[:v2] + A2
    K3 = S2[:v3a] + S1[v2:v2 + v3b] + A3
    vmode = O[0] if last == "o" else S3[0]
    leaves = [O + A2 + A3 + K1, S1 + K1, S2 + K2, S3 + K3]
    out = [x for x in O + S1[v2 + v3b:] + S2[v3a:] + S3 if x != vmode]
    if permuted:
        leaves = [list(rng.permutation(m)) for m in leaves]
        out = list(rng.permutation(out))
    leaves.append([vmode])
    n = next(labels)
    ext = np.full(n, 2, dtype=np.int64)
    data = [_cn(rng, [2] * len(l)) for l in leaves] if with_data else None
    net = Network(ext, [list(map(int, l)) for l in leaves], [int(x) for x in out], data,
                  name=f"chain3_k{k1}{k2}{k3}_v{v2}{v3a}{v3b}_r{log_rows}_{last}")
    return net, Tree([0, 5, 6, 7], [1, 2, 3, 4])


def chain_n_network(ks, vs, log_rows, last, seed, permuted=True, with_data=True):
    """A chain of n = len(ks) absorbs: T (outer modes O, then A_2 .. A_n, then
    K_1) takes W_1 (K_1 -> S_1, 2^ks[0] x 2^ks[0]); step q = 2 .. n reduces
    the product against W_q over K_q = vs[q - 1] modes drawn (seeded) from the
    modes the earlier W's brought in and still open, plus ks[q - 1] -
    vs[q - 1] further modes A_q of T (K_q -> S_q).  A last step contracts one
    mode of the chain's product with a vector (an outer mode for last = "o", a
    mode of S_n for "s").  All extents 2; T has 2^log_rows rows of 2^ks[0]
    entries."""
    rng = np.random.default_rng(seed)
    n = len(ks)
    na = [ks[q] - vs[q] for q in range(1, n)]
    assert min(na) >= 0
    n_outer = log_rows - sum(na)
    assert n_outer >= 2
    labels = iter(range(1000))
    take = lambda c: [next(labels) for _ in range(c)]
    O, K1 = take(n_outer), take(ks[0])
    S = [take(k) for k in ks]
    A = [take(c) for c in na]
    pool = list(S[0])
    ws = [S[0] + K1]
    for q in range(1, n):
        assert vs[q] <= len(pool)
        pick = [pool[i] for i in sorted(rng.choice(len(pool), size=vs[q], replace=False))]
        pool = [x for x in pool if x not in pick] + S[q]
        ws.append(S[q] + pick + A[q - 1])
    vmode = O[0] if last == "o" else S[-1][0]
    leaves = [O + sum(A, []) + K1] + ws
    out = [x for x in O + pool if x != vmode]
    if permuted:
        leaves = [list(rng.permutation(m)) for m in leaves]
        out = list(rng.permutation(out))
    leaves.append([vmode])
    nl = len(leaves)
    ext = np.full(next(labels), 2, dtype=np.int64)
    data = [_cn(rng, [2] * len(l)) for l in leaves] if with_data else None
    name = "chain{}_k{}_v{}_r{}_{}".format(n, "".join(map(str, ks)), "".join(map(str, vs[1:])), log_rows, last)
    net = Network(ext, [list(map(int, l)) for l in leaves], [int(x) for x in out], data, name=name)
    return net, Tree([0] + [nl + q for q in range(n)], list(range(1, n + 2)))


# (log2 K1, log2 K2, shared modes v, log2 rows of T, last-step mode); a
# phase with K <= 8 runs on the vector ALU, K >= 16 on the matrix cores
CASES = [(4, 4, 0, 16, "s"), (4, 4, 2, 17, "s"), (4, 4, 4, 16, "o"), (4, 5, 2, 17, "s"), (5, 4, 1, 16, "s"),
         (5, 5, 3, 17, "o"), (4, 5, 0, 16, "o"), (5, 5, 0, 18, "s"), (5, 4, 4, 17, "o"), (4, 4, 1, 19, "s"),
         (2, 2, 0, 16, "s"), (2, 2, 2, 17, "o"), (2, 3, 1, 16, "s"), (3, 2, 2, 17, "o"), (3, 3, 1, 16, "s"),
         (3, 3, 3, 18, "o"), (2, 2, 1, 19, "s"), (3, 4, 1, 17, "s"), (2, 5, 2, 16, "o"), (5, 3, 2, 17, "s"),
         (4, 2, 1, 16, "s"), (5, 2, 0, 16, "o"), (2, 4, 2, 17, "s"),
         (1, 1, 0, 16, "s"), (1, 2, 1, 17, "o"), (3, 1, 1, 16, "s"), (1, 3, 0, 16, "o")]


@pytest.mark.parametrize("case", CASES, ids=lambda c: "k{}_{}_v{}_r{}_{}".format(*c))
def test_fused_pair_matches_oracle(case):
    net, tree = chain_network(*case, seed=700 + sum(case[:4]))
    ks = _check(net, tree, expect_kernel="k_fused2", kind="fused")
    assert len(ks) == 1, ks


@pytest.mark.parametrize("case", [CASES[0], CASES[3], CASES[5], CASES[10], CASES[15]],
                         ids=["k16_16", "k16_32", "k32_32", "k4_4", "k8_8"])
def test_aligned_orders(case):
    net, tree = chain_network(*case, seed=31, permuted=False)
    _check(net, tree, expect_kernel="k_fused2", kind="fused")


# three-step chains (every K <= 8): (log2 K1, K2, K3, v2, v3a, v3b, log2 rows, last)
CHAIN3 = [(2, 2, 2, 1, 1, 0, 16, "s"), (2, 2, 2, 2, 0, 0, 17, "o"), (3, 2, 3, 1, 1, 1, 16, "s"),
          (2, 3, 2, 0, 2, 0, 17, "s"), (3, 3, 3, 2, 1, 0, 16, "o"), (2, 2, 3, 0, 1, 1, 18, "s")]


@pytest.mark.parametrize("case", CHAIN3, ids=lambda c: "k{}{}{}_v{}{}{}_r{}_{}".format(*c))
def test_fused_chain_of_three_matches_oracle(case):
    net, tree = chain3_network(*case, seed=800 + sum(case[:7]))
    ks = _check(net, tree, expect_kernel="k_fused2", kind="fused")
    assert len(ks) == 1 and ks[0].count(",") == 2, ks   # one k_fused2<K1,K2,K3> launch


# longer chains (every K <= 8, two of the pass's row bits left free): (log2 K
# of each step, shared modes of each later step, log2 rows, last)
CHAINN = [((2, 2, 2, 2), (0, 1, 1, 0), 16, "s"), ((2, 2, 2, 2, 2), (0, 0, 0, 1, 1), 16, "o"),
          ((2, 2, 2, 2, 2, 2), (0, 2, 1, 2, 1, 2), 17, "s"), ((3, 3, 3, 3), (0, 1, 2, 1), 16, "o"),
          ((2, 3, 3, 2), (0, 1, 2, 1), 17, "s"), ((3, 2, 2, 2, 3), (0, 1, 1, 1, 2), 16, "s"),
          ((2, 2, 2, 2, 2), (0, 1, 0, 1, 0), 18, "s"), ((3, 3, 3, 3, 3), (0, 2, 2, 2, 2), 16, "o"),
          ((1, 1, 1, 1), (0, 1, 0, 1), 17, "s"), ((2, 1, 1, 2), (0, 1, 1, 1), 16, "o"),
          ((1, 2, 2, 1), (0, 1, 1, 0), 16, "s"), ((1,) * 6, (0, 1, 1, 0, 1, 1), 17, "o"),
          ((3, 1, 1, 1, 3), (0, 1, 0, 1, 2), 16, "s"),
          # middle steps with different K
          ((2, 1, 2, 1, 2, 1), (0, 1, 1, 1, 1, 1), 16, "s"), ((3, 2, 1, 3, 2), (0, 1, 1, 1, 1), 16, "o"),
          ((2, 2, 3, 2), (0, 1, 2, 1), 17, "o")]


@pytest.mark.parametrize("case", CHAINN, ids=lambda c: "k{}_v{}_r{}_{}".format(
    "".join(map(str, c[0])), "".join(map(str, c[1][1:])), c[2], c[3]))
def test_fused_longer_chain_matches_oracle(case):
    import quantum_circuit_simulation_amd as qa
    ks, vs, log_rows, last = case
    net, tree = chain_n_network(ks, vs, log_rows, last, seed=900 + sum(ks) + sum(vs) + log_rows)
    plan = qa.Plan.from_network(net, tree)
    assert plan.stats()["fused_pairs"] == 1 and plan.fused(0)["nsteps"] == len(ks)
    kern = _check(net, tree, expect_kernel="k_fused2", kind="fused")
    assert len(kern) == 1 and kern[0].count(",") == 2, kern


def test_chain_stops_at_the_longest_chain():
    # seven steps that could each follow the last: the first six form one
    # chain, the seventh runs alone
    import quantum_circuit_simulation_amd as qa
    net, tree = chain_n_network((2,) * 7, (0, 2, 2, 2, 2, 2, 2), 16, "o", seed=95)
    plan = qa.Plan.from_network(net, tree)
    assert plan.stats()["fused_pairs"] == 1 and plan.fused(0)["step"] == list(range(6))
    _check(net, tree, expect_kernel="k_fused2", kind="fused")


def test_sliced_longer_chain():
    net, tree = chain_n_network((2, 2, 2, 2, 2), (0, 1, 0, 1, 0), 18, "o", seed=97)
    _check(net, tree, expect_kernel="k_fused2", kind="fused", sliced=[net.leaves[-1][0]])


def test_sliced_chain_of_three():
    net, tree = chain3_network(2, 2, 2, 1, 1, 0, 18, "o", seed=91)
    _check(net, tree, expect_kernel="k_fused2", kind="fused", sliced=[net.leaves[4][0]])


def test_fuse_off_runs_the_steps_alone():
    import quantum_circuit_simulation_amd as qa
    net, tree = chain_network(4, 4, 2, 17, "s", seed=5)
    assert qa.Plan.from_network(net, tree).stats()["fused_pairs"] == 1
    assert qa.Plan.from_network(net, tree, fuse=False).stats()["fused_pairs"] == 0
    assert _check(net, tree, kind="fused", fuse=False) == []


def test_sliced_pair():
    net, tree = chain_network(4, 4, 1, 18, "o", seed=77)
    # fix the closed outer mode of T (the last step's): T is staged per slice,
    # the pair runs on half the rows and the root accumulates the two slices
    _check(net, tree, expect_kernel="k_fused2", kind="fused", sliced=[net.leaves[3][0]])
