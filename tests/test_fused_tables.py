"""Host-side check of the fused-pair tables (no GPU): the planner's per-bit
tables of a fused pair (tnc_plan_fused) are applied in numpy exactly as the
pass kernel applies them - which rows of the long operand a pass reads,
where each first product goes in the second step's block, where each second
product is stored - and the result must equal the oracle's contraction of
the two steps in the second product's planned layout, with every entry
written once.  A wrong bit, offset or row choice in the tables fails here
before any kernel runs."""

import numpy as np
import pytest

import oracle
import quantum_circuit_simulation_amd as qa
from tests.test_gpu_fused import chain_network
from workloads.network import Network, Tree

CASES = [(4, 4, 0, 16, "s"), (4, 4, 2, 16, "o"), (4, 5, 2, 16, "s"), (5, 4, 1, 16, "s"), (5, 5, 3, 16, "o"),
         (4, 4, 4, 16, "s"), (5, 4, 4, 16, "o"), (4, 5, 0, 16, "o"), (2, 2, 0, 16, "s"), (2, 3, 2, 16, "o"),
         (3, 2, 1, 16, "s"), (3, 3, 3, 16, "o"), (3, 4, 1, 16, "s"), (5, 2, 2, 16, "o")]


def _bits_sum(idx, table, nbits):
    """sum over set bits b < nbits of idx of table[b] (idx an int array)."""
    out = np.zeros(np.shape(idx), dtype=np.int64)
    for b in range(nbits):
        out += ((idx >> b) & 1).astype(np.int64) * int(table[b])
    return out


def _planned(data, declared, planned):
    return np.transpose(data, [declared.index(x) for x in planned])


def _to_block(Y, pos_row, pos_col, nrow_bits, k_in, k_next):
    """Place products Y (round, wave, rows, k_in) in the next step's block
    [1024 / k_next rows][k_next + 2] by the per-bit tables."""
    nround = Y.shape[0]
    rows_next = 1024 // k_next
    pos = (_bits_sum(np.arange(Y.shape[2]), pos_row, nrow_bits)[:, None]
           + _bits_sum(np.arange(k_in), pos_col, k_in.bit_length() - 1)[None, :])
    assert len(np.unique(pos)) == pos.size and np.all(pos % (k_next + 2) < k_next)
    block = np.zeros((nround, 4, rows_next * (k_next + 2)), dtype=np.complex128)
    block[:, :, pos.reshape(-1)] = Y.reshape(nround, 4, -1)
    return block.reshape(nround, 4, rows_next, k_next + 2)[..., :k_next]


def emulate_pair(f, X, W1, W2, out_size, W3=None):
    """The pass kernel's index arithmetic over all rounds and waves (complex128);
    with W3, a chain of three."""
    k1, k2, k3 = f["k1"], f["k2"], f["k3"]
    kl = k3 if k3 else k2
    rows1, rows2 = 1024 // k1, 1024 // kl
    lb1, lb2 = rows1.bit_length() - 1, rows2.bit_length() - 1
    nround = f["rows"] // rows1 // 4
    rnd = np.arange(nround, dtype=np.int64)
    dep = rnd.copy()
    for p in f["hole"][:lb1 + 2]:
        dep = ((dep >> p) << (p + 1)) | (dep & ((1 << p) - 1))
    w = np.arange(4, dtype=np.int64)
    wrow = (w & 1) << f["wbit"][0] | (w >> 1) << f["wbit"][1]
    rho = np.arange(rows1, dtype=np.int64)
    spread = _bits_sum(rho, [1 << b for b in f["lrow"]], lb1)
    rows = dep[:, None, None] + wrow[None, :, None] + spread[None, None, :]
    Y1 = X[rows] @ W1.T                                   # (round, wave, rho, j)
    Y2 = _to_block(Y1, f["pos_row"], f["pos_col"], lb1, k1, k2) @ W2.T
    if k3:
        lbm = (1024 // k2).bit_length() - 1
        Y2 = _to_block(Y2, f["pos2_row"], f["pos2_col"], lbm, k2, k3) @ W3.T
    k2 = kl                                               # the stored product's columns
    base = _bits_sum(rnd, f["out_pass"][2:], f["nouter"] - 2)
    wpart = (w & 1) * f["out_pass"][0] + (w >> 1) * f["out_pass"][1]
    local = (_bits_sum(np.arange(rows2), f["out_row"], lb2)[:, None]
             + _bits_sum(np.arange(k2), f["out_col"], k2.bit_length() - 1)[None, :])
    addr = base[:, None, None, None] + wpart[None, :, None, None] + local[None, None]
    assert addr.min() >= 0 and addr.max() < out_size
    C = np.zeros(out_size, dtype=np.complex128)
    hits = np.zeros(out_size, dtype=np.int64)
    np.add.at(hits, addr.reshape(-1), 1)
    assert np.all(hits == 1), "every entry of the second product is written once"
    C[addr.reshape(-1)] = Y2.reshape(-1)
    return C


@pytest.mark.parametrize("case", CASES, ids=lambda c: "k{}_{}_v{}_r{}_{}".format(*c))
@pytest.mark.parametrize("permuted", [False, True], ids=["aligned", "permuted"])
def test_fused_tables_reproduce_the_two_steps(case, permuted):
    net, tree = chain_network(*case, seed=60 + sum(case[:4]), permuted=permuted)
    plan = qa.Plan.from_network(net, tree)
    assert plan.stats()["fused_pairs"] == 1
    f = plan.fused(0)
    assert (f["first"], f["second"], f["long1"], f["long2"]) == (0, 1, 0, 0)
    L = net.num_leaves
    order = [plan.tensor_order(t) for t in range(L + 2)]
    data = [np.asarray(d, dtype=np.complex128) for d in net.data]
    X = _planned(data[0], net.leaves[0], order[0]).reshape(f["rows"], f["k1"])
    W1 = _planned(data[1], net.leaves[1], order[1]).reshape(f["k1"], f["k1"])
    W2 = _planned(data[2], net.leaves[2], order[2]).reshape(f["k2"], f["k2"])
    T2_modes = order[L + 1]
    got = emulate_pair(f, X, W1, W2, int(np.prod([net.extents[x] for x in T2_modes])))
    sub = Network(net.extents, net.leaves[:3], T2_modes, net.data[:3], name="pair")
    ref = np.asarray(oracle.contract_network(sub, Tree([0, 3], [1, 2]))).reshape(-1)
    np.testing.assert_allclose(got, ref, rtol=0, atol=1e-9 * np.abs(ref).max())


@pytest.mark.parametrize("case", [(2, 2, 2, 1, 1, 0, 16, "s"), (3, 2, 3, 1, 1, 1, 16, "o"), (2, 3, 2, 0, 2, 0, 16, "s"),
                                  (3, 3, 3, 2, 1, 0, 16, "o")], ids=lambda c: "k{}{}{}_v{}{}{}".format(*c))
@pytest.mark.parametrize("permuted", [False, True], ids=["aligned", "permuted"])
def test_fused_chain_tables_reproduce_the_three_steps(case, permuted):
    from tests.test_gpu_fused import chain3_network
    net, tree = chain3_network(*case, seed=70 + sum(case[:7]), permuted=permuted)
    plan = qa.Plan.from_network(net, tree)
    assert plan.stats()["fused_pairs"] == 1
    f = plan.fused(0)
    assert (f["first"], f["second"], f["third"]) == (0, 1, 2) and f["long1"] == f["long2"] == f["long3"] == 0
    L = net.num_leaves
    order = [plan.tensor_order(t) for t in range(L + 3)]
    data = [np.asarray(d, dtype=np.complex128) for d in net.data]
    X = _planned(data[0], net.leaves[0], order[0]).reshape(f["rows"], f["k1"])
    W = [_planned(data[i], net.leaves[i], order[i]).reshape(k, k) for i, k in ((1, f["k1"]), (2, f["k2"]), (3, f["k3"]))]
    T3_modes = order[L + 2]
    got = emulate_pair(f, X, W[0], W[1], int(np.prod([net.extents[x] for x in T3_modes])), W3=W[2])
    sub = Network(net.extents, net.leaves[:4], T3_modes, net.data[:4], name="chain3")
    ref = np.asarray(oracle.contract_network(sub, Tree([0, 4, 5], [1, 2, 3]))).reshape(-1)
    np.testing.assert_allclose(got, ref, rtol=0, atol=1e-9 * np.abs(ref).max())
    for t in (L, L + 1):
        assert plan.tensor_offset(t) == (1 << 64) - 1   # neither earlier product is stored


def test_unfused_plan_has_no_tables():
    net, tree = chain_network(4, 4, 2, 16, "s", seed=3, with_data=False)
    plan = qa.Plan.from_network(net, tree, fuse=False)
    with pytest.raises(RuntimeError):
        plan.fused(0)
