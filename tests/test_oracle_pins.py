"""Pins of the oracle contractor against things other than itself: state-vector
simulation, a whole-network numpy.einsum, closed forms, invariances.

A plausible mistake in the oracle (a dropped term, a sign in the complex
product, a swapped stride, a wrong output permutation) fails at least one of
these: random complex data rules out sign/term errors, extents 1/2/3/5 and
random declared orders rule out index mix-ups, random output orders check the
final permutation.
"""

import numpy as np
import pytest

import oracle
from tests.brute import einsum_full, statevector
from tests.conftest import rel_err_ok
from workloads import circuits, lattice, randnet, trees
from workloads.network import Network, Tree, caterpillar

TOL128 = 1e-10


def _gates64(c):
    """Gate matrices rounded to complex64, as the network leaves hold them."""
    return [(a, b, u.astype(np.complex64).astype(np.complex128)) for a, b, u in c.gates]


def test_brickwork_amplitude_matches_statevector():
    c = circuits.brickwork(12, 8, 101)
    net = c.to_network()
    tree = trees.greedy_tree(net)
    amp = oracle.contract_network(net, tree)
    psi = statevector(12, _gates64(c))
    ok, err = rel_err_ok(amp, psi[0], TOL128)
    assert ok, err


def test_brickwork_all_open_matches_statevector():
    n = 10
    c = circuits.brickwork(n, 6, 7)
    net = c.to_network(open_qubits=range(n))
    tree = trees.greedy_tree(net)
    psi = oracle.contract_network(net, tree).reshape(-1)
    ref = statevector(n, _gates64(c))
    ok, err = rel_err_ok(psi, ref, TOL128)
    assert ok, err


def test_batch_amplitudes_with_shuffled_output_order():
    n = 10
    c = circuits.brickwork(n, 7, 11)
    order = [3, 0, 5, 1]
    bits = [0, 1, 1, 0, 1, 0, 0, 1, 1, 0]
    net = c.to_network(open_qubits=order, bits=bits, out_order=order)
    tree = trees.greedy_tree(net)
    got = oracle.contract_network(net, tree)          # axes = qubits 3, 0, 5, 1
    psi = statevector(n, _gates64(c)).reshape((2,) * n)
    idx = [slice(None) if q in order else bits[q] for q in range(n)]
    sub = psi[tuple(idx)]                              # axes = qubits 0, 1, 3, 5
    ref = np.transpose(sub, [2, 0, 3, 1])
    ok, err = rel_err_ok(got, ref, TOL128)
    assert ok, err


@pytest.mark.parametrize("seed", range(12))
def test_random_networks_match_einsum(seed):
    rng = np.random.default_rng(1000 + seed)
    net = randnet.random_network(rng, n_leaves=int(rng.integers(2, 7)), n_closed=int(rng.integers(1, 9)),
                                 n_open=int(rng.integers(0, 4)), max_leaf_elems=600)
    tree = randnet.random_tree(rng, net.num_leaves)
    if trees.tree_cost(net, tree)["max_elems"] > 1 << 16:
        pytest.skip("random tree too wide for the unit test")
    got = oracle.contract_network(net, tree)
    ref = einsum_full(net.extents, net.leaves, net.out_modes, net.data)
    ok, err = rel_err_ok(got, ref, TOL128)
    assert ok, err


def test_single_leaf_is_a_permutation():
    rng = np.random.default_rng(5)
    ext = np.array([2, 3, 5], dtype=np.int64)
    d = (rng.standard_normal((2, 3, 5)) + 1j * rng.standard_normal((2, 3, 5))).astype(np.complex64)
    got = oracle.contract([2, 3, 5], [[0, 1, 2]], [2, 0, 1], [d], [], [])
    assert np.array_equal(got, np.transpose(d, [2, 0, 1]).astype(np.complex128))


def test_outer_product():
    rng = np.random.default_rng(6)
    a = (rng.standard_normal(3) + 1j * rng.standard_normal(3)).astype(np.complex64)
    b = (rng.standard_normal(4) + 1j * rng.standard_normal(4)).astype(np.complex64)
    got = oracle.contract([3, 4], [[0], [1]], [1, 0], [a, b], [0], [1])
    ref = np.outer(b.astype(np.complex128), a.astype(np.complex128))
    assert np.allclose(got, ref, rtol=0, atol=1e-14)


def test_identity_circuit_closed_forms():
    n = 8
    c = circuits.Circuit(n)
    for t in range(4):
        for q in range(t % 2, n - 1, 2):
            c.add(q, q + 1, np.eye(4))
    net = c.to_network()
    amp = oracle.contract_network(net, trees.greedy_tree(net))
    assert amp == 1.0
    net_open = c.to_network(open_qubits=range(n))
    psi = oracle.contract_network(net_open, trees.greedy_tree(net_open)).reshape(-1)
    ref = np.zeros(2 ** n)
    ref[0] = 1
    assert np.array_equal(psi, ref)


def test_hadamard_layer_amplitudes():
    n = 8
    hh = np.kron(circuits.HADAMARD, circuits.HADAMARD)
    c = circuits.from_gates(n, [(q, q + 1, hh) for q in range(0, n, 2)])
    net = c.to_network(open_qubits=range(n))
    psi = oracle.contract_network(net, trees.greedy_tree(net)).reshape(-1)
    h32 = np.float64(np.float32(0.5))  # (1/sqrt 2)^2 rounded through complex64 entries
    assert np.allclose(psi, h32 ** (n // 2), rtol=1e-7)
    assert np.allclose(np.abs(psi) ** 2 * 2 ** n, 1.0, rtol=1e-6)


def _trace_network(n, u_layer):
    """tr(I . U) over n qubits: U on pairs (2i, 2i+1), then identity gates
    whose outputs are tied back to U's inputs."""
    ext, leaves, data = [], [], []

    def mode():
        ext.append(2)
        return len(ext) - 1

    for p in range(0, n, 2):
        i0, i1, o0, o1 = mode(), mode(), mode(), mode()
        leaves.append([o0, o1, i0, i1])
        data.append(u_layer.reshape(2, 2, 2, 2).astype(np.complex64))
        leaves.append([i0, i1, o0, o1])
        data.append(np.eye(4).reshape(2, 2, 2, 2).astype(np.complex64))
    return Network(np.array(ext, dtype=np.int64), leaves, [], data)


def test_trace_of_identity_is_dimension():
    n = 8
    net = _trace_network(n, np.eye(4))
    assert oracle.contract_network(net, trees.greedy_tree(net)) == 2.0 ** n


def test_trace_of_hadamard_pair_is_zero():
    net = _trace_network(2, np.kron(circuits.HADAMARD, circuits.HADAMARD))
    v = oracle.contract_network(net, trees.greedy_tree(net))
    assert abs(v) < 1e-12


def test_unit_norm_over_all_bitstrings():
    n = 10
    c = circuits.grid_fsim(2, 5, 6, 3)
    net = c.to_network(open_qubits=range(n))
    psi = oracle.contract_network(net, trees.greedy_tree(net))
    # gates are stored in complex64, so unitarity holds to single precision
    assert abs(np.sum(np.abs(psi) ** 2) - 1.0) < 1e-5


def test_grid_circuit_matches_statevector():
    c = circuits.grid_fsim(3, 4, 8, 9)
    net = c.to_network(open_qubits=[0, 5, 11])
    got = oracle.contract_network(net, trees.greedy_tree(net))
    psi = statevector(12, _gates64(c)).reshape((2,) * 12)
    idx = [slice(None) if q in (0, 5, 11) else 0 for q in range(12)]
    ok, err = rel_err_ok(got, psi[tuple(idx)], TOL128)
    assert ok, err


def test_peps_all_ones_closed_form():
    # all-ones sites scaled by 1/(0.5 D^(deg/2)) give Z = 2^(number of sites)
    # D = 4: the scale 1/(0.5 * 2^deg) is exact in float32, so Z is exact
    net = lattice.peps(3, 4, 0, fill=lambda i, j, shape, rng: np.ones(shape))
    z = oracle.contract_network(net, lattice.row_major_tree(3))
    assert z == 2.0 ** 9
    net = lattice.peps(4, 3, 0, fill=lambda i, j, shape, rng: np.ones(shape))
    z = oracle.contract_network(net, lattice.row_major_tree(4))
    assert abs(z - 2.0 ** 16) < 1e-5 * 2.0 ** 16


def test_peps_rank_one_sites_factorise_over_bonds():
    L, D = 3, 3
    rng = np.random.default_rng(17)
    vec = {}

    def fill(i, j, shape, _rng):
        modes = lattice.site_modes(L, i, j)
        t = np.ones(())
        for x in modes:
            v = rng.integers(1, 4, size=D).astype(np.float64)
            vec[(x, (i, j))] = v
            t = np.multiply.outer(t, v)
        return t

    net = lattice.peps(L, D, 0, fill=fill)
    z = oracle.contract_network(net, lattice.row_major_tree(L))
    expect = 1.0
    for i in range(L):
        for j in range(L):
            deg = len(lattice.site_modes(L, i, j))
            expect *= float(np.float32(1.0 / (0.5 * D ** (deg / 2.0))))
    bonds = {}
    for (x, site), v in vec.items():
        bonds.setdefault(x, []).append(v)
    for x, (u, v) in bonds.items():
        expect *= float(np.dot(u, v))
    assert abs(z - expect) < 1e-6 * abs(expect)


def test_slices_sum_to_unsliced():
    c = circuits.brickwork(8, 6, 21)
    net = c.to_network(open_qubits=[2])
    tree = trees.greedy_tree(net)
    full = oracle.contract_network(net, tree)
    sl = trees.choose_slices(net, tree, 3)
    acc = np.zeros_like(full)
    for v in range(8):
        fixed = {sl[0]: (v >> 2) & 1, sl[1]: (v >> 1) & 1, sl[2]: v & 1}
        acc += oracle.contract_network(net, tree, fixed=fixed)
    ok, err = rel_err_ok(acc, full, TOL128)
    assert ok, err


def test_result_independent_of_tree():
    c = circuits.grid_fsim(3, 3, 6, 4)
    net = c.to_network(open_qubits=[4])
    r1 = oracle.contract_network(net, trees.greedy_tree(net))
    r2 = oracle.contract_network(net, trees.greedy_tree(net, reverse_ties=True))
    r3 = oracle.contract_network(net, randnet.random_tree(np.random.default_rng(0), net.num_leaves))
    for r in (r2, r3):
        ok, err = rel_err_ok(r, r1, TOL128)
        assert ok, err


def test_sampled_entries_match_full_contraction():
    from workloads import sweep
    net, tree = sweep.network(3, 4, 3, permuted=True, seed=9, with_data=True)
    full = oracle.contract_network(net, tree).reshape(-1)
    idx = np.array([0, 5, 17, 100, full.size - 1])
    oa, ob = oracle.sample_gather(net.extents, net.leaves[0], net.leaves[1], net.out_modes, idx)
    a = net.data[0].reshape(-1)[oa]
    b = net.data[1].reshape(-1)[ob]
    got = oracle.dot_rows(a, b)
    assert np.allclose(got, full[idx], rtol=1e-13, atol=1e-13)


def test_monomial_circuit_amplitude_is_tracked_phase():
    from tests.brute import track_basis_state
    c = circuits.grid_monomial(3, 4, 8, 12)
    g64 = _gates64(c)
    bits, amp = track_basis_state(12, g64)
    assert abs(abs(amp) - 1.0) < 1e-6
    net = c.to_network(bits=bits)
    got = oracle.contract_network(net, trees.greedy_tree(net))
    ok, err = rel_err_ok(got, amp, TOL128)
    assert ok, err
    # any other bra gives exactly zero
    other = list(bits)
    other[5] ^= 1
    net0 = c.to_network(bits=other)
    assert oracle.contract_network(net0, trees.greedy_tree(net0)) == 0


def test_monomial_tracking_matches_statevector():
    from tests.brute import track_basis_state
    c = circuits.grid_monomial(2, 4, 8, 3)
    g = _gates64(c)
    bits, amp = track_basis_state(8, g)
    psi = statevector(8, g)
    idx = int("".join(map(str, bits)), 2)
    assert abs(psi[idx] - amp) < 1e-12
    assert abs(np.sum(np.abs(psi) ** 2) - 1) < 1e-6


def test_random_greedy_search_is_deterministic_and_valid():
    net = circuits.grid_fsim(3, 4, 8, 1).to_network(open_qubits=[0])
    t1 = trees.search_tree(net, trials=10, seed=3)
    t2 = trees.search_tree(net, trials=10, seed=3)
    assert t1.lhs == t2.lhs and t1.rhs == t2.rhs
    ref = oracle.contract_network(net, trees.greedy_tree(net))
    got = oracle.contract_network(net, t1)
    ok, err = rel_err_ok(got, ref, TOL128)
    assert ok, err


def test_complex128_leaves_are_read_at_full_precision():
    """A network whose exact value needs more than single precision: with
    complex128 leaves the oracle must reproduce the einsum to 1e-12."""
    rng = np.random.default_rng(77)
    net = randnet.random_network(rng, n_leaves=5, n_closed=7, n_open=2, max_leaf_elems=500)
    data = [(rng.standard_normal(d.shape) + 1j * rng.standard_normal(d.shape)) for d in net.data]
    tree = randnet.random_tree(rng, net.num_leaves)
    got = oracle.contract(net.extents, net.leaves, net.out_modes, data, tree.lhs, tree.rhs)
    ref = einsum_full(net.extents, net.leaves, net.out_modes, data)
    ok, err = rel_err_ok(got, ref, 1e-12)
    assert ok, err
    single = oracle.contract(net.extents, net.leaves, net.out_modes, [d.astype(np.complex64) for d in data],
                             tree.lhs, tree.rhs)
    assert np.max(np.abs(single - ref)) > 1e-9 * np.max(np.abs(ref))


def _cn(rng, shape):
    return ((rng.standard_normal(shape) + 1j * rng.standard_normal(shape)) / np.sqrt(2)).astype(np.complex64)


@pytest.mark.parametrize("ni,nj,k", [(5, 7, 3), (9, 4, 1), (3, 3, 27), (6, 11, 40), (1, 13, 2)])
def test_pair_block_is_a_times_b_transposed(ni, nj, k):
    """oracle.pair_block(a, b) = a @ b^T over K (no conjugate), against numpy's
    own complex128 matrix product on non-square blocks (so a transposed
    index into b, or a swapped i / j, reads the wrong entries)."""
    rng = np.random.default_rng(ni * 1000 + nj * 10 + k)
    a, b = _cn(rng, (ni, k)), _cn(rng, (nj, k))
    got = oracle.pair_block(a, b)
    ref = a.astype(np.complex128) @ b.astype(np.complex128).T
    assert got.shape == (ni, nj)
    assert np.max(np.abs(got - ref)) <= 1e-12 * max(1.0, np.max(np.abs(ref)))


def test_pair_block_closed_forms():
    """Identity rows of B give A back exactly; all-ones operands give k."""
    rng = np.random.default_rng(3)
    a = _cn(rng, (6, 9))
    eye = np.eye(9, dtype=np.complex64)
    assert np.array_equal(oracle.pair_block(a, eye), a.astype(np.complex128))
    ones_a = np.ones((4, 37), np.complex64)
    ones_b = np.ones((5, 37), np.complex64)
    assert np.array_equal(oracle.pair_block(ones_a, ones_b), np.full((4, 5), 37.0 + 0j))
    # (i * 1) * (i * 1) = -1 per term: the sign of the imaginary product
    ij = np.full((2, 5), 1j, np.complex64)
    assert np.array_equal(oracle.pair_block(ij, ij), np.full((2, 2), -5.0 + 0j))


def test_pair_block_matches_the_contractor_on_gathered_rows():
    """A pairwise network with extent-3 and extent-5 modes, contracted whole by
    the oracle contractor (pinned above against einsum and brute force); the
    block of randomly gathered rows of A and of B must equal the same block
    of the full product."""
    rng = np.random.default_rng(41)
    # modes: m0 (3), m1 (2) | n0 (5) | k0 (3), k1 (2)
    ext = [3, 2, 5, 3, 2]
    A_modes, B_modes, out = [0, 1, 3, 4], [2, 3, 4], [0, 1, 2]
    A, B = _cn(rng, (3, 2, 3, 2)), _cn(rng, (5, 3, 2))
    full = oracle.contract(ext, [A_modes, B_modes], out, [A, B], [0], [1]).reshape(6, 5)
    rows = rng.permutation(6)[:4]
    cols = rng.permutation(5)[:3]
    got = oracle.pair_block(A.reshape(6, 6)[rows], B.reshape(5, 6)[cols])
    assert np.max(np.abs(got - full[np.ix_(rows, cols)])) <= 1e-12 * np.max(np.abs(full))
    # K = {} (outer product): a column of A times a row of B
    a1, b1 = _cn(rng, (7, 1)), _cn(rng, (4, 1))
    outer = oracle.contract([7, 4], [[0], [1]], [0, 1], [a1.reshape(7), b1.reshape(4)], [0], [1])
    assert np.max(np.abs(oracle.pair_block(a1, b1) - outer)) <= 1e-14


def test_monomial_path_values_select_the_one_nonzero_slice():
    """For a monomial circuit every mode takes one value on the tracked
    basis-state path: fixing any modes to those values keeps the whole
    amplitude, fixing one of them to the other value gives exactly zero."""
    from tests.brute import monomial_mode_values, track_basis_state
    c = circuits.grid_monomial(3, 4, 8, 21)
    g64 = _gates64(c)
    bits, amp = track_basis_state(12, g64)
    net = c.to_network(bits=bits)
    vals, amp2 = monomial_mode_values(net, g64, 12)
    assert abs(amp2 - amp) < 1e-12
    tree = trees.greedy_tree(net)
    closed = trees.closed_modes(net)
    rng = np.random.default_rng(4)
    pick = [int(x) for x in rng.choice(closed, size=3, replace=False)]
    on = oracle.contract_network(net, tree, fixed={x: vals[x] for x in pick})
    ok, err = rel_err_ok(on, amp, TOL128)
    assert ok, err
    off = {x: vals[x] for x in pick}
    off[pick[1]] ^= 1
    assert oracle.contract_network(net, tree, fixed=off) == 0
