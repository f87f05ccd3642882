"""The one-GPU half of the distribution schedule (page "Parallelizing
Large-Scale Tensor Network Contraction on Multiple GPUs", sections 1.5-1.6:
a split tensor stays in contiguous blocks, one per GPU, and a Keep step is a
local GEMM on each GPU's own block).  For P = 8 schedules of a reduced grid
circuit and of a 4x4 lattice, every split step's local GEMM runs on the GPU
at its shard shape for two ranks (first and last): the operands' blocks at
the rank's digits of the split modes go through the C ABI, and the result is
compared with the oracle's contraction of the whole step with the reduced
split modes fixed (oracle ``fixed``), indexed at the kept split modes.
Per output entry: |g - r| <= 1e-4 * max(|r|, rms(r))."""

import math

import numpy as np
import pytest

import oracle
import quantum_circuit_simulation_amd as qa
from tests.conftest import rel_err_ok
from workloads import circuits, lattice, trees

pytestmark = pytest.mark.gpu

TOL = 1e-4
P = 8


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    yield


def _cases():
    g = circuits.grid_fsim(4, 5, 12, 31).to_network(name="grid4x5d12")
    gt, _, _ = trees.optimize_tree(g, trials=8, seed=3)
    p = lattice.peps(4, 8, 811)
    return [("grid4x5d12", g, gt, 8 << 10), ("peps4x4", p, lattice.row_major_tree(4), 8 << 10)]


def _digits(q, exts):
    out = []
    for e in reversed(exts):
        out.append(q % e)
        q //= e
    return out[::-1]


@pytest.mark.parametrize("case", range(2))
def test_split_steps_local_gemm_matches_oracle_slice(case):
    import torch
    name, net, tree, thr = _cases()[case]
    plan = qa.Plan.from_network(net, tree)
    steps, _ = plan.distribute(num_gpus=P, threshold_bytes=thr)
    split = [s for s, st in enumerate(steps) if st["tag_name"] != "replicated" and st["num_local"] > 0]
    assert split, "threshold splits nothing"
    ext = [int(e) for e in net.extents]
    checked = 0
    for s in split:
        st = steps[s]
        nd = plan.node(s)
        if 8.0 * nd["m"] * nd["n"] * nd["k"] > 4e10:
            continue
        oa, ob, oc = (plan.tensor_order(nd[k]) for k in ("lhs", "rhs", "out"))
        K = [x for x in oa if x in ob]
        rng = np.random.default_rng(1000 + s)
        A = ((rng.standard_normal([ext[x] for x in oa]) + 1j * rng.standard_normal([ext[x] for x in oa]))
             / np.sqrt(2)).astype(np.complex64)
        B = ((rng.standard_normal([ext[x] for x in ob]) + 1j * rng.standard_normal([ext[x] for x in ob]))
             / np.sqrt(2)).astype(np.complex64)
        loc = list(st["local_modes"])
        lexts = [ext[x] for x in loc]
        Q = math.prod(lexts)
        cnt = st["local_count"]
        assert cnt == -(-Q // P)
        for rank in (0, P - 1):
            for q in range(rank * cnt, min(Q, (rank + 1) * cnt))[:2]:
                dig = dict(zip(loc, _digits(q, lexts)))
                # GPU: the rank's blocks of the operands, the split modes gone
                a_sh = A[tuple(dig[x] if x in dig else slice(None) for x in oa)]
                b_sh = B[tuple(dig[x] if x in dig else slice(None) for x in ob)]
                ka = [x for x in oa if x not in dig]
                kb = [x for x in ob if x not in dig]
                kc = [x for x in oc if x not in dig]
                lab = {x: i for i, x in enumerate(dict.fromkeys(ka + kb + kc))}
                sp = qa.Plan([ext[x] for x in lab], [[lab[x] for x in ka], [lab[x] for x in kb]],
                             [lab[x] for x in kc], [0], [1])
                n0 = sp.node(0)
                assert {n0["m"], n0["n"]} == {st["local_m"], st["local_n"]} and n0["k"] == st["local_k"], (s, n0, st)
                dev = [torch.from_numpy(np.ascontiguousarray(a_sh)).cuda(),
                       torch.from_numpy(np.ascontiguousarray(b_sh)).cuda()]
                out = torch.empty(max(1, math.prod(ext[x] for x in kc)), dtype=torch.complex64, device="cuda")
                sp.execute(dev, out, qa.alloc_workspace(sp))
                torch.cuda.synchronize()
                got = out.cpu().numpy().astype(np.complex128)
                # oracle: the whole step with the reduced split modes fixed,
                # then the block of the kept split modes
                fixed = {x: v for x, v in dig.items() if x in K}
                full = oracle.contract(ext, [oa, ob], oc, [A, B], [0], [1], fixed=fixed)
                ref = full[tuple(dig[x] if x in dig else slice(None) for x in oc)].reshape(-1)
                ok, err = rel_err_ok(got, ref, TOL)
                print(f"[gpu] {name} step {s} {st['tag_name']} rank {rank} slice {q}/{Q}: "
                      f"local {n0['m']}x{n0['n']}x{n0['k']} err {err:.2e}", flush=True)
                assert ok, (s, rank, q, err)
                checked += 1
    assert checked >= 4, checked
