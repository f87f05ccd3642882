"""The skinny-step bench workload at its full sizes and in its launch
configuration (the same plans on the same seeded device pools), checked
against the oracle on sampled rows (all columns of each row: exact
complex128 sums over the gathered inputs) and, for the 2^30-long dot product,
on the whole result.  Also checks, over the whole output, that every entry
is finite and that mean |C|^2 / k is close to 1 (i.i.d. CN(0,1) inputs),
which catches rows that were skipped or written twice."""

import numpy as np
import pytest

import oracle
from tests.conftest import rel_err_ok
from workloads import sweep

pytestmark = pytest.mark.gpu
TOL = 1e-4


@pytest.fixture(scope="module")
def workload():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from bench import SkinnyWorkload
    wl = SkinnyWorkload()
    torch.cuda.synchronize()
    yield wl
    del wl
    torch.cuda.empty_cache()


@pytest.mark.parametrize("idx", range(5), ids=lambda i: "m%dn%dk%d" % tuple(
    __import__("bench").SkinnyWorkload.CASES[i]))
def test_skinny_bench_case_full_size(idx, workload):
    import torch
    wl = workload
    (lm, ln, lk), plan, m, n, k = wl.plans[idx]
    print(f"[gpu] skinny bench case m=2^{lm} n=2^{ln} k=2^{lk}", flush=True)
    C = wl.C[: m * n]
    C.fill_(float("nan"))
    plan.execute([wl.A[: m * k], wl.B[: n * k]], C, wl.ws)
    torch.cuda.synchronize()
    assert bool(torch.isfinite(torch.view_as_real(C)).all()), "non-finite or unwritten entries"
    ms = float((C.abs() ** 2).mean().item()) / k
    assert 0.8 < ms < 1.2 or m * n < 64, f"mean |C|^2 / k = {ms}"
    if m * n == 1:
        a = wl.A[:k].view(1, k).cpu().numpy()
        b = wl.B[:k].view(1, k).cpu().numpy()
        ref = oracle.dot_rows(a, b)
        got = C.cpu().numpy()
    else:
        rng = np.random.default_rng(idx)
        rows = np.unique(np.concatenate([rng.choice(m, size=min(m, 4096), replace=False), [0, m - 1]]))
        ri = torch.from_numpy(rows).cuda()
        a = wl.A[: m * k].view(m, k).index_select(0, ri).cpu().numpy()
        b = wl.B[: n * k].view(n, k).cpu().numpy()
        ref = oracle.pair_block(a, b)
        got = C.view(m, n).index_select(0, ri).cpu().numpy()
    ok, err = rel_err_ok(got, ref, TOL)
    assert ok, err
