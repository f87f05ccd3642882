"""Isolated pairwise contractions: C[M, N] = sum_K A[M, K] B[N, K].

Every mode has extent 2; A carries log2(m) + log2(k) modes and B carries
log2(n) + log2(k).  Mode labels: M = 0 .. a-1, N = a .. a+b-1,
K = a+b .. a+b+c-1 (K ascending, so the GEMM-aligned declaration already
matches the planner's K order).

* aligned:  A declared [M | K], B declared [N | K], output [M | N];
* permuted: the same modes, with A, B and the output each declared in a
  seeded random order (numpy default_rng(seed + 1_000_000)).

Entries are i.i.d. standard complex Gaussian CN(0, 1) = (x + i y)/sqrt(2).
"""

from __future__ import annotations

from typing import List, Tuple

import numpy as np

from .network import Network, Tree

EXPONENTS = (6, 10, 14, 18)       # log2 of m, n, k
K_MAX_EXP = 14                    # k <= 2^14


def cases() -> List[dict]:
    """All (m, n, k) combinations with their seeds; ``feasible`` is False when
    C alone would not fit one GPU (m = n = 2^18: 512 GiB)."""
    out = []
    idx = 0
    for a in EXPONENTS:
        for b in EXPONENTS:
            for c in EXPONENTS:
                if c > K_MAX_EXP:
                    continue
                out.append(dict(index=idx, logm=a, logn=b, logk=c, seed=200 + idx,
                                feasible=not (a == 18 and b == 18)))
                idx += 1
    return out


def network(logm: int, logn: int, logk: int, permuted: bool = False, seed: int = 0,
            with_data: bool = False) -> Tuple[Network, Tree]:
    a, b, c = logm, logn, logk
    M = list(range(a))
    N = list(range(a, a + b))
    K = list(range(a + b, a + b + c))
    A = M + K
    B = N + K
    out = M + N
    if permuted:
        prng = np.random.default_rng(seed + 1_000_000)
        A = [A[i] for i in prng.permutation(len(A))]
        B = [B[i] for i in prng.permutation(len(B))]
        out = [out[i] for i in prng.permutation(len(out))]
    extents = np.full(a + b + c, 2, dtype=np.int64)
    data = None
    if with_data:
        rng = np.random.default_rng(seed)
        data = [complex_gaussian(rng, (2,) * len(A)), complex_gaussian(rng, (2,) * len(B))]
    net = Network(extents, [A, B], out, data,
                  name=f"pair_m2^{a}_n2^{b}_k2^{c}" + ("_perm" if permuted else ""),
                  meta=dict(logm=a, logn=b, logk=c, permuted=permuted, seed=seed))
    return net, Tree([0], [1])


def complex_gaussian(rng: np.random.Generator, shape) -> np.ndarray:
    """CN(0,1) complex64: real and imaginary parts N(0, 1/2), drawn as one
    real block of shape (..., 2)."""
    x = rng.standard_normal(tuple(shape) + (2,), dtype=np.float32) * np.float32(np.sqrt(0.5))
    return x.view(np.complex64).reshape(shape)
