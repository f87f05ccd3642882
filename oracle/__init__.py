"""Oracle for exact tensor-network contraction.

TEST INFRASTRUCTURE.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
CPU-baseline leg of ``bench.py`` may import this package.  It is independent
of the GPU library: it shares no code with it and never imports it.

* ``contract``      - the naive complex128 contractor (C, OpenMP), evaluating
                      the network's full sum pairwise along a given tree;
* ``dot_rows``      - exact complex128 dot products for sampled entries;
* ``sample_gather`` - which input entries meet in a given output entry of a
                      pairwise contraction (for sampled checks at sizes the
                      full contractor cannot reach);
* ``planner``       - the mode-order / node / arena plan that the GPU
                      library must reproduce bit-exactly.

Source: "Parallelizing Large-Scale Tensor Network Contraction on Multiple
GPUs" (section 1.1 for the pairwise step, section 1.4 for lifetime ordering).
"""

from __future__ import annotations

import ctypes
import os
from typing import Optional, Sequence

import numpy as np

from . import planner  # noqa: F401

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_HERE, "liboracle.so")
_lib = None


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB_PATH):
        from .build import build
        build()
    lib = ctypes.CDLL(_LIB_PATH)
    P = ctypes.POINTER
    lib.oracle_contract.restype = ctypes.c_int
    lib.oracle_contract.argtypes = [
        ctypes.c_int32, P(ctypes.c_int64),
        ctypes.c_int32, P(ctypes.c_int32), P(ctypes.c_int32),
        P(ctypes.c_void_p), ctypes.c_int32,
        ctypes.c_int32, P(ctypes.c_int32), P(ctypes.c_int32),
        ctypes.c_int32, P(ctypes.c_int32),
        ctypes.c_int32, P(ctypes.c_int32), P(ctypes.c_int64),
        P(ctypes.c_double), ctypes.c_int32,
    ]
    lib.oracle_dot_rows.restype = None
    lib.oracle_dot_rows.argtypes = [ctypes.c_int64, ctypes.c_int64, P(ctypes.c_float), P(ctypes.c_float),
                                    P(ctypes.c_double), ctypes.c_int32]
    lib.oracle_pair_block.restype = None
    lib.oracle_pair_block.argtypes = [ctypes.c_int64, ctypes.c_int64, ctypes.c_int64, P(ctypes.c_float),
                                      P(ctypes.c_float), P(ctypes.c_double), ctypes.c_int32]
    lib.oracle_max_threads.restype = ctypes.c_int
    _lib = lib
    return lib


def max_threads() -> int:
    return int(_load().oracle_max_threads())


def _i32(a):
    return np.ascontiguousarray(np.asarray(a, dtype=np.int32))


def _i64(a):
    return np.ascontiguousarray(np.asarray(a, dtype=np.int64))


def _ptr(a, ct):
    return a.ctypes.data_as(ctypes.POINTER(ct))


def contract(extents, leaves, out_modes, data, lhs, rhs, fixed: Optional[dict] = None,
             threads: Optional[int] = None) -> np.ndarray:
    """Evaluate the network along the tree; returns complex128 with the shape
    of ``out_modes`` (a 0-d array for a scalar).  Leaf data are read as
    complex128 when every leaf is complex128, else as complex64."""
    lib = _load()
    ext = _i64(extents)
    rank = _i32([len(l) for l in leaves])
    modes = _i32([x for l in leaves for x in l]) if rank.sum() else np.zeros(1, np.int32)
    c128 = all(np.asarray(d).dtype == np.complex128 for d in data)
    dt = np.complex128 if c128 else np.complex64
    bufs = [np.ascontiguousarray(np.asarray(d, dtype=dt)) for d in data]
    for d, l in zip(bufs, leaves):
        assert d.size == int(np.prod([ext[x] for x in l], dtype=np.int64)), "leaf data size"
    ptrs = (ctypes.c_void_p * len(bufs))(*[d.ctypes.data for d in bufs])
    lhs_a, rhs_a = _i32(lhs), _i32(rhs)
    if lhs_a.size == 0:
        lhs_a = np.zeros(1, np.int32); rhs_a = np.zeros(1, np.int32)
    outm = _i32(out_modes) if len(out_modes) else np.zeros(1, np.int32)
    fixed = fixed or {}
    fm = _i32(list(fixed.keys())) if fixed else np.zeros(1, np.int32)
    fv = _i64(list(fixed.values())) if fixed else np.zeros(1, np.int64)
    shape = tuple(int(ext[x]) for x in out_modes)
    out = np.zeros(int(np.prod(shape, dtype=np.int64)) * 2, dtype=np.float64)
    nt = threads if threads else max_threads()
    rc = lib.oracle_contract(len(ext), _ptr(ext, ctypes.c_int64), len(leaves), _ptr(rank, ctypes.c_int32),
                             _ptr(modes, ctypes.c_int32), ptrs, int(c128), len(lhs), _ptr(lhs_a, ctypes.c_int32),
                             _ptr(rhs_a, ctypes.c_int32), len(out_modes), _ptr(outm, ctypes.c_int32),
                             len(fixed), _ptr(fm, ctypes.c_int32), _ptr(fv, ctypes.c_int64),
                             _ptr(out, ctypes.c_double), nt)
    if rc != 0:
        raise RuntimeError(f"oracle_contract failed with code {rc}")
    return out.view(np.complex128).reshape(shape)


def contract_network(net, tree, fixed=None, threads=None) -> np.ndarray:
    return contract(net.extents, net.leaves, net.out_modes, net.data, tree.lhs, tree.rhs,
                    fixed=fixed, threads=threads)


def dot_rows(a: np.ndarray, b: np.ndarray, threads: Optional[int] = None) -> np.ndarray:
    """a, b: complex64 [count, k].  Returns complex128 [count] = sum_l a*b."""
    a = np.ascontiguousarray(a, dtype=np.complex64)
    b = np.ascontiguousarray(b, dtype=np.complex64)
    assert a.shape == b.shape and a.ndim == 2
    cnt, k = a.shape
    out = np.zeros(2 * cnt, dtype=np.float64)
    _load().oracle_dot_rows(cnt, k, _ptr(a.view(np.float32), ctypes.c_float),
                            _ptr(b.view(np.float32), ctypes.c_float), _ptr(out, ctypes.c_double),
                            threads if threads else max_threads())
    return out.view(np.complex128)


def pair_block(a: np.ndarray, b: np.ndarray, threads: Optional[int] = None) -> np.ndarray:
    """a: complex64 [ni, k] rows of A, b: complex64 [nj, k] rows of B (K
    innermost, same K order).  Returns complex128 [ni, nj] = a @ b^T."""
    a = np.ascontiguousarray(a, dtype=np.complex64)
    b = np.ascontiguousarray(b, dtype=np.complex64)
    assert a.ndim == 2 and b.ndim == 2 and a.shape[1] == b.shape[1]
    ni, k = a.shape
    nj = b.shape[0]
    out = np.zeros(2 * ni * nj, dtype=np.float64)
    _load().oracle_pair_block(ni, nj, k, _ptr(a.view(np.float32), ctypes.c_float),
                              _ptr(b.view(np.float32), ctypes.c_float), _ptr(out, ctypes.c_double),
                              threads if threads else max_threads())
    return out.view(np.complex128).reshape(ni, nj)


def row_major_strides(extents, modes):
    st = {}
    s = 1
    for x in reversed(list(modes)):
        st[x] = s
        s *= int(extents[x])
    return st


def sample_gather(extents, a_modes: Sequence[int], b_modes: Sequence[int], out_modes: Sequence[int],
                  out_index: np.ndarray):
    """For a pairwise contraction with declared layouts ``a_modes``,
    ``b_modes`` and output layout ``out_modes``, return flat offsets
    (int64 [count, k]) into A and into B of the entries whose products sum to
    each requested output entry (flat index into the output layout).  K is
    enumerated in ascending mode label, last label fastest."""
    A, B = list(a_modes), list(b_modes)
    K = sorted(set(A) & set(B))
    sa = row_major_strides(extents, A)
    sb = row_major_strides(extents, B)
    so = row_major_strides(extents, out_modes)
    out_index = np.asarray(out_index, dtype=np.int64)
    base_a = np.zeros(out_index.shape, dtype=np.int64)
    base_b = np.zeros(out_index.shape, dtype=np.int64)
    for x in out_modes:
        digit = (out_index // so[x]) % int(extents[x])
        if x in sa:
            base_a += digit * sa[x]
        else:
            base_b += digit * sb[x]
    kk = int(np.prod([int(extents[x]) for x in K], dtype=np.int64)) if K else 1
    l = np.arange(kk, dtype=np.int64)
    ka = np.zeros(kk, dtype=np.int64)
    kb = np.zeros(kk, dtype=np.int64)
    r = l.copy()
    for x in reversed(K):
        d = r % int(extents[x])
        r //= int(extents[x])
        ka += d * sa[x]
        kb += d * sb[x]
    return base_a[:, None] + ka[None, :], base_b[:, None] + kb[None, :]
