"""Deterministic contraction-tree and slice-mode choices.

The source page ("Parallelizing Large-Scale Tensor Network Contraction on
Multiple GPUs", sections 3.3-3.4) takes its trees and slicing from an
external hyper-optimising path finder.  That tool is not available here, so
the trees are built by a plain greedy rule:

1. among live tensor pairs that share at least one mode, take the pair whose
   result has the fewest entries;
2. ties: the smallest (|C| - |A| - |B|), then the smallest (min id, max id);
3. when no pair shares a mode, take the outer product of the two lowest ids.

``tree_cost`` reports, for any tree, the per-step (m, n, k), the largest
intermediate and the operation count 8 m n k per step (complex64 on real
arithmetic), with a chosen set of modes fixed (sliced).
"""

from __future__ import annotations

from typing import Dict, Iterable, List, Optional, Sequence, Tuple

import numpy as np

from .network import Network, Tree


def _prod(ext, modes) -> int:
    p = 1
    for x in modes:
        p *= int(ext[x])
    return p


def greedy_tree(net: Network, reverse_ties: bool = False) -> Tree:
    """Greedy min-intermediate-size tree (rule in the module docstring).

    ``reverse_ties`` flips the last tie-break to the largest (min id, max id),
    giving a second, generally different, tree for order-invariance tests."""
    ext = net.extents
    L = net.num_leaves
    live: Dict[int, frozenset] = {i: frozenset(m) for i, m in enumerate(net.leaves)}
    size: Dict[int, int] = {i: _prod(ext, m) for i, m in live.items()}
    holders: Dict[int, set] = {}
    for i, ms in live.items():
        for x in ms:
            holders.setdefault(x, set()).add(i)
    lhs, rhs = [], []
    nxt = L
    while len(live) > 1:
        best = None
        seen = set()
        for x, hs in holders.items():
            if len(hs) < 2:
                continue
            a, b = sorted(hs)
            if (a, b) in seen:
                continue
            seen.add((a, b))
            K = live[a] & live[b]
            kk = _prod(ext, K)
            c = size[a] * size[b] // (kk * kk)
            tie = (a, b) if not reverse_ties else (-b, -a)
            key = (c, c - size[a] - size[b], tie)
            if best is None or key < best[0]:
                best = (key, a, b)
        if best is None:
            ids = sorted(live)
            a, b = ids[0], ids[1]
        else:
            _, a, b = best
        K = live[a] & live[b]
        C = (live[a] | live[b]) - K
        for x in live[a]:
            holders[x].discard(a)
        for x in live[b]:
            holders[x].discard(b)
        for x in K:
            holders.pop(x, None)
        del live[a], live[b]
        live[nxt] = C
        size[nxt] = _prod(ext, C)
        for x in C:
            holders.setdefault(x, set()).add(nxt)
        lhs.append(a)
        rhs.append(b)
        nxt += 1
    return Tree(lhs, rhs)


def tree_cost(net: Network, tree: Tree, sliced: Sequence[int] = ()) -> dict:
    """Sizes and operation counts of every step with ``sliced`` modes fixed."""
    ext = np.array(net.extents, dtype=np.int64).copy()
    for x in sliced:
        ext[x] = 1
    L = net.num_leaves
    modes = [frozenset(m) for m in net.leaves]
    steps = []
    max_elems = max([_prod(ext, m) for m in modes] + [1])
    flops = 0
    for a, b in zip(tree.lhs, tree.rhs):
        A, B = modes[a], modes[b]
        K = A & B
        m, n, k = _prod(ext, A - K), _prod(ext, B - K), _prod(ext, K)
        C = (A | B) - K
        modes.append(C)
        steps.append((m, n, k))
        max_elems = max(max_elems, m * n)
        flops += 8 * m * n * k
    return dict(steps=steps, max_elems=max_elems, flops=flops,
                num_slices=int(np.prod([int(net.extents[x]) for x in sliced], dtype=np.int64)) if sliced else 1)


def closed_modes(net: Network) -> List[int]:
    cnt: Dict[int, int] = {}
    for l in net.leaves:
        for x in l:
            cnt[x] = cnt.get(x, 0) + 1
    return sorted(x for x, c in cnt.items() if c == 2)


def choose_slices(net: Network, tree: Tree, s: int) -> List[int]:
    """Pick s closed modes greedily: each time the mode that minimises the
    sliced tree's largest intermediate, then its total flops, then the lowest
    label."""
    chosen: List[int] = []
    cands = closed_modes(net)
    for _ in range(s):
        best = None
        for x in cands:
            if x in chosen:
                continue
            c = tree_cost(net, tree, chosen + [x])
            key = (c["max_elems"], c["flops"], x)
            if best is None or key < best:
                best = key
        if best is None:
            break
        chosen.append(best[2])
    return chosen


def random_greedy_tree(net: Network, seed: int, alpha: float = 1.0, temperature: float = 0.3) -> Tree:
    """One randomized greedy contraction: among pairs sharing a mode, take the
    pair minimising log2|C| - alpha (log2|A| + log2|B|) plus Gumbel noise of
    scale `temperature` (temperature 0 gives a deterministic greedy)."""
    import heapq
    import math
    rng = np.random.default_rng(seed)
    ext = net.extents
    lg = {x: math.log2(float(ext[x])) for x in range(len(ext))}
    L = net.num_leaves
    live: Dict[int, frozenset] = {i: frozenset(m) for i, m in enumerate(net.leaves)}
    size = {i: sum(lg[x] for x in m) for i, m in live.items()}
    holders: Dict[int, set] = {}
    for i, ms in live.items():
        for x in ms:
            holders.setdefault(x, set()).add(i)
    heap = []

    def push(a, b):
        A, B = live[a], live[b]
        K = A & B
        kk = sum(lg[x] for x in K)
        c = size[a] + size[b] - 2 * kk
        score = c - alpha * (size[a] + size[b])
        if temperature > 0:
            score -= temperature * float(-np.log(-np.log(rng.random() + 1e-300) + 1e-300))
        heapq.heappush(heap, (score, a, b))

    for x, hs in holders.items():
        if len(hs) == 2:
            a, b = sorted(hs)
            push(a, b)
    lhs, rhs = [], []
    nxt = L
    while len(live) > 1:
        pair = None
        while heap:
            _, a, b = heapq.heappop(heap)
            if a in live and b in live:
                pair = (a, b)
                break
        if pair is None:
            ids = sorted(live)
            pair = (ids[0], ids[1])
        a, b = pair
        K = live[a] & live[b]
        C = (live[a] | live[b]) - K
        for x in live[a]:
            holders[x].discard(a)
        for x in live[b]:
            holders[x].discard(b)
        for x in K:
            holders.pop(x, None)
        del live[a], live[b]
        live[nxt] = C
        size[nxt] = sum(lg[x] for x in C)
        neigh = set()
        for x in C:
            holders.setdefault(x, set()).add(nxt)
            neigh |= holders[x]
        neigh.discard(nxt)
        for o in neigh:
            push(min(o, nxt), max(o, nxt))
        lhs.append(a)
        rhs.append(b)
        nxt += 1
    return Tree(lhs, rhs)


def search_tree(net: Network, trials: int, seed: int = 0, max_elems: Optional[int] = None,
                alphas=(0.5, 1.0, 1.5), temperatures=(0.1, 0.3, 1.0)) -> Tree:
    """Best of `trials` randomized greedy trees (seeded, deterministic), by
    (largest intermediate, total flops).  Stops early once a tree's largest
    intermediate is at most `max_elems` and no better width is found within
    the next trials/4 attempts."""
    rng = np.random.default_rng(seed)
    best = None
    best_key = None
    since = 0
    for t in range(trials):
        a = float(alphas[int(rng.integers(len(alphas)))])
        temp = float(temperatures[int(rng.integers(len(temperatures)))])
        tr = random_greedy_tree(net, int(rng.integers(1 << 31)), alpha=a, temperature=temp)
        c = tree_cost(net, tr)
        key = (c["max_elems"], c["flops"])
        if best_key is None or key < best_key:
            best, best_key, since = tr, key, 0
        else:
            since += 1
        if max_elems is not None and best_key[0] <= max_elems and since > trials // 4:
            break
    return best


def state_vector_tree(net: Network) -> Tree:
    """For a circuit network built by ``Circuit.to_network`` (kets first, then
    gates in time order, then bras): absorb the leaves in that order into one
    growing tensor, i.e. build the product state, apply every gate to the
    full state vector, then project the closed qubits.  Width 2^n; every gate
    step is a (2^(n-2) x 4 x 4) product with the state."""
    from .network import caterpillar
    return caterpillar(net.num_leaves)


def _bisect(W: np.ndarray, rng, imbalance: float, passes: int = 6) -> np.ndarray:
    """Balanced two-way split of a weighted graph (dense symmetric W, zero
    diagonal) with a small cut: the graph Laplacian's Fiedler vector, split
    at a random point inside the balance window, then Fiduccia-Mattheyses
    passes (move the unlocked vertex of largest cut reduction that keeps the
    balance, keep the best prefix of the moves).  Returns a boolean side per
    vertex."""
    n = W.shape[0]
    lo = max(1, int(np.floor(n * (1.0 - imbalance) / 2)))
    hi = min(n - 1, int(np.ceil(n * (1.0 + imbalance) / 2)))
    lap = np.diag(W.sum(axis=1)) - W
    _, vecs = np.linalg.eigh(lap)
    f = vecs[:, 1] + 1e-6 * rng.standard_normal(n)
    order = np.argsort(f)
    n0 = int(rng.integers(lo, hi + 1))          # vertices on side False
    side = np.zeros(n, dtype=bool)
    side[order[n0:]] = True
    for _ in range(passes):
        s = side.astype(np.float64)
        other = np.where(side, W @ (1.0 - s), W @ s)
        same = W.sum(axis=1) - other
        gain = other - same
        locked = np.zeros(n, dtype=bool)
        count0 = int(n - side.sum())
        cut = 0.0
        best, best_k = 0.0, 0
        moves = []
        for _step in range(n):
            can = ~locked & np.where(side, count0 + 1 <= hi, count0 - 1 >= lo)
            if not can.any():
                break
            g = np.where(can, gain + 1e-9 * rng.random(n), -np.inf)
            i = int(np.argmax(g))
            cut -= gain[i]
            new = not side[i]
            side[i] = new
            count0 += -1 if new else 1
            locked[i] = True
            # neighbours now on i's side lose 2 w, the others gain 2 w
            gain += np.where(side == new, -2.0, 2.0) * W[i]
            gain[i] = -gain[i]
            moves.append(i)
            if cut < best - 1e-12:
                best, best_k = cut, len(moves)
        for i in moves[best_k:]:
            side[i] = not side[i]
        if best_k == 0:
            break
    return side


def partition_tree(net: Network, seed: int = 0, imbalance: float = 0.2, cutoff: int = 10) -> Tree:
    """Contraction tree by recursive balanced bisection of the leaves: each
    set of leaves is split in two with a small cut (the closed modes joining
    the halves, weighted by log2 of their extents), both halves are
    contracted recursively and their results are contracted last; sets of at
    most ``cutoff`` leaves are contracted by the greedy rule (smallest result
    first).  Seeded; ``imbalance`` bounds each split's size ratio."""
    import math
    rng = np.random.default_rng(seed)
    L = net.num_leaves
    ext = net.extents
    lg = [math.log2(float(e)) for e in ext]
    W = np.zeros((L, L))
    holders: Dict[int, List[int]] = {}
    for i, ms in enumerate(net.leaves):
        for x in ms:
            holders.setdefault(x, []).append(i)
    for x, hs in holders.items():
        if len(hs) == 2:
            a, b = hs
            W[a, b] += lg[x]
            W[b, a] += lg[x]
    modes: Dict[int, frozenset] = {i: frozenset(m) for i, m in enumerate(net.leaves)}
    lhs: List[int] = []
    rhs: List[int] = []

    def contract(a: int, b: int) -> int:
        K = modes[a] & modes[b]
        c = L + len(lhs)
        modes[c] = (modes[a] | modes[b]) - K
        lhs.append(a)
        rhs.append(b)
        return c

    def size(ms) -> float:
        return sum(lg[x] for x in ms)

    def greedy(ids: List[int]) -> int:
        live = list(ids)
        while len(live) > 1:
            best = None
            for u in range(len(live)):
                for v in range(u + 1, len(live)):
                    a, b = live[u], live[v]
                    K = modes[a] & modes[b]
                    if not K:
                        continue
                    c = size(modes[a]) + size(modes[b]) - 2 * size(K)
                    key = (c, c - size(modes[a]) - size(modes[b]), min(a, b), max(a, b))
                    if best is None or key < best[0]:
                        best = (key, a, b)
            if best is None:
                a, b = sorted(live)[:2]
            else:
                a, b = best[1], best[2]
            live.remove(a)
            live.remove(b)
            live.append(contract(a, b))
        return live[0]

    def build(nodes: List[int]) -> int:
        if len(nodes) <= cutoff:
            return greedy(nodes)
        idx = np.array(nodes)
        side = _bisect(W[np.ix_(idx, idx)], rng, imbalance)
        p = [int(v) for v in idx[~side]]
        q = [int(v) for v in idx[side]]
        return contract(build(p), build(q))

    build(list(range(L)))
    return Tree(lhs, rhs)


def partition_search(net: Network, trials: int, seed: int = 0, imbalances=(0.05, 0.1, 0.2, 0.3, 0.45),
                     cutoffs=(6, 10, 16)) -> Tree:
    """Best of ``trials`` seeded partition trees (random imbalance and
    cutoff per trial) by (largest intermediate, total flops)."""
    rng = np.random.default_rng(seed)
    best, best_key = None, None
    for _ in range(trials):
        im = float(imbalances[int(rng.integers(len(imbalances)))])
        co = int(cutoffs[int(rng.integers(len(cutoffs)))])
        tr = partition_tree(net, seed=int(rng.integers(1 << 31)), imbalance=im, cutoff=co)
        c = tree_cost(net, tr)
        key = (c["max_elems"], c["flops"])
        if best_key is None or key < best_key:
            best, best_key = tr, key
    return best


# ---------------------------------------------------------------------------
# native tree and slice search (treeopt.cpp)

_TREEOPT = None


def _treeopt_lib():
    global _TREEOPT
    if _TREEOPT is None:
        import ctypes
        import os
        from . import treeopt_build
        if not os.path.exists(treeopt_build.LIB):
            treeopt_build.build()
        lib = ctypes.CDLL(treeopt_build.LIB)
        P = ctypes.POINTER
        lib.treeopt_search.restype = ctypes.c_int
        lib.treeopt_search.argtypes = [ctypes.c_int32, ctypes.c_int32, P(ctypes.c_double), P(ctypes.c_int32),
                                       P(ctypes.c_int32), P(ctypes.c_double), P(ctypes.c_int32),
                                       P(ctypes.c_int32), P(ctypes.c_int32), P(ctypes.c_int32),
                                       P(ctypes.c_double)]
        lib.treeopt_refine.restype = ctypes.c_int
        lib.treeopt_refine.argtypes = lib.treeopt_search.argtypes
        _TREEOPT = lib
    return _TREEOPT


def _treeopt_call(fn: str, net: Network, params, tree: Optional[Tree] = None, sliced: Sequence[int] = (),
                  max_sliced: int = 64):
    import ctypes
    import math
    lib = _treeopt_lib()
    L = net.num_leaves
    logw = np.ascontiguousarray([math.log2(float(e)) for e in net.extents], dtype=np.float64)
    rank = np.ascontiguousarray([len(l) for l in net.leaves], dtype=np.int32)
    modes = np.ascontiguousarray([x for l in net.leaves for x in l] or [0], dtype=np.int32)
    params = np.ascontiguousarray(params, dtype=np.float64)
    lhs = np.zeros(max(1, L - 1), np.int32)
    rhs = np.zeros(max(1, L - 1), np.int32)
    sl = np.zeros(max(1, max_sliced, len(sliced)), np.int32)
    if tree is not None:
        lhs[:L - 1] = tree.lhs
        rhs[:L - 1] = tree.rhs
    sl[:len(sliced)] = list(sliced)
    ns = ctypes.c_int32(len(sliced))
    st = np.zeros(4, np.float64)
    P = ctypes.POINTER
    rc = getattr(lib, fn)(L, len(net.extents), logw.ctypes.data_as(P(ctypes.c_double)),
                          rank.ctypes.data_as(P(ctypes.c_int32)), modes.ctypes.data_as(P(ctypes.c_int32)),
                          params.ctypes.data_as(P(ctypes.c_double)), lhs.ctypes.data_as(P(ctypes.c_int32)),
                          rhs.ctypes.data_as(P(ctypes.c_int32)), sl.ctypes.data_as(P(ctypes.c_int32)),
                          ctypes.byref(ns), st.ctypes.data_as(P(ctypes.c_double)))
    if rc != 0:
        raise RuntimeError(f"{fn} failed ({rc})")
    out = Tree([int(x) for x in lhs[:L - 1]], [int(x) for x in rhs[:L - 1]])
    return out, [int(x) for x in sl[:ns.value]], dict(log2_cost=float(st[0]), width=float(st[1]),
                                                      peak_log2=float(st[2]), trial=int(st[3]))


def optimize_tree(net: Network, trials: int = 64, seed: int = 0, max_log_width: float = 1e9,
                  max_log_peak: float = 1e9, reconf_k: int = 8, reconf_rounds: int = 4, imbalance=(0.0, 0.3),
                  cutoff=(6, 10), threads: int = 8, time_limit_s: float = 0.0, max_sliced: int = 64,
                  ridge: float = 0.0, score_ridge: float = 0.0):
    """Tree and sliced modes from the native search (recursive multilevel
    bisection, subtree reconfiguration, slicing interleaved with
    reconfiguration; see treeopt.cpp).  Slices until the widest sliced
    intermediate has at most 2^max_log_width entries and at most
    2^max_log_peak entries are live at once (in the returned step order).
    Returns (Tree, sliced modes, stats) with stats = dict(log2_cost: log2 of
    2^s * sum of m n k, width: log2 entries of the largest sliced
    intermediate, peak_log2, trial).  Deterministic for a given seed and
    parameters (the best trial wins, ties to the lowest index).  With
    ``ridge`` > 0 a step costs max(m n k, ridge (m k + n k + m n)) instead of
    m n k: its roofline time on a device doing ``ridge`` multiply-adds per
    entry moved (a complex64 step on MI355X: 157.3e12 / 8 flop per
    multiply-add against 8e12 / 8 entries per second gives 19.7).
    ``score_ridge`` > 0 ranks the finished trials by that roofline cost
    while each trial still minimises its own cost (log2_cost is then in
    roofline units)."""
    params = [trials, threads, seed, max_log_width, reconf_k, reconf_rounds, imbalance[0], imbalance[1],
              cutoff[0], cutoff[1], time_limit_s, max_sliced, max_log_peak, ridge, score_ridge]
    return _treeopt_call("treeopt_search", net, params, max_sliced=max_sliced)


def refine_tree(net: Network, tree: Tree, sliced: Sequence[int] = (), reconf_k: int = 10, reconf_rounds: int = 8,
                max_log_width: float = 1e9, max_log_peak: float = 1e9, seed: int = 0, max_sliced: int = 64,
                ridge: float = 0.0):
    """Reconfigure a given tree (frontier of ``reconf_k`` tensors) with its
    sliced modes, slicing further if a bound is exceeded; same returns as
    ``optimize_tree``."""
    params = [1, 1, seed, max_log_width, reconf_k, reconf_rounds, 0.0, 0.0, 1, 1, 0.0, max_sliced, max_log_peak,
              ridge, 0.0]
    return _treeopt_call("treeopt_refine", net, params, tree=tree, sliced=sliced, max_sliced=max_sliced)


def stored_tree(name: str, net: Optional[Network] = None):
    """(Tree, sliced modes, record) of a stored search result
    (``workloads/data/<name>.json``, written by ``workloads/make_trees.py``).
    With ``net`` given, checks that the record belongs to that network."""
    import json
    import os
    from . import make_trees
    with open(make_trees.path(name)) as f:
        rec = json.load(f)
    if net is not None and make_trees.structure_digest(net) != rec["network"]["structure_sha256"]:
        raise ValueError(f"stored tree {name} belongs to another network")
    return Tree(rec["lhs"], rec["rhs"]), list(rec["sliced"]), rec


def more_slices(net: Network, tree: Tree, sliced: Sequence[int], extra: int,
                max_log_width: Optional[float] = None, max_flop: Optional[float] = None) -> List[int]:
    """Extend ``sliced`` greedily: each time the mode held by the most
    intermediates of the largest (sliced) width, ties broken by the operation
    count of the steps holding it (slicing it removes the most work), then
    the lowest label.  Takes ``extra`` modes, or, with bounds given, as many
    as needed until the widest sliced intermediate has at most
    2^max_log_width entries and one slice at most max_flop (8 m n k)."""
    L = net.num_leaves
    sets = [0] * (L + len(tree.lhs))
    for i, l in enumerate(net.leaves):
        for x in l:
            sets[i] |= 1 << x
    for s, (a, b) in enumerate(zip(tree.lhs, tree.rhs)):
        sets[L + s] = sets[a] ^ sets[b]
    unions = [sets[a] | sets[b] for a, b in zip(tree.lhs, tree.rhs)]
    lw = [float(np.log2(float(e))) for e in net.extents]

    def size(bits):
        t = 0.0
        while bits:
            x = (bits & -bits).bit_length() - 1
            t += lw[x]
            bits &= bits - 1
        return t

    out = list(sliced)
    added = 0
    while True:
        mask = 0
        for x in out:
            mask |= 1 << x
        widths = [size(t & ~mask) for t in sets]
        w = max(widths)
        if max_log_width is None and added >= extra:
            break
        if max_log_width is not None:
            fl = sum(8.0 * 2.0 ** size(u & ~mask) for u in unions)
            if w <= max_log_width and (max_flop is None or fl <= max_flop):
                break
        contrib: Dict[int, float] = {}
        for u in unions:
            c = 2.0 ** size(u & ~mask)
            v = u & ~mask
            while v:
                x = (v & -v).bit_length() - 1
                contrib[x] = contrib.get(x, 0.0) + c
                v &= v - 1
        widest = [t & ~mask for t, wt in zip(sets, widths) if wt >= w - 1e-9]
        hits: Dict[int, int] = {}
        for t in widest:
            v = t
            while v:
                x = (v & -v).bit_length() - 1
                if lw[x] > 0:
                    hits[x] = hits.get(x, 0) + 1
                v &= v - 1
        if not hits:
            break
        x = max(hits, key=lambda y: (hits[y], contrib.get(y, 0.0), -y))
        out.append(x)
        added += 1
    return out
