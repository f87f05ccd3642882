"""Oracle for the execution plan: mode orders, node descriptors, launch
groups and arena offsets, which the GPU library's planner must reproduce
bit-exactly.

TEST INFRASTRUCTURE ONLY (see the package docstring).

Mode orders follow the reverse-tree "lifetime ordering" of the source page
("Parallelizing Large-Scale Tensor Network Contraction on Multiple GPUs",
section 1.4): the root takes the requested output order; walking the steps
from last to first, an operand's order is the order of its product with the
modes the product does not carry dropped, followed by the modes reduced at
that step.  The reduced modes are appended in ascending label order (the page
only says they are appended together; one common order for both operands is
what makes them a GEMM's K axis).

``death_sort_orders`` is an independent formulation used to pin the reverse
pass: every tensor's order is its modes sorted by the step at which each mode
is reduced, latest first (open modes count as never reduced and keep the
output order among themselves; modes reduced at the same step are in
ascending label order).  The page describes this as the emergent property of
the reverse pass (section 1.4, the paragraph after the algorithm).

Everything else (node classes, operand orientation, output runs, split-K,
grouping, fused chains and first-fit arena) is this project's own execution
design; the rules are restated here from their definitions.
"""

from __future__ import annotations

from dataclasses import dataclass, field
from typing import Dict, List, Optional, Sequence

INF = float("inf")

LIFETIME = 0
NAIVE = 1

CLASS_TINY = 0
CLASS_SKINNY = 1
CLASS_GEMM = 2

SKINNY_MAX_SIDE = 16        # skinny when the smaller of m, n is at most this
GEMM_NOMINAL_TILE = 128     # nominal tile edge used only by the split-K rule
EARLY_STAGE_MAX = 1 << 16   # staged leaves up to this many entries are copied before the first group
FUSE_PASS_ENTRIES = 1024    # entries of the long operand in one pass of a fused chain
FUSE_MIN_ROWS = 1 << 16     # fused chains need at least this many rows of the long operand
FUSE_MAX_STEPS = 6          # the longest fused chain
NONE = (1 << 64) - 1        # "not in the arena"


def _prod(ext, modes) -> int:
    p = 1
    for x in modes:
        p *= int(ext[x])
    return p


def _pow2_floor(v: int) -> int:
    p = 1
    while p * 2 <= v:
        p *= 2
    return p


def _ceil_div(a: int, b: int) -> int:
    return -(-a // b)


class PlanError(Exception):
    def __init__(self, code: str, msg: str = ""):
        super().__init__(f"{code}: {msg}")
        self.code = code


# ----------------------------------------------------------------------------
# validation and SSA bookkeeping


def validate(extents, leaves, out_modes, lhs, rhs, sliced=()):
    nm = len(extents)
    for e in extents:
        if int(e) < 1:
            raise PlanError("INVALID_NETWORK", "extent < 1")
    L = len(leaves)
    if L < 1:
        raise PlanError("INVALID_ARG", "no leaves")
    count = [0] * nm
    for l in leaves:
        if len(set(l)) != len(l):
            raise PlanError("UNSUPPORTED", "mode repeated within one leaf")
        for x in l:
            if not (0 <= x < nm):
                raise PlanError("INVALID_NETWORK", "mode label out of range")
            count[x] += 1
    if len(set(out_modes)) != len(out_modes):
        raise PlanError("INVALID_NETWORK", "repeated output mode")
    in_out = [False] * nm
    for x in out_modes:
        if not (0 <= x < nm):
            raise PlanError("INVALID_NETWORK", "output mode out of range")
        in_out[x] = True
    for x in range(nm):
        c = count[x] + (1 if in_out[x] else 0)
        if c > 2:
            raise PlanError("UNSUPPORTED", "mode in more than two tensors")
        if c == 1:
            raise PlanError("INVALID_NETWORK", "dangling mode")
        if in_out[x] and count[x] != 1:
            raise PlanError("INVALID_NETWORK", "open mode not on exactly one leaf")
    S = len(lhs)
    if S != L - 1 or len(rhs) != S:
        raise PlanError("INVALID_TREE", "number of steps must be leaves - 1")
    used = [False] * (L + S)
    for s in range(S):
        a, b = int(lhs[s]), int(rhs[s])
        for t in (a, b):
            if not (0 <= t < L + s) or used[t]:
                raise PlanError("INVALID_TREE", "bad or reused operand")
            used[t] = True
        if a == b:
            raise PlanError("INVALID_TREE", "operand used twice")
    sl = list(sliced)
    if len(set(sl)) != len(sl):
        raise PlanError("INVALID_ARG", "repeated sliced mode")
    for x in sl:
        if not (0 <= x < nm) or count[x] != 2:
            raise PlanError("INVALID_ARG", "sliced mode must be a closed mode")


def ssa_modes(leaves, lhs, rhs, sliced):
    """Mode sets of every SSA tensor (sliced modes removed), and per-step
    (K, M, N) sets."""
    sl = set(sliced)
    sets = [frozenset(x for x in l if x not in sl) for l in leaves]
    steps = []
    for a, b in zip(lhs, rhs):
        A, B = sets[a], sets[b]
        K = A & B
        steps.append((K, A - K, B - K))
        sets.append((A | B) - K)
    return sets, steps


def death_steps(leaves, lhs, rhs, sliced) -> Dict[int, float]:
    """Step index at which each (non-sliced) mode is reduced; open = inf."""
    _, steps = ssa_modes(leaves, lhs, rhs, sliced)
    d: Dict[int, float] = {}
    for l in leaves:
        for x in l:
            d[x] = INF
    for s, (K, _, _) in enumerate(steps):
        for x in K:
            d[x] = s
    return d


# ----------------------------------------------------------------------------
# orders


def lifetime_orders(leaves, out_modes, lhs, rhs, sliced=()) -> List[List[int]]:
    """Reverse pass over the tree: the product's order fixes each operand's
    retained modes, and the reduced modes (ascending label) go last."""
    L, S = len(leaves), len(lhs)
    sets, steps = ssa_modes(leaves, lhs, rhs, sliced)
    order: List[Optional[List[int]]] = [None] * (L + S)
    order[L + S - 1] = list(out_modes)
    for s in range(S - 1, -1, -1):
        K, _, _ = steps[s]
        c_order = order[L + s]
        reduced = sorted(K)
        for operand in (lhs[s], rhs[s]):
            kept = [x for x in c_order if x in sets[operand]]
            order[operand] = kept + reduced
    return order  # type: ignore[return-value]


def death_sort_orders(leaves, out_modes, lhs, rhs, sliced=()) -> List[List[int]]:
    """Independent formulation: sort each tensor's modes by death step,
    latest first; open modes first, in output order; equal deaths by label."""
    sets, _ = ssa_modes(leaves, lhs, rhs, sliced)
    death = death_steps(leaves, lhs, rhs, sliced)
    pos = {x: i for i, x in enumerate(out_modes)}

    def key(x):
        if death[x] == INF:
            return (0, pos[x])
        return (1, -death[x], x)

    return [sorted(ms, key=key) for ms in sets]


def naive_orders(leaves, lhs, rhs, sliced=()):
    """Forward order policy used for the ablation: intermediates keep
    [A's retained modes in A's order | B's retained modes in B's order];
    operands are re-laid as [retained | K ascending] whenever they differ."""
    L, S = len(leaves), len(lhs)
    sl = set(sliced)
    sets, steps = ssa_modes(leaves, lhs, rhs, sliced)
    order = [[x for x in l if x not in sl] for l in leaves] + [None] * S
    gemm_a, gemm_b = [], []
    for s in range(S):
        K, _, _ = steps[s]
        a, b = lhs[s], rhs[s]
        ra = [x for x in order[a] if x not in K]
        rb = [x for x in order[b] if x not in K]
        gemm_a.append(ra + sorted(K))
        gemm_b.append(rb + sorted(K))
        order[L + s] = ra + rb
    return order, gemm_a, gemm_b


# ----------------------------------------------------------------------------
# the plan


@dataclass
class Node:
    step: int
    lhs: int
    rhs: int
    out: int
    m: int
    n: int
    k: int
    cls: int
    swap: int
    splits: int
    group: int = -1
    row_runs: List[tuple] = field(default_factory=list)   # (size, stride), outermost first
    col_runs: List[tuple] = field(default_factory=list)
    inner_run: int = 1
    interleaved: int = 0
    copy_a: int = 0          # operand A is re-laid into the arena before the step
    copy_b: int = 0
    a_off: int = NONE        # arena offset of the GEMM's A operand (copy or intermediate)
    b_off: int = NONE
    c_off: int = NONE        # NONE = written to the output buffer
    scratch_off: int = NONE
    scratch_bytes: int = 0
    fuse_next: int = -1      # the next step of its fused chain
    fuse_prev: int = -1      # the previous step of its fused chain
    fused_with: int = -1     # earlier steps: the chain's last step; the last step: the chain's first


@dataclass
class Plan:
    order: List[List[int]]
    gemm_a: List[List[int]]
    gemm_b: List[List[int]]
    nodes: List[Node]
    groups: List[List[int]]
    arena_bytes: int
    tensor_off: List[int]
    root_permute: int
    root_off: int
    staged_leaf: List[int]
    flops: int
    flops_unsliced: int
    bytes: int
    max_elems: int
    num_slices: int
    fused: List[tuple] = field(default_factory=list)   # fused chains: their steps, in order


def _runs(c_order, ext, row_set):
    """Maximal runs of same-side modes along c_order (extent-1 modes skipped).
    Returns (row_runs, col_runs, inner_run, n_runs) with (size, stride) per
    run, stride = stride in C of the run's innermost mode."""
    eff = [x for x in c_order if int(ext[x]) > 1]
    stride = {}
    s = 1
    for x in reversed(eff):
        stride[x] = s
        s *= int(ext[x])
    runs = []  # (is_row, size, stride)
    for x in eff:
        side = x in row_set
        if runs and runs[-1][0] == side:
            r = runs[-1]
            runs[-1] = (side, r[1] * int(ext[x]), stride[x])
        else:
            runs.append((side, int(ext[x]), stride[x]))
    row_runs = [(sz, st) for side, sz, st in runs if side]
    col_runs = [(sz, st) for side, sz, st in runs if not side]
    inner = runs[-1][1] if runs else 1
    return row_runs, col_runs, inner, len(runs)


def _split_rule(cls, R, S, k, c64):
    """K split count: enough workgroups to fill the chip, K chunks of at
    least 64 (GEMM) / 1024 (skinny) entries.  Complex64 GEMM-class steps
    with R S <= 2^19 and K <= 512 are not split (the small-GEMM kernel
    splits their K inside each workgroup)."""
    if cls == CLASS_GEMM:
        if c64 and R * S <= 1 << 19 and k <= 512:
            return 1
        tiles = _ceil_div(R, GEMM_NOMINAL_TILE) * _ceil_div(S, GEMM_NOMINAL_TILE)
        if tiles >= 256 or k < 128:
            return 1
        return max(1, min(_pow2_floor(512 // tiles), _pow2_floor(k // 64)))
    if cls == CLASS_SKINNY:
        blocks = _ceil_div(R, 256)
        if blocks >= 512 or k < 2048:
            return 1
        return max(1, min(_pow2_floor(1024 // blocks), _pow2_floor(k // 1024)))
    return 1


class _Arena:
    """First-fit over a free list of [start, end) holes; the last hole is
    unbounded.  Frees coalesce with neighbours."""

    def __init__(self):
        self.free = [[0, None]]
        self.peak = 0

    def alloc(self, size: int) -> int:
        for h in self.free:
            start, end = h
            if end is None or end - start >= size:
                off = start
                h[0] = start + size
                if end is not None and h[0] == end:
                    self.free.remove(h)
                self.peak = max(self.peak, off + size)
                return off
        raise AssertionError("unreachable")

    def release(self, off: int, size: int):
        self.free.append([off, off + size])
        self.free.sort(key=lambda h: h[0])
        merged = []
        for h in self.free:
            if merged and merged[-1][1] is not None and merged[-1][1] == h[0]:
                merged[-1][1] = h[1]
            else:
                merged.append(list(h))
        self.free = merged


def _is_pow2(v: int) -> bool:
    return v >= 1 and (v & (v - 1)) == 0


def _log2(v: int) -> int:
    return v.bit_length() - 1


def fused_pairs(nodes, sets, ext, L, eb, policy, fuse=True):
    """Chains of steps run as one pass: a long tensor T absorbs a small one
    (K = S = 2, 4, 8, 16 or 32 entries) and the product T1 is at once the long
    operand of the next step, which reduces it against another small tensor
    (K = S = 2, 4, 8, 16 or 32; K = 2 only beside K <= 8), with every extent of the modes involved a power
    of two, T holding at least 2^16 rows, both steps outside the tiny class,
    neither split over K nor the root, T1 read in place, and the modes of the
    second step's K that T carries spanning at most 1024 / K1 index values (so
    that a pass over 1024 entries of T yields whole rows of the second step).
    A chain extends to the next step in the same way, one step at a time up to
    FUSE_MAX_STEPS steps, while every K of the chain is 2, 4 or 8 and the modes of T reduced by
    all later steps together span at most 1024 / K1 values (256 / K1 for
    chains of four or more, which leaves two of a pass's row bits to give its
    stores contiguous pieces).  Chains are taken in step order and do not
    overlap.  Complex64, lifetime order."""
    if not fuse or policy != LIFETIME or eb != 8:
        return []
    consumer = {}
    for nd in nodes:
        consumer[nd.lhs] = nd.step
        consumer[nd.rhs] = nd.step
    chains = []
    taken = set()

    def long_short(nd):
        # (long operand, its rows, the short side) with lhs taken when m >= n
        return (nd.lhs, nd.m, nd.n) if nd.m >= nd.n else (nd.rhs, nd.n, nd.m)

    def link(prev, s, ks):
        """The small operand of step s when it may follow step prev in a
        chain whose K so far are ks, else None."""
        c = nodes[s]
        t, _, sw = long_short(c)
        if c.cls == CLASS_TINY or c.splits > 1 or s == len(nodes) - 1:
            return None
        if t != L + prev or (c.copy_a if t == c.lhs else c.copy_b) or sw != c.k:
            return None
        if len(ks) == 1:
            if c.k not in (2, 4, 8, 16, 32) or (2 in (ks[0], c.k) and max(ks[0], c.k) > 8):
                return None   # a pair: K = 2 only beside K <= 8
        elif c.k not in (2, 4, 8) or any(k not in (2, 4, 8) for k in ks):
            return None   # a chain of three or more: every K 2, 4 or 8
        small = c.rhs if t == c.lhs else c.lhs
        if not all(_is_pow2(ext[x]) for x in sets[small]):
            return None
        return small

    for a in nodes:
        s1 = a.step
        if a.cls == CLASS_TINY or a.splits > 1 or s1 in taken or (L + s1) not in consumer:
            continue
        t, r1, s1w = long_short(a)
        if a.k not in (2, 4, 8, 16, 32) or s1w != a.k or not _is_pow2(r1) or r1 < FUSE_MIN_ROWS:
            continue
        small1 = a.rhs if t == a.lhs else a.lhs
        if not all(_is_pow2(ext[x]) for u in (t, small1) for x in sets[u]):
            continue
        chain, ks, bits_t = [s1], [a.k], 0
        while len(chain) < FUSE_MAX_STEPS and (L + chain[-1]) in consumer:
            s = consumer[L + chain[-1]]
            small = link(chain[-1], s, ks)
            if small is None:
                break
            # the modes of T that the chain's later steps reduce, in index bits;
            # a chain of four or more leaves two of the pass's rows free
            bits = bits_t + sum(_log2(ext[x]) for x in sets[t] if x in sets[small])
            if bits > _log2(FUSE_PASS_ENTRIES // a.k) - (2 if len(chain) >= 3 else 0):
                break
            chain.append(s)
            ks.append(nodes[s].k)
            bits_t = bits
        if len(chain) < 2:
            continue
        for x, y in zip(chain, chain[1:]):
            nodes[x].fuse_next, nodes[y].fuse_prev = y, x
        for x in chain[:-1]:
            nodes[x].fused_with = chain[-1]
        nodes[chain[-1]].fused_with = chain[0]
        taken.update(chain)
        chains.append(tuple(chain))
    return chains


def make_plan(extents, leaves, out_modes, lhs, rhs, policy=LIFETIME, sliced=(), align=256,
              tiny_mnk=1 << 17, max_group=256, dtype=0, fuse=True) -> Plan:
    """dtype 0: complex64 (8-byte entries), 1: complex128 (16-byte entries)."""
    eb = 16 if dtype == 1 else 8
    validate(extents, leaves, out_modes, lhs, rhs, sliced)
    L, S = len(leaves), len(lhs)
    sl = set(sliced)
    ext = [1 if x in sl else int(e) for x, e in enumerate(extents)]
    sets, steps = ssa_modes(leaves, lhs, rhs, sliced)
    declared = [[x for x in l if x not in sl] for l in leaves]
    has_sliced = [any(x in sl for x in l) for l in leaves]

    if policy == LIFETIME:
        order = lifetime_orders(leaves, out_modes, lhs, rhs, sliced)
        gemm_a = [order[a] for a in lhs]
        gemm_b = [order[b] for b in rhs]
        root_permute = 0
    else:
        order, gemm_a, gemm_b = naive_orders(leaves, lhs, rhs, sliced)
        root_permute = int(S > 0 and order[L + S - 1] != list(out_modes))

    staged_leaf = [0] * L
    nodes: List[Node] = []
    flops = flops_u = nbytes = 0
    max_elems = 0
    for s in range(S):
        K, M, N = steps[s]
        a, b = lhs[s], rhs[s]
        m, n, k = _prod(ext, M), _prod(ext, N), _prod(ext, K)
        mu = _prod(extents, M); nu = _prod(extents, N); ku = _prod(extents, K)
        flops += 8 * m * n * k
        flops_u += 8 * mu * nu * ku
        nbytes += eb * (m * k + n * k + m * n)
        max_elems = max(max_elems, m * n)
        if m * n * k <= tiny_mnk and m * k + n * k + m * n <= tiny_mnk // 4:
            cls = CLASS_TINY
        elif min(m, n) <= SKINNY_MAX_SIDE:
            cls = CLASS_SKINNY
        else:
            cls = CLASS_GEMM
        # C's order as the GEMM writes it
        c_order = order[L + s] if not (policy == NAIVE) else order[L + s]
        eff = [x for x in c_order if ext[x] > 1]
        if cls == CLASS_SKINNY:
            swap = int(n > m)
        else:
            swap = int(bool(eff) and eff[-1] in M)
        row_set = N if swap else M
        row_runs, col_runs, inner, nruns = _runs(c_order, ext, row_set)
        R, Sx = (n, m) if swap else (m, n)
        if cls == CLASS_GEMM and max(R, Sx, k) >= 1 << 31:
            raise PlanError("UNSUPPORTED", "GEMM step with a side or K of 2^31 or more")
        splits = _split_rule(cls, R, Sx, k, eb == 8)
        node = Node(step=s, lhs=a, rhs=b, out=L + s, m=m, n=n, k=k, cls=cls, swap=swap, splits=splits,
                    row_runs=row_runs, col_runs=col_runs, inner_run=inner, interleaved=int(nruns > 2))
        # operand copies
        for which, t, want in (("a", a, gemm_a[s]), ("b", b, gemm_b[s])):
            if t < L:
                need = has_sliced[t] or declared[t] != want
                if need:
                    staged_leaf[t] = 1
            else:
                need = order[t] != want
            setattr(node, "copy_" + which, int(need))
        if splits > 1:
            node.scratch_bytes = splits * R * Sx * eb
        nodes.append(node)

    fused = fused_pairs(nodes, sets, ext, L, eb, policy, fuse)

    # launch groups: the tiny steps between two non-tiny steps (a segment)
    # run in dependency-level order, one group per level (split at max_group
    # members, list order inside a level); non-tiny steps are groups of their
    # own.  Level = 0 unless an operand was produced in the same segment, then
    # one more than that producer's level.
    groups: List[List[int]] = []
    segment: List[int] = []

    def flush_segment():
        if not segment:
            return
        level = {}
        for s in segment:
            nd = nodes[s]
            lv = 0
            for t in (nd.lhs, nd.rhs):
                if t in level:
                    lv = max(lv, level[t] + 1)
            level[nd.out] = lv
        depth = max(level.values()) + 1
        for lv in range(depth):
            members = [s for s in segment if level[nodes[s].out] == lv]
            for i in range(0, len(members), max_group):
                groups.append(members[i:i + max_group])
        segment.clear()

    for s, nd in enumerate(nodes):
        if nd.cls == CLASS_TINY:
            segment.append(s)
        else:
            flush_segment()
            groups.append([s])
    flush_segment()
    for g, members in enumerate(groups):
        for s in members:
            nodes[s].group = g

    # arena
    def rbytes(elems):
        return _ceil_div(elems * eb, align) * align

    arena = _Arena()
    tensor_off = [NONE] * (L + S)
    elems_of = [_prod(ext, st) for st in sets]
    root = L + S - 1
    root_off = NONE
    # early staging: copies of leaves with at most EARLY_STAGE_MAX entries are
    # made in one launch before the first group, so they are allocated first
    # (in execution order, A before B) and freed with their consumer group
    early = set()
    for members in groups:
        for s in members:
            nd = nodes[s]
            for which, t in (("a", nd.lhs), ("b", nd.rhs)):
                if getattr(nd, "copy_" + which) and t < L and elems_of[t] <= EARLY_STAGE_MAX:
                    off = arena.alloc(rbytes(elems_of[t]))
                    setattr(nd, which + "_off", off)
                    if policy == LIFETIME:
                        tensor_off[t] = off
                    early.add((s, which))
    # a fused chain's earlier steps keep their operands until the chain's
    # launch (its last step's group) and never store their products
    deferred = {}
    for members in groups:
        to_free = []
        for s in members:
            nd = nodes[s]
            frees = deferred.setdefault(s, []) if nd.fuse_next >= 0 else to_free
            if nd.fuse_prev >= 0:
                # the chain's earlier steps: their operands stay until its last step
                frees.extend(deferred.pop(nd.fuse_prev))
            for which, t in (("a", nd.lhs), ("b", nd.rhs)):
                if (s, which) in early:
                    frees.append((getattr(nd, which + "_off"), rbytes(elems_of[t])))
                elif getattr(nd, "copy_" + which):
                    off = arena.alloc(rbytes(elems_of[t]))
                    frees.append((off, rbytes(elems_of[t])))
                    if t < L and policy == LIFETIME:
                        tensor_off[t] = off
                    setattr(nd, which + "_off", off)
                elif nd.fuse_prev >= 0 and t == L + nd.fuse_prev:
                    setattr(nd, which + "_off", NONE)
                elif t >= L:
                    setattr(nd, which + "_off", tensor_off[t])
                    frees.append((tensor_off[t], rbytes(elems_of[t])))
            if nd.fuse_next >= 0:
                nd.c_off = NONE
                continue
            if nd.out == root and not root_permute:
                nd.c_off = NONE
            else:
                nd.c_off = arena.alloc(rbytes(elems_of[nd.out]))
                tensor_off[nd.out] = nd.c_off
                if nd.out == root:
                    root_off = nd.c_off
            if nd.splits > 1:
                nd.scratch_off = arena.alloc(_ceil_div(nd.scratch_bytes, align) * align)
                to_free.append((nd.scratch_off, _ceil_div(nd.scratch_bytes, align) * align))
        for off, sz in to_free:
            arena.release(off, sz)
    if S == 0:
        staged_leaf = [0] * L
    return Plan(order=order, gemm_a=gemm_a, gemm_b=gemm_b, nodes=nodes, groups=groups,
                arena_bytes=arena.peak, tensor_off=tensor_off, root_permute=root_permute,
                root_off=root_off, staged_leaf=staged_leaf, flops=flops, flops_unsliced=flops_u,
                bytes=nbytes, max_elems=max_elems,
                num_slices=_prod(extents, sliced) if sliced else 1, fused=fused)
