"""Oracle for the distribution schedule over P GPUs: exhaustive search.

TEST INFRASTRUCTURE ONLY (see the package docstring).

Source: "Parallelizing Large-Scale Tensor Network Contraction on Multiple
GPUs", section 1.5 (prefix split of every tensor above a size threshold, the
Activate / Keep / Redistribute / Gather tags) and section 1.6 (keep-or-
redistribute choice along each chain of large tensors, cost of a step =
local GEMM time + communication time).  The page's formulas are stripped;
the readings below are the ones the library documents for the same call:

* a step output of more than ``threshold`` bytes (and not the root) is
  split; leaves are replicated.  A split is the shortest prefix of the
  tensor's lifetime order (extent-1 modes and excluded modes skipped) whose
  extents multiply to at least P; each GPU holds ceil(Q / P) of the Q
  slices;
* a step with replicated operands and a split output activates it on
  prefix(C); a split operand carries its split through the step (Keep) while
  none of its split modes is reduced there, or is re-split first onto
  prefix(T minus the step's reduced modes) (Redistribute; not onto its
  current split).  When both operands are split the larger carries on and
  the smaller is all-gathered first.  A step whose output is not split
  (small, or the root) gathers: all-reduce if split modes were reduced
  there, all-gather of the split output otherwise;
* t_gemm = count * max(eb (mk + nk + mn) / B_dev, 8 m n k / F_dev);
  t_comm = V / B_net + lambda * ceil(V / blk) for V bytes sent per GPU in
  contiguous blocks of blk bytes: a re-split of T sends (P - 1) |T| / P^2
  with blk = min(run, |T| / P^2), run = bytes right of the rightmost new
  split mode in the shard's layout (T's order minus the old split); an
  all-gather of T on D sends (P - 1) |T| / P with blk = min(run right of
  D's rightmost mode in T's order, |T| / P); an all-reduce of T sends
  2 (P - 1) |T| / P in 2 (P - 1) blocks.

Instead of a dynamic program, every keep/redistribute vector of every chain
is tried (2^(len - 1) per chain) and the cheapest valid one kept, so the
oracle is only for small chains.  Orders come from ``planner.lifetime_orders``.
"""

from __future__ import annotations

import itertools
import math
from typing import Dict, List, Optional, Sequence, Tuple

from .planner import lifetime_orders

REPLICATED, ACTIVATE, KEEP, REDISTRIBUTE, GATHER = range(5)


class Model:
    def __init__(self, extents, leaves, out_modes, lhs, rhs, eb, P, threshold, B_dev, F_dev, B_net, lam):
        self.ext = [int(e) for e in extents]
        self.L, self.S = len(leaves), len(lhs)
        self.lhs, self.rhs = list(lhs), list(rhs)
        self.order = lifetime_orders(leaves, out_modes, lhs, rhs)
        self.eb, self.P, self.threshold = eb, P, threshold
        self.B_dev, self.F_dev, self.B_net, self.lam = B_dev, F_dev, B_net, lam
        self.size = [eb * math.prod(self.ext[x] for x in o) for o in self.order]
        self.K = [[x for x in self.order[self.lhs[s]] if x in self.order[self.rhs[s]]] for s in range(self.S)]
        self.user = {}
        for s in range(self.S):
            self.user[self.lhs[s]] = s
            self.user[self.rhs[s]] = s

    # ---- sizes and splits
    def out(self, s):
        return self.L + s

    def is_big(self, t):
        return t >= self.L and self.P > 1 and self.size[t] > self.threshold

    def stays_whole(self, t):
        return (not self.is_big(t)) or t == self.L + self.S - 1

    def prefix(self, t, exclude=()) -> Optional[List[int]]:
        chosen, q = [], 1
        for x in self.order[t]:
            if self.ext[x] == 1 or x in exclude:
                continue
            chosen.append(x)
            q *= self.ext[x]
            if q >= self.P:
                return chosen
        return None

    # ---- costs
    def gemm_time(self, m, n, k, count):
        return count * max(self.eb * (m * k + n * k + m * n) / self.B_dev, 8.0 * m * n * k / self.F_dev)

    def sides(self, s):
        K = self.K[s]
        m = math.prod(self.ext[x] for x in self.order[self.lhs[s]] if x not in K)
        n = math.prod(self.ext[x] for x in self.order[self.rhs[s]] if x not in K)
        k = math.prod(self.ext[x] for x in K)
        return m, n, k

    def local_replicated(self, s):
        m, n, k = self.sides(s)
        return (m, n, k, 1), self.gemm_time(m, n, k, 1)

    def local_activate(self, s, D):
        m, n, k = self.sides(s)
        fl = math.prod(self.ext[x] for x in D if x in self.order[self.lhs[s]])
        fr = math.prod(self.ext[x] for x in D if x in self.order[self.rhs[s]])
        count = -(-fl * fr // self.P)
        return (m // fl, n // fr, k, count), self.gemm_time(m // fl, n // fr, k, count)

    def local_carried(self, s, side, D):
        """Operand `side` (0 lhs, 1 rhs) split on D, the other whole."""
        m, n, k = self.sides(s)
        K = self.K[s]
        f_side = math.prod(self.ext[x] for x in D if x not in K)
        f_k = math.prod(self.ext[x] for x in D if x in K)
        count = -(-(f_side * f_k) // self.P)
        if side == 0:
            lm, ln = m // f_side, n
        else:
            lm, ln = m, n // f_side
        lk = k // f_k
        return (lm, ln, lk, count), self.gemm_time(lm, ln, lk, count)

    def _blocks_time(self, v, blk):
        if v <= 0:
            return 0.0
        return v / self.B_net + self.lam * math.ceil(v / max(blk, 1.0))

    def _run_right_of(self, layout, cut):
        run = 1
        for x in reversed(layout):
            if x in cut:
                break
            run *= self.ext[x]
        return self.eb * run

    def resplit_time(self, t, old, new):
        piece = self.size[t] / (self.P * self.P)
        layout = [x for x in self.order[t] if x not in old]
        cut = [x for x in new if x not in old]
        blk = min(self._run_right_of(layout, cut), piece)
        return self._blocks_time((self.P - 1) * piece, blk)

    def allgather_time(self, t, D):
        shard = self.size[t] / self.P
        blk = min(self._run_right_of(self.order[t], D), shard)
        return self._blocks_time((self.P - 1) * shard, blk)

    def allreduce_time(self, t):
        v = 2.0 * (self.P - 1) * self.size[t] / self.P
        return v / self.B_net + self.lam * 2.0 * (self.P - 1)

    def gather_time(self, s, D):
        if any(x in self.K[s] for x in D):
            return self.allreduce_time(self.out(s))
        return self.allgather_time(self.out(s), D)

    # ---- structure
    def structure(self):
        """Which outputs are split; which operand carries a split into each
        step; which one is gathered when both are split."""
        split = [False] * (self.L + self.S)
        carry, gathered = [None] * self.S, [None] * self.S
        for s in range(self.S):
            a, b, c = self.lhs[s], self.rhs[s], self.out(s)
            if split[a] and split[b]:
                carry[s] = 1 if self.size[b] > self.size[a] else 0
                gathered[s] = 1 - carry[s]
            elif split[a] or split[b]:
                carry[s] = 0 if split[a] else 1
            if self.stays_whole(c):
                continue
            split[c] = carry[s] is not None or self.prefix(c) is not None
        return split, carry, gathered

    def chains(self, split, carry):
        """[(steps, merge step or None)] starting at every activation."""
        out = []
        for s0 in range(self.S):
            if not split[self.out(s0)] or carry[s0] is not None:
                continue
            steps, merge = [s0], None
            while split[self.out(steps[-1])]:
                t = self.out(steps[-1])
                if t not in self.user:
                    break
                c = self.user[t]
                side = 0 if self.lhs[c] == t else 1
                if carry[c] != side:
                    merge = c
                    break
                steps.append(c)
            out.append((steps, merge))
        return out

    def chain_cost(self, steps, merge, choice, split, carry):
        """Cost and per-step records of one chain under one keep (0) /
        redistribute (1) vector for steps[1:]; None if invalid."""
        recs = {}
        D = self.prefix(self.out(steps[0]))
        shape, tg = self.local_activate(steps[0], D)
        recs[steps[0]] = dict(tag=ACTIVATE, shape=shape, t_gemm=tg, t_comm=0.0, dist=list(D), local=list(D))
        total = tg
        for i in range(1, len(steps)):
            s, t = steps[i], self.out(steps[i - 1])
            whole = not split[self.out(s)]
            comm = 0.0
            if choice[i - 1]:
                if whole:
                    return None
                new = self.prefix(t, exclude=self.K[s])
                if new is None or sorted(new) == sorted(D):
                    return None
                comm += self.resplit_time(t, D, new)
                D = new
                tag = REDISTRIBUTE
            else:
                if not whole and any(x in self.K[s] for x in D):
                    return None
                tag = GATHER if whole else KEEP
            shape, tg = self.local_carried(s, carry[s], D)
            if whole:
                comm += self.gather_time(s, D)
            recs[s] = dict(tag=tag, shape=shape, t_gemm=tg, t_comm=comm, dist=[] if whole else list(D), local=list(D))
            total += tg + comm
        extra = 0.0
        if merge is not None:
            extra = self.allgather_time(self.out(steps[-1]), D)
            total += extra
        return total, recs, extra

    def best(self):
        """Cheapest schedule by exhaustive search: (total, records per step)."""
        split, carry, gathered = self.structure()
        recs: Dict[int, dict] = {}
        merge_extra: Dict[int, float] = {}
        total = 0.0
        for steps, merge in self.chains(split, carry):
            best = None
            for choice in itertools.product((0, 1), repeat=len(steps) - 1):
                r = self.chain_cost(steps, merge, choice, split, carry)
                if r is not None and (best is None or r[0] < best[0]):
                    best = r
            if best is None:
                raise ValueError(f"no feasible split along the chain from step {steps[0]}")
            total += best[0]
            recs.update(best[1])
            if merge is not None:
                merge_extra[merge] = merge_extra.get(merge, 0.0) + best[2]
        for s in range(self.S):
            if s not in recs:
                shape, tg = self.local_replicated(s)
                recs[s] = dict(tag=REPLICATED, shape=shape, t_gemm=tg, t_comm=0.0, dist=[], local=[])
                total += tg
        for s, e in merge_extra.items():
            recs[s]["t_comm"] += e
        return total, recs, carry, gathered

    def cost_of(self, tags):
        """(total, records) of the schedule whose per-step tags are given (a
        redistribute tag means the re-split before that step), or None if
        the schedule is invalid.  Used to check another planner's choice."""
        split, carry, _ = self.structure()
        total = 0.0
        recs: Dict[int, dict] = {}
        extra: Dict[int, float] = {}
        for steps, merge in self.chains(split, carry):
            choice = [1 if tags[s] == REDISTRIBUTE else 0 for s in steps[1:]]
            r = self.chain_cost(steps, merge, choice, split, carry)
            if r is None:
                return None
            total += r[0]
            recs.update(r[1])
            if merge is not None:
                extra[merge] = extra.get(merge, 0.0) + r[2]
        for s in range(self.S):
            if s not in recs:
                shape, tg = self.local_replicated(s)
                recs[s] = dict(tag=REPLICATED, shape=shape, t_gemm=tg, t_comm=0.0, dist=[], local=[])
                total += tg
        for s, e in extra.items():
            recs[s]["t_comm"] += e
        return total, recs


def model(net_extents, leaves, out_modes, lhs, rhs, eb=8, P=8, threshold=8 << 30, B_dev=8.0e12, F_dev=157.3e12,
          B_net=7 * 76.8e9, lam=5e-6) -> Model:
    return Model(net_extents, leaves, out_modes, lhs, rhs, eb, P, threshold, B_dev, F_dev, B_net, lam)
