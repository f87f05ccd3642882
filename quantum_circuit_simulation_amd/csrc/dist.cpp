// Distribution schedule of a plan over P GPUs (host only, launches nothing).
//
// Follows the page "Parallelizing Large-Scale Tensor Network Contraction on
// Multiple GPUs", section 1.5 (a tensor above the size threshold is split on
// the shortest prefix of its lifetime order whose extents multiply to at
// least P; steps are tagged Activate / Keep / Redistribute / Gather) and
// section 1.6 (along each chain of large tensors a one-dimensional dynamic
// program chooses, at every step, to keep the current split or to
// redistribute, under t = t_gemm + t_comm with t_gemm = max(bytes / B_dev,
// flops / F_dev) and t_comm = bytes / B_net + lambda * n_blk).  The page's
// formulas are stripped; the readings used here are stated at each function.
#include <algorithm>
#include <cmath>
#include <limits>
#include <string>
#include <vector>

#include "plan.hpp"

namespace tnc {

namespace {

constexpr double kInf = std::numeric_limits<double>::infinity();
using Modes = std::vector<int32_t>;

bool has(const Modes &s, int32_t x) { return std::find(s.begin(), s.end(), x) != s.end(); }

struct Dist {
  const PlanImpl &p;
  const tnc_dist_options &o;
  int64_t P;
  double eb;
  int32_t T;                          // tensors: L leaves + S step outputs
  std::vector<double> bytes;          // unsliced size of each tensor
  std::vector<Modes> kset;            // reduced modes of each step
  std::vector<int32_t> consumer;      // step consuming each tensor, -1 for the root

  Dist(const PlanImpl &plan, const tnc_dist_options &opt)
      : p(plan), o(opt), P(opt.num_gpus), eb((double)plan.elem_bytes), T(plan.L + plan.S) {
    bytes.resize(T);
    for (int32_t t = 0; t < T; ++t) {
      double e = 1;
      for (int32_t x : p.order[t]) e *= (double)p.extents[x];
      bytes[t] = eb * e;
    }
    consumer.assign(T, -1);
    kset.resize(p.S);
    for (int32_t s = 0; s < p.S; ++s) {
      const int32_t a = p.lhs[s], b = p.rhs[s];
      consumer[a] = consumer[b] = s;
      for (int32_t x : p.order[a])
        if (has(p.order[b], x)) kset[s].push_back(x);
    }
  }

  double ext(int32_t x) const { return (double)p.extents[x]; }
  double prod(const Modes &m) const {
    double v = 1;
    for (int32_t x : m) v *= ext(x);
    return v;
  }
  int32_t root() const { return T - 1; }
  bool big(int32_t t) const { return t >= p.L && P > 1 && bytes[t] > (double)o.threshold_bytes; }
  // an output that is small, or the root (which ends replicated in `out`)
  bool small_like(int32_t t) const { return !big(t) || t == root(); }

  // Shortest prefix of t's lifetime order, skipping extent-1 modes and modes
  // in `excl`, whose extents multiply to at least P.  False if none.
  bool prefix(int32_t t, const Modes &excl, Modes *d) const {
    d->clear();
    double q = 1;
    for (int32_t x : p.order[t]) {
      if (p.extents[x] <= 1 || has(excl, x)) continue;
      d->push_back(x);
      q *= ext(x);
      if (q >= (double)P) return true;
    }
    d->clear();
    return false;
  }

  // t_gemm of `count` sub-GEMMs (m, n, k): max(bytes / B_dev, flops / F_dev)
  // with bytes = entry size * (mk + nk + mn) and 8 mnk real flops per step.
  double t_gemm(double m, double n, double k, double count) const {
    const double by = eb * (m * k + n * k + m * n), fl = 8.0 * m * n * k;
    return count * std::max(by / o.hbm_bytes_per_s, fl / o.flops_per_s);
  }

  // Bytes of the contiguous runs that move when the layout `order` (minus
  // the modes in `skip`) is cut along the modes of `cut`: the product of the
  // extents right of the rightmost cut mode.  All of it if no mode is cut.
  double run_bytes(const Modes &order, const Modes &skip, const Modes &cut) const {
    double run = 1;
    for (auto it = order.rbegin(); it != order.rend(); ++it) {
      if (has(skip, *it)) continue;
      if (has(cut, *it)) return eb * run;
      run *= ext(*it);
    }
    return eb * run;
  }

  // Per-GPU time of sending V bytes in blocks of s_blk bytes.
  double send(double v, double blk) const {
    if (v <= 0) return 0;
    const double n_blk = std::ceil(v / std::max(blk, 1.0));
    return v / o.net_bytes_per_s + o.latency_s * n_blk;
  }

  // All-to-All re-split of tensor t from src to dst: each GPU keeps 1/P of
  // its shard and sends P - 1 pieces of |t| / P^2 bytes, in contiguous
  // blocks of the shard's layout cut along the new split modes.
  double t_redist(int32_t t, const Modes &src, const Modes &dst) const {
    const double piece = bytes[t] / (double)(P * P);
    Modes cut;
    for (int32_t x : dst)
      if (!has(src, x)) cut.push_back(x);
    const double blk = std::min(run_bytes(p.order[t], src, cut), piece);
    return send((double)(P - 1) * piece, blk);
  }

  // All-gather of t split on d: each GPU sends its shard of |t| / P bytes
  // to P - 1 peers, in blocks of t's layout cut along d.
  double t_allgather(int32_t t, const Modes &d) const {
    const double shard = bytes[t] / (double)P;
    const double blk = std::min(run_bytes(p.order[t], Modes{}, d), shard);
    return send((double)(P - 1) * shard, blk);
  }

  // All-reduce of partial sums of t (ring: 2 (P - 1) / P of |t| per GPU in
  // 2 (P - 1) contiguous messages).
  double t_allreduce(int32_t t) const {
    const double v = 2.0 * (double)(P - 1) * bytes[t] / (double)P;
    return v / o.net_bytes_per_s + o.latency_s * 2.0 * (double)(P - 1);
  }

  // One GPU's GEMM at step s when operand side x (0 lhs, 1 rhs) is split on
  // d: d's modes among x's kept modes divide x's side, those among the
  // reduced modes divide k; the GPU holds ceil(Q / P) of the Q slices.
  void local_split(int32_t s, int side, const Modes &d, tnc_dist_step *r) const {
    const int32_t xa = side == 0 ? p.lhs[s] : p.rhs[s], xo = side == 0 ? p.rhs[s] : p.lhs[s];
    double mx = 1, no = 1, k = 1, fm = 1, fk = 1;
    for (int32_t x : p.order[xa])
      if (!has(kset[s], x)) mx *= ext(x);
    for (int32_t x : p.order[xo])
      if (!has(kset[s], x)) no *= ext(x);
    for (int32_t x : kset[s]) k *= ext(x);
    for (int32_t x : d) (has(kset[s], x) ? fk : fm) *= ext(x);
    const double q = fm * fk, count = std::ceil(q / (double)P);
    const double lm = mx / fm, lk = k / fk;
    r->local_m = (int64_t)(side == 0 ? lm : no);
    r->local_n = (int64_t)(side == 0 ? no : lm);
    r->local_k = (int64_t)lk;
    r->local_count = (int64_t)count;
    r->t_gemm = t_gemm(lm, no, lk, count);
  }

  // Activation: C split on d = prefix(C); each GPU computes ceil(Q / P)
  // blocks of C from replicated operands.
  void local_activate(int32_t s, const Modes &d, tnc_dist_step *r) const {
    double m = 1, n = 1, k = 1, fl = 1, fr = 1;
    for (int32_t x : p.order[p.lhs[s]])
      if (!has(kset[s], x)) m *= ext(x);
    for (int32_t x : p.order[p.rhs[s]])
      if (!has(kset[s], x)) n *= ext(x);
    for (int32_t x : kset[s]) k *= ext(x);
    for (int32_t x : d) (has(p.order[p.lhs[s]], x) ? fl : fr) *= ext(x);
    const double count = std::ceil(fl * fr / (double)P);
    r->local_m = (int64_t)(m / fl);
    r->local_n = (int64_t)(n / fr);
    r->local_k = (int64_t)k;
    r->local_count = (int64_t)count;
    r->t_gemm = t_gemm(m / fl, n / fr, k, count);
  }

  void replicated(int32_t s, tnc_dist_step *r) const {
    double m = 1, n = 1, k = 1;
    for (int32_t x : p.order[p.lhs[s]])
      if (!has(kset[s], x)) m *= ext(x);
    for (int32_t x : p.order[p.rhs[s]])
      if (!has(kset[s], x)) n *= ext(x);
    for (int32_t x : kset[s]) k *= ext(x);
    r->local_m = (int64_t)m;
    r->local_n = (int64_t)n;
    r->local_k = (int64_t)k;
    r->local_count = 1;
    r->t_gemm = t_gemm(m, n, k, 1);
  }

  // Communication after a Gather step s whose operand is split on d:
  // partial sums (d meets the reduced modes) are all-reduced, otherwise the
  // split output is all-gathered.
  double t_gather_after(int32_t s, const Modes &d) const {
    const int32_t c = p.L + s;
    for (int32_t x : d)
      if (has(kset[s], x)) return t_allreduce(c);
    return t_allgather(c, d);
  }

  void set_modes(tnc_dist_step *r, int32_t out, const Modes &d) const {
    r->num_dist = 0;
    for (int32_t x : p.order[out])
      if (has(d, x)) r->dist_modes[r->num_dist++] = x;
  }

  void set_local(tnc_dist_step *r, const Modes &d) const {
    r->num_local = 0;
    for (int32_t x : d) r->local_modes[r->num_local++] = x;
  }
};

}  // namespace

tnc_status plan_distribution(const PlanImpl &p, const tnc_dist_options &o, tnc_dist_step *steps, double *total,
                             std::string *err) {
  Dist ds(p, o);
  const int32_t S = p.S, L = p.L;
  for (int32_t s = 0; s < S; ++s) {
    tnc_dist_step &r = steps[s];
    r = tnc_dist_step{};
    r.tag = TNC_DIST_REPLICATED;
    r.dist_operand = -1;
    r.gathered_operand = -1;
  }
  // Which step outputs are split, and which operand of each step carries a
  // split into it (the larger one when both do; the other is gathered).
  std::vector<char> split(ds.T, 0);
  std::vector<int> carry(S, -1), gathered(S, -1);
  for (int32_t s = 0; s < S; ++s) {
    const int32_t a = p.lhs[s], b = p.rhs[s], c = L + s;
    const bool da = split[a], db = split[b];
    if (da && db) {
      carry[s] = ds.bytes[b] > ds.bytes[a] ? 1 : 0;
      gathered[s] = 1 - carry[s];
    } else if (da || db) {
      carry[s] = da ? 0 : 1;
    }
    if (ds.small_like(c)) continue;
    if (carry[s] >= 0) {
      split[c] = 1;
    } else {
      Modes d;
      if (ds.prefix(c, Modes{}, &d)) split[c] = 1;
    }
  }
  // Chains: from each Activate step follow the carried tensor.
  std::vector<char> done(S, 0);
  for (int32_t s0 = 0; s0 < S; ++s0) {
    if (!split[L + s0] || carry[s0] >= 0) continue;
    std::vector<int32_t> ch{s0};
    int end_merge = -1;  // step where the chain's last tensor is gathered as the smaller operand
    for (;;) {
      const int32_t t = L + ch.back();
      if (!split[t]) break;
      const int32_t c = ds.consumer[t];
      if (c < 0) break;
      const int side = p.lhs[c] == t ? 0 : 1;
      if (carry[c] != side) {
        end_merge = c;
        break;
      }
      ch.push_back(c);
      if (!split[L + c]) break;
    }
    const int n = (int)ch.size();
    std::vector<Modes> gen(n);
    std::vector<char> gen_ok(n, 0);
    if (!ds.prefix(L + s0, Modes{}, &gen[0])) {
      *err = "activation without a feasible prefix";
      return TNC_ERR_UNSUPPORTED;
    }
    gen_ok[0] = 1;
    std::vector<std::vector<double>> f(n, std::vector<double>(n, kInf));
    std::vector<std::vector<int>> from(n, std::vector<int>(n, -1));
    tnc_dist_step tmp{};
    ds.local_activate(s0, gen[0], &tmp);
    f[0][0] = tmp.t_gemm;
    for (int i = 1; i < n; ++i) {
      const int32_t s = ch[i], t = L + ch[i - 1];
      const int side = carry[s];
      const bool gather = !split[L + s];
      auto disjoint = [&](const Modes &d) {
        for (int32_t x : d)
          if (has(ds.kset[s], x)) return false;
        return true;
      };
      for (int g = 0; g < i; ++g) {
        if (f[i - 1][g] == kInf || !gen_ok[g]) continue;
        if (!gather && !disjoint(gen[g])) continue;
        ds.local_split(s, side, gen[g], &tmp);
        double c = f[i - 1][g] + tmp.t_gemm;
        if (gather) c += ds.t_gather_after(s, gen[g]);
        f[i][g] = c;
        from[i][g] = g;
      }
      if (!gather && ds.prefix(t, ds.kset[s], &gen[i])) {
        gen_ok[i] = 1;
        Modes si = gen[i];
        std::sort(si.begin(), si.end());
        double best = kInf;
        int arg = -1;
        for (int g = 0; g < i; ++g) {
          if (f[i - 1][g] == kInf || !gen_ok[g]) continue;
          Modes sg = gen[g];
          std::sort(sg.begin(), sg.end());
          if (sg == si) continue;
          const double c = f[i - 1][g] + ds.t_redist(t, gen[g], gen[i]);
          if (c < best) {
            best = c;
            arg = g;
          }
        }
        if (arg >= 0) {
          ds.local_split(s, side, gen[i], &tmp);
          f[i][i] = best + tmp.t_gemm;
          from[i][i] = arg;
        }
      }
    }
    // final state, plus the all-gather of a tensor that a merge consumes
    double best = kInf;
    int gb = -1;
    for (int g = 0; g < n; ++g) {
      if (f[n - 1][g] == kInf) continue;
      double c = f[n - 1][g];
      if (end_merge >= 0) c += ds.t_allgather(L + ch[n - 1], gen[g]);
      if (c < best) {
        best = c;
        gb = g;
      }
    }
    if (gb < 0) {
      *err = "no feasible distribution along the chain starting at step " + std::to_string(s0) +
             " (a split mode is reduced and no other prefix covers P)";
      return TNC_ERR_UNSUPPORTED;
    }
    std::vector<int> use(n);
    use[n - 1] = gb;
    for (int i = n - 1; i > 0; --i) use[i - 1] = from[i][use[i]];
    for (int i = 0; i < n; ++i) {
      const int32_t s = ch[i];
      tnc_dist_step &r = steps[s];
      done[s] = 1;
      const Modes &d = gen[use[i]];
      ds.set_local(&r, d);
      if (i == 0) {
        r.tag = TNC_DIST_ACTIVATE;
        ds.local_activate(s, d, &r);
        ds.set_modes(&r, L + s, d);
        continue;
      }
      const bool gather = !split[L + s];
      r.dist_operand = carry[s];
      ds.local_split(s, carry[s], d, &r);
      if (use[i] == i) {
        r.tag = TNC_DIST_REDISTRIBUTE;
        r.t_comm += ds.t_redist(L + ch[i - 1], gen[use[i - 1]], d);
      } else {
        r.tag = gather ? TNC_DIST_GATHER : TNC_DIST_KEEP;
      }
      if (gather) {
        r.t_comm += ds.t_gather_after(s, d);
        r.num_dist = 0;
      } else {
        ds.set_modes(&r, L + s, d);
      }
    }
    if (end_merge >= 0) {
      steps[end_merge].t_comm += ds.t_allgather(L + ch[n - 1], gen[gb]);
      steps[end_merge].gathered_operand = gathered[end_merge];
    }
  }
  double tot = 0;
  for (int32_t s = 0; s < S; ++s) {
    if (!done[s]) ds.replicated(s, &steps[s]);
    tot += steps[s].t_gemm + steps[s].t_comm;
  }
  *total = tot;
  return TNC_OK;
}

}  // namespace tnc
