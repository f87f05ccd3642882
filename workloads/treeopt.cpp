// Contraction-tree and slice search for tensor networks (host only).
//
// The source page ("Parallelizing Large-Scale Tensor Network Contraction on
// Multiple GPUs", sections 1.1 and 2.3) takes its trees and slicing from an
// external hyper-optimising path finder that is not available here.  This
// file is an in-house stand-in built from published, general techniques,
// written from their definitions:
//
//  * recursive bisection of the leaf set: each set of leaves is split in two
//    with a small cut (modes joining the halves, weighted by log2 extent)
//    under a random balance bound, by a multilevel graph partitioner -
//    coarsening by heavy-edge matching, greedy growing of an initial part,
//    Fiduccia-Mattheyses refinement while uncoarsening;
//  * subtree reconfiguration: the subtree below a node is cut at a frontier
//    of up to k tensors, which are re-contracted by an exact dynamic program
//    over subsets (3^k splits) whenever that lowers the operation count;
//  * slicing interleaved with reconfiguration: modes are fixed one at a time,
//    each time the one in the widest intermediates that carries the most
//    operations, and the tree is re-optimised with the sliced extents, until
//    the widest sliced intermediate fits the bound.
//
// Cost model (section 1.1 of the page): a step with operand mode sets A, B
// costs m n k = 2^(log2 size of A | B) multiply-adds; a tree costs the sum
// over its steps; with s sliced modes of extent 2 every step runs 2^s times
// on the sliced extents.  Width = log2 entries of the largest intermediate.
#include <algorithm>
#include <atomic>
#include <chrono>
#include <cmath>
#include <cstdint>
#include <cstring>
#include <functional>
#include <limits>
#include <mutex>
#include <random>
#include <thread>
#include <vector>

namespace {

using u64 = uint64_t;
const double kInf = std::numeric_limits<double>::infinity();

struct Params {
  int32_t trials;          // trees to build (each fully optimised)
  int32_t threads;         // worker threads (>= 1)
  uint64_t seed;
  double max_log_width;    // bound on the sliced width (log2 entries)
  int32_t reconf_k;        // frontier size of subtree reconfiguration (2..12)
  int32_t reconf_rounds;   // reconfiguration sweeps per optimisation
  double imb_min, imb_max; // range of the balance bound of a bisection (0..1)
  int32_t cutoff_min, cutoff_max;  // leaf sets up to this size are solved exactly (<= 12)
  double time_limit_s;     // stop starting new trials after this many seconds (0: none)
  int32_t max_sliced;      // most modes to slice
  double max_log_peak;     // bound on log2 entries live at once in the emitted order
  double ridge;            // > 0: a step costs max(m n k, ridge (m k + n k + m n)) (roofline time in
                           // multiply-add units at `ridge` multiply-adds per entry moved)
  double score_ridge;      // the same for ranking finished trials only (0: rank by the search cost)
};

// ---------------------------------------------------------------------------
// bitsets of NW 64-bit words

template <int NW>
struct BS {
  u64 w[NW];
  void clear() { std::memset(w, 0, sizeof(w)); }
  void set(int i) { w[i >> 6] |= u64(1) << (i & 63); }
  bool test(int i) const { return (w[i >> 6] >> (i & 63)) & 1; }
};

template <int NW>
inline BS<NW> bor(const BS<NW> &a, const BS<NW> &b) {
  BS<NW> r;
  for (int i = 0; i < NW; ++i) r.w[i] = a.w[i] | b.w[i];
  return r;
}
template <int NW>
inline BS<NW> bxor(const BS<NW> &a, const BS<NW> &b) {
  BS<NW> r;
  for (int i = 0; i < NW; ++i) r.w[i] = a.w[i] ^ b.w[i];
  return r;
}
template <int NW>
inline bool bintersects(const BS<NW> &a, const BS<NW> &b) {
  for (int i = 0; i < NW; ++i)
    if (a.w[i] & b.w[i]) return true;
  return false;
}

// log2 size of a mode set: modes are grouped by log2 extent; sliced modes
// and modes of extent 1 weigh nothing.
template <int NW>
struct Sizer {
  std::vector<double> cw;          // weight of class c
  std::vector<BS<NW>> cmask;       // modes of class c that are not sliced
  double operator()(const BS<NW> &b) const {
    double s = 0;
    for (size_t c = 0; c < cw.size(); ++c) {
      int n = 0;
      for (int i = 0; i < NW; ++i) n += __builtin_popcountll(b.w[i] & cmask[c].w[i]);
      s += cw[c] * n;
    }
    return s;
  }
};

struct NetDesc {
  int L = 0, M = 0;
  std::vector<double> logw;             // per mode
  std::vector<std::vector<int>> leaf;   // modes per leaf
  // leaf graph: for each leaf, (neighbour leaf, weight) over closed modes
  std::vector<std::vector<std::pair<int, double>>> adj;
};

// ---------------------------------------------------------------------------
// multilevel bisection

struct Graph {
  int n = 0;
  std::vector<double> vw;                                  // vertex weight
  std::vector<std::vector<std::pair<int, double>>> adj;    // merged edges
};

double cut_of(const Graph &g, const std::vector<char> &side) {
  double c = 0;
  for (int v = 0; v < g.n; ++v)
    for (auto &e : g.adj[v])
      if (e.first > v && side[v] != side[e.first]) c += e.second;
  return c;
}

// Fiduccia-Mattheyses passes: move the unlocked vertex of largest gain whose
// move keeps side-0 weight within [lo, hi]; keep the best prefix of moves.
void fm_refine(const Graph &g, std::vector<char> &side, double lo, double hi, std::mt19937_64 &rng,
               int passes) {
  const int n = g.n;
  std::vector<double> gain(n);
  std::vector<char> locked(n);
  std::vector<int> moves;
  std::uniform_real_distribution<double> U(0.0, 1e-9);
  std::vector<double> jitter(n);
  for (int pass = 0; pass < passes; ++pass) {
    double w0 = 0;
    for (int v = 0; v < n; ++v)
      if (!side[v]) w0 += g.vw[v];
    for (int v = 0; v < n; ++v) {
      double gv = 0;
      for (auto &e : g.adj[v]) gv += side[e.first] != side[v] ? e.second : -e.second;
      gain[v] = gv;
      jitter[v] = U(rng);
    }
    std::fill(locked.begin(), locked.end(), 0);
    moves.clear();
    double cur = 0, best = 0;
    size_t best_k = 0;
    for (int step = 0; step < n; ++step) {
      int pick = -1;
      double pg = -kInf;
      for (int v = 0; v < n; ++v) {
        if (locked[v]) continue;
        double nw0 = side[v] ? w0 + g.vw[v] : w0 - g.vw[v];
        if (nw0 < lo - 1e-9 || nw0 > hi + 1e-9) continue;
        double gv = gain[v] + jitter[v];
        if (gv > pg) {
          pg = gv;
          pick = v;
        }
      }
      if (pick < 0) break;
      const int v = pick;
      cur -= gain[v];
      w0 = side[v] ? w0 + g.vw[v] : w0 - g.vw[v];
      side[v] = !side[v];
      locked[v] = 1;
      for (auto &e : g.adj[v]) gain[e.first] += side[e.first] == side[v] ? -2 * e.second : 2 * e.second;
      gain[v] = -gain[v];
      moves.push_back(v);
      if (cur < best - 1e-12) {
        best = cur;
        best_k = moves.size();
      }
    }
    for (size_t i = best_k; i < moves.size(); ++i) side[moves[i]] = !side[moves[i]];
    if (best_k == 0) break;
  }
}

// Grow side 0 from a random seed vertex, always adding the frontier vertex
// with the largest gain, until its weight reaches `target`.
void grow(const Graph &g, std::vector<char> &side, double target, std::mt19937_64 &rng) {
  const int n = g.n;
  std::fill(side.begin(), side.end(), 1);
  std::vector<double> conn(n, 0.0), deg(n, 0.0);
  for (int v = 0; v < n; ++v)
    for (auto &e : g.adj[v]) deg[v] += e.second;
  std::uniform_int_distribution<int> pickv(0, n - 1);
  std::uniform_real_distribution<double> U(0.0, 1e-9);
  double w0 = 0;
  int v = pickv(rng);
  while (true) {
    side[v] = 0;
    w0 += g.vw[v];
    if (w0 >= target) break;
    for (auto &e : g.adj[v]) conn[e.first] += e.second;
    int best = -1;
    double bg = -kInf;
    for (int u = 0; u < n; ++u) {
      if (!side[u]) continue;
      double gu = 2 * conn[u] - deg[u] + U(rng);
      if (conn[u] <= 0) gu -= 1e6;  // prefer connected growth
      if (gu > bg) {
        bg = gu;
        best = u;
      }
    }
    if (best < 0) break;
    v = best;
  }
}

// Heavy-edge matching; returns the coarse graph and the fine -> coarse map.
Graph coarsen(const Graph &g, std::vector<int> &cmap, std::mt19937_64 &rng) {
  const int n = g.n;
  std::vector<int> order(n);
  for (int i = 0; i < n; ++i) order[i] = i;
  std::shuffle(order.begin(), order.end(), rng);
  std::vector<int> match(n, -1);
  for (int v : order) {
    if (match[v] >= 0) continue;
    int best = -1;
    double bw = 0;
    for (auto &e : g.adj[v]) {
      int u = e.first;
      if (u == v || match[u] >= 0) continue;
      // heavy edge, scaled down for heavy vertices to keep coarse weights even
      double s = e.second / (g.vw[u] + g.vw[v]);
      if (s > bw) {
        bw = s;
        best = u;
      }
    }
    if (best >= 0) {
      match[v] = best;
      match[best] = v;
    } else {
      match[v] = v;
    }
  }
  cmap.assign(n, -1);
  int nc = 0;
  for (int v = 0; v < n; ++v) {
    if (cmap[v] >= 0) continue;
    cmap[v] = nc;
    if (match[v] != v) cmap[match[v]] = nc;
    ++nc;
  }
  Graph c;
  c.n = nc;
  c.vw.assign(nc, 0.0);
  c.adj.assign(nc, {});
  for (int v = 0; v < n; ++v) c.vw[cmap[v]] += g.vw[v];
  std::vector<double> acc(nc, 0.0);
  std::vector<int> touched;
  std::vector<std::vector<int>> members(nc);
  for (int v = 0; v < n; ++v) members[cmap[v]].push_back(v);
  for (int cv = 0; cv < nc; ++cv) {
    touched.clear();
    for (int v : members[cv])
      for (auto &e : g.adj[v]) {
        int cu = cmap[e.first];
        if (cu == cv) continue;
        if (acc[cu] == 0.0) touched.push_back(cu);
        acc[cu] += e.second;
      }
    for (int cu : touched) {
      c.adj[cv].push_back({cu, acc[cu]});
      acc[cu] = 0.0;
    }
  }
  return c;
}

// Split graph g in two: side[v] = 0 or 1, side-0 weight within [lo, hi].
void multilevel_bisect(const Graph &g, double lo, double hi, std::mt19937_64 &rng, std::vector<char> &side) {
  std::vector<Graph> levels{g};
  std::vector<std::vector<int>> maps;
  while (levels.back().n > 48) {
    std::vector<int> cmap;
    Graph c = coarsen(levels.back(), cmap, rng);
    if (c.n > 0.92 * levels.back().n) break;
    maps.push_back(std::move(cmap));
    levels.push_back(std::move(c));
  }
  const Graph &cg = levels.back();
  std::vector<char> best_side, s(cg.n);
  double best_cut = kInf;
  std::uniform_real_distribution<double> U01(0.0, 1.0);
  for (int t = 0; t < 8; ++t) {
    double target = lo + (hi - lo) * U01(rng);
    grow(cg, s, target, rng);
    fm_refine(cg, s, lo, hi, rng, 8);
    double w0 = 0;
    for (int v = 0; v < cg.n; ++v)
      if (!s[v]) w0 += cg.vw[v];
    if (w0 < lo - 1e-9 || w0 > hi + 1e-9) continue;
    double c = cut_of(cg, s);
    if (c < best_cut) {
      best_cut = c;
      best_side = s;
    }
  }
  if (best_side.empty()) {  // no balanced grown part: fall back to an ordered split
    best_side.assign(cg.n, 1);
    double w0 = 0;
    for (int v = 0; v < cg.n && w0 < lo; ++v) {
      best_side[v] = 0;
      w0 += cg.vw[v];
    }
  }
  side = best_side;
  for (int lv = (int)maps.size() - 1; lv >= 0; --lv) {
    const Graph &fine = levels[lv];
    std::vector<char> fs(fine.n);
    for (int v = 0; v < fine.n; ++v) fs[v] = side[maps[lv][v]];
    fm_refine(fine, fs, lo, hi, rng, 6);
    side.swap(fs);
  }
}

// ---------------------------------------------------------------------------
// trees

template <int NW>
struct TreeT {
  int L = 0;
  std::vector<int> left, right, parent;   // 2L - 1 nodes; leaves are 0 .. L-1
  std::vector<BS<NW>> legs;
  int root = -1;
  int next = 0;

  void init(int nleaves, const std::vector<BS<NW>> &leaf_legs) {
    L = nleaves;
    left.assign(2 * L - 1, -1);
    right.assign(2 * L - 1, -1);
    parent.assign(2 * L - 1, -1);
    legs.resize(2 * L - 1);
    for (int i = 0; i < L; ++i) legs[i] = leaf_legs[i];
    next = L;
    root = L == 1 ? 0 : -1;
  }
  int join(int a, int b) {
    int n = next++;
    left[n] = a;
    right[n] = b;
    parent[a] = n;
    parent[b] = n;
    legs[n] = bxor(legs[a], legs[b]);
    root = n;
    return n;
  }
};

// Optimal contraction of k <= 16 tensors by dynamic programming over
// subsets: best[T] = min over splits T = A + B of best[A] + best[B] +
// 2^(size(legs A | legs B)); intermediates (not the whole set) wider than
// max_w are not allowed.  Returns the cost (kInf if none) and fills split[].
// Cost of one step with operand sizes 2^a, 2^b, result 2^c and 2^u = m n k.
inline double step_cost(double u, double a, double b, double c, double ridge) {
  double f = std::exp2(u);
  if (ridge > 0) f = std::max(f, ridge * (std::exp2(a) + std::exp2(b) + std::exp2(c)));
  return f;
}

template <int NW>
double dp_contract(const std::vector<BS<NW>> &items, const Sizer<NW> &sz, double max_w, double ridge,
                   std::vector<uint32_t> &split, std::vector<BS<NW>> &legs, std::vector<double> &best) {
  const int k = (int)items.size();
  const uint32_t full = (1u << k) - 1;
  legs.assign(size_t(1) << k, BS<NW>{});
  best.assign(size_t(1) << k, kInf);
  split.assign(size_t(1) << k, 0);
  std::vector<double> wsz(size_t(1) << k, 0.0);
  for (uint32_t T = 1; T <= full; ++T) {
    int low = __builtin_ctz(T);
    uint32_t rest = T & (T - 1);
    if (rest == 0) {
      legs[T] = items[low];
      best[T] = 0.0;
    } else {
      legs[T] = bxor(legs[rest], items[low]);
    }
    wsz[T] = sz(legs[T]);
  }
  for (uint32_t T = 1; T <= full; ++T) {
    if ((T & (T - 1)) == 0) continue;
    if (T != full && wsz[T] > max_w + 1e-9) continue;
    const uint32_t lowbit = T & (~T + 1);
    double bc = kInf;
    uint32_t bs = 0;
    // sub runs over proper subsets holding T's lowest element
    for (uint32_t sub = (T - 1) & T; sub; sub = (sub - 1) & T) {
      if (!(sub & lowbit)) continue;
      uint32_t oth = T ^ sub;
      double c = best[sub] + best[oth];
      if (!(c < bc)) continue;
      c += step_cost(sz(bor(legs[sub], legs[oth])), wsz[sub], wsz[oth], wsz[T], ridge);
      if (c < bc) {
        bc = c;
        bs = sub;
      }
    }
    best[T] = bc;
    split[T] = bs;
  }
  return best[full];
}

template <int NW>
class Optimizer {
 public:
  Optimizer(const NetDesc &net, const Params &p) : net_(net), p_(p) {
    leaf_legs_.resize(net.L);
    for (int l = 0; l < net.L; ++l) {
      leaf_legs_[l].clear();
      for (int x : net.leaf[l]) leaf_legs_[l].set(x);
    }
    // weight classes
    std::vector<double> ws;
    for (double w : net.logw)
      if (w > 0 && std::find(ws.begin(), ws.end(), w) == ws.end()) ws.push_back(w);
    base_.cw = ws;
    base_.cmask.assign(ws.size(), BS<NW>{});
    for (auto &m : base_.cmask) m.clear();
    for (int x = 0; x < net.M; ++x)
      for (size_t c = 0; c < ws.size(); ++c)
        if (net.logw[x] == ws[c]) base_.cmask[c].set(x);
  }

  struct Result {
    std::vector<int> lhs, rhs, sliced;
    double log2_cost = kInf;   // log2 of 2^s * sum of m n k
    double width = 0;          // sliced width (log2 entries)
    double peak_log2 = 0;      // log2 entries of the peak live intermediates in the emitted order
    int trial = -1;
  };

  Result run() {
    Result best;
    std::mutex mu;
    std::atomic<int> next{0};
    const auto t0 = std::chrono::steady_clock::now();
    auto worker = [&]() {
      for (;;) {
        int t = next.fetch_add(1);
        if (t >= p_.trials) return;
        if (p_.time_limit_s > 0 && t > 0) {
          double el = std::chrono::duration<double>(std::chrono::steady_clock::now() - t0).count();
          if (el > p_.time_limit_s) return;
        }
        Result r = trial(t);
        std::lock_guard<std::mutex> lk(mu);
        if (r.log2_cost < best.log2_cost - 1e-12 ||
            (std::fabs(r.log2_cost - best.log2_cost) <= 1e-12 && r.trial < best.trial))
          best = r;
      }
    };
    int nt = std::max(1, p_.threads);
    std::vector<std::thread> pool;
    for (int i = 0; i < nt; ++i) pool.emplace_back(worker);
    for (auto &th : pool) th.join();
    return best;
  }

  // One trial: a bisection tree with random balance and leaf-set size,
  // reconfigured, then sliced down to the width bound with reconfiguration
  // after every sliced mode.
  Result trial(int t) {
    std::mt19937_64 rng(p_.seed * 0x9E3779B97F4A7C15ull + (u64)t * 0xD1B54A32D192ED03ull + 1);
    std::uniform_real_distribution<double> U01(0.0, 1.0);
    const double imb = p_.imb_min + (p_.imb_max - p_.imb_min) * U01(rng);
    std::uniform_int_distribution<int> cut_d(p_.cutoff_min, p_.cutoff_max);
    const int cutoff = cut_d(rng);
    TreeT<NW> tr;
    tr.init(net_.L, leaf_legs_);
    Sizer<NW> sz = base_;
    std::vector<int> all(net_.L);
    for (int i = 0; i < net_.L; ++i) all[i] = i;
    if (net_.L > 1) build(tr, all, imb, cutoff, sz, rng);
    BS<NW> sliced;
    sliced.clear();
    std::vector<int> sl;
    reconfigure(tr, sz, kInf, rng);
    while ((width(tr, sz) > p_.max_log_width + 1e-9 || peak(tr, sz) > p_.max_log_peak + 1e-9) &&
           (int)sl.size() < p_.max_sliced) {
      int x = pick_slice(tr, sz, sliced);
      if (x < 0) break;
      sliced.set(x);
      sl.push_back(x);
      for (auto &m : sz.cmask) m.w[x >> 6] &= ~(u64(1) << (x & 63));
      reconfigure(tr, sz, kInf, rng);
    }
    // a last pass that may not widen past the bound
    reconfigure(tr, sz, std::max(p_.max_log_width, width(tr, sz)), rng);
    Result r;
    r.trial = t;
    r.sliced = sl;
    r.width = width(tr, sz);
    double ns = 0;
    for (int x : sl) ns += net_.logw[x];
    r.log2_cost = std::log2(score_total(tr, sz)) + ns;
    emit(tr, sz, r);
    if (r.width > p_.max_log_width + 1e-9 || r.peak_log2 > p_.max_log_peak + 1e-9)
      r.log2_cost += 1000.0;  // bound not met
    return r;
  }

  // Load a given tree (SSA steps) with given sliced modes, reconfigure it
  // with the configured frontier size, slice further while a bound is
  // exceeded, and emit it again.
  Result refine(const int32_t *lhs, const int32_t *rhs, const std::vector<int> &sliced_in) {
    std::mt19937_64 rng(p_.seed * 0x9E3779B97F4A7C15ull + 7);
    TreeT<NW> tr;
    tr.init(net_.L, leaf_legs_);
    for (int s = 0; s + 1 < net_.L; ++s) tr.join(lhs[s], rhs[s]);
    Sizer<NW> sz = base_;
    BS<NW> sliced;
    sliced.clear();
    std::vector<int> sl = sliced_in;
    for (int x : sl) {
      sliced.set(x);
      for (auto &m : sz.cmask) m.w[x >> 6] &= ~(u64(1) << (x & 63));
    }
    reconfigure(tr, sz, std::max(p_.max_log_width, width(tr, sz)), rng);
    while ((width(tr, sz) > p_.max_log_width + 1e-9 || peak(tr, sz) > p_.max_log_peak + 1e-9) &&
           (int)sl.size() < p_.max_sliced) {
      int x = pick_slice(tr, sz, sliced);
      if (x < 0) break;
      sliced.set(x);
      sl.push_back(x);
      for (auto &m : sz.cmask) m.w[x >> 6] &= ~(u64(1) << (x & 63));
      reconfigure(tr, sz, std::max(p_.max_log_width, width(tr, sz)), rng);
    }
    Result r;
    r.trial = 0;
    r.sliced = sl;
    r.width = width(tr, sz);
    double ns = 0;
    for (int x : sl) ns += net_.logw[x];
    r.log2_cost = std::log2(score_total(tr, sz)) + ns;
    emit(tr, sz, r);
    return r;
  }

 private:
  const NetDesc &net_;
  const Params &p_;
  std::vector<BS<NW>> leaf_legs_;
  Sizer<NW> base_;

  double width(const TreeT<NW> &tr, const Sizer<NW> &sz) const {
    double w = 0;
    for (int n = 0; n < tr.next; ++n) w = std::max(w, sz(tr.legs[n]));
    return w;
  }
  double node_cost(const TreeT<NW> &tr, int n, const Sizer<NW> &sz) const {
    const BS<NW> &a = tr.legs[tr.left[n]], &b = tr.legs[tr.right[n]];
    return step_cost(sz(bor(a, b)), sz(a), sz(b), sz(tr.legs[n]), p_.ridge);
  }
  // the ranking cost of a finished tree (roofline units with score_ridge)
  double score_total(const TreeT<NW> &tr, const Sizer<NW> &sz) const {
    if (!(p_.score_ridge > 0)) return total(tr, sz);
    double s = 0;
    for (int n = tr.L; n < tr.next; ++n) {
      const BS<NW> &a = tr.legs[tr.left[n]], &b = tr.legs[tr.right[n]];
      s += step_cost(sz(bor(a, b)), sz(a), sz(b), sz(tr.legs[n]), p_.score_ridge);
    }
    return s;
  }
  double total(const TreeT<NW> &tr, const Sizer<NW> &sz) const {
    double s = 0;
    for (int n = tr.L; n < tr.next; ++n) s += node_cost(tr, n, sz);
    return s;
  }

  // contract a small set exactly (dynamic program), returns the subtree root
  int solve_small(TreeT<NW> &tr, const std::vector<int> &ids, const Sizer<NW> &sz) {
    std::vector<BS<NW>> items;
    for (int i : ids) items.push_back(tr.legs[i]);
    std::vector<uint32_t> split;
    std::vector<BS<NW>> legs;
    std::vector<double> best;
    dp_contract(items, sz, kInf, p_.ridge, split, legs, best);
    std::vector<int> node_of(size_t(1) << ids.size(), -1);
    for (size_t i = 0; i < ids.size(); ++i) node_of[size_t(1) << i] = ids[i];
    return emit_dp(tr, (1u << ids.size()) - 1, split, node_of);
  }
  int emit_dp(TreeT<NW> &tr, uint32_t T, const std::vector<uint32_t> &split, std::vector<int> &node_of) {
    if (node_of[T] >= 0) return node_of[T];
    uint32_t a = split[T], b = T ^ split[T];
    int na = emit_dp(tr, a, split, node_of);
    int nb = emit_dp(tr, b, split, node_of);
    return node_of[T] = tr.join(na, nb);
  }

  int build(TreeT<NW> &tr, const std::vector<int> &ids, double imb, int cutoff, const Sizer<NW> &sz,
            std::mt19937_64 &rng) {
    if (ids.size() == 1) return ids[0];
    if ((int)ids.size() <= cutoff) return solve_small(tr, ids, sz);
    // subgraph on ids
    Graph g;
    g.n = (int)ids.size();
    g.vw.assign(g.n, 1.0);
    g.adj.assign(g.n, {});
    std::vector<int> local(net_.L, -1);
    for (int i = 0; i < g.n; ++i) local[ids[i]] = i;
    for (int i = 0; i < g.n; ++i)
      for (auto &e : net_.adj[ids[i]])
        if (local[e.first] >= 0) g.adj[i].push_back({local[e.first], e.second});
    const double W = g.n;
    double lo = std::max(1.0, std::floor(W * (1.0 - imb) / 2.0));
    double hi = std::min(W - 1.0, std::ceil(W * (1.0 + imb) / 2.0));
    std::vector<char> side;
    multilevel_bisect(g, lo, hi, rng, side);
    std::vector<int> a, b;
    for (int i = 0; i < g.n; ++i) (side[i] ? b : a).push_back(ids[i]);
    if (a.empty() || b.empty()) {  // degenerate: split in half
      a.assign(ids.begin(), ids.begin() + ids.size() / 2);
      b.assign(ids.begin() + ids.size() / 2, ids.end());
    }
    int na = build(tr, a, imb, cutoff, sz, rng);
    int nb = build(tr, b, imb, cutoff, sz, rng);
    return tr.join(na, nb);
  }

  // Reconfigure every internal node's subtree (frontier of up to k
  // tensors, grown by repeatedly opening the widest internal frontier node),
  // for the configured number of sweeps or until nothing improves.
  void reconfigure(TreeT<NW> &tr, const Sizer<NW> &sz, double max_w, std::mt19937_64 &rng) {
    const int k = std::max(2, std::min(12, p_.reconf_k));
    std::vector<uint32_t> split;
    std::vector<BS<NW>> dlegs;
    std::vector<double> dbest;
    for (int round = 0; round < p_.reconf_rounds; ++round) {
      bool improved = false;
      std::vector<int> order;
      for (int n = tr.L; n < tr.next; ++n) order.push_back(n);
      std::shuffle(order.begin(), order.end(), rng);
      for (int n : order) {
        std::vector<int> front{tr.left[n], tr.right[n]};
        std::vector<int> inner{n};
        while ((int)front.size() < k) {
          int bi = -1;
          double bw = -1;
          for (size_t i = 0; i < front.size(); ++i) {
            int f = front[i];
            if (f < tr.L) continue;
            double w = sz(tr.legs[f]);
            if (w > bw) {
              bw = w;
              bi = (int)i;
            }
          }
          if (bi < 0) break;
          int f = front[bi];
          front[bi] = tr.left[f];
          front.push_back(tr.right[f]);
          inner.push_back(f);
        }
        if (front.size() < 3) continue;
        double cur = 0;
        for (int i : inner) cur += node_cost(tr, i, sz);
        std::vector<BS<NW>> items;
        for (int f : front) items.push_back(tr.legs[f]);
        double c = dp_contract(items, sz, max_w, p_.ridge, split, dlegs, dbest);
        if (!(c < cur * (1.0 - 1e-9))) continue;
        // rebuild: reuse the inner node ids, the top one (n) stays the root of the subtree
        std::vector<int> free_ids(inner.begin() + 1, inner.end());
        const int par = tr.parent[n];
        std::vector<int> node_of(size_t(1) << front.size(), -1);
        for (size_t i = 0; i < front.size(); ++i) node_of[size_t(1) << i] = front[i];
        const uint32_t full = (1u << front.size()) - 1;
        size_t fi = 0;
        std::function<int(uint32_t)> rec = [&](uint32_t T) -> int {
          if (node_of[T] >= 0) return node_of[T];
          int na = rec(split[T]);
          int nb = rec(T ^ split[T]);
          int id = (T == full) ? n : free_ids[fi++];
          tr.left[id] = na;
          tr.right[id] = nb;
          tr.parent[na] = id;
          tr.parent[nb] = id;
          tr.legs[id] = bxor(tr.legs[na], tr.legs[nb]);
          return node_of[T] = id;
        };
        rec(full);
        tr.parent[n] = par;
        improved = true;
      }
      if (!improved) break;
    }
  }

  // The mode to slice next: among modes of the widest intermediates, the
  // one held by most of them, then the one whose steps carry the most
  // operations (slicing it removes the largest share of the work).
  int pick_slice(const TreeT<NW> &tr, const Sizer<NW> &sz, const BS<NW> &sliced) const {
    double w = width(tr, sz);
    std::vector<double> contrib(net_.M, 0.0);
    std::vector<int> hits(net_.M, 0);
    for (int n = tr.L; n < tr.next; ++n) {
      BS<NW> u = bor(tr.legs[tr.left[n]], tr.legs[tr.right[n]]);
      double c = std::exp2(sz(u));
      for (int i = 0; i < NW; ++i)
        for (u64 b = u.w[i]; b; b &= b - 1) contrib[i * 64 + __builtin_ctzll(b)] += c;
    }
    for (int n = 0; n < tr.next; ++n) {
      if (sz(tr.legs[n]) < w - 1e-9) continue;
      for (int i = 0; i < NW; ++i)
        for (u64 b = tr.legs[n].w[i]; b; b &= b - 1) hits[i * 64 + __builtin_ctzll(b)]++;
    }
    int best = -1;
    for (int x = 0; x < net_.M; ++x) {
      if (sliced.test(x) || net_.logw[x] <= 0 || hits[x] == 0) continue;
      if (best < 0 || hits[x] > hits[best] || (hits[x] == hits[best] && contrib[x] > contrib[best])) best = x;
    }
    return best;
  }

  double peak(const TreeT<NW> &tr, const Sizer<NW> &sz) {
    Result tmp;
    emit(tr, sz, tmp);
    return tmp.peak_log2;
  }

  // Steps in execution order: depth first, at every node the child whose
  // subtree needs more live memory first (its result then waits while the
  // smaller subtree runs).
  void emit(const TreeT<NW> &tr, const Sizer<NW> &sz, Result &r) {
    const int N = tr.next;
    std::vector<double> peak(N, 0.0), size(N, 0.0);
    std::vector<char> first_left(N, 1);
    // post-order over the tree
    std::vector<int> post;
    {
      std::vector<std::pair<int, int>> st{{tr.root, 0}};
      while (!st.empty()) {
        auto &top = st.back();
        int n = top.first;
        if (n < tr.L || top.second == 2) {
          post.push_back(n);
          st.pop_back();
          continue;
        }
        int c = top.second == 0 ? tr.left[n] : tr.right[n];
        top.second++;
        st.push_back({c, 0});
      }
    }
    for (int n : post) {
      size[n] = n < tr.L ? 0.0 : std::exp2(sz(tr.legs[n]));
      if (n < tr.L) continue;
      int a = tr.left[n], b = tr.right[n];
      double pab = std::max({peak[a], size[a] + peak[b], size[a] + size[b] + size[n]});
      double pba = std::max({peak[b], size[b] + peak[a], size[a] + size[b] + size[n]});
      first_left[n] = pab <= pba;
      peak[n] = std::min(pab, pba);
    }
    r.peak_log2 = tr.root >= 0 && peak[tr.root] > 0 ? std::log2(peak[tr.root]) : 0.0;
    std::vector<int> ssa(N, -1);
    for (int l = 0; l < tr.L; ++l) ssa[l] = l;
    int nxt = tr.L;
    r.lhs.clear();
    r.rhs.clear();
    std::vector<std::pair<int, int>> st;
    if (tr.root >= tr.L) st.push_back({tr.root, 0});
    while (!st.empty()) {
      auto &top = st.back();
      int n = top.first;
      if (n < tr.L) {
        st.pop_back();
        continue;
      }
      int a = first_left[n] ? tr.left[n] : tr.right[n];
      int b = first_left[n] ? tr.right[n] : tr.left[n];
      if (top.second == 0) {
        top.second = 1;
        st.push_back({a, 0});
      } else if (top.second == 1) {
        top.second = 2;
        st.push_back({b, 0});
      } else {
        r.lhs.push_back(ssa[a]);
        r.rhs.push_back(ssa[b]);
        ssa[n] = nxt++;
        st.pop_back();
      }
    }
  }
};

template <int NW>
int run_nw(const NetDesc &net, const Params &p, int32_t *lhs, int32_t *rhs, int32_t *sliced, int32_t *nsliced,
           double *stats, bool refine) {
  Optimizer<NW> opt(net, p);
  typename Optimizer<NW>::Result r;
  if (refine) r = opt.refine(lhs, rhs, std::vector<int>(sliced, sliced + *nsliced));
  else r = opt.run();
  if (r.trial < 0) return 3;
  for (size_t i = 0; i < r.lhs.size(); ++i) {
    lhs[i] = r.lhs[i];
    rhs[i] = r.rhs[i];
  }
  *nsliced = (int32_t)r.sliced.size();
  for (size_t i = 0; i < r.sliced.size(); ++i) sliced[i] = r.sliced[i];
  stats[0] = r.log2_cost;
  stats[1] = r.width;
  stats[2] = r.peak_log2;
  stats[3] = r.trial;
  return 0;
}

}  // namespace

namespace {

int search_impl(int32_t L, int32_t M, const double *logw, const int32_t *leaf_rank, const int32_t *leaf_modes,
                const double *params, int32_t *lhs, int32_t *rhs, int32_t *sliced, int32_t *nsliced, double *stats,
                bool refine);

}  // namespace

extern "C" {

// Search a tree (and sliced modes) for a network of L leaves over M modes.
// logw[M]: log2 extent of each mode; leaf_rank[L] and the concatenated
// leaf_modes give each leaf's modes.  params (doubles, in order): trials,
// threads, seed, max_log_width, reconf_k, reconf_rounds, imb_min, imb_max,
// cutoff_min, cutoff_max, time_limit_s, max_sliced, max_log_peak, ridge,
// score_ridge.
// Outputs: lhs/rhs[L-1] (SSA steps in execution order), sliced[max_sliced]
// and *nsliced, stats[4] = {log2 of 2^s * sum m n k, sliced width, log2 peak
// live entries, winning trial}; the cost is in roofline units when
// score_ridge > 0.  Returns 0, or 1 (bad arguments), 2 (more
// than 2048 modes), 3 (no trial ran).
int treeopt_search(int32_t L, int32_t M, const double *logw, const int32_t *leaf_rank,
                   const int32_t *leaf_modes, const double *params, int32_t *lhs, int32_t *rhs, int32_t *sliced,
                   int32_t *nsliced, double *stats) {
  return search_impl(L, M, logw, leaf_rank, leaf_modes, params, lhs, rhs, sliced, nsliced, stats, false);
}

// Same arguments; lhs/rhs/sliced/nsliced hold a tree and its sliced modes on
// entry, which are reconfigured (params: trials and threads unused) and
// returned in the same form.
int treeopt_refine(int32_t L, int32_t M, const double *logw, const int32_t *leaf_rank,
                   const int32_t *leaf_modes, const double *params, int32_t *lhs, int32_t *rhs, int32_t *sliced,
                   int32_t *nsliced, double *stats) {
  return search_impl(L, M, logw, leaf_rank, leaf_modes, params, lhs, rhs, sliced, nsliced, stats, true);
}

}  // extern "C"

namespace {

int search_impl(int32_t L, int32_t M, const double *logw, const int32_t *leaf_rank, const int32_t *leaf_modes,
                const double *params, int32_t *lhs, int32_t *rhs, int32_t *sliced, int32_t *nsliced, double *stats,
                bool refine) {
  if (L < 1 || M < 0 || !logw || !leaf_rank || !params || !lhs || !rhs || !sliced || !nsliced || !stats) return 1;
  NetDesc net;
  net.L = L;
  net.M = M;
  net.logw.assign(logw, logw + M);
  net.leaf.resize(L);
  std::vector<std::vector<int>> holders(M);
  int64_t pos = 0;
  for (int l = 0; l < L; ++l) {
    for (int r = 0; r < leaf_rank[l]; ++r) {
      int x = leaf_modes[pos++];
      if (x < 0 || x >= M) return 1;
      net.leaf[l].push_back(x);
      holders[x].push_back(l);
    }
  }
  net.adj.assign(L, {});
  for (int x = 0; x < M; ++x) {
    if (holders[x].size() > 2) return 1;
    if (holders[x].size() == 2 && logw[x] > 0) {
      int a = holders[x][0], b = holders[x][1];
      net.adj[a].push_back({b, logw[x]});
      net.adj[b].push_back({a, logw[x]});
    }
  }
  // merge parallel edges
  for (auto &a : net.adj) {
    std::sort(a.begin(), a.end());
    std::vector<std::pair<int, double>> m;
    for (auto &e : a) {
      if (!m.empty() && m.back().first == e.first) m.back().second += e.second;
      else m.push_back(e);
    }
    a.swap(m);
  }
  Params p;
  p.trials = (int32_t)params[0];
  p.threads = (int32_t)params[1];
  p.seed = (uint64_t)params[2];
  p.max_log_width = params[3];
  p.reconf_k = (int32_t)params[4];
  p.reconf_rounds = (int32_t)params[5];
  p.imb_min = params[6];
  p.imb_max = params[7];
  p.cutoff_min = std::max(1, std::min(12, (int32_t)params[8]));
  p.cutoff_max = std::max(p.cutoff_min, std::min(12, (int32_t)params[9]));
  p.time_limit_s = params[10];
  p.max_sliced = (int32_t)params[11];
  p.max_log_peak = params[12];
  p.ridge = params[13];
  p.score_ridge = params[14];
  if (p.trials < 1) return 1;
  if (refine) {
    for (int s = 0; s + 1 < L; ++s)
      if (lhs[s] < 0 || rhs[s] < 0 || lhs[s] >= L + s || rhs[s] >= L + s || lhs[s] == rhs[s]) return 1;
    for (int i = 0; i < *nsliced; ++i)
      if (sliced[i] < 0 || sliced[i] >= M) return 1;
  }
  const int nw = (M + 63) / 64;
  if (nw <= 2) return run_nw<2>(net, p, lhs, rhs, sliced, nsliced, stats, refine);
  if (nw <= 4) return run_nw<4>(net, p, lhs, rhs, sliced, nsliced, stats, refine);
  if (nw <= 8) return run_nw<8>(net, p, lhs, rhs, sliced, nsliced, stats, refine);
  if (nw <= 16) return run_nw<16>(net, p, lhs, rhs, sliced, nsliced, stats, refine);
  if (nw <= 32) return run_nw<32>(net, p, lhs, rhs, sliced, nsliced, stats, refine);
  return 2;
}

}  // namespace
