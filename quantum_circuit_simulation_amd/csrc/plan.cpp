// Host planner: validation, lifetime ordering, step descriptors, launch
// groups, first-fit arena and the device descriptor blob.
#include "plan.hpp"

#include <algorithm>
#include <array>
#include <cstring>
#include <list>
#include <set>

namespace tnc {
namespace {

uint64_t round_up(uint64_t v, uint64_t a) { return (v + a - 1) / a * a; }

int64_t pow2_floor(int64_t v) {
  int64_t p = 1;
  while (p * 2 <= v) p *= 2;
  return p;
}

int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }

// product of extents of `modes`; returns false on int64 overflow
bool checked_prod(const std::vector<int64_t> &ext, const std::vector<int32_t> &modes, int64_t *out) {
  __int128 p = 1;
  for (int32_t x : modes) {
    p *= ext[x];
    if (p > (__int128)(INT64_MAX / 16)) return false;
  }
  *out = (int64_t)p;
  return true;
}

int64_t prod(const std::vector<int64_t> &ext, const std::vector<int32_t> &modes) {
  int64_t p = 1;
  for (int32_t x : modes) p *= ext[x];
  return p;
}

bool contains(const std::vector<int32_t> &v, int32_t x) { return std::find(v.begin(), v.end(), x) != v.end(); }

// First-fit arena over a sorted free list of holes; the last hole is unbounded.
class Arena {
 public:
  uint64_t alloc(uint64_t size) {
    for (auto it = holes_.begin(); it != holes_.end(); ++it) {
      if (it->second == kNone || it->second - it->first >= size) {
        uint64_t off = it->first;
        it->first += size;
        if (it->second != kNone && it->first == it->second) holes_.erase(it);
        peak_ = std::max(peak_, off + size);
        return off;
      }
    }
    return kNone;  // unreachable: the last hole is unbounded
  }
  void release(uint64_t off, uint64_t size) {
    auto it = holes_.begin();
    while (it != holes_.end() && it->first < off) ++it;
    it = holes_.insert(it, {off, off + size});
    // merge with the next hole
    auto nx = std::next(it);
    if (nx != holes_.end() && it->second == nx->first) {
      it->second = nx->second;
      holes_.erase(nx);
    }
    // merge with the previous hole
    if (it != holes_.begin()) {
      auto pv = std::prev(it);
      if (pv->second == it->first) {
        pv->second = it->second;
        holes_.erase(it);
      }
    }
  }
  uint64_t peak() const { return peak_; }

 private:
  std::list<std::pair<uint64_t, uint64_t>> holes_{{0, kNone}};
  uint64_t peak_ = 0;
};

int32_t split_rule(int32_t cls, int64_t R, int64_t S, int64_t k, bool c64) {
  // enough workgroups to fill the chip; K chunks of >= 64 (GEMM) / 1024 (skinny)
  if (cls == TNC_CLASS_GEMM) {
    // complex64 steps with R S <= 2^19 and K <= 512 run whole in the
    // small-GEMM kernel, which splits K over the waves of each block
    if (c64 && R * S <= (int64_t(1) << 19) && k <= 512) return 1;
    int64_t tiles = ceil_div(R, kGemmNominalTile) * ceil_div(S, kGemmNominalTile);
    if (tiles >= 256 || k < 128) return 1;
    return (int32_t)std::max<int64_t>(1, std::min(pow2_floor(512 / tiles), pow2_floor(k / 64)));
  }
  if (cls == TNC_CLASS_SKINNY) {
    int64_t blocks = ceil_div(R, 256);
    if (blocks >= 512 || k < 2048) return 1;
    return (int32_t)std::max<int64_t>(1, std::min(pow2_floor(1024 / blocks), pow2_floor(k / 1024)));
  }
  return 1;
}

// Output runs of C along `c_order` (extent-1 modes skipped).
void make_runs(const std::vector<int32_t> &c_order, const std::vector<int64_t> &ext,
               const std::vector<int32_t> &row_modes, Node *nd) {
  std::vector<int32_t> eff;
  for (int32_t x : c_order)
    if (ext[x] > 1) eff.push_back(x);
  std::vector<int64_t> stride(eff.size());
  int64_t s = 1;
  for (int p = (int)eff.size() - 1; p >= 0; --p) {
    stride[p] = s;
    s *= ext[eff[p]];
  }
  struct R3 { bool row; int64_t size, stride; };
  std::vector<R3> runs;
  for (size_t p = 0; p < eff.size(); ++p) {
    bool side = contains(row_modes, eff[p]);
    if (!runs.empty() && runs.back().row == side) {
      runs.back().size *= ext[eff[p]];
      runs.back().stride = stride[p];
    } else {
      runs.push_back({side, ext[eff[p]], stride[p]});
    }
  }
  nd->row_runs.clear();
  nd->col_runs.clear();
  for (auto &r : runs) (r.row ? nd->row_runs : nd->col_runs).push_back({r.size, r.stride});
  nd->inner_run = runs.empty() ? 1 : runs.back().size;
  nd->interleaved = runs.size() > 2 ? 1 : 0;
}

// Tile a large copy (see CopyOp).  Leaves c->tiled = 0 when no tile of at
// most kCopyTileMax entries covers both innermost runs.
void make_tile(CopyOp *c) {
  struct Dim { int64_t e, src; };
  std::vector<Dim> d;
  for (size_t q = 0; q < c->dims.size(); ++q) {
    // refine dims above 32 into (e / 32, 32) so a tile can take their inner part
    int64_t e = c->dims[q], st = c->src_strides[q];
    std::vector<Dim> parts;
    while (e > 32 && e % 32 == 0) {
      parts.push_back({32, st});
      st *= 32;
      e /= 32;
    }
    parts.push_back({e, st});
    for (auto it = parts.rbegin(); it != parts.rend(); ++it) d.push_back(*it);
  }
  const int n = (int)d.size();
  if (n < 2) return;
  std::vector<int64_t> dst(n);
  int64_t acc = 1;
  for (int q = n - 1; q >= 0; --q) {
    dst[q] = acc;
    acc *= d[q].e;
  }
  std::vector<char> in(n, 0);
  int64_t tprod = 1;
  for (int q = n - 1; q >= 0 && tprod < 32; --q) {  // innermost destination dims
    in[q] = 1;
    tprod *= d[q].e;
  }
  std::vector<int> by_src(n);
  for (int q = 0; q < n; ++q) by_src[q] = q;
  std::stable_sort(by_src.begin(), by_src.end(), [&](int a, int b) { return d[a].src < d[b].src; });
  int64_t sprod = 1;
  for (int q : by_src) {  // smallest source strides
    if (sprod >= 32) break;
    if (!in[q]) {
      in[q] = 1;
      tprod *= d[q].e;
    }
    sprod *= d[q].e;
  }
  for (int q = n - 1; q >= 0; --q)  // widen the tile along the destination while it fits
    if (!in[q] && tprod * d[q].e <= kCopyTileMax) {
      in[q] = 1;
      tprod *= d[q].e;
    }
  if (tprod > kCopyTileMax || tprod < 32) return;
  std::vector<int> tdst, tsrc, outer;
  for (int q = 0; q < n; ++q) (in[q] ? tdst : outer).push_back(q);
  tsrc = tdst;
  std::stable_sort(tsrc.begin(), tsrc.end(), [&](int a, int b) { return d[a].src < d[b].src; });
  std::vector<int64_t> lds_stride(n, 0);
  acc = 1;
  for (int i = (int)tdst.size() - 1; i >= 0; --i) {
    lds_stride[tdst[i]] = acc;
    acc *= d[tdst[i]].e;
  }
  c->tile = tprod;
  c->ld_src.assign(tprod, 0);
  c->ld_lds.assign(tprod, 0);
  c->st_dst.assign(tprod, 0);
  for (int64_t e = 0; e < tprod; ++e) {
    int64_t r = e, so = 0, lo = 0;
    for (int q : tsrc) {  // fastest = smallest source stride
      int64_t dg = r % d[q].e;
      r /= d[q].e;
      so += dg * d[q].src;
      lo += dg * lds_stride[q];
    }
    c->ld_src[e] = so;
    c->ld_lds[e] = lo;
    r = e;
    int64_t dof = 0;
    for (int i = (int)tdst.size() - 1; i >= 0; --i) {
      int q = tdst[i];
      int64_t dg = r % d[q].e;
      r /= d[q].e;
      dof += dg * dst[q];
    }
    c->st_dst[e] = dof;
  }
  c->outer_dims.clear();
  c->outer_src.clear();
  c->outer_dst.clear();
  c->outer_pow2 = 1;
  for (int q : outer) {
    c->outer_dims.push_back(d[q].e);
    c->outer_src.push_back(d[q].src);
    c->outer_dst.push_back(dst[q]);
    if ((d[q].e & (d[q].e - 1)) != 0) c->outer_pow2 = 0;
  }
  c->tiled = 1;
}

// Offsets of the bits of an index over power-of-two runs (innermost run
// last), lowest bit first; false if a run is not a power of two.
bool bit_offsets(const std::vector<Run> &runs, std::vector<int64_t> *out) {
  out->clear();
  for (int q = (int)runs.size() - 1; q >= 0; --q) {
    const int64_t sz = runs[q].size;
    if (sz < 1 || (sz & (sz - 1)) != 0) return false;
    for (int64_t b = 1; b < sz; b <<= 1) out->push_back(runs[q].stride * b);
  }
  return true;
}

int32_t log2_exact(int64_t v) {  // -1 unless v is a power of two
  if (v < 1 || (v & (v - 1)) != 0) return -1;
  int32_t b = 0;
  while ((int64_t(1) << b) < v) ++b;
  return b;
}

// Tables of a fused chain of n = 2 .. kFuseMaxSteps steps st[0 .. n-1], each
// step's product the next step's long operand (see FusedChain).  False when
// the chain does not have the required form.
bool make_fused_chain(const PlanImpl &p, const int32_t *st, int n, FusedChain *f) {
  struct Phase {
    int32_t lng = 0;                 // 0: the step's lhs is its long operand
    int64_t R = 0, K = 0;
    int32_t lr = 0, lk = 0, lb = 0;  // log2 of rows, K and the block's rows
    std::vector<int64_t> r, c;       // offsets in the step's product of its row / column bits
    std::vector<int32_t> tr, tc;     // the product's address bit of each row / column bit
  } ph[kFuseMaxSteps];
  if (n < 2 || n > kFuseMaxSteps) return false;
  // longer chains run every step on the vector ALU, the middle ones with one K
  auto kok = [n](int64_t k) { return k == 2 || k == 4 || k == 8 || (n == 2 && (k == 16 || k == 32)); };
  for (int q = 0; q < n; ++q) {
    const Node &nd = p.nodes[st[q]];
    Phase &h = ph[q];
    // each step is taken with its long operand as the rows, whatever the
    // orientation its own kernel would use
    h.lng = nd.m >= nd.n ? 0 : 1;
    h.R = h.lng == 0 ? nd.m : nd.n;
    const int64_t S = h.lng == 0 ? nd.n : nd.m;
    h.K = nd.k;
    if (!kok(h.K) || S != h.K) return false;
    if (q > 0 && ((h.lng == 0 ? nd.lhs : nd.rhs) != p.L + st[q - 1] || (h.lng == 0 ? nd.copy_a : nd.copy_b) != 0))
      return false;
    // the oriented rows of a node are its N side when swapped, else its M side
    const bool rows_are_runs = (h.lng == 1) == (nd.swap != 0);
    if (!bit_offsets(rows_are_runs ? nd.row_runs : nd.col_runs, &h.r) ||
        !bit_offsets(rows_are_runs ? nd.col_runs : nd.row_runs, &h.c))
      return false;
    h.lr = log2_exact(h.R);
    h.lk = log2_exact(h.K);
    h.lb = log2_exact(kFusePassEntries / h.K);
    if (h.lr < 0 || (int)h.r.size() != h.lr || (int)h.c.size() != h.lk) return false;
    if (q > 0 && h.lr != ph[q - 1].lr + ph[q - 1].lk - h.lk) return false;
    h.tr.assign(h.lr, 0);
    h.tc.assign(h.lk, 0);
    std::vector<char> seen(h.lr + h.lk, 0);
    for (int32_t i = 0; i < h.lr + h.lk; ++i) {
      const int32_t t = log2_exact(i < h.lr ? h.r[i] : h.c[i - h.lr]);
      if (t < 0 || t >= h.lr + h.lk || seen[t]) return false;
      seen[t] = 1;
      (i < h.lr ? h.tr[i] : h.tc[i - h.lr]) = t;
    }
  }
  // K = 2 steps run only beside vector-ALU steps (K <= 8)
  if ((ph[0].K == 2 || ph[1].K == 2) && (ph[0].K > 8 || ph[1].K > 8)) return false;
  const Phase &first = ph[0], &last = ph[n - 1];
  if (first.R < kFuseMinRows || first.lr - first.lb > kFuseOuterMax) return false;
  // A row bit of the first long operand passes through the chain: at each
  // later step it either lands in that step's K (it must then be local to a
  // pass, so that a pass holds whole rows of every step) or stays a row bit;
  // fin[] is its offset in the last product otherwise.
  std::vector<int32_t> local, cand, outer;
  std::vector<int64_t> fin(first.lr, 0);
  for (int32_t b = 0; b < first.lr; ++b) {
    int32_t t = first.tr[b];
    bool reduced = false;
    for (int q = 1; q < n && !reduced; ++q) {
      if (t < ph[q].lk) reduced = true;
      else t = ph[q].tr[t - ph[q].lk];
    }
    if (reduced) {
      local.push_back(b);
    } else {
      fin[b] = int64_t(1) << t;
      cand.push_back(b);
    }
  }
  // The pass's local rows (first.lb of them): those, then the row bits with
  // the smallest offsets in the last product, so that a pass's stores form
  // the longest contiguous pieces.  Rows of X are K1 contiguous entries, so
  // any choice loads whole rows.  A chain of four or more steps must leave
  // two local rows to that choice: with none left its stores fall apart into
  // pieces of a few entries.
  if ((int32_t)local.size() > first.lb - (n >= 4 ? 2 : 0)) return false;
  std::stable_sort(cand.begin(), cand.end(), [&](int32_t x, int32_t y) { return fin[x] < fin[y]; });
  for (int32_t b : cand) ((int32_t)local.size() < first.lb ? local : outer).push_back(b);
  std::sort(local.begin(), local.end());
  std::sort(outer.begin(), outer.end());
  // Each later step's block: the pass's bits of the previous product that are
  // not in this step's K, ascending, are the block's rows; a previous bit t
  // goes to place 2^t (t < lk) or (K + 2) 2^e (block row bit e).
  std::vector<int32_t> prow = local;  // the previous phase's local rows, ascending
  for (int q = 1; q < n; ++q) {
    const Phase &pv = ph[q - 1], &h = ph[q];
    std::vector<int32_t> up;
    for (int32_t i : prow)
      if (pv.tr[i] >= h.lk) up.push_back(pv.tr[i] - h.lk);
    for (int32_t c = 0; c < pv.lk; ++c)
      if (pv.tc[c] >= h.lk) up.push_back(pv.tc[c] - h.lk);
    std::sort(up.begin(), up.end());
    if ((int32_t)up.size() != h.lb) return false;
    auto pos = [&](int32_t t) -> int32_t {
      if (t < h.lk) return int32_t(1) << t;
      const int32_t e = (int32_t)(std::lower_bound(up.begin(), up.end(), t - h.lk) - up.begin());
      return (int32_t)(h.K + 2) << e;  // block rows are K + 2 entries apart
    };
    int32_t *pr = f->pos_row[q - 1], *pc = f->pos_col[q - 1];
    for (size_t i = 0; i < prow.size(); ++i) pr[i] = pos(pv.tr[prow[i]]);
    for (int32_t c = 0; c < pv.lk; ++c) pc[c] = pos(pv.tc[c]);
    prow = up;
  }
  for (int32_t e = 0; e < last.lb; ++e) f->out_row[e] = last.r[prow[e]];
  for (int32_t c = 0; c < last.lk; ++c) f->out_col[c] = last.c[c];
  f->nsteps = n;
  for (int q = 0; q < n; ++q) {
    f->step[q] = st[q];
    f->longop[q] = ph[q].lng;
    f->k[q] = (int32_t)ph[q].K;
  }
  f->rows = first.R;
  f->nouter = first.lr - first.lb;
  for (int32_t i = 0; i < first.lb; ++i) f->lrow[i] = local[i];
  // a workgroup runs four passes at once (bits 0 and 1 of the pass index):
  // they take the two outer row bits with the smallest offsets in the last
  // product, so that the four passes' stores join into longer pieces; the
  // rest count the workgroup's rounds, in ascending row-bit order
  if ((int32_t)outer.size() < 2) return false;
  {
    std::vector<int32_t> by = outer;
    std::stable_sort(by.begin(), by.end(), [&](int32_t x, int32_t y) { return fin[x] < fin[y]; });
    f->wbit[0] = by[0];
    f->wbit[1] = by[1];
    std::vector<int32_t> rest, holes(local);
    for (int32_t i : outer)
      if (i != by[0] && i != by[1]) rest.push_back(i);
    holes.push_back(by[0]);
    holes.push_back(by[1]);
    std::sort(holes.begin(), holes.end());
    for (size_t j = 0; j < holes.size(); ++j) f->hole[j] = holes[j];
    f->out_pass[0] = fin[by[0]];
    f->out_pass[1] = fin[by[1]];
    for (size_t q = 0; q < rest.size(); ++q) f->out_pass[2 + q] = fin[rest[q]];
  }
  // the kernel's writes must cover the last product exactly once: its
  // offsets, one per bit, are the distinct powers of two below its size
  std::vector<int64_t> outs(f->out_pass, f->out_pass + f->nouter);
  outs.insert(outs.end(), f->out_row, f->out_row + last.lb);
  outs.insert(outs.end(), f->out_col, f->out_col + last.lk);
  std::sort(outs.begin(), outs.end());
  if ((int32_t)outs.size() != last.lr + last.lk) return false;
  for (size_t i = 0; i < outs.size(); ++i)
    if (outs[i] != (int64_t(1) << i)) return false;
  return true;
}

tnc_status validate(PlanImpl *p, const tnc_network *net, const tnc_tree *tree) {
  const int32_t nm = net->num_modes;
  if (nm < 0) return TNC_ERR_INVALID_NETWORK;
  if (nm > 0 && !net->extents) return TNC_ERR_INVALID_ARG;
  for (int32_t x = 0; x < nm; ++x)
    if (net->extents[x] < 1) return TNC_ERR_INVALID_NETWORK;
  if (net->num_leaves < 1) return TNC_ERR_INVALID_ARG;
  if (!net->leaf_rank) return TNC_ERR_INVALID_ARG;
  const int32_t L = net->num_leaves;
  std::vector<int> count(nm, 0);
  int64_t pos = 0;
  p->leaves.resize(L);
  for (int32_t l = 0; l < L; ++l) {
    int32_t r = net->leaf_rank[l];
    if (r < 0) return TNC_ERR_INVALID_NETWORK;
    if (r > 0 && !net->leaf_modes) return TNC_ERR_INVALID_ARG;
    std::vector<int32_t> ms(net->leaf_modes + pos, net->leaf_modes + pos + r);
    pos += r;
    std::vector<int32_t> sorted_ms = ms;
    std::sort(sorted_ms.begin(), sorted_ms.end());
    if (std::adjacent_find(sorted_ms.begin(), sorted_ms.end()) != sorted_ms.end()) return TNC_ERR_UNSUPPORTED;
    for (int32_t x : ms) {
      if (x < 0 || x >= nm) return TNC_ERR_INVALID_NETWORK;
      count[x]++;
    }
    p->leaves[l] = std::move(ms);
  }
  if (net->out_rank < 0 || (net->out_rank > 0 && !net->out_modes)) return TNC_ERR_INVALID_ARG;
  std::vector<int32_t> out(net->out_modes, net->out_modes + net->out_rank);
  {
    std::vector<int32_t> so = out;
    std::sort(so.begin(), so.end());
    if (std::adjacent_find(so.begin(), so.end()) != so.end()) return TNC_ERR_INVALID_NETWORK;
  }
  std::vector<char> in_out(nm, 0);
  for (int32_t x : out) {
    if (x < 0 || x >= nm) return TNC_ERR_INVALID_NETWORK;
    in_out[x] = 1;
  }
  for (int32_t x = 0; x < nm; ++x) {
    int c = count[x] + (in_out[x] ? 1 : 0);
    if (c > 2) return TNC_ERR_UNSUPPORTED;
    if (c == 1) return TNC_ERR_INVALID_NETWORK;
    if (in_out[x] && count[x] != 1) return TNC_ERR_INVALID_NETWORK;
  }
  const int32_t S = tree->num_steps;
  if (S != L - 1) return TNC_ERR_INVALID_TREE;
  if (S > 0 && (!tree->lhs || !tree->rhs)) return TNC_ERR_INVALID_ARG;
  std::vector<char> used(L + S, 0);
  for (int32_t s = 0; s < S; ++s) {
    int32_t a = tree->lhs[s], b = tree->rhs[s];
    for (int32_t t : {a, b}) {
      if (t < 0 || t >= L + s || used[t]) return TNC_ERR_INVALID_TREE;
      used[t] = 1;
    }
    if (a == b) return TNC_ERR_INVALID_TREE;
  }
  // sliced modes
  const tnc_plan_options &o = p->opts;
  if (o.num_sliced < 0 || (o.num_sliced > 0 && !o.sliced_modes)) return TNC_ERR_INVALID_ARG;
  if (o.num_sliced > kMaxSliced) return TNC_ERR_UNSUPPORTED;
  std::vector<int32_t> sl(o.sliced_modes, o.sliced_modes + o.num_sliced);
  {
    std::vector<int32_t> ss = sl;
    std::sort(ss.begin(), ss.end());
    if (std::adjacent_find(ss.begin(), ss.end()) != ss.end()) return TNC_ERR_INVALID_ARG;
  }
  for (int32_t x : sl)
    if (x < 0 || x >= nm || count[x] != 2) return TNC_ERR_INVALID_ARG;

  p->num_modes = nm;
  p->extents.assign(net->extents, net->extents + nm);
  p->out_modes = out;
  p->lhs.assign(tree->lhs, tree->lhs + S);
  p->rhs.assign(tree->rhs, tree->rhs + S);
  p->sliced = sl;
  p->L = L;
  p->S = S;
  return TNC_OK;
}

}  // namespace

tnc_status build_plan(const tnc_network *net, const tnc_tree *tree, const tnc_plan_options *opts,
                      PlanImpl *p) {
  if (!net || !tree || !p) return TNC_ERR_INVALID_ARG;
  if (opts) p->opts = *opts;
  else tnc_plan_options_default(&p->opts);
  const tnc_plan_options &o = p->opts;
  if (o.align < 256 || (o.align & (o.align - 1)) != 0) return TNC_ERR_INVALID_ARG;
  if (o.max_group < 1) return TNC_ERR_INVALID_ARG;
  if (o.order != TNC_ORDER_LIFETIME && o.order != TNC_ORDER_NAIVE) return TNC_ERR_INVALID_ARG;
  if (net->dtype != TNC_C64 && net->dtype != TNC_C128) return TNC_ERR_INVALID_ARG;
  if (o.precision != TNC_PREC_EXACT && o.precision != TNC_PREC_BF16X3) return TNC_ERR_INVALID_ARG;
  if (o.precision == TNC_PREC_BF16X3 && net->dtype != TNC_C64) return TNC_ERR_INVALID_ARG;
  p->dtype = net->dtype;
  const uint64_t eb = net->dtype == TNC_C128 ? 16 : 8;  // bytes per entry
  p->elem_bytes = eb;
  tnc_status st = validate(p, net, tree);
  if (st != TNC_OK) return st;

  const int32_t L = p->L, S = p->S, T = L + S;
  p->ext = p->extents;
  for (int32_t x : p->sliced) p->ext[x] = 1;
  const std::vector<int64_t> &ext = p->ext;

  // ---- SSA mode sets (sliced modes removed), per-step K/M/N
  std::vector<std::vector<int32_t>> sets(T);  // sorted mode lists
  std::vector<std::vector<int32_t>> declared(L);
  std::vector<char> has_sliced(L, 0);
  for (int32_t l = 0; l < L; ++l) {
    for (int32_t x : p->leaves[l]) {
      if (contains(p->sliced, x)) has_sliced[l] = 1;
      else declared[l].push_back(x);
    }
    if ((int)declared[l].size() > kMaxRank) return TNC_ERR_UNSUPPORTED;
    sets[l] = declared[l];
    std::sort(sets[l].begin(), sets[l].end());
    int64_t tmp;
    if (!checked_prod(p->extents, p->leaves[l], &tmp)) return TNC_ERR_UNSUPPORTED;
  }
  std::vector<std::vector<int32_t>> K(S), M(S), N(S);
  for (int32_t s = 0; s < S; ++s) {
    const auto &A = sets[p->lhs[s]], &B = sets[p->rhs[s]];
    std::set_intersection(A.begin(), A.end(), B.begin(), B.end(), std::back_inserter(K[s]));
    std::set_difference(A.begin(), A.end(), K[s].begin(), K[s].end(), std::back_inserter(M[s]));
    std::set_difference(B.begin(), B.end(), K[s].begin(), K[s].end(), std::back_inserter(N[s]));
    std::vector<int32_t> C;
    std::set_union(M[s].begin(), M[s].end(), N[s].begin(), N[s].end(), std::back_inserter(C));
    if ((int)C.size() > kMaxRank) return TNC_ERR_UNSUPPORTED;
    int64_t tmp;
    if (!checked_prod(p->extents, C, &tmp)) return TNC_ERR_UNSUPPORTED;
    sets[L + s] = std::move(C);
  }

  // ---- orders
  p->order.assign(T, {});
  p->gemm_a.assign(S, {});
  p->gemm_b.assign(S, {});
  const bool naive = o.order == TNC_ORDER_NAIVE;
  if (!naive) {
    // Lifetime ordering (page section 1.4): a mode that stays alive longer
    // sits further left.  Each mode gets a rank: open modes outlive every
    // step and rank by their place in the output order; a closed mode ranks
    // by the step that reduces it, later steps first, and modes reduced by
    // the same step by ascending label, so that both operands of that step
    // carry the reduced modes innermost in one common order.  Every tensor
    // lists its modes by ascending rank, which puts each operand in the form
    // [modes it hands on to its product, in the product's order | reduced
    // modes]: the GEMM layout the page's reverse pass over the tree builds.
    std::vector<int64_t> rank_of(p->num_modes, 0);
    const int64_t nout = (int64_t)p->out_modes.size();
    for (int64_t i = 0; i < nout; ++i) rank_of[p->out_modes[i]] = i;
    for (int32_t s = 0; s < S; ++s)
      for (size_t q = 0; q < K[s].size(); ++q)  // K[s] is ascending
        rank_of[K[s][q]] = nout + (int64_t)(S - 1 - s) * (p->num_modes + 1) + (int64_t)q;
    for (int32_t t = 0; t < T; ++t) {
      std::vector<int32_t> o2 = sets[t];
      std::sort(o2.begin(), o2.end(), [&](int32_t a, int32_t b) { return rank_of[a] < rank_of[b]; });
      p->order[t] = std::move(o2);
    }
    for (int32_t s = 0; s < S; ++s) {
      p->gemm_a[s] = p->order[p->lhs[s]];
      p->gemm_b[s] = p->order[p->rhs[s]];
    }
    p->root_permute = 0;
  } else {
    for (int32_t l = 0; l < L; ++l) p->order[l] = declared[l];
    for (int32_t s = 0; s < S; ++s) {
      std::vector<int32_t> ra, rb;
      for (int32_t x : p->order[p->lhs[s]])
        if (!std::binary_search(K[s].begin(), K[s].end(), x)) ra.push_back(x);
      for (int32_t x : p->order[p->rhs[s]])
        if (!std::binary_search(K[s].begin(), K[s].end(), x)) rb.push_back(x);
      p->gemm_a[s] = ra;
      p->gemm_a[s].insert(p->gemm_a[s].end(), K[s].begin(), K[s].end());
      p->gemm_b[s] = rb;
      p->gemm_b[s].insert(p->gemm_b[s].end(), K[s].begin(), K[s].end());
      ra.insert(ra.end(), rb.begin(), rb.end());
      p->order[L + s] = ra;
    }
    p->root_permute = (S > 0 && p->order[T - 1] != p->out_modes) ? 1 : 0;
  }
  if (S == 0) p->order[0] = p->out_modes;

  // ---- nodes
  p->staged_leaf.assign(L, 0);
  p->nodes.assign(S, Node{});
  double flops = 0, flops_u = 0, bytes = 0;
  uint64_t max_elems = 0;
  for (int32_t s = 0; s < S; ++s) {
    Node &nd = p->nodes[s];
    nd.lhs = p->lhs[s];
    nd.rhs = p->rhs[s];
    nd.out = L + s;
    nd.is_root = (s == S - 1) ? 1 : 0;
    nd.m = prod(ext, M[s]);
    nd.n = prod(ext, N[s]);
    nd.k = prod(ext, K[s]);
    nd.mu = prod(p->extents, M[s]);
    nd.nu = prod(p->extents, N[s]);
    nd.ku = prod(p->extents, K[s]);
    flops += 8.0 * (double)nd.m * (double)nd.n * (double)nd.k;
    flops_u += 8.0 * (double)nd.mu * (double)nd.nu * (double)nd.ku;
    bytes += (double)eb * ((double)nd.m * nd.k + (double)nd.n * nd.k + (double)nd.m * nd.n);
    max_elems = std::max<uint64_t>(max_elems, (uint64_t)(nd.m * nd.n));
    __int128 mnk = (__int128)nd.m * nd.n * nd.k;
    // a tiny step runs in one workgroup: its flops and its entries are bounded
    const __int128 entries = (__int128)nd.m * nd.k + (__int128)nd.n * nd.k + (__int128)nd.m * nd.n;
    if (mnk <= (__int128)o.tiny_mnk && entries <= (__int128)(o.tiny_mnk / 4)) nd.cls = TNC_CLASS_TINY;
    else if (std::min(nd.m, nd.n) <= kSkinnyMaxSide) nd.cls = TNC_CLASS_SKINNY;
    else nd.cls = TNC_CLASS_GEMM;
    const auto &c_order = p->order[L + s];
    int32_t last_eff = -1;
    for (int32_t x : c_order)
      if (ext[x] > 1) last_eff = x;
    if (nd.cls == TNC_CLASS_SKINNY) nd.swap = nd.n > nd.m ? 1 : 0;
    else nd.swap = (last_eff >= 0 && std::binary_search(M[s].begin(), M[s].end(), last_eff)) ? 1 : 0;
    make_runs(c_order, ext, nd.swap ? N[s] : M[s], &nd);
    int64_t R = nd.swap ? nd.n : nd.m, Sx = nd.swap ? nd.m : nd.n;
    // the GEMM kernel indexes rows, columns and K with 32-bit integers
    if (nd.cls == TNC_CLASS_GEMM && (R >= (int64_t(1) << 31) || Sx >= (int64_t(1) << 31) ||
                                     nd.k >= (int64_t(1) << 31)))
      return TNC_ERR_UNSUPPORTED;
    nd.splits = split_rule(nd.cls, R, Sx, nd.k, eb == 8);
    if (nd.splits > 1) nd.scratch_bytes = (uint64_t)nd.splits * (uint64_t)R * (uint64_t)Sx * eb;
    // operand copies
    for (int w = 0; w < 2; ++w) {
      int32_t t = w == 0 ? nd.lhs : nd.rhs;
      const auto &want = w == 0 ? p->gemm_a[s] : p->gemm_b[s];
      int need;
      if (t < L) {
        need = (has_sliced[t] || declared[t] != want) ? 1 : 0;
        if (need) p->staged_leaf[t] = 1;
      } else {
        need = p->order[t] != want ? 1 : 0;
      }
      (w == 0 ? nd.copy_a : nd.copy_b) = need;
    }
  }
  if (S == 0) p->staged_leaf.assign(L, 0);

  // ---- fused chains: a non-tiny step whose product is at once the long
  // operand of another non-tiny step, both of the FusedChain form, extended
  // one step at a time while the chain keeps that form (up to kFuseMaxSteps);
  // chains do not overlap and are taken in step order
  p->fused.clear();
  if (o.fuse && !naive && eb == 8 && o.precision == TNC_PREC_EXACT) {
    std::vector<int32_t> consumer(T, -1);
    for (int32_t s = 0; s < S; ++s) {
      consumer[p->lhs[s]] = s;
      consumer[p->rhs[s]] = s;
    }
    for (int32_t s1 = 0; s1 < S; ++s1) {
      Node &a = p->nodes[s1];
      if (a.cls == TNC_CLASS_TINY || a.splits > 1 || a.fuse_prev >= 0 || a.is_root) continue;
      const int32_t s2 = consumer[L + s1];
      if (s2 < 0) continue;
      Node &b = p->nodes[s2];
      if (b.cls == TNC_CLASS_TINY || b.splits > 1 || b.is_root) continue;
      int32_t st[kFuseMaxSteps] = {s1, s2};
      FusedChain f;
      if (!make_fused_chain(*p, st, 2, &f)) continue;
      int n = 2;
      while (n < kFuseMaxSteps) {
        const int32_t sn = consumer[L + st[n - 1]];
        if (sn < 0) break;
        const Node &c = p->nodes[sn];
        if (c.cls == TNC_CLASS_TINY || c.splits > 1 || c.is_root) break;
        st[n] = sn;
        FusedChain g;
        if (!make_fused_chain(*p, st, n + 1, &g)) break;
        f = g;
        ++n;
      }
      for (int q = 0; q + 1 < n; ++q) {
        p->nodes[st[q]].fuse_next = st[q + 1];
        p->nodes[st[q + 1]].fuse_prev = st[q];
      }
      p->nodes[st[n - 1]].fused_index = (int32_t)p->fused.size();
      p->fused.push_back(f);
    }
  }

  // ---- launch groups: the tiny steps between two non-tiny steps (a segment)
  // run in dependency-level order, one group per level (split at max_group
  // members, list order inside a level); non-tiny steps are groups of their
  // own.  Level = 0 unless an operand was produced in the same segment, then
  // one more than that producer's level.
  p->groups.clear();
  {
    std::vector<int32_t> segment;
    std::vector<int32_t> level(T, -1);  // level of outputs produced in the open segment
    auto flush = [&]() {
      if (segment.empty()) return;
      int32_t depth = 0;
      for (int32_t s : segment) {
        const Node &nd = p->nodes[s];
        int32_t lv = 0;
        for (int32_t t : {nd.lhs, nd.rhs})
          if (level[t] >= 0) lv = std::max(lv, level[t] + 1);
        level[nd.out] = lv;
        depth = std::max(depth, lv + 1);
      }
      for (int32_t lv = 0; lv < depth; ++lv) {
        std::vector<int32_t> members;
        for (int32_t s : segment)
          if (level[p->nodes[s].out] == lv) members.push_back(s);
        for (size_t i = 0; i < members.size(); i += (size_t)o.max_group)
          p->groups.emplace_back(members.begin() + i,
                                 members.begin() + std::min(members.size(), i + (size_t)o.max_group));
      }
      for (int32_t s : segment) level[p->nodes[s].out] = -1;
      segment.clear();
    };
    for (int32_t s = 0; s < S; ++s) {
      if (p->nodes[s].cls == TNC_CLASS_TINY) {
        segment.push_back(s);
      } else {
        flush();
        p->groups.push_back({s});
      }
    }
    flush();
  }
  for (size_t g = 0; g < p->groups.size(); ++g)
    for (int32_t s : p->groups[g]) p->nodes[s].group = (int32_t)g;

  // ---- arena
  auto rbytes = [&](int64_t elems) { return round_up((uint64_t)elems * eb, o.align); };
  std::vector<int64_t> elems(T);
  for (int32_t t = 0; t < T; ++t) elems[t] = prod(ext, sets[t]);
  Arena arena;
  p->tensor_off.assign(T, kNone);
  // early staging: copies of leaves with at most kEarlyStageMax entries are
  // made in one launch before the first group, so they are allocated first
  // (in execution order, A before B) and freed with their consumer group
  std::vector<std::array<char, 2>> early(S, {0, 0});
  for (auto &members : p->groups)
    for (int32_t s : members) {
      Node &nd = p->nodes[s];
      for (int w = 0; w < 2; ++w) {
        int32_t t = w == 0 ? nd.lhs : nd.rhs;
        int32_t copy = w == 0 ? nd.copy_a : nd.copy_b;
        if (copy && t < L && elems[t] <= kEarlyStageMax) {
          uint64_t &off = w == 0 ? nd.a_off : nd.b_off;
          off = arena.alloc(rbytes(elems[t]));
          if (!naive) p->tensor_off[t] = off;
          early[s][w] = 1;
        }
      }
    }
  // a fused chain's earlier steps keep their operands until the chain's
  // launch (its last step's group) and store no product
  std::vector<std::vector<std::pair<uint64_t, uint64_t>>> deferred(S);
  for (auto &members : p->groups) {
    std::vector<std::pair<uint64_t, uint64_t>> to_free;
    for (int32_t s : members) {
      Node &nd = p->nodes[s];
      auto &frees = nd.fuse_next >= 0 ? deferred[s] : to_free;
      if (nd.fuse_prev >= 0) {
        // the chain's earlier steps: their operands stay until its last step
        auto &d = deferred[nd.fuse_prev];
        frees.insert(frees.end(), d.begin(), d.end());
      }
      for (int w = 0; w < 2; ++w) {
        int32_t t = w == 0 ? nd.lhs : nd.rhs;
        int32_t copy = w == 0 ? nd.copy_a : nd.copy_b;
        uint64_t &off = w == 0 ? nd.a_off : nd.b_off;
        if (early[s][w]) {
          frees.push_back({off, rbytes(elems[t])});
        } else if (copy) {
          off = arena.alloc(rbytes(elems[t]));
          frees.push_back({off, rbytes(elems[t])});
          if (t < L && !naive) p->tensor_off[t] = off;
        } else if (nd.fuse_prev >= 0 && t == L + nd.fuse_prev) {
          off = kNone;  // the previous product of its chain: never stored
        } else if (t >= L) {
          off = p->tensor_off[t];
          frees.push_back({off, rbytes(elems[t])});
        }
      }
      if (nd.fuse_next >= 0) {
        nd.c_off = kNone;
        continue;
      }
      if (nd.is_root && !p->root_permute) {
        nd.c_off = kNone;
      } else {
        nd.c_off = arena.alloc(rbytes(elems[nd.out]));
        p->tensor_off[nd.out] = nd.c_off;
      }
      if (nd.splits > 1) {
        uint64_t sb = round_up(nd.scratch_bytes, o.align);
        nd.scratch_off = arena.alloc(sb);
        to_free.push_back({nd.scratch_off, sb});
      }
    }
    for (auto &f : to_free) arena.release(f.first, f.second);
  }
  p->arena_bytes = arena.peak();

  // ---- copies and the launch program
  p->slice_extents.clear();
  for (int32_t x : p->sliced) p->slice_extents.push_back(p->extents[x]);
  auto leaf_strides = [&](int32_t l) {
    // declared row-major strides with full (unsliced) extents
    std::vector<int64_t> st(p->leaves[l].size());
    int64_t s = 1;
    for (int q = (int)p->leaves[l].size() - 1; q >= 0; --q) {
      st[q] = s;
      s *= p->extents[p->leaves[l][q]];
    }
    return st;
  };
  bool copy_bounds_ok = true;
  auto make_copy = [&](int32_t src_tensor, int32_t src_buf, uint64_t src_off, int32_t dst_buf, uint64_t dst_off,
                       const std::vector<int32_t> &dst_order, int32_t is_root) {
    CopyOp c;
    c.src_buf = src_buf;
    c.src_off_bytes = src_off;
    c.dst_buf = dst_buf;
    c.dst_off_bytes = dst_off;
    c.is_root = is_root;
    // source strides of every mode
    std::vector<int32_t> src_modes;
    std::vector<int64_t> src_st;
    if (src_tensor < L) {
      src_modes = p->leaves[src_tensor];
      src_st = leaf_strides(src_tensor);
    } else {
      src_modes = p->order[src_tensor];
      src_st.resize(src_modes.size());
      int64_t s = 1;
      for (int q = (int)src_modes.size() - 1; q >= 0; --q) {
        src_st[q] = s;
        s *= ext[src_modes[q]];
      }
    }
    auto stride_of = [&](int32_t x) -> int64_t {
      for (size_t q = 0; q < src_modes.size(); ++q)
        if (src_modes[q] == x) return src_st[q];
      return 0;
    };
    std::vector<int64_t> dims, sst;
    for (int32_t x : dst_order) {
      if (ext[x] <= 1) continue;
      int64_t d = ext[x], ss = stride_of(x);
      if (!dims.empty() && sst.back() == ss * d) {
        dims.back() *= d;
        sst.back() = ss;
      } else {
        dims.push_back(d);
        sst.push_back(ss);
      }
    }
    c.dims = dims;
    c.src_strides = sst;
    c.count = prod(ext, dst_order);
    for (int32_t x : p->sliced) c.slice_strides.push_back(src_tensor < L ? stride_of(x) : 0);
    // every source offset the copy can form must lie inside the source buffer
    int64_t src_size = src_tensor < L ? prod(p->extents, p->leaves[src_tensor]) : prod(ext, src_modes);
    int64_t max_off = 0;
    for (size_t q = 0; q < dims.size(); ++q) max_off += (dims[q] - 1) * sst[q];
    for (size_t t = 0; t < p->sliced.size(); ++t) max_off += (p->slice_extents[t] - 1) * c.slice_strides[t];
    if (max_off >= src_size) copy_bounds_ok = false;
    if (c.count >= kCopyTiledMin) make_tile(&c);
    return c;
  };
  p->copies.clear();
  p->program.clear();
  auto push_copy_op = [&](int32_t idx) {
    const int64_t kBig = int64_t(1) << 20;
    int64_t cnt = p->copies[idx].count;
    if (p->copies[idx].tiled) {
      p->program.push_back({OP_COPY_TILED, idx, 1, cnt});
      return;
    }
    if (!p->program.empty() && p->program.back().kind == OP_COPY && cnt <= kBig &&
        p->program.back().max_count <= kBig && p->program.back().first + p->program.back().count == idx) {
      p->program.back().count++;
      p->program.back().max_count = std::max(p->program.back().max_count, cnt);
    } else {
      p->program.push_back({OP_COPY, idx, 1, cnt});
    }
  };
  if (S == 0) {
    p->copies.push_back(make_copy(0, kBufLeaf0 + 0, 0, kBufOut, 0, p->out_modes, 1));
    push_copy_op(0);
  }
  std::vector<TinyDesc> tiny;
  std::vector<RunDev> runs;
  auto emit_copy = [&](int32_t s, int w) {
    Node &nd = p->nodes[s];
    int32_t t = w == 0 ? nd.lhs : nd.rhs;
    uint64_t dst = w == 0 ? nd.a_off : nd.b_off;
    const auto &want = w == 0 ? p->gemm_a[s] : p->gemm_b[s];
    int32_t src_buf = t < L ? kBufLeaf0 + t : kBufArena;
    uint64_t src_off = t < L ? 0 : p->tensor_off[t];
    p->copies.push_back(make_copy(t, src_buf, src_off, kBufArena, dst, want, 0));
    push_copy_op((int32_t)p->copies.size() - 1);
  };
  for (auto &members : p->groups)
    for (int32_t s : members)
      for (int w = 0; w < 2; ++w)
        if (early[s][w]) emit_copy(s, w);
  for (auto &members : p->groups) {
    // staging / re-layout copies of this group's operands
    for (int32_t s : members) {
      const Node &nd = p->nodes[s];
      for (int w = 0; w < 2; ++w)
        if ((w == 0 ? nd.copy_a : nd.copy_b) && !early[s][w]) emit_copy(s, w);
    }
    // compute
    const Node &first = p->nodes[members[0]];
    if (first.cls == TNC_CLASS_TINY) {
      Op op{OP_TINY_GROUP, (int32_t)tiny.size(), (int32_t)members.size(), 0};
      for (int32_t s : members) {
        Node &nd = p->nodes[s];
        nd.runs_index = (int32_t)runs.size();
        for (auto &r : nd.row_runs) runs.push_back({r.size, r.stride});
        for (auto &r : nd.col_runs) runs.push_back({r.size, r.stride});
        TinyDesc d{};
        auto operand = [&](int w, int32_t *buf, int64_t *off) {
          int32_t t = w == 0 ? nd.lhs : nd.rhs;
          int32_t copy = w == 0 ? nd.copy_a : nd.copy_b;
          uint64_t ao = w == 0 ? nd.a_off : nd.b_off;
          if (copy || t >= L) { *buf = kBufArena; *off = (int64_t)(ao / eb); }
          else { *buf = kBufLeaf0 + t; *off = 0; }
        };
        operand(nd.swap ? 1 : 0, &d.x_buf, &d.x_off);
        operand(nd.swap ? 0 : 1, &d.y_buf, &d.y_off);
        if (nd.c_off == kNone) { d.c_buf = kBufOut; d.c_off = 0; }
        else { d.c_buf = kBufArena; d.c_off = (int64_t)(nd.c_off / eb); }
        d.is_root = nd.is_root && !p->root_permute;
        d.R = (int32_t)(nd.swap ? nd.n : nd.m);
        d.S = (int32_t)(nd.swap ? nd.m : nd.n);
        d.K = (int32_t)nd.k;
        d.nrr = (int32_t)nd.row_runs.size();
        d.ncr = (int32_t)nd.col_runs.size();
        d.runs_index = nd.runs_index;
        tiny.push_back(d);
        op.max_count = std::max(op.max_count, (int64_t)d.R * d.S);
      }
      p->program.push_back(op);
    } else {
      Node &nd = p->nodes[members[0]];
      nd.runs_index = (int32_t)runs.size();
      for (auto &r : nd.row_runs) runs.push_back({r.size, r.stride});
      for (auto &r : nd.col_runs) runs.push_back({r.size, r.stride});
      if (nd.fuse_prev >= 0 && nd.fuse_next < 0)
        p->program.push_back({OP_FUSED, nd.fused_index, p->fused[nd.fused_index].nsteps, 0});
      else if (nd.fuse_next < 0 && nd.fuse_prev < 0)  // a chain's earlier steps run in its last step's launch
        p->program.push_back({first.cls == TNC_CLASS_SKINNY ? OP_SKINNY : OP_GEMM, members[0], 1, 0});
    }
  }
  if (p->root_permute) {
    p->copies.push_back(make_copy(T - 1, kBufArena, p->tensor_off[T - 1], kBufOut, 0, p->out_modes, 1));
    push_copy_op((int32_t)p->copies.size() - 1);
  }

  if (!copy_bounds_ok) return TNC_ERR_UNSUPPORTED;  // internal layout error: never launch it

  // ---- descriptor blob: [runs][copy descs][tiny descs][int64 table]
  std::vector<CopyDesc> cdesc;
  std::vector<int64_t> ints;
  for (auto &c : p->copies) {
    CopyDesc d{};
    d.src_buf = c.src_buf;
    d.dst_buf = c.dst_buf;
    d.rank = (int32_t)c.dims.size();
    d.is_root = c.is_root;
    d.src_off = (int64_t)(c.src_off_bytes / eb);
    d.dst_off = (int64_t)(c.dst_off_bytes / eb);
    d.count = c.count;
    d.ints_index = (int32_t)ints.size();
    d.tiled = c.tiled;
    if (!c.tiled) {
      ints.insert(ints.end(), c.dims.begin(), c.dims.end());
      ints.insert(ints.end(), c.src_strides.begin(), c.src_strides.end());
      ints.insert(ints.end(), c.slice_strides.begin(), c.slice_strides.end());
    } else {
      ints.push_back(c.tile);
      ints.push_back((int64_t)c.outer_dims.size());
      ints.push_back(c.outer_pow2);
      ints.insert(ints.end(), c.outer_dims.begin(), c.outer_dims.end());
      ints.insert(ints.end(), c.outer_src.begin(), c.outer_src.end());
      ints.insert(ints.end(), c.outer_dst.begin(), c.outer_dst.end());
      ints.insert(ints.end(), c.slice_strides.begin(), c.slice_strides.end());
      ints.insert(ints.end(), c.ld_src.begin(), c.ld_src.end());
      ints.insert(ints.end(), c.ld_lds.begin(), c.ld_lds.end());
      ints.insert(ints.end(), c.st_dst.begin(), c.st_dst.end());
    }
    cdesc.push_back(d);
  }
  auto append = [&](const void *src, size_t n) {
    size_t at = round_up(p->blob.size(), 16);
    p->blob.resize(at + n);
    if (n) std::memcpy(p->blob.data() + at, src, n);
    return (uint64_t)at;
  };
  p->blob.clear();
  p->blob_runs = append(runs.data(), runs.size() * sizeof(RunDev));
  p->blob_copies = append(cdesc.data(), cdesc.size() * sizeof(CopyDesc));
  p->blob_tiny = append(tiny.data(), tiny.size() * sizeof(TinyDesc));
  p->blob_ints = append(ints.data(), ints.size() * sizeof(int64_t));
  if (p->blob.empty()) p->blob.resize(16);

  p->ptab_bytes = round_up(8ull * (uint64_t)(2 + L), 256);
  p->blob_bytes = round_up(p->blob.size(), 256);
  p->header_bytes = p->ptab_bytes + p->blob_bytes;

  // ---- stats
  tnc_plan_stats &stt = p->stats;
  std::memset(&stt, 0, sizeof(stt));
  stt.num_leaves = L;
  stt.num_steps = S;
  stt.num_groups = (int32_t)p->groups.size();
  stt.min_inner_run = S > 0 ? INT32_MAX : 0;
  for (auto &nd : p->nodes) {
    if (nd.cls == TNC_CLASS_TINY) stt.nodes_tiny++;
    else if (nd.cls == TNC_CLASS_SKINNY) stt.nodes_skinny++;
    else stt.nodes_gemm++;
    if (nd.splits > 1) stt.nodes_split++;
    stt.nodes_interleaved += nd.interleaved;
    stt.min_inner_run = std::min<int32_t>(stt.min_inner_run, (int32_t)std::min<int64_t>(nd.inner_run, INT32_MAX));
    if (nd.lhs >= L) stt.relayouts += nd.copy_a;
    if (nd.rhs >= L) stt.relayouts += nd.copy_b;
  }
  for (int32_t l = 0; l < L; ++l) stt.staged_leaves += p->staged_leaf[l];
  stt.root_permute = p->root_permute;
  {
    __int128 ns = 1;
    for (int64_t e : p->slice_extents) {
      ns *= e;
      if (ns > (__int128)(INT64_MAX / 2)) return TNC_ERR_UNSUPPORTED;
    }
    stt.num_slices = (int64_t)ns;
  }
  if (o.slice_begin == 0 && o.slice_end == 0) {
    p->slice_begin = 0;
    p->slice_end = stt.num_slices;
  } else {
    if (o.slice_begin < 0 || o.slice_end <= o.slice_begin || o.slice_end > stt.num_slices)
      return TNC_ERR_INVALID_ARG;
    p->slice_begin = o.slice_begin;
    p->slice_end = o.slice_end;
  }
  stt.flops = flops;
  stt.flops_unsliced = flops_u;
  stt.bytes = bytes;
  stt.max_intermediate = max_elems;
  stt.header_bytes = p->header_bytes;
  stt.arena_bytes = p->arena_bytes;
  stt.workspace_bytes = p->header_bytes + p->arena_bytes;
  stt.fused_pairs = (int32_t)p->fused.size();
  if (o.capacity_bytes > 0 && stt.workspace_bytes > o.capacity_bytes) return TNC_ERR_OUT_OF_MEMORY;
  return TNC_OK;
}

}  // namespace tnc
