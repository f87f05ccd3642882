// Host-side plan of a tree contraction: mode orders, per-step GEMM
// descriptors, launch groups, arena offsets and the device descriptor blob.
//
// Mode orders follow the reverse-tree "lifetime ordering" of the page
// "Parallelizing Large-Scale Tensor Network Contraction on Multiple GPUs",
// section 1.4.  The rest (kernel classes, orientation, output runs, split-K,
// grouping, first-fit arena) is this library's execution design.
#pragma once

#include <cstdint>
#include <string>
#include <vector>

#include "../../include/tnc.h"
#include "device_desc.hpp"

namespace tnc {

constexpr uint64_t kNone = UINT64_MAX;
constexpr int kMaxRank = 64;
constexpr int64_t kSkinnyMaxSide = 16;   // skinny when min(m, n) <= this
constexpr int64_t kGemmNominalTile = 128;
constexpr int64_t kCopyTileMax = 1024;     // entries per LDS tile of a tiled copy
constexpr int64_t kCopyTiledMin = 1 << 16;  // copies at least this large use the tiled kernel
constexpr int64_t kEarlyStageMax = 1 << 16; // staged leaves up to this size are copied before the first group

struct Run {
  int64_t size;
  int64_t stride;  // stride in C (entries) of the run's innermost mode
};

// A copy of one tensor into a new layout (leaf staging, NAIVE re-layout,
// NAIVE root permute, single-leaf networks).
struct CopyOp {
  int32_t src_buf;             // buffer id: kBufArena, kBufOut, kBufLeaf0 + leaf
  uint64_t src_off_bytes;      // offset inside the source buffer
  int32_t dst_buf;
  uint64_t dst_off_bytes;
  int64_t count;               // entries copied
  int32_t is_root;             // destination is `out` (beta applies across slices)
  std::vector<int64_t> dims;   // destination dims, outermost first (merged, extent > 1)
  std::vector<int64_t> src_strides;
  std::vector<int64_t> slice_strides;  // per sliced mode: source stride (0 if absent)
  // Tiled variant (large copies): a tile over the innermost destination dims
  // and the smallest-source-stride dims goes through LDS; the tables give,
  // per tile entry, its source offset and LDS slot in source order, and its
  // destination offset in destination order.  Outer dims enumerate tiles.
  int32_t tiled = 0;
  int64_t tile = 0;
  std::vector<int64_t> ld_src, ld_lds, st_dst;
  std::vector<int64_t> outer_dims, outer_src, outer_dst;
  int32_t outer_pow2 = 0;
};

struct Node {
  int32_t lhs = -1, rhs = -1, out = -1;
  int64_t m = 1, n = 1, k = 1;        // with sliced modes fixed
  int64_t mu = 1, nu = 1, ku = 1;     // unsliced
  int32_t cls = TNC_CLASS_TINY;
  int32_t swap = 0;
  int32_t group = -1;
  int32_t splits = 1;
  std::vector<Run> row_runs, col_runs;
  int64_t inner_run = 1;
  int32_t interleaved = 0;
  int32_t copy_a = 0, copy_b = 0;
  uint64_t a_off = kNone, b_off = kNone, c_off = kNone;
  uint64_t scratch_off = kNone, scratch_bytes = 0;
  int32_t is_root = 0;
  // device run table location (entries into the blob's run array)
  int32_t runs_index = 0;
  // fused chains (see FusedChain): only the last step's product is stored;
  // every step of the chain runs in the launch of the last
  int32_t fuse_next = -1;    // the next step of its fused chain
  int32_t fuse_prev = -1;    // the previous step of its fused chain
  int32_t fused_index = -1;  // a chain's last step: index into PlanImpl::fused
};

// A chain of 2 .. kFuseMaxSteps complex64 steps run as one pass over the
// first step's long operand (k_fused2): each step's product is at once the
// next step's long operand, and each step absorbs a small tensor with K = S
// (2, 4, 8, 16 or 32 entries, K = 2 only beside K <= 8; in chains of three
// or more every K is 2, 4 or 8).  Built when every
// index is a power of two and a pass of kFusePassEntries entries of the long
// operand holds whole rows of every step; the tables give, per index bit, the
// place of an entry (see Fused2Args in kernels.hpp).
constexpr int64_t kFusePassEntries = 1024;
constexpr int32_t kFuseOuterMax = 48;
constexpr int32_t kFuseMaxSteps = 6;
constexpr int64_t kFuseMinRows = int64_t(1) << 16;  // smaller steps are not worth a pass
struct FusedChain {
  int32_t nsteps = 0;
  int32_t step[kFuseMaxSteps] = {};
  int32_t longop[kFuseMaxSteps] = {};  // 0: the step's lhs is its long operand, 1: its rhs
  int32_t k[kFuseMaxSteps] = {};       // each step's K (= its short side S)
  int64_t rows = 0;          // rows of the first step's long operand
  int32_t nouter = 0;
  int32_t lrow[9] = {};      // the pass's local row bits of the long operand, ascending
  int32_t wbit[2] = {};      // row bits set by bits 0, 1 of the pass index (a workgroup's four passes)
  int32_t hole[11] = {};     // lrow and wbit, ascending: the rest count the workgroup's rounds
  // [q]: the places of step q's products in step q + 1's block
  int32_t pos_row[kFuseMaxSteps - 1][9] = {}, pos_col[kFuseMaxSteps - 1][8] = {};
  int64_t out_row[9] = {}, out_col[8] = {};  // the last product's offsets
  int64_t out_pass[kFuseOuterMax] = {};
};

enum OpKind : int32_t { OP_COPY = 0, OP_TINY_GROUP = 1, OP_SKINNY = 2, OP_GEMM = 3, OP_COPY_TILED = 4,
                        OP_FUSED = 5 };

struct Op {
  OpKind kind;
  int32_t first;   // OP_COPY: first index into copy descriptors; TINY: first tiny desc;
                   // OP_FUSED: index into PlanImpl::fused; else node
  int32_t count;   // OP_COPY / OP_TINY_GROUP: descriptors in the launch
  int64_t max_count;  // OP_COPY: largest copy in the launch; OP_TINY_GROUP: largest member R S (grid sizing)
};

struct PlanImpl {
  // ---- inputs (copied)
  int32_t num_modes = 0;
  std::vector<int64_t> extents;      // as given
  std::vector<int64_t> ext;          // sliced modes set to 1
  std::vector<std::vector<int32_t>> leaves;
  std::vector<int32_t> out_modes;
  std::vector<int32_t> lhs, rhs;
  std::vector<int32_t> sliced;
  tnc_plan_options opts{};

  tnc_dtype dtype = TNC_C64;
  uint64_t elem_bytes = 8;                     // 8 (complex64) or 16 (complex128)

  // ---- derived
  int32_t L = 0, S = 0;
  std::vector<std::vector<int32_t>> order;     // planned order per SSA tensor
  std::vector<std::vector<int32_t>> gemm_a, gemm_b;
  std::vector<Node> nodes;
  std::vector<FusedChain> fused;
  std::vector<std::vector<int32_t>> groups;
  std::vector<uint64_t> tensor_off;
  std::vector<int32_t> staged_leaf;
  int32_t root_permute = 0;
  uint64_t arena_bytes = 0;
  uint64_t ptab_bytes = 0, blob_bytes = 0, header_bytes = 0;
  tnc_plan_stats stats{};

  // ---- execution program
  std::vector<CopyOp> copies;
  std::vector<Op> program;
  std::vector<uint8_t> blob;                   // host image of the device descriptor blob
  uint64_t blob_runs = 0, blob_copies = 0, blob_tiny = 0, blob_ints = 0;  // byte offsets in blob
  std::vector<int64_t> slice_extents;          // extents of sliced modes
  int64_t slice_begin = 0, slice_end = 1;      // slices tnc_execute runs
};

tnc_status build_plan(const tnc_network *net, const tnc_tree *tree, const tnc_plan_options *opts,
                      PlanImpl *p);

// Distribution schedule over P GPUs (dist.cpp); `steps` holds p.S records.
tnc_status plan_distribution(const PlanImpl &p, const tnc_dist_options &o, tnc_dist_step *steps, double *total,
                             std::string *err);

}  // namespace tnc
