// Descriptor layouts shared by the host planner and the HIP kernels.  The
// planner writes them into a blob that tnc_execute uploads into the head of
// the caller's workspace; grouped kernels read them from there.
#pragma once

#include <cstdint>

namespace tnc {

// Buffer ids used by descriptors; the device pointer table holds
// [arena base, out, leaf 0, leaf 1, ...].
enum : int32_t { kBufArena = 0, kBufOut = 1, kBufLeaf0 = 2 };

constexpr int kMaxSliced = 32;

struct RunDev {
  int64_t size;    // number of index values the run covers (product of its extents)
  int64_t stride;  // stride in C, in entries, of the run's innermost mode
};

// Permuting copy: dst (contiguous, dims outermost first) <- src (strided).
struct CopyDesc {
  int32_t src_buf, dst_buf;
  int32_t rank, is_root;
  int64_t src_off, dst_off;   // in complex64 entries
  int64_t count;
  int32_t ints_index;         // into the int64 table, see below
  int32_t tiled;              // 0: ints = dims[rank], src_strides[rank], slice[num_sliced]
                              // 1: ints = tile, n_outer, outer_pow2, outer_dims[n_outer],
                              //    outer_src[n_outer], outer_dst[n_outer], slice[num_sliced],
                              //    ld_src[tile], ld_lds[tile], st_dst[tile]
};

// One tiny pairwise step of a grouped launch, already oriented: C[i, j] =
// sum_l X[i, l] Y[j, l] with X = rows operand [R, K], Y = cols operand [S, K].
struct TinyDesc {
  int32_t x_buf, y_buf, c_buf, is_root;
  int64_t x_off, y_off, c_off;  // in complex64 entries
  int32_t R, S, K;
  int32_t nrr, ncr, runs_index; // output runs: rows then cols, in the run table
};

}  // namespace tnc
