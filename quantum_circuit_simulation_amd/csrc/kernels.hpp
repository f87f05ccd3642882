// Launchers of the gfx950 kernels (defined in kernels.hip).
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>

#include "device_desc.hpp"

namespace tnc {

struct SliceDigits {
  int32_t n;
  int32_t digit[kMaxSliced];
};

// Operands of one oriented pairwise step: C[i, j] = sum_l X[i, l] * Y[j, l],
// X row-major [R, K], Y row-major [S, K]; T = float2 (complex64) or double2
// (complex128).  C is written at rowoff(i) + coloff(j) through `runs` (nrr row
// runs then ncr col runs, outermost first).  beta = 1 adds into C.
// splits > 1: K is cut into `splits` chunks whose partial sums go to
// `scratch` [splits, R, S] and are then reduced into C.
template <typename T>
struct StepArgsT {
  const T *X;
  const T *Y;
  T *C;
  int64_t R, S, K;
  const RunDev *runs;
  int32_t nrr, ncr;
  int32_t beta;
  int32_t splits;
  T *scratch;
  int32_t prec;  // kPrecExact or kPrecBf16x3 (the plan's tnc_precision)
  int32_t pow2_runs;  // every row and column run has a power-of-two size
};
constexpr int32_t kPrecExact = 0;   // TNC_PREC_EXACT
constexpr int32_t kPrecBf16x3 = 1;  // TNC_PREC_BF16X3
using StepArgs = StepArgsT<float2>;    // complex64
using StepArgsZ = StepArgsT<double2>;  // complex128

// A chain of complex64 steps run as one pass over the first step's long
// operand (k_fused2): T1[i, j] = sum_l X[i, l] W[0][j, l] (K1 = S1 entries),
// then T2 = T1 W[1] on the second step's layout of T1 (K2 = S2), and so on
// for nsteps steps, without writing any product but the last.  Every mode
// has extent 2, so each place below is a sum over the set bits of an index.
// A pass is 1024 entries of X (1024 / K1 rows); within it, step q's block row
// bit b and column bit c put its product at pos_row[q][b] + pos_col[q][c]
// (complex entries) of step q + 1's input block [1024 / K rows][K + 2] (the
// first block's rows are the pass's rows); the last step's row bit e and
// column bit c add out_row[e] and out_col[c] to the offset in C, and bit q
// of the pass index adds out_pass[q].  The pass's rows of X are those whose
// row bits lrow[0 .. log2(1024 / K1) - 1] (ascending) vary.  A workgroup runs
// passes 4 r + w (w = 0 .. 3, one per wave) together: bits 0 and 1 of the
// pass index set row bits wbit[0] and wbit[1], and r fills the row bits
// outside hole[0 .. log2(1024 / K1) + 1] (lrow and wbit, ascending) in
// ascending order.
constexpr int kFuseEntries = 1024;
constexpr int kFuseMaxOuter = 48;
constexpr int kFuseMaxChain = 6;
struct Fused2Args {
  const float2 *X;                   // row-major [R, K1]
  const float2 *W[kFuseMaxChain];    // step q's small operand, row-major [K, K] (S rows)
  float2 *C;
  int64_t R;         // a multiple of 1024 / K1; R / (1024 / K1) = 2^nouter passes
  int32_t K1, K2;    // the first and second step's K: 2, 4, 8, 16 or 32 (K <= 8: vector-ALU
                     // phase; 2 only beside K <= 8)
  int32_t K3;        // 0 (a pair), or the last step's K (2, 4 or 8) in a chain of nsteps >= 3
                     // steps whose every K is 2, 4 or 8
  int32_t nsteps;
  int32_t kmid[kFuseMaxChain - 2];  // a chain's middle steps' K (steps 1 .. nsteps - 2)
  int32_t nouter;
  int32_t lrow[9], hole[11], wbit[2];
  int32_t pos_row[kFuseMaxChain - 1][9], pos_col[kFuseMaxChain - 1][8];
  int64_t out_row[9], out_col[8];
  int64_t out_pass[kFuseMaxOuter];
};

// `z` selects complex128 entries (16 bytes) instead of complex64 (8 bytes).
// Writes the pointer table [arena, out, leaves...] to ptab and copies
// blob_bytes (a multiple of 16) of descriptors from pinned host memory to
// blob_dst; one launch per 400 pointers, the blob with the first.
hipError_t launch_header(void **ptab, void *arena, void *out, const void *const *leaves, int32_t num_leaves,
                         const void *blob_src, void *blob_dst, uint64_t blob_bytes, hipStream_t stream);
hipError_t launch_copy(const CopyDesc *descs, int32_t count, int64_t max_count, const void *const *ptab,
                       const int64_t *ints, const SliceDigits &digits, int32_t beta, bool z, hipStream_t stream);
hipError_t launch_copy_tiled(const CopyDesc *desc, int64_t count, const void *const *ptab, const int64_t *ints,
                             const SliceDigits &digits, int32_t beta, bool z, hipStream_t stream);
// max_rs: the largest member's R S (sets the workgroups per member).
hipError_t launch_tiny(const TinyDesc *descs, int32_t count, int64_t max_rs, const void *const *ptab,
                       const RunDev *runs, int32_t beta, bool z, hipStream_t stream);
hipError_t launch_skinny(const StepArgs &a, hipStream_t stream);
hipError_t launch_gemm(const StepArgs &a, hipStream_t stream);
hipError_t launch_skinny_z(const StepArgsZ &a, hipStream_t stream);
hipError_t launch_fused2(const Fused2Args &a, hipStream_t stream);
hipError_t launch_gemm_z(const StepArgsZ &a, hipStream_t stream);

// Peak probes: `blocks` workgroups of 256 threads running `chains` (4 or 8)
// MFMA chains of `iters` steps each (writes blocks * 256 floats to out); a
// copy of n16 16-byte entries with `inflight` (1 or 4) loads per thread in
// flight.  device_cus(): compute units of the current device.
hipError_t launch_probe_mfma(float *out, int64_t blocks, int32_t iters, int32_t chains, hipStream_t stream);
hipError_t launch_probe_copy(const void *src, void *dst, int64_t n16, int32_t pattern, hipStream_t stream);
int32_t device_cus();

// Name of the kernel the last launcher call on this thread enqueued (a split
// K step appends "+k_split_reduce"); "" after clear_kernel_name().
const char *last_kernel_name();
void clear_kernel_name();

}  // namespace tnc
