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
