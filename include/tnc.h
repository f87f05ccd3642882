/*
 * tnc.h - exact tensor-network contraction along a fixed tree, on one
 * MI355X (gfx950) GPU.  C ABI of libtnc.so.
 *
 * The operation (page "Parallelizing Large-Scale Tensor Network Contraction
 * on Multiple GPUs", section 1.1): a network of leaf tensors joined by
 * shared modes is reduced by a binary tree of pairwise steps.  Each step
 * forms C[M, N] = sum over K of A[M, K] * B[N, K], where K are the modes
 * shared by the two operands (summed away) and M, N the modes each keeps.
 * The result is the network's full sum laid out in a caller-given order of
 * the open modes.
 *
 * How it runs: tnc_plan fixes, on the host, the memory order of every tensor
 * by the reverse-tree "lifetime ordering" of section 1.4 (the root takes the
 * requested output order; each operand's order is its product's order
 * restricted to the operand, followed by the reduced modes).  With those
 * orders both operands of every step are stored K-innermost, so every step
 * is a GEMM with no runtime transpose of intermediates.  tnc_plan also
 * decides each step's kernel, groups the many small steps into shared
 * launches, and lays all intermediates out in one arena.  tnc_execute then
 * only enqueues kernels on the caller's stream.
 *
 * Conventions common to all calls:
 *   - Tensors are dense, row-major in their mode order (first mode slowest),
 *     complex64 entries stored as interleaved (float re, float im), or, for a
 *     network declared TNC_C128, complex128 entries as interleaved
 *     (double re, double im).  All buffers of one plan share its dtype.
 *   - Mode labels are 0 .. num_modes-1.  Every mode appears in exactly two
 *     tensors counting the output: two leaves (closed mode, summed) or one
 *     leaf and the output (open mode).
 *   - No function throws; every failure is a tnc_status.  Functions that
 *     return an error leave their outputs untouched.
 *   - The library never allocates device memory.  The caller owns every
 *     device buffer.
 */
#ifndef TNC_H
#define TNC_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  TNC_OK = 0,
  TNC_ERR_INVALID_ARG = 1,        /* NULL pointer, bad option, bad sliced mode, bad id */
  TNC_ERR_INVALID_NETWORK = 2,    /* extent < 1, label out of range, dangling mode,
                                     open mode not on exactly one leaf */
  TNC_ERR_INVALID_TREE = 3,       /* steps != leaves - 1, operand id out of range or reused */
  TNC_ERR_UNSUPPORTED = 4,        /* mode in more than two tensors (hyperedge / batch mode),
                                     a mode repeated inside one leaf, rank > 64,
                                     a size that overflows 64 bits,
                                     a GEMM-class step with m, n or k >= 2^31 */
  TNC_ERR_OUT_OF_MEMORY = 5,      /* planned workspace exceeds options.capacity_bytes */
  TNC_ERR_WORKSPACE_TOO_SMALL = 6,/* tnc_execute got less workspace than planned */
  TNC_ERR_HIP = 7                 /* a HIP runtime call or kernel launch failed */
} tnc_status;

/* Entry type of every buffer of a plan.  C64 steps run on FP32 matrix cores
 * (FP32 accumulation, the precision the page's own kernels use); C128 steps
 * run on FP64 matrix cores for callers that need double precision. */
typedef enum { TNC_C64 = 0, TNC_C128 = 1 } tnc_dtype;

/* Mode-order policy.  LIFETIME: the page's reverse-tree ordering (section
 * 1.4); intermediates are never re-laid.  NAIVE: the ablation baseline of
 * section 1.3 - each product keeps [A's kept modes | B's kept modes] and
 * every operand that is not already [kept | K] is permuted before its GEMM;
 * the root is permuted into the output order at the end. */
typedef enum { TNC_ORDER_LIFETIME = 0, TNC_ORDER_NAIVE = 1 } tnc_order_policy;

/* Kernel class of a step. */
typedef enum { TNC_CLASS_TINY = 0, TNC_CLASS_SKINNY = 1, TNC_CLASS_GEMM = 2 } tnc_kernel_class;

typedef struct tnc_plan_s *tnc_plan_t;

/* The network.  Arrays are read during tnc_plan only (the plan copies them). */
typedef struct {
  int32_t num_modes;
  const int64_t *extents;     /* [num_modes], each >= 1 */
  int32_t num_leaves;         /* >= 1 */
  const int32_t *leaf_rank;   /* [num_leaves] */
  const int32_t *leaf_modes;  /* concatenated mode lists, each in its buffer's row-major order */
  int32_t out_rank;
  const int32_t *out_modes;   /* [out_rank]: the result's mode order */
  tnc_dtype dtype;            /* TNC_C64 or TNC_C128 */
} tnc_network;

/* The tree, in SSA form: leaves are ids 0 .. L-1, step s creates id L + s
 * from operands lhs[s] and rhs[s]; each id is consumed once; the last step
 * creates the root.  Steps execute in list order. */
typedef struct {
  int32_t num_steps;          /* = num_leaves - 1 */
  const int32_t *lhs;
  const int32_t *rhs;
} tnc_tree;

/* Plan options; pass NULL for the defaults shown. */
typedef struct {
  tnc_order_policy order;     /* TNC_ORDER_LIFETIME */
  int32_t num_sliced;         /* 0: number of closed modes fixed per slice */
  const int32_t *sliced_modes;/* NULL: closed modes to slice over; tnc_execute sums the
                                 prod(extents) slices into `out` (page section 1.1) */
  uint64_t align;             /* 256: arena alignment in bytes (power of two, >= 256) */
  uint64_t capacity_bytes;    /* 0: no limit; else fail with OUT_OF_MEMORY above it */
  uint64_t tiny_mnk;          /* 131072: steps with m*n*k <= this and at most tiny_mnk / 4
                                 operand + output entries share grouped launches */
  int32_t max_group;          /* 256: most steps in one grouped launch */
  int32_t precision;          /* TNC_PREC_EXACT: arithmetic of GEMM-class complex64 steps */
  int64_t slice_begin;        /* 0, 0: all slices.  Otherwise tnc_execute runs only slices */
  int64_t slice_end;          /*   slice_begin <= sigma < slice_end (0 <= begin < end <= number of
                                   slices) and leaves their sum in `out`: partial sums that add up to
                                   the whole result, e.g. one range per process or per call */
  int32_t fuse;               /* 1: where a long tensor absorbs a small one (2, 4, 8, 16 or 32
                                 entries of K, as many outputs; 2 only beside K <= 8) and the product
                                 is reduced at once against another such small tensor (and, all K
                                 2, 4 or 8, up to
                                 TNC_FUSE_MAX_STEPS steps in a row), the chain runs in one pass
                                 over the long operand and only its last product is stored
                                 (complex64, exact, lifetime order, every extent a power of two,
                                 long side >= 2^16 rows).  0: every step runs on its own. */
} tnc_plan_options;

/* Arithmetic of the GEMM-class steps of a complex64 plan.  EXACT: FP32
 * matrix cores on the FP32 entries (products exact, FP32 accumulation).
 * BF16X3: each FP32 entry is split into bf16 hi + lo (round to nearest
 * even twice) and each product is hi*hi + hi*lo + lo*hi on the bf16 matrix
 * cores with FP32 accumulation; the dropped lo*lo term and the split leave
 * about 2^-16 relative error per product.  This is the split / emulated
 * precision variant the page lists among the extensions (page 1, the
 * outlook on extended and mixed precision); it is opt-in and never the
 * default.  Complex128 plans accept only EXACT. */
typedef enum { TNC_PREC_EXACT = 0, TNC_PREC_BF16X3 = 1 } tnc_precision;

/* Fill `opts` with the defaults. */
void tnc_plan_options_default(tnc_plan_options *opts);

/*
 * Build a plan.  Host only: no HIP call is made.  On success *plan owns a
 * copy of everything it needs.
 * Errors: INVALID_ARG, INVALID_NETWORK, INVALID_TREE, UNSUPPORTED,
 * OUT_OF_MEMORY (see tnc_status).
 */
tnc_status tnc_plan(const tnc_network *net, const tnc_tree *tree, const tnc_plan_options *opts,
                    tnc_plan_t *plan);

void tnc_plan_destroy(tnc_plan_t plan);

/* Device workspace the plan needs, in bytes (header + arena). */
tnc_status tnc_plan_workspace_bytes(tnc_plan_t plan, uint64_t *bytes);

typedef struct {
  int32_t num_leaves, num_steps, num_groups;
  int32_t nodes_tiny, nodes_skinny, nodes_gemm, nodes_split;
  int32_t nodes_interleaved;     /* steps whose output interleaves A- and B-modes */
  int32_t min_inner_run;         /* shortest innermost output run, in entries */
  int32_t staged_leaves;         /* leaves copied into the arena before use */
  int32_t relayouts;             /* operand re-layouts of intermediates (NAIVE only) */
  int32_t root_permute;          /* 1 if the root is permuted into `out` (NAIVE) */
  int64_t num_slices;            /* product of sliced extents (1 if unsliced) */
  double flops;                  /* sum of 8 m n k over steps of one slice */
  double flops_unsliced;         /* same for the tree with nothing sliced */
  double bytes;                  /* sum of 8 (m k + n k + m n) over steps of one slice */
  uint64_t max_intermediate;     /* largest step output, in entries */
  uint64_t header_bytes;         /* workspace prefix holding kernel descriptors */
  uint64_t arena_bytes;          /* arena high-water mark */
  uint64_t workspace_bytes;      /* header_bytes + arena_bytes */
  int32_t fused_pairs;           /* fused chains (2 .. TNC_FUSE_MAX_STEPS steps) run as one pass
                                    each (tnc_plan_options.fuse) */
} tnc_plan_stats;

tnc_status tnc_plan_stats_get(tnc_plan_t plan, tnc_plan_stats *stats);

/* Planned mode order of SSA tensor `id` (0 .. L+S-1).  `modes` must hold 64
 * entries; *rank receives the order's length. */
tnc_status tnc_plan_tensor_order(tnc_plan_t plan, int32_t id, int32_t *modes, int32_t *rank);

/* Arena offset (bytes, from the arena start) of SSA tensor `id`: a staged
 * leaf copy or an intermediate.  UINT64_MAX: read in place (leaf), written
 * to `out` (root) or never stored (a fused chain's products but the last). */
tnc_status tnc_plan_tensor_offset(tnc_plan_t plan, int32_t id, uint64_t *offset);

typedef struct {
  int32_t lhs, rhs, out;         /* SSA ids */
  int32_t kernel_class;          /* tnc_kernel_class */
  int32_t swap;                  /* 1: the kernel's row operand is B (C is produced transposed) */
  int32_t group;                 /* launch group */
  int32_t splits;                /* K split count (> 1: partial sums in scratch, then a reduce) */
  int32_t row_runs, col_runs;    /* number of output runs per side */
  int32_t inner_run;             /* entries in the innermost output run */
  int32_t interleaved;
  int32_t copy_a, copy_b;        /* operand copied/permuted into the arena before the step */
  int64_t m, n, k;
  uint64_t a_off, b_off, c_off;  /* arena offsets of the GEMM operands / product
                                    (UINT64_MAX: leaf in place or `out`) */
  uint64_t scratch_off, scratch_bytes;
  int32_t fused_with;            /* fused chains (all their steps run in the last step's launch):
                                    for an earlier step the chain's last step, for the last step
                                    the chain's first; -1 if not fused */
} tnc_node_info;

tnc_status tnc_plan_node(tnc_plan_t plan, int32_t step, tnc_node_info *info);

/* A fused chain's pass tables (index 0 .. fused_pairs - 1, in step order),
 * for inspection and host-side checks.  The chain runs steps step[0 ..
 * nsteps - 1] (2 .. TNC_FUSE_MAX_STEPS; unused entries -1): each step's long
 * operand is the previous step's product (the first step's: its lhs for
 * longop = 0, else its rhs) and its small operand has k[q] x k[q] entries
 * (2, 4, 8, 16 or 32, 2 only beside k <= 8; in chains of three or more
 * every k is 2, 4 or 8).  Every index is a sum
 * of one offset per set bit.  A pass takes 1024 entries of the first long
 * operand X (row-major [rows, k[0]]): its local row rho (0 .. 1024/k[0] - 1)
 * is X row spread(rho) + round part + wave part, where spread puts bit j of
 * rho at row bit lrow[j]; the workgroup's four passes w = 0 .. 3 add
 * (w & 1) << wbit[0] and (w >> 1) << wbit[1]; a round index fills the row
 * bits outside hole[] (lrow and wbit, ascending) in ascending order.  Step
 * q's product of its block row l and column j goes to complex entry
 * sum pos_row[q][bits of l] + sum pos_col[q][bits of j] of step q + 1's block
 * [1024/k[q + 1] rows][k[q + 1] + 2] (step 0's block rows are the pass's rows
 * rho); the last step's product of block row l and column j goes to offset
 * sum out_row[bits of l] + sum out_col[bits of j] + (w & 1) out_pass[0]
 * + (w >> 1) out_pass[1] + sum out_pass[2 + q] over bits q of the round.
 * Errors: INVALID_ARG (no such chain). */
#define TNC_FUSE_MAX_STEPS 6
typedef struct {
  int32_t nsteps;
  int32_t step[TNC_FUSE_MAX_STEPS];
  int32_t longop[TNC_FUSE_MAX_STEPS];
  int32_t k[TNC_FUSE_MAX_STEPS];
  int64_t rows;
  int32_t nouter;
  int32_t lrow[9], hole[11], wbit[2];
  int32_t pos_row[TNC_FUSE_MAX_STEPS - 1][9], pos_col[TNC_FUSE_MAX_STEPS - 1][8];
  int64_t out_row[9], out_col[8];
  int64_t out_pass[48];
} tnc_fused_info;

tnc_status tnc_plan_fused(tnc_plan_t plan, int32_t index, tnc_fused_info *info);

/*
 * Run the plan.
 *   leaves[L]   device pointers to the leaf buffers (declared orders); a leaf
 *               that a fused chain reads in place as its long operand must be
 *               16-byte aligned (INVALID_ARG otherwise, before any launch)
 *   out         device pointer, prod(out extents) entries of the plan's dtype,
 *               overwritten
 *   workspace   device pointer, >= tnc_plan_workspace_bytes, 256-byte aligned
 *   stream      hipStream_t to enqueue on (NULL = the default stream)
 * Asynchronous: returns once the work is enqueued; no host synchronisation
 * and no device allocation.  The first call on a plan outside stream capture
 * allocates a pinned host copy of the plan's step descriptors (a few KB to a
 * few MB, freed by tnc_plan_destroy) which a kernel then reads on every call;
 * a call captured into a graph before that copy exists records an ordinary
 * host-to-device copy of the descriptors instead.  The caller keeps the plan,
 * leaves, out and workspace alive until the stream has finished; a HIP graph
 * that captured a call reads the plan's host descriptors on every replay, so
 * the plan must also outlive every such graph.  One plan may run concurrently on different
 * streams given distinct workspaces and outputs.  A sliced plan loops over its
 * slices (all of them, or options.slice_begin .. slice_end - 1) and leaves
 * their sum in `out`.  Slice sigma fixes the sliced modes to the digits of
 * sigma in the mixed radix of their extents, the first sliced mode most
 * significant.
 * Errors: INVALID_ARG, WORKSPACE_TOO_SMALL, HIP (pinned allocation or launch
 * failure; faults surface at the caller's next synchronisation).
 */
tnc_status tnc_execute(tnc_plan_t plan, const void *const *leaves, void *out, void *workspace,
                       uint64_t workspace_bytes, void *stream);

/*
 * Profiling: run the plan like tnc_execute, with a pair of HIP events around
 * every launch, and report each launch's kernel and time.  Synchronous: it
 * waits for the stream after every slice to read the events (so it is for
 * measurement, not for production runs), and it creates HIP events.
 *   ops[max_ops]  caller-owned records, one per launch of the plan's program
 *                 plus one (index 0) for the descriptor header; at most
 *                 3 * num_steps + 2 are needed
 *   *num_ops      records written
 * A launch of a sliced plan runs once per slice: `ms` sums them and
 * `launches` counts them.  Errors: INVALID_ARG (also when max_ops is too
 * small; tnc_last_error says how many are needed), WORKSPACE_TOO_SMALL, HIP.
 */
typedef enum {
  TNC_OP_COPY = 0,          /* permuting copies (leaf staging, naive-order re-layouts) */
  TNC_OP_TINY_GROUP = 1,    /* one grouped launch of small steps */
  TNC_OP_SKINNY = 2,        /* one step with a side of at most 16 */
  TNC_OP_GEMM = 3,          /* one matrix-core GEMM step */
  TNC_OP_COPY_TILED = 4,    /* one large permuting copy through LDS tiles */
  TNC_OP_HEADER = 5,        /* pointer table and descriptor upload */
  TNC_OP_FUSED = 6          /* one pass running a fused chain of steps (`step`: its last) */
} tnc_op_kind;

typedef struct {
  int32_t kind;             /* tnc_op_kind */
  int32_t step;             /* the step of a SKINNY, GEMM or FUSED launch, else -1 */
  int32_t count;            /* copies or steps in the launch */
  int32_t launches;         /* times the launch ran */
  double ms;                /* its total time over those runs */
  char kernel[64];          /* the kernel the launcher chose, e.g. "k_cgemm_tile<128,128>" */
} tnc_op_timing;

tnc_status tnc_execute_timed(tnc_plan_t plan, const void *const *leaves, void *out, void *workspace,
                             uint64_t workspace_bytes, void *stream, tnc_op_timing *ops, int32_t max_ops,
                             int32_t *num_ops);

/*
 * Run the plan without allocating anything: for callers that cannot allocate
 * (code under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc).  Same arguments and results as tnc_execute, except that the
 * workspace is a static array inside the library, one copy per GPU of
 * TNC_NOALLOC_MAX_WORKSPACE_BYTES bytes, held from the library's load until
 * the process ends.  The call makes no hipMalloc, hipFree, hipHostMalloc or
 * other allocation: if the plan already has its pinned descriptor copy (from
 * an earlier tnc_execute) a kernel reads it, otherwise the descriptors are
 * uploaded by a host-to-device copy from the plan's own host memory.  The
 * first call on a device looks up that device's copy of the array (with the
 * device current).  Nothing in the workspace needs to start at zero: every
 * region a call reads was written earlier in the same call.  All calls on
 * one GPU share its array, so two calls whose work overlaps in time on the
 * same GPU (other streams, other threads) race and corrupt each other's
 * results; serialise them.
 * Errors: INVALID_ARG, WORKSPACE_TOO_SMALL (the plan's workspace exceeds
 * TNC_NOALLOC_MAX_WORKSPACE_BYTES; checked before any HIP call), HIP.
 */
#define TNC_NOALLOC_MAX_WORKSPACE_BYTES (UINT64_C(64) << 20)
tnc_status tnc_execute_noalloc(tnc_plan_t plan, const void *const *leaves, void *out, void *stream);

/*
 * Distribution schedule over P GPUs (host only; launches nothing).
 *
 * "Parallelizing Large-Scale Tensor Network Contraction on Multiple GPUs",
 * section 1.5: an intermediate larger than a threshold (8 GiB on the page)
 * is split over P GPUs on the shortest prefix of its lifetime order whose
 * extents multiply to at least P, so each GPU holds one contiguous block;
 * every step is tagged Activate, Keep, Redistribute or Gather.  Section 1.6:
 * along each chain of split tensors a one-dimensional dynamic program picks,
 * before every step, keeping the current split (allowed while none of its
 * modes is reduced by the step) or an All-to-All re-split onto the fresh
 * prefix of the tensor's order that avoids the step's reduced modes, under
 * the cost t = t_gemm + t_comm:
 *   t_gemm = count * max(bytes / B_dev, 8 m n k / F_dev) for the GPU's
 *            sub-GEMMs (m, n, k), bytes = entry size * (mk + nk + mn);
 *   t_comm = V / B_net + lambda * n_blk, V the bytes one GPU sends and
 *            n_blk the contiguous blocks they fall into (a re-split moves
 *            P - 1 pieces of |T| / P^2; blocks end where the new split modes
 *            cut the shard's layout).
 * The page's formulas are stripped; these are readings of its words.  The
 * remaining rules are this library's: leaves stay replicated; a step whose
 * operands are both split gathers the smaller one (all-gather); a small
 * output (or the root) of a split operand is all-gathered, or all-reduced
 * when split modes were reduced (partial sums).  Ties in the program keep
 * the earlier choice; any optimal schedule is correct.
 */
typedef enum {
  TNC_DIST_REPLICATED = 0,   /* replicated operands, output not split: every GPU runs the whole step */
  TNC_DIST_ACTIVATE = 1,     /* replicated operands, output above the threshold: each GPU computes its block */
  TNC_DIST_KEEP = 2,         /* the split operand keeps its split; local GEMM, no communication */
  TNC_DIST_REDISTRIBUTE = 3, /* the split operand is re-split (All-to-All) before the local GEMM */
  TNC_DIST_GATHER = 4        /* output not split: gathered (or all-reduced) after the local GEMM */
} tnc_dist_tag;

typedef struct {
  int32_t num_gpus;          /* P, 1 .. 65536 (1: nothing is split) */
  uint64_t threshold_bytes;  /* step outputs above this many bytes are split */
  double hbm_bytes_per_s;    /* B_dev, > 0 */
  double flops_per_s;        /* F_dev (matrix peak for the plan's dtype), > 0 */
  double net_bytes_per_s;    /* B_net: bytes per second one GPU sends to its peers, > 0 */
  double latency_s;          /* lambda: cost of one message block, >= 0 */
} tnc_dist_options;

typedef struct {
  int32_t tag;               /* tnc_dist_tag */
  int32_t dist_operand;      /* 0 lhs or 1 rhs: the split operand the step continues; -1 none */
  int32_t gathered_operand;  /* 0 or 1: a second split operand all-gathered before the step; -1 none */
  int32_t num_dist;          /* modes the output is split on (0: not split) */
  int32_t dist_modes[16];    /* those modes, in the output's planned order */
  int32_t num_local;         /* modes the local GEMM is split on (the operand's split after any */
  int32_t local_modes[16];   /*   re-split, or the activated output's split); one GPU runs the step */
                             /*   with these fixed, local_count times (0: whole step) */
  int64_t local_m;           /* one GPU's sub-GEMM: lhs-side extent, */
  int64_t local_n;           /*   rhs-side extent, */
  int64_t local_k;           /*   reduced extent, */
  int64_t local_count;       /*   and how many such sub-GEMMs it runs */
  double t_gemm;             /* seconds of local GEMM (cost model) */
  double t_comm;             /* seconds of communication charged to this step */
} tnc_dist_step;

/* MI355X defaults for an 8-GPU node: P = 8, threshold 8 GiB, B_dev 8 TB/s,
 * F_dev 157.3 TFLOP/s (C64) or 78.6 (C128), B_net 537.6 GB/s (7 xGMI links
 * of 76.8 GB/s per direction), lambda 5 us.  Errors: INVALID_ARG. */
tnc_status tnc_dist_options_default(tnc_dist_options *opts, tnc_dtype dtype);

/* Compute the schedule of `plan` (its unsliced tree).  steps[num_steps] is
 * caller-owned and fully written; *total_s = sum of t_gemm + t_comm.
 * Errors: INVALID_ARG (NULL, options out of range), UNSUPPORTED (a chain
 * with no feasible split, e.g. a split tensor whose surviving modes cannot
 * be cut P ways); outputs are untouched on error. */
tnc_status tnc_plan_distribute(tnc_plan_t plan, const tnc_dist_options *opts, tnc_dist_step *steps,
                               double *total_s);

/*
 * Measurement probe (not part of a contraction): the current device's
 * sustained FP32 matrix-core rate (4 or 8 independent chains of the 32x32x2
 * FP32 MFMA per wave, 2 or 4 waves per SIMD, no memory traffic) and HBM copy
 * rate (16-byte copy of bytes / 2 from the first half of `buffer` to the
 * second: grid-stride with 1 or 4 loads in flight per thread, or one
 * contiguous 256 KiB chunk per workgroup with plain or nontemporal loads and
 * stores), each the best over those launch shapes of three timed runs after
 * one untimed run.  `buffer`: caller-owned device memory of `bytes` >= 64 MiB,
 * 256-byte aligned, overwritten.  Synchronous.  These are the measured
 * denominators beside the published peaks (157.3 TFLOP/s, 8 TB/s).
 * Errors: INVALID_ARG, HIP.
 */
tnc_status tnc_probe_peaks(void *buffer, uint64_t bytes, void *stream, double *mfma_tflops, double *copy_gbps);

/* Static text for a status code. */
const char *tnc_status_string(tnc_status status);

/* Detail of the most recent failure on the calling thread (e.g. which launch
 * failed and the HIP error string), or "" if none.  Valid until the thread's
 * next tnc_* call. */
const char *tnc_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* TNC_H */
