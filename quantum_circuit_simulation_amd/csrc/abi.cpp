// extern "C" entry points of libtnc.so (declared in include/tnc.h) and the
// executor that turns a plan's launch program into kernel launches.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <mutex>
#include <new>
#include <string>
#include <vector>

#include "kernels.hpp"
#include "plan.hpp"

struct tnc_plan_s {
  tnc::PlanImpl impl;
  // pinned host copy of the descriptor blob (blob_bytes, zero padded), made by
  // the first tnc_execute and read by the upload kernel on every call
  std::mutex pin_mu;
  void *blob_pinned = nullptr;
  ~tnc_plan_s() {
    if (blob_pinned) (void)hipHostFree(blob_pinned);
  }
};

namespace {

thread_local std::string g_last_error;

bool debug_sync() {
  static int v = -1;
  if (v < 0) {
    const char *e = std::getenv("TNC_DEBUG_SYNC");
    v = (e && e[0] == '1') ? 1 : 0;
  }
  return v == 1;
}

tnc_status check(hipError_t e, hipStream_t stream, const char *what) {
  if (e == hipSuccess && debug_sync()) e = hipStreamSynchronize(stream);
  if (e != hipSuccess) {
    g_last_error = std::string(what) + ": " + hipGetErrorString(e);
    return TNC_ERR_HIP;
  }
  return TNC_OK;
}

static_assert(tnc::kFuseEntries == tnc::kFusePassEntries && tnc::kFuseMaxOuter == tnc::kFuseOuterMax &&
                  tnc::kFuseMaxChain == tnc::kFuseMaxSteps && TNC_FUSE_MAX_STEPS == tnc::kFuseMaxSteps,
              "fused-pair pass size and table length agree between planner and kernel");
#define TNC_SAME_TABLE(f) \
  (sizeof(tnc_fused_info::f) == sizeof(tnc::FusedChain::f) && sizeof(tnc::Fused2Args::f) == sizeof(tnc::FusedChain::f))
static_assert(TNC_SAME_TABLE(lrow) && TNC_SAME_TABLE(hole) && TNC_SAME_TABLE(wbit) && TNC_SAME_TABLE(pos_row) &&
                  TNC_SAME_TABLE(pos_col) && TNC_SAME_TABLE(out_row) && TNC_SAME_TABLE(out_col) &&
                  TNC_SAME_TABLE(out_pass),
              "the fused chain's per-bit tables have one layout in the planner, the ABI and the kernel arguments");
#undef TNC_SAME_TABLE

const char *op_name(int kind) {
  switch (kind) {
    case tnc::OP_COPY: return "k_copy launch";
    case tnc::OP_COPY_TILED: return "k_copy_tiled launch";
    case tnc::OP_TINY_GROUP: return "k_tiny launch";
    case tnc::OP_SKINNY: return "k_skinny launch";
    case tnc::OP_GEMM: return "k_cgemm launch";
    case tnc::OP_FUSED: return "k_fused2 launch";
  }
  return "launch";
}

}  // namespace

extern "C" {

void tnc_plan_options_default(tnc_plan_options *o) {
  if (!o) return;
  std::memset(o, 0, sizeof(*o));
  o->order = TNC_ORDER_LIFETIME;
  o->num_sliced = 0;
  o->sliced_modes = nullptr;
  o->align = 256;
  o->capacity_bytes = 0;
  o->tiny_mnk = 131072;
  o->max_group = 256;
  o->precision = TNC_PREC_EXACT;
  o->slice_begin = 0;
  o->slice_end = 0;
  o->fuse = 1;
}

tnc_status tnc_plan(const tnc_network *net, const tnc_tree *tree, const tnc_plan_options *opts,
                    tnc_plan_t *plan) {
  g_last_error.clear();
  if (!plan) return TNC_ERR_INVALID_ARG;
  tnc_plan_s *p = new (std::nothrow) tnc_plan_s();
  if (!p) return TNC_ERR_OUT_OF_MEMORY;
  tnc_status st;
  try {
    st = tnc::build_plan(net, tree, opts, &p->impl);
  } catch (const std::bad_alloc &) {
    st = TNC_ERR_OUT_OF_MEMORY;
  } catch (...) {
    st = TNC_ERR_INVALID_ARG;
  }
  if (st != TNC_OK) {
    delete p;
    return st;
  }
  // the plan keeps no pointer into the caller's arrays
  p->impl.opts.sliced_modes = nullptr;
  *plan = p;
  return TNC_OK;
}

void tnc_plan_destroy(tnc_plan_t plan) { delete plan; }

tnc_status tnc_plan_workspace_bytes(tnc_plan_t plan, uint64_t *bytes) {
  if (!plan || !bytes) return TNC_ERR_INVALID_ARG;
  *bytes = plan->impl.stats.workspace_bytes;
  return TNC_OK;
}

tnc_status tnc_plan_stats_get(tnc_plan_t plan, tnc_plan_stats *stats) {
  if (!plan || !stats) return TNC_ERR_INVALID_ARG;
  *stats = plan->impl.stats;
  return TNC_OK;
}

tnc_status tnc_plan_tensor_order(tnc_plan_t plan, int32_t id, int32_t *modes, int32_t *rank) {
  if (!plan || !modes || !rank) return TNC_ERR_INVALID_ARG;
  const auto &p = plan->impl;
  if (id < 0 || id >= p.L + p.S) return TNC_ERR_INVALID_ARG;
  const auto &o = p.order[id];
  if ((int)o.size() > tnc::kMaxRank) return TNC_ERR_UNSUPPORTED;
  for (size_t i = 0; i < o.size(); ++i) modes[i] = o[i];
  *rank = (int32_t)o.size();
  return TNC_OK;
}

tnc_status tnc_plan_tensor_offset(tnc_plan_t plan, int32_t id, uint64_t *offset) {
  if (!plan || !offset) return TNC_ERR_INVALID_ARG;
  const auto &p = plan->impl;
  if (id < 0 || id >= p.L + p.S) return TNC_ERR_INVALID_ARG;
  *offset = p.tensor_off[id];
  return TNC_OK;
}

tnc_status tnc_plan_node(tnc_plan_t plan, int32_t step, tnc_node_info *info) {
  if (!plan || !info) return TNC_ERR_INVALID_ARG;
  const auto &p = plan->impl;
  if (step < 0 || step >= p.S) return TNC_ERR_INVALID_ARG;
  const tnc::Node &n = p.nodes[step];
  std::memset(info, 0, sizeof(*info));
  info->lhs = n.lhs;
  info->rhs = n.rhs;
  info->out = n.out;
  info->kernel_class = n.cls;
  info->swap = n.swap;
  info->group = n.group;
  info->splits = n.splits;
  info->row_runs = (int32_t)n.row_runs.size();
  info->col_runs = (int32_t)n.col_runs.size();
  info->inner_run = (int32_t)(n.inner_run > INT32_MAX ? INT32_MAX : n.inner_run);
  info->interleaved = n.interleaved;
  info->copy_a = n.copy_a;
  info->copy_b = n.copy_b;
  info->m = n.m;
  info->n = n.n;
  info->k = n.k;
  info->a_off = n.a_off;
  info->b_off = n.b_off;
  info->c_off = n.c_off;
  info->scratch_off = n.scratch_off;
  info->scratch_bytes = n.scratch_bytes;
  // earlier steps of a fused chain: the step whose launch runs them (the
  // chain's last); the last step: the chain's first
  int32_t w = -1;
  if (n.fuse_next >= 0) {
    w = n.fuse_next;
    while (p.nodes[w].fuse_next >= 0) w = p.nodes[w].fuse_next;
  } else if (n.fuse_prev >= 0) {
    w = n.fuse_prev;
    while (p.nodes[w].fuse_prev >= 0) w = p.nodes[w].fuse_prev;
  }
  info->fused_with = w;
  return TNC_OK;
}

tnc_status tnc_plan_fused(tnc_plan_t plan, int32_t index, tnc_fused_info *info) {
  if (!plan || !info) return TNC_ERR_INVALID_ARG;
  const auto &p = plan->impl;
  if (index < 0 || index >= (int32_t)p.fused.size()) return TNC_ERR_INVALID_ARG;
  const tnc::FusedChain &f = p.fused[index];
  std::memset(info, 0, sizeof(*info));
  info->nsteps = f.nsteps;
  for (int q = 0; q < tnc::kFuseMaxSteps; ++q) {
    info->step[q] = q < f.nsteps ? f.step[q] : -1;
    info->longop[q] = f.longop[q];
    info->k[q] = f.k[q];
  }
  info->rows = f.rows;
  info->nouter = f.nouter;
  std::memcpy(info->hole, f.hole, sizeof(f.hole));
  std::memcpy(info->lrow, f.lrow, sizeof(f.lrow));
  std::memcpy(info->pos_row, f.pos_row, sizeof(f.pos_row));
  std::memcpy(info->pos_col, f.pos_col, sizeof(f.pos_col));
  std::memcpy(info->out_row, f.out_row, sizeof(f.out_row));
  std::memcpy(info->out_col, f.out_col, sizeof(f.out_col));
  info->wbit[0] = f.wbit[0];
  info->wbit[1] = f.wbit[1];
  static_assert(sizeof(info->out_pass) / sizeof(info->out_pass[0]) == tnc::kFuseOuterMax, "out_pass length");
  for (int i = 0; i < tnc::kFuseOuterMax; ++i) info->out_pass[i] = f.out_pass[i];
  return TNC_OK;
}

}  // extern "C"

namespace {

// Per-launch timing for tnc_execute_timed: an event pair around every
// launch of the program, read back after each slice.
struct OpTimer {
  std::vector<hipEvent_t> ev;   // 2 per op: [header, program ops...]
  std::vector<tnc_op_timing> *ops = nullptr;
  hipError_t err = hipSuccess;
  ~OpTimer() {
    for (hipEvent_t e : ev)
      if (e) (void)hipEventDestroy(e);
  }
  void record(size_t i, int end, hipStream_t s) {
    if (err == hipSuccess) err = hipEventRecord(ev[2 * i + end], s);
  }
  // after a slice: wait, add each op's time, keep its kernel name
  void collect(hipStream_t s) {
    if (err == hipSuccess) err = hipStreamSynchronize(s);
    for (size_t i = 0; err == hipSuccess && i < ops->size(); ++i) {
      float ms = 0;
      err = hipEventElapsedTime(&ms, ev[2 * i], ev[2 * i + 1]);
      (*ops)[i].ms += ms;
      (*ops)[i].launches += 1;
    }
  }
};

// Runs `plan` with its workspace at `workspace`.  may_pin: the first call on
// the plan outside stream capture may allocate the pinned descriptor copy;
// without it, a plan that has no pinned copy yet uploads its descriptors
// with a host-to-device copy from the plan's own host memory.
tnc_status run_plan(tnc_plan_t plan, const void *const *leaves, void *out, void *workspace,
                    uint64_t workspace_bytes, void *stream_ptr, bool may_pin, OpTimer *tm = nullptr) {
  const tnc::PlanImpl &p = plan->impl;
  // an error left behind by an earlier, unrelated HIP call is not ours
  (void)hipGetLastError();
  for (int32_t l = 0; l < p.L; ++l)
    if (!leaves[l]) return TNC_ERR_INVALID_ARG;
  // a fused chain reads its long operand with 16-byte loads; a leaf read in
  // place must be 16-byte aligned (checked before anything is enqueued)
  for (const auto &f : p.fused) {
    const tnc::Node &n1 = p.nodes[f.step[0]];
    const int32_t t = f.longop[0] == 0 ? n1.lhs : n1.rhs;
    const int32_t copied = f.longop[0] == 0 ? n1.copy_a : n1.copy_b;
    if (t < p.L && !copied && (reinterpret_cast<uintptr_t>(leaves[t]) & 15) != 0) {
      g_last_error = "leaf " + std::to_string(t) + " is the long operand of a fused chain and must be 16-byte "
                     "aligned (or plan with fuse = 0)";
      return TNC_ERR_INVALID_ARG;
    }
  }
  if (workspace_bytes < p.stats.workspace_bytes) return TNC_ERR_WORKSPACE_TOO_SMALL;
  if (!workspace || (reinterpret_cast<uintptr_t>(workspace) & 255) != 0) return TNC_ERR_INVALID_ARG;
  hipStream_t stream = reinterpret_cast<hipStream_t>(stream_ptr);

  char *ws = static_cast<char *>(workspace);
  void **ptab = reinterpret_cast<void **>(ws);
  char *blob = ws + p.ptab_bytes;
  char *arena = ws + p.header_bytes;

  // The pinned descriptor copy is made by the first call outside stream
  // capture; a call captured before it exists records a plain copy from the
  // plan's host memory instead (a memcpy node of the graph).
  const void *pinned = nullptr;
  {
    std::lock_guard<std::mutex> lock(plan->pin_mu);
    if (!plan->blob_pinned && may_pin) {
      hipStreamCaptureStatus cs = hipStreamCaptureStatusNone;
      if (hipStreamIsCapturing(stream, &cs) != hipSuccess) {
        (void)hipGetLastError();
        cs = hipStreamCaptureStatusActive;
      }
      if (cs == hipStreamCaptureStatusNone) {
        void *h = nullptr;
        hipError_t e = hipHostMalloc(&h, p.blob_bytes, hipHostMallocDefault);
        if (e != hipSuccess || !h) {
          (void)hipGetLastError();
          g_last_error = std::string("pinned descriptor copy (hipHostMalloc): ") + hipGetErrorString(e);
          return TNC_ERR_HIP;
        }
        std::memset(h, 0, p.blob_bytes);
        std::memcpy(h, p.blob.data(), p.blob.size());
        plan->blob_pinned = h;
      }
    }
    pinned = plan->blob_pinned;
  }
  tnc_status st;
  if (tm) tm->record(0, 0, stream);
  if (pinned) {
    st = check(tnc::launch_header(ptab, arena, out, leaves, p.L, pinned, blob, p.blob_bytes, stream), stream,
               "k_header launch");
  } else {
    st = check(hipMemcpyAsync(blob, p.blob.data(), p.blob.size(), hipMemcpyHostToDevice, stream), stream,
               "descriptor upload (hipMemcpyAsync)");
    if (st == TNC_OK)
      st = check(tnc::launch_header(ptab, arena, out, leaves, p.L, nullptr, blob, 0, stream), stream,
                 "k_header launch");
  }
  if (st != TNC_OK) return st;
  if (tm) tm->record(0, 1, stream);

  const auto *runs = reinterpret_cast<const tnc::RunDev *>(blob + p.blob_runs);
  const auto *cdesc = reinterpret_cast<const tnc::CopyDesc *>(blob + p.blob_copies);
  const auto *tdesc = reinterpret_cast<const tnc::TinyDesc *>(blob + p.blob_tiny);
  const auto *ints = reinterpret_cast<const int64_t *>(blob + p.blob_ints);

  auto resolve = [&](int32_t buf, uint64_t off_bytes) -> char * {
    if (buf == tnc::kBufArena) return arena + off_bytes;
    if (buf == tnc::kBufOut) return static_cast<char *>(out) + off_bytes;
    return const_cast<char *>(static_cast<const char *>(leaves[buf - tnc::kBufLeaf0])) + off_bytes;
  };
  auto operand = [&](const tnc::Node &nd, int w) -> const void * {
    int32_t t = w == 0 ? nd.lhs : nd.rhs;
    int32_t copy = w == 0 ? nd.copy_a : nd.copy_b;
    uint64_t off = w == 0 ? nd.a_off : nd.b_off;
    if (copy || t >= p.L) return arena + off;
    return leaves[t];
  };
  const bool z = p.dtype == TNC_C128;

  const int64_t s_begin = p.slice_begin, s_end = p.slice_end;
  tnc::SliceDigits sd{};
  sd.n = (int32_t)p.slice_extents.size();
  for (int64_t sigma = s_begin; sigma < s_end; ++sigma) {
    // digits of sigma over the sliced extents, first sliced mode most significant
    int64_t r = sigma;
    for (int t = sd.n - 1; t >= 0; --t) {
      sd.digit[t] = (int32_t)(r % p.slice_extents[t]);
      r /= p.slice_extents[t];
    }
    const int32_t beta = sigma > s_begin ? 1 : 0;
    for (size_t oi = 0; oi < p.program.size(); ++oi) {
      const tnc::Op &op = p.program[oi];
      hipError_t e = hipSuccess;
      if (tm) {
        tm->record(oi + 1, 0, stream);
        tnc::clear_kernel_name();
      }
      switch (op.kind) {
        case tnc::OP_COPY:
          e = tnc::launch_copy(cdesc + op.first, op.count, op.max_count, ptab, ints, sd, beta, z, stream);
          break;
        case tnc::OP_COPY_TILED:
          e = tnc::launch_copy_tiled(cdesc + op.first, op.max_count, ptab, ints, sd, beta, z, stream);
          break;
        case tnc::OP_TINY_GROUP:
          e = tnc::launch_tiny(tdesc + op.first, op.count, op.max_count, ptab, runs, beta, z, stream);
          break;
        case tnc::OP_SKINNY:
        case tnc::OP_GEMM: {
          const tnc::Node &nd = p.nodes[op.first];
          tnc::StepArgsT<float2> a{};
          a.X = reinterpret_cast<const float2 *>(operand(nd, nd.swap ? 1 : 0));
          a.Y = reinterpret_cast<const float2 *>(operand(nd, nd.swap ? 0 : 1));
          a.C = reinterpret_cast<float2 *>(nd.c_off == tnc::kNone ? resolve(tnc::kBufOut, 0)
                                                                   : resolve(tnc::kBufArena, nd.c_off));
          a.R = nd.swap ? nd.n : nd.m;
          a.S = nd.swap ? nd.m : nd.n;
          a.K = nd.k;
          a.runs = runs + nd.runs_index;
          a.nrr = (int32_t)nd.row_runs.size();
          a.ncr = (int32_t)nd.col_runs.size();
          a.beta = (nd.is_root && !p.root_permute) ? beta : 0;
          a.splits = nd.splits;
          a.scratch = nd.splits > 1 ? reinterpret_cast<float2 *>(arena + nd.scratch_off) : nullptr;
          a.prec = p.opts.precision;
          a.pow2_runs = 1;
          for (const auto *side : {&nd.row_runs, &nd.col_runs})
            for (const auto &r : *side)
              if (r.size < 1 || (r.size & (r.size - 1)) != 0) a.pow2_runs = 0;
          if (z) {
            // same fields, complex128 entries
            tnc::StepArgsZ az{};
            az.X = reinterpret_cast<const double2 *>(a.X);
            az.Y = reinterpret_cast<const double2 *>(a.Y);
            az.C = reinterpret_cast<double2 *>(a.C);
            az.R = a.R;
            az.S = a.S;
            az.K = a.K;
            az.runs = a.runs;
            az.nrr = a.nrr;
            az.ncr = a.ncr;
            az.beta = a.beta;
            az.splits = a.splits;
            az.scratch = reinterpret_cast<double2 *>(a.scratch);
            az.pow2_runs = a.pow2_runs;
            e = op.kind == tnc::OP_GEMM ? tnc::launch_gemm_z(az, stream) : tnc::launch_skinny_z(az, stream);
          } else {
            e = op.kind == tnc::OP_GEMM ? tnc::launch_gemm(a, stream) : tnc::launch_skinny(a, stream);
          }
          break;
        }
        case tnc::OP_FUSED: {
          const tnc::FusedChain &f = p.fused[op.first];
          const int ns = f.nsteps;
          const tnc::Node &n1 = p.nodes[f.step[0]], &nl = p.nodes[f.step[ns - 1]];
          tnc::Fused2Args fa{};
          fa.X = reinterpret_cast<const float2 *>(operand(n1, f.longop[0]));
          for (int q = 0; q < ns; ++q)
            fa.W[q] = reinterpret_cast<const float2 *>(operand(p.nodes[f.step[q]], 1 - f.longop[q]));
          fa.C = reinterpret_cast<float2 *>(resolve(tnc::kBufArena, nl.c_off));
          fa.R = f.rows;
          fa.K1 = f.k[0];
          fa.K2 = f.k[1];
          fa.K3 = ns > 2 ? f.k[ns - 1] : 0;
          fa.nsteps = ns;
          for (int q = 1; q + 1 < ns; ++q) fa.kmid[q - 1] = f.k[q];
          fa.nouter = f.nouter;
          fa.wbit[0] = f.wbit[0];
          fa.wbit[1] = f.wbit[1];
          std::memcpy(fa.hole, f.hole, sizeof(f.hole));
          std::memcpy(fa.lrow, f.lrow, sizeof(f.lrow));
          std::memcpy(fa.pos_row, f.pos_row, sizeof(f.pos_row));
          std::memcpy(fa.pos_col, f.pos_col, sizeof(f.pos_col));
          std::memcpy(fa.out_row, f.out_row, sizeof(f.out_row));
          std::memcpy(fa.out_col, f.out_col, sizeof(f.out_col));
          for (int i = 0; i < tnc::kFuseMaxOuter && i < tnc::kFuseOuterMax; ++i) fa.out_pass[i] = f.out_pass[i];
          e = tnc::launch_fused2(fa, stream);
          break;
        }
      }
      st = check(e, stream, op_name(op.kind));
      if (st != TNC_OK) return st;
      if (tm) {
        tm->record(oi + 1, 1, stream);
        std::snprintf((*tm->ops)[oi + 1].kernel, sizeof((*tm->ops)[oi + 1].kernel), "%s",
                      tnc::last_kernel_name());
      }
    }
    if (tm) {
      tm->collect(stream);
      if (tm->err != hipSuccess) return check(tm->err, stream, "per-launch timing events");
      // the header runs once per call, not per slice
      if (sigma + 1 < s_end) (*tm->ops)[0].launches -= 1;
    }
  }
  return TNC_OK;
}

// Static workspace of tnc_execute_noalloc: one copy per GPU, held from the
// library's load until the process ends.  Host code never passes `scratch`
// itself to a kernel or a copy (on the host the name is only a stand-in);
// it uses the device address that hipGetSymbolAddress returns per device.
constexpr uint64_t kScratchBytes = TNC_NOALLOC_MAX_WORKSPACE_BYTES;
__device__ __align__(256) unsigned char scratch[kScratchBytes];

constexpr int kMaxScratchDevices = 64;
std::mutex g_scratch_mu;
void *g_scratch_ptr[kMaxScratchDevices] = {};

// Device address of `scratch` on the current device, looked up once per
// device (with that device current).
tnc_status scratch_for_current_device(void **ptr) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) {
    (void)hipGetLastError();
    g_last_error = std::string("hipGetDevice: ") + hipGetErrorString(e);
    return TNC_ERR_HIP;
  }
  if (dev < 0 || dev >= kMaxScratchDevices) {
    g_last_error = "device index beyond the static scratch table";
    return TNC_ERR_INVALID_ARG;
  }
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void *a = nullptr;
    e = hipGetSymbolAddress(&a, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !a) {
      (void)hipGetLastError();
      g_last_error = std::string("hipGetSymbolAddress(scratch): ") + hipGetErrorString(e);
      return TNC_ERR_HIP;
    }
    g_scratch_ptr[dev] = a;
  }
  *ptr = g_scratch_ptr[dev];
  return TNC_OK;
}

}  // namespace

extern "C" {

tnc_status tnc_execute(tnc_plan_t plan, const void *const *leaves, void *out, void *workspace,
                       uint64_t workspace_bytes, void *stream_ptr) {
  g_last_error.clear();
  if (!plan || !leaves || !out) return TNC_ERR_INVALID_ARG;
  return run_plan(plan, leaves, out, workspace, workspace_bytes, stream_ptr, true);
}

tnc_status tnc_execute_timed(tnc_plan_t plan, const void *const *leaves, void *out, void *workspace,
                             uint64_t workspace_bytes, void *stream_ptr, tnc_op_timing *ops, int32_t max_ops,
                             int32_t *num_ops) {
  g_last_error.clear();
  if (!plan || !leaves || !out || !ops || !num_ops) return TNC_ERR_INVALID_ARG;
  const tnc::PlanImpl &p = plan->impl;
  const size_t n = p.program.size() + 1;
  if (max_ops < 0 || (size_t)max_ops < n) {
    g_last_error = "ops holds " + std::to_string(max_ops) + " records, the plan has " + std::to_string(n);
    return TNC_ERR_INVALID_ARG;
  }
  std::vector<tnc_op_timing> rec(n);
  for (size_t i = 0; i < n; ++i) {
    std::memset(&rec[i], 0, sizeof(rec[i]));
    rec[i].step = -1;
    rec[i].count = 1;
  }
  rec[0].kind = TNC_OP_HEADER;
  std::snprintf(rec[0].kernel, sizeof(rec[0].kernel), "k_header");
  for (size_t i = 1; i < n; ++i) {
    const tnc::Op &op = p.program[i - 1];
    rec[i].kind = op.kind == tnc::OP_COPY ? TNC_OP_COPY
                  : op.kind == tnc::OP_COPY_TILED ? TNC_OP_COPY_TILED
                  : op.kind == tnc::OP_TINY_GROUP ? TNC_OP_TINY_GROUP
                  : op.kind == tnc::OP_SKINNY ? TNC_OP_SKINNY
                  : op.kind == tnc::OP_FUSED ? TNC_OP_FUSED : TNC_OP_GEMM;
    if (op.kind == tnc::OP_SKINNY || op.kind == tnc::OP_GEMM) rec[i].step = op.first;
    if (op.kind == tnc::OP_FUSED) {
      const tnc::FusedChain &f = p.fused[op.first];
      rec[i].step = f.step[f.nsteps - 1];
      rec[i].count = f.nsteps;
    }
    if (op.kind == tnc::OP_COPY || op.kind == tnc::OP_TINY_GROUP) rec[i].count = op.count;
  }
  OpTimer tm;
  tm.ops = &rec;
  tm.ev.assign(2 * n, nullptr);
  for (auto &e : tm.ev) {
    hipError_t r = hipEventCreate(&e);
    if (r != hipSuccess) {
      (void)hipGetLastError();
      e = nullptr;
      g_last_error = std::string("hipEventCreate: ") + hipGetErrorString(r);
      return TNC_ERR_HIP;
    }
  }
  tnc_status st = run_plan(plan, leaves, out, workspace, workspace_bytes, stream_ptr, true, &tm);
  if (st != TNC_OK) return st;
  for (size_t i = 0; i < n; ++i) ops[i] = rec[i];
  *num_ops = (int32_t)n;
  return TNC_OK;
}

tnc_status tnc_probe_peaks(void *buffer, uint64_t bytes, void *stream_ptr, double *mfma_tflops,
                           double *copy_gbps) {
  g_last_error.clear();
  const int32_t cus = tnc::device_cus();
  const uint64_t need_mfma = (uint64_t)4 * cus * 256 * sizeof(float);
  if (!buffer || !mfma_tflops || !copy_gbps || bytes < (uint64_t(64) << 20) || bytes < need_mfma ||
      (reinterpret_cast<uintptr_t>(buffer) & 255) != 0)
    return TNC_ERR_INVALID_ARG;
  hipStream_t stream = reinterpret_cast<hipStream_t>(stream_ptr);
  (void)hipGetLastError();
  hipEvent_t e0 = nullptr, e1 = nullptr;
  hipError_t e = hipEventCreate(&e0);
  if (e == hipSuccess) e = hipEventCreate(&e1);
  const int32_t iters = 20000;
  double best_mfma = 0, best_copy = 0;
  const int64_t half16 = (int64_t)(bytes / 2 / 16);
  char *buf = static_cast<char *>(buffer);
  auto timed = [&](auto launch, float *ms) {
    if (e == hipSuccess) e = hipEventRecord(e0, stream);
    if (e == hipSuccess) e = launch();
    if (e == hipSuccess) e = hipEventRecord(e1, stream);
    if (e == hipSuccess) e = hipEventSynchronize(e1);
    if (e == hipSuccess) e = hipEventElapsedTime(ms, e0, e1);
  };
  // launch shapes: 4 or 8 chains per wave at 2 or 4 waves per SIMD; copies
  // with 1 or 4 loads in flight per thread.  Best of three runs after one
  // untimed run, best over the shapes.
  for (int32_t waves : {2, 4})
    for (int32_t chains : {4, 8}) {
      const int64_t blocks = (int64_t)waves * cus;
      for (int rep = 0; rep < 4 && e == hipSuccess; ++rep) {
        float ms = 0.f;
        timed([&] { return tnc::launch_probe_mfma(static_cast<float *>(buffer), blocks, iters, chains, stream); },
              &ms);
        // flops: blocks x 4 waves x iters x chains x (32 x 32 x 2 x 2)
        const double tf = (double)blocks * 4 * iters * chains * 4096.0 / (ms * 1e-3) / 1e12;
        if (e == hipSuccess && rep > 0 && tf > best_mfma) best_mfma = tf;
      }
    }
  // copy patterns: grid-stride with 1 or 4 loads in flight per thread, one
  // contiguous chunk per workgroup with plain or nontemporal accesses
  for (int32_t pattern : {0, 1, 2, 3})
    for (int rep = 0; rep < 4 && e == hipSuccess; ++rep) {
      float ms = 0.f;
      timed([&] { return tnc::launch_probe_copy(buf, buf + half16 * 16, half16, pattern, stream); }, &ms);
      const double gbps = 2.0 * (double)half16 * 16 / (ms * 1e-3) / 1e9;
      if (e == hipSuccess && rep > 0 && gbps > best_copy) best_copy = gbps;
    }
  if (e0) (void)hipEventDestroy(e0);
  if (e1) (void)hipEventDestroy(e1);
  if (e != hipSuccess) {
    g_last_error = std::string("peak probe: ") + hipGetErrorString(e);
    (void)hipGetLastError();
    return TNC_ERR_HIP;
  }
  *mfma_tflops = best_mfma;
  *copy_gbps = best_copy;
  return TNC_OK;
}

tnc_status tnc_execute_noalloc(tnc_plan_t plan, const void *const *leaves, void *out, void *stream_ptr) {
  g_last_error.clear();
  if (!plan || !leaves || !out) return TNC_ERR_INVALID_ARG;
  if (plan->impl.stats.workspace_bytes > kScratchBytes) {
    g_last_error = "plan needs " + std::to_string(plan->impl.stats.workspace_bytes) +
                   " bytes of workspace; the static scratch holds " + std::to_string(kScratchBytes);
    return TNC_ERR_WORKSPACE_TOO_SMALL;
  }
  void *ws = nullptr;
  tnc_status st = scratch_for_current_device(&ws);
  if (st != TNC_OK) return st;
  return run_plan(plan, leaves, out, ws, kScratchBytes, stream_ptr, false);
}

tnc_status tnc_dist_options_default(tnc_dist_options *o, tnc_dtype dtype) {
  if (!o || (dtype != TNC_C64 && dtype != TNC_C128)) return TNC_ERR_INVALID_ARG;
  o->num_gpus = 8;
  o->threshold_bytes = uint64_t(8) << 30;
  o->hbm_bytes_per_s = 8.0e12;
  o->flops_per_s = dtype == TNC_C128 ? 78.6e12 : 157.3e12;
  o->net_bytes_per_s = 7 * 76.8e9;
  o->latency_s = 5e-6;
  return TNC_OK;
}

tnc_status tnc_plan_distribute(tnc_plan_t plan, const tnc_dist_options *o, tnc_dist_step *steps, double *total) {
  g_last_error.clear();
  if (!plan || !o || (!steps && plan->impl.S > 0) || !total) return TNC_ERR_INVALID_ARG;
  if (o->num_gpus < 1 || o->num_gpus > 65536 || !(o->hbm_bytes_per_s > 0) || !(o->flops_per_s > 0) ||
      !(o->net_bytes_per_s > 0) || !(o->latency_s >= 0))
    return TNC_ERR_INVALID_ARG;
  const auto &p = plan->impl;
  std::vector<tnc_dist_step> tmp(p.S);
  double tot = 0;
  std::string err;
  tnc_status st;
  try {
    st = tnc::plan_distribution(p, *o, tmp.data(), &tot, &err);
  } catch (const std::bad_alloc &) {
    return TNC_ERR_OUT_OF_MEMORY;
  }
  if (st != TNC_OK) {
    g_last_error = err;
    return st;
  }
  for (int32_t s = 0; s < p.S; ++s) steps[s] = tmp[s];
  *total = tot;
  return TNC_OK;
}

const char *tnc_last_error(void) { return g_last_error.c_str(); }

const char *tnc_status_string(tnc_status s) {
  switch (s) {
    case TNC_OK: return "TNC_OK";
    case TNC_ERR_INVALID_ARG: return "TNC_ERR_INVALID_ARG";
    case TNC_ERR_INVALID_NETWORK: return "TNC_ERR_INVALID_NETWORK";
    case TNC_ERR_INVALID_TREE: return "TNC_ERR_INVALID_TREE";
    case TNC_ERR_UNSUPPORTED: return "TNC_ERR_UNSUPPORTED";
    case TNC_ERR_OUT_OF_MEMORY: return "TNC_ERR_OUT_OF_MEMORY";
    case TNC_ERR_WORKSPACE_TOO_SMALL: return "TNC_ERR_WORKSPACE_TOO_SMALL";
    case TNC_ERR_HIP: return "TNC_ERR_HIP";
  }
  return "TNC_ERR_UNKNOWN";
}

}  // extern "C"
