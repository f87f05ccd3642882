"""ctypes binding of libtnc.so (include/tnc.h).

Argument marshalling only: every step of the contraction runs in the HIP
library.  PyTorch supplies device memory and the stream; nothing here falls
back to a CPU path.  If the library has not been built this module raises on
import (build it with ``python quantum_circuit_simulation_amd/build.py``).
"""

from __future__ import annotations

import ctypes
import os
from typing import List, Optional, Sequence

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libtnc.so")

TNC_OK = 0
STATUS = {0: "TNC_OK", 1: "TNC_ERR_INVALID_ARG", 2: "TNC_ERR_INVALID_NETWORK", 3: "TNC_ERR_INVALID_TREE",
          4: "TNC_ERR_UNSUPPORTED", 5: "TNC_ERR_OUT_OF_MEMORY", 6: "TNC_ERR_WORKSPACE_TOO_SMALL",
          7: "TNC_ERR_HIP"}
TNC_C64, TNC_C128 = 0, 1
PREC_EXACT, PREC_BF16X3 = 0, 1
ORDER_LIFETIME, ORDER_NAIVE = 0, 1
CLASS_TINY, CLASS_SKINNY, CLASS_GEMM = 0, 1, 2
NONE = (1 << 64) - 1
FUSE_MAX_STEPS = 6  # TNC_FUSE_MAX_STEPS: the longest fused chain

P = ctypes.POINTER


class TncError(RuntimeError):
    def __init__(self, code: int, where: str, detail: str = ""):
        super().__init__(f"{where}: {STATUS.get(code, code)}" + (f" ({detail})" if detail else ""))
        self.code = code
        self.name = STATUS.get(code, str(code))


class Network(ctypes.Structure):
    _fields_ = [("num_modes", ctypes.c_int32), ("extents", P(ctypes.c_int64)),
                ("num_leaves", ctypes.c_int32), ("leaf_rank", P(ctypes.c_int32)),
                ("leaf_modes", P(ctypes.c_int32)), ("out_rank", ctypes.c_int32),
                ("out_modes", P(ctypes.c_int32)), ("dtype", ctypes.c_int)]


class Tree(ctypes.Structure):
    _fields_ = [("num_steps", ctypes.c_int32), ("lhs", P(ctypes.c_int32)), ("rhs", P(ctypes.c_int32))]


class PlanOptions(ctypes.Structure):
    _fields_ = [("order", ctypes.c_int), ("num_sliced", ctypes.c_int32), ("sliced_modes", P(ctypes.c_int32)),
                ("align", ctypes.c_uint64), ("capacity_bytes", ctypes.c_uint64), ("tiny_mnk", ctypes.c_uint64),
                ("max_group", ctypes.c_int32), ("precision", ctypes.c_int32), ("slice_begin", ctypes.c_int64),
                ("slice_end", ctypes.c_int64), ("fuse", ctypes.c_int32)]


class PlanStats(ctypes.Structure):
    _fields_ = [("num_leaves", ctypes.c_int32), ("num_steps", ctypes.c_int32), ("num_groups", ctypes.c_int32),
                ("nodes_tiny", ctypes.c_int32), ("nodes_skinny", ctypes.c_int32), ("nodes_gemm", ctypes.c_int32),
                ("nodes_split", ctypes.c_int32), ("nodes_interleaved", ctypes.c_int32),
                ("min_inner_run", ctypes.c_int32), ("staged_leaves", ctypes.c_int32),
                ("relayouts", ctypes.c_int32), ("root_permute", ctypes.c_int32), ("num_slices", ctypes.c_int64),
                ("flops", ctypes.c_double), ("flops_unsliced", ctypes.c_double), ("bytes", ctypes.c_double),
                ("max_intermediate", ctypes.c_uint64), ("header_bytes", ctypes.c_uint64),
                ("arena_bytes", ctypes.c_uint64), ("workspace_bytes", ctypes.c_uint64),
                ("fused_pairs", ctypes.c_int32)]

    def as_dict(self):
        return {name: getattr(self, name) for name, _ in self._fields_}


class NodeInfo(ctypes.Structure):
    _fields_ = [("lhs", ctypes.c_int32), ("rhs", ctypes.c_int32), ("out", ctypes.c_int32),
                ("kernel_class", ctypes.c_int32), ("swap", ctypes.c_int32), ("group", ctypes.c_int32),
                ("splits", ctypes.c_int32), ("row_runs", ctypes.c_int32), ("col_runs", ctypes.c_int32),
                ("inner_run", ctypes.c_int32), ("interleaved", ctypes.c_int32), ("copy_a", ctypes.c_int32),
                ("copy_b", ctypes.c_int32), ("m", ctypes.c_int64), ("n", ctypes.c_int64), ("k", ctypes.c_int64),
                ("a_off", ctypes.c_uint64), ("b_off", ctypes.c_uint64), ("c_off", ctypes.c_uint64),
                ("scratch_off", ctypes.c_uint64), ("scratch_bytes", ctypes.c_uint64),
                ("fused_with", ctypes.c_int32)]

    def as_dict(self):
        return {name: getattr(self, name) for name, _ in self._fields_}


class FusedInfo(ctypes.Structure):
    _fields_ = [("nsteps", ctypes.c_int32), ("step", ctypes.c_int32 * FUSE_MAX_STEPS),
                ("longop", ctypes.c_int32 * FUSE_MAX_STEPS), ("k", ctypes.c_int32 * FUSE_MAX_STEPS),
                ("rows", ctypes.c_int64), ("nouter", ctypes.c_int32), ("lrow", ctypes.c_int32 * 9),
                ("hole", ctypes.c_int32 * 11), ("wbit", ctypes.c_int32 * 2),
                ("pos_row", (ctypes.c_int32 * 9) * (FUSE_MAX_STEPS - 1)),
                ("pos_col", (ctypes.c_int32 * 8) * (FUSE_MAX_STEPS - 1)),
                ("out_row", ctypes.c_int64 * 9), ("out_col", ctypes.c_int64 * 8), ("out_pass", ctypes.c_int64 * 48)]

    def as_dict(self):
        def plain(v):
            return [plain(x) for x in v] if isinstance(v, ctypes.Array) else v
        d = {name: plain(getattr(self, name)) for name, _ in self._fields_}
        n = d["nsteps"]   # the chain's own entries only
        for name in ("step", "longop", "k"):
            d[name] = d[name][:n]
        for name in ("pos_row", "pos_col"):
            d[name] = d[name][:n - 1]
        return d


class DistOptions(ctypes.Structure):
    _fields_ = [("num_gpus", ctypes.c_int32), ("threshold_bytes", ctypes.c_uint64),
                ("hbm_bytes_per_s", ctypes.c_double), ("flops_per_s", ctypes.c_double),
                ("net_bytes_per_s", ctypes.c_double), ("latency_s", ctypes.c_double)]


class DistStep(ctypes.Structure):
    _fields_ = [("tag", ctypes.c_int32), ("dist_operand", ctypes.c_int32), ("gathered_operand", ctypes.c_int32),
                ("num_dist", ctypes.c_int32), ("dist_modes", ctypes.c_int32 * 16), ("num_local", ctypes.c_int32),
                ("local_modes", ctypes.c_int32 * 16), ("local_m", ctypes.c_int64),
                ("local_n", ctypes.c_int64), ("local_k", ctypes.c_int64), ("local_count", ctypes.c_int64),
                ("t_gemm", ctypes.c_double), ("t_comm", ctypes.c_double)]

    def as_dict(self):
        d = {name: getattr(self, name) for name, _ in self._fields_ if name not in ("dist_modes", "local_modes")}
        d["dist_modes"] = [int(self.dist_modes[i]) for i in range(self.num_dist)]
        d["local_modes"] = [int(self.local_modes[i]) for i in range(self.num_local)]
        return d


DIST_TAGS = ["replicated", "activate", "keep", "redistribute", "gather"]


class OpTiming(ctypes.Structure):
    _fields_ = [("kind", ctypes.c_int32), ("step", ctypes.c_int32), ("count", ctypes.c_int32),
                ("launches", ctypes.c_int32), ("ms", ctypes.c_double), ("kernel", ctypes.c_char * 64)]


OP_KINDS = ["copy", "tiny_group", "skinny", "gemm", "copy_tiled", "header", "fused"]

EXPORTS = ["tnc_plan_options_default", "tnc_plan", "tnc_plan_destroy", "tnc_plan_workspace_bytes",
           "tnc_plan_stats_get", "tnc_plan_tensor_order", "tnc_plan_tensor_offset", "tnc_plan_node",
           "tnc_execute", "tnc_status_string", "tnc_last_error", "tnc_dist_options_default",
           "tnc_plan_distribute", "tnc_execute_noalloc", "tnc_execute_timed", "tnc_probe_peaks", "tnc_plan_fused"]
NOALLOC_MAX_WORKSPACE_BYTES = 64 << 20  # TNC_NOALLOC_MAX_WORKSPACE_BYTES

_lib = None


def load_library(path: str = LIB_PATH):
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise ImportError(f"{path} is missing: build it with `python quantum_circuit_simulation_amd/build.py`")
    # Let torch bring in its HIP runtime first, so that the library binds to
    # the same runtime (and sees the same devices, streams and allocations)
    # rather than loading a second copy from the system ROCm.
    try:
        import torch  # noqa: F401
    except ImportError:
        pass
    lib = ctypes.CDLL(path)
    lib.tnc_plan_options_default.argtypes = [P(PlanOptions)]
    lib.tnc_plan_options_default.restype = None
    lib.tnc_plan.argtypes = [P(Network), P(Tree), P(PlanOptions), P(ctypes.c_void_p)]
    lib.tnc_plan.restype = ctypes.c_int
    lib.tnc_plan_destroy.argtypes = [ctypes.c_void_p]
    lib.tnc_plan_destroy.restype = None
    lib.tnc_plan_workspace_bytes.argtypes = [ctypes.c_void_p, P(ctypes.c_uint64)]
    lib.tnc_plan_workspace_bytes.restype = ctypes.c_int
    lib.tnc_plan_stats_get.argtypes = [ctypes.c_void_p, P(PlanStats)]
    lib.tnc_plan_stats_get.restype = ctypes.c_int
    lib.tnc_plan_tensor_order.argtypes = [ctypes.c_void_p, ctypes.c_int32, P(ctypes.c_int32), P(ctypes.c_int32)]
    lib.tnc_plan_tensor_order.restype = ctypes.c_int
    lib.tnc_plan_tensor_offset.argtypes = [ctypes.c_void_p, ctypes.c_int32, P(ctypes.c_uint64)]
    lib.tnc_plan_tensor_offset.restype = ctypes.c_int
    lib.tnc_plan_node.argtypes = [ctypes.c_void_p, ctypes.c_int32, P(NodeInfo)]
    lib.tnc_plan_node.restype = ctypes.c_int
    lib.tnc_plan_fused.argtypes = [ctypes.c_void_p, ctypes.c_int32, P(FusedInfo)]
    lib.tnc_plan_fused.restype = ctypes.c_int
    lib.tnc_execute.argtypes = [ctypes.c_void_p, P(ctypes.c_void_p), ctypes.c_void_p, ctypes.c_void_p,
                                ctypes.c_uint64, ctypes.c_void_p]
    lib.tnc_execute.restype = ctypes.c_int
    lib.tnc_execute_noalloc.argtypes = [ctypes.c_void_p, P(ctypes.c_void_p), ctypes.c_void_p, ctypes.c_void_p]
    lib.tnc_execute_noalloc.restype = ctypes.c_int
    lib.tnc_execute_timed.argtypes = [ctypes.c_void_p, P(ctypes.c_void_p), ctypes.c_void_p, ctypes.c_void_p,
                                      ctypes.c_uint64, ctypes.c_void_p, P(OpTiming), ctypes.c_int32,
                                      P(ctypes.c_int32)]
    lib.tnc_execute_timed.restype = ctypes.c_int
    lib.tnc_probe_peaks.argtypes = [ctypes.c_void_p, ctypes.c_uint64, ctypes.c_void_p, P(ctypes.c_double),
                                    P(ctypes.c_double)]
    lib.tnc_probe_peaks.restype = ctypes.c_int
    lib.tnc_status_string.argtypes = [ctypes.c_int]
    lib.tnc_status_string.restype = ctypes.c_char_p
    lib.tnc_last_error.argtypes = []
    lib.tnc_last_error.restype = ctypes.c_char_p
    lib.tnc_dist_options_default.argtypes = [P(DistOptions), ctypes.c_int]
    lib.tnc_dist_options_default.restype = ctypes.c_int
    lib.tnc_plan_distribute.argtypes = [ctypes.c_void_p, P(DistOptions), P(DistStep), P(ctypes.c_double)]
    lib.tnc_plan_distribute.restype = ctypes.c_int
    _lib = lib
    return lib


def _check(code: int, where: str):
    if code != TNC_OK:
        detail = ""
        if _lib is not None:
            detail = (_lib.tnc_last_error() or b"").decode(errors="replace")
        raise TncError(code, where, detail)


def _i32(a):
    a = np.ascontiguousarray(np.asarray(a, dtype=np.int32))
    return a if a.size else np.zeros(1, dtype=np.int32)


def _i64(a):
    a = np.ascontiguousarray(np.asarray(a, dtype=np.int64))
    return a if a.size else np.zeros(1, dtype=np.int64)


class Plan:
    """A tnc plan built from a network description and a tree (host only)."""

    def __init__(self, extents, leaves: Sequence[Sequence[int]], out_modes: Sequence[int], lhs, rhs,
                 order: int = ORDER_LIFETIME, sliced: Sequence[int] = (), align: int = 256,
                 capacity_bytes: int = 0, tiny_mnk: int = 1 << 17, max_group: int = 256, dtype: int = TNC_C64,
                 precision: int = 0, slice_range: Optional[Sequence[int]] = None, fuse: bool = True):
        lib = load_library()
        self._lib = lib
        self.num_leaves = len(leaves)
        self.num_steps = len(lhs)
        ext = _i64(extents)
        rank = _i32([len(l) for l in leaves])
        modes = _i32([x for l in leaves for x in l])
        outm = _i32(out_modes)
        lhs_a, rhs_a = _i32(lhs), _i32(rhs)
        sl = _i32(sliced)
        self._keep = (ext, rank, modes, outm, lhs_a, rhs_a, sl)
        net = Network(len(extents), ext.ctypes.data_as(P(ctypes.c_int64)), len(leaves),
                      rank.ctypes.data_as(P(ctypes.c_int32)), modes.ctypes.data_as(P(ctypes.c_int32)),
                      len(out_modes), outm.ctypes.data_as(P(ctypes.c_int32)), int(dtype))
        self.dtype = int(dtype)
        tree = Tree(len(lhs), lhs_a.ctypes.data_as(P(ctypes.c_int32)), rhs_a.ctypes.data_as(P(ctypes.c_int32)))
        opts = PlanOptions()
        lib.tnc_plan_options_default(ctypes.byref(opts))
        opts.order = order
        opts.num_sliced = len(sliced)
        opts.sliced_modes = sl.ctypes.data_as(P(ctypes.c_int32))
        opts.align = align
        opts.capacity_bytes = capacity_bytes
        opts.tiny_mnk = tiny_mnk
        opts.max_group = max_group
        opts.precision = precision
        opts.fuse = 1 if fuse else 0
        if slice_range is not None:
            opts.slice_begin, opts.slice_end = int(slice_range[0]), int(slice_range[1])
        h = ctypes.c_void_p()
        _check(lib.tnc_plan(ctypes.byref(net), ctypes.byref(tree), ctypes.byref(opts), ctypes.byref(h)), "tnc_plan")
        self._h = h
        ext_list = [int(e) for e in extents]
        self.out_shape = tuple(ext_list[int(x)] for x in out_modes)
        self.leaf_shapes = [tuple(ext_list[int(x)] for x in l) for l in leaves]
        self._leaf_numel = [int(np.prod(sh, dtype=np.int64)) for sh in self.leaf_shapes]
        self._out_numel = int(np.prod(self.out_shape, dtype=np.int64))

    @classmethod
    def from_network(cls, net, tree, **kw) -> "Plan":
        return cls(net.extents, net.leaves, net.out_modes, tree.lhs, tree.rhs, **kw)

    def __del__(self):
        h = getattr(self, "_h", None)
        if h is not None and h.value:
            self._lib.tnc_plan_destroy(h)
            self._h = None

    @property
    def handle(self):
        return self._h

    @property
    def workspace_bytes(self) -> int:
        v = ctypes.c_uint64()
        _check(self._lib.tnc_plan_workspace_bytes(self._h, ctypes.byref(v)), "tnc_plan_workspace_bytes")
        return int(v.value)

    def stats(self) -> dict:
        s = PlanStats()
        _check(self._lib.tnc_plan_stats_get(self._h, ctypes.byref(s)), "tnc_plan_stats_get")
        return s.as_dict()

    def tensor_order(self, tid: int) -> List[int]:
        buf = (ctypes.c_int32 * 64)()
        r = ctypes.c_int32()
        _check(self._lib.tnc_plan_tensor_order(self._h, tid, buf, ctypes.byref(r)), "tnc_plan_tensor_order")
        return [int(buf[i]) for i in range(r.value)]

    def tensor_offset(self, tid: int) -> int:
        v = ctypes.c_uint64()
        _check(self._lib.tnc_plan_tensor_offset(self._h, tid, ctypes.byref(v)), "tnc_plan_tensor_offset")
        return int(v.value)

    def node(self, step: int) -> dict:
        n = NodeInfo()
        _check(self._lib.tnc_plan_node(self._h, step, ctypes.byref(n)), "tnc_plan_node")
        return n.as_dict()

    def fused(self, index: int) -> dict:
        """Pass tables of fused chain `index` (tnc_plan_fused); the per-step
        lists (step, longop, k, and pos_row / pos_col per transition) hold the
        chain's own entries only."""
        f = FusedInfo()
        _check(self._lib.tnc_plan_fused(self._h, index, ctypes.byref(f)), "tnc_plan_fused")
        return f.as_dict()

    def distribute(self, **overrides):
        """Distribution schedule over P GPUs (tnc_plan_distribute).  Keyword
        overrides of the MI355X defaults: num_gpus, threshold_bytes,
        hbm_bytes_per_s, flops_per_s, net_bytes_per_s, latency_s.  Returns
        (list of per-step dicts with a "tag_name", total seconds)."""
        o = DistOptions()
        _check(self._lib.tnc_dist_options_default(ctypes.byref(o), self.dtype), "tnc_dist_options_default")
        for k, v in overrides.items():
            if not hasattr(o, k):
                raise TypeError(f"unknown distribution option {k}")
            setattr(o, k, v)
        steps = (DistStep * max(1, self.num_steps))()
        tot = ctypes.c_double()
        _check(self._lib.tnc_plan_distribute(self._h, ctypes.byref(o), steps, ctypes.byref(tot)),
               "tnc_plan_distribute")
        out = []
        for i in range(self.num_steps):
            d = steps[i].as_dict()
            d["tag_name"] = DIST_TAGS[d["tag"]]
            out.append(d)
        return out, float(tot.value)

    def execute_ptrs(self, leaf_ptrs: Sequence[int], out_ptr: int, ws_ptr: int, ws_bytes: int, stream: int = 0):
        """Raw-pointer form: device addresses as Python ints."""
        arr = (ctypes.c_void_p * max(1, len(leaf_ptrs)))(*[int(p) for p in leaf_ptrs])
        _check(self._lib.tnc_execute(self._h, arr, ctypes.c_void_p(int(out_ptr)), ctypes.c_void_p(int(ws_ptr)),
                                     ctypes.c_uint64(int(ws_bytes)), ctypes.c_void_p(int(stream))), "tnc_execute")

    def check_buffers(self, leaves, out, workspace):
        """Raise ValueError unless every buffer has the plan's entry count,
        dtype and layout and all of them sit on one GPU.  The C ABI receives
        bare pointers, so a short buffer would otherwise be read or written
        past its end by the kernels."""
        import torch
        if len(leaves) != self.num_leaves:
            raise ValueError(f"wrong number of leaves: {len(leaves)} given, plan has {self.num_leaves}")
        want = torch.complex128 if self.dtype == TNC_C128 else torch.complex64
        for i, (t, need) in enumerate(zip(leaves, self._leaf_numel)):
            if t.numel() != need:
                raise ValueError(f"leaf {i} holds {t.numel()} entries, its modes need {need}")
        need = self._out_numel
        if out.numel() != need:
            raise ValueError(f"out holds {out.numel()} entries, the output modes need {need}")
        if workspace is not None and workspace.numel() * workspace.element_size() < self.workspace_bytes:
            raise ValueError(f"workspace holds {workspace.numel() * workspace.element_size()} bytes, "
                             f"the plan needs {self.workspace_bytes}")
        for t in list(leaves) + [out]:
            if t.dtype != want or not t.is_contiguous():
                raise ValueError(f"leaves and out must be contiguous {want} tensors")
        devices = {t.device for t in list(leaves) + [out] + ([workspace] if workspace is not None else [])}
        if len(devices) != 1 or next(iter(devices)).type != "cuda":
            raise ValueError(f"leaves, out and workspace must all be on one GPU (got {sorted(map(str, devices))})")

    def execute_noalloc_ptrs(self, leaf_ptrs: Sequence[int], out_ptr: int, stream: int = 0):
        """tnc_execute_noalloc: the library's static per-GPU workspace."""
        arr = (ctypes.c_void_p * max(1, len(leaf_ptrs)))(*[int(p) for p in leaf_ptrs])
        _check(self._lib.tnc_execute_noalloc(self._h, arr, ctypes.c_void_p(int(out_ptr)),
                                             ctypes.c_void_p(int(stream))), "tnc_execute_noalloc")

    def execute_noalloc(self, leaves, out, stream=None):
        """Like ``execute`` but with the library's static per-GPU workspace
        (at most ``NOALLOC_MAX_WORKSPACE_BYTES``); calls that overlap in time
        on one GPU share it and race."""
        import torch
        self.check_buffers(leaves, out, None)
        if stream is None:
            stream = torch.cuda.current_stream()
        s = stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream)
        self.execute_noalloc_ptrs([t.data_ptr() for t in leaves], out.data_ptr(), s)

    def bind(self, leaves, out, workspace, stream=None):
        """Check the buffers once and return a callable that enqueues
        tnc_execute on them with no further Python-side work (for loops that
        run one plan many times on the same buffers; the buffers must stay
        alive and unchanged in size while the callable is used)."""
        import torch
        self.check_buffers(leaves, out, workspace)
        if stream is None:
            stream = torch.cuda.current_stream()
        s = ctypes.c_void_p(stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream))
        arr = (ctypes.c_void_p * max(1, len(leaves)))(*[int(t.data_ptr()) for t in leaves])
        args = (self._h, arr, ctypes.c_void_p(int(out.data_ptr())), ctypes.c_void_p(int(workspace.data_ptr())),
                ctypes.c_uint64(workspace.numel() * workspace.element_size()), s)
        keep = (list(leaves), out, workspace, self)
        fn = self._lib.tnc_execute

        def run():
            code = fn(*args)
            if code != TNC_OK:
                _check(code, "tnc_execute")
        run.keep = keep
        return run

    def execute_timed(self, leaves, out, workspace, stream=None):
        """tnc_execute_timed: run once with HIP events around every launch
        (synchronous).  Returns one dict per launch of the program (index 0:
        the descriptor header) with kind, step, count, launches, ms (summed
        over slices) and kernel name."""
        import torch
        self.check_buffers(leaves, out, workspace)
        if stream is None:
            stream = torch.cuda.current_stream()
        s = stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream)
        cap = 3 * self.num_steps + 8
        recs = (OpTiming * cap)()
        n = ctypes.c_int32(0)
        arr = (ctypes.c_void_p * max(1, len(leaves)))(*[int(t.data_ptr()) for t in leaves])
        _check(self._lib.tnc_execute_timed(self._h, arr, ctypes.c_void_p(int(out.data_ptr())),
                                           ctypes.c_void_p(int(workspace.data_ptr())),
                                           ctypes.c_uint64(workspace.numel() * workspace.element_size()),
                                           ctypes.c_void_p(s), recs, cap, ctypes.byref(n)), "tnc_execute_timed")
        return [{"kind": OP_KINDS[r.kind], "step": r.step, "count": r.count, "launches": r.launches, "ms": r.ms,
                 "kernel": r.kernel.decode()} for r in recs[:n.value]]

    def execute(self, leaves, out, workspace, stream=None):
        """leaves: torch complex64 tensors on the GPU (declared layouts), out:
        complex64 tensor of the output size, workspace: uint8 tensor of at
        least ``workspace_bytes``.  Enqueued on ``stream`` (default: torch's
        current stream); returns without synchronising.  A HIP graph that
        captured this call reads the plan's descriptors on every replay, so
        keep this Plan alive as long as any such graph."""
        import torch
        self.check_buffers(leaves, out, workspace)
        if stream is None:
            stream = torch.cuda.current_stream()
        s = stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream)
        self.execute_ptrs([t.data_ptr() for t in leaves], out.data_ptr(), workspace.data_ptr(),
                          workspace.numel() * workspace.element_size(), s)


def probe_peaks(buffer, stream=None):
    """tnc_probe_peaks on a uint8 device tensor (>= 64 MiB, overwritten):
    returns (sustained FP32 MFMA TFLOP/s, HBM copy GB/s) of the device."""
    import torch
    lib = load_library()
    if stream is None:
        stream = torch.cuda.current_stream()
    s = stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream)
    f, c = ctypes.c_double(), ctypes.c_double()
    _check(lib.tnc_probe_peaks(ctypes.c_void_p(buffer.data_ptr()), buffer.numel() * buffer.element_size(),
                               ctypes.c_void_p(s), ctypes.byref(f), ctypes.byref(c)), "tnc_probe_peaks")
    return float(f.value), float(c.value)


def alloc_workspace(plan: Plan, device="cuda"):
    import torch
    n = max(256, plan.workspace_bytes)
    return torch.empty(n, dtype=torch.uint8, device=device)
