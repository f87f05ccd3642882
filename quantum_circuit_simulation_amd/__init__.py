"""Exact tensor-network contraction along a fixed tree on one MI355X.

The contraction itself runs in ``libtnc.so`` (C ABI, ``include/tnc.h``):
a host planner applies reverse-tree lifetime ordering so every pairwise step
is a transpose-free complex64 GEMM, and hand-written gfx950 kernels execute
the plan.  This package is the thin Python binding over that library.
"""

from .tnc import (CLASS_GEMM, CLASS_SKINNY, CLASS_TINY, NONE, ORDER_LIFETIME, ORDER_NAIVE, PREC_BF16X3, PREC_EXACT, TNC_C64,
                  TNC_C128, Plan,
                  TncError, alloc_workspace, load_library)

__all__ = ["Plan", "TncError", "alloc_workspace", "load_library", "ORDER_LIFETIME", "ORDER_NAIVE", "CLASS_TINY",
           "CLASS_SKINNY", "CLASS_GEMM", "NONE", "TNC_C64", "TNC_C128", "PREC_EXACT",
           "PREC_BF16X3"]
