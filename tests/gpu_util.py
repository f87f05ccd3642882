"""Helpers for the GPU parity tests: run a network through the C-ABI
library on cuda:0 and read the result back."""

import numpy as np

import quantum_circuit_simulation_amd as qa


def to_device(arrays, dtype=np.complex64):
    import torch
    return [torch.from_numpy(np.ascontiguousarray(a, dtype=dtype)).to("cuda") for a in arrays]


def run(net, tree, leaves_dev=None, sync=True, **plan_kw):
    """Plan, allocate, execute; returns (result complex128 ndarray, plan).
    With dtype=TNC_C128 the leaves go to the GPU as complex128."""
    import torch
    plan = qa.Plan.from_network(net, tree, **plan_kw)
    z = plan_kw.get("dtype", qa.TNC_C64) == qa.TNC_C128
    if leaves_dev is None:
        leaves_dev = to_device(net.data, np.complex128 if z else np.complex64)
    size = int(np.prod(plan.out_shape, dtype=np.int64)) if plan.out_shape else 1
    out = torch.empty(size, dtype=torch.complex128 if z else torch.complex64, device="cuda")
    ws = qa.alloc_workspace(plan)
    plan.execute(leaves_dev, out, ws)
    torch.cuda.synchronize()
    return out.cpu().numpy().astype(np.complex128).reshape(plan.out_shape), plan
