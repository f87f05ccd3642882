"""Helpers for the GPU parity tests: run a network through the C-ABI
library on cuda:0 and read the result back."""

import numpy as np

import quantum_circuit_simulation_amd as qa


def to_device(arrays):
    import torch
    return [torch.from_numpy(np.ascontiguousarray(a, dtype=np.complex64)).to("cuda") for a in arrays]


def run(net, tree, leaves_dev=None, sync=True, **plan_kw):
    """Plan, allocate, execute; returns (result complex128 ndarray, plan)."""
    import torch
    plan = qa.Plan.from_network(net, tree, **plan_kw)
    if leaves_dev is None:
        leaves_dev = to_device(net.data)
    size = int(np.prod(plan.out_shape, dtype=np.int64)) if plan.out_shape else 1
    out = torch.empty(size, dtype=torch.complex64, device="cuda")
    ws = qa.alloc_workspace(plan)
    plan.execute(leaves_dev, out, ws)
    torch.cuda.synchronize()
    return out.cpu().numpy().astype(np.complex128).reshape(plan.out_shape), plan
