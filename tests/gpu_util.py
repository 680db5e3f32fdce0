"""Helpers shared by the GPU parity tests: upload seeded inputs, run a stage
through the C ABI, download results."""

import numpy as np
import torch

from pipeline_schedules_amd import pps


def tdtype(dtype):
    return torch.bfloat16 if dtype == "bf16" else torch.float32


def to_dev(a, dtype):
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to("cuda").to(tdtype(dtype))


def to_host(t):
    return t.detach().float().cpu().numpy().astype(np.float64)


def upload_params(params, block, dtype):
    """Device weights in the ABI order [(chunk*L + block)*nw + w]."""
    out = []
    for p in params:
        if block == "swiglu":
            out += [to_dev(p["Wg"], dtype), to_dev(p["Wu"], dtype), to_dev(p["Wd"], dtype),
                    torch.from_numpy(p["gamma"].astype(np.float32)).cuda()]
        else:
            out += [torch.from_numpy(p["W"].astype(np.float32)).cuda(),
                    torch.from_numpy(p["b"].astype(np.float32)).cuda()]
    return out


def grad_shapes(block, d, f):
    if block == "swiglu":
        return {"Wg": (0, (d, f)), "Wu": (1, (d, f)), "Wd": (2, (f, d)), "gamma": (3, (d,))}
    return {"W": (0, (d, d)), "b": (1, (d,))}


def run_stage(stage, ops, xs_dev, dys_dev, T, d, dtype):
    """Issue ``ops`` (op, mb, chunk, ...) on the stage.  xs_dev / dys_dev are
    indexed [chunk][mb].  Returns ys, dxs as [chunk][mb] device tensors."""
    v = len(xs_dev)
    M = len(xs_dev[0])
    ys = [[torch.empty((T, d), dtype=tdtype(dtype), device="cuda") for _ in range(M)] for _ in range(v)]
    dxs = [[torch.empty((T, d), dtype=tdtype(dtype), device="cuda") for _ in range(M)] for _ in range(v)]
    for op, mb, c, *_ in ops:
        if op == pps.OP_F:
            stage.forward(mb, c, xs_dev[c][mb], ys[c][mb])
        elif op == pps.OP_B:
            stage.backward(mb, c, dys_dev[c][mb], dxs[c][mb])
        else:
            stage.backward_weight(mb, c)
    stage.sync()
    return ys, dxs


def stage_grads(stage, nblocks, block, d, f, chunk=0):
    out = []
    for b in range(nblocks):
        g = {}
        for key, (which, shape) in grad_shapes(block, d, f).items():
            g[key] = to_host(stage.grad(chunk, b, which, shape))
        out.append(g)
    return out
