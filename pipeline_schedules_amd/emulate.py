"""Single-GPU emulation of a P-stage pipeline with P stage handles.

Every stage's op list comes from ``pps_make_schedule``; the ops of all stages
are issued in order of their unit-cost start time (ties by stage index), on
one HIP stream, so every op finds its inputs ready.  Stage k's forward output
of micro-batch i is stage k+1's input; stage k+1's input gradient is stage
k's output gradient ([1F1B §5.2] send_to_next / send_to_prev, here device
buffers handed over on one GPU).  The last stage's output gradient is the
loss gradient divided by M ([1F1B §5.2]), with the linear-probe loss
L = (1/M) sum_i <y_i, G_i>, i.e. dy_i = G_i / M, computed with ``pps_scale``.

[1F1B] = page "2. 1F1B" (sgdbs.github.io AI_Infra notes).
"""

from __future__ import annotations

import torch

from . import pps


def run_pipeline(stages, xs, Gs, dtype, kind=pps.ONE_F_ONE_B):
    """Run one pass of all stages.  ``stages[k]`` is a ``pps.Stage`` for
    stage k (same P, M, kind, v=1); ``xs``/``Gs`` are M device tensors [T,d].

    Returns (ys_last, dxs_first): the last stage's outputs and the first
    stage's input gradients, per micro-batch.
    """
    P = len(stages)
    M = len(xs)
    T, d = xs[0].shape
    tdt = xs[0].dtype
    stream = torch.cuda.current_stream()
    act = [[torch.empty((T, d), dtype=tdt, device=xs[0].device) for _ in range(M)] for _ in range(P)]
    grad = [[torch.empty((T, d), dtype=tdt, device=xs[0].device) for _ in range(M)] for _ in range(P)]
    loss_grad = [torch.empty((T, d), dtype=tdt, device=xs[0].device) for _ in range(M)]
    for i in range(M):
        pps.scale(loss_grad[i], Gs[i], T * d, 1.0 / M, dtype, stream)
    ops = []
    for k in range(P):
        for op in pps.make_schedule(P, M, k, 1, kind):
            ops.append((op[5], k, op))
    ops.sort(key=lambda t: (t[0], t[1]))
    for _t, k, (op, mb, chunk, *_rest) in ops:
        st = stages[k]
        if op == pps.OP_F:
            x = xs[mb] if k == 0 else act[k - 1][mb]
            st.forward(mb, chunk, x, act[k][mb])
        elif op == pps.OP_B:
            dy = loss_grad[mb] if k == P - 1 else grad[k + 1][mb]
            st.backward(mb, chunk, dy, grad[k][mb])
        else:
            st.backward_weight(mb, chunk)
    for st in stages:
        st.sync()
    return act[P - 1], grad[0]
