"""Float64 numerics oracle of one pipeline stage -- TEST INFRASTRUCTURE ONLY.

See ``oracle/__init__.py`` for who may import this and for the page legend.

The pages define the schedule, not the layers of a stage; the stage blocks
below are the plain definitions of the blocks named by the workloads:

* SwiGLU block (RMSNorm, gated MLP, residual)::

      r = (mean_j x_j^2 + eps)^(-1/2)        one scalar per token (row)
      n = x * r * gamma
      g = n Wg,  u = n Wu                   weights stored [in, out]
      h = silu(g) * u,   silu(g) = g * sigmoid(g)
      y = x + h Wd

* toy block (two per stage in the smallest workload)::

      z = x W + b,  y = GELU(z) = z * Phi(z)   (exact, erf-based)

Backward passes are hand-derived from those definitions by the chain rule.
The weight-gradient / input-gradient split follows [GPipe->ZB Zero Bubble]:
for Y = X W with output gradient G, the input gradient is G W^T (needed by
the previous stage at once) and the weight gradient is X^T G (can wait).
Gradient accumulation over micro-batches and one step at the end follows
[1F1B §5.1] (PipeDream-Flush: same weights for all micro-batches, gradients
summed, equal to one large-batch step).

All arithmetic is numpy float64; matrix products use ``@`` (a library
primitive), nothing is blocked, fused or reordered.
"""

from __future__ import annotations

import numpy as np
from scipy.special import erf

EPS = 1e-6  # RMSNorm epsilon (a reading: the pages do not define the block)


# ---------------------------------------------------------------------------
# SwiGLU block
# ---------------------------------------------------------------------------

def sigmoid(z):
    return 1.0 / (1.0 + np.exp(-z))


def silu(z):
    return z * sigmoid(z)


def rmsnorm_forward(x, gamma, eps=EPS):
    """r = (mean(x^2) + eps)^(-1/2) per row; n = x * r * gamma."""
    x = np.asarray(x, dtype=np.float64)
    r = 1.0 / np.sqrt(np.mean(x * x, axis=-1) + eps)
    n = x * r[:, None] * np.asarray(gamma, dtype=np.float64)[None, :]
    return n, r


def swiglu_forward(x, p, eps=EPS):
    """Forward of one SwiGLU block.  ``p`` has Wg, Wu [d,f], Wd [f,d], gamma [d].

    Returns (y, saved) where ``saved`` holds what the backward needs.
    """
    x = np.asarray(x, dtype=np.float64)
    n, r = rmsnorm_forward(x, p["gamma"], eps)
    g = n @ p["Wg"]
    u = n @ p["Wu"]
    h = silu(g) * u
    y = x + h @ p["Wd"]
    return y, {"x": x, "r": r, "n": n, "g": g, "u": u, "h": h}


def swiglu_backward_input(s, dy, p):
    """Input-gradient half (B) of one SwiGLU block's backward.

    Returns (dx, wsaved, dgamma) with ``wsaved`` = what the weight-gradient
    half (W) needs.  dgamma is produced here because it needs dn.
    """
    dy = np.asarray(dy, dtype=np.float64)
    x, r, g, u = s["x"], s["r"], s["g"], s["u"]
    d = x.shape[1]
    dh = dy @ p["Wd"].T
    sg = sigmoid(g)
    du = dh * g * sg                          # d/du of silu(g)*u
    dg = dh * u * sg * (1.0 + g * (1.0 - sg))  # d/dg of silu(g)*u
    dn = dg @ p["Wg"].T + du @ p["Wu"].T
    gamma = np.asarray(p["gamma"], dtype=np.float64)
    dgamma = np.sum(dn * x * r[:, None], axis=0)
    a = dn * gamma[None, :]
    # d r / d x_i = -r^3 x_i / d
    dx = dy + r[:, None] * a - (r ** 3)[:, None] * x * (np.sum(a * x, axis=1) / d)[:, None]
    return dx, {"n": s["n"], "h": s["h"], "dy": dy, "dg": dg, "du": du}, dgamma


def swiglu_backward_weight(ws):
    """Weight-gradient half (W): dWd = h^T dy, dWg = n^T dg, dWu = n^T du."""
    return {
        "Wg": ws["n"].T @ ws["dg"],
        "Wu": ws["n"].T @ ws["du"],
        "Wd": ws["h"].T @ ws["dy"],
    }


def swiglu_backward(s, dy, p):
    """Unsplit backward: returns (dx, grads) with grads keys Wg, Wu, Wd, gamma."""
    dx, ws, dgamma = swiglu_backward_input(s, dy, p)
    grads = swiglu_backward_weight(ws)
    grads["gamma"] = dgamma
    return dx, grads


def swiglu_block_at(x, dy, p, rows, wsel, gsel, eps=EPS):
    """One SwiGLU block's forward and backward, evaluated only where asked.

    The same definitions as ``swiglu_forward`` / ``swiglu_backward``, for
    blocks too wide to evaluate whole in float64 on the host:

    * ``rows``: token indices; y and dx are token-local, so their rows need
      only the sampled tokens' inputs.
    * ``wsel``: {"Wg"|"Wu"|"Wd": (I, J)}; dW[I][:, J] is a sum over every
      token, so it needs every token's n (or h) at the columns I and dg/du (or
      dy) at the columns J.
    * ``gsel``: feature indices K; dgamma[K] needs every token's dn at K,
      which needs every token's dg and du in full.

    Returns (y_rows, dx_rows, {"Wg"|"Wu"|"Wd": dW block}, dgamma_at_K).
    """
    x = np.asarray(x, dtype=np.float64)
    dy = np.asarray(dy, dtype=np.float64)
    d = x.shape[1]
    y_rows, s = swiglu_forward(x[rows], p, eps)
    dx_rows, _, _ = swiglu_backward_input(s, dy[rows], p)

    # every token: g, u (and h), dh, then dg, du
    n, r = rmsnorm_forward(x, p["gamma"], eps)
    g = n @ p["Wg"]
    u = n @ p["Wu"]
    h = silu(g) * u
    dh = dy @ p["Wd"].T
    sg = sigmoid(g)
    du = dh * g * sg
    dg = dh * u * sg * (1.0 + g * (1.0 - sg))
    dW = {}
    for key, (I, J) in wsel.items():
        if key == "Wd":
            dW[key] = h[:, I].T @ dy[:, J]
        elif key == "Wg":
            dW[key] = n[:, I].T @ dg[:, J]
        else:
            dW[key] = n[:, I].T @ du[:, J]
    dn_k = dg @ p["Wg"][gsel, :].T + du @ p["Wu"][gsel, :].T
    dgamma = np.sum(dn_k * x[:, gsel] * r[:, None], axis=0)
    return y_rows, dx_rows, dW, dgamma


# ---------------------------------------------------------------------------
# Toy block: Linear (with bias) + exact GELU
# ---------------------------------------------------------------------------

def phi_cdf(z):
    return 0.5 * (1.0 + erf(z / np.sqrt(2.0)))


def phi_pdf(z):
    return np.exp(-0.5 * z * z) / np.sqrt(2.0 * np.pi)


def gelu(z):
    return z * phi_cdf(z)


def toy_forward(x, p):
    """z = x W + b; y = GELU(z).  ``p`` has W [d_in, d_out], b [d_out]."""
    x = np.asarray(x, dtype=np.float64)
    z = x @ p["W"] + np.asarray(p["b"], dtype=np.float64)[None, :]
    return gelu(z), {"x": x, "z": z}


def toy_backward_input(s, dy, p):
    dy = np.asarray(dy, dtype=np.float64)
    z = s["z"]
    dz = dy * (phi_cdf(z) + z * phi_pdf(z))
    dx = dz @ p["W"].T
    return dx, {"x": s["x"], "dz": dz}


def toy_backward_weight(ws):
    return {"W": ws["x"].T @ ws["dz"], "b": np.sum(ws["dz"], axis=0)}


def toy_backward(s, dy, p):
    dx, ws = toy_backward_input(s, dy, p)
    return dx, toy_backward_weight(ws)


BLOCKS = {
    "swiglu": (swiglu_forward, swiglu_backward_input, swiglu_backward_weight),
    "toy": (lambda x, p, eps=EPS: toy_forward(x, p),
            lambda s, dy, p: toy_backward_input(s, dy, p) + (None,),
            toy_backward_weight),
}


# ---------------------------------------------------------------------------
# A stage = L blocks in sequence
# ---------------------------------------------------------------------------

def zero_grads(params):
    return [{k: np.zeros(np.shape(v), dtype=np.float64) for k, v in p.items()} for p in params]


def stage_forward(x, params, block="swiglu", eps=EPS):
    fwd = BLOCKS[block][0]
    saved = []
    for p in params:
        x, s = fwd(x, p, eps)
        saved.append(s)
    return x, saved


def stage_backward_input(saved, dy, params, block="swiglu"):
    """Input-gradient pass over the blocks in reverse.

    Returns (dx, wsaved_per_block, dgamma_per_block).
    """
    bwd_in = BLOCKS[block][1]
    ws_all = [None] * len(params)
    dgam = [None] * len(params)
    for b in reversed(range(len(params))):
        dy, ws, dg = bwd_in(saved[b], dy, params[b])
        ws_all[b] = ws
        dgam[b] = dg
    return dy, ws_all, dgam


def accumulate_weight_grads(acc, ws_all, dgam, block="swiglu"):
    bwd_w = BLOCKS[block][2]
    for b, ws in enumerate(ws_all):
        g = bwd_w(ws)
        for key, val in g.items():
            acc[b][key] += val
        if dgam[b] is not None:
            acc[b]["gamma"] += dgam[b]


def stage_backward(saved, dy, params, acc, block="swiglu"):
    dx, ws_all, dgam = stage_backward_input(saved, dy, params, block)
    accumulate_weight_grads(acc, ws_all, dgam, block)
    return dx


def full_batch_step(xs, dys, params, block="swiglu", eps=EPS):
    """Non-pipelined reference ([Sched §09]: compare against the gradients
    of the un-pipelined step): concatenate the micro-batches along rows, run
    one forward and one backward, gradients summed over all rows.

    Returns (ys, dxs, grads) with ys/dxs split back per micro-batch.
    """
    sizes = [np.shape(x)[0] for x in xs]
    X = np.concatenate([np.asarray(x, dtype=np.float64) for x in xs], axis=0)
    DY = np.concatenate([np.asarray(d, dtype=np.float64) for d in dys], axis=0)
    Y, saved = stage_forward(X, params, block, eps)
    acc = zero_grads(params)
    DX = stage_backward(saved, DY, params, acc, block)
    cut = np.cumsum(sizes)[:-1]
    return np.split(Y, cut), np.split(DX, cut), acc


def run_stage_ops(ops, xs, dys, params, block="swiglu", eps=EPS, recompute=False, trace=None):
    """Execute one stage's op list in order, as the executor does.

    ``ops`` is a list of (kind, mb, chunk) with kinds 0=F, 1=B, 2=W (only
    chunk 0 here).  A dict plays the activation stash: F stores, B pops
    ([1F1B §5.2] activations dict).  Gradients accumulate in op order.

    ``recompute``: the stash keeps only the stage input, and B first runs the
    forward again from it to get back what the blocks saved ([GPipe→ZB
    "GPipe 2018年"]: only the boundary between devices is kept, each layer's
    forward is redone when the backward reaches it).  Not defined with W ops.
    ``trace``, if a list, receives after each op the number of stash entries
    and the float64 elements they hold.
    Returns (ys, dxs, grads).
    """
    stash, pend = {}, {}
    ys, dxs = {}, {}
    acc = zero_grads(params)
    split = any(o[0] == 2 for o in ops)
    assert not (split and recompute)
    for kind, i, _c in ops:
        if kind == 0:
            ys[i], saved = stage_forward(xs[i], params, block, eps)
            stash[i] = np.array(xs[i], dtype=np.float64, copy=True) if recompute else saved
        elif kind == 1:
            saved = stash.pop(i)
            if recompute:
                _, saved = stage_forward(saved, params, block, eps)
            dxs[i], ws_all, dgam = stage_backward_input(saved, dys[i], params, block)
            if split:
                pend[i] = (ws_all, dgam)
            else:
                accumulate_weight_grads(acc, ws_all, dgam, block)
        else:
            ws_all, dgam = pend.pop(i)
            accumulate_weight_grads(acc, ws_all, dgam, block)
        if trace is not None:
            held = sum(e.size if recompute else sum(a.size for blk in e for a in blk.values())
                       for e in stash.values())
            trace.append((len(stash), held))
    assert not stash and not pend
    M = len(xs)
    return [ys[i] for i in range(M)], [dxs[i] for i in range(M)], acc


def linear_probe_loss(ys, Gs):
    """L = (1/M) sum_i <y_i, G_i>; its output gradient is G_i / M
    ([1F1B §5.2]: the last stage divides the loss gradient by M)."""
    M = len(ys)
    return sum(float(np.sum(np.asarray(y) * np.asarray(g))) for y, g in zip(ys, Gs)) / M


def pipeline_model_step(xs, Gs, stage_params, block="swiglu", eps=EPS):
    """Reference for the P-stage emulation: the whole P*L-block model on the
    full batch, with the linear-probe loss (dy_i = G_i / M at the output).

    Returns (ys_last, dxs_first, grads_per_stage).
    """
    M = len(xs)
    sizes = [np.shape(x)[0] for x in xs]
    cut = np.cumsum(sizes)[:-1]
    X = np.concatenate([np.asarray(x, dtype=np.float64) for x in xs], axis=0)
    saved_all = []
    for params in stage_params:
        X, saved = stage_forward(X, params, block, eps)
        saved_all.append(saved)
    DY = np.concatenate([np.asarray(g, dtype=np.float64) for g in Gs], axis=0) / M
    grads = []
    for params, saved in zip(reversed(stage_params), reversed(saved_all)):
        acc = zero_grads(params)
        DY = stage_backward(saved, DY, params, acc, block)
        grads.append(acc)
    grads.reverse()
    return np.split(X, cut), np.split(DY, cut), grads


def rel_l2(a, ref):
    """||a - ref||_2 / ||ref||_2 in float64 over the whole tensor."""
    a = np.asarray(a, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    den = np.linalg.norm(ref.ravel())
    num = np.linalg.norm((a - ref).ravel())
    if den == 0.0:
        return 0.0 if num == 0.0 else float("inf")
    return float(num / den)


def executed_flops_per_block_microbatch(T, d, f, recompute=False):
    """GEMM FLOPs actually run per block per micro-batch: the algorithmic
    18Tdf, plus the forward's 6Tdf again when B recomputes it."""
    return (24 if recompute else 18) * T * d * f


def flops_per_block_microbatch(T, d, f):
    """Algorithmic F+B FLOPs of one SwiGLU block on one micro-batch:
    forward 6Tdf (gate/up 4Tdf + down 2Tdf), input-gradient 6Tdf, weight
    gradient 6Tdf.  Norm and elementwise work is not counted."""
    return 18 * T * d * f
