"""Pins of the float64 numerics oracle.  CPU only.

Each block's backward (hand-derived in the oracle) is pinned to torch.autograd
in float64 on the CPU (an independent derivation of the same gradients from
the forward definition) and to central finite differences; the forward to
closed forms and invariants; the pipelined result to the full-batch step
([Sched §09]; [1F1B §4.5]: synchronous 1F1B equals one large-batch step).
"""

import math

import numpy as np
import pytest
import torch

from oracle import numerics as N
from oracle import schedule as S


def _rand_swiglu(rng, d, f, gamma_random=True):
    p = {
        "Wg": rng.normal(0, 0.3, (d, f)),
        "Wu": rng.normal(0, 0.3, (d, f)),
        "Wd": rng.normal(0, 0.3, (f, d)),
        "gamma": 1.0 + rng.normal(0, 0.2, (d,)) if gamma_random else np.ones(d),
    }
    return p


def _torch_swiglu(x, p, eps):
    r = torch.rsqrt((x * x).mean(dim=-1, keepdim=True) + eps)
    n = x * r * p["gamma"]
    g = n @ p["Wg"]
    u = n @ p["Wu"]
    return x + (torch.nn.functional.silu(g) * u) @ p["Wd"]


@pytest.mark.parametrize("T,d,f", [(5, 8, 16), (7, 16, 24), (1, 4, 4)])
def test_swiglu_backward_matches_autograd(T, d, f):
    rng = np.random.default_rng(1)
    p = _rand_swiglu(rng, d, f)
    x = rng.normal(0, 1, (T, d))
    dy = rng.normal(0, 1, (T, d))
    y, s = N.swiglu_forward(x, p, eps=1e-3)
    dx, grads = N.swiglu_backward(s, dy, p)

    tp = {k: torch.tensor(v, dtype=torch.float64, requires_grad=True) for k, v in p.items()}
    tx = torch.tensor(x, dtype=torch.float64, requires_grad=True)
    ty = _torch_swiglu(tx, tp, 1e-3)
    ty.backward(torch.tensor(dy, dtype=torch.float64))
    np.testing.assert_allclose(y, ty.detach().numpy(), rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(dx, tx.grad.numpy(), rtol=1e-10, atol=1e-12)
    for k in ("Wg", "Wu", "Wd", "gamma"):
        np.testing.assert_allclose(grads[k], tp[k].grad.numpy(), rtol=1e-10, atol=1e-12)


def test_swiglu_block_at_matches_autograd():
    # The entry-sampled evaluation used at full width equals torch.autograd's
    # gradients of the same block at those entries (rows of y and dx, blocks
    # of every dW, entries of dgamma).
    rng = np.random.default_rng(11)
    T, d, f = 29, 16, 24
    p = _rand_swiglu(rng, d, f)
    x = rng.normal(0, 1, (T, d))
    dy = rng.normal(0, 1, (T, d))
    tp = {k: torch.tensor(v, dtype=torch.float64, requires_grad=True) for k, v in p.items()}
    tx = torch.tensor(x, dtype=torch.float64, requires_grad=True)
    ty = _torch_swiglu(tx, tp, 1e-3)
    ty.backward(torch.tensor(dy, dtype=torch.float64))
    rows = np.array([0, 3, 17, 28])
    wsel = {"Wg": (np.array([1, 5, 15]), np.array([0, 7, 23])), "Wu": (np.array([2, 9]), np.array([4, 11, 20])),
            "Wd": (np.array([0, 13, 22]), np.array([3, 15]))}
    gsel = np.array([0, 6, 15])
    y_r, dx_r, dW, dgam = N.swiglu_block_at(x, dy, p, rows, wsel, gsel, eps=1e-3)
    np.testing.assert_allclose(y_r, ty.detach().numpy()[rows], rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(dx_r, tx.grad.numpy()[rows], rtol=1e-10, atol=1e-12)
    for k, (I, J) in wsel.items():
        np.testing.assert_allclose(dW[k], tp[k].grad.numpy()[np.ix_(I, J)], rtol=1e-10, atol=1e-12)
    np.testing.assert_allclose(dgam, tp["gamma"].grad.numpy()[gsel], rtol=1e-10, atol=1e-12)


def test_toy_backward_matches_autograd():
    rng = np.random.default_rng(2)
    p = {"W": rng.normal(0, 0.5, (6, 6)), "b": rng.normal(0, 0.5, (6,))}
    x = rng.normal(0, 1, (4, 6))
    dy = rng.normal(0, 1, (4, 6))
    y, s = N.toy_forward(x, p)
    dx, grads = N.toy_backward(s, dy, p)
    tW = torch.tensor(p["W"], requires_grad=True)
    tb = torch.tensor(p["b"], requires_grad=True)
    tx = torch.tensor(x, requires_grad=True)
    ty = torch.nn.functional.gelu(tx @ tW + tb, approximate="none")
    ty.backward(torch.tensor(dy))
    np.testing.assert_allclose(y, ty.detach().numpy(), rtol=1e-12, atol=1e-14)
    np.testing.assert_allclose(dx, tx.grad.numpy(), rtol=1e-10, atol=1e-13)
    np.testing.assert_allclose(grads["W"], tW.grad.numpy(), rtol=1e-10, atol=1e-13)
    np.testing.assert_allclose(grads["b"], tb.grad.numpy(), rtol=1e-10, atol=1e-13)


def test_stage_gradients_finite_differences():
    # Tiny shapes (d=8, f=16, T=4, L=2): central differences of the
    # linear-probe loss <y, G> against every gradient of the stage.
    rng = np.random.default_rng(3)
    d, f, T, L = 8, 16, 4, 2
    params = [_rand_swiglu(rng, d, f) for _ in range(L)]
    x = rng.normal(0, 1, (T, d))
    G = rng.normal(0, 1, (T, d))
    eps = 1e-2

    def loss(params, x):
        y, _ = N.stage_forward(x, params, "swiglu", eps)
        return float(np.sum(y * G))

    y, saved = N.stage_forward(x, params, "swiglu", eps)
    acc = N.zero_grads(params)
    dx = N.stage_backward(saved, G, params, acc, "swiglu")
    h = 1e-6
    for b in range(L):
        for key in ("Wg", "Wu", "Wd", "gamma"):
            arr = params[b][key]
            flat = arr.reshape(-1)
            for idx in rng.choice(flat.size, size=min(6, flat.size), replace=False):
                old = flat[idx]
                flat[idx] = old + h
                lp = loss(params, x)
                flat[idx] = old - h
                lm = loss(params, x)
                flat[idx] = old
                fd = (lp - lm) / (2 * h)
                assert abs(fd - acc[b][key].reshape(-1)[idx]) < 1e-6 * max(1.0, abs(fd))
    for idx in range(x.size):
        xp = x.copy().reshape(-1)
        xp[idx] += h
        lp = loss(params, xp.reshape(x.shape))
        xp[idx] -= 2 * h
        lm = loss(params, xp.reshape(x.shape))
        fd = (lp - lm) / (2 * h)
        assert abs(fd - dx.reshape(-1)[idx]) < 1e-6 * max(1.0, abs(fd))


def test_toy_gradients_finite_differences():
    rng = np.random.default_rng(4)
    params = [{"W": rng.normal(0, 0.5, (5, 5)), "b": rng.normal(0, 0.5, (5,))} for _ in range(2)]
    x = rng.normal(0, 1, (3, 5))
    G = rng.normal(0, 1, (3, 5))
    y, saved = N.stage_forward(x, params, "toy")
    acc = N.zero_grads(params)
    dx = N.stage_backward(saved, G, params, acc, "toy")
    h = 1e-6
    for b in range(2):
        for key in ("W", "b"):
            flat = params[b][key].reshape(-1)
            for idx in range(flat.size):
                old = flat[idx]
                flat[idx] = old + h
                lp = float(np.sum(N.stage_forward(x, params, "toy")[0] * G))
                flat[idx] = old - h
                lm = float(np.sum(N.stage_forward(x, params, "toy")[0] * G))
                flat[idx] = old
                assert abs((lp - lm) / (2 * h) - acc[b][key].reshape(-1)[idx]) < 1e-7


def test_closed_form_zero_down_projection():
    # Wd = 0: y = x, dx = dy exactly, dWg = dWu = 0, dgamma = 0, dWd = h^T dy.
    rng = np.random.default_rng(5)
    d, f, T = 12, 20, 9
    p = _rand_swiglu(rng, d, f)
    p["Wd"] = np.zeros((f, d))
    x = rng.normal(0, 1, (T, d))
    dy = rng.normal(0, 1, (T, d))
    y, s = N.swiglu_forward(x, p)
    assert np.array_equal(y, x)
    dx, g = N.swiglu_backward(s, dy, p)
    assert np.array_equal(dx, dy)
    assert not g["Wg"].any() and not g["Wu"].any() and not g["gamma"].any()
    n = s["n"]
    gg = n @ p["Wg"]
    h = gg / (1 + np.exp(-gg)) * (n @ p["Wu"])
    np.testing.assert_allclose(g["Wd"], h.T @ dy, rtol=1e-13)


def test_closed_form_zero_gate():
    # Wg = 0: g = 0, silu(0) = 0 so h = 0 and y = x; dWd = 0; the only
    # non-zero weight gradient is dWg = n^T (dh * u * 1/2).
    rng = np.random.default_rng(6)
    d, f, T = 8, 8, 5
    p = _rand_swiglu(rng, d, f)
    p["Wg"] = np.zeros((d, f))
    x = rng.normal(0, 1, (T, d))
    dy = rng.normal(0, 1, (T, d))
    y, s = N.swiglu_forward(x, p)
    assert np.array_equal(y, x)
    dx, g = N.swiglu_backward(s, dy, p)
    assert not g["Wd"].any() and not g["Wu"].any()
    dh = dy @ p["Wd"].T
    np.testing.assert_allclose(g["Wg"], s["n"].T @ (dh * s["u"] * 0.5), rtol=1e-12)


def test_rmsnorm_invariants():
    rng = np.random.default_rng(7)
    x = rng.normal(0, 3, (6, 10))
    n, r = N.rmsnorm_forward(x, np.ones(10), eps=0.0)
    np.testing.assert_allclose(np.mean(n * n, axis=1), 1.0, rtol=1e-14)
    n2, _ = N.rmsnorm_forward(7.5 * x, np.ones(10), eps=0.0)
    np.testing.assert_allclose(n2, n, rtol=1e-13)
    # a row of constant c has r = 1/sqrt(c^2 + eps)
    c = np.full((1, 4), 2.0)
    _, rc = N.rmsnorm_forward(c, np.ones(4), eps=0.25)
    assert rc[0] == 1.0 / math.sqrt(4.25)


def test_rmsnorm_backward_identity():
    # x . (dx - dy) = eps * r^3 * (a . x) per row, a = dn * gamma
    # (zero when eps = 0: the norm is scale invariant).
    rng = np.random.default_rng(8)
    d, f, T = 16, 24, 6
    p = _rand_swiglu(rng, d, f)
    x = rng.normal(0, 1, (T, d))
    dy = rng.normal(0, 1, (T, d))
    for eps in (0.0, 0.5):
        y, s = N.swiglu_forward(x, p, eps)
        dx, _ws, _dg = N.swiglu_backward_input(s, dy, p)
        dh = dy @ p["Wd"].T
        sg = 1 / (1 + np.exp(-s["g"]))
        dn = (dh * s["u"] * sg * (1 + s["g"] * (1 - sg))) @ p["Wg"].T + (dh * s["g"] * sg) @ p["Wu"].T
        a = dn * p["gamma"]
        lhs = np.sum(x * (dx - dy), axis=1)
        rhs = eps * s["r"] ** 3 * np.sum(a * x, axis=1)
        np.testing.assert_allclose(lhs, rhs, atol=1e-11)


def test_activation_reference_values():
    assert N.sigmoid(np.array(0.0)) == 0.5
    assert N.silu(np.array(0.0)) == 0.0
    # GELU(1) = Phi(1) = 0.8413447460685429 (standard normal table)
    assert abs(float(N.gelu(np.array(1.0))) - 0.8413447460685429) < 1e-15
    z = np.linspace(-4, 4, 33)
    np.testing.assert_allclose(N.gelu(-z), N.gelu(z) - z, atol=1e-14)
    # GELU'(0) = 1/2
    assert abs(float(N.phi_cdf(0.0) + 0.0 * N.phi_pdf(0.0)) - 0.5) < 1e-16


def _toy_cfg_params(rng, L, d):
    return [{"W": rng.normal(0, 0.3, (d, d)), "b": rng.normal(0, 0.3, (d,))} for _ in range(L)]


@pytest.mark.parametrize("block", ["swiglu", "toy"])
def test_pipelined_orders_equal_full_batch(block):
    # 1F1B order, GPipe order and the ZB1P split order give the full-batch
    # outputs, input gradients and summed weight gradients.
    rng = np.random.default_rng(9)
    P, M, k, T, d, f, L = 4, 6, 1, 5, 8, 12, 2
    if block == "swiglu":
        params = [_rand_swiglu(rng, d, f) for _ in range(L)]
    else:
        params = _toy_cfg_params(rng, L, d)
    xs = [rng.normal(0, 1, (T, d)) for _ in range(M)]
    dys = [rng.normal(0, 1, (T, d)) for _ in range(M)]
    ys_f, dxs_f, g_f = N.full_batch_step(xs, dys, params, block)
    orders = {
        "1f1b": S.one_f_one_b(P, M, k),
        "gpipe": S.gpipe(P, M, k),
        "zb1p": S.simulate_zb(P, M, 1)[0][k],
    }
    for name, ops in orders.items():
        ys, dxs, g = N.run_stage_ops(ops, xs, dys, params, block)
        for i in range(M):
            assert N.rel_l2(ys[i], ys_f[i]) < 1e-14
            assert N.rel_l2(dxs[i], dxs_f[i]) < 1e-14
        for b in range(L):
            for key in g[b]:
                assert N.rel_l2(g[b][key], g_f[b][key]) < 1e-13, (name, b, key)


@pytest.mark.parametrize("block", ["swiglu", "toy"])
def test_recompute_mode_equals_stash_mode(block):
    # Recomputing the forward inside B from the stashed stage input gives the
    # very arrays the forward saved, so every result is bit-identical; the
    # stash then holds T*d elements per entry whatever the depth L, against
    # L blocks' worth when the forward's tensors are kept.
    rng = np.random.default_rng(12)
    P, M, k, T, d, f = 4, 6, 1, 5, 8, 12
    held_per_entry = {}
    for L in (1, 3):
        params = ([_rand_swiglu(rng, d, f) for _ in range(L)] if block == "swiglu"
                  else _toy_cfg_params(rng, L, d))
        xs = [rng.normal(0, 1, (T, d)) for _ in range(M)]
        dys = [rng.normal(0, 1, (T, d)) for _ in range(M)]
        for ops, peak in ((S.one_f_one_b(P, M, k), P - k), (S.gpipe(P, M, k), M)):
            tr_s, tr_r = [], []
            ys, dxs, g = N.run_stage_ops(ops, xs, dys, params, block, trace=tr_s)
            ys_r, dxs_r, g_r = N.run_stage_ops(ops, xs, dys, params, block, recompute=True, trace=tr_r)
            for i in range(M):
                assert np.array_equal(ys[i], ys_r[i]) and np.array_equal(dxs[i], dxs_r[i])
            for b in range(L):
                for key in g[b]:
                    assert np.array_equal(g[b][key], g_r[b][key]), (L, b, key)
            assert [n for n, _ in tr_s] == [n for n, _ in tr_r]
            assert max(n for n, _ in tr_r) == peak
            for n, held in tr_r:
                assert held == n * T * d
            per = {held // n for n, held in tr_s if n}
            assert len(per) == 1
            held_per_entry[L] = per.pop()
    if block == "swiglu":   # x, n [T,d]; r [T]; g, u, h [T,f] per block
        per_block = 2 * T * d + T + 3 * T * f
    else:                   # x, z [T,d] per block
        per_block = 2 * T * d
    assert held_per_entry == {1: per_block, 3: 3 * per_block}
    assert N.executed_flops_per_block_microbatch(T, d, f, True) / N.flops_per_block_microbatch(T, d, f) == 4 / 3


def test_token_independence():
    # Rows are independent: the forward of a batch is the row-concatenation
    # of the forwards of its parts.
    rng = np.random.default_rng(10)
    params = [_rand_swiglu(rng, 8, 12) for _ in range(2)]
    x = rng.normal(0, 1, (9, 8))
    y, _ = N.stage_forward(x, params)
    for i in range(9):
        yi, _ = N.stage_forward(x[i:i + 1], params)
        np.testing.assert_allclose(yi[0], y[i], rtol=1e-13, atol=1e-13)


def test_pipeline_model_probe_gradient():
    # The linear-probe loss L = (1/M) sum <y_i, G_i> has dL/dy_i = G_i / M;
    # check the P-stage reference model's input gradient by finite differences.
    rng = np.random.default_rng(11)
    P, M, T, d = 2, 3, 2, 5
    stage_params = [_toy_cfg_params(rng, 2, d) for _ in range(P)]
    xs = [rng.normal(0, 1, (T, d)) for _ in range(M)]
    Gs = [rng.normal(0, 1, (T, d)) for _ in range(M)]
    ys, dxs, grads = N.pipeline_model_step(xs, Gs, stage_params, "toy")

    def loss(xs):
        X = np.concatenate(xs)
        for p in stage_params:
            X, _ = N.stage_forward(X, p, "toy")
        return N.linear_probe_loss(np.split(X, M), Gs)

    h = 1e-6
    for i in range(M):
        for idx in range(T * d):
            xp = [x.copy() for x in xs]
            xp[i].reshape(-1)[idx] += h
            lp = loss(xp)
            xp[i].reshape(-1)[idx] -= 2 * h
            lm = loss(xp)
            assert abs((lp - lm) / (2 * h) - dxs[i].reshape(-1)[idx]) < 1e-8


def test_rel_l2():
    a = np.array([3.0, 4.0])
    assert N.rel_l2(a, a) == 0.0
    assert abs(N.rel_l2(np.array([3.0, 5.0]), a) - 0.2) < 1e-15
