"""Seeded random stage configurations against the float64 oracle.

Each case draws a pipeline shape (P, k, M), a schedule kind, a block count,
a dtype and token/feature sizes that mix ragged and whole 256-wide tiles,
plus sometimes the recompute mode, then checks the op log against the
oracle's schedule exactly and every output, input gradient and weight
gradient against the oracle's full-batch step (rel-L2 <= 2e-2 bf16,
<= 1e-5 fp32)."""

import numpy as np
import pytest

from oracle import schedule as S

pytestmark = pytest.mark.gpu

TOL = {"bf16": 2e-2, "fp32": 1e-5}
SIZES_T = [1, 7, 64, 255, 256, 300, 512]
SIZES_F = [8, 40, 136, 256, 264, 392, 512]


@pytest.fixture(scope="module")
def env():
    import torch
    from pipeline_schedules_amd import pps
    from tests import gpu_util as G
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    pps.lib()
    return torch, pps, G


def _draw(case):
    rng = np.random.default_rng(20260 + case)
    P = int(rng.integers(1, 5))
    k = int(rng.integers(0, P))
    M = int(rng.integers(1, 7))
    kind = ["1f1b", "gpipe", "zb1p", "zb2p"][int(rng.integers(0, 4))]
    dtype = ["bf16", "fp32"][int(rng.integers(0, 2))]
    L = int(rng.integers(1, 3))
    T = int(rng.choice(SIZES_T))
    d = int(rng.choice(SIZES_F))
    f = int(rng.choice(SIZES_F))
    recompute = kind in ("1f1b", "gpipe") and bool(rng.integers(0, 3) == 0)
    if case % 4 == 0:   # bf16 on whole tiles: the dh epilogue's T-contiguous outputs
        dtype, T, f = "bf16", int(rng.choice([256, 512])), int(rng.choice([256, 512]))
    elif case % 4 == 1:   # recompute mode
        kind, recompute = ["1f1b", "gpipe"][int(rng.integers(0, 2))], True
    return dict(P=P, k=k, M=M, kind=kind, dtype=dtype, L=L, T=T, d=d, f=f, recompute=recompute)


@pytest.mark.parametrize("case", range(48))
def test_random_stage(env, case):
    from pipeline_schedules_amd.configs import StageConfig
    from pipeline_schedules_amd.inputs import make_inputs
    from tests.test_gpu_stage import _check, _run_single
    torch, pps, G = env
    c = _draw(case)
    print(c, flush=True)
    cfg = StageConfig(f"random{case}", P=c["P"], M=c["M"], k=c["k"], v=1, kind=c["kind"], block="swiglu",
                      dtype=c["dtype"], L=c["L"], d=c["d"], f=c["f"], T=c["T"])
    inp = make_inputs(cfg, gamma="random")
    flags = pps.FLAG_RECOMPUTE if c["recompute"] else 0
    got = _run_single(env, cfg, inp, c["kind"], flags=flags)
    _check(cfg, got, inp, TOL[c["dtype"]])
    # the stash never holds more than the schedule's peak
    peak = max(o[4] for o in S.stage_ops(cfg.P, cfg.M, cfg.k, 1, {"1f1b": S.ONE_F_ONE_B, "gpipe": S.GPIPE,
                                                                   "zb1p": S.ZB1P, "zb2p": S.ZB2P}[c["kind"]]))
    assert got[3]["peak_live_entries"] == peak
