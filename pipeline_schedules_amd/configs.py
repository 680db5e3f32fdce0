"""Named stage workloads.

Each preset fixes the pipeline shape (P stages, M micro-batches, stage index
k, v virtual chunks per device, schedule kind) and the stage's blocks (block
type, dtype, L blocks per chunk, model dim d, ffn dim f, T tokens per
micro-batch).  The shapes are the workloads the executor is built and
measured for; the 80-layer / 8-stage / v=2 layout and the micro-batch of 2
sequences follow the [lpnh] article's example (lpnh.cn/news/2768528).
"""

from __future__ import annotations

from dataclasses import dataclass, replace


@dataclass(frozen=True)
class StageConfig:
    name: str
    P: int
    M: int
    k: int
    v: int
    kind: str          # "1f1b" (interleaved when v > 1), "gpipe", "zb1p", "zb2p"
    block: str         # "swiglu" or "toy"
    dtype: str         # "bf16" or "fp32"
    L: int             # blocks per chunk
    d: int
    f: int             # ffn dim (toy block: output dim == d)
    T: int             # tokens (rows) per micro-batch
    eps: float = 1e-6
    seed: int = 0
    w_std: float = 0.02
    x_std: float = 1.0
    g_std: float = 0.01

    def with_(self, **kw) -> "StageConfig":
        return replace(self, **kw)

    @property
    def blocks_per_stage(self) -> int:
        return self.L * self.v

    def flops_per_microbatch(self) -> int:
        """Algorithmic F+B FLOPs of this stage on one micro-batch.

        SwiGLU: 18*T*d*f per block (forward 6, input grad 6, weight grad 6).
        Toy: 3 GEMMs of 2*T*d*d per block.
        """
        if self.block == "swiglu":
            return 18 * self.T * self.d * self.f * self.blocks_per_stage
        return 6 * self.T * self.d * self.d * self.blocks_per_stage


# Smallest workload: 2 stages x 4 micro-batches, each stage two
# Linear(64->64)+GELU layers, micro-batch 8x64, fp32.
C1_TOY = StageConfig("c1_toy", P=2, M=4, k=0, v=1, kind="1f1b", block="toy",
                     dtype="fp32", L=2, d=64, f=64, T=8)

# 4 stages x 6 micro-batches; each stage 2 SwiGLU blocks d=1024 f=2816;
# micro-batch 4x512 tokens; bf16.
C2_SMALL = StageConfig("c2_swiglu_p4m6", P=4, M=6, k=0, v=1, kind="1f1b",
                       block="swiglu", dtype="bf16", L=2, d=1024, f=2816, T=2048)

# One stage (k=0 of P=8, stash 8) of an 80-layer model: 10 SwiGLU blocks
# d=8192 f=28672, micro-batch 2x4096 tokens, M=16; bf16.
C3_SLICE = StageConfig("c3_80layer_p8_stage0", P=8, M=16, k=0, v=1, kind="1f1b",
                       block="swiglu", dtype="bf16", L=10, d=8192, f=28672, T=8192)

# The same slice, interleaved v=2: two chunks of 5 blocks.
C4_INTERLEAVED = C3_SLICE.with_(name="c4_80layer_p8_v2", v=2, L=5)

# Zero-Bubble split: P=4, M=32, 8 blocks d=4096 f=14336, micro-batch 4x2048.
C5_ZB = StageConfig("c5_zb1p_p4m32", P=4, M=32, k=0, v=1, kind="zb1p",
                    block="swiglu", dtype="bf16", L=8, d=4096, f=14336, T=8192)

# The same stage under ZB2P (2(P-k)-1 warmup forwards, W budget 2P, larger stash).
C6_ZB2P = C5_ZB.with_(name="c6_zb2p_p4m32", kind="zb2p")

# The same stage unsplit (plain 1F1B): the reference point for the cost of the split.
C5_UNSPLIT = C5_ZB.with_(name="c5u_1f1b_p4m32", kind="1f1b")

PRESETS = {c.name: c for c in (C1_TOY, C2_SMALL, C3_SLICE, C4_INTERLEAVED, C5_ZB, C6_ZB2P, C5_UNSPLIT)}
