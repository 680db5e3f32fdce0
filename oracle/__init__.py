"""CPU oracle for the 1F1B pipeline-stage executor -- TEST INFRASTRUCTURE ONLY.

This package is the plain, slow, obviously-correct reference that the HIP path
is checked against.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import it.  The product library under
``pipeline_schedules_amd/`` never imports, links or executes anything here, and
nothing here imports the product library.

Modules
-------
schedule  -- integer schedule generation (GPipe, 1F1B, interleaved 1F1B,
             ZB1P/ZB2P) and a unit-cost dependency simulator of all P stages.
numerics  -- float64 forward/backward of the stage blocks (RMSNorm + SwiGLU
             MLP with residual; the toy Linear+GELU block), the full-batch
             step and the P-stage reference model.

Page legend used in citations throughout this package
-----------------------------------------------------
[1F1B]        page "2. 1F1B" (sgdbs.github.io, AI_Infra notes, PipelineParallel)
[GPipe->ZB]   page "流水线并行：从 GPipe 到 1F1B 与 Zero Bubble" (dlog.com.cn)
[Sched]       page "流水线调度：GPipe、1F1B、交错与计算通信重叠" (xuujii.github.io)
[Megatron-PP] page "Megatron-LM 分布式训练（三）：流水线并行 PP 与 1F1B 调度"
              (swordlidev.github.io)
[lpnh]        article lpnh.cn/news/2768528 on 1F1B / interleaved scheduling
"""
