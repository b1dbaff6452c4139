"""CPU oracle for the LoGRA sketch / merge / predicted-KL hot path.

TEST INFRASTRUCTURE ONLY.  Nothing in the library imports this package: only
the tests, the smoke check and the benchmark's CPU-baseline leg may use it.
It is a plain, slow, fp64 NumPy restatement of what the method computes, so a
reader can check each function against the source pages by eye.  It shares no
code, constants module or helper with the HIP path.

Sources (cited by short tag in every module):
  [LoGRA] wispaper.ai research summary of "LoGRA: Scaling LLM Reinforcement
          Learning with Low-Rank Gradient Sketches".  Sections:
            Sketch - "草图如何取代完整梯度缓冲" (how the sketch replaces the
                     full gradient buffer)
            Sync   - "同一份草图也压缩策略同步开销" (the same sketch also
                     compresses policy sync)
            PKL    - "预测 KL 控制防止过大更新破坏学习" (predicted-KL control)
            Rank   - "投影秩比基刷新更重要" (projection rank matters more than
                     basis refresh)
  [EVAL]  cloud.baidu.com evaluation guide for low-rank gradient compression
          schemes, section 3 (description of the evaluated mechanism).
  [SALMON11] Salmon, Moraes, Dror, Shaw, "Parallel Random Numbers: As Easy as
          1, 2, 3", SC'11 (Philox4x64-10).
  [BOXMULLER58] Box & Muller, "A Note on the Generation of Random Normal
          Deviates", Ann. Math. Statist. 1958.

Notation (the only reading under which the pages' shapes type-check):
  W  d x k  layer weight, Y = X @ W.T   (d = out features, k = in features)
  X  T x k  layer input saved for backward (bf16 values)
  dY T x d  gradient of the layer output (bf16 values)
  G  = dY.T @ X            d x k  (never formed on the GPU path)
  A  r x k  seeded projection
  S  = G @ A.T             d x r  (fp32 accumulator on the GPU path)

Parity status per function:
  bf16, philox, projection (Rademacher), sketch, merge, kl, controller:
      pinned (see tests/test_oracle_*.py).
  projection (Gaussian): the generator's statistics are pinned; its exact
      element values are "parity unpinned" (fp64 Box-Muller here vs fp32
      hardware transcendentals on the GPU, compared to within one bf16 ulp).
  optim (stateful sketch update rules): "parity unpinned" - the pages name
      stateful sketch optimizers without defining one; the textbook momentum
      and Adam rules used here are pinned against closed forms only.
"""

from . import bf16, philox, projection, sketch, merge, kl, optim  # noqa: F401
