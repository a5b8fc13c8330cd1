"""CPU oracle for the encoder-layer forward with padding removal (TEST INFRASTRUCTURE).

A plain, slow, obviously correct float64 NumPy implementation of what the GPU
library computes. It exists only to check the GPU path: the tests, the smoke
check and the benchmark's CPU-baseline leg are the only code allowed to import
it. The GPU library never calls it, and it shares no code with the GPU library
(no kernels, headers, helpers or tables); the only module both sides' callers
use is the seeded input generator, which holds no arithmetic of the method.

Pages cited by title (the reference is a set of web pages):
  [KS]  Kuaishou heterogeneous-computing article, "GPU底层优化 | 如何让Transformer在GPU上
        跑得更快？" ("How to make Transformer run faster on GPU"), Figs. 6-11.
  [SW]  NVIDIA talk on Swin Transformer, "大規模なビジュアル モデルを使用してトレーニングと
        推論を高速化するにはどうすればよいですか?" ("How to accelerate training and inference
        of large visual models"), sections 1 (Swin introduction), 2 (training),
        3 (inference).
  [TRT] "通過稀疏支持和Transformer優化增強AI推理" (TensorRT 8 overview).
  [P5]  "揭秘Transformer模型：速度优化与量化技术" (speed optimisation and quantisation).

Modules:
  encoder  offsets, padding removal/rebuild, the post-LN encoder layer and stack
  int8     int8-GEMM variant of the layer (quantise, int32 accumulate, dequantise)
  swin     shifted-window attention block with relative-position bias
  sparse   2:4 structured-sparse projection weights (magnitude pruning, compressed form)

Every function is pinned by tests under tests/ (test_oracle_*.py) against brute
force, a textbook library routine, closed forms or invariants; none is "parity
unpinned".
"""
from . import encoder, int8, sparse, swin  # noqa: F401
