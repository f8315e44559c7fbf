"""CPU oracle for SageBwd-style INT8 trainable attention.

TEST INFRASTRUCTURE ONLY. Nothing in the product path may import, call or link
anything here: only the test suite, the smoke check and the benchmark's CPU
baseline leg use it. It shares no code with the HIP kernels and imports nothing
from the product package.

Two references, both plain and slow, written from the pages:

  oracle.quant  - the quantised algorithm (O-Q): QK-norm and K-smoothing and the
                  per-block INT8 quantisation of Q, K, V and dO specified operation by
                  operation in float32 (so the GPU's codes and scales must match bit
                  for bit), then the tiled forward and backward in float64 with the
                  in-kernel quantisation of P~, P and dS on the same tiles as the
                  kernels use.
  oracle.exact  - full-precision float64 attention with QK-norm (O-X), forward and
                  backward, no quantisation.

Citations name the page and paragraph. "SageBwd article" is the page
"SageBwd: a trainable low-bit attention mechanism" (aitrends.kr, article 8227);
its paragraphs are named by topic: precision split, QK-norm, K-smoothing,
per-block kernels, dS magnitude bound, gradient amplification, Q-smoothing.

Parity status: every function is pinned by the tests named in its docstring
(finite differences, closed forms, library routines, identity-quantiser and
lossless-quantiser reductions, quantisation error bounds). None is "parity
unpinned"; the end-to-end quantised values are pinned only through those
reductions, since the pages print no worked numeric example.
"""
