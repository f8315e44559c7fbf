"""SageBwd-style trainable INT8 attention for AMD MI355X (gfx950).

The compute path is libsagebwd.so (hand-written HIP kernels behind the C ABI declared in
include/sagebwd.h); `api` is a thin ctypes binding with the same entry-point names, and
`autograd` wraps it as a torch.autograd.Function.
`workloads` draws the seeded synthetic inputs. Importing this package does not load the
library; the first call through `api` does, and fails loudly if it was not built.
"""
__all__ = ["api", "autograd", "workloads"]
