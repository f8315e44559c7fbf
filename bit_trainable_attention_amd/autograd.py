"""PyTorch autograd wrapper over the C ABI (argument marshalling only).

`sagebwd_attention(q, k, v, ...)` runs the quantisation prologue and the INT8 forward and
returns O (and optionally the row logsumexp); `O.backward(dO)` runs the library's backward
and delivers dQ, dK, dV with respect to the raw q, k, v handed in (the RMSNorm backward of
QK-norm included; K-smoothing contributes nothing, SageBwd article, K-smoothing paragraph).
Every step runs in libsagebwd.so; there is no CPU path.

Layouts: "bhnd" takes [B, H, N, d] tensors, "bnhd" the [B, N, H, d] layout of a fused
projection output; the kernels read and write either layout in place (sagebwd_params.layout),
so neither costs a copy of a contiguous input. O and the gradients come back in the layout of
the inputs.
"""
from __future__ import annotations

from typing import Optional, Tuple, Union

import torch
from torch.autograd.function import once_differentiable

from . import api

_DTYPES = {torch.float16: "fp16", torch.bfloat16: "bf16"}
# prologue tensors the backward reads (the V codes are only the forward's)
_SAVED = ("Qc", "Kc", "Qs", "Ks", "q_rstd", "k_rstd")
_SAVED_QS = _SAVED + ("q_mean", "kbias")


class SageBwdAttention(torch.autograd.Function):
    """Autograd node: forward = prologue + INT8 forward, backward = the library's backward."""

    @staticmethod
    def forward(ctx, q, k, v, q_gain, k_gain, causal: bool, qk_norm: bool, k_smooth: bool, blk: int,
                eps: float, sm_scale: float, dq_mode: int, q_smooth: bool, layout: str, normed_grads: bool,
                fmt: str, split: str):
        if q.dtype not in _DTYPES:
            raise TypeError(f"q, k, v must be float16 or bfloat16, got {q.dtype}")
        if q.dim() != 4:
            raise ValueError(f"expected 4-d {layout} tensors, got shape {tuple(q.shape)}")
        if layout == "bnhd":
            B, N, H, d = q.shape
        else:
            B, H, N, d = q.shape
        gained = q_gain is not None
        if gained != (k_gain is not None):
            raise ValueError("q_gain and k_gain go together")
        p = api.make_params(B, H, N, d, blk, causal, qk_norm, k_smooth, _DTYPES[q.dtype], eps=eps,
                            sm_scale=sm_scale, dq_mode=dq_mode, q_smooth=q_smooth, layout=layout,
                            qk_gain=gained, normed_grads=normed_grads, fmt=fmt, split=split)
        q, k, v = q.contiguous(), k.contiguous(), v.contiguous()
        gains = (q_gain.detach().float().contiguous(), k_gain.detach().float().contiguous()) if gained else (None, None)
        pro = api.sagebwd_quant_prologue(p, q, k, v, q_gain=gains[0], k_gain=gains[1])
        O, lse = api.sagebwd_forward(p, pro, V=v)
        ctx.params = p
        ctx.saved_names = _SAVED_QS if q_smooth else _SAVED
        ctx.gain_dtypes = (q_gain.dtype, k_gain.dtype) if gained else None
        ctx.save_for_backward(q, k, v, O, lse, *(pro[n] for n in ctx.saved_names), *(gains if gained else ()))
        ctx.mark_non_differentiable(lse)
        # lse carries no gradient: without this, autograd would fill a zero tensor for it on
        # every backward (a kernel launch and a write of B*H*N floats)
        ctx.set_materialize_grads(False)
        return O, lse

    @staticmethod
    @once_differentiable   # the backward runs in the library: no second derivative through it
    def backward(ctx, dO, _dlse):
        if dO is None:   # O took no part in the loss (grads are not materialised)
            return (None,) * 17
        q, k, v, O, lse, *saved = ctx.saved_tensors
        pro = dict(zip(ctx.saved_names, saved[:len(ctx.saved_names)]))
        gains = saved[len(ctx.saved_names):] if ctx.gain_dtypes else (None, None)
        g = api.sagebwd_backward(ctx.params, q, k, v, pro, O, lse, dO.contiguous(), q_gain=gains[0],
                                 k_gain=gains[1])
        dgq = dgk = None
        if ctx.gain_dtypes:
            dgq, dgk = g["dq_gain"].to(ctx.gain_dtypes[0]), g["dk_gain"].to(ctx.gain_dtypes[1])
        return (g["dQ"], g["dK"], g["dV"], dgq, dgk) + (None,) * 12


def sagebwd_attention(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, causal: bool = True,
                      qk_norm: bool = True, k_smooth: bool = True, blk: int = 128, eps: float = 1e-6,
                      sm_scale: float = 0.0, layout: str = "bhnd", return_lse: bool = False,
                      dq_mode: int = 0, q_smooth: bool = False, q_gain: Optional[torch.Tensor] = None,
                      k_gain: Optional[torch.Tensor] = None,
                      normed_grads: bool = False,
                      fmt: str = "int8", split: str = "sagebwd") -> Union[torch.Tensor, Tuple[torch.Tensor, torch.Tensor]]:
    """SageBwd-style INT8 attention with gradients (see the module docstring).

    sm_scale <= 0 selects 1/sqrt(d); q_smooth selects the Q-smoothing variant (the query
    mean is subtracted before quantising and added back through the key bias and dK_bias).
    q_gain, k_gain: optional learnable QK-norm gains [H, d] (both or neither; they receive
    gradients). normed_grads: q.grad and k.grad become the gradients with respect to the
    normalised Q^, K^ (for a caller that applies its own RMSNorm backward). fmt: "int8" or
    "fp8" (e4m3 codes for the quantised products; not with q_smooth). split: "sagebwd" (six of
    the seven products quantised) or "qattn" (the Full-Stack FP4 page's split: QK^T and the dS
    products quantised, PV, P^T dO and dO V^T in 16 bits; not with q_smooth). The lse returned
    with return_lse is float32 [B, H, N] (natural log) and carries no gradient.
    """
    if fmt not in ("int8", "fp8"):
        raise ValueError(f"fmt must be 'int8' or 'fp8', got {fmt!r}")
    if split not in ("sagebwd", "qattn"):
        raise ValueError(f"split must be 'sagebwd' or 'qattn', got {split!r}")
    if layout not in ("bhnd", "bnhd"):
        raise ValueError(f"layout must be 'bhnd' or 'bnhd', got {layout!r}")
    O, lse = SageBwdAttention.apply(q, k, v, q_gain, k_gain, bool(causal), bool(qk_norm), bool(k_smooth), int(blk),
                                    float(eps), float(sm_scale), int(dq_mode), bool(q_smooth), layout,
                                    bool(normed_grads), str(fmt), str(split))
    if not return_lse:
        return O
    # the library's lse holds N rounded up to whole blocks (padding rows +inf): the first N
    N = q.shape[1] if layout == "bnhd" else q.shape[2]
    return O, lse[..., :N]
