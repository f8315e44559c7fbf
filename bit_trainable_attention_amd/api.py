"""Thin Python binding of the C ABI (include/sagebwd.h); names follow the C entry points.

Argument marshalling only: every step of the attention runs in the HIP kernels of
libsagebwd.so. PyTorch provides device memory and the stream. Before a call is made,
each tensor is checked on the host against the shape, dtype, device and layout that the
parameters imply, so a kernel is never launched on a buffer of the wrong size.
"""
from __future__ import annotations

import ctypes
from typing import Dict, Optional

import torch

from . import _lib

_TORCH_DTYPE = {_lib.SAGEBWD_FP16: torch.float16, _lib.SAGEBWD_BF16: torch.bfloat16}


def make_params(B: int, H: int, N: int, d: int, blk: int, causal: bool, qk_norm: bool, k_smooth: bool,
                dtype: str, eps: float = 1e-6, sm_scale: float = 0.0, dq_mode: int = 0,
                q_smooth: bool = False, layout: str = "bhnd", qk_gain: bool = False,
                normed_grads: bool = False, fmt: str = "int8", split: str = "sagebwd") -> _lib.Params:
    """dq_mode: 0 auto, 1 dS spill, 2 float32 atomics; layout of the 16-bit tensors:
    "bhnd" [B,H,N,d] or "bnhd" [B,N,H,d]; qk_gain: learnable QK-norm gains [H,d];
    normed_grads: dQ, dK with respect to the normalised Q^, K^; fmt: code format of the
    quantised products, "int8" or "fp8" (e4m3); split: "sagebwd" (six of seven products
    quantised) or "qattn" (QK^T and the dS products) (include/sagebwd.h)."""
    dt = {"fp16": _lib.SAGEBWD_FP16, "bf16": _lib.SAGEBWD_BF16}[dtype]
    lay = {"bhnd": _lib.LAYOUT_BHND, "bnhd": _lib.LAYOUT_BNHD}[layout]
    return _lib.Params(B, H, N, d, blk, int(causal), int(qk_norm), int(k_smooth), eps, sm_scale, dt, dq_mode,
                       int(q_smooth), lay, int(qk_gain), int(normed_grads),
                       {"int8": _lib.FMT_INT8, "fp8": _lib.FMT_FP8}[fmt],
                       {"sagebwd": _lib.SPLIT_SAGEBWD, "qattn": _lib.SPLIT_QATTN}[split])


def sagebwd_status_string(status: int) -> str:
    return _lib.load().sagebwd_status_string(status).decode()


def sagebwd_last_error() -> str:
    """Detail of the last SAGEBWD_ERR_HIP on this thread ("" if none)."""
    return _lib.load().sagebwd_last_error().decode()


def _check(status: int, what: str) -> None:
    if status != 0:
        detail = f"; {sagebwd_last_error()}" if _lib.STATUS.get(status) == "SAGEBWD_ERR_HIP" else ""
        raise RuntimeError(f"{what}: {_lib.STATUS.get(status, status)} ({sagebwd_status_string(status)}){detail}")


def _stream(device: torch.device, stream: Optional[torch.cuda.Stream]) -> ctypes.c_void_p:
    s = stream if stream is not None else torch.cuda.current_stream(device)
    return ctypes.c_void_p(s.cuda_stream)


def _want(t: torch.Tensor, name: str, shape, dtype, device) -> None:
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a tensor")
    if t.device.type != "cuda":
        raise ValueError(f"{name}: the library takes device tensors only, got one on {t.device}")
    if tuple(t.shape) != tuple(shape) or t.dtype != dtype or t.device != device or not t.is_contiguous():
        raise ValueError(f"{name}: expected contiguous {dtype} {tuple(shape)} on {device}, got "
                         f"{t.dtype} {tuple(t.shape)} on {t.device} (contiguous={t.is_contiguous()})")


def _ptr(t: Optional[torch.Tensor]) -> ctypes.c_void_p:
    return ctypes.c_void_p(0 if t is None else t.data_ptr())


def padded_n(p: _lib.Params) -> int:
    """Tokens per head of the library's own arrays: N rounded up to whole blocks."""
    return -(-p.N // p.blk) * p.blk


def _shapes(p: _lib.Params):
    Np = padded_n(p)
    x16 = (p.B, p.N, p.H, p.d) if p.layout == _lib.LAYOUT_BNHD else (p.B, p.H, p.N, p.d)
    return dict(x=(p.B, p.H, Np, p.d), x16=x16, xt=(p.B, p.H, p.d, Np), s=(p.B, p.H, Np // p.blk),
                r=(p.B, p.H, Np), m=(p.B, p.H, p.d))


def sagebwd_prologue_workspace_bytes(p: _lib.Params) -> int:
    return int(_lib.load().sagebwd_prologue_workspace_bytes(ctypes.byref(p)))


def sagebwd_backward_workspace_bytes(p: _lib.Params) -> int:
    return int(_lib.load().sagebwd_backward_workspace_bytes(ctypes.byref(p)))


PACKET_BYTES = {64: 17408, 128: 33792}


SPILL_LIMIT = 16 << 30


def backward_workspace_layout(p: _lib.Params) -> Dict[str, int]:
    """Byte offsets of the backward workspace regions, as documented in include/sagebwd.h."""
    def up(x):
        return (x + 255) // 256 * 256
    bh, nt, nb = p.B * p.H, padded_n(p) // 64, padded_n(p) // p.blk
    r = p.blk // 64
    tiles = nb * nt - r * nb * (nb - 1) // 2 if p.causal else nb * nt
    off = {"packet_bytes": PACKET_BYTES[p.d], "packets": 0, "tiles_per_head": tiles, "tiles_per_head_q": nt}
    after = up(bh * nt * PACKET_BYTES[p.d])
    ktp, dsp, dsm = up(bh * nb * p.d * p.blk), up(bh * tiles * 64 * p.blk), up(bh * tiles * (p.blk // 64) * 4)
    # one head's dS tiles must stay below 4 GiB (the dQ pass addresses them with 32-bit offsets)
    fits = tiles * 64 * p.blk < (1 << 32)
    spill = fits and (p.dq_mode == 1 or (p.dq_mode == 0 and ktp + dsp + dsm <= SPILL_LIMIT))
    off["spill"] = int(spill)
    if spill:
        off["ktp"] = after
        off["dsp"] = after + ktp
        off["dsm"] = after + ktp + dsp
        off["total"] = after + ktp + dsp + dsm
    else:
        off["dq_acc"] = after
        off["total"] = after + up(4 * bh * padded_n(p) * p.d)
    if p.qk_gain:
        off["gq"] = off["total"]
        off["gk"] = off["gq"] + up(4 * bh * nt * p.d)
        off["total"] = off["gk"] + up(4 * bh * nb * p.d)
    return off


def _gains(p: _lib.Params, q_gain, k_gain, dev):
    if not p.qk_gain:
        return None, None
    for name, g in (("q_gain", q_gain), ("k_gain", k_gain)):
        if g is None:
            raise ValueError(f"{name} is required with qk_gain")
        _want(g, name, (p.H, p.d), torch.float32, dev)
    return q_gain, k_gain


def sagebwd_quant_prologue(p: _lib.Params, Q: torch.Tensor, K: torch.Tensor, V: torch.Tensor,
                           out: Optional[Dict[str, torch.Tensor]] = None,
                           workspace: Optional[torch.Tensor] = None,
                           stream: Optional[torch.cuda.Stream] = None,
                           q_gain: Optional[torch.Tensor] = None,
                           k_gain: Optional[torch.Tensor] = None) -> Dict[str, torch.Tensor]:
    """QK-norm (with the gains [H,d] when p.qk_gain) -> K-smoothing (and Q-smoothing) ->
    per-block INT8 codes/scales. Returns the prologue tensors; with q_smooth also q_mean
    [B,H,d] and kbias [B,H,N]."""
    out, q_gain, k_gain = _prologue_outputs(p, Q, K, V, out, q_gain, k_gain)
    dev = Q.device
    need = sagebwd_prologue_workspace_bytes(p)
    if need and workspace is None:
        workspace = torch.empty(need, dtype=torch.uint8, device=dev)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    st = _lib.load().sagebwd_quant_prologue(ctypes.byref(p), *_prologue_ptrs(p, Q, K, V, out, q_gain, k_gain),
                                            _ptr(workspace), ws_bytes, _stream(dev, stream))
    _check(st, "sagebwd_quant_prologue")
    return out


def sagebwd_quant_prologue_noalloc(p: _lib.Params, Q: torch.Tensor, K: torch.Tensor, V: torch.Tensor,
                                   out: Optional[Dict[str, torch.Tensor]] = None,
                                   stream: Optional[torch.cuda.Stream] = None,
                                   q_gain: Optional[torch.Tensor] = None,
                                   k_gain: Optional[torch.Tensor] = None) -> Dict[str, torch.Tensor]:
    """The allocation-free prologue (include/sagebwd.h): the library's call allocates nothing,
    its scratch is a static per-device array. Pass preallocated `out` tensors for a call
    that allocates nothing on this side either (with out=None they are allocated here)."""
    out, q_gain, k_gain = _prologue_outputs(p, Q, K, V, out, q_gain, k_gain)
    st = _lib.load().sagebwd_quant_prologue_noalloc(
        ctypes.byref(p), *_prologue_ptrs(p, Q, K, V, out, q_gain, k_gain), _stream(Q.device, stream))
    _check(st, "sagebwd_quant_prologue_noalloc")
    return out


def _prologue_ptrs(p, Q, K, V, out, q_gain, k_gain):
    return [_ptr(Q), _ptr(K), _ptr(V),
            _ptr(out["Qc"]), _ptr(out["Kc"]), _ptr(out["Vtc"]), _ptr(out["Qs"]), _ptr(out["Ks"]), _ptr(out["Vs"]),
            _ptr(out["q_rstd"]), _ptr(out["k_rstd"]), _ptr(out["k_mean"]),
            _ptr(out.get("q_mean") if p.q_smooth else None), _ptr(out.get("kbias") if p.q_smooth else None),
            _ptr(q_gain), _ptr(k_gain)]


def _prologue_outputs(p, Q, K, V, out, q_gain, k_gain):
    """Check the prologue's inputs and outputs (allocating the outputs when out is None)."""
    dev = Q.device
    sh = _shapes(p)
    dt = _TORCH_DTYPE[p.dtype]
    for name, t in (("Q", Q), ("K", K), ("V", V)):
        _want(t, name, sh["x16"], dt, dev)
    q_gain, k_gain = _gains(p, q_gain, k_gain, dev)
    if out is None:
        out = dict(
            Qc=torch.empty(sh["x"], dtype=torch.int8, device=dev),
            Kc=torch.empty(sh["x"], dtype=torch.int8, device=dev),
            Vtc=torch.empty(sh["xt"], dtype=torch.int8, device=dev),
            Qs=torch.empty(sh["s"], dtype=torch.float32, device=dev),
            Ks=torch.empty(sh["s"], dtype=torch.float32, device=dev),
            Vs=torch.empty(sh["s"], dtype=torch.float32, device=dev),
            q_rstd=torch.empty(sh["r"], dtype=torch.float32, device=dev),
            k_rstd=torch.empty(sh["r"], dtype=torch.float32, device=dev),
            k_mean=torch.empty(sh["m"], dtype=torch.float32, device=dev),
        )
        if p.q_smooth:
            out["q_mean"] = torch.empty(sh["m"], dtype=torch.float32, device=dev)
            out["kbias"] = torch.empty(sh["r"], dtype=torch.float32, device=dev)
    wanted = [("Qc", "x", torch.int8), ("Kc", "x", torch.int8), ("Vtc", "xt", torch.int8),
              ("Qs", "s", torch.float32), ("Ks", "s", torch.float32), ("Vs", "s", torch.float32),
              ("q_rstd", "r", torch.float32), ("k_rstd", "r", torch.float32), ("k_mean", "m", torch.float32)]
    if p.q_smooth:
        wanted += [("q_mean", "m", torch.float32), ("kbias", "r", torch.float32)]
    for name, key, tdt in wanted:
        _want(out[name], name, sh[key], tdt, dev)
    return out, q_gain, k_gain


def sagebwd_forward(p: _lib.Params, pro: Dict[str, torch.Tensor], O: Optional[torch.Tensor] = None,
                    lse: Optional[torch.Tensor] = None,
                    stream: Optional[torch.cuda.Stream] = None, V: Optional[torch.Tensor] = None):
    """Forward from the prologue tensors (and their kbias with q_smooth). With the Q-Attn split
    the raw V (the prologue's input) is required: PV runs in 16 bits. Returns (O, lse)."""
    dev = pro["Qc"].device
    sh = _shapes(p)
    qattn = p.split == _lib.SPLIT_QATTN
    wanted = [("Qc", "x", torch.int8), ("Kc", "x", torch.int8), ("Qs", "s", torch.float32), ("Ks", "s", torch.float32)]
    if not qattn:
        wanted += [("Vtc", "xt", torch.int8), ("Vs", "s", torch.float32)]
    else:
        if V is None:
            raise ValueError("the Q-Attn split's forward needs the raw V")
        _want(V, "V", sh["x16"], _TORCH_DTYPE[p.dtype], dev)
    if p.q_smooth:
        wanted.append(("kbias", "r", torch.float32))
    for name, key, tdt in wanted:
        _want(pro[name], name, sh[key], tdt, dev)
    if O is None:
        O = torch.empty(sh["x16"], dtype=_TORCH_DTYPE[p.dtype], device=dev)
    if lse is None:
        lse = torch.empty(sh["r"], dtype=torch.float32, device=dev)
    _want(O, "O", sh["x16"], _TORCH_DTYPE[p.dtype], dev)
    _want(lse, "lse", sh["r"], torch.float32, dev)
    st = _lib.load().sagebwd_forward(
        ctypes.byref(p), _ptr(pro["Qc"]), _ptr(pro["Kc"]), _ptr(pro["Vtc"]),
        _ptr(pro["Qs"]), _ptr(pro["Ks"]), _ptr(pro["Vs"]), _ptr(pro["kbias"] if p.q_smooth else None),
        _ptr(V if qattn else None), _ptr(O), _ptr(lse), _stream(dev, stream))
    _check(st, "sagebwd_forward")
    return O, lse


def _backward_args(p, Q, K, V, pro, O, lse, dO, grads, workspace, q_gain=None, k_gain=None):
    dev = Q.device
    q_gain, k_gain = _gains(p, q_gain, k_gain, dev)
    sh = _shapes(p)
    dt = _TORCH_DTYPE[p.dtype]
    for name, t in (("Q", Q), ("K", K), ("V", V), ("O", O), ("dO", dO)):
        _want(t, name, sh["x16"], dt, dev)
    wanted = [("Qc", "x", torch.int8), ("Kc", "x", torch.int8), ("Qs", "s", torch.float32),
              ("Ks", "s", torch.float32), ("q_rstd", "r", torch.float32), ("k_rstd", "r", torch.float32)]
    if p.q_smooth:
        wanted += [("q_mean", "m", torch.float32), ("kbias", "r", torch.float32)]
    for name, key, tdt in wanted:
        _want(pro[name], name, sh[key], tdt, dev)
    _want(lse, "lse", sh["r"], torch.float32, dev)
    if grads is None:
        grads = {n: torch.empty(sh["x16"], dtype=dt, device=dev) for n in ("dQ", "dK", "dV")}
    for n in ("dQ", "dK", "dV"):
        _want(grads[n], n, sh["x16"], dt, dev)
    if p.qk_gain:
        for n in ("dq_gain", "dk_gain"):
            if n not in grads:
                grads[n] = torch.empty((p.H, p.d), dtype=torch.float32, device=dev)
            _want(grads[n], n, (p.H, p.d), torch.float32, dev)
    need = sagebwd_backward_workspace_bytes(p)
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=dev)
    ws_bytes = workspace.numel() * workspace.element_size()
    args = [_ptr(Q), _ptr(K), _ptr(V), _ptr(pro["Qc"]), _ptr(pro["Kc"]),
            _ptr(pro["Qs"]), _ptr(pro["Ks"]), _ptr(pro["q_rstd"]), _ptr(pro["k_rstd"]),
            _ptr(pro["q_mean"] if p.q_smooth else None), _ptr(pro["kbias"] if p.q_smooth else None),
            _ptr(q_gain), _ptr(k_gain),
            _ptr(O), _ptr(lse), _ptr(dO), _ptr(grads["dQ"]), _ptr(grads["dK"]), _ptr(grads["dV"]),
            _ptr(grads.get("dq_gain")), _ptr(grads.get("dk_gain")),
            _ptr(workspace), ws_bytes]
    return args, grads, workspace


def sagebwd_backward(p: _lib.Params, Q: torch.Tensor, K: torch.Tensor, V: torch.Tensor,
                     pro: Dict[str, torch.Tensor], O: torch.Tensor, lse: torch.Tensor, dO: torch.Tensor,
                     grads: Optional[Dict[str, torch.Tensor]] = None,
                     workspace: Optional[torch.Tensor] = None,
                     stream: Optional[torch.cuda.Stream] = None,
                     q_gain: Optional[torch.Tensor] = None,
                     k_gain: Optional[torch.Tensor] = None) -> Dict[str, torch.Tensor]:
    """Backward. Returns dict(dQ, dK, dV, workspace) and, with p.qk_gain, dq_gain, dk_gain."""
    args, grads, workspace = _backward_args(p, Q, K, V, pro, O, lse, dO, grads, workspace, q_gain, k_gain)
    st = _lib.load().sagebwd_backward(ctypes.byref(p), *args, _stream(Q.device, stream))
    _check(st, "sagebwd_backward")
    out = dict(grads)
    out["workspace"] = workspace
    return out


def sagebwd_backward_part(p: _lib.Params, part: int, Q: torch.Tensor, K: torch.Tensor, V: torch.Tensor,
                          pro: Dict[str, torch.Tensor], O: torch.Tensor, lse: torch.Tensor, dO: torch.Tensor,
                          grads: Dict[str, torch.Tensor], workspace: torch.Tensor,
                          stream: Optional[torch.cuda.Stream] = None,
                          q_gain: Optional[torch.Tensor] = None, k_gain: Optional[torch.Tensor] = None) -> None:
    """One stage (0: pre, 1: main, 2: the dQ pass) of the backward; see include/sagebwd.h."""
    args, _, _ = _backward_args(p, Q, K, V, pro, O, lse, dO, grads, workspace, q_gain, k_gain)
    st = _lib.load().sagebwd_backward_part(ctypes.byref(p), int(part), *args, _stream(Q.device, stream))
    _check(st, f"sagebwd_backward_part({part})")
