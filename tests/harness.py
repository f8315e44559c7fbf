"""Shared helpers for the parity tests: build the oracle's Spec from a workload and the
tile constants documented in include/sagebwd.h, move seeded inputs to the GPU, run the
HIP path through the C ABI, and compare."""
from __future__ import annotations

import os
import re
from typing import Dict, Optional, Sequence

import numpy as np

from bit_trainable_attention_amd import workloads as wl
from oracle import quant as oq

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "sagebwd.h")


def header_constants() -> Dict[str, int]:
    text = open(HEADER).read()
    return {m.group(1): int(m.group(2)) for m in re.finditer(r"#define\s+SAGEBWD_(\w+)\s+(\d+)", text)}


def header_functions() -> list:
    text = open(HEADER).read()
    return sorted(set(re.findall(r"^\s*(?:size_t|sagebwd_status|const char\*)\s+(sagebwd_\w+)\s*\(", text, re.M)))


def spec_for(w: wl.Workload, dtype: Optional[str] = None, normed_grads: bool = False, fmt: str = "int8",
             split: str = "sagebwd") -> oq.Spec:
    c = header_constants()
    qa = split == "qattn"
    return oq.Spec(N=w.N, d=w.d, blk=w.blk, causal=w.causal, qk_norm=w.qk_norm, k_smooth=w.k_smooth,
                   dtype=dtype or w.dtype, eps=w.eps, sm_scale=w.sm_scale,
                   fwd_tq=c["FWD_TILE_Q"], fwd_tk=min(w.blk, c["QATTN_FWD_TILE_K"]) if qa else w.blk,
                   bwd_tq=w.blk, bwd_pk=c["BWD_P_TILE_K"],
                   bwd_sk=min(w.blk, c["BWD_DS_TILE_K"]), q_smooth=w.q_smooth, normed_grads=normed_grads,
                   fmt=fmt, split=split)


def rel_l2(a, b) -> float:
    a = np.asarray(a, np.float64).ravel()
    b = np.asarray(b, np.float64).ravel()
    return float(np.linalg.norm(a - b) / max(np.linalg.norm(b), 1e-300))


# Per-row bar next to the whole-tensor rel-L2 bar (2e-3), derived before measuring: a row of
# an output holds d = 64..128 values whose quantisation errors are averaged, so rows whose
# error is concentrated (a query attending to a few keys, a key seen by few queries) may sit a
# few times above the tensor-wide figure; 10x covers that. A localised bug (one wrong value per
# row, e.g. at a tile edge) moves its row by about one value's share of the row norm, at least
# 1/sqrt(d) >= 0.088, far above the bar. Rows with a norm below the tensor's RMS row norm are
# judged against that RMS norm (an absolute floor), so a tiny row's relative noise does not
# count as a fault.
ROW_TOL = 2e-2


def row_norm_floor(b) -> np.ndarray:
    """Per row (all axes but the last, flattened) of b: max(||b_i||, RMS_i ||b_i||), the
    denominator of the per-row bar."""
    b = np.asarray(b, np.float64)
    nb = np.linalg.norm(b.reshape(-1, b.shape[-1]), axis=1)
    return np.maximum(nb, max(float(np.sqrt(np.mean(nb * nb))), 1e-300))


def row_rel(a, b) -> np.ndarray:
    """Per row (flattened as row_norm_floor) of ||a_i - b_i|| / max(||b_i||, RMS_i ||b_i||)."""
    a = np.asarray(a, np.float64)
    b = np.asarray(b, np.float64)
    d = b.shape[-1]
    return np.linalg.norm(a.reshape(-1, d) - b.reshape(-1, d), axis=1) / row_norm_floor(b)


def row_rel_max(a, b) -> float:
    """max over rows (all axes but the last) of ||a_i - b_i|| / max(||b_i||, RMS_i ||b_i||)."""
    return float(np.max(row_rel(a, b)))


def cosine(a, b) -> float:
    a = np.asarray(a, np.float64).ravel()
    b = np.asarray(b, np.float64).ravel()
    return float(a @ b / max(np.linalg.norm(a) * np.linalg.norm(b), 1e-300))


def host_inputs(w: wl.Workload) -> Dict[str, np.ndarray]:
    x = wl.make_inputs(w)
    out = {k: x[k] for k in ("Q", "K", "V", "dO")}
    for k in ("Q", "K", "V", "dO"):
        out[k + "f"] = wl.bits_to_f32(x[k], w.dtype)
    return out


# ------------------------------------------------------------------------------- GPU side

def params_for(w: wl.Workload, dq_mode: int = 0, layout: str = "bhnd", qk_gain: bool = False,
               normed_grads: bool = False, fmt: str = "int8", split: str = "sagebwd"):
    from bit_trainable_attention_amd import api
    return api.make_params(w.B, w.H, w.N, w.d, w.blk, w.causal, w.qk_norm, w.k_smooth, w.dtype, eps=w.eps,
                           dq_mode=dq_mode, q_smooth=w.q_smooth, layout=layout, qk_gain=qk_gain,
                           normed_grads=normed_grads, fmt=fmt, split=split)


def to_device(bits: np.ndarray, dtype: str):
    import torch
    t = torch.from_numpy(np.ascontiguousarray(bits).view(np.int16))
    t = t.view(torch.float16 if dtype == "fp16" else torch.bfloat16)
    return t.to("cuda:0")


def f32_to_device_dtype(x: np.ndarray, dtype: str):
    """float64/32 values already representable in dtype -> device tensor of dtype."""
    return to_device(wl.f32_to_bits(np.asarray(x, np.float32), dtype), dtype)


def gpu_run(w: wl.Workload, x: Dict[str, np.ndarray], stages=("prologue", "forward", "backward"),
            pro_in=None, O_in=None, lse_in=None, dq_mode: int = 0, layout: str = "bhnd",
            gains=None, normed_grads: bool = False, fmt: str = "int8",
            split: str = "sagebwd") -> Dict[str, np.ndarray]:
    """Run the HIP path and return host copies (numpy) of everything it produced. With
    layout "bnhd" the 16-bit tensors are handed to the library as [B,N,H,d] (a transposed
    copy of the same values) and its O, dQ, dK, dV are returned transposed back. gains:
    optional (q_gain, k_gain) float32 [H, d] arrays (learnable QK-norm gains); their
    gradients come back as dq_gain, dk_gain. fmt: "int8" or "fp8" codes (FP8 codes come back
    as their uint8 bit patterns, like the oracle's)."""
    import torch
    from bit_trainable_attention_amd import api
    p = params_for(w, dq_mode, layout, qk_gain=gains is not None, normed_grads=normed_grads, fmt=fmt, split=split)
    gq = gk = None
    if gains is not None:
        gq, gk = (torch.from_numpy(np.ascontiguousarray(g, dtype=np.float32)).to("cuda:0") for g in gains)
    tr = (lambda t: t.transpose(1, 2).contiguous()) if layout == "bnhd" else (lambda t: t)
    back = (lambda t: t.transpose(1, 2)) if layout == "bnhd" else (lambda t: t)
    Q, K, V, dO = (tr(to_device(x[k], w.dtype)) for k in ("Q", "K", "V", "dO"))
    if O_in is not None:
        O_in = tr(O_in)
    res: Dict[str, np.ndarray] = {}
    pro = pro_in
    if "prologue" in stages:
        pro = api.sagebwd_quant_prologue(p, Q, K, V, q_gain=gq, k_gain=gk)
    O, lse = O_in, lse_in
    if "forward" in stages:
        O, lse = api.sagebwd_forward(p, pro, V=V)
    if "backward" in stages:
        g = api.sagebwd_backward(p, Q, K, V, pro, O, lse, dO, q_gain=gq, k_gain=gk)
    torch.cuda.synchronize()
    if "prologue" in stages:
        for k, v in pro.items():
            res[k] = v.cpu().numpy()
    if "forward" in stages:
        res["O"] = back(O).float().cpu().numpy().astype(np.float64)
        res["LSE"] = lse[:, :, :w.N].cpu().numpy()      # (rows from N on: padding)
    if "backward" in stages:
        for k in ("dQ", "dK", "dV"):
            res[k] = back(g[k]).float().cpu().numpy().astype(np.float64)
        if gains is not None:
            res["dq_gain"] = g["dq_gain"].cpu().numpy().astype(np.float64)
            res["dk_gain"] = g["dk_gain"].cpu().numpy().astype(np.float64)
        lay = api.backward_workspace_layout(p)
        npk = w.B * w.H * lay["tiles_per_head_q"] * lay["packet_bytes"]   # only the packet region is decoded
        ws = g["workspace"][:npk].cpu().numpy()
        res.update(decode_packets(ws, lay, w))
    if fmt == "fp8":
        for k in ("Qc", "Kc", "Vtc", "dOtc"):
            if k in res:
                res[k] = res[k].view(np.uint8)
    return res


def decode_packets(ws: np.ndarray, lay: Dict[str, int], w: wl.Workload) -> Dict[str, np.ndarray]:
    """Read the dO codes (channel-major, natural token order), the dO block scales and D
    back out of the backward workspace's tile packets (layout in include/sagebwd.h)."""
    Np = -(-w.N // w.blk) * w.blk
    d, P, nt = w.d, lay["packet_bytes"], Np // 64
    pk = ws[lay["packets"]:lay["packets"] + w.B * w.H * nt * P].reshape(w.B, w.H, nt, P)
    rows = pk[..., 192 * d:256 * d].view(np.int8).reshape(w.B, w.H, nt, d, 4, 16)  # [.., c, slot, 16]
    c = np.arange(d)
    slot_of = np.arange(4)[None, :] ^ ((c[:, None] >> 1) & 3)                        # logical chunk -> slot
    logical = np.take_along_axis(rows, slot_of[None, None, None, :, :, None], axis=-2).reshape(w.B, w.H, nt, d, 64)
    u = np.arange(64)
    pos = 16 * ((u >> 2) & 3) + 4 * (u >> 4) + (u & 3)
    codes = logical[..., pos]                                                         # [B,H,nt,d,64]
    dOtc = np.moveaxis(codes, 2, 3).reshape(w.B, w.H, d, Np)
    base = 256 * d
    Dv = pk[..., base + 256:base + 512].copy().view(np.float32).reshape(w.B, w.H, Np)
    sdo_tiles = pk[..., base + 516:base + 520].copy().view(np.float32).reshape(w.B, w.H, nt)
    dOs = sdo_tiles[..., :: w.blk // 64]
    return {"dOtc": dOtc, "dOs": dOs, "Dvec": Dv}


def check_prologue(g: Dict[str, np.ndarray], o: Dict[str, np.ndarray], check_v: bool = True) -> None:
    """The GPU prologue's codes, scales, rstd and K mean (and query mean with Q-smoothing)
    equal the oracle's bit for bit; the key bias (float32 on the GPU, any summation order)
    is within float32 rounding of the oracle's float64 value. check_v False skips the V codes
    (the Q-Attn split's oracle keeps V's own values; the products never read the V codes)."""
    keys = ["Qc", "Kc", "Qs", "Ks", "q_rstd", "k_rstd", "k_mean"] + (["Vs"] if check_v else [])
    if "kbias" in g:
        keys.append("q_mean")
        kb = np.asarray(o["kbias"], np.float64)
        err = np.max(np.abs(g["kbias"].astype(np.float64) - kb))
        # a float32 dot product over d terms: a few ulps of the largest term's magnitude
        assert err <= 1e-5 * max(1.0, float(np.max(np.abs(kb)))), err
    for k in keys:
        assert g[k].dtype == o[k].dtype, k
        assert np.array_equal(g[k], o[k]), (k, int(np.sum(g[k] != o[k])))
    if check_v:
        assert np.array_equal(g["Vtc"], np.swapaxes(o["Vc"], -1, -2)), \
            int(np.sum(g["Vtc"] != np.swapaxes(o["Vc"], -1, -2)))


def pro_to_device(pro: Dict[str, np.ndarray]):
    """The oracle's prologue outputs as device tensors in the C ABI layout (for staged tests)."""
    import torch
    out = {}
    for k in ("Qc", "Kc", "Qs", "Ks", "Vs", "q_rstd", "k_rstd", "k_mean"):
        out[k] = torch.from_numpy(np.ascontiguousarray(pro[k])).to("cuda:0")
    if np.any(pro.get("q_mean", 0)):
        out["q_mean"] = torch.from_numpy(np.ascontiguousarray(pro["q_mean"])).to("cuda:0")
        out["kbias"] = torch.from_numpy(np.ascontiguousarray(pro["kbias"], dtype=np.float32)).to("cuda:0")
    out["Vtc"] = torch.from_numpy(np.ascontiguousarray(np.swapaxes(pro["Vc"], -1, -2))).to("cuda:0")
    return out


def slice_heads(x: Dict[str, np.ndarray], w: wl.Workload, heads: Sequence[int]) -> Dict[str, np.ndarray]:
    """Select flattened heads (b*H + h) of every [B,H,...] array, as a B=1, H=len(heads) set."""
    out = {}
    for k, v in x.items():
        if isinstance(v, np.ndarray) and v.ndim >= 2 and v.shape[:2] == (w.B, w.H):
            f = v.reshape((w.B * w.H,) + v.shape[2:])[list(heads)]
            out[k] = f.reshape((1, len(heads)) + v.shape[2:])
        else:
            out[k] = v
    return out
