"""Guard bands: every output of the three calls (prologue codes, scales and statistics; O and
lse; dQ, dK, dV and the gains' gradients) and the backward workspace is placed inside a larger
device buffer whose bytes before and after it hold a sentinel pattern. After the calls the
sentinels must be intact (no write past either end of any output) and the outputs must equal
those of a run on plain tensors bit for bit; every call's inputs (Q, K, V, dO, the gains, the
prologue's outputs as the forward's and backward's inputs, O and lse) must be unchanged. Cases: ragged N (the 16-bit tensors hold exactly
N tokens, the library's own arrays Np), the in-place [B,N,H,d] layout, gains, both dQ modes,
Q-smoothing and the FP8 recipe."""
import numpy as np
import pytest

from bit_trainable_attention_amd import workloads as wl
from tests.harness import host_inputs, params_for, to_device

pytestmark = pytest.mark.gpu
W = wl.WORKLOADS

PAD = 4096          # guard bytes on each side (a multiple of 256: outputs stay aligned)
SENTINEL = 0xA5


class Guarded:
    """Device buffers with PAD sentinel bytes before and after each tensor view."""

    def __init__(self):
        self.bufs = []

    def like(self, t):
        import torch
        nbytes = t.numel() * t.element_size()
        buf = torch.full((nbytes + 2 * PAD,), SENTINEL, dtype=torch.uint8, device=t.device)
        view = buf[PAD:PAD + nbytes].view(t.dtype).view(t.shape)
        self.bufs.append((buf, nbytes))
        return view

    def bytes(self, n, device):
        import torch
        buf = torch.full((n + 2 * PAD,), SENTINEL, dtype=torch.uint8, device=device)
        self.bufs.append((buf, n))
        return buf[PAD:PAD + n]

    def check(self):
        for i, (buf, n) in enumerate(self.bufs):
            h = buf.cpu().numpy()
            assert np.all(h[:PAD] == SENTINEL), f"buffer {i}: write before the start"
            assert np.all(h[PAD + n:] == SENTINEL), f"buffer {i}: write past the end"


def _run(w, layout, dq_mode, gains, fmt, guard):
    import torch
    from bit_trainable_attention_amd import api
    x = host_inputs(w)
    p = params_for(w, dq_mode=dq_mode, layout=layout, qk_gain=gains, fmt=fmt)
    tr = (lambda t: t.transpose(1, 2).contiguous()) if layout == "bnhd" else (lambda t: t)
    Q, K, V, dO = (tr(to_device(x[k], w.dtype)) for k in ("Q", "K", "V", "dO"))
    gq = gk = None
    if gains:
        rng = np.random.default_rng(600 + w.N)
        gq, gk = (torch.from_numpy((1 + 0.3 * rng.standard_normal((w.H, w.d))).astype(np.float32)).to("cuda:0")
                  for _ in range(2))
    G = Guarded()
    ref = api.sagebwd_quant_prologue(p, Q, K, V, q_gain=gq, k_gain=gk)       # shapes only
    # inputs are never written: snapshots of every call's inputs, compared after the calls
    before = {"Q": Q.clone(), "K": K.clone(), "V": V.clone(), "dO": dO.clone()}
    if gains:
        before.update(q_gain=gq.clone(), k_gain=gk.clone())
    now = {"Q": Q, "K": K, "V": V, "dO": dO, "q_gain": gq, "k_gain": gk}
    pro = {k: (G.like(v) if guard else torch.empty_like(v)) for k, v in ref.items()}
    need = api.sagebwd_prologue_workspace_bytes(p)
    pws = (G.bytes(need, Q.device) if guard else torch.empty(need, dtype=torch.uint8, device=Q.device)) if need else None
    api.sagebwd_quant_prologue(p, Q, K, V, out=pro, workspace=pws, q_gain=gq, k_gain=gk)
    before.update({"pro." + k: v.clone() for k, v in pro.items()})
    now.update({"pro." + k: v for k, v in pro.items()})
    O0, lse0 = api.sagebwd_forward(p, pro)
    O = G.like(O0) if guard else torch.empty_like(O0)
    lse = G.like(lse0) if guard else torch.empty_like(lse0)
    api.sagebwd_forward(p, pro, O=O, lse=lse)
    before.update(O=O.clone(), lse=lse.clone())
    now.update(O=O, lse=lse)
    grads = {n: (G.like(Q) if guard else torch.empty_like(Q)) for n in ("dQ", "dK", "dV")}
    if gains:
        for n in ("dq_gain", "dk_gain"):
            t = torch.empty((w.H, w.d), dtype=torch.float32, device=Q.device)
            grads[n] = G.like(t) if guard else t
    bneed = api.sagebwd_backward_workspace_bytes(p)
    bws = G.bytes(bneed, Q.device) if guard else torch.empty(bneed, dtype=torch.uint8, device=Q.device)
    api.sagebwd_backward(p, Q, K, V, pro, O, lse, dO, grads=grads, workspace=bws, q_gain=gq, k_gain=gk)
    torch.cuda.synchronize()
    if guard:
        G.check()
    for k, t in before.items():   # the prologue's, the forward's and the backward's inputs
        assert torch.equal(now[k], t), f"input {k} was written"
    def host(t):   # 16-bit tensors as their bit patterns (numpy has no bfloat16)
        return t.view(torch.int16).cpu().numpy() if t.element_size() == 2 else t.cpu().numpy()

    out = {k: host(v) for k, v in pro.items()}
    out.update(O=host(O), lse=host(lse))
    out.update({k: host(v) for k, v in grads.items()})
    return out


CASES = [
    ("ragged_d128_blk128_spill", W["n8192_d128"].with_shape(B=1, H=2, N=200), "bhnd", 1, False, "int8"),
    ("ragged_d64_bnhd_atomic_gains", W["llama325m"].with_shape(B=2, H=3, N=130), "bnhd", 2, True, "int8"),
    ("ragged_d128_blk64_bnhd_gains_spill", W["n8192_d128"].with_shape(B=2, H=2, N=333, blk=64), "bnhd", 1, True,
     "int8"),
    ("d64_blk128_qsmooth", W["bf16_d64"].with_shape(B=1, H=2, N=256, blk=128, q_smooth=True, q_bias_var=4.0),
     "bhnd", 0, False, "int8"),
    ("fp8_ragged_d128_atomic", W["n8192_d128"].with_shape(B=1, H=2, N=300), "bhnd", 2, False, "fp8"),
    ("fp8_d64_bnhd_spill", W["bf16_d64"].with_shape(B=1, H=2, N=384), "bnhd", 1, False, "fp8"),
]


@pytest.mark.parametrize("name,w,layout,dq_mode,gains,fmt", CASES)
def test_outputs_stay_inside_their_buffers(name, w, layout, dq_mode, gains, fmt):
    print(f"[guard] {name}: B{w.B} H{w.H} N{w.N} d{w.d} blk{w.blk} {w.dtype} layout={layout} dq_mode={dq_mode} "
          f"gains={gains} fmt={fmt} q_smooth={w.q_smooth}", flush=True)
    a = _run(w, layout, dq_mode, gains, fmt, guard=True)
    b = _run(w, layout, dq_mode, gains, fmt, guard=False)
    for k in b:
        if dq_mode == 2 and k in ("dQ", "dq_gain"):
            continue   # float32 atomics: the summation order varies between runs
        assert np.array_equal(a[k], b[k], equal_nan=True), k
    # padding queries of a ragged last block get lse = +inf (every output element is written)
    Np = -(-w.N // w.blk) * w.blk
    assert np.all(np.isposinf(a["lse"][..., w.N:Np])) and np.all(np.isfinite(a["lse"][..., :w.N]))


@pytest.mark.parametrize("dq_mode", [1, 2])
def test_nonfinite_inputs_stay_memory_safe(dq_mode):
    """NaN and infinite inputs give unspecified results (the header), but memory-safe ones: with
    NaN, +inf and -inf planted in Q, K, V and dO, every output still lands inside its guarded
    buffer (no kernel indexes memory by a data value), in both dQ modes."""
    import torch
    from bit_trainable_attention_amd import api
    w = W["n8192_d128"].with_shape(B=1, H=2, N=300)
    print(f"[guard] non-finite inputs: B{w.B} H{w.H} N{w.N} d{w.d} dq_mode={dq_mode}", flush=True)
    x = host_inputs(w)
    p = params_for(w, dq_mode=dq_mode)
    ins = {k: to_device(x[k], w.dtype) for k in ("Q", "K", "V", "dO")}
    for i, k in enumerate(ins):                     # a NaN, a +inf and a -inf in every input
        flat = ins[k].view(-1)
        flat[7 + 100 * i] = float("nan")
        flat[5000 + 100 * i] = float("inf")
        flat[-3 - 100 * i] = float("-inf")
    G = Guarded()
    ref = api.sagebwd_quant_prologue(p, ins["Q"], ins["K"], ins["V"])
    pro = {k: G.like(v) for k, v in ref.items()}
    need = api.sagebwd_prologue_workspace_bytes(p)
    pws = G.bytes(need, ins["Q"].device) if need else None
    api.sagebwd_quant_prologue(p, ins["Q"], ins["K"], ins["V"], out=pro, workspace=pws)
    O0, lse0 = api.sagebwd_forward(p, pro)
    O, lse = G.like(O0), G.like(lse0)
    api.sagebwd_forward(p, pro, O=O, lse=lse)
    grads = {n: G.like(ins["Q"]) for n in ("dQ", "dK", "dV")}
    bws = G.bytes(api.sagebwd_backward_workspace_bytes(p), ins["Q"].device)
    api.sagebwd_backward(p, ins["Q"], ins["K"], ins["V"], pro, O, lse, ins["dO"], grads=grads, workspace=bws)
    torch.cuda.synchronize()
    G.check()
