"""The C ABI library loads, exports every entry point include/sagebwd.h declares, and
rejects bad arguments before doing anything on a device. No call here reaches a kernel:
every call either fails validation or is a documented no-op (N == 0)."""
import ctypes
import re

import pytest

from bit_trainable_attention_amd import _lib
from tests.harness import HEADER, header_constants, header_functions


def header_path():
    return HEADER

lib = _lib.load()  # fails loudly if the library was not built


def P(**kw):
    base = dict(B=1, H=2, N=256, d=64, blk=64, causal=1, qk_norm=1, k_smooth=1, eps=1e-6, sm_scale=0.0,
                dtype=_lib.SAGEBWD_FP16, dq_mode=0, q_smooth=0, layout=_lib.LAYOUT_BHND, qk_gain=0,
                normed_grads=0, fmt=_lib.FMT_INT8, split=_lib.SPLIT_SAGEBWD)
    base.update(kw)
    return _lib.Params(**base)


FAKE = 0x10000  # an aligned, never dereferenced address
MIS = 0x10001   # misaligned


def test_exports_every_header_symbol():
    names = header_functions()
    assert set(names) == set(_lib.SIGNATURES), names
    for n in names:
        assert hasattr(lib, n)


def test_header_tile_constants_match_binding():
    c = header_constants()
    assert (c["FWD_TILE_Q"], c["BWD_P_TILE_K"], c["BWD_DS_TILE_K"], c["QATTN_FWD_TILE_K"]) == \
        (_lib.FWD_TILE_Q, _lib.BWD_P_TILE_K, _lib.BWD_DS_TILE_K, _lib.QATTN_FWD_TILE_K)


def test_status_strings():
    for code, name in _lib.STATUS.items():
        s = lib.sagebwd_status_string(code).decode()
        assert s and s != "unknown status", (code, name)
    assert lib.sagebwd_status_string(12345).decode() == "unknown status"


def test_last_error_empty_without_failures():
    # argument errors are reported by status alone; only a failed enqueue records detail
    assert _prologue(P(d=96)) == -3
    assert lib.sagebwd_last_error().decode() == ""


def _prologue(p, ptr=FAKE, ws=FAKE, ws_bytes=1 << 40):
    return lib.sagebwd_quant_prologue(ctypes.byref(p), *([ptr] * 16), ws, ws_bytes, None)


def _prologue_noalloc(p, ptr=FAKE):
    return lib.sagebwd_quant_prologue_noalloc(ctypes.byref(p), *([ptr] * 16), None)


def _forward(p, ptr=FAKE):
    return lib.sagebwd_forward(ctypes.byref(p), *([ptr] * 10), None)


def _backward(p, ptr=FAKE, ws=FAKE, ws_bytes=1 << 40):
    return lib.sagebwd_backward(ctypes.byref(p), *([ptr] * 21), ws, ws_bytes, None)


@pytest.mark.parametrize("call", [_prologue, _prologue_noalloc, _forward, _backward])
def test_invalid_params_rejected(call):
    assert call(P(d=96)) == -3
    assert call(P(d=32)) == -3
    assert call(P(blk=32)) == -3
    assert call(P(dtype=7)) == -3
    assert call(P(eps=-1.0)) == -3
    assert call(P(dq_mode=3)) == -3
    assert call(P(layout=2)) == -3
    assert call(P(layout=-1)) == -3
    assert call(P(qk_gain=1, qk_norm=0)) == -3   # gains need QK-norm
    assert call(P(normed_grads=1, qk_norm=0)) == -3
    assert call(P(normed_grads=1, qk_gain=1)) == -3
    assert call(P(fmt=2)) == -3
    assert call(P(fmt=-1)) == -3
    assert call(P(fmt=_lib.FMT_FP8, q_smooth=1)) == -3   # Q-smoothing sums INT8 codes
    assert call(P(split=2)) == -3
    assert call(P(split=-1)) == -3
    assert call(P(split=_lib.SPLIT_QATTN, q_smooth=1)) == -3
    assert call(P(B=-1)) == -2
    assert call(P(N=-64)) == -2
    assert call(P(B=1 << 13, H=1 << 12)) == -2
    assert call(P(N=(1 << 22) + 64)) == -2   # per-head byte offsets must fit in 31 bits
    assert call(P(), ptr=0) == -1          # null tensors
    assert call(P(), ptr=MIS) == -4        # misaligned tensors


def test_null_params_rejected():
    assert lib.sagebwd_forward(None, *([FAKE] * 10), None) == -1
    assert lib.sagebwd_backward_workspace_bytes(None) == 0
    assert lib.sagebwd_prologue_workspace_bytes(None) == 0


def test_workspace_checks():
    p = P()
    need = lib.sagebwd_backward_workspace_bytes(ctypes.byref(p))
    n = 1 * 2 * 256 * 64
    up = lambda x: (x + 255) // 256 * 256
    # auto -> dS spill at this size: packets, K^T packets, dS tiles, multipliers
    tiles = 4 * 4 - 4 * 3 // 2          # nb * nt - (blk/64) * nb * (nb - 1) / 2, causal
    assert need == up(2 * 4 * 17408) + up(2 * 4 * 64 * 64) + up(2 * tiles * 64 * 64) + up(2 * tiles * 4)
    atomic = lib.sagebwd_backward_workspace_bytes(ctypes.byref(P(dq_mode=2)))
    assert atomic == up(2 * 4 * 17408) + up(4 * n)
    assert _backward(p, ws_bytes=need - 1) == -5
    assert _backward(p, ws=0) == -1
    assert _backward(p, ws=MIS) == -4
    pw = lib.sagebwd_prologue_workspace_bytes(ctypes.byref(p))
    assert pw == up(4 * 2 * 4 * 64)
    assert _prologue(p, ws_bytes=pw - 1) == -5
    assert _prologue(p, ws=0) == -1
    # smoothing off: the prologue needs no scratch
    assert lib.sagebwd_prologue_workspace_bytes(ctypes.byref(P(k_smooth=0))) == 0


def test_spill_needs_per_head_tiles_below_4gib():
    # causal N = 131072, blk 128: one head's dS tiles need 8.6 GB > 4 GiB of 32-bit offsets
    big = dict(B=1, H=1, N=131072, d=128, blk=128)
    assert lib.sagebwd_backward_workspace_bytes(ctypes.byref(P(dq_mode=1, **big))) == 0
    assert _backward(P(dq_mode=1, **big)) == -3
    # auto falls back to the atomic layout (packets + float32 dQ accumulator)
    up = lambda x: (x + 255) // 256 * 256
    auto = lib.sagebwd_backward_workspace_bytes(ctypes.byref(P(dq_mode=0, **big)))
    assert auto == up(131072 // 64 * 33792) + up(4 * 131072 * 128)
    # N = 65536 still spills (2.1 GB per head)
    assert lib.sagebwd_backward_workspace_bytes(ctypes.byref(P(dq_mode=1, B=1, H=1, N=65536, d=128, blk=128))) > 0


@pytest.mark.parametrize("kw", [
    dict(), dict(dq_mode=2), dict(causal=0), dict(N=200), dict(d=128, blk=128), dict(qk_gain=1),
    dict(B=1, H=1, N=65536, d=128, blk=128), dict(B=1, H=1, N=131072, d=128, blk=128),
    dict(B=1, H=1, N=131072, d=128, blk=128, causal=0, dq_mode=2)])
def test_binding_layout_matches_library(kw):
    # the binding's documented workspace offsets (which tests use to decode the packets)
    # end where the library's workspace size says, in both dQ modes and past the spill limit
    from bit_trainable_attention_amd import api
    p = P(**kw)
    lay = api.backward_workspace_layout(p)
    assert lay["total"] == lib.sagebwd_backward_workspace_bytes(ctypes.byref(p))


def test_empty_is_a_noop():
    # N == 0 (or B == 0 / H == 0): nothing is enqueued and pointers are not inspected
    for p in (P(N=0), P(B=0), P(H=0)):
        assert _prologue(p, ptr=0, ws=0, ws_bytes=0) == 0
        assert _forward(p, ptr=0) == 0
        assert _backward(p, ptr=0, ws=0, ws_bytes=0) == 0


def test_backward_part_rejects_bad_part():
    p = P()
    for part in (-1, 3, 99):
        assert lib.sagebwd_backward_part(ctypes.byref(p), part, *([FAKE] * 21), FAKE, 1 << 40, None) == -3
    assert lib.sagebwd_backward_part(ctypes.byref(P(d=96)), 0, *([FAKE] * 21), FAKE, 1 << 40, None) == -3
    assert lib.sagebwd_backward_part(ctypes.byref(p), 1, *([FAKE] * 21), FAKE, 0, None) == -5


def test_binding_rejects_host_tensors():
    # host tensors never reach the C ABI (there is no CPU path): the binding and the autograd
    # wrapper refuse them before any library call
    import torch
    from bit_trainable_attention_amd import api
    from bit_trainable_attention_amd.autograd import sagebwd_attention
    q = torch.zeros(1, 2, 128, 64, dtype=torch.float16)
    p = api.make_params(1, 2, 128, 64, 64, True, True, True, "fp16")
    with pytest.raises(ValueError, match="device tensors only"):
        api.sagebwd_quant_prologue(p, q, q, q)
    with pytest.raises(ValueError, match="device tensors only"):
        sagebwd_attention(q, q, q, blk=64)
    with pytest.raises(ValueError, match="layout"):
        sagebwd_attention(q, q, q, blk=64, layout="nhd")


def test_q_smooth_arguments():
    # the query mean / key bias pointers are required with q_smooth and ignored (NULL is
    # fine) without; the prologue scratch grows by the queries' block sums
    def pro_with(p, qm, kb):
        ptrs = [FAKE] * 12 + [qm, kb, FAKE, FAKE]
        return lib.sagebwd_quant_prologue(ctypes.byref(p), *ptrs, FAKE, 1 << 40, None)
    assert pro_with(P(q_smooth=1), 0, FAKE) == -1
    assert pro_with(P(q_smooth=1), FAKE, 0) == -1
    assert pro_with(P(q_smooth=1), MIS, FAKE) == -4
    fw = lambda p, kb: lib.sagebwd_forward(ctypes.byref(p), *([FAKE] * 6), kb, FAKE, FAKE, FAKE, None)
    assert fw(P(q_smooth=1), 0) == -1
    bw = lambda p, qm, kb: lib.sagebwd_backward(ctypes.byref(p), *([FAKE] * 9), qm, kb, *([FAKE] * 10),
                                                FAKE, 1 << 40, None)
    assert bw(P(q_smooth=1), 0, FAKE) == -1
    assert bw(P(q_smooth=1), FAKE, 0) == -1
    up = lambda x: (x + 255) // 256 * 256
    part = up(4 * 2 * 4 * 64)
    assert lib.sagebwd_prologue_workspace_bytes(ctypes.byref(P(q_smooth=1))) == 2 * part
    assert lib.sagebwd_prologue_workspace_bytes(ctypes.byref(P(q_smooth=1, k_smooth=0))) == part
    # the q_smooth-only scratch must still be passed
    assert lib.sagebwd_quant_prologue(ctypes.byref(P(q_smooth=1, k_smooth=0)), *([FAKE] * 16), FAKE,
                                      part - 1, None) == -5


def test_qk_gain_arguments():
    # with qk_gain the gains (prologue, backward) and their gradients (backward) are required,
    # and the backward workspace grows by the gains' partial sums
    def pro_with(p, qg, kg):
        return lib.sagebwd_quant_prologue(ctypes.byref(p), *([FAKE] * 14), qg, kg, FAKE, 1 << 40, None)
    assert pro_with(P(qk_gain=1), 0, FAKE) == -1
    assert pro_with(P(qk_gain=1), FAKE, 0) == -1
    assert pro_with(P(qk_gain=1), MIS, FAKE) == -4

    def bw(p, qg, kg, dqg, dkg):
        return lib.sagebwd_backward(ctypes.byref(p), *([FAKE] * 11), qg, kg, *([FAKE] * 6), dqg, dkg,
                                    FAKE, 1 << 40, None)
    assert bw(P(qk_gain=1), 0, FAKE, FAKE, FAKE) == -1
    assert bw(P(qk_gain=1), FAKE, FAKE, FAKE, 0) == -1
    assert bw(P(qk_gain=1), FAKE, FAKE, MIS, FAKE) == -4
    up = lambda x: (x + 255) // 256 * 256
    base = lib.sagebwd_backward_workspace_bytes(ctypes.byref(P()))
    gains = lib.sagebwd_backward_workspace_bytes(ctypes.byref(P(qk_gain=1)))
    assert gains == base + up(4 * 2 * 4 * 64) + up(4 * 2 * 4 * 64)   # N/64 and N/blk tiles of d floats


def test_fp8_workspace_sizes_equal_int8():
    # FP8 codes keep the INT8 byte layouts: every buffer and workspace has the same size
    for kw in (dict(), dict(dq_mode=2), dict(k_smooth=0), dict(N=200)):
        a, b = P(**kw), P(fmt=_lib.FMT_FP8, **kw)
        assert lib.sagebwd_backward_workspace_bytes(ctypes.byref(a)) == \
            lib.sagebwd_backward_workspace_bytes(ctypes.byref(b))
        assert lib.sagebwd_prologue_workspace_bytes(ctypes.byref(a)) == \
            lib.sagebwd_prologue_workspace_bytes(ctypes.byref(b))


def test_noalloc_rejects_problems_beyond_its_scratch():
    """The allocation-free prologue refuses a problem whose scratch exceeds the static array,
    after the argument checks and before any HIP call (on a host without a GPU a HIP call
    would fail with SAGEBWD_ERR_HIP instead)."""
    big = P(B=64, H=64, N=32768, d=128, blk=128)       # K block sums: 4096 heads x 256 blocks x 128 x 4 B
    assert lib.sagebwd_prologue_workspace_bytes(ctypes.byref(big)) > _lib.NOALLOC_SCRATCH_BYTES
    assert _prologue_noalloc(big) == -7
    assert lib.sagebwd_status_string(-7).decode() != "unknown status"
    assert _prologue_noalloc(big, ptr=MIS) == -4         # argument errors still come first
    assert _prologue_noalloc(big, ptr=0) == -1
    assert _prologue_noalloc(P(N=0)) == 0                # an empty problem enqueues nothing
    # a problem at the limit passes the size check (and would then look up the device)
    text = open(header_path()).read()
    m = re.search(r"#define\s+SAGEBWD_NOALLOC_SCRATCH_BYTES\s+\((\d+)ull\s*<<\s*(\d+)\)", text)
    assert m and int(m.group(1)) << int(m.group(2)) == _lib.NOALLOC_SCRATCH_BYTES


def test_qattn_forward_needs_raw_v():
    """The Q-Attn split's forward reads the raw 16-bit V (its PV is 16-bit) and not the V codes:
    a null V is an argument error, misaligned V too."""
    qa = P(split=_lib.SPLIT_QATTN)
    fw = lambda p, vtc, vs, v: lib.sagebwd_forward(ctypes.byref(p), FAKE, FAKE, vtc, FAKE, FAKE, vs, None, v,
                                                   FAKE, FAKE, None)
    assert fw(qa, FAKE, FAKE, 0) == -1
    assert fw(qa, FAKE, FAKE, MIS) == -4
    assert fw(P(), FAKE, 0, FAKE) == -1       # the SageBwd split still needs the V codes


def test_binding_layout_matches_library_random():
    # 400 seeded parameter sets (N log-uniform in 1..2^18, so that some spill and some take the
    # atomic layout; both dQ requests; gains; Q-smoothing; both formats and splits; ragged N):
    # wherever the library accepts the parameters, the binding's documented workspace layout
    # ends exactly at the size the library asks for
    import numpy as np
    from bit_trainable_attention_amd import api
    rng = np.random.default_rng(20261204)
    checked = 0
    for _ in range(400):
        d = int(rng.choice([64, 128]))
        kw = dict(B=int(rng.integers(1, 9)), H=int(rng.integers(1, 17)), N=int(np.exp(rng.uniform(0, np.log(1 << 18)))),
                  d=d, blk=int(rng.choice([64, 128])), causal=int(rng.integers(2)), dq_mode=int(rng.integers(3)),
                  qk_gain=int(rng.integers(2)), q_smooth=int(rng.random() < 0.2),
                  fmt=int(rng.choice([_lib.FMT_INT8, _lib.FMT_FP8])), split=int(rng.choice([_lib.SPLIT_SAGEBWD, _lib.SPLIT_QATTN])))
        p = P(**kw)
        n = lib.sagebwd_backward_workspace_bytes(ctypes.byref(p))
        if n == 0:
            continue   # a rejected combination (or an explicit spill past its limit)
        checked += 1
        assert api.backward_workspace_layout(p)["total"] == n, kw
    assert checked > 100
