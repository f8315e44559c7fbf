#!/usr/bin/env python3
"""Throughput of the SageBwd-style INT8 attention hot path on one MI355X.

A step is one pass of the whole path over one batch of synthetic input resident in HBM:
quantisation prologue -> INT8 forward -> INT8/FP16 backward (all kernels). The workload is
B2 H16 N8192 d128, causal, fp16, QK-norm and K-smoothing on, 128-token quantisation blocks.
Throughput counts the seven attention matmuls: 14*d operations per visible (query, key) pair
(12*d in INT8, 2*d in FP16), for the whole step.

Prints ONE JSON line on stdout; diagnostics go to stderr.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

# MI355X published dense peaks (TOP/s): INT8 5.0 POPS, FP16/BF16 2.5 PFLOPS.
PEAK_I8 = 5000.0
PEAK_F16 = 2500.0
PROFILE_TRAFFIC = os.path.join(ROOT, "profiles", "bwd_main_n8192_d128_traffic.txt")
KERNEL_SOURCES = [os.path.join(ROOT, "bit_trainable_attention_amd", "csrc", f)
                  for f in ("backward.hip", "common.hpp")]


def weighted_peak(n_i8: int, n_f16: int) -> float:
    tot = n_i8 + n_f16
    return 1.0 / ((n_i8 / tot) / PEAK_I8 + (n_f16 / tot) / PEAK_F16)


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def kernel_source_hash() -> str:
    h = hashlib.sha256()
    for f in KERNEL_SOURCES:
        with open(f, "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()


def traffic_from_profile():
    """HBM bytes per bwd_main launch from the committed rocprofv3 counter summary, or None
    if there is none or the kernel source changed since it was taken."""
    if not os.path.exists(PROFILE_TRAFFIC):
        return None
    with open(PROFILE_TRAFFIC) as f:
        d = json.load(f)
    if d.get("source_sha256") != kernel_source_hash():
        return None
    return d.get("hbm_bytes_per_launch")


def cpu_baseline(w, x, heads: int, fmt: str = "int8"):
    """The plain CPU oracle (as it stands) on `heads` heads of the same workload."""
    from threadpoolctl import threadpool_info
    from oracle import quant as oq
    from tests.harness import spec_for
    from bit_trainable_attention_amd import workloads as wl
    ws = w.with_shape(B=1, H=heads)
    sl = lambda a: np.ascontiguousarray(a.reshape((-1,) + a.shape[2:])[:heads].reshape((1, heads) + a.shape[2:]))
    Qf, Kf, Vf, dOf = (wl.bits_to_f32(sl(x[k]), w.dtype) for k in ("Q", "K", "V", "dO"))
    spec = spec_for(ws, fmt=fmt)
    t0 = time.perf_counter()
    oq.run(Qf, Kf, Vf, dOf, spec)
    dt = time.perf_counter() - t0
    threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    model = "unknown CPU"
    try:
        with open("/proc/cpuinfo") as f:
            model = next((ln.split(":", 1)[1].strip() for ln in f if ln.startswith("model name")), model)
    except OSError:
        pass
    return dict(value=ws.algorithmic_ops() / dt / 1e12, unit="TOPS", cores=int(threads), kind="oracle",
                sample=f"{heads} of {w.B * w.H} heads (B1 H{heads} N{w.N} d{w.d}), quantised oracle "
                       f"prologue+forward+backward, float64 numpy, {dt:.1f} s on {model}",
                seconds=dt)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="n8192_d128")
    ap.add_argument("--cpu-heads", type=int, default=8)
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="MiB",
                    help="before warm-up, run one plain device-to-device copy of this many MiB "
                         "(a known-traffic kernel for scaling the FETCH_SIZE / WRITE_SIZE counters)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--q-smooth", action="store_true",
                    help="time the Q-smoothing variant on the same inputs (default: off, as the metric)")
    ap.add_argument("--layout", default="bhnd", choices=("bhnd", "bnhd"),
                    help="memory layout of the 16-bit tensors handed to the library (default [B,H,N,d])")
    ap.add_argument("--fmt", default="int8", choices=("int8", "fp8"),
                    help="code format of the six quantised products (default INT8, as the metric)")
    ap.add_argument("--split", default="sagebwd", choices=("sagebwd", "qattn"),
                    help="precision split: six of seven products quantised (default, the metric) or the "
                         "Q-Attn split (QK^T and the dS products quantised, PV, P^T dO, dO V^T in 16 bits)")
    ap.add_argument("--dq-mode", default="auto", choices=("auto", "spill", "atomic"),
                    help="how the backward reduces dQ over key blocks (default: the library's choice)")
    ap.add_argument("--no-autograd", action="store_true",
                    help="skip the extra timing of the same step through the autograd wrapper")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: the library has no multi-GPU path "
              "(the attention shards over heads with no communication between them).", file=sys.stderr)
        sys.exit(2)

    import torch
    from bit_trainable_attention_amd import api
    from bit_trainable_attention_amd import workloads as wl
    w = wl.WORKLOADS[args.workload]
    if args.q_smooth:
        w = w.with_shape(q_smooth=True)

    def to_device(bits):
        t = torch.from_numpy(np.ascontiguousarray(bits).view(np.int16))
        return t.view(torch.float16 if w.dtype == "fp16" else torch.bfloat16).to("cuda:0")

    log(f"[bench] workload {w.name}: B{w.B} H{w.H} N{w.N} d{w.d} {w.dtype} causal={w.causal} "
        f"qk_norm={w.qk_norm} k_smooth={w.k_smooth} blk={w.blk}")
    x = wl.make_inputs(w)
    p = api.make_params(w.B, w.H, w.N, w.d, w.blk, w.causal, w.qk_norm, w.k_smooth, w.dtype, eps=w.eps,
                        q_smooth=w.q_smooth, layout=args.layout, fmt=args.fmt,
                        dq_mode={"auto": 0, "spill": 1, "atomic": 2}[args.dq_mode], split=args.split)
    dev = torch.device("cuda:0")
    Q, K, V, dO = (to_device(x[k]) for k in ("Q", "K", "V", "dO"))
    if args.layout == "bnhd":
        Q, K, V, dO = (t.transpose(1, 2).contiguous() for t in (Q, K, V, dO))
    pro = api.sagebwd_quant_prologue(p, Q, K, V)
    pro_ws = torch.empty(max(api.sagebwd_prologue_workspace_bytes(p), 1), dtype=torch.uint8, device=dev)
    O, lse = api.sagebwd_forward(p, pro, V=V)
    grads = {n: torch.empty_like(Q) for n in ("dQ", "dK", "dV")}
    bws = torch.empty(api.sagebwd_backward_workspace_bytes(p), dtype=torch.uint8, device=dev)
    torch.cuda.synchronize()

    if args.copy_calibration > 0:
        n = args.copy_calibration << 20
        src = torch.ones(n // 4, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst

    stages = ["prologue", "forward", "bwd_pre", "bwd_main", "bwd_dq"]

    def step(ev):
        ev[0].record()
        api.sagebwd_quant_prologue(p, Q, K, V, out=pro, workspace=pro_ws)
        ev[1].record()
        api.sagebwd_forward(p, pro, O=O, lse=lse, V=V)
        ev[2].record()
        for part in range(3):
            api.sagebwd_backward_part(p, part, Q, K, V, pro, O, lse, dO, grads, bws)
            ev[3 + part].record()

    mk = lambda: [torch.cuda.Event(enable_timing=True) for _ in range(6)]
    for _ in range(args.warmup):
        step(mk())
    torch.cuda.synchronize()
    evs = [mk() for _ in range(args.steps)]
    t_start = torch.cuda.Event(enable_timing=True)
    t_end = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t_start.record()
    for i in range(args.steps):
        step(evs[i])
    t_end.record()
    torch.cuda.synchronize()
    total_ms = t_start.elapsed_time(t_end)
    ms_per_step = total_ms / args.steps
    stage_ms = {s: float(np.mean([e[j].elapsed_time(e[j + 1]) for e in evs])) for j, s in enumerate(stages)}
    per_step = np.array([e[0].elapsed_time(e[5]) for e in evs])
    step_stats = {"median": float(np.median(per_step)), "min": float(per_step.min()),
                  "p90": float(np.percentile(per_step, 90))}

    pairs = w.visible_pairs()
    ops = w.algorithmic_ops()
    value = ops / (ms_per_step * 1e-3) / 1e12
    peak_step = weighted_peak(6, 1)
    # bwd_main's products depend on where dQ = dS K runs: with the dS spill (the default at this
    # size) bwd_main does the recomputed QK^T, dV, dK (INT8) and dP (FP16), 8*d ops per visible
    # pair against a 3:1 INT8/FP16 peak, and the dQ pass does dQ (2*d INT8 ops per pair); with
    # float32 atomics bwd_main does all five (10*d, 4:1) and the dQ pass only the epilogue
    spill = bool(api.backward_workspace_layout(p)["spill"])
    n_i8_main = 3 if spill else 4
    ops_main = (2 * n_i8_main + 2) * w.d * pairs
    ach_main = ops_main / (stage_ms["bwd_main"] * 1e-3) / 1e12
    peak_main = weighted_peak(n_i8_main, 1)
    ops_dq = 2 * w.d * pairs if spill else 0
    traffic = traffic_from_profile() if args.fmt == "int8" else None   # (counters of the INT8 kernel)
    # each stage's own ideal: the stages with products at their dense MFMA peaks (forward: QK^T
    # and PV in INT8; bwd_main as above; the dQ pass: dS K in INT8), the others at 8 TB/s of
    # their algorithmic HBM bytes (E = B*H*N*d elements: the prologue reads Q, K, V and writes
    # three code tensors, 9E; bwd_pre reads dO, O, Qc, Kc and writes the packets, 11E). The dS
    # spill is the dQ pass's working traffic, not algorithmic bytes; without it the dQ pass is
    # the RMSNorm backward over the float32 accumulator (reads 4E + Q 2E, writes dQ 2E)
    E = w.B * w.H * w.N * w.d
    hbm = 8e12
    stage_ideal_ms = {"prologue": 9 * E / hbm * 1e3, "forward": 4 * w.d * pairs / (PEAK_I8 * 1e12) * 1e3,
                      "bwd_pre": 11 * E / hbm * 1e3, "bwd_main": ops_main / (peak_main * 1e12) * 1e3,
                      "bwd_dq": ops_dq / (PEAK_I8 * 1e12) * 1e3 if spill else 8 * E / hbm * 1e3}
    log(f"[bench] {ms_per_step:.3f} ms/step, {value:.1f} TOPS = {100 * value / peak_step:.1f}% of the "
        f"{peak_step:.0f} TOPS INT8/FP16 (6:1) dense peak; stages (ms): "
        + ", ".join(f"{k} {v:.3f}" for k, v in stage_ms.items()))
    fwd_ops = 4 * w.d * pairs
    log(f"[bench] forward {fwd_ops / (stage_ms['forward'] * 1e-3) / 1e12:.1f} TOPS (INT8 peak {PEAK_I8:.0f}); "
        f"bwd_main {ach_main:.1f} TOPS ({n_i8_main}:1 INT8/FP16 peak {peak_main:.0f}); dQ pass "
        + (f"{ops_dq / (stage_ms['bwd_dq'] * 1e-3) / 1e12:.1f} TOPS (INT8 peak {PEAK_I8:.0f})" if spill
           else "epilogue only (atomic dQ)"))

    autograd_ms = None
    if not args.no_autograd:
        # the same step through torch.autograd (bit_trainable_attention_amd.autograd): the
        # wrapper's own outputs, workspaces and saved tensors come from torch's allocator
        from bit_trainable_attention_amd.autograd import sagebwd_attention
        qg, kg, vg = (t.detach().clone().requires_grad_() for t in (Q, K, V))

        def ag_step():
            for t in (qg, kg, vg):
                t.grad = None
            o = sagebwd_attention(qg, kg, vg, causal=w.causal, qk_norm=w.qk_norm, k_smooth=w.k_smooth,
                                  blk=w.blk, eps=w.eps, q_smooth=w.q_smooth, layout=args.layout, fmt=args.fmt,
                                  split=args.split)
            o.backward(dO)

        # (as many warm-up steps as the main timing: the first steps also grow the allocator's
        # pool for the wrapper's own tensors)
        for _ in range(max(args.warmup, 5)):
            ag_step()
        n_ag = max(1, min(args.steps, 10))
        a0, a1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        a0.record()
        for _ in range(n_ag):
            ag_step()
        a1.record()
        torch.cuda.synchronize()
        autograd_ms = a0.elapsed_time(a1) / n_ag
        log(f"[bench] autograd wrapper: {autograd_ms:.3f} ms/step over {n_ag} steps")
        del qg, kg, vg

    out = {
        "metric": ("INT8" if args.fmt == "int8" else "FP8 (e4m3)")
        + " attention fwd+bwd TOPS at B2 H16 N8192 d128 causal; % of MFMA peak",
        "value": round(value, 2),
        "unit": "TOPS",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "int8+fp16" if args.fmt == "int8" else "fp8e4m3+fp16",
        "data": "synthetic",
        "config": {"workload": f"{w.name}: B{w.B} H{w.H} N{w.N} d{w.d} causal {w.dtype} QK-norm "
                               f"K-smoothing blk{w.blk}{' Q-smoothing' if w.q_smooth else ''} (prologue+fwd+bwd)",
                   "B": w.B, "H": w.H, "N": w.N, "d": w.d, "causal": w.causal, "blk": w.blk,
                   "dtype": w.dtype, "q_smooth": w.q_smooth, "layout": args.layout, "fmt": args.fmt,
                   "parallelism": "single GPU"},
        "frac_of_peak": round(value / peak_step, 4),
        "step_ms": {k: round(v, 4) for k, v in step_stats.items()},
        "stages_ms": {k: round(v, 4) for k, v in stage_ms.items()},
        "stages_frac_of_ideal": {k: round(stage_ideal_ms[k] / stage_ms[k], 4) for k in stage_ms},
        "roofline": {"kernel": "bwd_main", "bound": "mfma", "achieved": round(ach_main, 2),
                     "peak": round(peak_main, 1), "unit": "TFLOP/s", "frac": round(ach_main / peak_main, 4),
                     "traffic": traffic,
                     "ops_per_pair": (2 * n_i8_main + 2) * w.d, "pairs": pairs,
                     "mix": f"{n_i8_main}:1 INT8:FP16 ({'dS spill: dQ in the dQ pass' if spill else 'atomic dQ'})"},
        "dq_pass": ({"ops_per_pair": 2 * w.d, "achieved": round(ops_dq / (stage_ms["bwd_dq"] * 1e-3) / 1e12, 2),
                     "peak": PEAK_I8, "unit": "TOPS", "frac": round(ops_dq / (stage_ms["bwd_dq"] * 1e-3) / 1e12
                                                                   / PEAK_I8, 4)} if spill else None),
        "cpu_baseline": None,
        "autograd_ms_per_step": None if autograd_ms is None else round(autograd_ms, 4),
    }
    if not args.no_cpu_baseline:
        log(f"[bench] CPU oracle baseline on {args.cpu_heads} head(s)...")
        cb = cpu_baseline(w, x, args.cpu_heads, args.fmt)
        log(f"[bench] CPU oracle: {cb['seconds']:.1f} s, {cb['value']:.5f} TOPS, {cb['cores']} threads")
        cb.pop("seconds")
        out["cpu_baseline"] = cb
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
