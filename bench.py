#!/usr/bin/env python3
"""Throughput of the Inkling MoE feed-forward on one MI355X (gfx950).

One step = one inkling_moe_forward call (router logits, selection, permutation,
grouped gate_up GEMM + SwiGLU, grouped down GEMM, shared down GEMM + combine)
over one batch of synthetic hidden states that are already resident in HBM.

Default workload: prefill, T=8192 tokens, hidden=6144, 128 routed experts
(top-8), 2 shared experts, intermediate 2048, bf16 weights.  The same run also
times the decode shape (T=32, same weights) for its HBM GB/s.

Prints ONE JSON line.  `roofline` covers the dominant kernel (the grouped
gate_up GEMM) timed live with HIP events recorded on the library's stream;
`cpu_baseline` times the fp64 CPU oracle on a bounded token sample.
"""
from __future__ import annotations

import argparse
import ctypes
import hashlib
import json
import os
import re
import sys
import time

import numpy as np

PEAK_BF16_TFLOPS = 2500.0
PEAK_F32_TFLOPS = 157.3
PEAK_HBM_GBS = 8000.0

ROOT = os.path.dirname(os.path.abspath(__file__))
# HBM bytes per launch of the gate_up kernel, from two rocprofv3 --pmc runs
# (FETCH_SIZE, WRITE_SIZE), scaled by the copy-kernel factor; valid only while
# the GEMM sources hash to the value recorded beside them.
TRAFFIC_PROFILE = os.path.join(ROOT, "profiles", "gate_up_prefill_h6144_traffic.md")
GEMM_SOURCES = [os.path.join(ROOT, "mixture_experts_feed_amd", "csrc", f) for f in ("gemm.hip", "common.h")]


def log(msg):
    print(msg, file=sys.stderr, flush=True)


class HipEvents:
    """hipEvent_t handles through the HIP runtime that torch already loaded."""

    def __init__(self):
        self.hip = ctypes.CDLL("libamdhip64.so.7")
        self.hip.hipEventCreate.argtypes = [ctypes.POINTER(ctypes.c_void_p)]
        self.hip.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p, ctypes.c_void_p]
        self.hip.hipEventDestroy.argtypes = [ctypes.c_void_p]

    def create(self, n):
        arr = (ctypes.c_void_p * n)()
        for i in range(n):
            h = ctypes.c_void_p()
            rc = self.hip.hipEventCreate(ctypes.byref(h))
            if rc != 0:
                raise RuntimeError(f"hipEventCreate failed: {rc}")
            arr[i] = h.value
        return arr

    def elapsed_ms(self, a, b):
        ms = ctypes.c_float()
        rc = self.hip.hipEventElapsedTime(ctypes.byref(ms), ctypes.c_void_p(a), ctypes.c_void_p(b))
        if rc != 0:
            raise RuntimeError(f"hipEventElapsedTime failed: {rc}")
        return float(ms.value)

    def destroy(self, arr):
        for h in arr:
            self.hip.hipEventDestroy(ctypes.c_void_p(h))


def run_timed(torch, B, call, steps, warmup, events: HipEvents, record=(), per_step=None):
    """Warmup, then `steps` timed calls.  `record` holds the stage boundaries
    (0..INKLING_STAGE_EVENTS-1) at which hipEvents are recorded on the library's
    stream during the timed calls ("all" = every boundary); an event record costs
    a few microseconds, so the headline run records only what it reports.
    Returns (ms_per_step from the wall clock, {stage index: mean ms} for stages
    whose both boundaries were recorded); `per_step`, if a list, receives each
    step's duration in ms from events at the first and last boundaries
    (inkling_moe_forward calls only: the other entry points record none)."""
    n_ev = B.INKLING_STAGE_EVENTS
    idx = set(range(n_ev)) if record == "all" else set(record)
    if per_step is not None:
        idx |= {0, n_ev - 1}
    for _ in range(warmup):
        call()
    torch.cuda.synchronize()
    sets = []
    for _ in range(steps if idx else 0):
        arr = (ctypes.c_void_p * n_ev)()
        made = events.create(len(idx))
        for j, i in enumerate(sorted(idx)):
            arr[i] = made[j]
        sets.append(arr)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(steps):
        if idx:
            B.set_stage_events(sets[i])
        call()
    if idx:
        B.set_stage_events(None)
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    stage = {}
    for s_i in range(1, n_ev):
        if s_i - 1 in idx and s_i in idx:
            stage[s_i - 1] = float(np.mean([events.elapsed_ms(ev[s_i - 1], ev[s_i]) for ev in sets]))
    if per_step is not None:
        per_step.extend(events.elapsed_ms(ev[0], ev[n_ev - 1]) for ev in sets)
    for ev in sets:
        events.destroy([h for h in ev if h])
    return (t1 - t0) * 1e3 / steps, stage


def gemm_source_hash():
    h = hashlib.sha256()
    for f in GEMM_SOURCES:
        with open(f, "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()


def recorded_traffic(workload):
    """Measured HBM bytes per gate_up launch on `workload`, or None when the
    counters were taken on another workload, the kernel source changed since
    they were taken, or none were taken."""
    if not os.path.exists(TRAFFIC_PROFILE):
        return None
    text = open(TRAFFIC_PROFILE).read()
    m_h = re.search(r"^source_sha256:\s*([0-9a-f]{64})\s*$", text, re.M)
    m_b = re.search(r"^hbm_bytes_per_launch:\s*([0-9.eE+]+)\s*$", text, re.M)
    m_w = re.search(r"^workload:\s*(\S+)\s*$", text, re.M)
    if not m_h or not m_b or not m_w or m_h.group(1) != gemm_source_hash() or m_w.group(1) != workload:
        return None
    return float(m_b.group(1))


def copy_calibration(torch, mib):
    """A plain device-to-device copy of `mib` MiB (read mib, write mib), for
    scaling FETCH_SIZE / WRITE_SIZE to bytes."""
    n = mib * (1 << 20) // 4
    src = torch.empty(n, dtype=torch.float32, device="cuda:0")
    dst = torch.empty_like(src)
    src.fill_(1.0)
    torch.cuda.synchronize()
    for _ in range(3):
        dst.copy_(src)
    torch.cuda.synchronize()
    log(f"[bench] copied {mib} MiB three times")


def cpu_baseline(inp, w, n_tokens):
    """The fp64 oracle on the first n_tokens tokens of the same workload."""
    import torch
    import oracle
    from threadpoolctl import threadpool_info

    x = inp["x"][:n_tokens].float().cpu().numpy()
    bank = inp["gate_bank"].cpu().numpy()
    bias = inp["bias"].cpu().numpy()
    host_w = {k: inp[k].cpu() for k in ("w_gu", "w_d", "wsh_gu", "wsh_d")}

    class View:
        def __init__(self, t):
            self.t = t

        def __len__(self):
            return self.t.shape[0]

        def __getitem__(self, e):
            return self.t[int(e)].float().numpy()

    t0 = time.perf_counter()
    oracle.moe_forward(x, bank, bias, View(host_w["w_gu"]), View(host_w["w_d"]), View(host_w["wsh_gu"]),
                       View(host_w["wsh_d"]), w.top_k, w.route_scale, w.global_scale)
    dt = time.perf_counter() - t0
    flops = 2.0 * n_tokens * w.hidden * w.n_total + 6.0 * n_tokens * (w.top_k + w.n_shared) * w.hidden * w.intermediate
    threads = max([p.get("num_threads", 1) for p in threadpool_info() if p.get("user_api") == "blas"] or [1])
    return {"value": flops / dt / 1e12, "unit": "TFLOP/s", "cores": int(threads), "kind": "oracle",
            "sample": f"first {n_tokens} of {w.T} tokens of the same workload, all experts; "
                      f"{dt:.2f} s wall, {n_tokens / dt:.1f} tokens/s, fp64 numpy "
                      f"({len(os.sched_getaffinity(0))} cores in the affinity mask)"}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="prefill_h6144")
    ap.add_argument("--decode-workload", default="decode_h6144")
    ap.add_argument("--no-decode", action="store_true")
    ap.add_argument("--no-dense", action="store_true", help="skip the InklingDenseMLP line")
    ap.add_argument("--no-backward", action="store_true", help="skip the backward line")
    ap.add_argument("--no-others", action="store_true", help="skip the small and skewed workload lines")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-tokens", type=int, default=4096)
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="MIB",
                    help="only run a plain device copy of MIB MiB (counter calibration) and exit")
    args = ap.parse_args()

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: the library has no multi-GPU path "
              "(token sharding across GPUs is a design note, not code). Run with --gpus 1.", file=sys.stderr)
        sys.exit(2)

    import torch
    from mixture_experts_feed_amd import binding as B
    from mixture_experts_feed_amd import workloads as wl

    if not torch.cuda.is_available():
        print("no GPU visible", file=sys.stderr)
        sys.exit(1)
    dev = "cuda:0"
    if args.copy_calibration:
        copy_calibration(torch, args.copy_calibration)
        return
    B.load()
    w = wl.WORKLOADS[args.workload]
    log(f"[bench] drawing inputs for {w.name}")
    inp = wl.make_inputs(w, device=dev)
    torch.cuda.synchronize()
    S = w.n_shared
    dims = B.make_dims(w.T, w.hidden, w.n_routed, w.top_k, S, w.intermediate, w.torch_dtype)
    ws = B.alloc_workspace(dims, dev)
    out = torch.empty_like(inp["x"])

    def call():
        B.forward(inp["x"], inp["gate_bank"], inp["bias"], inp["w_gu"], inp["w_d"], inp["wsh_gu"], inp["wsh_d"],
                  w.top_k, w.route_scale, w.global_scale, out=out, workspace=ws)

    events = HipEvents()
    gu = B.STAGES.index("gate_up")   # stage i lies between boundaries i and i+1
    log(f"[bench] timing {args.steps} steps after {args.warmup} warmup")
    step_ms = []
    ms, st = run_timed(torch, B, call, args.steps, args.warmup, events, record=(gu, gu + 1), per_step=step_ms)
    _, st_all = run_timed(torch, B, call, args.steps, 2, events, record="all")
    flops = w.flops_alg()
    tflops = flops / (ms * 1e-3) / 1e12
    tok_s = w.T / (ms * 1e-3)
    stages = {n: round(st_all[i], 4) for i, n in enumerate(B.STAGES)}
    log(f"[bench] {ms:.3f} ms/step, {tflops:.1f} TFLOP/s, stages {stages}")

    # dominant kernel: grouped gate_up GEMM (routed + shared), 2*H*2I flops per (token, expert) pair,
    # its mean duration from the events around it in the timed run
    gu_flops = 2.0 * w.T * (w.top_k + S) * w.hidden * 2 * w.intermediate
    gu_ms = st[gu]
    gu_tflops = gu_flops / (gu_ms * 1e-3) / 1e12
    peak = PEAK_BF16_TFLOPS if w.dtype == "bf16" else PEAK_F32_TFLOPS
    roofline = {"kernel": "moe_gemm_kernel gate_up (routed + shared, SwiGLU epilogue)", "bound": "mfma",
                "achieved": round(gu_tflops, 2), "peak": peak, "unit": "TFLOP/s",
                "frac": round(gu_tflops / peak, 4), "traffic": recorded_traffic(w.name),
                "per_launch": {"flops": gu_flops, "avg_ms": round(gu_ms, 4)}}

    result = {
        "metric": "MoE-FFN TFLOP/s & tokens/s (hidden=6144,T=8192) + decode HBM GB/s, 1 GPU",
        "value": round(tflops, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 4),
        # each step's own duration from the hipEvents around it (value and
        # ms_per_step come from the wall clock over all steps)
        "ms_median": round(float(np.median(step_ms)), 4),
        "ms_min": round(float(np.min(step_ms)), 4),
        "ms_max": round(float(np.max(step_ms)), 4),
        "TFLOP_s_at_median": round(flops / (float(np.median(step_ms)) * 1e-3) / 1e12, 2),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": w.dtype,
        "data": "synthetic (seeded; N(0,1) hidden states, N(0,0.02) weights, U(+-0.05) gate bank and bias)",
        "config": {"workload": w.name, "T": w.T, "hidden": w.hidden, "n_routed": w.n_routed, "top_k": w.top_k,
                   "n_shared": S, "intermediate": w.intermediate, "route_scale": w.route_scale,
                   "global_scale": w.global_scale},
        "tokens_per_s": round(tok_s, 1),
        "flops_per_step": flops,
        "stage_ms": stages,   # separate pass with every stage boundary recorded
        "roofline": roofline,
    }

    if not args.no_decode:
        wd = wl.WORKLOADS[args.decode_workload]
        dinp = wl.make_inputs(wd, device=dev, with_experts=False)
        for k in ("w_gu", "w_d", "wsh_gu", "wsh_d"):
            dinp[k] = inp[k]
        ddims = B.make_dims(wd.T, wd.hidden, wd.n_routed, wd.top_k, wd.n_shared, wd.intermediate, wd.torch_dtype)
        dws = B.alloc_workspace(ddims, dev)
        dout = torch.empty_like(dinp["x"])
        routing = {}

        def dcall():
            r = B.forward(dinp["x"], dinp["gate_bank"], dinp["bias"], dinp["w_gu"], dinp["w_d"], dinp["wsh_gu"],
                          dinp["wsh_d"], wd.top_k, wd.route_scale, wd.global_scale, out=dout, workspace=dws,
                          return_routing=not routing)
            if isinstance(r, tuple):
                routing.update(r[1])

        dcall()
        torch.cuda.synchronize()
        n_touched = int((routing["expert_counts"] > 0).sum().item())
        d_steps = []
        dms, _ = run_timed(torch, B, dcall, max(20, args.steps), args.warmup, events, per_step=d_steps)
        _, dstage = run_timed(torch, B, dcall, max(20, args.steps), 2, events, record="all")
        eb = 2 if wd.dtype == "bf16" else 4
        bytes_alg = (3 * wd.hidden * wd.intermediate * eb * (n_touched + wd.n_shared)
                     + 4 * wd.hidden * (wd.n_routed + wd.n_shared) + 4 * wd.n_routed + 2 * eb * wd.T * wd.hidden)
        result["decode"] = {"workload": wd.name, "T": wd.T, "ms_per_step": round(dms, 4),
                            "ms_median": round(float(np.median(d_steps)), 4),
                            "ms_min": round(float(np.min(d_steps)), 4), "ms_max": round(float(np.max(d_steps)), 4),
                            "hbm_GBps": round(bytes_alg / (dms * 1e-3) / 1e9, 1),
                            "frac_of_peak": round(bytes_alg / (dms * 1e-3) / 1e9 / PEAK_HBM_GBS, 4),
                            "bytes_alg": bytes_alg, "n_touched_experts": n_touched,
                            "stage_ms": {n: round(dstage[i], 4) for i, n in enumerate(B.STAGES)}}
        log(f"[bench] decode {dms:.3f} ms, {result['decode']['hbm_GBps']} GB/s")

    if not args.no_others and w.name == "prefill_h6144":
        # the other two TFLOP/s workloads: skewed routing (same weights) and the small bf16 shape
        result["other_workloads"] = {}
        for oname in ("skewed_h6144", "small_bf16", "ep8_shard_h6144"):
            ow = wl.WORKLOADS[oname]
            same_shape = ow.hidden == w.hidden and ow.intermediate == w.intermediate and ow.n_shared == S
            oinp = wl.make_inputs(ow, device=dev, with_experts=not same_shape)
            if same_shape:
                # the prefill weights (the first n_routed routed experts)
                oinp["w_gu"], oinp["w_d"] = inp["w_gu"][:ow.n_routed], inp["w_d"][:ow.n_routed]
                oinp["wsh_gu"], oinp["wsh_d"] = inp["wsh_gu"], inp["wsh_d"]
            odims = B.make_dims(ow.T, ow.hidden, ow.n_routed, ow.top_k, ow.n_shared, ow.intermediate, ow.torch_dtype)
            ows = B.alloc_workspace(odims, dev)
            oout = torch.empty_like(oinp["x"])

            def ocall():
                B.forward(oinp["x"], oinp["gate_bank"], oinp["bias"], oinp["w_gu"], oinp["w_d"], oinp["wsh_gu"],
                          oinp["wsh_d"], ow.top_k, ow.route_scale, ow.global_scale, out=oout, workspace=ows)

            o_steps = []
            oms, _ = run_timed(torch, B, ocall, args.steps, args.warmup, events, per_step=o_steps)
            otf = ow.flops_alg() / (oms * 1e-3) / 1e12
            result["other_workloads"][oname] = {"T": ow.T, "hidden": ow.hidden, "ms_per_step": round(oms, 4),
                                                "ms_median": round(float(np.median(o_steps)), 4),
                                                "ms_min": round(float(np.min(o_steps)), 4),
                                                "ms_max": round(float(np.max(o_steps)), 4),
                                                "TFLOP_s": round(otf, 2), "tokens_per_s": round(ow.T / (oms * 1e-3), 1),
                                                "frac_of_peak": round(otf / PEAK_BF16_TFLOPS, 4)}
            log(f"[bench] {oname} {oms:.3f} ms, {otf:.1f} TFLOP/s")
            del oinp, ows, oout

    if not args.no_dense:
        # InklingDenseMLP of the first layer (intermediate 24576) on the same token count
        dw = wl.DENSE_WORKLOADS["dense_h6144"]
        dn = wl.dense_inputs(dw, device=dev)
        ddims = B.make_dense_dims(dw.T, dw.hidden, dw.intermediate, dw.torch_dtype)
        dws = torch.empty(max(1, B.dense_workspace_size(ddims)), dtype=torch.uint8, device=dev)
        dout = torch.empty_like(dn["x"])

        def dense_call():
            B.dense_mlp_forward(dn["x"], dn["gate_up"], dn["down"], dw.global_scale, out=dout, workspace=dws)

        dms, _ = run_timed(torch, B, dense_call, args.steps, args.warmup, events)
        dtf = dw.flops_alg() / (dms * 1e-3) / 1e12
        result["dense_mlp"] = {"workload": dw.name, "T": dw.T, "hidden": dw.hidden, "intermediate": dw.intermediate,
                               "ms_per_step": round(dms, 4), "TFLOP_s": round(dtf, 2),
                               "frac_of_peak": round(dtf / PEAK_BF16_TFLOPS, 4), "flops_per_step": dw.flops_alg()}
        log(f"[bench] dense MLP {dms:.3f} ms, {dtf:.1f} TFLOP/s")
        del dn, dws, dout

    if not args.no_backward:
        # backward of the same prefill step: gradients of <dout, out>
        bw_steps = max(3, args.steps // 4)
        dout_b = torch.randn(inp["x"].shape, generator=torch.Generator().manual_seed(7)).to(inp["x"].dtype).to(dev)
        bdims = B.make_dims(w.T, w.hidden, w.n_routed, w.top_k, S, w.intermediate, w.torch_dtype)
        bws = torch.empty(B.backward_workspace_size(bdims), dtype=torch.uint8, device=dev)
        f32 = dict(dtype=torch.float32, device=dev)
        grads = {"dx": torch.empty_like(inp["x"]), "d_gate_bank": torch.empty(tuple(inp["gate_bank"].shape), **f32),
                 "d_w_gu": torch.empty(tuple(inp["w_gu"].shape), **f32), "d_w_d": torch.empty(tuple(inp["w_d"].shape), **f32),
                 "d_wsh_gu": torch.empty(tuple(inp["wsh_gu"].shape), **f32),
                 "d_wsh_d": torch.empty(tuple(inp["wsh_d"].shape), **f32)}

        def bw_call():
            B.backward(inp["x"], inp["gate_bank"], inp["bias"], inp["w_gu"], inp["w_d"], inp["wsh_gu"], inp["wsh_d"],
                       w.top_k, w.route_scale, w.global_scale, dout_b, workspace=bws, grads=grads)

        bms, _ = run_timed(torch, B, bw_call, bw_steps, 2, events)
        # algorithmic: dact, dx, d down, d gate_up (12 T (k+S) H I) and the gate bank (2 T H (E+S));
        # the gate_up recompute (4 T (k+S) H I) is reported beside it
        bw_flops = 12.0 * w.T * (w.top_k + S) * w.hidden * w.intermediate + 2.0 * w.T * w.hidden * w.n_total
        re_flops = 4.0 * w.T * (w.top_k + S) * w.hidden * w.intermediate
        btf = bw_flops / (bms * 1e-3) / 1e12
        result["backward"] = {"workload": w.name, "ms_per_step": round(bms, 4), "TFLOP_s": round(btf, 2),
                              "frac_of_peak": round(btf / PEAK_BF16_TFLOPS, 4), "flops_alg": bw_flops,
                              "recompute_flops": re_flops,
                              "TFLOP_s_with_recompute": round((bw_flops + re_flops) / (bms * 1e-3) / 1e12, 2)}
        log(f"[bench] backward {bms:.3f} ms, {btf:.1f} TFLOP/s algorithmic")

        # the same backward with bf16 weight gradients (each the fp32 gradient
        # rounded once): half the gradient bytes written
        bf = dict(dtype=torch.bfloat16, device=dev)
        grads16 = dict(grads, d_w_gu=torch.empty(tuple(inp["w_gu"].shape), **bf),
                       d_w_d=torch.empty(tuple(inp["w_d"].shape), **bf),
                       d_wsh_gu=torch.empty(tuple(inp["wsh_gu"].shape), **bf),
                       d_wsh_d=torch.empty(tuple(inp["wsh_d"].shape), **bf))

        def bw16_call():
            B.backward(inp["x"], inp["gate_bank"], inp["bias"], inp["w_gu"], inp["w_d"], inp["wsh_gu"], inp["wsh_d"],
                       w.top_k, w.route_scale, w.global_scale, dout_b, workspace=bws, grads=grads16)

        b16ms, _ = run_timed(torch, B, bw16_call, bw_steps, 2, events)
        b16tf = bw_flops / (b16ms * 1e-3) / 1e12
        result["backward_bf16_weight_grads"] = {"workload": w.name, "ms_per_step": round(b16ms, 4),
                                                "TFLOP_s": round(b16tf, 2),
                                                "frac_of_peak": round(b16tf / PEAK_BF16_TFLOPS, 4)}
        log(f"[bench] backward, bf16 weight gradients {b16ms:.3f} ms, {b16tf:.1f} TFLOP/s algorithmic")
        del grads16

        # training step: the training forward keeps the gate_up projections,
        # and the backward reads them instead of recomputing
        saved = torch.empty(B.saved_size(bdims), dtype=torch.uint8, device=dev)
        tr_out = torch.empty_like(inp["x"])

        def train_call():
            B.forward(inp["x"], inp["gate_bank"], inp["bias"], inp["w_gu"], inp["w_d"], inp["wsh_gu"], inp["wsh_d"],
                      w.top_k, w.route_scale, w.global_scale, out=tr_out, workspace=ws, saved=saved)
            B.backward(inp["x"], inp["gate_bank"], inp["bias"], inp["w_gu"], inp["w_d"], inp["wsh_gu"], inp["wsh_d"],
                       w.top_k, w.route_scale, w.global_scale, dout_b, workspace=bws, grads=grads, saved=saved)

        tms, _ = run_timed(torch, B, train_call, bw_steps, 2, events)
        ttf = (w.flops_alg() + bw_flops) / (tms * 1e-3) / 1e12
        result["train_step"] = {"workload": w.name, "ms_per_step": round(tms, 4), "TFLOP_s": round(ttf, 2),
                                "frac_of_peak": round(ttf / PEAK_BF16_TFLOPS, 4),
                                "saved_bytes": B.saved_size(bdims),
                                "note": "inkling_moe_forward_train + inkling_moe_backward from the saved projections"}
        log(f"[bench] training step (forward keeping h + backward) {tms:.3f} ms, {ttf:.1f} TFLOP/s algorithmic")
        del bws, grads, dout_b, saved, tr_out

    if not args.no_cpu_baseline:
        log(f"[bench] timing the CPU oracle on {args.cpu_tokens} tokens")
        result["cpu_baseline"] = cpu_baseline(inp, w, args.cpu_tokens)

    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
