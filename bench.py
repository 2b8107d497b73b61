"""Benchmark of one rank's tensor-parallel layer shard on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W]

Prints ONE JSON line.  The timed step is the whole prefill hot path of rank 0
of a 7B-shaped layer split two ways (hidden 4096, 16 of 32 heads x 128,
SwiGLU 5504 of 11008, RMSNorm, RoPE, bf16, batch 1 x 2048 tokens, causal):
ATTN stage (RMSNorm, Q/K/V projection with RoPE and KV-cache write, causal
attention, row-parallel output projection) -> reduce of the two ranks'
partials + residual -> MLP stage (RMSNorm, gate/up projection with SwiGLU,
row-parallel down projection) -> reduce.  Rank 1's partials are computed once
before timing (they stand for the other GPU's contribution).

`value` is the shard step's algorithmic FLOPs (GEMMs + causal attention) per
second.  `roofline` covers the dominant kernel (the gate/up projection GEMM),
timed with HIP events on its launch stream inside the timed steps.  `decode`
reports batch-1 decode of rank 0 of the 7B layer split four ways against a
1024-position cache, in microseconds per token per layer, over a stack of
distinct layer copies whose weights (0.8 GB) exceed the 256 MB Infinity Cache.
`cpu_baseline` times the CPU oracle (NumPy float64) on the same prefill step.
"""

from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "shard-layer prefill TFLOP/s (% MFMA peak) + decode µs/token/layer (% HBM BW)"
PEAK_BF16_TFLOPS = 2500.0      # MI355X dense bf16 MFMA
PEAK_HBM_GBPS = 8000.0         # MI355X HBM3E


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--decode-layers", type=int, default=8)
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    ap.add_argument("--no-decode", action="store_true")
    return ap.parse_args()


def prefill_flops(w, t):
    """Algorithmic FLOPs of one rank's prefill step: the four projections
    plus causal attention (QK^T and PV over the causal half)."""
    d = w.hidden // w.heads
    hl, kvl, fl = w.heads // t, w.kv_heads // t, w.ffn // t
    T = w.batch * w.seq
    nqkv = (hl + 2 * kvl) * d
    gemm = {
        "gemm_qkv": 2 * T * w.hidden * nqkv,
        "gemm_out": 2 * T * hl * d * w.hidden,
        "gemm_up": 2 * T * w.hidden * 2 * fl,
        "gemm_down": 2 * T * fl * w.hidden,
    }
    attn = 2 * w.batch * hl * w.seq * w.seq * d
    return gemm, attn


def decode_bytes(w, t, L):
    """Algorithmic HBM bytes of one decode token on one rank at cache length
    L: the rank's bf16 weights once, K/V of positions 0..L read, one K/V
    position written (activations are a few KB and left out)."""
    d = w.hidden // w.heads
    hl, kvl, fl = w.heads // t, w.kv_heads // t, w.ffn // t
    weights = 2 * ((hl + 2 * kvl) * d * w.hidden + w.hidden * hl * d + 2 * fl * w.hidden + w.hidden * fl)
    kv = 2 * 2 * kvl * d * (L + 1) + 2 * 2 * kvl * d
    per_kernel = {
        "gemv_qkv": 2 * (hl + 2 * kvl) * d * w.hidden,
        "gemv_out": 2 * w.hidden * hl * d,
        "gemv_up": 2 * 2 * fl * w.hidden,
        "gemv_down": 2 * w.hidden * fl,
        "attn_decode": 2 * 2 * kvl * d * (L + 1),
    }
    return weights + kv, per_kernel


def source_sha(name):
    p = os.path.join(ROOT, "tensor_transformer_layer_tp_amd", "csrc", name)
    return hashlib.sha256(open(p, "rb").read()).hexdigest()[:16]


def traffic_for(kernel, src, launches_per_step):
    """HBM bytes per launch from the committed rocprofv3 counter summary, if
    it was taken on the current kernel source; else None."""
    p = os.path.join(ROOT, "profiles", "traffic.json")
    if not os.path.exists(p):
        return None
    rec = json.load(open(p)).get(kernel)
    if not rec or rec.get("source_sha") != source_sha(src):
        return None
    return rec.get("bytes_per_launch")


def timed(fn, steps, warmup, stream):
    import torch
    for _ in range(warmup):
        fn()
    torch.cuda.synchronize()
    t0 = torch.cuda.Event(enable_timing=True)
    t1 = torch.cuda.Event(enable_timing=True)
    t0.record(stream)
    for _ in range(steps):
        fn()
    t1.record(stream)
    torch.cuda.synchronize()
    return t0.elapsed_time(t1) / steps


def bench_prefill(args, torch, T):
    from tensor_transformer_layer_tp_amd import ATTN, MLP, Shard, partial_reduce, synth
    w = synth.WORKLOADS["7b-t2-prefill"]
    t = w.tp
    raw = synth.draw_workload(w)
    dev = {k: synth.to_storage(v, "bf16").cuda() for k, v in raw.items()}
    wdev = {k: v for k, v in dev.items() if k != "x"}
    x = dev["x"]
    shards = [Shard(w.hidden, w.heads, w.kv_heads, w.ffn, t, r) for r in range(t)]
    for sh in shards:
        sh.load_weights(wdev)
        sh.reserve(w.batch * w.seq)
    B, S, h = w.batch, w.seq, w.hidden
    kv = shards[0].kv_cache(B, S)
    # the other rank's partials (the contribution a second GPU would send)
    pa = [torch.empty((B, S, h), dtype=torch.float32, device="cuda") for _ in range(t)]
    pm = [torch.empty((B, S, h), dtype=torch.float32, device="cuda") for _ in range(t)]
    hbuf = torch.empty_like(x)
    ybuf = torch.empty_like(x)
    for r in range(1, t):
        shards[r].prefill(ATTN, x, None, out=pa[r])
    shards[0].prefill(ATTN, x, kv, out=pa[0])
    partial_reduce(pa, residual=x, out=hbuf)
    for r in range(1, t):
        shards[r].prefill(MLP, hbuf, out=pm[r])
    torch.cuda.synchronize()
    sh = shards[0]
    stream = torch.cuda.current_stream()

    def step():
        sh.prefill(ATTN, x, kv, out=pa[0])
        partial_reduce(pa, residual=x, out=hbuf)
        sh.prefill(MLP, hbuf, out=pm[0])
        partial_reduce(pm, residual=hbuf, out=ybuf)

    # timed region: the kernel timer brackets the dominant kernel (gate/up
    # projection) with events on its launch stream inside these same steps
    dom = "gemm_up"
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    sh.timing(True, kinds=[dom])
    ms = timed(step, args.steps, 0, stream)
    dom_times = sh.timing_read()[dom]
    # per-kernel breakdown: a second pass with every kernel bracketed
    sh.timing(True)
    ms_marked = timed(step, args.steps, 0, stream)
    ktimes = sh.timing_read()
    sh.timing(False)
    gemm, attn = prefill_flops(w, t)
    total = sum(gemm.values()) + attn
    kern = {k: {"avg_us": 1e3 * v[0] / v[1], "launches": v[1]} for k, v in ktimes.items()}
    for k, f in gemm.items():
        if k in kern:
            kern[k]["tflops"] = f / (kern[k]["avg_us"] * 1e-6) / 1e12
    if "attn_prefill" in kern:
        kern["attn_prefill"]["tflops"] = attn / (kern["attn_prefill"]["avg_us"] * 1e-6) / 1e12
    gemm_us = sum(kern[k]["avg_us"] for k in gemm if k in kern)
    dom_us = 1e3 * dom_times[0] / dom_times[1]
    achieved = gemm[dom] / (dom_us * 1e-6) / 1e12
    traffic = traffic_for("gemm_up_7b_t2", "gemm_bf16.hip", 1)
    out = {
        "w": w, "ms": ms, "ms_marked": ms_marked, "dom_us": dom_us, "flops": total, "gemm_flops": sum(gemm.values()),
        "attn_flops": attn, "kernels": kern, "gemm_us": gemm_us,
        "roofline": {"bound": "mfma", "achieved": round(achieved, 2), "peak": PEAK_BF16_TFLOPS,
                     "unit": "TFLOP/s", "frac": round(achieved / PEAK_BF16_TFLOPS, 4), "traffic": traffic,
                     "kernel": "gemm (gate/up projection + SwiGLU epilogue), M=2048 N=11008 K=4096",
                     "avg_us": round(dom_us, 3), "launches": dom_times[1], "flops_per_launch": gemm[dom]},
        "state": (w, raw),
    }
    for s_ in shards:
        s_.close()
    kv.close()
    return out


def bench_decode(args, torch):
    from tensor_transformer_layer_tp_amd import ATTN, MLP, Shard, partial_reduce, synth
    w = synth.WORKLOADS["7b-t4-decode"]
    t, L0 = w.tp, w.kv_len
    raw = synth.draw_workload(w)
    dev = {k: synth.to_storage(v, "bf16").cuda() for k, v in raw.items()}
    wdev = {k: v for k, v in dev.items() if k not in ("k_cache", "v_cache", "x_dec")}
    nl = args.decode_layers
    cap = L0 + args.warmup + 2 * args.steps + 4
    layers = []
    for _ in range(nl):
        sh = Shard(w.hidden, w.heads, w.kv_heads, w.ffn, t, 0)
        sh.load_weights(wdev)
        kv = sh.kv_cache(1, cap)
        kfull = torch.zeros(kv.shape, dtype=torch.bfloat16, device="cuda")
        vfull = torch.zeros(kv.shape, dtype=torch.bfloat16, device="cuda")
        kvl = w.kv_heads // t
        kfull[:, :, :L0] = dev["k_cache"][:, :kvl]
        vfull[:, :, :L0] = dev["v_cache"][:, :kvl]
        kv.write(kfull, vfull)
        kv.length = L0
        layers.append((sh, kv))
    del wdev
    # the other ranks' partials: fixed buffers standing for the other GPUs
    others = [torch.randn((1, w.hidden), device="cuda", dtype=torch.float32) * 0.1 for _ in range(t - 1)]
    x0 = dev["x_dec"]
    pa = torch.empty((1, w.hidden), dtype=torch.float32, device="cuda")
    pm = torch.empty_like(pa)
    hb = torch.empty_like(x0)
    yb = [torch.empty_like(x0) for _ in range(2)]
    stream = torch.cuda.current_stream()

    def step():
        x = x0
        for i, (sh, kv) in enumerate(layers):
            sh.decode(ATTN, x, kv, out=pa)
            partial_reduce([pa, *others], residual=x, out=hb)
            sh.decode(MLP, hb, out=pm)
            y = yb[i & 1]
            partial_reduce([pm, *others], residual=hb, out=y)
            x = y

    ms = timed(step, args.steps, args.warmup, stream)
    # per-kernel durations from a separate pass with event markers
    for sh, _ in layers:
        sh.timing(True)
    timed(step, args.steps, 0, stream)
    agg = {}
    for sh, _ in layers:
        for k, (tot, n) in sh.timing_read().items():
            a = agg.setdefault(k, [0.0, 0])
            a[0] += tot
            a[1] += n
        sh.timing(False)
    L_avg = L0 + args.warmup + args.steps + (args.steps - 1) / 2.0   # mean cache length of the timed steps
    nbytes, per_kernel = decode_bytes(w, t, int(L_avg))
    us = 1e3 * ms / nl
    kern = {k: {"avg_us": 1e3 * v[0] / v[1], "launches": v[1]} for k, v in agg.items()}
    for k, b in per_kernel.items():
        if k in kern:
            kern[k]["GBps"] = b / (kern[k]["avg_us"] * 1e-6) / 1e9
    dom = "gemv_up"
    ach = per_kernel[dom] / (kern[dom]["avg_us"] * 1e-6) / 1e9
    for sh, kv in layers:
        sh.close()
        kv.close()
    return {
        "workload": "7b-t4-decode: hidden 4096, rank 0 of t=4 (8 of 32 heads x 128, SwiGLU 2752 of 11008), "
                    f"bf16, batch 1, cache {L0}+ positions, {nl} distinct layer copies",
        "us_per_token_layer": round(us, 3),
        "bytes_per_token_layer": nbytes,
        "hbm_GBps": round(nbytes / (us * 1e-6) / 1e9, 1),
        "hbm_frac": round(nbytes / (us * 1e-6) / 1e9 / PEAK_HBM_GBPS, 4),
        "kernels": {k: {kk: round(vv, 3) if isinstance(vv, float) else vv for kk, vv in v.items()}
                    for k, v in kern.items()},
        "roofline": {"bound": "hbm", "achieved": round(ach, 1), "peak": PEAK_HBM_GBPS, "unit": "GB/s",
                     "frac": round(ach / PEAK_HBM_GBPS, 4), "traffic": None,
                     "kernel": "gemv_kernel (gate/up + SwiGLU, fused RMSNorm), N=5504 K=4096",
                     "bytes_per_launch": per_kernel[dom]},
    }


def cpu_baseline(state):
    """The CPU oracle (NumPy float64) on the same rank-0 prefill step; the
    other rank's partials are computed first, outside the timed part."""
    import numpy as np
    from threadpoolctl import threadpool_info

    from oracle import layer as O
    w, raw = state
    from tensor_transformer_layer_tp_amd import synth
    ex = {k: synth.to_storage(v, "bf16").float().numpy() for k, v in raw.items()}
    spec = O.Spec(w.hidden, w.heads, w.kv_heads, w.ffn)
    x = ex["x"]
    a1 = O.attn_stage(x, ex, spec, w.tp, 1)["partial"]
    a0 = O.attn_stage(x, ex, spec, w.tp, 0)["partial"]
    h = O.reduce([a0, a1], x, spec)
    m1 = O.mlp_stage(h, ex, spec, w.tp, 1)["partial"]
    steps, t_tot = 0, 0.0
    while steps < 5 and (t_tot < 10.0 or steps == 0):
        t0 = time.perf_counter()
        a0 = O.attn_stage(x, ex, spec, w.tp, 0)["partial"]
        hh = O.reduce([a0, a1], x, spec)
        m0 = O.mlp_stage(hh, ex, spec, w.tp, 0)["partial"]
        O.reduce([m0, m1], hh, spec)
        t_tot += time.perf_counter() - t0
        steps += 1
    threads = max([p.get("num_threads", 1) for p in threadpool_info() if p.get("user_api") == "blas"] or [1])
    return steps, t_tot, threads


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only (got --gpus {args.gpus}); multi-GPU runs are not part of this "
              "build", file=sys.stderr)
        sys.exit(2)
    import torch
    torch.cuda.set_device(0)
    pre = bench_prefill(args, torch, None)
    dec = None if args.no_decode else bench_decode(args, torch)
    w = pre["w"]
    tflops = pre["flops"] / (pre["ms"] * 1e-3) / 1e12
    line = {
        "metric": METRIC,
        "value": round(tflops, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(pre["ms"], 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded N(0,1) activations, N(0,0.02) weights, random-init)",
        "config": {
            "workload": "7b-t2-prefill: rank 0 of a 7B-shaped layer split t=2 (hidden 4096, 16 of 32 heads x 128, "
                        "SwiGLU 5504 of 11008, RMSNorm, RoPE), bf16, batch 1 x seq 2048, causal; step = ATTN stage "
                        "+ reduce + MLP stage + reduce",
            "global_batch": w.batch, "seq_len": w.seq, "parallelism": "tp2 shard (rank 0) on 1 GPU",
        },
        "mfma_frac": round(tflops / PEAK_BF16_TFLOPS, 4),
        "flops_per_step": pre["flops"],
        "gemm_tflops": round(pre["gemm_flops"] / (pre["gemm_us"] * 1e-6) / 1e12, 2),
        "gemm_mfma_frac": round(pre["gemm_flops"] / (pre["gemm_us"] * 1e-6) / 1e12 / PEAK_BF16_TFLOPS, 4),
        "ms_per_step_all_kernels_bracketed": round(pre["ms_marked"], 4),
        "kernels": {k: {kk: round(vv, 3) if isinstance(vv, float) else vv for kk, vv in v.items()}
                    for k, v in pre["kernels"].items()},
        "roofline": pre["roofline"],
    }
    if dec is not None:
        line["decode"] = dec
    if not args.no_cpu:
        steps, secs, threads = cpu_baseline(pre["state"])
        line["cpu_baseline"] = {
            "value": round(pre["flops"] * steps / secs / 1e12, 5), "unit": "TFLOP/s", "cores": threads,
            "kind": "oracle",
            "sample": f"{steps} full rank-0 prefill step(s) of the same workload (B=1, S=2048) in NumPy float64, "
                      f"{secs:.1f} s",
        }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
